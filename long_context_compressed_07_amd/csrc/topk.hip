// csa_topk kernels: per-query selection of the k highest-scoring visible entries.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 and yudonglee.me "DeepSeek-V4 详解" 2.2
// Step 3 (only the top-k compressed rows by indexer score enter attention). Ties go to the lower
// index and the output lists indices in ascending order (this library's reading).
//
// Algorithm (deterministic: the result depends only on the keys' order). Scores map to
// order-preserving 32-bit keys, held in registers, PER per thread: wave v of a workgroup holds
// 64 PER consecutive positions as groups of 256, lane l keys 4 l .. 4 l + 3 of each group
// (key_pos), so that every load instruction of a wave reads one contiguous span. The selection is
// bound by vector ALU work per key (few workgroups per CU, one key per lane and instruction), so
// each step keeps that work small. Single-stage rows first look for the
// k-th largest key K in equal-width score bins (kth_key_by_value: one histogram, then a direct
// ranking of the few keys in K's bin). Otherwise, and when that bin is crowded, K is found by a
// radix select: the block's largest and smallest keys fix the bits every key shares; then, from
// the highest differing bit down, each level counts in an LDS histogram the next digit (at most 11
// bits) of the keys that match the digits found so far, and a block scan over the histogram
// locates the digit of the k-th key and its rank among the keys of that digit. Starting at the
// highest differing bit spreads clustered keys over the histogram, which keeps LDS atomic
// conflicts low. Compaction keeps every key > K and the lowest-position keys == K: per-wave
// counts from ballots, one exchange of them between the waves, then each selected key's output
// offset from lane-mask counts (mbcnt) in position order; selected positions are staged in LDS and
// written out with coalesced stores.
//
// Rows of up to kChunk (8192) visible entries: one 256-thread workgroup per row; rows of up to
// kWideChunk (32768): one 1024-thread workgroup per row (the same code, 32 keys per thread).
// Longer rows in a call with few rows (a decode step: one row per sequence) take the
// sampled-threshold path below, which spreads each row over many workgroups. Other longer rows:
// stage 1 runs the same selection on chunks of kWideChunk entries (several 1024-thread
// workgroups per row) and writes each chunk's local top-k (ascending); stage 2 selects the row's
// top-k among the concatenated candidates, with the 256-thread form when they fit in it. The
// union of the chunks' top-k contains the row's top-k under the same tie rule, so the result is
// exact. Every chunk before a row's last visible one holds kWideChunk >= k entries and so yields
// exactly k candidates: a row's candidates are the first n slots of its [chunks][k] block, in
// entry order.
#include <mutex>

#include "common.h"

namespace csa {
namespace {

constexpr int kChunk = 8192;      // single-stage limit of the 256-thread row kernel
constexpr int kWideChunk = 32768; // 1024-thread row kernel limit and entries per stage-1 chunk
constexpr int kCandMax = 32768;   // candidates per row in stage 2
constexpr int kPer = 32;          // keys per thread
constexpr int kBins = 2048;       // LDS ints per histogram (11-bit digits); two per workgroup
constexpr int kMaxK = 2048;       // largest k staged in LDS (and largest k of rows > kChunk)

// Order-preserving map float -> uint32 (larger float -> larger key); -0.0 and +0.0 map alike.
// Finite scores give keys >= 1; padding keys are 0.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Barrier for LDS hand-offs: waits for this wave's LDS operations only, so global loads and
// stores stay in flight across it.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// DPP controls (GFX9 encoding): shift right within a row of 16 lanes, and broadcasts of lane 15
// of each row to the next row / of lane 31 to rows 2 and 3.
constexpr int kRowShr = 0x110;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;

template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp(int fill, int x) {
  return __builtin_amdgcn_update_dpp(fill, x, CTRL, ROWS, 0xf, false);
}

// Inclusive prefix sum over the wave's 64 lanes.
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += dpp<kRowShr + 1, 0xf>(0, x);
  x += dpp<kRowShr + 2, 0xf>(0, x);
  x += dpp<kRowShr + 4, 0xf>(0, x);
  x += dpp<kRowShr + 8, 0xf>(0, x);
  x += dpp<kRowBcast15, 0xa>(0, x);
  x += dpp<kRowBcast31, 0xc>(0, x);
  return x;
}

// Running max / min in lane order (lane 63 holds the wave's result).
__device__ __forceinline__ uint32_t wave_incl_max(uint32_t x) {
  x = max(x, (uint32_t)dpp<kRowShr + 1, 0xf>(0, (int)x));
  x = max(x, (uint32_t)dpp<kRowShr + 2, 0xf>(0, (int)x));
  x = max(x, (uint32_t)dpp<kRowShr + 4, 0xf>(0, (int)x));
  x = max(x, (uint32_t)dpp<kRowShr + 8, 0xf>(0, (int)x));
  x = max(x, (uint32_t)dpp<kRowBcast15, 0xa>(0, (int)x));
  x = max(x, (uint32_t)dpp<kRowBcast31, 0xc>(0, (int)x));
  return x;
}

__device__ __forceinline__ uint32_t wave_incl_min(uint32_t x) {
  x = min(x, (uint32_t)dpp<kRowShr + 1, 0xf>(-1, (int)x));
  x = min(x, (uint32_t)dpp<kRowShr + 2, 0xf>(-1, (int)x));
  x = min(x, (uint32_t)dpp<kRowShr + 4, 0xf>(-1, (int)x));
  x = min(x, (uint32_t)dpp<kRowShr + 8, 0xf>(-1, (int)x));
  x = min(x, (uint32_t)dpp<kRowBcast15, 0xa>(-1, (int)x));
  x = min(x, (uint32_t)dpp<kRowBcast31, 0xc>(-1, (int)x));
  return x;
}

__device__ __forceinline__ int lane63(int x) { return __builtin_amdgcn_readlane(x, 63); }

// Position of key i of this thread within its workgroup's span of NT PER positions: wave v holds
// [64 PER v, 64 PER (v + 1)) as PER / 4 groups of 256 positions, lane l positions 4 l .. 4 l + 3
// of each group. Position order is (wave, group, lane, key within the lane's four).
template <int PER>
__device__ __forceinline__ int key_pos(int i) {
  static_assert(PER % 4 == 0, "groups of four keys per lane");
  return (int)(threadIdx.x / kWave) * (kWave * PER) + 256 * (i >> 2) +
         4 * (int)(threadIdx.x & (kWave - 1)) + (i & 3);
}

// Number of set bits of the wave mask m in lanes below this one, plus acc.
__device__ __forceinline__ int mbcnt(uint64_t m, int acc) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, (uint32_t)acc));
}

// Exclusive prefix sum (in thread order) of a per-thread count over the block, and the total.
// s_tmp: NT / 64 ints.
template <int NT>
__device__ __forceinline__ int block_scan(int a, int* s_tmp, int& total) {
  constexpr int NW = NT / kWave;
  const int wv = threadIdx.x / kWave;
  const int ia = wave_incl_sum(a);
  if ((threadIdx.x & (kWave - 1)) == kWave - 1) s_tmp[wv] = ia;
  lds_sync();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = s_tmp[w];
    before += w < wv ? c : 0;
    total += c;
  }
  lds_sync();   // s_tmp is free again
  return before + ia - a;
}

// Largest key and smallest nonzero key of the block. s_tmp: 2 NT / 64 ints.
template <int NT, int PER>
__device__ __forceinline__ void block_range(const uint32_t (&kv)[PER], int* s_tmp,
                                            uint32_t& mx, uint32_t& mn) {
  constexpr int NW = NT / kWave;
  uint32_t a = 0, b = ~0u;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    a = max(a, kv[i]);
    b = min(b, kv[i] == 0u ? ~0u : kv[i]);
  }
  a = lane63((int)wave_incl_max(a));
  b = lane63((int)wave_incl_min(b));
  const int wv = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) {
    s_tmp[wv] = (int)a;
    s_tmp[NW + wv] = (int)b;
  }
  lds_sync();
  mx = 0;
  mn = ~0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    mx = max(mx, (uint32_t)s_tmp[w]);
    mn = min(mn, (uint32_t)s_tmp[NW + w]);
  }
  lds_sync();
}

// Given a histogram of kBins digit values, finds the digit d holding the kk-th largest key (digits
// above d hold fewer than kk keys, digits >= d at least kk) and turns kk into the rank of that key
// among the keys of digit d, and count into the number of keys of digit d. Every thread returns the
// same d, kk and count. s_tmp: NT / 64 + 3 ints.
template <int NT>
__device__ __forceinline__ uint32_t find_digit(const int* hist, int& kk, int* s_tmp, int& count) {
  constexpr int B = kBins / NT;
  static_assert(B >= 2 && B % 2 == 0, "bins per thread");
  int* s_res = s_tmp + NT / kWave;
  const int t = threadIdx.x;
  int h[B];
  int local = 0;
#pragma unroll
  for (int b = 0; b < B; b += 2) {
    const int2 v = reinterpret_cast<const int2*>(hist + t * B)[b / 2];
    h[b] = v.x;
    h[b + 1] = v.y;
    local += v.x + v.y;
  }
  int total;
  const int before = block_scan<NT>(local, s_tmp, total);
  int acc = total - before - local;   // keys in the digits of higher threads
  if (acc < kk && kk <= acc + local) {
#pragma unroll
    for (int b = B - 1; b >= 0; --b) {
      if (acc < kk && kk <= acc + h[b]) {
        s_res[0] = t * B + b;
        s_res[1] = kk - acc;
        s_res[2] = h[b];
      }
      acc += h[b];
    }
  }
  lds_sync();
  kk = s_res[1];
  count = s_res[2];
  const uint32_t d = (uint32_t)s_res[0];
  lds_sync();   // s_res is free again
  return d;
}

__device__ __forceinline__ void clear_hist(int* hist, int nt) {
  for (int i = threadIdx.x; i < 2 * kBins / 4; i += nt) reinterpret_cast<int4*>(hist)[i] = int4{0, 0, 0, 0};
}

// The score a nonzero key stands for (inverse of score_key; both zeros give +0.0).
__device__ __forceinline__ float key_score(uint32_t u) {
  return __uint_as_float(u ^ ((int32_t)u < 0 ? 0x80000000u : 0xffffffffu));
}

// First pass of kth_key for scores spread over their range: kBins bins of equal width in score
// between the smallest real score f0 and the largest (scale = kBins / width). A key's bin never
// decreases as its score grows, so the bin that holds the k-th largest key follows from the bin
// counts, and for scores without heavy clustering that bin holds a few keys (far fewer LDS atomic
// conflicts than the radix digits of the sign and exponent bits). Those keys are gathered in
// position order and ranked against each other. Returns false, with hist zero again, when that
// bin holds more than NT keys; otherwise the k-th largest key and *need_eq as kth_key.
template <int NT, int PER>
__device__ bool kth_key_by_value(const uint32_t (&kv)[PER], int k, float f0, float scale,
                                 int* hist, int* s_tmp, uint32_t* kth, int* need_eq) {
  auto bin = [&](uint32_t key) {
    const int b = (int)((key_score(key) - f0) * scale);   // >= 0: key_score(key) >= f0
    return b < kBins - 1 ? b : kBins - 1;
  };
  // Each key's bin, kept from the histogram pass for the gather below: two 16-bit fields per
  // word, 0xffff for padding keys.
  uint32_t bp[(PER + 1) / 2];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    uint32_t b = 0xffffu;
    if (kv[i] != 0u) {
      b = (uint32_t)bin(kv[i]);
      atomicAdd(&hist[b], 1);
    }
    if (i & 1)
      bp[i >> 1] |= b << 16;
    else
      bp[i >> 1] = b;
  }
  auto bin_of = [&](int i) { return (bp[i >> 1] >> (16 * (i & 1))) & 0xffffu; };
  lds_sync();
  int kk = k, count;
  const int d = (int)find_digit<NT>(hist, kk, s_tmp, count);
  if (count > NT) {   // hist zero again for the radix passes
    for (int i = threadIdx.x; i < kBins / 4; i += NT) reinterpret_cast<int4*>(hist)[i] = int4{0, 0, 0, 0};
    lds_sync();
    return false;
  }
  // The keys of bin d (in any order: only their values matter), into the second histogram's space.
  uint32_t* s_cand = reinterpret_cast<uint32_t*>(hist + kBins);
  int mine = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) mine += bin_of(i) == (uint32_t)d;
  int total;
  int off = block_scan<NT>(mine, s_tmp, total);
  if (mine > 0) {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (bin_of(i) == (uint32_t)d) s_cand[off++] = kv[i];
  }
  // Padded with zero keys (below every real key) to a multiple of 16 for the 16-byte reads.
  const int t = threadIdx.x;
  const int n16 = (count + 15) & ~15;   // <= NT
  if (t >= count && t < n16) s_cand[t] = 0u;
  lds_sync();
  // The kk-th largest among them: the key with fewer than kk larger keys and at least kk keys
  // larger or equal (every copy of it writes the same values).
  int* s_res = s_tmp + NT / kWave;
  if (t < count) {
    const uint32_t my = s_cand[t];
    int gt = 0, eq = 0;
    const uint4* c4 = reinterpret_cast<const uint4*>(s_cand);
    for (int j = 0; j < n16 / 4; j += 4) {
      uint4 v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = c4[j + u];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        gt += (v[u].x > my) + (v[u].y > my) + (v[u].z > my) + (v[u].w > my);
        eq += (v[u].x == my) + (v[u].y == my) + (v[u].z == my) + (v[u].w == my);
      }
    }
    if (gt < kk && kk <= gt + eq) {
      s_res[0] = (int)my;
      s_res[1] = kk - gt;
    }
  }
  lds_sync();
  *kth = (uint32_t)s_res[0];
  *need_eq = s_res[1];
  lds_sync();   // s_res is free again
  return true;
}

// The k-th largest of the block's keys (1 <= k <= number of real keys; padding keys are 0, below
// every real key), and in *need_eq how many keys equal to it belong to the top k. hist: 2 kBins
// ints, zero on entry (clear_hist, then an LDS barrier); s_tmp: 2 NT / 64 + 2 ints. With BY_VALUE,
// scores with a finite, nonzero range take the equal-width bins first; clustered ones (more than
// NT keys in the k-th key's bin) and non-finite ranges take the radix select below. The bins pay
// where several workgroups share a CU's LDS (one workgroup per row, many rows: 568 -> 365 us for
// 32768 rows of up to 8192 scores); the chunk and merge kernels of long rows run with about one
// workgroup per CU, where the radix alone measured faster (12.2 vs 13.8 us per chunk launch).
template <int NT, bool BY_VALUE, int PER>
__device__ uint32_t kth_key(const uint32_t (&kv)[PER], int k, int* hist, int* s_tmp,
                            int* need_eq) {
  uint32_t mx, mn;
  block_range<NT>(kv, s_tmp, mx, mn);
  if (mx == mn) {   // one distinct real key
    *need_eq = k;
    return mx;
  }
  if constexpr (BY_VALUE) {
    const float f0 = key_score(mn);
    const float width = key_score(mx) - f0;
    const float scale = (float)kBins / width;
    // NaN fails every comparison; an infinite score makes width or scale infinite.
    if (width > 0.f && width <= 3.4028235e38f && scale <= 3.4028235e38f) {
      uint32_t K;
      if (kth_key_by_value<NT, PER>(kv, k, f0, scale, hist, s_tmp, &K, need_eq)) return K;
    }
  }
  const int p = 31 - __builtin_clz(mx ^ mn);   // highest bit in which real keys differ
  // Keys matching the digits found so far: (key & pmask) == prefix. The bits above p are shared
  // by every real key; a padding key matches only if they are all zero, and then it sits below
  // every real key in the lowest digit, which leaves the k-th largest unchanged.
  uint32_t pmask = p == 31 ? 0u : ~0u << (p + 1);
  uint32_t prefix = mx & pmask;
  int kk = k;
  int lo = p + 1;
  int level = 0;
  while (lo > 0) {
    const int hi = lo - 1;
    lo = hi >= 10 ? hi - 10 : 0;
    const uint32_t dmask = (2u << (hi - lo)) - 1u;
    int* h = hist + (level & 1) * kBins;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      if ((kv[i] & pmask) == prefix) atomicAdd(&h[(kv[i] >> lo) & dmask], 1);
    }
    lds_sync();
    int count;
    const uint32_t d = find_digit<NT>(h, kk, s_tmp, count);
    // This histogram serves the level after next: clear it (every thread has read it).
    for (int i = threadIdx.x; i < kBins / 4; i += NT) reinterpret_cast<int4*>(h)[i] = int4{0, 0, 0, 0};
    prefix |= d << lo;
    pmask |= dmask << lo;
    ++level;
  }
  *need_eq = kk;
  return prefix;
}

// Calls put(o, j, key) for the top k in ascending position order o = 0 .. k-1 (j = key_pos(i) for
// key kv[i]): keys > K and the first need_eq keys == K. The block's numbers of keys > K and == K
// go to *tot_gt and *tot_eq when given. Ends with an LDS barrier. s_tmp: 2 NT / 64 ints.
template <int NT, int PER, typename Put>
__device__ void compact(const uint32_t (&kv)[PER], uint32_t K, int need_eq, int k, int* s_tmp,
                        Put put, int* tot_gt = nullptr, int* tot_eq = nullptr) {
  // Padding keys (0) are below every real key, and K is a real key (>= 1), so they never count.
  constexpr int NW = NT / kWave;
  const int wv = threadIdx.x / kWave;
  int gl = 0, el = 0;   // this lane's keys > K and == K
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    gl += kv[i] > K;
    el += kv[i] == K;
  }
  // The wave's counts, both in one sum (at most 64 PER < 2^16 each).
  const int both = wave_incl_sum(gl | (el << 16));
  if ((threadIdx.x & (kWave - 1)) == kWave - 1) {
    s_tmp[wv] = both & 0xffff;
    s_tmp[NW + wv] = both >> 16;
  }
  lds_sync();
  int g_before = 0, e_before = 0, tg = 0, te = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int g = s_tmp[w], e = s_tmp[NW + w];
    g_before += w < wv ? g : 0;
    e_before += w < wv ? e : 0;
    tg += g;
    te += e;
  }
  lds_sync();   // s_tmp is free again
  if (tot_gt != nullptr) *tot_gt = tg;
  if (tot_eq != nullptr) *tot_eq = te;
  const int ne = need_eq < 0 ? 0 : need_eq;
  // Selected keys before this wave, and keys == K before the current group.
  int off = g_before + (e_before < ne ? e_before : ne);
  int eseen = e_before;
  const bool take_all_eq = te <= ne;   // uniform: every key == K belongs to the top k
  const int p0 = key_pos<PER>(0);
#pragma unroll
  for (int q = 0; q < PER / 4; ++q) {
    bool sel[4];
    if (take_all_eq) {
#pragma unroll
      for (int c = 0; c < 4; ++c) sel[c] = kv[4 * q + c] >= K;
    } else {
      bool e[4];
      uint64_t me[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        e[c] = kv[4 * q + c] == K;
        me[c] = __ballot(e[c]);
      }
      // Rank of each key == K among the row's keys == K, in position order.
      int r = mbcnt(me[3], mbcnt(me[2], mbcnt(me[1], mbcnt(me[0], eseen))));
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        sel[c] = kv[4 * q + c] > K || (e[c] && r < ne);
        r += e[c];
      }
      eseen += __popcll(me[0]) + __popcll(me[1]) + __popcll(me[2]) + __popcll(me[3]);
    }
    uint64_t ms[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) ms[c] = __ballot(sel[c]);
    int o = mbcnt(ms[3], mbcnt(ms[2], mbcnt(ms[1], mbcnt(ms[0], off))));
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (sel[c] && (unsigned)o < (unsigned)k) put(o, p0 + 256 * q + c, kv[4 * q + c]);
      o += sel[c];
    }
    off += __popcll(ms[0]) + __popcll(ms[1]) + __popcll(ms[2]) + __popcll(ms[3]);
  }
  lds_sync();
}

// Score value of element j of a row: fp32, or bf16 (widened exactly to fp32).
__device__ __forceinline__ float score_at(const float* row, int64_t j) { return row[j]; }
__device__ __forceinline__ float score_at(const uint16_t* row, int64_t j) {
  return __uint_as_float((uint32_t)row[j] << 16);
}

// Loads this thread's keys (positions key_pos(i)) of a row of n scores, 0 beyond n: one 16-byte
// load per group of four that lies inside a 16-byte aligned row, element by element otherwise.
// The row is read once per selection: non-temporal loads (about 2% faster than ordinary loads
// for the 32K prefill's rows: 311 -> 306 us, the two timed in alternation).
typedef float f32x4 __attribute__((ext_vector_type(4)));
template <int PER>
__device__ __forceinline__ void load_keys(const float* row, int n, uint32_t (&kv)[PER]) {
  const int p0 = key_pos<PER>(0);
  if ((reinterpret_cast<uintptr_t>(row) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const int p = p0 + 256 * q;
      if (p + 4 <= n) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(row + p));
        kv[4 * q] = score_key(v.x);
        kv[4 * q + 1] = score_key(v.y);
        kv[4 * q + 2] = score_key(v.z);
        kv[4 * q + 3] = score_key(v.w);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) kv[4 * q + c] = p + c < n ? score_key(row[p + c]) : 0u;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = p0 + 256 * (i >> 2) + (i & 3);
      kv[i] = p < n ? score_key(row[p]) : 0u;
    }
  }
}

// bf16 scores: one 8-byte load of four codes per group (the same conditions, 8-byte aligned
// rows); each code is the high half of its fp32 value.
template <int PER>
__device__ __forceinline__ void load_keys(const uint16_t* row, int n, uint32_t (&kv)[PER]) {
  const int p0 = key_pos<PER>(0);
  if ((reinterpret_cast<uintptr_t>(row) & 7) == 0) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const int p = p0 + 256 * q;
      if (p + 4 <= n) {
        const uint2 v = *reinterpret_cast<const uint2*>(row + p);
        kv[4 * q] = score_key(__uint_as_float(v.x << 16));
        kv[4 * q + 1] = score_key(__uint_as_float(v.x & 0xffff0000u));
        kv[4 * q + 2] = score_key(__uint_as_float(v.y << 16));
        kv[4 * q + 3] = score_key(__uint_as_float(v.y & 0xffff0000u));
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          kv[4 * q + c] = p + c < n ? score_key(score_at(row, p + c)) : 0u;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = p0 + 256 * (i >> 2) + (i & 3);
      kv[i] = p < n ? score_key(score_at(row, p)) : 0u;
    }
  }
}

// The same for keys already mapped (stage-2 candidates).
template <int PER>
__device__ __forceinline__ void load_mapped(const uint32_t* keys, int n, uint32_t (&kv)[PER]) {
  const int p0 = key_pos<PER>(0);
  if ((reinterpret_cast<uintptr_t>(keys) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const int p = p0 + 256 * q;
      if (p + 4 <= n) {
        const uint4 v = *reinterpret_cast<const uint4*>(keys + p);
        kv[4 * q] = v.x;
        kv[4 * q + 1] = v.y;
        kv[4 * q + 2] = v.z;
        kv[4 * q + 3] = v.w;
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) kv[4 * q + c] = p + c < n ? keys[p + c] : 0u;
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int p = p0 + 256 * (i >> 2) + (i & 3);
      kv[i] = p < n ? keys[p] : 0u;
    }
  }
}

// Single stage: one workgroup per query row (n_vis <= NT * kPer). For 256 threads, five waves per
// SIMD (at most 96 VGPRs: room for the keys' bins beside the keys): 307 us for 32768 rows of up
// to 8192 scores, against 321 us at six waves without the bins kept.
template <int NT, typename S>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(NT == 256 ? 5 : 4, NT == 256 ? 5 : 4)))
topk_row_kernel(TopkArgs a) {
  __shared__ int s_tmp[2 * NT / kWave + 2];
  __shared__ __attribute__((aligned(16))) int s_hist[2 * kBins];
  const int qi = blockIdx.x;
  const int n = (int)n_visible(a.Q.pos[qi], a.m, a.N);
  int32_t* out = a.idx + (int64_t)qi * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += NT) out[i] = i < n ? i : -1;
    return;
  }
  uint32_t kv[kPer];
  load_keys(static_cast<const S*>(a.scores) + (int64_t)qi * a.ld_scores, n, kv);
  clear_hist(s_hist, NT);
  lds_sync();
  int need_eq;
  const uint32_t K = kth_key<NT, true>(kv, a.k, s_hist, s_tmp, &need_eq);
  if (a.k <= kMaxK) {   // staged in LDS, then coalesced stores
    compact<NT>(kv, K, need_eq, a.k, s_tmp, [&](int o, int j, uint32_t) { s_hist[o] = j; });
    for (int i = threadIdx.x; i < a.k; i += NT) out[i] = s_hist[i];
  } else {
    compact<NT>(kv, K, need_eq, a.k, s_tmp, [&](int o, int j, uint32_t) { out[o] = j; });
  }
}

// Stage 1: chunk c of query row qi; writes the chunk's local top-k (or all of its visible
// entries) as (key, index) pairs in ascending index order.
template <int NT, typename S>
__global__ void __launch_bounds__(NT) topk_chunk_kernel(TopkArgs a, int n_chunks,
                                                        uint32_t* cand_key, int32_t* cand_idx) {
  constexpr int kChunkN = NT * kPer;   // entries per chunk: one key segment per thread
  __shared__ int s_tmp[2 * NT / kWave + 2];
  __shared__ __attribute__((aligned(16))) int s_hist[2 * kBins];
  const int qi = blockIdx.x / n_chunks;
  const int c = blockIdx.x - qi * n_chunks;
  const int64_t nv = n_visible(a.Q.pos[qi], a.m, a.N);
  const int64_t base = (int64_t)c * kChunkN;
  const int64_t slot = (int64_t)qi * n_chunks + c;
  int32_t* oi = cand_idx + slot * a.k;
  uint32_t* ok = cand_key + slot * a.k;
  const int n = base >= nv ? 0 : (int)(nv - base < kChunkN ? nv - base : kChunkN);
  const S* row = static_cast<const S*>(a.scores) + (int64_t)qi * a.ld_scores + base;
  if (n <= a.k) {
    for (int j = threadIdx.x; j < n; j += NT) {
      oi[j] = (int32_t)(base + j);
      ok[j] = score_key(score_at(row, j));
    }
    return;
  }
  uint32_t kv[kPer];
  load_keys(row, n, kv);
  clear_hist(s_hist, NT);
  lds_sync();
  int need_eq;
  const uint32_t K = kth_key<NT, false>(kv, a.k, s_hist, s_tmp, &need_eq);
  int* s_pos = s_hist;
  uint32_t* s_key = reinterpret_cast<uint32_t*>(s_hist + kMaxK);
  compact<NT>(kv, K, need_eq, a.k, s_tmp, [&](int o, int j, uint32_t key) {
    s_pos[o] = j;
    s_key[o] = key;
  });
  for (int i = threadIdx.x; i < a.k; i += NT) {
    oi[i] = (int32_t)base + s_pos[i];
    ok[i] = s_key[i];
  }
}

// Stage 2: the row's top-k among its candidates (n <= NT * kPer).
template <int NT>
__global__ void __launch_bounds__(NT) topk_merge_kernel(TopkArgs a, int n_chunks,
                                                        const uint32_t* cand_key,
                                                        const int32_t* cand_idx) {
  __shared__ int s_tmp[2 * NT / kWave + 2];
  __shared__ __attribute__((aligned(16))) int s_hist[2 * kBins];
  const int qi = blockIdx.x;
  int32_t* out = a.idx + (int64_t)qi * a.k;
  const int64_t nv = n_visible(a.Q.pos[qi], a.m, a.N);
  int n = 0;
  if (nv > 0) {
    const int64_t last = (nv - 1) / kWideChunk;
    const int64_t in_last = nv - last * kWideChunk;
    n = (int)(last * a.k + (in_last < a.k ? in_last : a.k));
  }
  const int32_t* cidx = cand_idx + (int64_t)qi * n_chunks * a.k;
  if (n <= a.k) {   // no more visible entries than k: every candidate, in order
    for (int i = threadIdx.x; i < a.k; i += NT) out[i] = i < n ? cidx[i] : -1;
    return;
  }
  uint32_t kv[kPer];
  load_mapped(cand_key + (int64_t)qi * n_chunks * a.k, n, kv);
  clear_hist(s_hist, NT);
  lds_sync();
  int need_eq;
  const uint32_t K = kth_key<NT, NT == 256>(kv, a.k, s_hist, s_tmp, &need_eq);
  compact<NT>(kv, K, need_eq, a.k, s_tmp, [&](int o, int j, uint32_t) { s_hist[o] = j; });
  // Entry indices of the selected candidates, gathered eight at a time.
  for (int i0 = 0; i0 < a.k; i0 += 8 * NT) {
    int32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * NT + (int)threadIdx.x;
      const int j = i < a.k ? s_hist[i] : 0;
      v[u] = cidx[(unsigned)j < (unsigned)n ? j : 0];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * NT + (int)threadIdx.x;
      if (i < a.k) out[i] = v[u];
    }
  }
}

// ---- Sampled threshold: rows longer than kChunk when there are few of them ---------------------
// One workgroup per row picks a threshold key T from evenly spaced samples (topk_sample_kernel);
// workgroups of kFiltN entries then write the row's keys at or above T, with their positions, as
// one candidate list per workgroup in position order (topk_filter_kernel); one workgroup per row
// gathers the lists (in workgroup order, so the candidates stay in position order) and selects the
// top k among them (topk_select_kernel). With C keys at or above T: C >= k means the row's k-th
// key is at or above T, so every key of the top k is a candidate and the top k of the candidates
// (ties to the lower position) is the row's; a sample that misjudged the row (C < k), or too many
// candidates (a list past kCandCap, or C past kSelCap), sends the row to an exact selection over
// all of its keys in the select workgroup. Every case yields the unique top k, so which one ran
// never shows in the result. These kernels run 1024 threads, few keys each: a decode call has too
// few rows to fill the GPU, so each workgroup's latency, not the throughput, sets the time.
constexpr int kSNT = 1024;                   // threads of the sampled path's workgroups
constexpr int kSampPer = 2;                  // samples per thread
constexpr int kSamp = kSNT * kSampPer;       // samples per row
constexpr int kFiltPer = 8;                  // entries per thread of a filter workgroup
constexpr int kFiltN = kSNT * kFiltPer;      // entries per filter workgroup
constexpr int kSelCap = kSNT * kFiltPer;     // keys one select workgroup ranks
constexpr int kCandCap = 512;                // candidates one filter workgroup may list
constexpr int kMaxFilt = 64;                 // filter workgroups per row

// Samples of a row of n > 0 keys: positions floor(i n / s), i < s = min(n, kSamp). T is the r-th
// largest sample: s evenly spaced samples hold about k s / n keys at or above the row's k-th key;
// twice that plus 16 makes a shortfall unlikely unless the scores line up with the sample
// positions, and then the exact fallback still gives the right result.
__host__ __device__ __forceinline__ int sample_rank(int64_t n, int k) {
  const int64_t s = n < kSamp ? n : kSamp;
  const int64_t r = 2 * ((k * s + n - 1) / n) + 16;
  return (int)(r < s ? r : s);
}

template <typename S>
__global__ void __launch_bounds__(kSNT) topk_sample_kernel(TopkArgs a, uint32_t* thr) {
  __shared__ int s_tmp[2 * kSNT / kWave + 2];
  __shared__ __attribute__((aligned(16))) int s_hist[2 * kBins];
  const int qi = blockIdx.x;
  const int64_t nv = n_visible(a.Q.pos[qi], a.m, a.N);
  if (nv <= a.k) return;   // the select kernel writes such rows without a threshold
  const S* row = static_cast<const S*>(a.scores) + (int64_t)qi * a.ld_scores;
  const int64_t s = nv < kSamp ? nv : kSamp;
  uint32_t kv[kSampPer];
#pragma unroll
  for (int u = 0; u < kSampPer; ++u) {
    const int64_t i = (int64_t)threadIdx.x * kSampPer + u;
    kv[u] = i < s ? score_key(score_at(row, i * nv / s)) : 0u;
  }
  clear_hist(s_hist, kSNT);
  lds_sync();
  int need_eq;
  const uint32_t T = kth_key<kSNT, true>(kv, sample_rank(nv, a.k), s_hist, s_tmp, &need_eq);
  if (threadIdx.x == 0) thr[qi] = T;
}

// Candidates of filter workgroup c of row qi, entries c kFiltN + 1024 u + t (u < kFiltPer): the
// keys >= T and their positions, in position order ((u, wave, lane) order), as the list
// cand[qi][c][0 .. count) with count in counts[qi][c] (a count past kCandCap: the list overflowed,
// only its first kCandCap entries are written). Entries past the visible ones have key 0, below
// every real T.
template <typename S>
__global__ void __launch_bounds__(kSNT) topk_filter_kernel(TopkArgs a, int n_f, const uint32_t* thr,
                                                           int* counts, uint2* cand) {
  constexpr int NW = kSNT / kWave;
  __shared__ int s_off[kFiltPer * NW];
  const int qi = blockIdx.x / n_f;
  const int c = blockIdx.x - qi * n_f;
  const int64_t nv = n_visible(a.Q.pos[qi], a.m, a.N);
  const int64_t base = (int64_t)c * kFiltN;
  int* cnt = counts + (int64_t)qi * n_f + c;
  if (nv <= a.k || base >= nv) {   // no candidates here (rows of at most k entries: none read)
    if (threadIdx.x == 0) *cnt = 0;
    return;
  }
  const S* row = static_cast<const S*>(a.scores) + (int64_t)qi * a.ld_scores;
  uint32_t kv[kFiltPer];
#pragma unroll
  for (int u = 0; u < kFiltPer; ++u) {
    const int64_t j = base + (int64_t)u * kSNT + threadIdx.x;
    kv[u] = j < nv ? score_key(score_at(row, j)) : 0u;
  }
  const uint32_t T = thr[qi];
  const int lane = threadIdx.x & (kWave - 1), v = threadIdx.x / kWave;
  uint64_t m[kFiltPer];
#pragma unroll
  for (int u = 0; u < kFiltPer; ++u) {
    m[u] = __ballot(kv[u] >= T);
    if (lane == 0) s_off[u * NW + v] = __popcll(m[u]);
  }
  lds_sync();
  // Exclusive prefix of the (u, wave) counts in position order, by wave 0 (two per lane).
  if (v == 0) {
    const int a0 = s_off[2 * lane], a1 = s_off[2 * lane + 1];
    const int inc = wave_incl_sum(a0 + a1);
    s_off[2 * lane] = inc - a0 - a1;
    s_off[2 * lane + 1] = inc - a1;
    if (lane == kWave - 1) *cnt = inc;
  }
  lds_sync();
  uint2* dst = cand + ((int64_t)qi * n_f + c) * kCandCap;
#pragma unroll
  for (int u = 0; u < kFiltPer; ++u) {
    const int o = mbcnt(m[u], s_off[u * NW + v]);
    if (kv[u] >= T && o < kCandCap)
      dst[o] = make_uint2(kv[u], (uint32_t)(base + (int64_t)u * kSNT + threadIdx.x));
  }
}

// Exact top k of a whole row of n > k keys by one workgroup, kFiltN keys per pass: the same radix
// select as kth_key (digits of the block's highest differing bit downwards) with the histograms
// summed over passes, then an ordered compaction pass. The fallback of the sampled path.
template <typename S>
__device__ void select_row_passes(const S* row, int64_t n, int k, int32_t* out, int* hist,
                                  int* s_tmp) {
  constexpr int NT = kSNT;
  uint32_t mx = 0, mn = ~0u;
  for (int64_t b0 = 0; b0 < n; b0 += kFiltN) {
    uint32_t kv[kFiltPer];
    load_keys(row + b0, (int)(n - b0 < kFiltN ? n - b0 : kFiltN), kv);
    uint32_t bx, bn;
    block_range<NT>(kv, s_tmp, bx, bn);
    mx = max(mx, bx);
    mn = min(mn, bn);
  }
  uint32_t K = mx;
  int kk = k;
  if (mx != mn) {
    const int p = 31 - __builtin_clz(mx ^ mn);
    uint32_t pmask = p == 31 ? 0u : ~0u << (p + 1);
    uint32_t prefix = mx & pmask;
    int lo = p + 1;
    while (lo > 0) {
      const int hi = lo - 1;
      lo = hi >= 10 ? hi - 10 : 0;
      const uint32_t dmask = (2u << (hi - lo)) - 1u;
      clear_hist(hist, NT);
      lds_sync();
      for (int64_t b0 = 0; b0 < n; b0 += kFiltN) {
        uint32_t kv[kFiltPer];
        load_keys(row + b0, (int)(n - b0 < kFiltN ? n - b0 : kFiltN), kv);
#pragma unroll
        for (int i = 0; i < kFiltPer; ++i)
          if ((kv[i] & pmask) == prefix) atomicAdd(&hist[(kv[i] >> lo) & dmask], 1);
      }
      lds_sync();
      int count;
      const uint32_t d = find_digit<NT>(hist, kk, s_tmp, count);
      prefix |= d << lo;
      pmask |= dmask << lo;
    }
    K = prefix;
  }
  // kk keys equal to K belong to the top k, the first ones in row order.
  int written = 0, eq_left = kk;
  for (int64_t b0 = 0; b0 < n && written < k; b0 += kFiltN) {
    uint32_t kv[kFiltPer];
    load_keys(row + b0, (int)(n - b0 < kFiltN ? n - b0 : kFiltN), kv);
    int tot_gt, tot_eq;
    compact<NT>(kv, K, eq_left, k - written, s_tmp,
                [&](int o, int j, uint32_t) { out[written + o] = (int32_t)(b0 + j); }, &tot_gt,
                &tot_eq);
    const int taken = eq_left < tot_eq ? eq_left : tot_eq;
    written += tot_gt + taken;
    eq_left -= taken;
  }
}

template <typename S>
__global__ void __launch_bounds__(kSNT) topk_select_kernel(TopkArgs a, int n_f, const int* counts,
                                                           const uint2* cand) {
  constexpr int NT = kSNT;
  __shared__ int s_tmp[2 * NT / kWave + 2];
  __shared__ __attribute__((aligned(16))) int s_hist[2 * kBins];
  __shared__ uint32_t s_key[kSelCap];   // candidates in position order
  __shared__ int s_pos[kSelCap];
  __shared__ int s_start[kMaxFilt + 1];
  __shared__ int s_bad;
  const int qi = blockIdx.x;
  const int64_t nv = n_visible(a.Q.pos[qi], a.m, a.N);
  int32_t* out = a.idx + (int64_t)qi * a.k;
  if (nv <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += NT) out[i] = i < nv ? i : -1;
    return;
  }
  const S* row = static_cast<const S*>(a.scores) + (int64_t)qi * a.ld_scores;
  const int k = a.k;
  // Where each filter workgroup's list goes (wave 0: one list per lane, n_f <= 64).
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    const int cn = lane < n_f ? counts[(int64_t)qi * n_f + lane] : 0;
    const int inc = wave_incl_sum(cn);
    s_start[lane] = inc - cn;
    if (lane == kWave - 1) {
      s_start[kMaxFilt] = inc;
      s_bad = inc < k || inc > kSelCap;
    }
    if (cn > kCandCap) s_bad = 1;   // any lane: an overflowed list
  }
  lds_sync();
  const int C = s_start[kMaxFilt];
  if (s_bad) {
    select_row_passes(row, nv, k, out, s_hist, s_tmp);
    return;
  }
  // Gather the lists: list c by the kSNT / kMaxFilt threads 16 c .. 16 c + 15, all loads issued
  // before any store.
  {
    constexpr int kTpl = NT / kMaxFilt;                  // threads per list
    constexpr int kPerT = kCandCap / kTpl;               // candidates per thread at most
    const int c = threadIdx.x / kTpl, r = threadIdx.x % kTpl;
    const int st = c < n_f ? s_start[c] : 0;
    const int cn = c < n_f ? s_start[c + 1] - st : 0;
    const uint2* src = cand + ((int64_t)qi * n_f + (c < n_f ? c : 0)) * kCandCap;
    uint2 v[kPerT];
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
      const int j = r + kTpl * i;
      v[i] = j < cn ? src[j] : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int i = 0; i < kPerT; ++i) {
      const int j = r + kTpl * i;
      if (j < cn) {
        s_key[st + j] = v[i].x;
        s_pos[st + j] = (int)v[i].y;
      }
    }
  }
  lds_sync();
  uint32_t kv[kFiltPer];
#pragma unroll
  for (int u = 0; u < kFiltPer; ++u) {
    const int j = key_pos<kFiltPer>(u);
    kv[u] = j < C ? s_key[j] : 0u;
  }
  clear_hist(s_hist, NT);
  lds_sync();
  int need_eq;
  const uint32_t K = kth_key<NT, true>(kv, k, s_hist, s_tmp, &need_eq);
  compact<NT>(kv, K, need_eq, k, s_tmp, [&](int o, int j, uint32_t) { s_hist[o] = s_pos[j]; });
  for (int i = threadIdx.x; i < k; i += NT) out[i] = s_hist[i];
}

int n_chunks_for(int64_t N) { return (int)((N + kWideChunk - 1) / kWideChunk); }

}  // namespace

// The sampled path serves rows longer than kWideChunk when they occupy few filter workgroups (a
// latency-bound call) and k is small enough for the candidate list to fit one select workgroup
// with a wide margin: about 2 k + 16 N / kSamp candidates are expected. Rows of up to kWideChunk
// keep the single 1024-thread workgroup, which measured as fast as the three sampled-path
// launches at 32768 entries (24 against 25 us for 64 rows) and faster below.
bool use_sampled(int nq, int64_t N, int k) {
  const int64_t n_f = (N + kFiltN - 1) / kFiltN;
  const int64_t s = N < kSamp ? N : kSamp;
  return N > kWideChunk && n_f <= kMaxFilt && k <= kMaxK && (int64_t)nq * n_f <= 2048 &&
         2 * (int64_t)k + 16 * ((N + s - 1) / s) <= kSelCap / 2;
}

// Sampled-path workspace: thresholds [nq], list counts [nq][n_f], lists [nq][n_f][kCandCap].
size_t align256(size_t b) { return (b + 255) / 256 * 256; }
size_t sampled_counts_offset(int nq) { return align256((size_t)nq * sizeof(uint32_t)); }
size_t sampled_lists_offset(int nq, int n_f) {
  return sampled_counts_offset(nq) + align256((size_t)nq * n_f * sizeof(int));
}

size_t topk_workspace(int nq, int64_t N, int k) {
  if (use_sampled(nq, N, k)) {
    const int n_f = (int)((N + kFiltN - 1) / kFiltN);
    return sampled_lists_offset(nq, n_f) + (size_t)nq * n_f * kCandCap * sizeof(uint2);
  }
  if (N <= kWideChunk) return 0;
  const int nc = n_chunks_for(N);
  return (size_t)nq * nc * (size_t)k * (sizeof(uint32_t) + sizeof(int32_t));
}

bool topk_supported(int64_t N, int k) {
  return N <= kWideChunk || (k <= kMaxK && (int64_t)n_chunks_for(N) * k <= kCandMax);
}

namespace {

template <typename S>
hipError_t launch_topk_t(const TopkArgs& a, hipStream_t s) {
  if (a.N <= kChunk) {
    topk_row_kernel<256, S><<<a.Q.nq, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  if (use_sampled(a.Q.nq, a.N, a.k)) {
    const int n_f = (int)((a.N + kFiltN - 1) / kFiltN);
    char* ws = static_cast<char*>(a.ws);
    uint32_t* thr = reinterpret_cast<uint32_t*>(ws);
    int* counts = reinterpret_cast<int*>(ws + sampled_counts_offset(a.Q.nq));
    uint2* lists = reinterpret_cast<uint2*>(ws + sampled_lists_offset(a.Q.nq, n_f));
    topk_sample_kernel<S><<<a.Q.nq, kSNT, 0, s>>>(a, thr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    topk_filter_kernel<S><<<(unsigned)((int64_t)a.Q.nq * n_f), kSNT, 0, s>>>(a, n_f, thr, counts,
                                                                            lists);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    topk_select_kernel<S><<<a.Q.nq, kSNT, 0, s>>>(a, n_f, counts, lists);
    return hipGetLastError();
  }
  if (a.N <= kWideChunk) {
    topk_row_kernel<1024, S><<<a.Q.nq, 1024, 0, s>>>(a);
    return hipGetLastError();
  }
  const int nc = n_chunks_for(a.N);
  uint32_t* cand_key = static_cast<uint32_t*>(a.ws);
  int32_t* cand_idx = reinterpret_cast<int32_t*>(cand_key + (size_t)a.Q.nq * nc * a.k);
  topk_chunk_kernel<1024, S><<<(unsigned)((int64_t)a.Q.nq * nc), 1024, 0, s>>>(a, nc, cand_key,
                                                                              cand_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Stage 2 block size: kPer candidate keys per thread.
  const int64_t cand = (int64_t)nc * a.k;
  if (cand <= 256 * kPer) {
    topk_merge_kernel<256><<<a.Q.nq, 256, 0, s>>>(a, nc, cand_key, cand_idx);
  } else if (cand <= 512 * kPer) {
    topk_merge_kernel<512><<<a.Q.nq, 512, 0, s>>>(a, nc, cand_key, cand_idx);
  } else {
    topk_merge_kernel<1024><<<a.Q.nq, 1024, 0, s>>>(a, nc, cand_key, cand_idx);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.Q.nq == 0) return hipSuccess;
  return a.bf16 ? launch_topk_t<uint16_t>(a, s) : launch_topk_t<float>(a, s);
}

// ---- Scratch of the no-allocation top-k (csa_topk_noalloc) -------------------------------------
// A file-scope device array that every call on a GPU shares: each GPU the library runs on holds
// its own copy until the process ends. Host code never passes the array's name (a host-side
// stand-in) to a kernel: it takes the device address from hipGetSymbolAddress, once per device,
// with that device current, and passes that.
namespace {
__device__ __align__(256) unsigned char scratch[kTopkScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t topk_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace csa
