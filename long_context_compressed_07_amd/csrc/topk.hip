// csa_topk kernels: per-query selection of the k highest-scoring visible entries.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 and yudonglee.me "DeepSeek-V4 详解" 2.2
// Step 3 (only the top-k compressed rows by indexer score enter attention). Ties go to the lower
// index and the output lists indices in ascending order (this library's reading).
//
// Algorithm (deterministic: the result depends only on the keys' order). Scores map to order-preserving 32-bit keys. Each
// thread holds a contiguous segment of PER keys in registers. Single-stage rows first look for the
// k-th largest key K in equal-width score bins (kth_key_by_value: one histogram, then a direct
// ranking of the few keys in K's bin). Otherwise, and when that bin is crowded, K is found by a
// radix select: the block's largest and smallest keys fix the bits every key shares; then, from
// the highest differing bit down, each level counts in an LDS histogram the next digit (at most 11
// bits) of the keys that match the digits found so far, and a block scan over the histogram
// locates the digit of the k-th key and its rank among the keys of that digit. Starting at the
// highest differing bit spreads clustered keys over the histogram, which keeps LDS atomic
// conflicts low. Compaction keeps every key > K and the lowest-position keys == K: two block scans
// give every segment its output offset; selected positions are staged in LDS and written out with
// coalesced stores.
//
// Rows of up to kChunk visible entries: one workgroup per row. Longer rows: stage 1 runs the same
// selection on chunks of kChunk entries (many workgroups per row) and writes each chunk's local
// top-k (ascending); stage 2 selects the row's top-k among the concatenated candidates. The union
// of the chunks' top-k contains the row's top-k under the same tie rule, so the result is exact.
// Every chunk before a row's last visible one holds kChunk >= k entries and so yields exactly k
// candidates: a row's candidates are the first n slots of its [chunks][k] block, in entry order.
#include "common.h"

namespace csa {
namespace {

constexpr int kChunk = 8192;      // entries per stage-1 chunk (and single-stage limit)
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
template <int NT>
__device__ __forceinline__ void block_range(const uint32_t (&kv)[kPer], int* s_tmp,
                                            uint32_t& mx, uint32_t& mn) {
  constexpr int NW = NT / kWave;
  uint32_t a = 0, b = ~0u;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
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
template <int NT>
__device__ bool kth_key_by_value(const uint32_t (&kv)[kPer], int k, float f0, float scale,
                                 int* hist, int* s_tmp, uint32_t* kth, int* need_eq) {
  auto bin = [&](uint32_t key) {
    const int b = (int)((key_score(key) - f0) * scale);   // >= 0: key_score(key) >= f0
    return b < kBins - 1 ? b : kBins - 1;
  };
#pragma unroll
  for (int i = 0; i < kPer; ++i)
    if (kv[i] != 0u) atomicAdd(&hist[bin(kv[i])], 1);
  lds_sync();
  int kk = k, count;
  const int d = (int)find_digit<NT>(hist, kk, s_tmp, count);
  if (count > NT) {   // hist zero again for the radix passes
    for (int i = threadIdx.x; i < kBins / 4; i += NT) reinterpret_cast<int4*>(hist)[i] = int4{0, 0, 0, 0};
    lds_sync();
    return false;
  }
  // The keys of bin d, in position order, into the second histogram's space.
  uint32_t* s_cand = reinterpret_cast<uint32_t*>(hist + kBins);
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) mine += kv[i] != 0u && bin(kv[i]) == d;
  int total;
  int off = block_scan<NT>(mine, s_tmp, total);
  if (mine > 0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i)
      if (kv[i] != 0u && bin(kv[i]) == d) s_cand[off++] = kv[i];
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
template <int NT, bool BY_VALUE>
__device__ uint32_t kth_key(const uint32_t (&kv)[kPer], int k, int* hist, int* s_tmp,
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
      if (kth_key_by_value<NT>(kv, k, f0, scale, hist, s_tmp, &K, need_eq)) return K;
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
    for (int i = 0; i < kPer; ++i) {
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

// Calls put(o, j, key) for the top k in ascending position order o = 0 .. k-1 (j = PER t + i for
// key kv[i] of thread t): keys > K and the first need_eq keys == K. Ends with an LDS barrier.
template <int NT, typename Put>
__device__ void compact(const uint32_t (&kv)[kPer], uint32_t K, int need_eq, int k, int* s_tmp,
                        Put put) {
  // Padding keys (0) are below every real key, and K is a real key (>= 1), so they never count.
  const int j0 = threadIdx.x * kPer;
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    gt += kv[i] > K;
    eq += kv[i] == K;
  }
  int total;
  const int eq_before = block_scan<NT>(eq, s_tmp, total);
  int take_eq = need_eq - eq_before;
  take_eq = take_eq < 0 ? 0 : (take_eq > eq ? eq : take_eq);
  int off = block_scan<NT>(gt + take_eq, s_tmp, total);
  int eq_left = take_eq;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    bool take = kv[i] > K;
    if (kv[i] == K && eq_left > 0) {
      take = true;
      --eq_left;
    }
    if (take && (unsigned)off < (unsigned)k) put(off, j0 + i, kv[i]);
    off += take;
  }
  lds_sync();
}

// Loads keys [PER t, PER t + PER) of a row of n scores (0 beyond n): 16-byte loads for whole,
// aligned segments, element by element only for the segment holding the row's end.
__device__ __forceinline__ void load_keys(const float* row, int n, uint32_t (&kv)[kPer]) {
  const int j0 = threadIdx.x * kPer;
  const float* src = row + j0;
  if (j0 + kPer <= n && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const float4 v = reinterpret_cast<const float4*>(src)[q];
      kv[4 * q] = score_key(v.x);
      kv[4 * q + 1] = score_key(v.y);
      kv[4 * q + 2] = score_key(v.z);
      kv[4 * q + 3] = score_key(v.w);
    }
  } else {
    const int m = n - j0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) kv[i] = i < m ? score_key(src[i]) : 0u;
  }
}

// The same for keys already mapped (stage-2 candidates).
__device__ __forceinline__ void load_mapped(const uint32_t* keys, int n, uint32_t (&kv)[kPer]) {
  const int j0 = threadIdx.x * kPer;
  const uint32_t* src = keys + j0;
  if (j0 + kPer <= n && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const uint4 v = reinterpret_cast<const uint4*>(src)[q];
      kv[4 * q] = v.x;
      kv[4 * q + 1] = v.y;
      kv[4 * q + 2] = v.z;
      kv[4 * q + 3] = v.w;
    }
  } else {
    const int m = n - j0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) kv[i] = i < m ? src[i] : 0u;
  }
}

// Single stage: one workgroup per query row (n_vis <= kChunk = NT * kPer). Six waves per SIMD (at
// most 80 VGPRs, no spills): 370 -> 336 us for 32768 rows of up to 8192 scores against five.
template <int NT>
__global__ void __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(6, 6)))
topk_row_kernel(TopkArgs a) {
  static_assert(NT * kPer == kChunk, "one key segment per thread");
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
  load_keys(a.scores + (int64_t)qi * a.ld_scores, n, kv);
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
template <int NT>
__global__ void __launch_bounds__(NT) topk_chunk_kernel(TopkArgs a, int n_chunks,
                                                        uint32_t* cand_key, int32_t* cand_idx) {
  static_assert(NT * kPer == kChunk, "one key segment per thread");
  __shared__ int s_tmp[2 * NT / kWave + 2];
  __shared__ __attribute__((aligned(16))) int s_hist[2 * kBins];
  const int qi = blockIdx.x / n_chunks;
  const int c = blockIdx.x - qi * n_chunks;
  const int64_t nv = n_visible(a.Q.pos[qi], a.m, a.N);
  const int64_t base = (int64_t)c * kChunk;
  const int64_t slot = (int64_t)qi * n_chunks + c;
  int32_t* oi = cand_idx + slot * a.k;
  uint32_t* ok = cand_key + slot * a.k;
  const int n = base >= nv ? 0 : (int)(nv - base < kChunk ? nv - base : kChunk);
  const float* row = a.scores + (int64_t)qi * a.ld_scores + base;
  if (n <= a.k) {
    for (int j = threadIdx.x; j < n; j += NT) {
      oi[j] = (int32_t)(base + j);
      ok[j] = score_key(row[j]);
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
    const int64_t last = (nv - 1) / kChunk;
    const int64_t in_last = nv - last * kChunk;
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
  const uint32_t K = kth_key<NT, false>(kv, a.k, s_hist, s_tmp, &need_eq);
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

int n_chunks_for(int64_t N) { return (int)((N + kChunk - 1) / kChunk); }

}  // namespace

size_t topk_workspace(int nq, int64_t N, int k) {
  if (N <= kChunk) return 0;
  const int nc = n_chunks_for(N);
  return (size_t)nq * nc * (size_t)k * (sizeof(uint32_t) + sizeof(int32_t));
}

bool topk_supported(int64_t N, int k) {
  return N <= kChunk || (k <= kMaxK && (int64_t)n_chunks_for(N) * k <= kCandMax);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.Q.nq == 0) return hipSuccess;
  if (a.N <= kChunk) {
    topk_row_kernel<256><<<a.Q.nq, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  const int nc = n_chunks_for(a.N);
  uint32_t* cand_key = static_cast<uint32_t*>(a.ws);
  int32_t* cand_idx = reinterpret_cast<int32_t*>(cand_key + (size_t)a.Q.nq * nc * a.k);
  topk_chunk_kernel<256><<<(unsigned)((int64_t)a.Q.nq * nc), 256, 0, s>>>(a, nc, cand_key,
                                                                         cand_idx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Stage 2 block size: kPer candidate keys per thread.
  const int64_t cand = (int64_t)nc * a.k;
  if (cand <= 128 * kPer) {
    topk_merge_kernel<128><<<a.Q.nq, 128, 0, s>>>(a, nc, cand_key, cand_idx);
  } else if (cand <= 256 * kPer) {
    topk_merge_kernel<256><<<a.Q.nq, 256, 0, s>>>(a, nc, cand_key, cand_idx);
  } else if (cand <= 512 * kPer) {
    topk_merge_kernel<512><<<a.Q.nq, 512, 0, s>>>(a, nc, cand_key, cand_idx);
  } else {
    topk_merge_kernel<1024><<<a.Q.nq, 1024, 0, s>>>(a, nc, cand_key, cand_idx);
  }
  return hipGetLastError();
}

}  // namespace csa
