// csa_topk kernels: per-query selection of the k highest-scoring visible entries.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 and yudonglee.me "DeepSeek-V4 详解" 2.2
// Step 3 (only the top-k compressed rows by indexer score enter attention). Ties go to the lower
// index and the output lists indices in ascending order (this library's reading).
//
// Algorithm (integer work only, deterministic). Scores map to order-preserving 32-bit keys. Each
// thread holds a contiguous segment of PER keys in registers. The k-th largest key K is found by a
// three-level radix select over 11-, 11- and 10-bit digits: each level counts, in an LDS histogram,
// the next digit of the keys that share the digits found so far, and a block scan over the
// histogram locates the digit of the k-th key and its rank within that digit.
// Compaction keeps every key > K and the lowest-index keys == K: two block scans give every
// segment its output offset, and indices are written in ascending order.
//
// Rows of up to kChunk visible entries: one workgroup per row. Longer rows: stage 1 runs the same
// selection on chunks of kChunk entries (many workgroups per row) and writes each chunk's local
// top-k (ascending); stage 2 selects the row's top-k among the concatenated candidates. The union
// of the chunks' top-k contains the row's top-k under the same tie rule, so the result is exact.
#include "common.h"

namespace csa {
namespace {

constexpr int kChunk = 8192;      // entries per stage-1 chunk (and single-stage limit)
constexpr int kCandMax = 32768;   // candidates per row in stage 2

// Order-preserving map float -> uint32 (larger float -> larger key); -0.0 and +0.0 map alike.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum (in thread order) of a per-thread count over the block, and the total.
template <int NT>
__device__ __forceinline__ int block_scan(int a, int* s_tmp, int& total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  int ia = a;   // inclusive wave scan
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int x = __shfl_up(ia, o);
    if (lane >= o) ia += x;
  }
  if (lane == kWave - 1) s_tmp[wv] = ia;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int c = s_tmp[w];
    if (w < wv) before += c;
    total += c;
  }
  __syncthreads();
  return before + ia - a;
}

// Radix digits of the k-th key search: bits [31:21], [20:10] and [9:0] of a key.
constexpr int kHistBins = 2048;   // LDS ints per histogram; two histograms per workgroup

// Given a histogram of NB digit values, finds the digit d holding the kk-th largest key (digits
// above d hold fewer than kk keys, digits >= d at least kk) and turns kk into the rank of that key
// among the keys of digit d. Every thread returns the same d and kk.
template <int NT, int NB>
__device__ __forceinline__ uint32_t find_digit(const int* hist, int& kk, int* s_tmp) {
  static_assert(NB % NT == 0, "bins per thread");
  constexpr int B = NB / NT;
  int* s_res = s_tmp + NT / kWave;
  const int t = threadIdx.x;
  int h[B];
  int local = 0;
#pragma unroll
  for (int b = 0; b < B; ++b) {
    h[b] = hist[t * B + b];
    local += h[b];
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
      }
      acc += h[b];
    }
  }
  __syncthreads();
  kk = s_res[1];
  return (uint32_t)s_res[0];
}

// The k-th largest of the block's keys (1 <= k <= number of real keys; padding keys are 0, below
// every real key), and in *need_eq how many keys equal to it belong to the top k. Radix select from
// the top digit down: each level histograms (LDS atomics) the next digit of the keys that share the
// digits found so far, then locates the k-th key's digit. s_hist holds 2 kHistBins ints; s_tmp
// holds NT / 64 + 2 ints.
template <int NT, int PER>
__device__ uint32_t kth_key(const uint32_t (&kv)[PER], int k, int* s_hist, int* s_tmp,
                            int* need_eq) {
  int* hA = s_hist;
  int* hB = s_hist + kHistBins;
  for (int i = threadIdx.x; i < 2 * kHistBins; i += NT) s_hist[i] = 0;
  __syncthreads();
  int kk = k;
#pragma unroll
  for (int i = 0; i < PER; ++i) atomicAdd(&hA[kv[i] >> 21], 1);
  __syncthreads();
  const uint32_t d0 = find_digit<NT, 2048>(hA, kk, s_tmp);
  for (int i = threadIdx.x; i < 1024; i += NT) hA[i] = 0;   // level 2 reuses hA[0, 1024)
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if ((kv[i] >> 21) == d0) atomicAdd(&hB[(kv[i] >> 10) & 2047u], 1);
  }
  __syncthreads();
  const uint32_t hi = (d0 << 11) | find_digit<NT, 2048>(hB, kk, s_tmp);
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    if ((kv[i] >> 10) == hi) atomicAdd(&hA[kv[i] & 1023u], 1);
  }
  __syncthreads();
  const uint32_t K = (hi << 10) | find_digit<NT, 1024>(hA, kk, s_tmp);
  *need_eq = kk;
  return K;
}

// Writes, in ascending position order, index_of(j) for the positions j (j = PER t + i for key
// kv[i] of thread t) of the top k: keys > K and the first need_eq keys == K; with out_key, also
// the selected keys.
template <int NT, int PER, typename F>
__device__ void compact_regs(const uint32_t (&kv)[PER], uint32_t K, int need_eq,
                             int* s_tmp, F index_of, int32_t* out, uint32_t* out_key = nullptr) {
  // Padding keys (0) are below every real key, and K is a real key (>= 1), so they never count.
  const int j0 = threadIdx.x * PER;
  int gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
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
  for (int i = 0; i < PER; ++i) {
    bool take = kv[i] > K;
    if (kv[i] == K && eq_left > 0) {
      take = true;
      --eq_left;
    }
    if (take) {
      out[off] = index_of(j0 + i);
      if (out_key != nullptr) out_key[off] = kv[i];
      ++off;
    }
  }
}

// Loads keys [PER t, PER t + PER) of a row of n scores (0 beyond n): 16-byte loads for whole,
// aligned segments, element by element only for the segment holding the row's end.
template <int PER>
__device__ __forceinline__ void load_keys(const float* row, int n, uint32_t (&kv)[PER]) {
  const int j0 = threadIdx.x * PER;
  const float* src = row + j0;
  if (j0 + PER <= n && (reinterpret_cast<uintptr_t>(src) & 15) == 0) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const float4 v = reinterpret_cast<const float4*>(src)[q];
      kv[4 * q] = score_key(v.x);
      kv[4 * q + 1] = score_key(v.y);
      kv[4 * q + 2] = score_key(v.z);
      kv[4 * q + 3] = score_key(v.w);
    }
  } else {
    const int m = n - j0;
#pragma unroll
    for (int i = 0; i < PER; ++i) kv[i] = i < m ? score_key(src[i]) : 0u;
  }
}

// The same from keys already in LDS (n of them).
template <int PER>
__device__ __forceinline__ void load_keys_lds(const uint32_t* keys, int n, uint32_t (&kv)[PER]) {
  const int j0 = threadIdx.x * PER;
  if (j0 + PER <= n) {
#pragma unroll
    for (int q = 0; q < PER / 4; ++q) {
      const uint4 v = reinterpret_cast<const uint4*>(keys + j0)[q];
      kv[4 * q] = v.x;
      kv[4 * q + 1] = v.y;
      kv[4 * q + 2] = v.z;
      kv[4 * q + 3] = v.w;
    }
  } else {
    const int m = n - j0;
#pragma unroll
    for (int i = 0; i < PER; ++i) kv[i] = i < m ? keys[j0 + i] : 0u;
  }
}

struct Identity {
  __device__ int32_t operator()(int j) const { return j; }
};

struct Offset {
  int32_t base;
  __device__ int32_t operator()(int j) const { return base + j; }
};

// Single stage: one workgroup per query row (n_vis <= kChunk).
template <int NT>
__global__ void __launch_bounds__(NT) topk_row_kernel(TopkArgs a) {
  constexpr int PER = kChunk / NT;
  __shared__ int s_tmp[NT / kWave + 2];
  __shared__ int s_hist[2 * kHistBins];
  const int qi = blockIdx.x;
  const int n = (int)n_visible(a.Q.pos[qi], a.m, a.N);
  int32_t* out = a.idx + (int64_t)qi * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += NT) out[i] = i < n ? i : -1;
    return;
  }
  uint32_t kv[PER];
  load_keys<PER>(a.scores + (int64_t)qi * a.ld_scores, n, kv);
  int need_eq;
  const uint32_t K = kth_key<NT, PER>(kv, a.k, s_hist, s_tmp, &need_eq);
  compact_regs<NT, PER>(kv, K, need_eq, s_tmp, Identity{}, out);
}

// Stage 1: chunk c of query row qi; writes the chunk's local top-k (or all of its visible
// entries) as (key, index) pairs in ascending index order, and their count.
template <int NT>
__global__ void __launch_bounds__(NT) topk_chunk_kernel(TopkArgs a, int n_chunks,
                                                        uint32_t* cand_key, int32_t* cand_idx,
                                                        int* cand_cnt) {
  constexpr int PER = kChunk / NT;
  __shared__ int s_tmp[NT / kWave + 2];
  __shared__ int s_hist[2 * kHistBins];
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
    if (threadIdx.x == 0) cand_cnt[slot] = n;
    return;
  }
  uint32_t kv[PER];
  load_keys<PER>(row, n, kv);
  int need_eq;
  const uint32_t K = kth_key<NT, PER>(kv, a.k, s_hist, s_tmp, &need_eq);
  compact_regs<NT, PER>(kv, K, need_eq, s_tmp, Offset{(int32_t)base}, oi, ok);
  if (threadIdx.x == 0) cand_cnt[slot] = a.k;
}

// Maps a position of the concatenated candidate list to its entry index.
struct CandIndex {
  const int* off;        // LDS: start of each chunk's candidates, n_chunks + 1 values
  int n_chunks;
  int k;
  const int32_t* idx;    // this row's candidate indices, [n_chunks][k]
  __device__ int32_t operator()(int j) const {
    int lo = 0, hi = n_chunks - 1;   // last chunk c with off[c] <= j
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (off[mid] <= j) lo = mid; else hi = mid - 1;
    }
    return idx[(int64_t)lo * k + (j - off[lo])];
  }
};

// Stage 2: the row's top-k among its chunks' candidates (concatenated in chunk order, so positions
// ascend with entry index).
template <int NT>
__global__ void __launch_bounds__(NT) topk_merge_kernel(TopkArgs a, int n_chunks,
                                                        const uint32_t* cand_key,
                                                        const int32_t* cand_idx,
                                                        const int* cand_cnt) {
  constexpr int PER = 32;
  extern __shared__ __attribute__((aligned(16))) uint32_t s_cand[];   // up to kCandMax keys
  __shared__ int s_tmp[NT / kWave + 2];
  __shared__ int s_hist[2 * kHistBins];
  __shared__ int s_off[64 + 1];
  const int qi = blockIdx.x;
  int32_t* out = a.idx + (int64_t)qi * a.k;
  if (threadIdx.x == 0) {
    int o = 0;
    for (int c = 0; c < n_chunks; ++c) {
      s_off[c] = o;
      o += cand_cnt[(int64_t)qi * n_chunks + c];
    }
    s_off[n_chunks] = o;
  }
  __syncthreads();
  const int n = s_off[n_chunks];
  const int32_t* cidx = cand_idx + (int64_t)qi * n_chunks * a.k;
  if (n <= a.k) {   // no more visible entries than k: every candidate, in order
    for (int c = 0; c < n_chunks; ++c) {
      const int cnt = s_off[c + 1] - s_off[c];
      for (int i = threadIdx.x; i < cnt; i += NT) out[s_off[c] + i] = cidx[(int64_t)c * a.k + i];
    }
    for (int i = n + threadIdx.x; i < a.k; i += NT) out[i] = -1;
    return;
  }
  // Candidates -> LDS (coalesced; eight loads in flight per thread), then each thread takes its
  // segment into registers.
  const uint32_t* ckeys = cand_key + (int64_t)qi * n_chunks * a.k;
  for (int c0 = 0; c0 < n_chunks; c0 += 8) {
    for (int i = threadIdx.x; i < a.k; i += NT) {
      uint32_t v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u;
        v[u] = (c < n_chunks && i < s_off[c + 1] - s_off[c]) ? ckeys[(int64_t)c * a.k + i] : 0u;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int c = c0 + u;
        if (c < n_chunks && i < s_off[c + 1] - s_off[c]) s_cand[s_off[c] + i] = v[u];
      }
    }
  }
  __syncthreads();
  uint32_t kv[PER];
  load_keys_lds<PER>(s_cand, n, kv);
  int need_eq;
  const uint32_t K = kth_key<NT, PER>(kv, a.k, s_hist, s_tmp, &need_eq);
  // Selected positions -> LDS (the keys are in registers now; the scans inside compact_regs
  // order these writes after every thread's reads of s_cand), then their entry indices are
  // gathered eight at a time.
  int32_t* s_pos = reinterpret_cast<int32_t*>(s_cand);
  compact_regs<NT, PER>(kv, K, need_eq, s_tmp, Identity{}, s_pos);
  __syncthreads();
  const CandIndex ci{s_off, n_chunks, a.k, cidx};
  for (int i0 = 0; i0 < a.k; i0 += 8 * NT) {
    int32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * NT + (int)threadIdx.x;
      v[u] = i < a.k ? ci(s_pos[i]) : 0;
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
  return (size_t)nq * nc * ((size_t)k * (sizeof(uint32_t) + sizeof(int32_t)) + sizeof(int));
}

bool topk_supported(int64_t N, int k) {
  return N <= kChunk ||
         (k <= 2048 && n_chunks_for(N) <= 64 && (int64_t)n_chunks_for(N) * k <= kCandMax);
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
  int* cand_cnt = reinterpret_cast<int*>(cand_idx + (size_t)a.Q.nq * nc * a.k);
  topk_chunk_kernel<256><<<(unsigned)((int64_t)a.Q.nq * nc), 256, 0, s>>>(a, nc, cand_key,
                                                                         cand_idx, cand_cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // Stage 2 block size: 32 candidate keys per thread.
  const int64_t cand = (int64_t)nc * a.k;
  const size_t lds = (size_t)cand * sizeof(uint32_t);
  auto merge = [&](auto kern, int nt) -> hipError_t {
    if (lds > 64 * 1024) {
      hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (e2 != hipSuccess) return e2;
    }
    kern<<<a.Q.nq, nt, lds, s>>>(a, nc, cand_key, cand_idx, cand_cnt);
    return hipGetLastError();
  };
  if (cand <= 128 * 32) return merge(&topk_merge_kernel<128>, 128);
  if (cand <= 256 * 32) return merge(&topk_merge_kernel<256>, 256);
  if (cand <= 512 * 32) return merge(&topk_merge_kernel<512>, 512);
  return merge(&topk_merge_kernel<1024>, 1024);
}

}  // namespace csa
