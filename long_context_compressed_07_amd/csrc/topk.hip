// csa_topk kernels: per-query selection of the k highest-scoring visible entries.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 and yudonglee.me "DeepSeek-V4 详解" 2.2
// Step 3 (only the top-k compressed rows by indexer score enter attention). Ties go to the lower
// index and the output lists indices in ascending order (this library's reading).
//
// Algorithm (integer work only, deterministic). Scores map to order-preserving 32-bit keys held in
// LDS. A most-significant-digit radix select with 11/11/10-bit digits (2048-bin LDS histograms,
// threshold bin found by a parallel suffix scan) yields the k-th largest key K and how many keys
// equal to K are still needed. Compaction keeps every key > K and the lowest-index keys == K: each
// thread owns a contiguous segment, two block scans give every segment its output offset, and
// indices are written in ascending order.
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

// Radix select over n keys in LDS: returns K (the k-th largest key) and, in *need_eq, how many
// keys equal to K belong to the top k. Requires n > k >= 1.
template <int NT>
__device__ uint32_t radix_select(const uint32_t* keys, int n, int k, int* s_hist, int* s_tmp,
                                 int* need_eq) {
  constexpr int kBins = 2048;
  constexpr int NW = NT / kWave;
  uint32_t prefix = 0, pmask = 0;
  int remaining = k;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3ffu : 0x7ffu;
    for (int i = threadIdx.x; i < kBins; i += NT) s_hist[i] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += NT) {
      const uint32_t key = keys[j];
      if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & dmask], 1);
    }
    __syncthreads();
    // Threshold bin: the highest bin whose suffix count (bins >= it) reaches `remaining`.
    // Thread t owns kPer bins counted down from 2047 - kPer t.
    constexpr int kPer = kBins / NT;
    int local = 0;
    const int top = kBins - 1 - kPer * threadIdx.x;
#pragma unroll
    for (int i = 0; i < kPer; ++i) local += s_hist[top - i];
    int total;
    const int before = block_scan<NT>(local, s_tmp, total);
    if (before < remaining && before + local >= remaining) {
      int cum = before, bin = top;
      for (int i = 0; i < kPer - 1; ++i, --bin) {
        const int c = s_hist[bin];
        if (cum + c >= remaining) break;
        cum += c;
      }
      s_tmp[NW] = bin;
      s_tmp[NW + 1] = remaining - cum;
    }
    __syncthreads();
    prefix |= (uint32_t)s_tmp[NW] << shift;
    pmask |= dmask << shift;
    remaining = s_tmp[NW + 1];
    __syncthreads();
  }
  *need_eq = remaining;
  return prefix;
}

// Writes, in ascending position order, index_of(j) for the positions j of the top k (keys > K and
// the first need_eq keys == K) into out[0..).
template <int NT, typename F>
__device__ void compact(const uint32_t* keys, int n, uint32_t K, int need_eq, int* s_tmp,
                        F index_of, int32_t* out) {
  const int seg = (n + NT - 1) / NT;
  const int j0 = threadIdx.x * seg < n ? threadIdx.x * seg : n;
  const int j1 = j0 + seg < n ? j0 + seg : n;
  int gt = 0, eq = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t key = keys[j];
    gt += key > K;
    eq += key == K;
  }
  int total;
  const int eq_before = block_scan<NT>(eq, s_tmp, total);
  int take_eq = need_eq - eq_before;
  take_eq = take_eq < 0 ? 0 : (take_eq > eq ? eq : take_eq);
  int off = block_scan<NT>(gt + take_eq, s_tmp, total);
  int eq_left = take_eq;
  for (int j = j0; j < j1; ++j) {
    const uint32_t key = keys[j];
    bool take = key > K;
    if (key == K && eq_left > 0) {
      take = true;
      --eq_left;
    }
    if (take) out[off++] = index_of(j);
  }
}

struct Identity {
  __device__ int32_t operator()(int j) const { return j; }
};

// Single stage: one workgroup per query row (n_vis <= kChunk).
template <int NT>
__global__ void __launch_bounds__(NT) topk_row_kernel(TopkArgs a) {
  __shared__ uint32_t s_keys[kChunk];
  __shared__ int s_hist[2048];
  __shared__ int s_tmp[NT / kWave + 2];
  const int qi = blockIdx.x;
  const int n = (int)n_visible(a.Q.pos[qi], a.m, a.N);
  int32_t* out = a.idx + (int64_t)qi * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += NT) out[i] = i < n ? i : -1;
    return;
  }
  const float* row = a.scores + (int64_t)qi * a.ld_scores;
  for (int j = threadIdx.x; j < n; j += NT) s_keys[j] = score_key(row[j]);
  __syncthreads();
  int need_eq;
  const uint32_t K = radix_select<NT>(s_keys, n, a.k, s_hist, s_tmp, &need_eq);
  compact<NT>(s_keys, n, K, need_eq, s_tmp, Identity{}, out);
}

// Stage 1: chunk c of query row qi; writes the chunk's local top-k (or all of its visible
// entries) as (key, index) pairs in ascending index order, and their count.
template <int NT>
__global__ void __launch_bounds__(NT) topk_chunk_kernel(TopkArgs a, int n_chunks,
                                                        uint32_t* cand_key, int32_t* cand_idx,
                                                        int* cand_cnt) {
  __shared__ uint32_t s_keys[kChunk];
  __shared__ int s_hist[2048];
  __shared__ int s_tmp[NT / kWave + 2];
  const int qi = blockIdx.x / n_chunks;
  const int c = blockIdx.x - qi * n_chunks;
  const int64_t nv = n_visible(a.Q.pos[qi], a.m, a.N);
  const int64_t base = (int64_t)c * kChunk;
  const int64_t slot = (int64_t)qi * n_chunks + c;
  int32_t* oi = cand_idx + slot * a.k;
  uint32_t* ok = cand_key + slot * a.k;
  const int n = base >= nv ? 0 : (int)(nv - base < kChunk ? nv - base : kChunk);
  const float* row = a.scores + (int64_t)qi * a.ld_scores + base;
  for (int j = threadIdx.x; j < n; j += NT) s_keys[j] = score_key(row[j]);
  __syncthreads();
  if (n <= a.k) {
    for (int j = threadIdx.x; j < n; j += NT) {
      oi[j] = (int32_t)(base + j);
      ok[j] = s_keys[j];
    }
    if (threadIdx.x == 0) cand_cnt[slot] = n;
    return;
  }
  int need_eq;
  const uint32_t K = radix_select<NT>(s_keys, n, a.k, s_hist, s_tmp, &need_eq);
  // The histogram is free now: it receives the selected chunk positions (k <= 2048).
  compact<NT>(s_keys, n, K, need_eq, s_tmp, Identity{}, s_hist);
  __syncthreads();
  for (int i = threadIdx.x; i < a.k; i += NT) {
    const int j = s_hist[i];
    ok[i] = s_keys[j];
    oi[i] = (int32_t)(base + j);
  }
  if (threadIdx.x == 0) cand_cnt[slot] = a.k;
}

// Maps a position of the concatenated candidate list to its entry index.
struct CandIndex {
  const int* off;        // LDS: start of each chunk's candidates, n_chunks + 1 values
  int n_chunks;
  int k;
  const int32_t* idx;    // this row's candidate indices, [n_chunks][k]
  __device__ int32_t operator()(int j) const {
    int c = 0;
    while (c + 1 < n_chunks && off[c + 1] <= j) ++c;
    return idx[(int64_t)c * k + (j - off[c])];
  }
};

// Stage 2: the row's top-k among its chunks' candidates (concatenated in chunk order, so positions
// ascend with entry index).
template <int NT>
__global__ void __launch_bounds__(NT) topk_merge_kernel(TopkArgs a, int n_chunks,
                                                        const uint32_t* cand_key,
                                                        const int32_t* cand_idx,
                                                        const int* cand_cnt) {
  extern __shared__ uint32_t s_cand[];          // up to kCandMax keys
  __shared__ int s_hist[2048];
  __shared__ int s_tmp[NT / kWave + 2];
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
  for (int c = 0; c < n_chunks; ++c) {
    const int cnt = s_off[c + 1] - s_off[c];
    const uint32_t* src = cand_key + ((int64_t)qi * n_chunks + c) * a.k;
    for (int i = threadIdx.x; i < cnt; i += NT) s_cand[s_off[c] + i] = src[i];
  }
  __syncthreads();
  if (n <= a.k) {   // no more visible entries than k: every candidate, in order
    for (int c = 0; c < n_chunks; ++c) {
      const int cnt = s_off[c + 1] - s_off[c];
      for (int i = threadIdx.x; i < cnt; i += NT) out[s_off[c] + i] = cidx[(int64_t)c * a.k + i];
    }
    for (int i = n + threadIdx.x; i < a.k; i += NT) out[i] = -1;
    return;
  }
  int need_eq;
  const uint32_t K = radix_select<NT>(s_cand, n, a.k, s_hist, s_tmp, &need_eq);
  compact<NT>(s_cand, n, K, need_eq, s_tmp, CandIndex{s_off, n_chunks, a.k, cidx}, out);
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
  const size_t lds = (size_t)nc * a.k * sizeof(uint32_t);
  if (lds > 64 * 1024) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_merge_kernel<1024>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  topk_merge_kernel<1024><<<a.Q.nq, 1024, lds, s>>>(a, nc, cand_key, cand_idx, cand_cnt);
  return hipGetLastError();
}

}  // namespace csa
