// csa_topk kernels: per-query selection of the k highest-scoring visible entries.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 and yudonglee.me "DeepSeek-V4 详解" 2.2
// Step 3 (only the top-k compressed rows by indexer score enter attention). Ties go to the lower
// index and the output lists indices in ascending order (this library's reading).
//
// Algorithm (integer work only, deterministic): scores map to order-preserving 32-bit keys; a
// most-significant-digit radix select (4 passes of 8 bits, LDS histograms) finds the k-th largest
// key K and how many entries equal to K are still needed; a final in-order pass keeps every key
// > K and the lowest-index keys == K, compacted with wavefront ballots and a block scan.
#include <atomic>

#include "common.h"

namespace csa {
namespace {

constexpr int kTopkThreads = 256;

// Order-preserving map float -> uint32 (larger float -> larger key); -0.0 and +0.0 map alike.
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix count of `flag` over the block (in thread order) and the block total.
__device__ __forceinline__ int block_excl_scan(bool flag, int* s_wave, int& total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wv = threadIdx.x / kWave;
  const unsigned long long bal = __ballot(flag);
  const int in_wave = __popcll(bal & ((1ull << lane) - 1ull));
  if (lane == 0) s_wave[wv] = __popcll(bal);
  __syncthreads();
  int before = 0;
  total = 0;
  for (int w = 0; w < kTopkThreads / kWave; ++w) {
    const int c = s_wave[w];
    before += w < wv ? c : 0;
    total += c;
  }
  __syncthreads();
  return before + in_wave;
}

// One workgroup per query row. When the row fits (cache_cap keys), its keys are copied once into
// dynamic LDS and every pass reads LDS; otherwise the passes re-read the scores.
__global__ void __launch_bounds__(kTopkThreads) topk_block_kernel(TopkArgs a, int cache_cap) {
  extern __shared__ uint32_t s_keys[];
  __shared__ int s_hist[256];
  __shared__ int s_wave[kTopkThreads / kWave];
  __shared__ int s_sel[2];
  const int qi = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t nv = n_visible(a.Q.pos[qi], a.m, a.N);
  int32_t* out = a.idx + (int64_t)qi * a.k;
  const float* row = a.scores + (int64_t)qi * a.ld_scores;
  if (nv <= a.k) {
    for (int i = tid; i < a.k; i += kTopkThreads) out[i] = i < nv ? i : -1;
    return;
  }
  const bool cached = nv <= cache_cap;
  if (cached) {
    for (int64_t j = tid; j < nv; j += kTopkThreads) s_keys[j] = score_key(row[j]);
  }
  auto key_at = [&](int64_t j) -> uint32_t { return cached ? s_keys[j] : score_key(row[j]); };
  uint32_t prefix = 0, pmask = 0;
  int remaining = a.k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kTopkThreads) s_hist[i] = 0;
    __syncthreads();
    for (int64_t j = tid; j < nv; j += kTopkThreads) {
      const uint32_t key = key_at(j);
      if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, bin = 255;
      for (; bin > 0; --bin) {
        if (cum + s_hist[bin] >= remaining) break;
        cum += s_hist[bin];
      }
      s_sel[0] = bin;
      s_sel[1] = remaining - cum;
    }
    __syncthreads();
    prefix |= (uint32_t)s_sel[0] << shift;
    pmask |= 255u << shift;
    remaining = s_sel[1];
    __syncthreads();
  }
  // prefix is the k-th largest key; `remaining` entries equal to it are taken (lowest first).
  int emitted = 0, eq_seen = 0;
  for (int64_t c0 = 0; c0 < nv; c0 += kTopkThreads) {
    const int64_t j = c0 + tid;
    const uint32_t key = j < nv ? key_at(j) : 0u;
    const bool gt = j < nv && key > prefix;
    const bool eq = j < nv && key == prefix;
    int eq_total, take_total;
    const int eq_rank = block_excl_scan(eq, s_wave, eq_total);
    const bool take = gt || (eq && eq_seen + eq_rank < remaining);
    const int slot = block_excl_scan(take, s_wave, take_total);
    if (take) out[emitted + slot] = (int32_t)j;
    emitted += take_total;
    eq_seen += eq_total;
  }
  for (int i = emitted + tid; i < a.k; i += kTopkThreads) out[i] = -1;
}

}  // namespace

size_t topk_workspace(int /*nq*/, int64_t /*N*/, int /*k*/) { return 0; }

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.Q.nq == 0) return hipSuccess;
  constexpr int kMaxCache = 32768;                 // keys (128 KiB of LDS)
  // Dynamic LDS above 64 KiB needs a per-device opt-in; remember it per device (thread-safe).
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&topk_block_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            kMaxCache * (int)sizeof(uint32_t));
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit, std::memory_order_release);
  }
  const int cap = a.N < kMaxCache ? (int)a.N : kMaxCache;
  topk_block_kernel<<<a.Q.nq, kTopkThreads, (size_t)cap * sizeof(uint32_t), s>>>(a, cap);
  return hipGetLastError();
}

}  // namespace csa
