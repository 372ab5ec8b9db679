// csa_cache_append: decode-time maintenance of the compressed caches, one new token per sequence.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 (CSA step one: m adjacent tokens pooled
// into one row with softmax weights that carry a position bias; HCA the same with m' = 128) and
// yudonglee.me "DeepSeek-V4 详解" 2.2 Step 1 / 2.3 Step 1; jaylab-temp.pages.dev "DeepSeek-V4 —
// 百万 Token 上下文的高效 MoE 模型" 其他技术细节 (cache rows: fp8 latent, bf16 RoPE dims). Reading: the
// tokens of the block being filled wait in a caller-owned fp32 staging ring; the token that
// completes a block turns it into that block's entry, pooled (pool.h: the arithmetic and order of
// csa_compress, so the entry is bitwise the one csa_compress would build) and stored by the same
// rules; the raw row of the token goes to the raw store, a ring addressed (p - pos0) mod rows, in
// the same row format. Indexer keys (hongke120.com/20112.html 4.1 lists them as their own cache)
// are maintained by a second call with d_r = 0, no raw store, and an e4m3 key store.
//
// One workgroup per sequence; thread t owns channels t, t + 256, ... of the row, so the pooled
// value of a channel needs only that thread's registers and the staged rows of earlier calls.
// The row maxima for the fp8 scales are reduced through LDS.
#include "append.h"
#include "attend_keys.h"
#include "pool.h"

namespace csa {
namespace {

constexpr int kAppThreads = 256;
constexpr int kAppMaxCh = 4;   // channels per thread: d <= 1024

template <typename TIn>
__device__ __forceinline__ float load_in(const void* p, int64_t off);
template <>
__device__ __forceinline__ float load_in<float>(const void* p, int64_t off) {
  return static_cast<const float*>(p)[off];
}
template <>
__device__ __forceinline__ float load_in<uint16_t>(const void* p, int64_t off) {
  return bf16_to_f32(static_cast<const uint16_t*>(p)[off]);
}

// Stores channel c of a row: latent as f32 / bf16 / e4m3 (value / sigma), RoPE as f32 for an f32
// store and bf16 otherwise (the csa_compress store rules).
__device__ __forceinline__ void store_value(const OutStore& o, int64_t row, int c, float v,
                                            float sigma) {
  if (c >= o.d_c) {
    const int rc = c - o.d_c;
    if (o.dtype == CSA_F32)
      static_cast<float*>(o.r)[row * o.ld_r + rc] = v;
    else
      static_cast<uint16_t*>(o.r)[row * o.ld_r + rc] = f32_to_bf16(v);
  } else if (o.dtype == CSA_F32) {
    static_cast<float*>(o.c)[row * o.ld_c + c] = v;
  } else if (o.dtype == CSA_BF16) {
    static_cast<uint16_t*>(o.c)[row * o.ld_c + c] = f32_to_bf16(v);
  } else {
    static_cast<uint8_t*>(o.c)[row * o.ld_c + c] = e4m3_code(v, sigma);
  }
}

template <typename TIn>
__global__ void __launch_bounds__(kAppThreads) append_kernel(AppendArgs a) {
  __shared__ uint32_t s_amax[2];   // |latent| maxima: raw row, entry row (non-negative floats)
  const int b = blockIdx.x, t = threadIdx.x;
  const int d = a.d_c + a.d_r;
  const int64_t p = a.pos[b];
  const int slot = (int)(p % a.m);
  const bool close = (p + 1) % a.m == 0;
  const bool raw_ok = a.raw.c != nullptr && a.raw.rows > 0;
  const int64_t rrow = raw_ok ? ring_row(p, a.raw_pos0 != nullptr ? a.raw_pos0[b] : 0, a.raw.rows)
                              : 0;
  const int64_t erow = (p + 1) / a.m - 1;
  const bool ent_ok = close && erow >= 0 && erow < a.ent.rows;
  if (t < 2) s_amax[t] = 0u;
  __syncthreads();
  // Phase 1: every load of the token rows first (the staging ring may alias nothing the
  // compiler can prove, so loads are kept ahead of all stores).
  float xv[kAppMaxCh], gv[kAppMaxCh], ev[kAppMaxCh];
#pragma unroll
  for (int u = 0; u < kAppMaxCh; ++u) {
    const int c = t + u * kAppThreads;
    const int cc = c < d ? c : d - 1;
    xv[u] = load_in<TIn>(a.x_new, (int64_t)b * d + cc);
    gv[u] = load_in<TIn>(a.g_new, (int64_t)b * d + cc);
    ev[u] = 0.f;
  }
  float* sx = a.stage_x + (int64_t)b * a.m * d;
  float* sg = a.stage_g + (int64_t)b * a.m * d;
  float am_x = 0.f, am_e = 0.f;
#pragma unroll
  for (int u = 0; u < kAppMaxCh; ++u)
    if (t + u * kAppThreads < a.d_c) am_x = fmaxf(am_x, fabsf(xv[u]));
  if (ent_ok) {
    // Phase 2: the block's pooling in the shared order (chunks of 4 positions); the new token's
    // row comes from registers, the earlier ones from the staging ring.
#pragma unroll
    for (int u = 0; u < kAppMaxCh; ++u) {
      const int c = t + u * kAppThreads;
      const int cc = c < d ? c : d - 1;
      PoolAcc pa = pool_start();
      for (int i0 = 0; i0 < a.m; i0 += 4) {
        const int cnt = a.m - i0 < 4 ? a.m - i0 : 4;
        float ai[4], xi[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int i = i0 + (q < cnt ? q : 0);
          const bool mine = i == slot;
          ai[q] = (mine ? gv[u] : sg[(int64_t)i * d + cc]) + a.bias[i];
          xi[q] = mine ? xv[u] : sx[(int64_t)i * d + cc];
        }
        pool_fold(pa, ai, xi, cnt);
      }
      ev[u] = pool_value(pa);
      if (c < a.d_c) am_e = fmaxf(am_e, fabsf(ev[u]));
    }
  }
  // Phase 3: the stores.
#pragma unroll
  for (int u = 0; u < kAppMaxCh; ++u) {
    const int c = t + u * kAppThreads;
    if (c >= d) continue;
    sx[(int64_t)slot * d + c] = xv[u];
    sg[(int64_t)slot * d + c] = gv[u];
  }
  atomicMax(&s_amax[0], __float_as_uint(am_x));
  atomicMax(&s_amax[1], __float_as_uint(am_e));
  __syncthreads();
  const float sig_x = e4m3_row_scale(__uint_as_float(s_amax[0]));
  const float sig_e = e4m3_row_scale(__uint_as_float(s_amax[1]));
  const int64_t rg = (int64_t)b * a.raw.rows + rrow;
  const int64_t eg = (int64_t)b * a.ent.rows + erow;
  if (t == 0 && raw_ok && a.raw.dtype == CSA_E4M3) a.raw.scale[rg] = sig_x;
  if (t == 0 && ent_ok && a.ent.dtype == CSA_E4M3) a.ent.scale[eg] = sig_e;
#pragma unroll
  for (int u = 0; u < kAppMaxCh; ++u) {
    const int c = t + u * kAppThreads;
    if (c >= d) continue;
    if (raw_ok) store_value(a.raw, rg, c, xv[u], sig_x);
    if (ent_ok) store_value(a.ent, eg, c, ev[u], sig_e);
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  if (a.in_dtype == CSA_F32)
    append_kernel<float><<<a.B, kAppThreads, 0, s>>>(a);
  else
    append_kernel<uint16_t><<<a.B, kAppThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace csa
