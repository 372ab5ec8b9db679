// csa_compress kernels: softmax-gated pooling of m consecutive token rows into one entry.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 (CSA step one: m adjacent tokens' KV
// merged with position-biased softmax weights) and yudonglee.me "DeepSeek-V4 详解" 2.2 Step 1 /
// 2.3 Step 1 (m = 4 for CSA, m' = 128 for HCA). Per channel c of block j:
//   a_i = g[jm+i][c] + bias[i],  w = softmax_i(a),  e[j][c] = sum_i w_i x[jm+i][c].
//
// pool_kernel streams x and g once (HBM-bound): one thread owns VEC consecutive channels of one
// entry (16-byte loads, consecutive threads on consecutive channels of a row) and folds the m
// positions in chunks of 4 with a running max (pool.h, the order every pooling kernel shares).
// project_pool_kernel is the fp32 projection mode: x = hidden * w_x and g = hidden * w_g are
// formed tile by tile in LDS and pooled in registers, so x and g never reach HBM (only the raw x
// rows the sliding window needs are written).
#include "pool.h"

namespace csa {
namespace {

// Vector loads of token rows; the pooling reads each row once, so the loads are non-temporal.
template <typename TIn>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void load(const void* base, int64_t off, float* out) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 v = __builtin_nontemporal_load(
        reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + off));
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
};
template <>
struct Vec<uint16_t> {
  static constexpr int N = 8;
  __device__ static void load(const void* base, int64_t off, float* out) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + off));
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(w[i] << 16);
      out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// Writes VEC pooled values of channels [ch, ch + VEC) of entry row (b, j).
template <int VEC>
__device__ void store_entry(const OutStore& o, int64_t b, int64_t j, int ch, const float* e,
                            float sigma) {
  const int64_t row = b * o.rows + j;
  if (ch >= o.d_c) {  // RoPE part: bf16 (fp32 when the store is fp32)
    const int rc = ch - o.d_c;
    if (o.dtype == CSA_F32) {
      float* p = static_cast<float*>(o.r) + row * o.ld_r + rc;
#pragma unroll
      for (int v = 0; v < VEC; ++v) p[v] = e[v];
    } else {
      uint16_t* p = static_cast<uint16_t*>(o.r) + row * o.ld_r + rc;
#pragma unroll
      for (int v = 0; v < VEC; ++v) p[v] = f32_to_bf16(e[v]);
    }
    return;
  }
  if (o.dtype == CSA_F32) {
    float* p = static_cast<float*>(o.c) + row * o.ld_c + ch;
#pragma unroll
    for (int v = 0; v < VEC; ++v) p[v] = e[v];
  } else if (o.dtype == CSA_BF16) {
    uint16_t* p = static_cast<uint16_t*>(o.c) + row * o.ld_c + ch;
#pragma unroll
    for (int v = 0; v < VEC; ++v) p[v] = f32_to_bf16(e[v]);
  } else {
    uint8_t* p = static_cast<uint8_t*>(o.c) + row * o.ld_c + ch;
#pragma unroll
    for (int v = 0; v < VEC; ++v) p[v] = e4m3_code(e[v], sigma);
  }
}

template <typename TIn>
__global__ void __launch_bounds__(256) pool_kernel(CompressArgs a, int cpr, int rows_per_wg) {
  constexpr int VEC = Vec<TIn>::N;
  __shared__ uint32_t s_amax[256];
  const int tid = threadIdx.x;
  const int lr = tid / cpr;
  const int cv = tid - lr * cpr;
  const int64_t nb = a.T / a.m;
  const int64_t gr = (int64_t)blockIdx.x * rows_per_wg + lr;
  const bool active = lr < rows_per_wg && gr < (int64_t)a.B * nb;
  const int d = a.d_c + a.d_r;
  const int ch = cv * VEC;
  if (tid < rows_per_wg) s_amax[tid] = 0u;

  float acc[VEC];
  int64_t b = 0, j = 0;
  if (active) {
    b = gr / nb;
    j = gr - b * nb;
    PoolAcc pa[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) pa[v] = pool_start();
    const int64_t base = (b * a.T + j * a.m) * d + ch;
    for (int i0 = 0; i0 < a.m; i0 += 4) {
      float xv[4][VEC], av[4][VEC];
      const int cnt = a.m - i0 < 4 ? a.m - i0 : 4;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if (p < cnt) {
          Vec<TIn>::load(a.x, base + (int64_t)(i0 + p) * d, xv[p]);
          Vec<TIn>::load(a.g, base + (int64_t)(i0 + p) * d, av[p]);
          const float bi = a.bias[i0 + p];
#pragma unroll
          for (int v = 0; v < VEC; ++v) av[p][v] += bi;
        }
      }
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        const float ai[4] = {av[0][v], av[1][v], av[2][v], av[3][v]};
        const float xi[4] = {xv[0][v], xv[1][v], xv[2][v], xv[3][v]};
        pool_fold(pa[v], ai, xi, cnt);
      }
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = pool_value(pa[v]);
  }
  float sigma = 0.f;
  if (a.out.dtype == CSA_E4M3) {
    __syncthreads();
    if (active && ch < a.d_c) {
      float am = 0.f;
#pragma unroll
      for (int v = 0; v < VEC; ++v) am = fmaxf(am, fabsf(acc[v]));
      atomicMax(&s_amax[lr], __float_as_uint(am));
    }
    __syncthreads();
    if (active) {
      sigma = e4m3_row_scale(__uint_as_float(s_amax[lr]));
      if (cv == 0) a.out.scale[b * a.out.rows + j] = sigma;
    }
  }
  if (active) store_entry<VEC>(a.out, b, j, ch, acc, sigma);
}

// fp32 projection + pooling on fp32 MFMA. A workgroup of 4 waves takes 64 tokens x 32 channels:
// wave w forms the 32 x 32 tile of tokens 32 (w & 1) .. + 32 of x (w < 2) or g (w >= 2) with
// mfma_f32_32x32x2_f32 over the model dims, from 32-dim slices of hidden and weights staged in LDS
// (the next slice loaded during the current one). In the MFMA's output layout a lane holds one
// channel and tokens 8 q + 4 (lane >> 5) + (0..3), q < 4: every block of m in {1, 2, 4} tokens
// is lane-local. The g waves hand their tiles to the x waves through LDS; the x waves store the
// raw rows and pool.
__global__ void __launch_bounds__(256) project_pool_kernel(CompressArgs a) {
  typedef float floatx16 __attribute__((ext_vector_type(16)));
  constexpr int TK = 32;
  constexpr int TC = 32;
  __shared__ float sh[64][TK + 1];
  __shared__ float sw[2][TK][TC];        // w_x, w_g slices
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63;
  const int64_t b = blockIdx.z;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * TC;
  const int d = a.d_c + a.d_r;
  const int dm = a.d_model;
  const int tg = w & 1, mat = w >> 1;    // token group, matrix (0: x, 1: g)
  // Staging: hidden 64 tokens x 32 dims (two float4 per thread), w_x (threads 0-127) or w_g
  // (128-255) 32 dims x 32 channels (two float4 per thread).
  const int tok = tid >> 2, kq = (tid & 3) * 4;
  const int wt = tid & 127, wr = wt >> 3, wc = (wt & 7) * 4;
  const float* W = tid < 128 ? a.w_x : a.w_g;
  float4 hv[2], wv[2];
  auto load_slice = [&](int k0) {
    const int64_t t = t0 + tok;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int k = k0 + kq + 16 * u;
      hv[u] = t < a.T && k < dm ? *reinterpret_cast<const float4*>(a.hidden + (b * a.T + t) * dm + k)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
      const int kr = k0 + wr + 16 * u;
      wv[u] = kr < dm ? *reinterpret_cast<const float4*>(W + (int64_t)kr * d + c0 + wc)
                      : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  floatx16 acc = floatx16{};
  const int arow = 32 * tg + (lane & 31), kl = lane >> 5, bcol = lane & 31;
  load_slice(0);
  for (int k0 = 0; k0 < dm; k0 += TK) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kk = kq + 16 * u;
      sh[tok][kk] = hv[u].x; sh[tok][kk + 1] = hv[u].y; sh[tok][kk + 2] = hv[u].z; sh[tok][kk + 3] = hv[u].w;
      *reinterpret_cast<float4*>(&sw[tid < 128 ? 0 : 1][wr + 16 * u][wc]) = wv[u];
    }
    __syncthreads();
    if (k0 + TK < dm) load_slice(k0 + TK);
#pragma unroll
    for (int kk = 0; kk < TK; kk += 2)
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(sh[arow][kk + kl], sw[mat][kk + kl][bcol], acc, 0, 0, 0);
    __syncthreads();
  }
  // g tiles to the x waves (through the idle hidden tile: 2 x 16 x 64 floats).
  float* red = &sh[0][0];
  if (mat == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[(tg * 16 + i) * 64 + lane] = acc[i];
  }
  __syncthreads();
  if (mat == 1) return;
  float gv[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) gv[i] = red[(tg * 16 + i) * 64 + lane];
  const int ch = c0 + (lane & 31);
  // Token of element i: t0 + 32 tg + 8 (i >> 2) + 4 (lane >> 5) + (i & 3).
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t t = t0 + 32 * tg + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    if (t < a.T) a.raw_x_out[(b * a.T + t) * d + ch] = acc[i];
  }
  const int m = a.m;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t tq = t0 + 32 * tg + 8 * q + 4 * (lane >> 5);   // first of this lane's four tokens
    for (int blk = 0; blk < 4 / m; ++blk) {
      const int64_t tb = tq + blk * m;
      if (tb + m > a.T) break;
      float ai[4], xi[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * q + blk * m + (i < m ? i : 0);
        ai[i] = gv[e] + a.bias[i < m ? i : 0];
        xi[i] = acc[e];
      }
      PoolAcc pa = pool_start();
      pool_fold(pa, ai, xi, m);
      const float ev = pool_value(pa);
      store_entry<1>(a.out, b, tb / m, ch, &ev, 0.f);
    }
  }
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  const int d = a.d_c + a.d_r;
  const int64_t nb = a.T / a.m;
  if (a.hidden != nullptr) {
    if (a.T == 0) return hipSuccess;
    dim3 grid((unsigned)((a.T + 63) / 64), (unsigned)(d / 32), (unsigned)a.B);
    project_pool_kernel<<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  if (nb == 0) return hipSuccess;
  const int vec = a.in_dtype == CSA_F32 ? 4 : 8;
  const int cpr = d / vec;
  const int rows_per_wg = cpr >= 256 ? 1 : 256 / cpr;
  const int threads = rows_per_wg * cpr;
  const int64_t total = (int64_t)a.B * nb;
  const unsigned grid = (unsigned)((total + rows_per_wg - 1) / rows_per_wg);
  if (a.in_dtype == CSA_F32)
    pool_kernel<float><<<grid, threads, 0, s>>>(a, cpr, rows_per_wg);
  else
    pool_kernel<uint16_t><<<grid, threads, 0, s>>>(a, cpr, rows_per_wg);
  return hipGetLastError();
}

}  // namespace csa
