// csa_compress kernels: softmax-gated pooling of m consecutive token rows into one entry.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 (CSA step one: m adjacent tokens' KV
// merged with position-biased softmax weights) and yudonglee.me "DeepSeek-V4 详解" 2.2 Step 1 /
// 2.3 Step 1 (m = 4 for CSA, m' = 128 for HCA). Per channel c of block j:
//   a_i = g[jm+i][c] + bias[i],  w = softmax_i(a),  e[j][c] = sum_i w_i x[jm+i][c].
//
// pool_kernel streams x and g once (HBM-bound): one thread owns VEC consecutive channels of one
// entry (16-byte loads, consecutive threads on consecutive channels of a row) and folds the m
// positions in chunks of 4 with a running max, so each element costs 1 + 1/4 exponentials.
// project_pool_kernel is the fp32 projection mode: x = hidden * w_x and g = hidden * w_g are
// formed tile by tile in LDS and pooled in registers, so x and g never reach HBM (only the raw x
// rows the sliding window needs are written).
#include "common.h"

namespace csa {
namespace {

template <typename TIn>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int N = 4;
  __device__ static void load(const void* base, int64_t off, float* out) {
    const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  }
};
template <>
struct Vec<uint16_t> {
  static constexpr int N = 8;
  __device__ static void load(const void* base, int64_t off, float* out) {
    const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
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
    for (int v = 0; v < VEC; ++v)
      p[v] = (uint8_t)(sigma > 0.0f ? f32_to_e4m3(__fdiv_rn(e[v], sigma)) : 0u);
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

  float acc[VEC], sum[VEC], mx[VEC];
  int64_t b = 0, j = 0;
  if (active) {
    b = gr / nb;
    j = gr - b * nb;
#pragma unroll
    for (int v = 0; v < VEC; ++v) { acc[v] = 0.f; sum[v] = 0.f; mx[v] = -INFINITY; }
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
        float cm = av[0][v];
#pragma unroll
        for (int p = 1; p < 4; ++p)
          if (p < cnt) cm = fmaxf(cm, av[p][v]);
        const float nm = fmaxf(mx[v], cm);
        const float c1 = __expf(mx[v] - nm);
        float s = sum[v] * c1, ac = acc[v] * c1;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          if (p < cnt) {
            const float e = __expf(av[p][v] - nm);
            s += e;
            ac = fmaf(e, xv[p][v], ac);
          }
        }
        sum[v] = s;
        acc[v] = ac;
        mx[v] = nm;
      }
    }
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = __fdiv_rn(acc[v], sum[v]);
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
      sigma = __fdiv_rn(__uint_as_float(s_amax[lr]), 448.0f);
      if (cv == 0) a.out.scale[b * a.out.rows + j] = sigma;
    }
  }
  if (active) store_entry<VEC>(a.out, b, j, ch, acc, sigma);
}

// fp32 projection + pooling. Tile: 64 tokens x 64 channels of both x and g; thread (ty, tx) owns
// tokens [4ty, 4ty+4) and channels [4tx, 4tx+4), so every block of m in {1, 2, 4} tokens is
// thread-local.
__global__ void __launch_bounds__(256) project_pool_kernel(CompressArgs a) {
  constexpr int TK = 16;
  __shared__ float sh[64][TK + 1];
  __shared__ float swx[TK][64];
  __shared__ float swg[TK][64];
  const int tid = threadIdx.x;
  const int ty = tid >> 4, tx = tid & 15;
  const int64_t b = blockIdx.z;
  const int64_t t0 = (int64_t)blockIdx.x * 64;
  const int c0 = blockIdx.y * 64;
  const int d = a.d_c + a.d_r;
  const int dm = a.d_model;
  float ax[4][4] = {}, ag[4][4] = {};
  for (int k0 = 0; k0 < dm; k0 += TK) {
    {
      const int tok = tid >> 2, kq = (tid & 3) * 4;
      const int64_t t = t0 + tok;
      float4 hv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (t < a.T && k0 + kq < dm)
        hv = *reinterpret_cast<const float4*>(a.hidden + (b * a.T + t) * dm + k0 + kq);
      sh[tok][kq] = hv.x; sh[tok][kq + 1] = hv.y; sh[tok][kq + 2] = hv.z; sh[tok][kq + 3] = hv.w;
      const int wr = tid >> 4, wc = (tid & 15) * 4;
      float4 wx = make_float4(0.f, 0.f, 0.f, 0.f), wg = wx;
      if (k0 + wr < dm) {
        wx = *reinterpret_cast<const float4*>(a.w_x + (int64_t)(k0 + wr) * d + c0 + wc);
        wg = *reinterpret_cast<const float4*>(a.w_g + (int64_t)(k0 + wr) * d + c0 + wc);
      }
      *reinterpret_cast<float4*>(&swx[wr][wc]) = wx;
      *reinterpret_cast<float4*>(&swg[wr][wc]) = wg;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float h[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) h[r] = sh[ty * 4 + r][kk];
      const float4 wx = *reinterpret_cast<const float4*>(&swx[kk][tx * 4]);
      const float4 wg = *reinterpret_cast<const float4*>(&swg[kk][tx * 4]);
      const float wxv[4] = {wx.x, wx.y, wx.z, wx.w};
      const float wgv[4] = {wg.x, wg.y, wg.z, wg.w};
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          ax[r][c] = fmaf(h[r], wxv[c], ax[r][c]);
          ag[r][c] = fmaf(h[r], wgv[c], ag[r][c]);
        }
    }
    __syncthreads();
  }
  const int ch = c0 + tx * 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t t = t0 + ty * 4 + r;
    if (t < a.T) {
      float* p = a.raw_x_out + (b * a.T + t) * d + ch;
#pragma unroll
      for (int c = 0; c < 4; ++c) p[c] = ax[r][c];
    }
  }
  const int m = a.m;
  for (int blk = 0; blk < 4 / m; ++blk) {
    const int64_t tb = t0 + ty * 4 + blk * m;  // first token of the block
    if (tb + m > a.T) break;
    float e[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float mxv = -INFINITY;
      for (int i = 0; i < m; ++i) mxv = fmaxf(mxv, ag[blk * m + i][c] + a.bias[i]);
      float s = 0.f, acc = 0.f;
      for (int i = 0; i < m; ++i) {
        const float w = __expf(ag[blk * m + i][c] + a.bias[i] - mxv);
        s += w;
        acc = fmaf(w, ax[blk * m + i][c], acc);
      }
      e[c] = __fdiv_rn(acc, s);
    }
    store_entry<4>(a.out, b, tb / m, ch, e, 0.f);
  }
}

}  // namespace

hipError_t launch_compress(const CompressArgs& a, hipStream_t s) {
  const int d = a.d_c + a.d_r;
  const int64_t nb = a.T / a.m;
  if (a.hidden != nullptr) {
    if (a.T == 0) return hipSuccess;
    dim3 grid((unsigned)((a.T + 63) / 64), (unsigned)(d / 64), (unsigned)a.B);
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
