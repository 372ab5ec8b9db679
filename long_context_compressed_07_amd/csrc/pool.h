// The pooling arithmetic of one channel, shared by every kernel that builds a compressed entry
// (csa_compress's pool_kernel and project_pool_kernel, csa_cache_append's append_kernel), so that
// an entry pooled at prefill and the same entry pooled at decode are bitwise equal.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 and yudonglee.me "DeepSeek-V4 详解"
// 2.2 Step 1 / 2.3 Step 1: the m positions of a block are merged per channel with softmax weights
// of the gate logits plus a position bias, e = sum_i softmax_i(a) x_i, a_i = g_i + bias_i.
//
// Order of the arithmetic: positions are folded in chunks of up to 4 in position order with a
// running maximum (each chunk rescales the running sums once by exp(old max - new max)), and the
// result is the correctly rounded quotient of the two sums. Each element costs 1 + 1/4
// exponentials.
#pragma once

#include "common.h"

namespace csa {

struct PoolAcc {
  float mx;    // running maximum of the logits folded so far
  float sum;   // sum of exp(a_i - mx)
  float acc;   // sum of exp(a_i - mx) x_i
};

__device__ __forceinline__ PoolAcc pool_start() { return PoolAcc{-INFINITY, 0.f, 0.f}; }

// Folds cnt (1..4) positions with logits a[] and values x[] into the running state.
__device__ __forceinline__ void pool_fold(PoolAcc& p, const float (&a)[4], const float (&x)[4],
                                          int cnt) {
  float cm = a[0];
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (i < cnt) cm = fmaxf(cm, a[i]);
  const float nm = fmaxf(p.mx, cm);
  const float c1 = __expf(p.mx - nm);
  float s = p.sum * c1, ac = p.acc * c1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < cnt) {
      const float e = __expf(a[i] - nm);
      s += e;
      ac = fmaf(e, x[i], ac);
    }
  }
  p.mx = nm;
  p.sum = s;
  p.acc = ac;
}

__device__ __forceinline__ float pool_value(const PoolAcc& p) { return __fdiv_rn(p.acc, p.sum); }

// Row scale of an e4m3 entry row from the largest latent magnitude, and one stored code.
__device__ __forceinline__ float e4m3_row_scale(float amax) { return __fdiv_rn(amax, 448.0f); }
__device__ __forceinline__ uint8_t e4m3_code(float v, float sigma) {
  return (uint8_t)(sigma > 0.0f ? f32_to_e4m3(__fdiv_rn(v, sigma)) : 0u);
}

}  // namespace csa
