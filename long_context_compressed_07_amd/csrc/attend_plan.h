// Work decomposition shared by the MFMA attention kernels, their split-K combine and the fp32
// fixup pass.
#pragma once

#include "csa_internal.h"

namespace csa {

struct AttnPlan {
  int ksw;            // fp16-staging kernel: key splits inside a workgroup (4 / ksw head groups)
  int rg;             // DMA kernels: 32-head row groups per workgroup (bf16: 2, fp8: 4)
  int head_groups;    // workgroups per query along heads
  int n_split;        // workgroups per query along keys
  int f8_dma;         // 1: fp8 rows staged by DMA and converted in LDS (attend_fp8.hip)
  int pp;             // 1: bf16, 64 heads per workgroup, QK and PV wave roles (attend_pp.hip)
  _Float16* ws_o;     // [nq][n_split][H][512] partial outputs normalised by their l, n_split > 1
  float* ws_ml;       // [nq][n_split][H][2] partial (max in log2 units, sum)
  int* flags;         // [nq][head_groups][n_split] 1 = some head left the range of P
};

// Log-sum-exp merge of the n_split partials of one head, 8 output dims [d0, d0 + 8): partial s
// holds o_s / l_s (fp16) and (m_s in log2 units, l_s); out = sum_s (l_s 2^(m_s - mx)) (o_s / l_s) /
// sum_s l_s 2^(m_s - mx), taken in batches of 8 splits (all loads issued before use) with a
// running maximum; writes the 8 dims of out and, for d0 == 0, the head's lse.
__device__ __forceinline__ void merge_partials8(const AttendArgs& a, const AttnPlan& plan, int qi,
                                                int head, int d0) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  constexpr int kDc = 512;
  constexpr int kBatch = 8;
  const int64_t p0 = (int64_t)qi * plan.n_split * a.H + head;   // partial index of split 0
  const int64_t ps = a.H;                                        // stride between splits
  float mx = -INFINITY, lsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < plan.n_split; s0 += kBatch) {
    float2 ml[kBatch];
    h8 v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const bool in = s0 + u < plan.n_split;
      const int64_t pidx = p0 + (int64_t)(in ? s0 + u : s0) * ps;
      ml[u] = *reinterpret_cast<const float2*>(plan.ws_ml + pidx * 2);
      v[u] = *reinterpret_cast<const h8*>(plan.ws_o + pidx * kDc + d0);
      if (!in) ml[u].x = -INFINITY;
    }
    float nm = mx;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) nm = fmaxf(nm, ml[u].x);
    const float r = mx == -INFINITY ? 0.f : exp2f(mx - nm);
    lsum *= r;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= r;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float wgt = ml[u].x == -INFINITY ? 0.f : exp2f(ml[u].x - nm) * ml[u].y;
      lsum += wgt;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += wgt * (float)v[u][j];
    }
    mx = nm;
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  float* dst = a.out + ((int64_t)qi * a.H + head) * kDc + d0;
  typedef float f32x4 __attribute__((ext_vector_type(4)));   // final outputs: non-temporal
  __builtin_nontemporal_store(f32x4{acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv},
                              reinterpret_cast<f32x4*>(dst));
  __builtin_nontemporal_store(f32x4{acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv},
                              reinterpret_cast<f32x4*>(dst + 4));
  if (a.lse != nullptr && d0 == 0)
    a.lse[(int64_t)qi * a.H + head] =
        lsum > 0.f ? (mx + __log2f(lsum)) * 0.6931471805599453f : -INFINITY;
}


// The work item of this workgroup. Workgroups go to the 8 XCDs in turn (workgroup b to XCD
// b mod 8); this mapping gives each XCD contiguous runs of items, so that the key splits and head
// groups of one query, and neighbouring queries, share that XCD's L2. Grids of at least 8 x 2048
// items are dealt out in runs of 512 (run r to XCD r mod 8), so that every XCD gets its share of
// each region of the item range: under causality the first queries' key lists are short, and
// one contiguous range per XCD would leave the XCD holding them idle at the end. Smaller grids
// give each XCD one contiguous range. The last gridDim.x mod 8 workgroups keep their own index.
__device__ __forceinline__ int xcd_item() {
  constexpr int kRun = 512;
  const int b = blockIdx.x, n = gridDim.x;
  const int n8 = n & ~7;
  if (b >= n8) return b;
  const int m = n8 >> 3;              // items per XCD
  const int x = b & 7, j = b >> 3;    // XCD, and this workgroup's rank on it
  if (m < 4 * kRun || m % kRun != 0) return x * m + j;
  return ((j / kRun) * 8 + x) * kRun + j % kRun;
}

// Four values of a normalised partial output row (o / l in fp16; zeros when l == 0).
__device__ __forceinline__ void store_partial4(_Float16* dst, float a, float b, float c, float d,
                                               float inv) {
  typedef _Float16 h4 __attribute__((ext_vector_type(4)));
  *reinterpret_cast<h4*>(dst) = h4{(_Float16)(a * inv), (_Float16)(b * inv), (_Float16)(c * inv),
                                   (_Float16)(d * inv)};
}

hipError_t launch_attend_fp8(const AttendArgs& a, const AttnPlan& p, hipStream_t s);
hipError_t launch_attend_pp(const AttendArgs& a, const AttnPlan& p, hipStream_t s);

}  // namespace csa
