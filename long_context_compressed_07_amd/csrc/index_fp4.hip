// csa_index_mxfp4: lightning-indexer scores from MXFP4 queries and keys, stored as bf16.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek", V4 的其他升级 (the indexer's QK path runs in FP4
// with fine-grained scales; FP4 values widen losslessly to FP8 because FP8 has two more exponent
// bits that absorb the scales; index scores drop to BF16, which makes the top-k selection 2x
// faster); jaylab-temp.pages.dev 其他技术细节 (FP4 for the indexer QK path). The score is the one
// of csa_index: s[j] = sum_h w[h] * ReLU(qI[h] . kI[j]).
//
// Format (OCP MX): E2M1 codes, two per byte (element 2i in the low nibble of byte i), one E8M0
// scale per 32 consecutive values; d_I = 64 gives 32 bytes of codes and 2 scale bytes per vector.
// gfx950's scaled MFMA takes exactly this: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in
// FP4 reads, per lane, one 32-value block (16 bytes) and its E8M0 scale. Products of two E2M1
// values are exact, so every per-block dot product is exact in fp32; the head sum is fp32 and the
// score is rounded to bf16 (round to nearest even) once.
//
// Work: a workgroup streams a range of one query's keys. The query's 8 heads are the rows of the
// A operand (rows 8..31 zero), 32 keys the columns of B; lane l then holds heads 4 (l / 32) + r
// (r < 4) of key l % 32 in its accumulators, and one exchange with lane l ^ 32 completes the head
// sum. Each wave issues the loads of 8 MFMA steps (256 keys) before using them.
#include "common.h"

namespace csa {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kFp4Batch = 8;                  // MFMA steps per wave with their loads in flight
constexpr int kFp4PerIter = 4 * 32 * kFp4Batch;   // keys per workgroup iteration (1024)
constexpr int kFmtFp4 = 4;                    // f8f6f4 operand format code of E2M1

__global__ void __launch_bounds__(256) index_mxfp4_kernel(IndexFp4Args a, int64_t per_wg, int nx) {
  const int qi = blockIdx.x / nx;
  const int chunk = blockIdx.x - qi * nx;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int64_t b = a.Q.seq[qi];
  const int64_t nv = n_visible(a.Q.pos[qi], a.m, a.N);
  const int64_t j0 = (int64_t)chunk * per_wg;
  const int64_t j1 = j0 + per_wg < nv ? j0 + per_wg : nv;
  if (j0 >= j1) return;
  // A: head col (rows 0..7 real), values 32 half + [0, 32) of its vector, with that block's scale.
  const int h = col & 7;
  const int64_t qrow = (int64_t)qi * 8 + h;
  const uint4 qv = *reinterpret_cast<const uint4*>(a.q_i + qrow * 32 + 16 * half);
  const int qs = a.q_i_scale[qrow * 2 + half];
  const v8i A = col < 8 ? v8i{(int)qv.x, (int)qv.y, (int)qv.z, (int)qv.w, 0, 0, 0, 0}
                        : v8i{0, 0, 0, 0, 0, 0, 0, 0};
  const int sa = col < 8 ? qs : 127;
  float wh[4];   // weights of the heads in accumulator rows 0..3 of this lane
#pragma unroll
  for (int r = 0; r < 4; ++r) wh[r] = a.w[(int64_t)qi * 8 + 4 * half + r];
  const uint8_t* kb = a.k_i + b * a.N * 32;
  const uint8_t* ks = a.k_i_scale + b * a.N * 2;
  uint16_t* out = a.scores + (int64_t)qi * a.ld_scores;
  // Keys past the range are clamped to its last one (loaded, not stored): no branches on loads.
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  for (int64_t base = j0 + 32 * kFp4Batch * w; base < j1; base += kFp4PerIter) {
    uint4 v[kFp4Batch];
    int sc[kFp4Batch];
#pragma unroll
    for (int u = 0; u < kFp4Batch; ++u) {
      int64_t ent = base + 32 * u + col;
      ent = ent < j1 ? ent : j1 - 1;
      // Keys are read once: non-temporal loads.
      const u32x4 kv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + ent * 32 + 16 * half));
      v[u] = make_uint4(kv.x, kv.y, kv.z, kv.w);
      sc[u] = __builtin_nontemporal_load(ks + ent * 2 + half);
    }
#pragma unroll
    for (int u = 0; u < kFp4Batch; ++u) {
      const v8i B = v8i{(int)v[u].x, (int)v[u].y, (int)v[u].z, (int)v[u].w, 0, 0, 0, 0};
      floatx16 acc = floatx16{};
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, B, acc, kFmtFp4, kFmtFp4, 0, sa, 0,
                                                            sc[u]);
      float p = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) p = fmaf(wh[r], fmaxf(acc[r], 0.f), p);
      p += __shfl_xor(p, 32);
      const int64_t ent = base + 32 * u + col;
      if (half == 0 && ent < j1) out[ent] = f32_to_bf16(p);
    }
  }
}

}  // namespace

hipError_t launch_index_fp4(const IndexFp4Args& a, hipStream_t s) {
  if (a.Q.nq == 0 || a.N == 0) return hipSuccess;
  // Enough workgroups to keep every CU streaming: >= 2048 in total, >= 1024 keys each.
  int64_t per_wg = (a.N * a.Q.nq + 2047) / 2048;
  per_wg = per_wg < kFp4PerIter ? kFp4PerIter : per_wg;
  per_wg = (per_wg + kFp4PerIter - 1) / kFp4PerIter * kFp4PerIter;
  const int64_t nx = (a.N + per_wg - 1) / per_wg;
  index_mxfp4_kernel<<<(unsigned)(nx * a.Q.nq), 256, 0, s>>>(a, per_wg, (int)nx);
  return hipGetLastError();
}

}  // namespace csa
