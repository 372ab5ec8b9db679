// Fast csa_index kernels for the indexer shape of the workloads: H_I = 8 heads of d_I = 64.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 and yudonglee.me "DeepSeek-V4 详解" 2.2
// Step 2 (lightning indexer, FP8 accelerated); score s = sum_h w_h ReLU(qI_h . kI_j).
//
// index_bf16_mfma_kernel (many queries, bf16): a workgroup takes 32 consecutive queries of one
// sequence; rows of the contraction are (query, head) pairs, 4 queries x 8 heads per 32-row
// MFMA tile, columns are entries. The rows are ordered so that in the 32x32 output tile a lane
// holds all 8 heads of two queries for one entry: the ReLU-weighted head sum stays in registers.
// Entry blocks of 128 rows are staged once in LDS and read as B fragments by all four waves. Only
// visible entries (j < n_vis of each query) are computed and written.
//
// index_fp8_stream_kernel (decode, e4m3 with per-row scales): each wave step reads 16 entries
// (1 KiB, one 16-byte load per lane, fully coalesced), widens the codes to fp16 and runs two
// 16x16x32 MFMAs with the query's heads as rows; ReLU(s_q s_k q.k) = s_q s_k ReLU(q.k) lets the
// scales fold into the head weights and the row scale.
#include "common.h"

namespace csa {
namespace {

typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kQ = 32;          // queries per workgroup
constexpr int kE = 128;         // entries per staged block
constexpr int kRowK = 64 + 8;   // LDS row stride of a staged key (bf16 elements)

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ void index_one_query_generic(const IndexArgs& a, int qi) {
  const int64_t b = a.Q.seq[qi];
  const int64_t nv = n_visible(a.Q.pos[qi], a.m, a.N);
  for (int64_t j = threadIdx.x; j < nv; j += blockDim.x) {
    float s = 0.f;
    for (int h = 0; h < a.H_I; ++h) {
      float dot = 0.f;
      for (int e = 0; e < a.d_I; ++e)
        dot = fmaf(load_vec(a.q_i, a.dtype, ((int64_t)qi * a.H_I + h) * a.d_I + e),
                   load_vec(a.k_i, a.dtype, (b * a.N + j) * a.d_I + e), dot);
      s = fmaf(a.w[(int64_t)qi * a.H_I + h], fmaxf(dot, 0.f), s);
    }
    a.scores[(int64_t)qi * a.ld_scores + j] = s;
  }
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
index_bf16_mfma_kernel(IndexArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k[kE * kRowK];
  __shared__ float s_w[kQ * 8];
  __shared__ int64_t s_nv[kQ];
  __shared__ int s_uniform;
  // The last query blocks first: under causality they see the most entries, and starting them
  // first shortens the tail of the grid.
  const int q0 = (gridDim.x - 1 - blockIdx.x) * kQ;
  const int nqw = a.Q.nq - q0 < kQ ? a.Q.nq - q0 : kQ;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, hi = lane >> 5;
  const int64_t b = a.Q.seq[q0];
  if (tid == 0) s_uniform = 1;
  __syncthreads();
  if (tid < nqw) {
    if (a.Q.seq[q0 + tid] != b) s_uniform = 0;
    s_nv[tid] = n_visible(a.Q.pos[q0 + tid], a.m, a.N);
  } else if (tid < kQ) {
    s_nv[tid] = 0;
  }
  for (int i = tid; i < kQ * 8; i += 256)
    s_w[i] = (i / 8) < nqw ? a.w[(int64_t)(q0 + i / 8) * 8 + (i % 8)] : 0.f;
  __syncthreads();
  if (!s_uniform) {  // queries of several sequences: no shared key blocks
    for (int qq = 0; qq < nqw; ++qq) index_one_query_generic(a, q0 + qq);
    return;
  }
  int64_t nmax = 0;
  for (int i = 0; i < kQ; ++i) nmax = s_nv[i] > nmax ? s_nv[i] : nmax;

  // A fragments: wave w owns queries q0 + 8 w + [0, 8) as two 32-row tiles. Row r of a tile
  // holds head 4 ((r >> 3) & 1) + (r & 3) of query 2 ((r >> 2) & 1) + (r >> 4), so that in the
  // 32x32 output layout each lane holds all 8 heads of two queries for its entry.
  bf16x8 af[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = lane & 31;
    const int qq = 8 * w + 4 * rt + 2 * ((row >> 2) & 1) + (row >> 4);
    const int h = 4 * ((row >> 3) & 1) + (row & 3);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (qq < nqw)
        v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q_i) +
                                            ((int64_t)(q0 + qq) * 8 + h) * 64 + 16 * s + 8 * hi);
      af[rt][s] = as_bf16x8(v);
    }
  }
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_i) + b * a.N * 64;
  // Entries [e0, e0 + 128): 128 rows x 128 bytes, 16 bytes per thread-task; the next block's
  // loads are issued before the current block's MFMAs, so their latency hides behind them.
  uint4 pre[4];
  auto load_block = [&](int64_t e0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int t = tid + 256 * it;
      const int r = t >> 3, c = t & 7;
      pre[it] = e0 + r < a.N ? *reinterpret_cast<const uint4*>(kbase + (e0 + r) * 64 + 8 * c)
                             : make_uint4(0u, 0u, 0u, 0u);
    }
  };
  load_block(0);
  for (int64_t e0 = 0; e0 < nmax; e0 += kE) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int t = tid + 256 * it;
      const int r = t >> 3, c = t & 7;
      *reinterpret_cast<uint4*>(s_k + r * kRowK + 8 * c) = pre[it];
    }
    __syncthreads();
    if (e0 + kE < nmax) load_block(e0 + kE);
#pragma unroll
    for (int ct = 0; ct < kE / 32; ++ct) {
      if (e0 + 32 * ct >= nmax) break;
      bf16x8 bfr[4];
#pragma unroll
      for (int s = 0; s < 4; ++s)
        bfr[s] = as_bf16x8(*reinterpret_cast<const uint4*>(s_k + (32 * ct + (lane & 31)) * kRowK +
                                                           16 * s + 8 * hi));
      const int64_t ent = e0 + 32 * ct + (lane & 31);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        floatx16 acc = floatx16{};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[rt][s], bfr[s], acc, 0, 0, 0);
        // acc[8 u + e] = head e of query 8 w + 4 rt + 2 hi + u (u = 0, 1), entry `ent`.
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int ql = 8 * w + 4 * rt + 2 * hi + u;
          const float* wq = s_w + ql * 8;
          float p = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) p = fmaf(wq[e], fmaxf(acc[8 * u + e], 0.f), p);
          if (ql < nqw && ent < s_nv[ql]) a.scores[(int64_t)(q0 + ql) * a.ld_scores + ent] = p;
        }
      }
    }
    __syncthreads();
  }
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));

// 8 e4m3 codes (two dwords) -> 8 fp16 values, exactly (every e4m3 value is an fp16 value).
__device__ __forceinline__ half8 e4m3x8_to_f16(uint32_t lo, uint32_t hi) {
  typedef float float2v __attribute__((ext_vector_type(2)));
  const float2v p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
  const float2v p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
  const float2v p2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
  const float2v p3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
  return half8{(_Float16)p0.x, (_Float16)p0.y, (_Float16)p1.x, (_Float16)p1.y,
               (_Float16)p2.x, (_Float16)p2.y, (_Float16)p3.x, (_Float16)p3.y};
}

// Workgroup (query qi, chunk c) covers entries [c * per_wg, (c + 1) * per_wg) (per_wg a multiple
// of 512); each wave step handles 16 entries. The fp8 codes are widened exactly to fp16 and contracted with the fp16
// MFMA (fp32 accumulation): the fp8 MFMA's own accumulation is narrower than fp32, which would
// move scores by ~2^-14 of the row maximum and with them near-boundary selections.
__global__ void __launch_bounds__(256) index_fp8_stream_kernel(IndexArgs a, int64_t per_wg,
                                                               int nx) {
  const int qi = blockIdx.x / nx;
  const int chunk = blockIdx.x - qi * nx;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int64_t b = a.Q.seq[qi];
  const int64_t nv = n_visible(a.Q.pos[qi], a.m, a.N);
  const int64_t j0 = (int64_t)chunk * per_wg;
  const int64_t j1 = j0 + per_wg < nv ? j0 + per_wg : nv;
  if (j0 >= j1) return;
  // A fragments: head `col` (< 8 real), dims 16 g + 8 s + [0, 8) for k-step s.
  // (Loads are unconditional, from clamped indices, so that they are all in flight together.)
  const uint8_t* qp =
      static_cast<const uint8_t*>(a.q_i) + ((int64_t)qi * 8 + (col & 7)) * 64 + 16 * g;
  const uint4 qv = *reinterpret_cast<const uint4*>(qp);
  float wh[4];   // w_h * scale_q,h for the heads of this lane's accumulators (4 g + i)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = (4 * g + i) & 7;
    wh[i] = a.w[(int64_t)qi * 8 + h] * a.q_i_scale[(int64_t)qi * 8 + h];
    wh[i] = g < 2 ? wh[i] : 0.f;
  }
  const half8 zero8 = half8{0, 0, 0, 0, 0, 0, 0, 0};
  const half8 a0 = col < 8 ? e4m3x8_to_f16(qv.x, qv.y) : zero8;
  const half8 a1 = col < 8 ? e4m3x8_to_f16(qv.z, qv.w) : zero8;
  const uint8_t* kb = static_cast<const uint8_t*>(a.k_i) + b * a.N * 64;
  const float* ks = a.k_i_scale + b * a.N;
  float* out = a.scores + (int64_t)qi * a.ld_scores;
  // Batches of 8 steps per wave (128 entries; 512 per workgroup): all 8 row loads and scale loads
  // are issued before any is used. Rows past the end are clamped to the last entry (loaded, not
  // stored), so the loads need no branches.
  for (int64_t base = j0 + 128 * w; base < j1; base += 512) {
    uint4 v[8];
    float sc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      int64_t ent = base + 16 * u + col;
      ent = ent < j1 ? ent : j1 - 1;
      v[u] = *reinterpret_cast<const uint4*>(kb + ent * 64 + 16 * g);
      sc[u] = ks[ent];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, e4m3x8_to_f16(v[u].x, v[u].y), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, e4m3x8_to_f16(v[u].z, v[u].w), acc, 0, 0, 0);
      // acc[i] = q-head (4 g + i) . entry (codes); groups 0, 1 hold the 8 real heads.
      float p = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) p = fmaf(wh[i], fmaxf(acc[i], 0.f), p);
      p += __shfl_xor(p, 16);
      const int64_t ent = base + 16 * u + col;
      if (g == 0 && ent < j1) out[ent] = p * sc[u];
    }
  }
}

}  // namespace

bool index_fast(const IndexArgs& a, hipStream_t s, hipError_t* err) {
  if (a.H_I != 8 || a.d_I != 64) return false;
  if (((uintptr_t)a.q_i | (uintptr_t)a.k_i) & 15u) return false;   // 16-byte vector loads
  if (a.dtype == CSA_BF16 && a.Q.nq >= 64) {
    index_bf16_mfma_kernel<<<(unsigned)((a.Q.nq + kQ - 1) / kQ), 256, 0, s>>>(a);
    *err = hipGetLastError();
    return true;
  }
  if (a.dtype == CSA_E4M3) {
    // Enough workgroups to keep every CU streaming: >= 2048 in total, >= 1024 entries each.
    int64_t per_wg = (a.N * a.Q.nq + 2047) / 2048;
    per_wg = per_wg < 1024 ? 1024 : per_wg;
    per_wg = (per_wg + 511) / 512 * 512;
    const int64_t nx = (a.N + per_wg - 1) / per_wg;
    if (nx == 0) { *err = hipSuccess; return true; }
    index_fp8_stream_kernel<<<(unsigned)(nx * a.Q.nq), 256, 0, s>>>(a, per_wg, (int)nx);
    *err = hipGetLastError();
    return true;
  }
  return false;
}

}  // namespace csa
