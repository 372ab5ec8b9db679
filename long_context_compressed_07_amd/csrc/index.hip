// csa_index kernels: lightning-indexer scores s[i][j] = sum_h w[i][h] * ReLU(qI[i][h] . kI[j]).
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 (a light indexer scores every compressed
// row against the current query) and yudonglee.me "DeepSeek-V4 详解" 2.2 Step 2 (like the V3.2
// lightning indexer, FP8 accelerated). The ReLU-weighted head sum is this library's reading.
//
// index_generic_kernel: one thread per (query, entry), any dtype and d_I; the query's heads are
// dequantised once into LDS. It is the reference kernel and the fallback for shapes without a
// specialised path.
#include "common.h"

namespace csa {
namespace {

__global__ void __launch_bounds__(256) index_generic_kernel(IndexArgs a, int tiles) {
  extern __shared__ float smem[];
  const int qi = blockIdx.x / tiles;
  const int64_t j0 = (int64_t)(blockIdx.x - qi * tiles) * 256;
  const int64_t pos = a.Q.pos[qi];
  const int64_t b = a.Q.seq[qi];
  const int64_t nv = n_visible(pos, a.m, a.N);
  if (j0 >= nv) return;  // uniform for the whole block
  const int hd = a.H_I * a.d_I;
  float* sq = smem;
  float* sw = smem + hd;
  for (int e = threadIdx.x; e < hd; e += blockDim.x) {
    float v = load_vec(a.q_i, a.dtype, (int64_t)qi * hd + e);
    if (a.dtype == CSA_E4M3) v *= a.q_i_scale[(int64_t)qi * a.H_I + e / a.d_I];
    sq[e] = v;
  }
  for (int h = threadIdx.x; h < a.H_I; h += blockDim.x) sw[h] = a.w[(int64_t)qi * a.H_I + h];
  __syncthreads();
  const int64_t j = j0 + threadIdx.x;
  if (j >= nv) return;
  const int64_t krow = (b * a.N + j) * a.d_I;
  const float ks = a.dtype == CSA_E4M3 ? a.k_i_scale[b * a.N + j] : 1.0f;
  float s = 0.f;
  for (int h = 0; h < a.H_I; ++h) {
    float dot = 0.f;
    for (int e = 0; e < a.d_I; ++e) dot = fmaf(sq[h * a.d_I + e], load_vec(a.k_i, a.dtype, krow + e), dot);
    s = fmaf(sw[h], fmaxf(dot * ks, 0.f), s);
  }
  a.scores[(int64_t)qi * a.ld_scores + j] = s;
}

}  // namespace

bool index_fast(const IndexArgs& a, hipStream_t s, hipError_t* err);

hipError_t launch_index(const IndexArgs& a, hipStream_t s) {
  if (a.Q.nq == 0 || a.N == 0) return hipSuccess;
  hipError_t err;
  if (index_fast(a, s, &err)) return err;
  const int tiles = (int)((a.N + 255) / 256);
  const size_t shm = sizeof(float) * ((size_t)a.H_I * a.d_I + a.H_I);
  index_generic_kernel<<<(unsigned)((int64_t)tiles * a.Q.nq), 256, shm, s>>>(a, tiles);
  return hipGetLastError();
}

}  // namespace csa
