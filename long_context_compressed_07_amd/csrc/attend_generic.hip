// Reference attention kernel for csa_attend / hca_attend: one workgroup per (query, head), fp32
// arithmetic, any store dtype and any d_c <= 1024. It serves the fp32 workloads, shapes without a
// specialised MFMA path, and as the GPU-side cross-check of the MFMA kernels.
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 (CSA: selected compressed rows plus a
// short window of recent raw KV, MQA over a shared KV; HCA: dense attention over the heavily
// compressed rows) and the MLA section (key row = [latent; RoPE key], value row = latent);
// yudonglee.me "DeepSeek-V4 详解" 2.2 Step 4 and 2.3 Step 2.
//
// Keys are processed in chunks of 256: each thread forms one key's logit, the block takes the
// chunk max and rescales the running sum and output (online softmax), then every thread
// accumulates its output dimensions over the chunk's keys.
#include "attend_keys.h"

namespace csa {
namespace {

constexpr int kThreads = 256;

__device__ float block_reduce(float v, float* s_red, bool is_max) {
  v = is_max ? wave_max(v) : wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  if (lane == 0) s_red[wv] = v;
  __syncthreads();
  float r = s_red[0];
  for (int w = 1; w < kThreads / kWave; ++w) r = is_max ? fmaxf(r, s_red[w]) : r + s_red[w];
  __syncthreads();
  return r;
}

__global__ void __launch_bounds__(kThreads) attend_generic_kernel(AttendArgs a) {
  extern __shared__ float smem[];
  const int qi = blockIdx.x / a.H;
  const int h = blockIdx.x - qi * a.H;
  const int d_c = a.ent.d_c, d_r = a.ent.d_r, d = d_c + d_r;
  float* sq = smem;                 // [d]
  float* sp = sq + d;               // [256] probabilities of the chunk
  float* s_red = sp + kThreads;     // [4]
  int64_t* s_row = reinterpret_cast<int64_t*>(s_red + 8);   // [256] row of each key (-1: none)
  int* s_src = reinterpret_cast<int*>(s_row + kThreads);    // [256] 0 = entries, 1 = raw
  const KeyList kl = make_key_list(a, qi);
  for (int e = threadIdx.x; e < d; e += kThreads)
    sq[e] = load_vec(a.q, a.q_dtype, ((int64_t)qi * a.H + h) * d + e);
  __syncthreads();
  constexpr int kMaxPer = 4;        // output dims per thread: d_c <= 1024
  float o[kMaxPer] = {0.f, 0.f, 0.f, 0.f};
  float run_max = -INFINITY, run_sum = 0.f;
  for (int64_t c0 = 0; c0 < kl.total; c0 += kThreads) {
    const int64_t kk = c0 + threadIdx.x;
    int src = 0;
    int64_t row = -1;
    float logit = -INFINITY;
    if (kk < kl.total) {
      row = key_row(a, kl, kk, src);
      if (row >= 0) {
        const Store& st = src ? a.raw : a.ent;
        float dc = 0.f, dr = 0.f;
        for (int e = 0; e < d_c; ++e) dc = fmaf(sq[e], load_c(st, kl.b, row, e), dc);
        for (int e = 0; e < d_r; ++e) dr = fmaf(sq[d_c + e], load_r(st, kl.b, row, e), dr);
        logit = a.sm_scale * fmaf(dc, row_scale(st, kl.b, row), dr);
      }
    }
    s_row[threadIdx.x] = row;
    s_src[threadIdx.x] = src;
    const float cmax = block_reduce(logit, s_red, true);
    const float new_max = fmaxf(run_max, cmax);
    float p = 0.f;
    if (row >= 0 && new_max > -INFINITY) p = expf(logit - new_max);
    sp[threadIdx.x] = p;
    const float csum = block_reduce(p, s_red, false);
    const float corr = run_max > -INFINITY ? expf(run_max - new_max) : 0.f;
    run_sum = run_sum * corr + csum;
#pragma unroll
    for (int r = 0; r < kMaxPer; ++r) o[r] *= corr;
    run_max = new_max;
    const int64_t cnt = kl.total - c0 < kThreads ? kl.total - c0 : kThreads;
    for (int j = 0; j < cnt; ++j) {
      const float pj = sp[j];
      if (pj == 0.f) continue;
      const int64_t rj = s_row[j];
      const Store& st = s_src[j] ? a.raw : a.ent;
      const float w = pj * row_scale(st, kl.b, rj);
#pragma unroll
      for (int r = 0; r < kMaxPer; ++r) {
        const int e = threadIdx.x + r * kThreads;
        if (e < d_c) o[r] = fmaf(w, load_c(st, kl.b, rj, e), o[r]);
      }
    }
    __syncthreads();
  }
  const int64_t ob = ((int64_t)qi * a.H + h) * d_c;
  const float inv = run_sum > 0.f ? 1.0f / run_sum : 0.f;
#pragma unroll
  for (int r = 0; r < kMaxPer; ++r) {
    const int e = threadIdx.x + r * kThreads;
    if (e < d_c) a.out[ob + e] = o[r] * inv;
  }
  if (a.lse != nullptr && threadIdx.x == 0)
    a.lse[(int64_t)qi * a.H + h] = run_sum > 0.f ? run_max + logf(run_sum) : -INFINITY;
}

}  // namespace

hipError_t launch_attend_generic(const AttendArgs& a, hipStream_t s) {
  const int d = a.ent.d_c + a.ent.d_r;
  const size_t shm = sizeof(float) * (d + kThreads + 8) + sizeof(int64_t) * kThreads +
                     sizeof(int) * kThreads;
  attend_generic_kernel<<<(unsigned)((int64_t)a.Q.nq * a.H), kThreads, shm, s>>>(a);
  return hipGetLastError();
}

}  // namespace csa
