// Reference attention of one (query, head) by a 256-thread block, fp32 arithmetic, any store dtype
// and any d_c <= 1024 (shared by the reference kernel and the MFMA path's fixup kernel).
//
// Method: deepseek.csdn.net "一文搞懂 DeepSeek" V4 改进一 (CSA: selected compressed rows plus a
// short window of recent raw KV, MQA over a shared KV; HCA: dense attention over the heavily
// compressed rows) and the MLA section (key row = [latent; RoPE key], value row = latent);
// yudonglee.me "DeepSeek-V4 详解" 2.2 Step 4 and 2.3 Step 2.
//
// Keys are processed in chunks of 256: each thread forms one key's logit, the block takes the
// chunk max and rescales the running sum and output (online softmax), then every thread
// accumulates its output dimensions over the chunk's keys.
#pragma once

#include "attend_keys.h"

namespace csa {

constexpr int kGenThreads = 256;


static __device__ float block_reduce(float v, float* s_red, bool is_max) {
  v = is_max ? wave_max(v) : wave_sum(v);
  const int lane = threadIdx.x & (kWave - 1), wv = threadIdx.x / kWave;
  if (lane == 0) s_red[wv] = v;
  __syncthreads();
  float r = s_red[0];
  for (int w = 1; w < kGenThreads / kWave; ++w) r = is_max ? fmaxf(r, s_red[w]) : r + s_red[w];
  __syncthreads();
  return r;
}

// Attention of query qi, head h by the calling 256-thread block; smem holds at least
// generic_smem_bytes(d) bytes.
static __device__ void attend_generic_one(const AttendArgs& a, int qi, int h, float* smem) {
  const int d_c = a.ent.d_c, d_r = a.ent.d_r, d = d_c + d_r;
  float* sq = smem;                 // [d]
  float* sp = sq + d;               // [256] probabilities of the chunk
  float* s_red = sp + kGenThreads;     // [4]
  int64_t* s_row = reinterpret_cast<int64_t*>(s_red + 8);   // [256] row of each key (-1: none)
  int* s_src = reinterpret_cast<int*>(s_row + kGenThreads);    // [256] 0 = entries, 1 = raw
  const KeyList kl = make_key_list(a, qi);
  for (int e = threadIdx.x; e < d; e += kGenThreads)
    sq[e] = load_vec(a.q, a.q_dtype, ((int64_t)qi * a.H + h) * d + e);
  __syncthreads();
  constexpr int kMaxPer = 4;        // output dims per thread: d_c <= 1024
  float o[kMaxPer] = {0.f, 0.f, 0.f, 0.f};
  float run_max = -INFINITY, run_sum = 0.f;
  for (int64_t c0 = 0; c0 < kl.total; c0 += kGenThreads) {
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
    const int64_t cnt = kl.total - c0 < kGenThreads ? kl.total - c0 : kGenThreads;
    for (int j = 0; j < cnt; ++j) {
      const float pj = sp[j];
      if (pj == 0.f) continue;
      const int64_t rj = s_row[j];
      const Store& st = s_src[j] ? a.raw : a.ent;
      const float w = pj * row_scale(st, kl.b, rj);
#pragma unroll
      for (int r = 0; r < kMaxPer; ++r) {
        const int e = threadIdx.x + r * kGenThreads;
        if (e < d_c) o[r] = fmaf(w, load_c(st, kl.b, rj, e), o[r]);
      }
    }
    __syncthreads();
  }
  const int64_t ob = ((int64_t)qi * a.H + h) * d_c;
  const float inv = run_sum > 0.f ? 1.0f / run_sum : 0.f;
#pragma unroll
  for (int r = 0; r < kMaxPer; ++r) {
    const int e = threadIdx.x + r * kGenThreads;
    if (e < d_c) a.out[ob + e] = o[r] * inv;
  }
  if (a.lse != nullptr && threadIdx.x == 0)
    a.lse[(int64_t)qi * a.H + h] = run_sum > 0.f ? run_max + logf(run_sum) : -INFINITY;
}


__host__ __device__ constexpr size_t generic_smem_bytes(int d) {
  return sizeof(float) * (d + kGenThreads + 8) + sizeof(int64_t) * kGenThreads + sizeof(int) * kGenThreads;
}

}  // namespace csa
