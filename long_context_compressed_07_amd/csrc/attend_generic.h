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

// The arithmetic of attend_generic_one (an online softmax over chunks of keys; within a chunk the
// same sums in the same order), with chunks of `chunk` keys whose rows are first copied into LDS
// by the whole block (the chunk boundaries, where the running sums are rescaled, differ, so results
// agree to rounding): row elements are read once, by the lanes of a wave across each row, instead
// of one row per thread in the logits and one dependent load per key in the output sums. A chunk holds `chunk` keys (at most kGenThreads); rows are stored with a
// stride of d + 1 floats so that the threads of the logit loop, one key each, read different banks.
__host__ __device__ constexpr int staged_row_stride(int d) { return d + 1; }

// Floats ahead of the 8-byte row indices: the query (d rounded up to even), probabilities and
// row scales of the chunk, the reduction slots.
__host__ __device__ constexpr int staged_floats(int d) { return ((d + 3) & ~3) + 2 * kGenThreads + 8; }

__host__ __device__ constexpr size_t staged_fixed_bytes(int d) {
  return sizeof(float) * staged_floats(d) + 2 * sizeof(uint64_t) * kGenThreads;
}

// Keys per chunk that fit `budget` bytes of LDS (at least 1, at most kGenThreads).
__host__ __device__ constexpr int staged_chunk(int d, size_t budget) {
  const size_t row = sizeof(float) * (size_t)staged_row_stride(d);
  const size_t fixed = staged_fixed_bytes(d);
  const size_t n = budget > fixed ? (budget - fixed) / row : 0;
  return n < 1 ? 1 : (n > (size_t)kGenThreads ? kGenThreads : (int)n);
}

__host__ __device__ constexpr size_t staged_smem_bytes(int d, int chunk) {
  return staged_fixed_bytes(d) + sizeof(float) * (size_t)staged_row_stride(d) * chunk;
}

// A load through a global-memory pointer: the store pointers come from the argument struct, so
// the compiler cannot tell them from LDS and would emit flat loads, which also count as LDS
// operations and make every wait for an LDS read a wait for the row loads as well.
template <typename T>
__device__ __forceinline__ T gload(const void* base, int64_t off) {
  typedef __attribute__((address_space(1))) const T GT;
  return ((GT*)base)[off];
}

// The chunk's cnt rows into sk (row j at j * ld) from the rows' addresses in s_cptr / s_rptr (0:
// no row; the row's c part, then its r part, of dtype DT). Wave v copies rows v, v + 4, ..., 16
// rows at a time, its lanes across each row's elements (64 apart), so a row's address is one
// wave-uniform value and 32 loads per lane are in flight before their LDS stores.
template <int DT>
__device__ __forceinline__ float staged_elem(uint64_t cp, uint64_t rp, int e, int d_c) {
  if (e < d_c) {
    const void* c = (const void*)(uintptr_t)cp;
    if constexpr (DT == CSA_F32) return gload<float>(c, e);
    if constexpr (DT == CSA_BF16) return bf16_to_f32(gload<uint16_t>(c, e));
    return e4m3_to_f32(gload<uint8_t>(c, e));
  }
  const void* r = (const void*)(uintptr_t)rp;
  if constexpr (DT == CSA_F32) return gload<float>(r, e - d_c);
  return bf16_to_f32(gload<uint16_t>(r, e - d_c));
}

template <int DT>
__device__ void stage_rows(int d_c, int cnt, int d, int ld, const uint64_t* s_cptr,
                           const uint64_t* s_rptr, float* sk) {
  constexpr int kRows = 16, kCols = 2;   // per wave and batch: 16 rows x 2 x 64 elements
  const int wv = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  constexpr int kWaves = kGenThreads / kWave;
  for (int j0 = wv; j0 < cnt; j0 += kWaves * kRows)
    for (int e0 = 0; e0 < d; e0 += kWave * kCols) {
      float v[kRows][kCols];
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int j = j0 + kWaves * r;
        const uint64_t cp = j < cnt ? s_cptr[j] : 0;
        const uint64_t rp = j < cnt ? s_rptr[j] : 0;
#pragma unroll
        for (int q = 0; q < kCols; ++q) {
          const int e = e0 + lane + kWave * q;
          v[r][q] = cp != 0 && e < d ? staged_elem<DT>(cp, rp, e, d_c) : 0.f;
        }
      }
#pragma unroll
      for (int r = 0; r < kRows; ++r) {
        const int j = j0 + kWaves * r;
#pragma unroll
        for (int q = 0; q < kCols; ++q) {
          const int e = e0 + lane + kWave * q;
          if (j < cnt && e < d) sk[j * ld + e] = v[r][q];
        }
      }
    }
}

static __device__ void attend_generic_staged(const AttendArgs& a, int qi, int h, float* smem,
                                             int chunk) {
  const int d_c = a.ent.d_c, d_r = a.ent.d_r, d = d_c + d_r;
  const int ld = staged_row_stride(d);
  float* sq = smem;                                // [d]
  float* sp = sq + ((d + 3) & ~3);                 // [kGenThreads] probabilities of the chunk
  float* s_scale = sp + kGenThreads;               // [kGenThreads] row scale of each key
  float* s_red = s_scale + kGenThreads;            // [8]
  // [kGenThreads] address of each key's c row (0: no row) and r row
  uint64_t* s_cptr = reinterpret_cast<uint64_t*>(smem + staged_floats(d));
  uint64_t* s_rptr = s_cptr + kGenThreads;
  float* sk = reinterpret_cast<float*>(s_rptr + kGenThreads);     // [chunk][ld]
  const KeyList kl = make_key_list(a, qi);
  const int csz = a.ent.dtype == CSA_F32 ? 4 : (a.ent.dtype == CSA_BF16 ? 2 : 1);
  const int rsz = a.ent.dtype == CSA_F32 ? 4 : 2;
  for (int e = threadIdx.x; e < d; e += kGenThreads)
    sq[e] = load_vec(a.q, a.q_dtype, ((int64_t)qi * a.H + h) * d + e);
  constexpr int kMaxPer = 4;             // output dims per thread: d_c <= 1024
  float o[kMaxPer] = {0.f, 0.f, 0.f, 0.f};
  float run_max = -INFINITY, run_sum = 0.f;
  for (int64_t c0 = 0; c0 < kl.total; c0 += chunk) {
    const int cnt = (int)(kl.total - c0 < chunk ? kl.total - c0 : chunk);
    if ((int)threadIdx.x < cnt) {
      int src = 0;
      const int64_t row = key_row(a, kl, c0 + threadIdx.x, src);
      uint64_t cp = 0, rp = 0;
      float sc = 0.f;
      if (row >= 0) {
        const Store& st = src ? a.raw : a.ent;
        const int64_t gr = kl.b * st.rows + row;
        cp = (uint64_t)(uintptr_t)st.c + (uint64_t)(gr * st.ld_c * csz);
        rp = st.r != nullptr ? (uint64_t)(uintptr_t)st.r + (uint64_t)(gr * st.ld_r * rsz) : 0;
        sc = row_scale(st, kl.b, row);
      }
      s_cptr[threadIdx.x] = cp;
      s_rptr[threadIdx.x] = rp;
      s_scale[threadIdx.x] = sc;
    }
    __syncthreads();
    // The chunk's rows (entries and raw rows share the dtype).
    if (a.ent.dtype == CSA_F32)
      stage_rows<CSA_F32>(d_c, cnt, d, ld, s_cptr, s_rptr, sk);
    else if (a.ent.dtype == CSA_BF16)
      stage_rows<CSA_BF16>(d_c, cnt, d, ld, s_cptr, s_rptr, sk);
    else
      stage_rows<CSA_E4M3>(d_c, cnt, d, ld, s_cptr, s_rptr, sk);
    __syncthreads();
    float logit = -INFINITY;
    const bool my_key = (int)threadIdx.x < cnt && s_cptr[threadIdx.x] != 0;
    if (my_key) {
      const float* kr = sk + threadIdx.x * ld;
      float dc = 0.f, dr = 0.f;
#pragma unroll 8
      for (int e = 0; e < d_c; ++e) dc = fmaf(sq[e], kr[e], dc);
#pragma unroll 8
      for (int e = 0; e < d_r; ++e) dr = fmaf(sq[d_c + e], kr[d_c + e], dr);
      logit = a.sm_scale * fmaf(dc, s_scale[threadIdx.x], dr);
    }
    const float cmax = block_reduce(logit, s_red, true);
    const float new_max = fmaxf(run_max, cmax);
    float p = 0.f;
    if (my_key && new_max > -INFINITY) p = expf(logit - new_max);
    sp[threadIdx.x] = p;
    const float csum = block_reduce(p, s_red, false);
    const float corr = run_max > -INFINITY ? expf(run_max - new_max) : 0.f;
    run_sum = run_sum * corr + csum;
#pragma unroll
    for (int r = 0; r < kMaxPer; ++r) o[r] *= corr;
    run_max = new_max;
    // Output sums in key order, four keys per step; a key without a row has p = 0 and a zero
    // row, so no key is skipped (a test on p would serialise every step on its LDS read).
    int j = 0;
    for (; j + 4 <= cnt; j += 4) {
      const float4 p4 = *reinterpret_cast<const float4*>(sp + j);
      const float4 s4 = *reinterpret_cast<const float4*>(s_scale + j);
      const float w[4] = {p4.x * s4.x, p4.y * s4.y, p4.z * s4.z, p4.w * s4.w};
#pragma unroll
      for (int r = 0; r < kMaxPer; ++r) {
        const int e = threadIdx.x + r * kGenThreads;
        if (e < d_c) {
#pragma unroll
          for (int u = 0; u < 4; ++u) o[r] = fmaf(w[u], sk[(j + u) * ld + e], o[r]);
        }
      }
    }
    for (; j < cnt; ++j) {
      const float w = sp[j] * s_scale[j];
#pragma unroll
      for (int r = 0; r < kMaxPer; ++r) {
        const int e = threadIdx.x + r * kGenThreads;
        if (e < d_c) o[r] = fmaf(w, sk[j * ld + e], o[r]);
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

}  // namespace csa
