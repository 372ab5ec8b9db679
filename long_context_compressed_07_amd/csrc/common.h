// Device-side helpers shared by the kernels: storage-format conversions and small reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "csa_internal.h"

namespace csa {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// OCP E4M3FN byte -> fp32 (exact). Encoding: sign, 4-bit exponent (bias 7), 3-bit fraction;
// exponent 0 is subnormal (fraction * 2^-9); S.1111.111 is NaN; no infinities.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t s = (b & 0x80u) << 24;
  const uint32_t e = (b >> 3) & 0xFu;
  const uint32_t f = b & 0x7u;
  float v;
  if (e == 0) {
    v = (float)f * 0.001953125f;  // 2^-9
  } else if (e == 0xF && f == 0x7) {
    v = __uint_as_float(0x7fc00000u);
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (f << 20));
  }
  return __uint_as_float(__float_as_uint(v) | s);
}

// fp32 -> OCP E4M3FN byte, round to nearest even, saturating to +-448 (NaN -> 0x7F).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  const uint32_t s = (u >> 24) & 0x80u;
  u &= 0x7fffffffu;
  if (u > 0x7f800000u) return 0x7Fu;
  const float a = __uint_as_float(u);
  if (a >= 448.0f) return s | 0x7Eu;
  if (a < 0.015625f) {                          // below 2^-6: subnormal grid of step 2^-9
    const uint32_t q = (uint32_t)rintf(a * 512.0f);  // 0..8 (8 is the smallest normal)
    return s | q;
  }
  const int e32 = (int)(u >> 23) - 127;         // -6 .. 8
  const uint32_t mant = u & 0x7fffffu;
  const uint32_t r = (mant + 0x7ffffu + ((mant >> 20) & 1u)) >> 20;  // 0..8, 8 carries
  return s | ((uint32_t)((e32 + 7) << 3) + r);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
  for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Number of entries of an m-fold compressed store visible to a query at absolute position pos.
__device__ __forceinline__ int64_t n_visible(int64_t pos, int m, int64_t n_entries) {
  const int64_t v = (pos + 1) / m;
  return v < n_entries ? (v < 0 ? 0 : v) : n_entries;
}

// Element e of row `row` of sequence b's c part, as fp32 (scale not applied).
__device__ __forceinline__ float load_c(const Store& st, int64_t b, int64_t row, int e) {
  const int64_t off = (b * st.rows + row) * st.ld_c + e;
  switch (st.dtype) {
    case CSA_F32: return static_cast<const float*>(st.c)[off];
    case CSA_BF16: return bf16_to_f32(static_cast<const uint16_t*>(st.c)[off]);
    default: return e4m3_to_f32(static_cast<const uint8_t*>(st.c)[off]);
  }
}

__device__ __forceinline__ float load_r(const Store& st, int64_t b, int64_t row, int e) {
  const int64_t off = (b * st.rows + row) * st.ld_r + e;
  if (st.dtype == CSA_F32) return static_cast<const float*>(st.r)[off];
  return bf16_to_f32(static_cast<const uint16_t*>(st.r)[off]);
}

__device__ __forceinline__ float row_scale(const Store& st, int64_t b, int64_t row) {
  return st.dtype == CSA_E4M3 ? st.scale[b * st.rows + row] : 1.0f;
}

__device__ __forceinline__ float load_vec(const void* p, int dtype, int64_t off) {
  switch (dtype) {
    case CSA_F32: return static_cast<const float*>(p)[off];
    case CSA_BF16: return bf16_to_f32(static_cast<const uint16_t*>(p)[off]);
    default: return e4m3_to_f32(static_cast<const uint8_t*>(p)[off]);
  }
}

}  // namespace csa
