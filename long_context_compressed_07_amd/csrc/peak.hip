// Measured dense bf16 MFMA throughput of the device, reported beside the datasheet peak when
// kernels are rated against the matrix-core roofline. Every wave runs kChains independent
// accumulation chains of mfma_f32_32x32x16_bf16 (32 x 32 x 16 x 2 flops each) on operands held in
// registers; the loop touches no memory, so the rate is the matrix cores' issue rate.
#include "common.h"
#include "csa_internal.h"

namespace csa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;
constexpr int kPeakThreads = 256;
constexpr int kPeakBlocks = 768;    // 3 per CU: one pass over 256 CUs (3 waves per SIMD fit)

__global__ void __launch_bounds__(kPeakThreads) peak_mfma_kernel(int iters, float* sink) {
  const uint32_t t = threadIdx.x;
  // Finite operands near 1.0 (bf16 bit patterns 0x3f80 + small mantissa offsets).
  const bf16x8 a = __builtin_bit_cast(
      bf16x8, make_uint4(0x3f803f80u + (t & 15u), 0x3f803f81u, 0x3f823f80u, 0x3f803f83u));
  const bf16x8 b = __builtin_bit_cast(
      bf16x8, make_uint4(0x3f843f80u, 0x3f803f85u + (t & 7u), 0x3f803f80u, 0x3f863f80u));
  floatx16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) acc[c] = floatx16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int c = 0; c < kChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  // One value per wave keeps every chain live.
  if ((t & (kWave - 1)) == 0) sink[blockIdx.x * (kPeakThreads / kWave) + t / kWave] = s;
}

}  // namespace

int peak_sink_floats() { return kPeakBlocks * (kPeakThreads / kWave); }

hipError_t peak_mfma_bf16(int iters, float* sink, double* tflops, hipStream_t s) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) {
    peak_mfma_kernel<<<kPeakBlocks, kPeakThreads, 0, s>>>(iters / 10 + 1, sink);   // warm-up
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  if (e == hipSuccess) {
    peak_mfma_kernel<<<kPeakBlocks, kPeakThreads, 0, s>>>(iters, sink);
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e == hipSuccess) {
    const double flops = (double)kPeakBlocks * (kPeakThreads / kWave) * iters * kChains * 32.0 *
                         32.0 * 16.0 * 2.0;
    *tflops = ms > 0.f ? flops / (ms * 1e-3) / 1e12 : 0.0;
  }
  if (e0 != nullptr) hipEventDestroy(e0);
  if (e1 != nullptr) hipEventDestroy(e1);
  return e;
}

}  // namespace csa
