// Matrix-core throughput probe (include/pa_probe.h): back-to-back independent bf16 MFMAs.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Each wave keeps NACC accumulators, so no instruction waits on the one before it; the
// operands stay in registers (no memory traffic in the loop).  Every lane folds its
// accumulators into one word of sink so nothing is removed.
template <int NACC>
__global__ __launch_bounds__(512) void mfma16_loop(int iters, float* sink) {
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = static_cast<__bf16>(static_cast<float>((threadIdx.x + j) & 7) * 0.125f);
    b[j] = static_cast<__bf16>(static_cast<float>((threadIdx.x * 3 + j) & 7) * 0.0625f);
  }
  f32x4 acc[NACC];
#pragma unroll
  for (int k = 0; k < NACC; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < NACC; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NACC; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

template <int NACC>
__global__ __launch_bounds__(512) void mfma32_loop(int iters, float* sink) {
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = static_cast<__bf16>(static_cast<float>((threadIdx.x + j) & 7) * 0.125f);
    b[j] = static_cast<__bf16>(static_cast<float>((threadIdx.x * 3 + j) & 7) * 0.0625f);
  }
  f32x16 acc[NACC];
#pragma unroll
  for (int k = 0; k < NACC; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < NACC; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NACC; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" int32_t pa_probe_mfma(int32_t shape, int32_t workgroups, int32_t waves_per_wg,
                                 int32_t iters, float* sink, double* flops, void* stream) {
  if (!sink || !flops || workgroups < 1 || workgroups > 65536 || iters < 1 ||
      (waves_per_wg != 1 && waves_per_wg != 2 && waves_per_wg != 4 && waves_per_wg != 8) ||
      (shape != 16 && shape != 32))
    return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int threads = 64 * waves_per_wg;
  const double waves = static_cast<double>(workgroups) * waves_per_wg;
  if (shape == 16) {
    constexpr int kAcc = 8;  // 16 x 16 x 32 x 2 flop each
    hipLaunchKernelGGL(mfma16_loop<kAcc>, dim3(workgroups), dim3(threads), 0, st, iters, sink);
    *flops = waves * iters * kAcc * (16.0 * 16 * 32 * 2);
  } else {
    constexpr int kAcc = 4;  // 32 x 32 x 16 x 2 flop each
    hipLaunchKernelGGL(mfma32_loop<kAcc>, dim3(workgroups), dim3(threads), 0, st, iters, sink);
    *flops = waves * iters * kAcc * (32.0 * 32 * 16 * 2);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}
