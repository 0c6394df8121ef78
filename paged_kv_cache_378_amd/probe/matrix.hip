// Matrix-core throughput probe (include/pa_probe.h): back-to-back independent bf16 MFMAs, with
// the shader clock each workgroup ran at.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Operand set k of this lane.  Fixed: a sparse pattern (multiples of 1/8 and 1/16), the same
// for every k.  Random: bf16 words with random sign, exponent 2^-1 or 2^0 and mantissa (values
// of magnitude 0.5 .. 2, like unit-variance data), different for every lane and set, so
// consecutive instructions see unrelated bits.
__device__ inline void make_operands(bool random, int k, bf16x8& a, bf16x8& b) {
  if (!random) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[j] = static_cast<__bf16>(static_cast<float>((threadIdx.x + j) & 7) * 0.125f);
      b[j] = static_cast<__bf16>(static_cast<float>((threadIdx.x * 3 + j) & 7) * 0.0625f);
    }
    return;
  }
  u32x4 ua, ub;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t x = (blockIdx.x * 1024u + threadIdx.x) * 2654435761u ^ (k * 4 + j) * 0x9e3779b9u;
    x ^= x >> 15;
    x *= 0x2c1b3c6du;
    x ^= x >> 12;
    x *= 0x297a2d39u;
    x ^= x >> 15;
    const uint32_t y = x * 0x85ebca6bu ^ (x >> 13);
    // keep sign (bit 15) and mantissa (bits 0-6), exponent 126 or 127 from bit 7
    ua[j] = (x & 0x80ff80ffu) | 0x3f003f00u;
    ub[j] = (y & 0x80ff80ffu) | 0x3f003f00u;
  }
  a = __builtin_bit_cast(bf16x8, ua);
  b = __builtin_bit_cast(bf16x8, ub);
}

__device__ inline void record_clock(uint64_t* clocks, uint64_t t0, uint64_t r0) {
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (clocks && threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// Each wave keeps NACC accumulators, each with its own operand set, so no instruction waits on
// the one before it; the operands stay in registers (no memory traffic and no other
// instruction in the loop).  Every lane folds its accumulators into one word of sink so
// nothing is removed.
template <int NACC>
__global__ __launch_bounds__(512) void mfma16_loop(int iters, bool random, float* sink, uint64_t* clocks) {
  bf16x8 a[NACC], b[NACC];
  f32x4 acc[NACC];
#pragma unroll
  for (int k = 0; k < NACC; ++k) {
    make_operands(random, k, a[k], b[k]);
    acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < NACC; ++k) acc[k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[k], b[k], acc[k], 0, 0, 0);
  }
  record_clock(clocks, t0, r0);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NACC; ++k) s += acc[k][0] + acc[k][1] + acc[k][2] + acc[k][3];
  sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

template <int NACC>
__global__ __launch_bounds__(512) void mfma32_loop(int iters, bool random, float* sink, uint64_t* clocks) {
  bf16x8 a[NACC], b[NACC];
  f32x16 acc[NACC];
#pragma unroll
  for (int k = 0; k < NACC; ++k) {
    make_operands(random, k, a[k], b[k]);
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[k][e] = 0.f;
  }
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < NACC; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[k], acc[k], 0, 0, 0);
  }
  record_clock(clocks, t0, r0);
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < NACC; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  sink[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" int32_t pa_probe_mfma(int32_t shape, int32_t operands, int32_t workgroups,
                                 int32_t waves_per_wg, int32_t iters, float* sink, uint64_t* clocks,
                                 double* flops, void* stream) {
  if (!sink || !flops || workgroups < 1 || workgroups > 65536 || iters < 1 ||
      (waves_per_wg != 1 && waves_per_wg != 2 && waves_per_wg != 4 && waves_per_wg != 8) ||
      (shape != 16 && shape != 32) || (operands != 0 && operands != 1))
    return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int threads = 64 * waves_per_wg;
  const double waves = static_cast<double>(workgroups) * waves_per_wg;
  const bool random = operands == 1;
  if (shape == 16) {
    constexpr int kAcc = 8;  // 16 x 16 x 32 x 2 flop each
    hipLaunchKernelGGL(mfma16_loop<kAcc>, dim3(workgroups), dim3(threads), 0, st, iters, random, sink, clocks);
    *flops = waves * iters * kAcc * (16.0 * 16 * 32 * 2);
  } else {
    constexpr int kAcc = 4;  // 32 x 32 x 16 x 2 flop each
    hipLaunchKernelGGL(mfma32_loop<kAcc>, dim3(workgroups), dim3(threads), 0, st, iters, random, sink, clocks);
    *flops = waves * iters * kAcc * (32.0 * 32 * 16 * 2);
  }
  return hipGetLastError() == hipSuccess ? 0 : -7;
}
