// Device helpers shared by the gfx950 kernels of libpa.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa.h"
#include "pa_status.h"

namespace pa {

constexpr int kWave = 64;  // CDNA wavefront width

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// (1, 1): the second operand of a dot2 that sums a pair of bf16 values into an fp32 total
constexpr bf16x2 kOnes2 = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};

// 16-byte load of K/V pool data.  Each byte is read once per call, so the load is marked
// non-temporal (measured ~2% faster on the Llama-3-70B-shaped decode batch).
__device__ __forceinline__ bf16x8 ld_kv16(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

// The same load without the non-temporal hint, for K/V lines other workgroups will read again
// soon (blocks shared by several sequences).
__device__ __forceinline__ bf16x8 ld_kv16_keep(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

// Round-to-nearest-even float -> bf16 bits (NaN stays a quiet NaN with its sign).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static float load(const float* p) { return *p; }
  __device__ static float to_f32(float v) { return v; }
  __device__ static float from_f32(float v) { return v; }
};
template <> struct Elem<uint16_t> {  // bf16 carried as raw bits
  __device__ static float to_f32(uint16_t v) { return bf16_to_f32(v); }
  __device__ static uint16_t from_f32(float v) { return f32_to_bf16(v); }
};

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, kWave); }

// NaN-propagating max (llvm.maximum; v_maximum_f32 / v_maximum3_f32 on gfx950).  fmaxf is
// IEEE maxNum, which first canonicalizes every operand the compiler cannot prove canonical --
// one extra VALU instruction per matrix-core result it is applied to.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }

// Max over lane pairs (i, i ^ 16) and (i, i ^ 32) with gfx950's row-swap instructions
// (VALU, no LDS round trip as a generic shuffle has).  Swapping odd 16-lane rows of one copy of
// v with even rows of another leaves every lane holding its own value and its xor-16
// partner's; the 32-lane swap does the same for the xor-32 partner.
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Chunk permutation for K tiles staged in LDS (rows of D bf16 = D/8 16-byte chunks): chunk c
// of key row `key` is stored at chunk c ^ kswz(key).  The matrix-core operand read has 16
// lanes read the same chunk of 16 keys that differ in bits 0-1 and 3-4; without the
// permutation keys 16 apart land in the same LDS banks.  kswz maps those keys to distinct values.
template <int D>
__device__ __forceinline__ int kswz(int key) {
  constexpr int kMask = D / 8 - 1;  // chunks per row - 1
  return ((key & 3) | (((key >> 3) & 3) << 2)) & kMask;
}

// 2^x by the hardware instruction alone: exact at -inf (0), results below 2^-126 flush to 0
// (harmless for softmax weights, which are summed against weights near 1).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Agent-scope (device-coherent) 4-byte accesses: on a multi-XCD device they are performed past
// the XCD-local L2, so values one workgroup stores are seen by a workgroup on another XCD
// without a whole-cache write-back or invalidation.
__device__ __forceinline__ void st_agent(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Two consecutive floats (8-byte aligned) in one agent-scope store.
__device__ __forceinline__ void st_agent2(float* p, float x, float y) {
  const uint64_t v = static_cast<uint64_t>(__float_as_uint(x)) | (static_cast<uint64_t>(__float_as_uint(y)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4): lane i writes at
// lds + 16 i, where lds must be the same for the whole wave.  Asynchronous: counted by vmcnt.
// The builtin exists only for the device; the host pass sees an empty body.
__device__ __forceinline__ void load16_to_lds(const void* src, void* lds) {
#if __HIP_DEVICE_COMPILE__
  __builtin_amdgcn_load_to_lds(const_cast<void*>(src), (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
#endif
}

// Workgroup barrier for data exchanged through LDS only: the wave's LDS operations complete
// before it, its global stores may still be in flight.  (__syncthreads also waits for those:
// ~1 us at each barrier that follows a pass of stores.)
__device__ __forceinline__ void lds_barrier() {
#if __HIP_DEVICE_COMPILE__
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#endif
}

// Index of this wave in its workgroup, as a wave-uniform (scalar) value.  Without the
// readfirstlane the compiler treats threadIdx.x / 64 as divergent, so every loop bounded by
// it becomes exec-masked vector control flow instead of a scalar loop.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
}

// Error check after a launch.
inline pa_status launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline int elem_bytes(int32_t dtype) {
  return dtype == PA_DTYPE_F32 ? 4 : dtype == PA_DTYPE_BF16 ? 2 : 0;
}

}  // namespace pa
