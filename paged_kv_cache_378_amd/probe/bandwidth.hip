// HBM read-bandwidth probes (include/pa_probe.h): a streaming read and a gather of 4 KiB chunks.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pa_probe.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kChunkVecs = 4096 / 16;  // 16-byte vectors per 4 KiB chunk

// Iteration k of a thread reads vectors i + (k * L + l) * nthr, l < L: L loads in flight per
// lane, consecutive threads on consecutive vectors.  n is a multiple of L * nthr.
template <int L>
__global__ __launch_bounds__(kThreads) void read_stream(const u32x4* __restrict__ p, size_t n,
                                                        uint32_t* sink) {
  const size_t nthr = static_cast<size_t>(gridDim.x) * kThreads;
  const size_t tid = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0;
  for (size_t i = tid; i < n; i += L * nthr) {
    u32x4 v[L];
#pragma unroll
    for (int l = 0; l < L; ++l) v[l] = __builtin_nontemporal_load(p + i + l * nthr);
#pragma unroll
    for (int l = 0; l < L; ++l) acc ^= v[l][0] ^ v[l][1] ^ v[l][2] ^ v[l][3];
  }
  sink[tid] = acc;
}

// Wave w takes list entries w * C, w * C + 1, ... (C per iteration), then jumps by all waves.
template <int C>
__global__ __launch_bounds__(kThreads) void read_gather(const u32x4* __restrict__ p,
                                                        const int32_t* __restrict__ order,
                                                        int nchunks, uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int wave = (blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int nwaves = (gridDim.x * kThreads) >> 6;
  uint32_t acc = 0;
  for (int j0 = wave * C; j0 < nchunks; j0 += nwaves * C) {
    u32x4 v[C][4];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      int id = order[min(j0 + c, nchunks - 1)];
      id = id < 0 ? 0 : (id >= nchunks ? nchunks - 1 : id);
      const u32x4* base = p + static_cast<size_t>(id) * kChunkVecs;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[c][k] = __builtin_nontemporal_load(base + k * 64 + lane);
    }
#pragma unroll
    for (int c = 0; c < C; ++c)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc ^= v[c][k][0] ^ v[c][k][3];
  }
  sink[blockIdx.x * kThreads + threadIdx.x] = acc;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int32_t launched() { return hipGetLastError() == hipSuccess ? 0 : -7; }

}  // namespace

extern "C" int32_t pa_probe_read_stream(const void* buf, size_t nbytes, int32_t workgroups,
                                        int32_t loads, uint32_t* sink, size_t* read_bytes,
                                        void* stream) {
  if (!buf || !sink || !read_bytes || !aligned16(buf) || workgroups < 1 || workgroups > 65536 ||
      (loads != 1 && loads != 2 && loads != 4 && loads != 8))
    return -1;
  const size_t step = static_cast<size_t>(workgroups) * kThreads * static_cast<size_t>(loads);
  const size_t n = nbytes / 16 / step * step;
  *read_bytes = n * 16;
  if (n == 0) return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4* p = static_cast<const u32x4*>(buf);
  switch (loads) {
    case 1: hipLaunchKernelGGL(read_stream<1>, dim3(workgroups), dim3(kThreads), 0, st, p, n, sink); break;
    case 2: hipLaunchKernelGGL(read_stream<2>, dim3(workgroups), dim3(kThreads), 0, st, p, n, sink); break;
    case 4: hipLaunchKernelGGL(read_stream<4>, dim3(workgroups), dim3(kThreads), 0, st, p, n, sink); break;
    case 8: hipLaunchKernelGGL(read_stream<8>, dim3(workgroups), dim3(kThreads), 0, st, p, n, sink); break;
    default: return -1;
  }
  return launched();
}

extern "C" int32_t pa_probe_read_gather(const void* buf, const int32_t* order, int32_t nchunks,
                                        int32_t per_wave, int32_t workgroups, uint32_t* sink,
                                        void* stream) {
  if (!buf || !order || !sink || !aligned16(buf) || nchunks < 1 || workgroups < 1 ||
      workgroups > 65536)
    return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const u32x4* p = static_cast<const u32x4*>(buf);
  switch (per_wave) {
    case 1: hipLaunchKernelGGL(read_gather<1>, dim3(workgroups), dim3(kThreads), 0, st, p, order, nchunks, sink); break;
    case 2: hipLaunchKernelGGL(read_gather<2>, dim3(workgroups), dim3(kThreads), 0, st, p, order, nchunks, sink); break;
    case 4: hipLaunchKernelGGL(read_gather<4>, dim3(workgroups), dim3(kThreads), 0, st, p, order, nchunks, sink); break;
    default: return -1;
  }
  return launched();
}
