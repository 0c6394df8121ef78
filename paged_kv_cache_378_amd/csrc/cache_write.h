// The slot scatter of a step's new tokens (and, optionally, the block-table entries they
// create), as a device function: pa_cache_write / pa_cache_append launch it on its own, and
// pa_decode_step runs it in the same launch as the decode planning.
//
// "Taming the Tail", "The Hidden Tax" -- each step stores only the new token's K/V;
// "vLLM PagedAttention" (tinycto), "1. Underlying Mechanism" -- a step writes the new token's
// entries and nothing else.  A workgroup moves a group of whole tokens: it reads the group's
// slots (and lengths) once into LDS, then each thread moves 16-byte chunks of key rows
// (coalesced read, coalesced write into the K pool) and scatters the matching value chunks
// into the transposed V blocks (one element every B elements).
#pragma once

#include "device_common.h"

namespace pa {

// Resident block table to patch; tables == nullptr for a plain cache write.
struct TablePatch {
  int32_t* tables;
  const int32_t* ctx_lens;  // lengths after the step
  int tokens_each, max_blocks;
};

// Reads a step's slot or length.  With `sys` set the value may live in page-locked host memory
// that the host rewrites between launches: a system-scope load fetches it past the GPU caches,
// so a line cached by an earlier launch is never reused.
__device__ __forceinline__ int32_t ld_step(const int32_t* p, bool sys) {
  return sys ? __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) : *p;
}

struct CacheWriteArgs {
  const void* key;
  const void* value;
  void* k_cache;
  void* v_cache;
  const int32_t* slots;
  int64_t T;         // tokens
  int Hkv, D, B;
  int tok_per_wg;    // tokens per workgroup (write_tokens_per_wg)
  int64_t n_slots;   // num_blocks * B
  TablePatch tp;
  bool sys;          // slots / tp.ctx_lens may be page-locked host memory (see ld_step)
};

constexpr int kWriteThreads = 256;
constexpr int kWriteChunksPerThread = 1;  // 16-byte chunks per thread per round
constexpr int kWriteChunksPerWG = kWriteThreads * kWriteChunksPerThread;
constexpr int kMaxTokPerWG = 64;

// Tokens per workgroup: as many whole tokens (all kv-heads) as one round of the workgroup
// moves, at least one.
inline int write_tokens_per_wg(int Hkv, int D, int elt_bytes) {
  const int64_t per_token = static_cast<int64_t>(Hkv) * D * elt_bytes / 16;
  const int64_t t = kWriteChunksPerWG / per_token;
  return static_cast<int>(t < 1 ? 1 : (t > kMaxTokPerWG ? kMaxTokPerWG : t));
}

// Workgroup wg writes tokens [wg * tok_per_wg, ...).  Each round first requests its key and
// value chunks, then (first round) the group's slots and lengths -- one request per
// workgroup, so with the slots in host memory the bus round trip is paid once and overlaps
// the chunk loads -- and then stores.
template <typename T>
__device__ __forceinline__ void cache_write_wg(const CacheWriteArgs& a, int64_t wg) {
  constexpr int VEC = 16 / sizeof(T);
  __shared__ int32_t s_slot[kMaxTokPerWG], s_len[kMaxTokPerWG];
  const int64_t t0 = wg * a.tok_per_wg;
  if (t0 >= a.T) return;  // uniform over the workgroup
  const int ntok = static_cast<int>(a.T - t0 < a.tok_per_wg ? a.T - t0 : a.tok_per_wg);
  const int D = a.D, B = a.B, Hkv = a.Hkv;
  const int per_row = D / VEC;
  const int64_t per_token = static_cast<int64_t>(per_row) * Hkv;
  const int64_t total = ntok * per_token;
  const T* key = static_cast<const T*>(a.key);
  const T* value = static_cast<const T*>(a.value);
  T* k_cache = static_cast<T*>(a.k_cache);
  T* v_cache = static_cast<T*>(a.v_cache);
  const TablePatch& tp = a.tp;
  for (int64_t base = 0; base < total; base += kWriteChunksPerWG) {
    uint4 kv[kWriteChunksPerThread], vv[kWriteChunksPerThread];
#pragma unroll
    for (int u = 0; u < kWriteChunksPerThread; ++u) {
      const int64_t j = base + threadIdx.x + u * kWriteThreads;
      if (j < total) {
        const int64_t src = (t0 * Hkv) * D + j * VEC;  // token-major rows: chunk j in order
        kv[u] = *reinterpret_cast<const uint4*>(key + src);
        vv[u] = *reinterpret_cast<const uint4*>(value + src);
      }
    }
    if (base == 0) {
      if (static_cast<int>(threadIdx.x) < ntok) {
        const int64_t t = t0 + threadIdx.x;
        s_slot[threadIdx.x] = ld_step(a.slots + t, a.sys);
        if (tp.tables) s_len[threadIdx.x] = ld_step(tp.ctx_lens + t / tp.tokens_each, a.sys);
      }
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < kWriteChunksPerThread; ++u) {
      const int64_t j = base + threadIdx.x + u * kWriteThreads;
      if (j >= total) continue;
      const int k = static_cast<int>(j / per_token);
      const int rem = static_cast<int>(j - k * per_token);
      const int h = rem / per_row, c = rem - h * per_row;
      const int32_t slot = s_slot[k];
      if (slot < 0 || slot >= a.n_slots) continue;  // padding or out of the pool: not written
      const int64_t p = slot / B;
      const int o = slot % B;
      if (tp.tables && c == 0 && h == 0) {
        // The token's logical block now lives in physical block p.  Tokens of one sequence
        // that share a block write the same value.
        const int64_t t = t0 + k;
        const int64_t r = t / tp.tokens_each;
        const int64_t pos = static_cast<int64_t>(s_len[k]) - tp.tokens_each + t % tp.tokens_each;
        if (pos >= 0 && pos < static_cast<int64_t>(tp.max_blocks) * B)
          tp.tables[r * tp.max_blocks + pos / B] = static_cast<int32_t>(p);
      }
      *reinterpret_cast<uint4*>(k_cache + ((p * Hkv + h) * B + o) * D + static_cast<int64_t>(c) * VEC) = kv[u];
      T vals[VEC];
      __builtin_memcpy(vals, &vv[u], 16);
      T* dst = v_cache + ((p * Hkv + h) * D + static_cast<int64_t>(c) * VEC) * B + o;
#pragma unroll
      for (int e = 0; e < VEC; ++e) dst[static_cast<int64_t>(e) * B] = vals[e];
    }
  }
}

inline CacheWriteArgs make_cache_write_args(const void* key, const void* value, void* k_cache,
                                            void* v_cache, const int32_t* slots, int32_t T,
                                            int32_t Hkv, int32_t D, int32_t B,
                                            int32_t num_blocks, int32_t dtype,
                                            const TablePatch& tp) {
  CacheWriteArgs w{};
  w.key = key;
  w.value = value;
  w.k_cache = k_cache;
  w.v_cache = v_cache;
  w.slots = slots;
  w.T = T;
  w.Hkv = Hkv;
  w.D = D;
  w.B = B;
  w.tok_per_wg = write_tokens_per_wg(Hkv, D, elem_bytes(dtype));
  w.n_slots = static_cast<int64_t>(num_blocks) * B;
  w.tp = tp;
  return w;
}

// Workgroups of a cache write.
inline int64_t cache_write_wgs(const CacheWriteArgs& w) {
  return (w.T + w.tok_per_wg - 1) / w.tok_per_wg;
}

}  // namespace pa
