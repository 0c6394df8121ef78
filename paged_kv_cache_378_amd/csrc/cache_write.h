// The slot scatter of a step's new tokens (and, optionally, the block-table entries they
// create), as a device function: pa_cache_write / pa_cache_append launch it on its own, and
// pa_decode_step runs it in the same launch as the decode planning.
//
// "Taming the Tail", "The Hidden Tax" -- each step stores only the new token's K/V;
// "vLLM PagedAttention" (tinycto), "1. Underlying Mechanism" -- a step writes the new token's
// entries and nothing else.  One thread moves one 16-byte chunk of a token's key row (coalesced
// read, coalesced write into the K pool) and scatters the matching value chunk into the
// transposed V block (one element every B elements).
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
  int64_t n_chunks;  // tokens * Hkv * (16-byte chunks per row)
  int Hkv, D, B;
  int64_t n_slots;   // num_blocks * B
  TablePatch tp;
  bool sys;          // slots / tp.ctx_lens may be page-locked host memory (see ld_step)
};

constexpr int kWriteThreads = 256;

template <typename T>
__device__ __forceinline__ void cache_write_chunk(const CacheWriteArgs& a, int64_t i) {
  constexpr int VEC = 16 / sizeof(T);
  if (i >= a.n_chunks) return;
  const int D = a.D, B = a.B, Hkv = a.Hkv;
  const int per_row = D / VEC;
  const int c = static_cast<int>(i % per_row);
  const int64_t th = i / per_row;
  const int h = static_cast<int>(th % Hkv);
  const int64_t t = th / Hkv;
  const int64_t src = (t * Hkv + h) * D + static_cast<int64_t>(c) * VEC;
  const T* key = static_cast<const T*>(a.key);
  const T* value = static_cast<const T*>(a.value);
  T* k_cache = static_cast<T*>(a.k_cache);
  T* v_cache = static_cast<T*>(a.v_cache);
  // The token's data, its slot and (for the table patch) its sequence's length are all
  // requested before any of them is used: with the slots and lengths in host memory the
  // step pays one round trip over the bus, not two.
  const uint4 kv = *reinterpret_cast<const uint4*>(key + src);
  const uint4 vv = *reinterpret_cast<const uint4*>(value + src);
  const TablePatch& tp = a.tp;
  const bool patch = tp.tables && c == 0 && h == 0;
  const int64_t r = t / tp.tokens_each;
  const int32_t slot = ld_step(a.slots + t, a.sys);
  const int32_t len = patch ? ld_step(tp.ctx_lens + r, a.sys) : 0;
  if (slot < 0 || slot >= a.n_slots) return;  // padding or out of the pool: not written
  const int64_t p = slot / B;
  const int o = slot % B;
  if (patch) {
    // The token's logical block now lives in physical block p.  Tokens of one sequence that
    // share a block write the same value.
    const int64_t pos = static_cast<int64_t>(len) - tp.tokens_each + t % tp.tokens_each;
    if (pos >= 0 && pos < static_cast<int64_t>(tp.max_blocks) * B)
      tp.tables[r * tp.max_blocks + pos / B] = static_cast<int32_t>(p);
  }
  *reinterpret_cast<uint4*>(k_cache + ((p * Hkv + h) * B + o) * D + static_cast<int64_t>(c) * VEC) = kv;

  T vals[VEC];
  __builtin_memcpy(vals, &vv, 16);
  T* dst = v_cache + ((p * Hkv + h) * D + static_cast<int64_t>(c) * VEC) * B + o;
#pragma unroll
  for (int e = 0; e < VEC; ++e) dst[static_cast<int64_t>(e) * B] = vals[e];
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
  w.n_chunks = static_cast<int64_t>(T) * Hkv * (D * elem_bytes(dtype) / 16);
  w.Hkv = Hkv;
  w.D = D;
  w.B = B;
  w.n_slots = static_cast<int64_t>(num_blocks) * B;
  w.tp = tp;
  return w;
}

}  // namespace pa
