// The slot scatter of a step's new tokens (and, optionally, the block-table entries they
// create), as a device function: pa_cache_write / pa_cache_append launch it on its own, and
// pa_decode_step runs it in the same launch as the decode planning.
//
// "Taming the Tail", "The Hidden Tax" -- each step stores only the new token's K/V;
// "vLLM PagedAttention" (tinycto), "1. Underlying Mechanism" -- a step writes the new token's
// entries and nothing else.  A workgroup moves a group of whole tokens: it reads the group's
// slots (and lengths) once into LDS, then each thread moves a 16-byte chunk of a key row
// (coalesced read, coalesced write into the K pool) and value elements into the transposed V
// blocks (lanes in row order, so neighbouring lanes' elements share cache lines).
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

// Workgroup wg writes tokens [wg * tok_per_wg, ...).  Each round first requests its key
// chunks and value elements, then (first round) the group's slots and lengths -- both bus
// requests issued back to back, one round trip per workgroup when they live in host memory,
// overlapping the HBM loads -- and then stores.  Keys move as 16-byte chunks (a key row is
// contiguous in the pool).  Values move one element per lane: a token's value row becomes a
// column of the transposed V block, so consecutive lanes take consecutive rows d and each
// store instruction covers a few whole cache lines of the block rather than one element in
// each of 64 lines.
template <typename T>
__device__ __forceinline__ void cache_write_wg(const CacheWriteArgs& a, int64_t wg) {
  constexpr int VEC = 16 / sizeof(T);
  static_assert(kWriteChunksPerThread == 1, "one key chunk and VEC value elements per thread");
  typedef typename std::conditional<sizeof(T) == 2, uint32_t, T>::type Wide;
  // Per token of the group: physical block (-1: padding or outside the pool, not written),
  // offset in it, length after the step.
  __shared__ int32_t s_blk[kMaxTokPerWG], s_off[kMaxTokPerWG], s_len[kMaxTokPerWG];
  const int64_t t0 = wg * a.tok_per_wg;
  if (t0 >= a.T) return;  // uniform over the workgroup
  const int ntok = static_cast<int>(a.T - t0 < a.tok_per_wg ? a.T - t0 : a.tok_per_wg);
  const int D = a.D, B = a.B, Hkv = a.Hkv;
  // Indices within the group fit 32 bits: at most kMaxTokPerWG tokens of Hkv * D elements.
  const int per_row = D / VEC;
  const int row_elems = Hkv * D;  // a token's elements
  const int per_token = per_row * Hkv;
  const int total = ntok * per_token;
  const T* key = static_cast<const T*>(a.key) + t0 * row_elems;
  const T* value = static_cast<const T*>(a.value) + t0 * row_elems;
  T* k_cache = static_cast<T*>(a.k_cache);
  T* v_cache = static_cast<T*>(a.v_cache);
  const TablePatch& tp = a.tp;
  for (int base = 0; base < total; base += kWriteChunksPerWG) {
    const int j = base + static_cast<int>(threadIdx.x);  // this thread's key chunk
    uint4 kv{};
    if (j < total) kv = *reinterpret_cast<const uint4*>(key + static_cast<int64_t>(j) * VEC);
    // Value elements in full registers (16-bit halves packed into one register would make
    // each load wait for the previous one); a lane past the end re-reads element 0.
    Wide vv[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int i = base * VEC + static_cast<int>(threadIdx.x) + e * kWriteThreads;
      vv[e] = static_cast<Wide>(value[i < total * VEC ? i : 0]);
    }
    if (base == 0) {
      if (static_cast<int>(threadIdx.x) < ntok) {
        const int32_t t = static_cast<int32_t>(t0) + static_cast<int32_t>(threadIdx.x);
        const int32_t* lp = tp.tables ? tp.ctx_lens + t / tp.tokens_each : nullptr;
        const int32_t sl = ld_step(a.slots + t, a.sys);
        const int32_t ln = lp ? ld_step(lp, a.sys) : 0;
        const bool ok = sl >= 0 && sl < a.n_slots;
        s_blk[threadIdx.x] = ok ? sl / B : -1;
        s_off[threadIdx.x] = ok ? sl % B : 0;
        s_len[threadIdx.x] = ln;
      }
      __syncthreads();
    }
    if (j < total) {
      const int k = j / per_token;
      const int rem = j - k * per_token;
      const int h = rem / per_row, c = rem - h * per_row;
      const int64_t p = s_blk[k];
      if (p >= 0) {
        const int o = s_off[k];
        if (tp.tables && c == 0 && h == 0) {
          // The token's logical block now lives in physical block p.  Tokens of one sequence
          // that share a block write the same value.
          const int64_t t = t0 + k;
          const int64_t r = t / tp.tokens_each;
          const int64_t pos = static_cast<int64_t>(s_len[k]) - tp.tokens_each + t % tp.tokens_each;
          if (pos >= 0 && pos < static_cast<int64_t>(tp.max_blocks) * B)
            tp.tables[r * tp.max_blocks + pos / B] = static_cast<int32_t>(p);
        }
        // Non-temporal, like the V elements below: the new rows are read once, by the next
        // kernel, and leave the L2 first instead of crowding the lines other work keeps
        // (decode step after the write: Llama-3-70B-shaped batch 0.2852-0.2869 -> 0.279-0.28 ms).
        __builtin_nontemporal_store(__builtin_bit_cast(u32x4, kv), reinterpret_cast<u32x4*>(
            k_cache + ((p * Hkv + h) * B + o) * D + static_cast<int64_t>(c) * VEC));
      }
    }
    // Element i = (token k, head h, row d); the next one this thread takes is kWriteThreads on.
    int i = base * VEC + static_cast<int>(threadIdx.x);
    int k = i / row_elems;
    int h = (i - k * row_elems) / D;
    int d = i - k * row_elems - h * D;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (i >= total * VEC) break;
      const int64_t p = s_blk[k];
      if (p >= 0)
        __builtin_nontemporal_store(static_cast<T>(vv[e]), &v_cache[((p * Hkv + h) * D + d) * B + s_off[k]]);
      i += kWriteThreads;
      d += kWriteThreads;
      while (d >= D) {
        d -= D;
        if (++h == Hkv) {
          h = 0;
          ++k;
        }
      }
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
__host__ __device__ inline int64_t cache_write_wgs(const CacheWriteArgs& w) {
  return (w.T + w.tok_per_wg - 1) / w.tok_per_wg;
}

}  // namespace pa
