// Cache write (slot scatter) and copy-on-write block copy on gfx950.
//
// Cache write: "Taming the Tail", "The Hidden Tax" -- each step stores only the new token's
// K/V; "vLLM PagedAttention" (tinycto), "1. Underlying Mechanism" -- a step writes the new
// token's entries and nothing else.  Block copy: KV-cache chapter, "PagedAttention: borrowing virtual memory" -- a
// writer into a shared block first gets a private copy.
//
// Both are pure bit copies and HBM-bound.  One thread moves one 16-byte chunk of a token's
// key row (coalesced read, coalesced write into the K pool); the same thread scatters the
// matching value chunk into the transposed V block (one element every B elements).

#include "device_common.h"

namespace pa {

// Resident block table to patch (pa_cache_append); tables == nullptr for a plain cache write.
struct TablePatch {
  int32_t* tables;
  const int32_t* ctx_lens;
  int tokens_each, max_blocks;
};

template <typename T>
__global__ __launch_bounds__(256) void cache_write_kernel(
    const T* __restrict__ key, const T* __restrict__ value, T* __restrict__ k_cache,
    T* __restrict__ v_cache, const int32_t* __restrict__ slots, int64_t n_chunks, int Hkv,
    int D, int B, int64_t n_slots, TablePatch tp) {
  constexpr int VEC = 16 / sizeof(T);
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_chunks) return;
  const int per_row = D / VEC;
  const int c = static_cast<int>(i % per_row);
  const int64_t th = i / per_row;
  const int h = static_cast<int>(th % Hkv);
  const int64_t t = th / Hkv;
  const int32_t slot = slots[t];
  if (slot < 0 || slot >= n_slots) return;  // padding or out of the pool: not written
  const int64_t p = slot / B;
  const int o = slot % B;
  if (tp.tables && c == 0 && h == 0) {
    // The token's logical block now lives in physical block p.  Tokens of one sequence that
    // share a block write the same value.
    const int64_t r = t / tp.tokens_each;
    const int64_t pos = static_cast<int64_t>(tp.ctx_lens[r]) - tp.tokens_each + t % tp.tokens_each;
    if (pos >= 0 && pos < static_cast<int64_t>(tp.max_blocks) * B)
      tp.tables[r * tp.max_blocks + pos / B] = static_cast<int32_t>(p);
  }
  const int64_t src = (t * Hkv + h) * D + static_cast<int64_t>(c) * VEC;

  const uint4 kv = *reinterpret_cast<const uint4*>(key + src);
  *reinterpret_cast<uint4*>(k_cache + ((p * Hkv + h) * B + o) * D + static_cast<int64_t>(c) * VEC) = kv;

  const uint4 vv = *reinterpret_cast<const uint4*>(value + src);
  T vals[VEC];
  __builtin_memcpy(vals, &vv, 16);
  T* dst = v_cache + ((p * Hkv + h) * D + static_cast<int64_t>(c) * VEC) * B + o;
#pragma unroll
  for (int e = 0; e < VEC; ++e) dst[static_cast<int64_t>(e) * B] = vals[e];
}

// One workgroup per pair; each copies the whole block (all kv-heads and slots) of both pools.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint4* __restrict__ k_cache,
                                                          uint4* __restrict__ v_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int num_blocks, int64_t block_vecs) {
  const int64_t pr = blockIdx.x;
  const int32_t src = pairs[2 * pr];
  const int32_t dst = pairs[2 * pr + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const uint4* ks = k_cache + src * block_vecs;
  const uint4* vs = v_cache + src * block_vecs;
  uint4* kd = k_cache + dst * block_vecs;
  uint4* vd = v_cache + dst * block_vecs;
  for (int64_t i = threadIdx.x; i < block_vecs; i += blockDim.x) {
    const uint4 a = ks[i];
    const uint4 b = vs[i];
    kd[i] = a;
    vd[i] = b;
  }
}

static pa_status check_pool_shape(const char* who, int32_t Hkv, int32_t D, int32_t B,
                                  int32_t dtype) {
  if (elem_bytes(dtype) == 0) return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d not supported", who, dtype);
  if (Hkv <= 0) return fail(PA_ERR_INVALID_ARG, "%s: Hkv %d <= 0", who, Hkv);
  if (D != 64 && D != 128) return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", who, D);
  if (B != 16 && B != 32) return fail(PA_ERR_UNSUPPORTED, "%s: block size %d not in {16, 32}", who, B);
  return PA_OK;
}

static pa_status launch_cache_write(const char* who, const void* key, const void* value,
                                    void* k_cache, void* v_cache, const int32_t* slot_mapping,
                                    int32_t T, int32_t Hkv, int32_t D, int32_t B,
                                    int32_t num_blocks, int32_t dtype, const TablePatch& tp,
                                    void* stream) {
  const int eb = elem_bytes(dtype);
  const int64_t n_chunks = static_cast<int64_t>(T) * Hkv * (D * eb / 16);
  const int64_t n_slots = static_cast<int64_t>(num_blocks) * B;
  const dim3 grid(static_cast<unsigned>((n_chunks + 255) / 256));
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == PA_DTYPE_F32)
    hipLaunchKernelGGL(cache_write_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(key), static_cast<const float*>(value),
                       static_cast<float*>(k_cache), static_cast<float*>(v_cache), slot_mapping,
                       n_chunks, Hkv, D, B, n_slots, tp);
  else
    hipLaunchKernelGGL(cache_write_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(key), static_cast<const uint16_t*>(value),
                       static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache),
                       slot_mapping, n_chunks, Hkv, D, B, n_slots, tp);
  return launch_status(who);
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_cache_write(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int32_t* slot_mapping, int32_t T,
                                    int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks,
                                    int32_t dtype, void* stream) {
  if (pa_status st = check_pool_shape("pa_cache_write", Hkv, D, B, dtype)) return st;
  if (T < 0 || num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "pa_cache_write: T %d, num_blocks %d", T, num_blocks);
  if (T == 0) return ok();
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "pa_cache_write: NULL pointer");
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARG, "pa_cache_write: pointers must be 16-byte aligned");
  return launch_cache_write("pa_cache_write", key, value, k_cache, v_cache, slot_mapping, T, Hkv,
                            D, B, num_blocks, dtype, TablePatch{nullptr, nullptr, 1, 0}, stream);
}

extern "C" pa_status pa_cache_append(const void* key, const void* value, void* k_cache,
                                     void* v_cache, const int32_t* slot_mapping, int32_t S,
                                     int32_t tokens_each, int32_t* block_tables,
                                     int32_t max_blocks, const int32_t* ctx_lens, int32_t Hkv,
                                     int32_t D, int32_t B, int32_t num_blocks, int32_t dtype,
                                     void* stream) {
  if (pa_status st = check_pool_shape("pa_cache_append", Hkv, D, B, dtype)) return st;
  if (S < 0 || tokens_each < 0 || num_blocks <= 0 || max_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "pa_cache_append: S %d, tokens_each %d, num_blocks %d, max_blocks %d",
                S, tokens_each, num_blocks, max_blocks);
  const int64_t T = static_cast<int64_t>(S) * tokens_each;
  if (T > INT32_MAX) return fail(PA_ERR_INVALID_ARG, "pa_cache_append: S * tokens_each too large");
  if (T == 0) return ok();
  if (!key || !value || !k_cache || !v_cache || !slot_mapping || !block_tables || !ctx_lens)
    return fail(PA_ERR_INVALID_ARG, "pa_cache_append: NULL pointer");
  if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARG, "pa_cache_append: pointers must be 16-byte aligned");
  return launch_cache_write("pa_cache_append", key, value, k_cache, v_cache, slot_mapping,
                            static_cast<int32_t>(T), Hkv, D, B, num_blocks, dtype,
                            TablePatch{block_tables, ctx_lens, tokens_each, max_blocks}, stream);
}

extern "C" pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t P,
                                    int32_t num_blocks, int32_t Hkv, int32_t D, int32_t B,
                                    int32_t dtype, void* stream) {
  if (pa_status st = check_pool_shape("pa_copy_blocks", Hkv, D, B, dtype)) return st;
  if (P < 0 || num_blocks <= 0) return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: P %d, num_blocks %d", P, num_blocks);
  if (P == 0) return ok();
  if (!k_cache || !v_cache || !pairs) return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: NULL pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARG, "pa_copy_blocks: pools must be 16-byte aligned");
  const int64_t block_vecs = static_cast<int64_t>(Hkv) * B * D * elem_bytes(dtype) / 16;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(P), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(k_cache), static_cast<uint4*>(v_cache), pairs, num_blocks,
                     block_vecs);
  return launch_status("pa_copy_blocks");
}
