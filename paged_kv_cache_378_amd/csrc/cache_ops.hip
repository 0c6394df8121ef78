// Cache write (slot scatter), copy-on-write block copy and swap copies on gfx950.
//
// Cache write: the device function in cache_write.h.  Block copy: KV-cache chapter,
// "PagedAttention: borrowing virtual memory" -- a writer into a shared block first gets a
// private copy.  Both are pure bit copies and HBM-bound.  Swap copies: "Taming the Tail",
// "Infrastructure Scale" -- a paused request's KV-cache moves to CPU RAM and back; whole
// blocks between the pools and page-locked host memory, bound by the host link.

#include "cache_write.h"
#include "device_common.h"
#include "host_memory.h"

namespace pa {

template <typename T>
__global__ __launch_bounds__(kWriteThreads) void cache_write_kernel(CacheWriteArgs a) {
  cache_write_wg<T>(a, blockIdx.x);
}

// Prefill-sized writes (many tokens, usually consecutive slots of each sequence): a workgroup
// takes kTileTok consecutive tokens of one kv-head.  Key rows go from the loaded registers to
// the pool (each a contiguous row of its block).  Value rows are staged in LDS and then stored
// transposed: the lanes of a 32-thread group take the tile's tokens at one dim, so the stores
// of consecutive slots of a block land in one contiguous run of its V^T row (the per-token
// path stores one element per lane of a single token).  Bit copy, like the per-token path;
// slot < 0 or outside the pool: not written.
constexpr int kTileTok = 32;
constexpr int kTiledMinTokens = 1024;  // fewer tokens: the per-token path (decode steps)

template <typename T>
__global__ __launch_bounds__(kWriteThreads) void cache_write_tiled_kernel(CacheWriteArgs a) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int kMaxPer = kTileTok * (128 * 4 / 16) / kWriteThreads;  // chunks per thread, max
  // V rows of the tile's tokens: row j at word j * stride; one pad word per row puts the
  // transposed reads (32 tokens at one dim) on 32 different banks
  extern __shared__ uint32_t s_v[];
  __shared__ int32_t s_blk[kTileTok], s_off[kTileTok], s_len[kTileTok];
  const int D = a.D, B = a.B, Hkv = a.Hkv;
  const int h = blockIdx.y;
  const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTileTok;
  const int ntok = static_cast<int>(a.T - t0 < kTileTok ? a.T - t0 : kTileTok);
  const int row_words = D * static_cast<int>(sizeof(T)) / 4, stride = row_words + 1;
  const int chunks = D / VEC;  // 16-byte chunks of a (token, kv-head) row
  const int total = ntok * chunks;
  const int tid = static_cast<int>(threadIdx.x);
  const T* key = static_cast<const T*>(a.key);
  const T* value = static_cast<const T*>(a.value);
  const TablePatch& tp = a.tp;
  u32x4 kr[kMaxPer], vr[kMaxPer];  // vector types: HIP's uint4 struct kept these in scratch
#pragma unroll
  for (int r = 0; r < kMaxPer; ++r) {
    const int c = tid + r * kWriteThreads;
    if (c < total) {
      const int j = c / chunks, q = c - j * chunks;
      const int64_t src = ((t0 + j) * Hkv + h) * D + static_cast<int64_t>(q) * VEC;
      kr[r] = *reinterpret_cast<const u32x4*>(key + src);
      vr[r] = *reinterpret_cast<const u32x4*>(value + src);
    }
  }
  if (tid < ntok) {  // slots (and lengths) after the row loads: one bus round trip overlaps them
    const int32_t t = static_cast<int32_t>(t0) + tid;
    const int32_t* lp = tp.tables ? tp.ctx_lens + t / tp.tokens_each : nullptr;
    const int32_t sl = ld_step(a.slots + t, a.sys);
    const int32_t ln = lp ? ld_step(lp, a.sys) : 0;
    const bool ok = sl >= 0 && sl < a.n_slots;
    s_blk[tid] = ok ? sl / B : -1;
    s_off[tid] = ok ? sl % B : 0;
    s_len[tid] = ln;
  }
  __syncthreads();
  T* k_cache = static_cast<T*>(a.k_cache);
  T* v_cache = static_cast<T*>(a.v_cache);
#pragma unroll
  for (int r = 0; r < kMaxPer; ++r) {
    const int c = tid + r * kWriteThreads;
    if (c < total) {
      const int j = c / chunks, q = c - j * chunks;
      const int64_t p = s_blk[j];
      if (p >= 0)
        *reinterpret_cast<u32x4*>(k_cache + ((p * Hkv + h) * B + s_off[j]) * D +
                                  static_cast<int64_t>(q) * VEC) = kr[r];
      uint32_t* row = s_v + j * stride + q * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k) row[k] = vr[r][k];
    }
  }
  if (tp.tables && h == 0 && tid < ntok && s_blk[tid] >= 0) {
    // the token's logical block now lives in physical block s_blk (tokens of one sequence that
    // share a block write the same value)
    const int64_t t = t0 + tid;
    const int64_t rr = t / tp.tokens_each;
    const int64_t pos = static_cast<int64_t>(s_len[tid]) - tp.tokens_each + t % tp.tokens_each;
    if (pos >= 0 && pos < static_cast<int64_t>(tp.max_blocks) * B)
      tp.tables[rr * tp.max_blocks + pos / B] = s_blk[tid];
  }
  __syncthreads();
  const int j = tid % kTileTok;
  if (j < ntok) {
    const int64_t p = s_blk[j];
    if (p >= 0) {
      const int o = s_off[j];
      for (int d = tid / kTileTok; d < D; d += kWriteThreads / kTileTok) {
        const uint32_t wv = s_v[j * stride + (sizeof(T) == 2 ? d >> 1 : d)];
        const uint32_t e = sizeof(T) == 2 ? (d & 1 ? wv >> 16 : wv & 0xFFFFu) : wv;
        v_cache[((p * Hkv + h) * D + d) * B + o] = __builtin_bit_cast(T, static_cast<
            typename std::conditional<sizeof(T) == 2, uint16_t, uint32_t>::type>(e));
      }
    }
  }
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

// One workgroup per (block, K or V slab).  A block's K slab ([Hkv, B, D]) and V slab
// ([Hkv, D, B]) are each contiguous in their pool; the host buffer holds block i's K slab then
// its V slab.  to_host: pool -> host with ordinary stores (written back over the bus when the
// kernel ends); else host -> pool with system-coherent 16-byte loads, which never use a line
// an earlier kernel left in a GPU cache.
__global__ __launch_bounds__(256) void swap_blocks_kernel(uint4* __restrict__ k_cache,
                                                          uint4* __restrict__ v_cache,
                                                          uint4* __restrict__ host,
                                                          const int32_t* __restrict__ blocks,
                                                          int num_blocks, int64_t slab_vecs,
                                                          int to_host, int blocks_on_host) {
  const int64_t i = blockIdx.x;
  const int which = blockIdx.y;  // 0: K, 1: V
  const int32_t blk = ld_step(blocks + i, blocks_on_host != 0);
  if (blk < 0 || blk >= num_blocks) return;  // outside the pool: skipped
  uint4* pool = (which == 0 ? k_cache : v_cache) + static_cast<int64_t>(blk) * slab_vecs;
  uint4* hb = host + (2 * i + which) * slab_vecs;
  if (to_host) {
    for (int64_t e = threadIdx.x; e < slab_vecs; e += blockDim.x) hb[e] = pool[e];
  } else {
    // 16-byte loads with the system-coherence bits (sc0 sc1) through a buffer resource over
    // the slab (raw, untyped: the resource word CDNA3/4 kernels use for plain buffers)
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        hb, 0, static_cast<int>(slab_vecs * 16), 0x00020000);
    u32x4* dst = reinterpret_cast<u32x4*>(pool);
    for (int64_t e = threadIdx.x; e < slab_vecs; e += blockDim.x)
      dst[e] = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(e * 16), 0, 1 | 16);
  }
}

static pa_status check_pool_shape(const char* who, int32_t Hkv, int32_t D, int32_t B,
                                  int32_t dtype) {
  if (elem_bytes(dtype) == 0) return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d not supported", who, dtype);
  if (Hkv <= 0) return fail(PA_ERR_INVALID_ARG, "%s: Hkv %d <= 0", who, Hkv);
  if (D != 64 && D != 128) return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", who, D);
  if (B != 16 && B != 32 && B != 64)
    return fail(PA_ERR_UNSUPPORTED, "%s: block size %d not in {16, 32, 64}", who, B);
  return PA_OK;
}

static pa_status launch_cache_write(const char* who, const void* key, const void* value,
                                    void* k_cache, void* v_cache, const int32_t* slot_mapping,
                                    int32_t T, int32_t Hkv, int32_t D, int32_t B,
                                    int32_t num_blocks, int32_t dtype, const TablePatch& tp,
                                    void* stream) {
  const CacheWriteArgs w = make_cache_write_args(key, value, k_cache, v_cache, slot_mapping, T,
                                                 Hkv, D, B, num_blocks, dtype, tp);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (T >= kTiledMinTokens && Hkv <= 65535) {
    const dim3 tg(static_cast<unsigned>((T + kTileTok - 1) / kTileTok), static_cast<unsigned>(Hkv));
    const size_t lds = static_cast<size_t>(kTileTok) * (D * elem_bytes(dtype) / 4 + 1) * 4;
    if (dtype == PA_DTYPE_F32)
      hipLaunchKernelGGL(cache_write_tiled_kernel<float>, tg, dim3(kWriteThreads), lds, s, w);
    else
      hipLaunchKernelGGL(cache_write_tiled_kernel<uint16_t>, tg, dim3(kWriteThreads), lds, s, w);
    return launch_status(who);
  }
  const dim3 grid(static_cast<unsigned>(cache_write_wgs(w)));
  if (dtype == PA_DTYPE_F32)
    hipLaunchKernelGGL(cache_write_kernel<float>, grid, dim3(kWriteThreads), 0, s, w);
  else
    hipLaunchKernelGGL(cache_write_kernel<uint16_t>, grid, dim3(kWriteThreads), 0, s, w);
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

extern "C" pa_status pa_swap_blocks(void* k_cache, void* v_cache, void* host,
                                    const int32_t* blocks, int32_t n, int32_t to_host,
                                    int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks,
                                    int32_t dtype, void* stream) {
  if (pa_status st = check_pool_shape("pa_swap_blocks", Hkv, D, B, dtype)) return st;
  if (n < 0 || num_blocks <= 0 || (to_host != 0 && to_host != 1))
    return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: n %d, num_blocks %d, to_host %d", n,
                num_blocks, to_host);
  if (n == 0) return ok();
  if (n > 65535 * 32768) return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: n too large");
  if (!k_cache || !v_cache || !host || !blocks)
    return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: NULL pointer");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(host))
    return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: pools and host buffer must be 16-byte aligned");
  bool host_is_host = false, blocks_on_host = false;
  if (pa_status st = memory_kind("pa_swap_blocks", "host", host, &host_is_host)) return st;
  if (!host_is_host)
    return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: host must be page-locked host memory");
  if (pa_status st = memory_kind("pa_swap_blocks", "blocks", blocks, &blocks_on_host)) return st;
  const int64_t slab_vecs = static_cast<int64_t>(Hkv) * B * D * elem_bytes(dtype) / 16;
  if (slab_vecs * 16 > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "pa_swap_blocks: a block slab exceeds 2 GiB");
  hipLaunchKernelGGL(swap_blocks_kernel, dim3(static_cast<unsigned>(n), 2), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<uint4*>(k_cache),
                     static_cast<uint4*>(v_cache), static_cast<uint4*>(host), blocks, num_blocks,
                     slab_vecs, to_host, blocks_on_host ? 1 : 0);
  return launch_status("pa_swap_blocks");
}
