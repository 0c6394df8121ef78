/*
 * pa.h -- C ABI of the paged KV-cache library (libpa.so) for AMD Instinct MI355X (gfx950).
 *
 * The library implements the hot path of PagedAttention as described on three pages:
 *   [TT]  "Taming the Tail: How PagedAttention Solves the KV-Cache Fragmentation Crisis in
 *         Multi-Tenant LLM Serving" (architects-blueprint blog);
 *   [VP]  "vLLM PagedAttention: Eliminating KV Cache Memory Fragmentation & 4x Throughput"
 *         (tinycto.tv);
 *   [KC]  the grade-12 KV-cache chapter of aicomputerinstitute.com.
 *
 * Two halves sit behind this header:
 *   - a host block manager (free pool, per-block reference counts, fork with copy-on-write,
 *     block tables and slot mappings), pure C++, no GPU needed;
 *   - HIP kernels for gfx950 that operate on a physical pool of fixed-size blocks.
 *
 * Conventions for every function:
 *   - The return value is a pa_status; PA_OK is 0, errors are negative.  After an error,
 *     pa_last_error() returns a message (thread-local, valid until the next call on that
 *     thread).  No C++ exception crosses this boundary.
 *   - Block-manager calls are all-or-nothing: when they return an error nothing changed.
 *   - Device calls take device pointers the CALLER owns and a hipStream_t passed as void*
 *     (NULL = the null stream).  They only enqueue work: no allocation, no synchronisation.
 *     Every argument visible on the host (sizes, dtype, alignment) is checked before any
 *     launch; contents of device memory cannot be checked there (use pa_validate_tables on a
 *     host copy).  Kernels never read or write outside the buffers described by the sizes
 *     passed in: a slot, block id or context length out of range is skipped or clamped and the
 *     affected outputs are set to NaN, never dereferenced.
 *   - A handle (pa_bm) is not thread-safe: one scheduler thread per handle.
 *
 * Pool layout (the pages fix only the address rule: physical block times block size plus offset,
 * [TT] "Under the Hood: The CUDA Kernel Engineering"; the rest is this library's choice):
 *   k_cache: [num_blocks, Hkv, B, D]  -- key of token at offset o of block p, kv-head h is
 *                                        the contiguous row k_cache[p][h][o][0..D)
 *   v_cache: [num_blocks, Hkv, D, B]  -- its value is the column v_cache[p][h][0..D)[o]
 *                                        (values are stored transposed inside each block)
 *   slot = p * B + o.   Block tables: int32 [S, max_blocks], row s lists the physical blocks of
 *   sequence s in logical order, padded with -1.  All arrays are C-contiguous.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t pa_status;

enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = -1,   /* bad size, pointer, id or precondition                     */
  PA_ERR_OUT_OF_BLOCKS = -2, /* the free pool cannot satisfy the request (state unchanged) */
  PA_ERR_UNKNOWN_SEQ = -3,   /* a sequence id that the manager does not hold               */
  PA_ERR_SEQ_EXISTS = -4,    /* a sequence id that is already in use                       */
  PA_ERR_UNSUPPORTED = -5,   /* dtype / head_dim / block size / group combination not built */
  PA_ERR_WORKSPACE = -6,     /* workspace missing or smaller than the size query returned  */
  PA_ERR_HIP = -7,           /* the HIP runtime reported an error at launch                */
  PA_ERR_SWAPPED = -8        /* the sequence is swapped out (pa_bm_swap_in it first)       */
};

enum { PA_DTYPE_F32 = 0, PA_DTYPE_BF16 = 1 };

/* Message of the last error on this thread ("" if none).  Never NULL. */
const char* pa_last_error(void);

/* Version of this ABI (bumped on any incompatible change). */
int32_t pa_abi_version(void);

/* ======================================================================================
 * Host block manager.
 *
 * [TT] "How the Architecture Works": logical blocks of a sequence map through its block table
 * to physical blocks anywhere in the pool; a new block is taken from the free block pool when
 * the current one is full.  [VP] "1. Underlying Mechanism": B=16 (or 32) tokens per block;
 * token 17 takes a new block; a forked child shares the parent's blocks and copy-on-write
 * gives it private copies.  [KC] "PagedAttention: borrowing virtual memory": one reference
 * count per physical block; a block rejoins the pool only at count zero; a sequence about to
 * write into a shared block first receives a private copy.
 *
 * Fixed policy (the pages leave it open; this is part of the contract, so block tables, slot
 * mappings and copy lists are reproducible bit for bit):
 *   - the free pool is FIFO: allocation takes the front, a freed block is appended at the
 *     back; a freed sequence releases its blocks in logical order;
 *   - appends to a batch are served in batch order; a sequence copies its last block iff the
 *     block is partly filled and its count is above one at that sequence's turn (of k sharers
 *     appending in one call, the first k-1 copy, the last writes in place); the copy covers the
 *     whole block (all kv-heads, all slots, K and V);
 *   - a batch names each sequence at most once.
 * ====================================================================================== */

typedef struct pa_bm pa_bm;

typedef struct {
  int32_t num_blocks;       /* pool size                                                  */
  int32_t block_size;       /* B                                                          */
  int32_t free_blocks;      /* blocks with count 0                                        */
  int32_t used_blocks;      /* blocks with count >= 1                                     */
  int32_t shared_blocks;    /* blocks with count >= 2                                     */
  int32_t num_seqs;         /* live sequences                                             */
  int64_t logical_blocks;   /* sum over sequences of table entries                        */
  int64_t live_tokens;      /* sum over sequences of their token counts                   */
  int64_t tail_waste_slots; /* logical_blocks * B - live_tokens (unused slots in last blocks) */
  int64_t forks;            /* pa_bm_fork calls so far                                    */
  int64_t cow_copies;       /* block copies issued by copy-on-write so far                */
  double usage;             /* used_blocks / num_blocks: the pool saturation to monitor,
                               [TT] "Summing it Up", item 3                                */
  int32_t swapped_seqs;     /* sequences swapped out (not counted in num_seqs)            */
  int64_t swapped_tokens;   /* tokens those sequences hold in host memory                 */
  int64_t swap_outs;        /* pa_bm_swap_out calls so far                                */
  int64_t swap_ins;         /* pa_bm_swap_in calls so far                                 */
  int32_t cached_blocks;    /* prefix-cache tree nodes (each holds one block reference)   */
  int64_t cache_hit_blocks; /* blocks pa_bm_add_seq_cached reused so far                  */
  int64_t cache_evictions;  /* tree nodes evicted so far                                  */
} pa_bm_stats_t;

/* Create a manager over physical blocks [0, num_blocks) of block_size tokens each.
 * init_free_order: NULL (ids in increasing order) or a host array of num_blocks ints that is a
 * permutation of [0, num_blocks), giving the initial FIFO order.  *out receives the handle. */
pa_status pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* init_free_order,
                       pa_bm** out);

/* Destroy a handle (NULL is accepted).  Device memory is not touched. */
pa_status pa_bm_destroy(pa_bm* bm);

/* New sequence holding n_tokens >= 0 tokens (a prefill): takes ceil(n/B) blocks.
 * slots_out: NULL or a host array of n_tokens ints receiving the slot of positions 0..n-1. */
pa_status pa_bm_add_seq(pa_bm* bm, int64_t seq_id, int32_t n_tokens, int32_t* slots_out);

/* Append tokens_each >= 0 tokens to each of n_seqs distinct sequences, in batch order
 * (tokens_each = 1 is one decode step; larger values append a chunk).
 * slots_out:      host array of n_seqs * tokens_each ints (sequence-major) receiving slots.
 * copy_pairs_out: host array of pairs_cap * 2 ints receiving the copy-on-write pairs
 *                 (src_block, dst_block) in the order made; may be NULL if pairs_cap == 0.
 * n_copies_out:   receives the number of pairs written.
 * The pairs must be applied (pa_copy_blocks) before the new tokens are written
 * (pa_cache_write), on the same stream.  Errors: PA_ERR_OUT_OF_BLOCKS if the pool cannot
 * hold the new blocks and copies; PA_ERR_INVALID_ARG if more than pairs_cap copies are
 * needed or an id repeats; PA_ERR_UNKNOWN_SEQ.  On error nothing changes. */
pa_status pa_bm_append_slots(pa_bm* bm, const int64_t* seq_ids, int32_t n_seqs,
                             int32_t tokens_each, int32_t* slots_out, int32_t* copy_pairs_out,
                             int32_t pairs_cap, int32_t* n_copies_out);

/* pa_bm_append_slots that also writes lens_out[i] (host array of n_seqs ints), the length of
 * seq_ids[i] after the call, in the same pass: the host half of one serving step (slots,
 * copy-on-write pairs and the new context lengths) in one call.  The host cost of block
 * management is one of the overheads [VP] "3. Production Failure Modes" says to watch; once
 * the handle's scratch has grown to the batch size, a step allocates no host memory.  Errors
 * and failure atomicity as pa_bm_append_slots (lens_out is not written on error). */
pa_status pa_bm_append_step(pa_bm* bm, const int64_t* seq_ids, int32_t n_seqs,
                            int32_t tokens_each, int32_t* slots_out, int32_t* lens_out,
                            int32_t* copy_pairs_out, int32_t pairs_cap, int32_t* n_copies_out);

/* Zero-copy fork ([VP] "Zero-Copy Forking & Parallel Sampling"): child receives the parent's
 * table and length; every block's count goes up by one.  No device work. */
pa_status pa_bm_fork(pa_bm* bm, int64_t parent_id, int64_t child_id);

/* Drop a sequence; each of its blocks' counts goes down by one and blocks reaching zero are
 * appended to the free pool in logical order ([KC] answer A6). */
pa_status pa_bm_free_seq(pa_bm* bm, int64_t seq_id);

/* Block tables and context lengths of n sequences.
 * tables_out: host [n, max_blocks] ints, row i = physical blocks of seq_ids[i], padded -1.
 * ctx_lens_out: host [n] ints (NULL allowed).  PA_ERR_INVALID_ARG if a sequence holds more
 * than max_blocks blocks. */
pa_status pa_bm_block_tables(pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t max_blocks,
                             int32_t* tables_out, int32_t* ctx_lens_out);

/* Token count of one sequence. */
pa_status pa_bm_seq_len(pa_bm* bm, int64_t seq_id, int32_t* n_out);

/* Token counts of n sequences (host array lens_out[n]); the context lengths of a step without
 * rebuilding the block tables.  PA_ERR_UNKNOWN_SEQ names the first unknown id (lens_out may be
 * partly written then). */
pa_status pa_bm_seq_lens(pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t* lens_out);

/* Reference count of one physical block. */
pa_status pa_bm_refcount(pa_bm* bm, int32_t block, int32_t* out);

/* The free pool, front first: writes min(cap, free) ids to out and the full count to *n_out. */
pa_status pa_bm_free_list(pa_bm* bm, int32_t* out, int32_t cap, int32_t* n_out);

/* Pool statistics ([TT] "Summing it Up": monitor the physical block pool saturation). */
pa_status pa_bm_stats(pa_bm* bm, pa_bm_stats_t* out);

/* Preemption by swapping ([TT] "Infrastructure Scale": when the pool runs out of physical
 * blocks, a request can be paused and its KV-cache moved to CPU RAM).
 *
 * pa_bm_swap_out: *n_out receives k = ceil(len / B), and blocks_out[0..k) the sequence's
 * physical blocks in logical order, as they are before the call.  Its references are then
 * released as in pa_bm_free_seq (blocks reaching count zero rejoin the pool in logical order),
 * and the sequence is swapped: it keeps its id and length and holds no blocks.  The caller
 * copies those k blocks to host memory (pa_swap_blocks, to_host = 1) before anything can
 * write into them again -- enqueued on the stream that later writes run on, that is
 * automatic.  Only pa_bm_swap_in, pa_bm_free_seq, pa_bm_seq_len and pa_bm_seq_lens accept a
 * swapped sequence; the other calls return PA_ERR_SWAPPED.  PA_ERR_INVALID_ARG if cap < k
 * (*n_out still receives k; nothing changes).
 *
 * pa_bm_swap_in: the swapped sequence takes k fresh blocks from the front of the pool, in
 * logical order, each with count 1, written to blocks_out (k to *n_out).  Blocks it shared
 * before the swap come back as private copies.  The caller copies the saved K/V into them
 * (pa_swap_blocks, to_host = 0) before a kernel reads the sequence.  PA_ERR_OUT_OF_BLOCKS if
 * fewer than k blocks are free, PA_ERR_INVALID_ARG if the sequence is live or cap < k;
 * nothing changes on error. */
pa_status pa_bm_swap_out(pa_bm* bm, int64_t seq_id, int32_t* blocks_out, int32_t cap,
                         int32_t* n_out);
pa_status pa_bm_swap_in(pa_bm* bm, int64_t seq_id, int32_t* blocks_out, int32_t cap,
                        int32_t* n_out);

/* Prefix cache ([KC] "RadixAttention": cached token sequences form a radix tree; a new request
 * reuses the K/V blocks of its longest cached prefix and prefills only the rest; when memory
 * runs low the least recently used leaves are evicted, reference counting protecting what
 * running requests use; [KC] answer A3: only whole blocks that are entirely prefix are shared).
 * A tree node is one full block of B token ids under its parent, and holds one reference to
 * its physical block.
 *
 * pa_bm_cache_insert: the first n_tokens token ids of a live sequence (the caller vouches that
 * they are its tokens and that their K/V are written) -- its first floor(n_tokens / B) blocks
 * become cached, each under its content; a content already cached keeps its existing block.
 * *n_added_out (NULL allowed) receives the number of new nodes.
 *
 * pa_bm_add_seq_cached: a new sequence of n_tokens token ids.  The longest chain of cached
 * full blocks matching its first tokens is reused (each block gains a reference);
 * *n_cached_out receives their token count (a multiple of B), and the rest get fresh blocks
 * as in pa_bm_add_seq.  slots_out (NULL allowed): the slots of all n_tokens positions; only
 * positions >= *n_cached_out need a prefill and a cache write.
 *
 * Eviction: a call that needs more blocks than the pool holds (adds, appends, swap-ins) first
 * evicts exactly the shortfall -- each time the tree leaf with the oldest use (ties: the
 * oldest node) among those only the tree references -- and the freed blocks join the back of
 * the pool.  If the tree cannot cover the shortfall the call fails with PA_ERR_OUT_OF_BLOCKS
 * and nothing changes.  An insert or a cached add marks every node it passes as used, at one
 * step of a counter.  pa_bm_cache_evict evicts up to n_blocks such leaves on demand. */
pa_status pa_bm_cache_insert(pa_bm* bm, int64_t seq_id, const int32_t* tokens, int32_t n_tokens,
                             int32_t* n_added_out);
pa_status pa_bm_add_seq_cached(pa_bm* bm, int64_t seq_id, const int32_t* tokens,
                               int32_t n_tokens, int32_t* slots_out, int32_t* n_cached_out);
pa_status pa_bm_cache_evict(pa_bm* bm, int32_t n_blocks, int32_t* n_evicted_out);

/* Truncate a live sequence to its first n_keep tokens (0 <= n_keep <= len), e.g. to roll back
 * rejected speculative tokens.  Blocks past ceil(n_keep / B) are released in logical order
 * (blocks reaching count zero rejoin the pool).  A kept last block that is shared stays
 * shared; the next append copies it first, as for any shared partial block.  No device work:
 * slots past the new length are simply never read. */
pa_status pa_bm_truncate(pa_bm* bm, int64_t seq_id, int32_t n_keep);

/* Share groups of a batch for pa_decode_shared / pa_decode_step_shared ([TT] "Complex Memory
 * Sharing": sequences forked from one prompt, or admitted through the prefix cache, read the
 * same physical blocks for their shared part).  Sequences of seq_ids whose tables start with
 * the same physical blocks are grouped, at most max_members (2..4) per group: the tables are
 * ordered so that common physical prefixes are adjacent, and the tree of those prefixes is
 * walked from its deepest nodes up -- at each node the sequences not yet grouped form groups
 * of max_members sharing that node's tokens; a smaller remainder is grouped there when that
 * saves at least the reads it could save one level up (a group of k saves (k - 1) * L
 * reads), else left to the parent.  Groups sharing fewer than min_tokens tokens are left
 * out.  groups_out: host [cap, 5] ints, one row per group: the
 * number of tokens L every member holds in the same physical blocks (positions below every
 * member's length), then the members as indices into seq_ids, ascending, -1 padded.
 * *n_groups_out receives the number of groups (rows ordered by their first member);
 * PA_ERR_INVALID_ARG if it exceeds cap (at most n / 2 are ever needed).  Host only. */
pa_status pa_bm_share_groups(pa_bm* bm, const int64_t* seq_ids, int32_t n, int32_t max_members,
                             int32_t min_tokens, int32_t* groups_out, int32_t cap,
                             int32_t* n_groups_out);

/* ---- host utilities ---------------------------------------------------------------- */

typedef struct {
  int64_t total_actual_tokens; /* sum of lengths                                   */
  int64_t paged_slots;         /* B * sum ceil(len / B)                            */
  int64_t naive_slots;         /* max_seq_len * n                                  */
  double paged_fragmentation_pct;  /* 100 (paged - actual) / paged   (unrounded) */
  double naive_fragmentation_pct;  /* 100 (naive - actual) / naive   (unrounded) */
  double memory_reduction_factor;  /* naive / paged                  (unrounded) */
} pa_accounting_t;

/* Slot accounting of n request lengths (host arrays), as [KC] "Worked Example 1" computes it for
 * its four requests: the tokens held, the slots paged blocks of block_size reserve, the slots a
 * contiguous reservation of max_seq_len per request reserves, both waste percentages and their
 * ratio.  No manager state is read (the name groups it with the block-manager calls).
 * PA_ERR_INVALID_ARG for n, block_size or max_seq_len <= 0, a negative length, or all lengths
 * zero. */
pa_status pa_bm_accounting(const int32_t* lens, int32_t n, int32_t block_size,
                           int32_t max_seq_len, pa_accounting_t* out);

/* Host check of a block table before upload: every entry a sequence uses (the first
 * ceil(ctx_len/B)) lies in [0, num_blocks), 1 <= ctx_len <= max_blocks * B.  PA_OK or
 * PA_ERR_INVALID_ARG naming the first bad row. */
pa_status pa_validate_tables(const int32_t* tables, const int32_t* ctx_lens, int32_t S,
                             int32_t max_blocks, int32_t block_size, int32_t num_blocks);

/* ======================================================================================
 * Device operations (HIP, gfx950).  Supported: dtype F32 or BF16; head_dim D in {64, 128};
 * block size B in {16, 32, 64}; Hq a multiple of Hkv.  Tensors are C-contiguous; every pointer
 * must be 16-byte aligned.
 * ====================================================================================== */

/* Cache write (each step stores only the new token's K/V: [TT] "The Hidden Tax"; [VP]
 * "1. Underlying Mechanism").  For t in [0, T): if slot_mapping[t] is in
 * [0, num_blocks * B) the key key[t] ([Hkv, D]) goes to k_cache[slot / B][h][slot % B][:] and
 * value[t] to v_cache[slot / B][h][:][slot % B]; other slots (negative: padding) are skipped.
 * Bit copy, no arithmetic.  Slots within one call must be distinct.
 * key, value: device [T, Hkv, D] of dtype;  slot_mapping: device int32 [T]. */
pa_status pa_cache_write(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int32_t* slot_mapping, int32_t T, int32_t Hkv, int32_t D,
                         int32_t B, int32_t num_blocks, int32_t dtype, void* stream);

/* The device half of one serving step in one launch: the cache write above plus the block-table
 * entries the step created, so that block tables and context lengths can stay resident on the
 * device from step to step and only the step's slots and new lengths cross the bus ([TT] "How
 * the Architecture Works": a sequence's table gains an entry when its last block is full; [KC]
 * "PagedAttention: borrowing virtual memory": a copy-on-write replaces the shared last block).
 * The batch is S sequences, each appending tokens_each tokens (1 = decode, C = a chunk), in the
 * order pa_bm_append_slots returns their slots.  For t in [0, S * tokens_each): row
 * r = t / tokens_each sits at position pos = ctx_lens[r] - tokens_each + t % tokens_each
 * (ctx_lens holds the lengths AFTER the step); its key/value go to slot_mapping[t] exactly as in
 * pa_cache_write, and block_tables[r][pos / B] = slot_mapping[t] / B.  This is the one entry
 * of the row a step can change: a new block at a block boundary, or the private copy that
 * replaced a shared last block.  Tokens with a slot outside [0, num_blocks * B) or a position
 * outside [0, max_blocks * B) are skipped (not written anywhere).
 * key, value: device [S * tokens_each, Hkv, D]; slot_mapping: device int32 [S * tokens_each];
 * block_tables: device int32 [S, max_blocks], updated in place; ctx_lens: device int32 [S]. */
pa_status pa_cache_append(const void* key, const void* value, void* k_cache, void* v_cache,
                          const int32_t* slot_mapping, int32_t S, int32_t tokens_each,
                          int32_t* block_tables, int32_t max_blocks, const int32_t* ctx_lens,
                          int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks, int32_t dtype,
                          void* stream);

/* Copy-on-write block copies ([KC] "PagedAttention: borrowing virtual memory"): for each of
 * the P pairs (src, dst) in device int32 [P, 2], physical block dst of both pools becomes a
 * bit copy of block src.  Pairs as produced by pa_bm_append_slots: distinct dst, no dst is
 * also a src; ids outside [0, num_blocks) are skipped.  Enqueue before pa_cache_write. */
pa_status pa_copy_blocks(void* k_cache, void* v_cache, const int32_t* pairs, int32_t P,
                         int32_t num_blocks, int32_t Hkv, int32_t D, int32_t B, int32_t dtype,
                         void* stream);

/* Workspace bytes pa_decode needs for S sequences of at most max_ctx_len tokens.
 * partition_tokens: the split-K partition length pa_decode will be called with (0 = the
 * library's choice; the size returned then covers any choice it makes). */
pa_status pa_decode_workspace_size(int32_t S, int32_t Hq, int32_t D, int32_t max_ctx_len,
                                   int32_t partition_tokens, size_t* bytes);

/* Paged decode attention: one query token per sequence and head over the sequence's cached
 * K/V, reached through its block table ([TT] "Under the Hood: The CUDA Kernel Engineering":
 * key/value addresses come from the block table, access stays coalesced, the unaligned last
 * block is handled; [KC] "Common misconception": the same scores and softmax as dense
 * attention).
 *
 *   out[s, h, :] = sum_j softmax_j(scale * q[s,h,:] . K_s[j, h / (Hq/Hkv), :]) V_s[j, ...]
 *   over the ctx_lens[s] tokens of sequence s (including the one written this step).
 *
 * q, out: device [S, Hq, D] of dtype (out is rounded to nearest-even for BF16).
 * block_tables: device int32 [S, max_blocks]; ctx_lens: device int32 [S], each in
 * [1, max_blocks * B] and <= max_ctx_len.  Positions >= ctx_len of a sequence never influence
 * its output (NaN or Inf there is harmless).  scale: positive and finite.  Computation: fp32
 * accumulation; split-K over partitions of partition_tokens tokens (0 = library's choice, else
 * a multiple of 32 and of B in [32, 8192]) followed by a merge.  workspace: device buffer of at least
 * pa_decode_workspace_size(S, Hq, D, max_ctx_len, partition_tokens) bytes (may be NULL if
 * that size is 0).  Deterministic: results depend on logical positions only, not on which
 * physical blocks hold them. */
pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* ctx_lens, int32_t S, int32_t Hq,
                    int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks, int32_t max_blocks,
                    int32_t max_ctx_len, float scale, int32_t dtype, int32_t partition_tokens,
                    void* workspace, size_t workspace_bytes, void* stream);

/* pa_decode with share groups ([TT] "Complex Memory Sharing": requests that share a prompt read
 * its blocks from one physical copy).  groups: device int32 [n_groups, 5], rows as
 * pa_bm_share_groups writes them: L, then up to 4 member sequences (indices in [0, S), -1
 * padded); 0 <= n_groups <= S.  The caller promises that every member holds the same keys and
 * values as its group's first member at positions [0, L) -- true for blocks a fork or the
 * prefix cache shares, and it stays true after copy-on-write (the copies are bit copies) as
 * long as no member is truncated below L.  Each group's range is then read once for several
 * members: on the matrix cores (bf16, 3 to 8 query heads per kv-head) one work item serves
 * 16 / (Hq/Hkv) members (at most 4), their heads side by side in the same 16-column operand, and
 * each member merges that result with its own tokens [L, n) like any other partition.  The
 * result is the same attention (it differs from pa_decode's only by the order of its fp32
 * sums).  The device plan checks each group: a member index out of range, an invalid length,
 * or a sequence already taken by an earlier group drops that member; L is cut to the members'
 * shortest length and rounded down to a multiple of 32; a group left with fewer than two
 * members or L < 32 is ignored.  Other shapes and dtypes ignore the groups.  A wrong promise
 * gives wrong outputs for that group's members, never an access outside the buffers.  The
 * workspace is the one pa_decode_workspace_size reports. */
pa_status pa_decode_shared(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* ctx_lens, int32_t S,
                           int32_t Hq, int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks,
                           int32_t max_blocks, int32_t max_ctx_len, float scale, int32_t dtype,
                           int32_t partition_tokens, const int32_t* groups, int32_t n_groups,
                           void* workspace, size_t workspace_bytes, void* stream);

/* One decode step of a serving loop on the device, fused: the cache write and block-table patch
 * of pa_cache_append for one new token per sequence (tokens_each = 1), then pa_decode over the
 * updated tables.  The decode's planning work runs in the same launch as the cache write (the
 * two are independent), so the step costs one kernel launch fewer than pa_cache_append followed
 * by pa_decode, with bit-identical results.
 * key, value: device [S, Hkv, D] of dtype (the new tokens).
 * slot_mapping: int32 [S], the new tokens' slots.  block_tables: device int32 [S, max_blocks],
 * updated in place.  ctx_lens: device int32 [S], the lengths the decode reads.
 * new_ctx_lens: int32 [S], the lengths AFTER the step (including the new token), or NULL when
 * ctx_lens already holds them; when given, the step copies them into ctx_lens.
 * slot_mapping and new_ctx_lens may each be device memory or page-locked host memory
 * (hipHostMalloc, a pinned torch tensor), so a serving loop needs no separate upload of its
 * per-step metadata: for S <= 384 the call copies page-locked buffers into the first kernel's
 * arguments; for larger batches that kernel reads host memory directly, and such a buffer must
 * then not be rewritten before the step has completed on the stream.
 * q, out, the pools, max_ctx_len, scale, partition_tokens and the workspace are as in
 * pa_decode (the size query is the same).  Errors as in pa_cache_append and pa_decode, and
 * PA_ERR_INVALID_ARG when slot_mapping or new_ctx_lens is pageable host memory; nothing is
 * launched when one is returned. */
pa_status pa_decode_step(void* out, const void* q, const void* key, const void* value,
                         void* k_cache, void* v_cache, const int32_t* slot_mapping,
                         int32_t* block_tables, int32_t* ctx_lens, const int32_t* new_ctx_lens,
                         int32_t S, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                         int32_t num_blocks, int32_t max_blocks, int32_t max_ctx_len, float scale,
                         int32_t dtype, int32_t partition_tokens, void* workspace,
                         size_t workspace_bytes, void* stream);

/* pa_decode_step with share groups (as in pa_decode_shared). */
pa_status pa_decode_step_shared(void* out, const void* q, const void* key, const void* value,
                                void* k_cache, void* v_cache, const int32_t* slot_mapping,
                                int32_t* block_tables, int32_t* ctx_lens,
                                const int32_t* new_ctx_lens, int32_t S, int32_t Hq, int32_t Hkv,
                                int32_t D, int32_t B, int32_t num_blocks, int32_t max_blocks,
                                int32_t max_ctx_len, float scale, int32_t dtype,
                                int32_t partition_tokens, const int32_t* groups,
                                int32_t n_groups, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Bytes of device scratch pa_decode_step_noalloc holds on each GPU it runs on, in MiB. */
#define PA_NOALLOC_SCRATCH_MIB 96

/* pa_decode_step without the workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * The decode's scratch (queue, work list, merge counters, partial results) is a file-scope
 * device array of PA_NOALLOC_SCRATCH_MIB MiB inside the library; each GPU the library runs on
 * holds its own copy until the process ends.  This call allocates nothing (no hipMalloc, no
 * hipFree, no allocating library routine); the caller still owns every input and output.
 * Arguments, results and errors are those of pa_decode_step, plus PA_ERR_WORKSPACE (before
 * any device work) when the batch needs more scratch than the array holds -- the size
 * pa_decode_workspace_size(S, Hq, D, max_ctx_len, partition_tokens) reports; e.g. 256
 * sequences of 64 query heads, D = 128, fit up to max_ctx_len = 10,240 with automatic
 * partitions.  Every call on one GPU shares that GPU's array, and the array keeps the last
 * call's contents (each call initialises what it reads): calls that overlap on one GPU (two
 * streams or two threads) race and must be serialised by the caller. */
pa_status pa_decode_step_noalloc(void* out, const void* q, const void* key, const void* value,
                                 void* k_cache, void* v_cache, const int32_t* slot_mapping,
                                 int32_t* block_tables, int32_t* ctx_lens,
                                 const int32_t* new_ctx_lens, int32_t S, int32_t Hq, int32_t Hkv,
                                 int32_t D, int32_t B, int32_t num_blocks, int32_t max_blocks,
                                 int32_t max_ctx_len, float scale, int32_t dtype,
                                 int32_t partition_tokens, void* stream);

/* Whole-block copies between the pools and host memory, for swapping a paused request's
 * KV-cache to CPU RAM and back ([TT] "Infrastructure Scale"; pa_bm_swap_out / pa_bm_swap_in
 * give the block lists).
 * host: page-locked host memory (hipHostMalloc, a pinned torch tensor) of n * 2 * Hkv * B * D
 *   elements of dtype: block i's K slab (its [Hkv, B, D] part of the K pool, laid out as
 *   there) followed by its V slab ([Hkv, D, B]).  The kernel reads or writes it directly over
 *   the bus; nothing else may touch it until the copy has completed on the stream.
 * blocks: int32 [n] physical block ids, device memory or page-locked host memory; ids outside
 *   [0, num_blocks) are skipped.
 * to_host = 1: pools -> host (swap out); 0: host -> pools (swap in).
 * Errors: PA_ERR_INVALID_ARG for a pageable or device `host`, a pageable `blocks`, NULL or
 * misaligned pointers; PA_ERR_UNSUPPORTED for shapes the pools do not support. */
pa_status pa_swap_blocks(void* k_cache, void* v_cache, void* host, const int32_t* blocks,
                         int32_t n, int32_t to_host, int32_t Hkv, int32_t D, int32_t B,
                         int32_t num_blocks, int32_t dtype, void* stream);

/* Chunked-query paged attention (prefill of the tokens past a cached prefix, [KC]
 * "RadixAttention": only the tokens past the divergence need a prefill pass).  Each of the S
 * sequences has ctx_lens[s] tokens in the pool INCLUDING its C new ones (already written by
 * pa_cache_write); query row i (0 <= i < C) sits at position ctx_lens[s] - C + i and attends
 * to positions 0 .. ctx_lens[s] - C + i (causal inside the chunk).
 * q, out: device [S, C, Hq, D] (BF16).  ctx_lens[s] in [C, max_blocks * B].  scale: positive
 * and finite.  fp32 accumulation on the matrix cores.  No workspace. */
pa_status pa_chunk_attend(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, const int32_t* ctx_lens, int32_t S,
                          int32_t C, int32_t Hq, int32_t Hkv, int32_t D, int32_t B,
                          int32_t num_blocks, int32_t max_blocks, float scale, int32_t dtype,
                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
