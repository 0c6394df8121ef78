// Paged decode attention on gfx950: split-K over context partitions and their merge.
//
// What is computed ("vLLM PagedAttention" (tinycto), FAQ: paging leaves the result of standard
// multi-head attention unchanged; KV-cache chapter, "Common misconception": the same scores and
// softmax, the memory is only gathered through the block table):
//
//   out[s, h] = sum_j softmax_j(scale * q[s, h] . K_s[j, h / g]) V_s[j, h / g]
//
// over the ctx_len tokens of sequence s, where token j lives in physical block
// table[s][j / B] at offset j % B ("Taming the Tail", "Under the Hood: The CUDA Kernel
// Engineering": key/value addresses come from the block table, accesses stay coalesced, the
// unaligned last block is handled).
//
// Work decomposition (chosen for CDNA4, not taken from the pages):
//   * a work item is one partition of PT tokens of one (sequence, kv-head); NW = 4 waves split
//     the partition's 32-token tiles round-robin and each keeps its own online-softmax state
//     (reference max m, sum l, unnormalised output o relative to m), scores in the log2
//     domain; the matrix-core kernel moves m only when a score passes it by 2^8;
//   * one workgroup plans: it turns the context lengths into a work list, longest first --
//     every full partition, then the partial last partitions by decreasing length.  It runs as
//     a one-workgroup kernel (pa_decode) or as workgroup 0 of the step's first kernel beside
//     the cache write (pa_decode_step).  The decode kernel is persistent (about as many
//     workgroups as the chip holds at once) and pulls items from that list through atomic
//     counters, claiming the next item as the current one's tiles end; a batch that
//     shares prefix blocks is claimed per XCD so each kv-head stays in one XCD's L2.  No
//     workgroup is launched for a partition that does not exist, and the short items fill
//     the tail;
//   * the partition's block-table slice is staged in LDS once (loaded together with the
//     context length), so tile loads never wait on a dependent table load;
//   * the four wave states are merged through LDS; a single-partition sequence writes its
//     final output directly.  Otherwise the partition stores (m, l, o/l) and the workgroup
//     that finishes the last partition of that (sequence, kv-head) merges them (the
//     FlashAttention-style tiling the KV-cache chapter mentions in "Common misconception");
//   * GQA groups (bf16, g >= 3): QK^T and PV are real dense contractions of g heads against
//     the tile, done on the matrix cores (v_mfma_f32_16x16x32_bf16).  S^T = K Q^T puts 16
//     tokens on the rows and the (padded) 16 heads on the columns; O^T = V^T P^T contracts
//     over tokens.  K is loaded as whole 256-byte rows and re-laid out through LDS into the
//     operand layout; the V pool is stored transposed per block so 8 consecutive tokens of
//     one dim are contiguous and load straight into the PV operand registers;
//   * one query head per kv-head (g in {1, 2}) or fp32: a VALU kernel; LPT lanes share one
//     token's dot product (reduced with cross-lane shuffles), the round max uses shuffles, and
//     the PV update broadcasts the round's weights through a per-wave LDS slot.
//
// Tiles beyond the context are never formed; lanes whose token lies past ctx_len load a
// clamped in-range address and their score is set to -inf and their V elements to zero, so
// values past the end (even NaN) cannot reach the output.

#include <climits>
#include <cstddef>
#include <cstring>
#include <cmath>
#include <map>
#include <mutex>
#include <utility>

#include "cache_write.h"
#include "device_common.h"
#include "host_memory.h"

namespace pa {

constexpr int kNW = 4;            // waves per workgroup
constexpr int kXcd = 8;           // XCDs of an MI355X (one work queue each)
constexpr int kMaxPT = 8192;      // largest partition (tokens)
constexpr int kMinAutoPT = 1024;  // smallest partition the automatic choice uses (below it the
                                  // per-item start-up and the merge outweigh the parallelism:
                                  // 32,768 tokens at batch 1 take 0.065 ms at 256, 0.040 at 1,024)
constexpr int kMaxAutoPT = 4096;  // largest partition the automatic choice uses
constexpr int kAutoPTStep = 256;  // the automatic choice is a multiple of this (whole blocks)
constexpr int kPtSlot = 11;       // queue[kPtSlot]: the partition length the plan used
constexpr int kPmaxSlot = 12;     // queue[kPmaxSlot]: partial-result slots per (sequence, head)
constexpr int kGroupMembers = 4;  // sequences a share group may name
constexpr int kGroupRec = 1 + kGroupMembers;  // caller's record: tokens, members
constexpr int kVGroupRec = 2 + kGroupMembers;  // validated record: tokens, members, count
constexpr int kFuseTail = 256;    // a group member's own tokens past the group's range, up to
                                  // this many, are read by the group's last item (no item of
                                  // their own, no merge when the range is one partition)
constexpr int kPlanThreads = 256;
constexpr int kMaxBuckets = kMaxPT / 32 + 1;  // partial partitions bucketed by 32-token tiles
constexpr int kPlanKeep = 2048;  // sequences whose lengths the plan keeps in LDS between passes
constexpr int kShareBits = 10;   // first-block set of the sharing test: 1024 slots
constexpr int kShareSlots = 1 << kShareBits;
constexpr int kShareProbes = 16;
constexpr float kLog2e = 1.4426950408889634f;

// A work-list entry is two int4: (sequence s, or -1 - group for a share-group item; partial
// slot; first token; end token) and the member sequences ((s, -1, -1, -1) for a sequence's own
// item).  Each entry stands for Hkv items, one per kv-head.
struct DecodeArgs {
  void* out;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* tables;
  const int32_t* ctx_lens;
  float* part_o;    // [S, Hq, Pmax, D]  partition outputs (normalised)
  float2* part_ml;  // [S, Hq, Pmax]     (max in log2 units, sum)
  int4* items;      // work list: entries (see above), longest first
  int* queue;       // [0] number of items, [2 + x] next unclaimed slot of XCD x
  int* done;        // [S, Hkv] partitions finished (split sequences), zeroed by the plan
  int* nparts;      // [S] partial results of each sequence (written by the plan)
  const int32_t* groups;  // caller's share groups [ngroups][kGroupRec] (device), or null
  int* vgroups;     // [ngroups][kVGroupRec] the groups as the plan accepted them
  int ngroups;      // groups given
  int gmem;         // sequences one group item serves (16 / G on the matrix cores; 0: no groups)
  int S, Hq, Hkv, G, max_blocks, num_blocks, PT, Pmax;
  int len_cap;      // min(max_blocks * B, max_ctx_len): longest context the call may see
  float scale_log2;
};

// Clamp a context length to what the table and the workspace can describe (len_cap);
// `bad` marks an invalid length, whose outputs become NaN.
__device__ __forceinline__ int eff_len(int n, int cap, bool& bad) {
  bad = (n < 1) || (n > cap);
  return n < 0 ? 0 : (n > cap ? cap : n);
}

// Element k of a 4-entry array by selects on constant indices: a runtime index into a local
// array makes the compiler keep the array in scratch memory (a 12% slower decode, measured).
__device__ __forceinline__ int pick4(const int (&v)[kGroupMembers], int k) {
  return k == 0 ? v[0] : k == 1 ? v[1] : k == 2 ? v[2] : v[3];
}

// ---------------------------------------------------------------------------------------
// Shared epilogue: merge the NW wave states held in LDS and store.
// s_ml[w][c] = (m, l); s_o[w][c][d] = unnormalised output of wave w relative to its own m, for
// the ncols columns of the item: column c is head c % G of member c / G.  A member with one
// partition gets its final output, the others a partial result in slot `slot`.
// ---------------------------------------------------------------------------------------
template <typename T, int D, int HMAX>
__device__ void finish_partition(const DecodeArgs& a, const int (&mem)[kGroupMembers],
                                 const int (&np)[kGroupMembers], int ncols, int kvh, int slot,
                                 bool bad, float (*s_ml)[HMAX][2], float (*s_o)[HMAX][D]) {
  // A thread finishes four consecutive dims of one column: the column's wave weights are
  // computed once for the four, the LDS reads and the store are 16-byte ones.  (One dim per
  // thread recomputed the weights per output and, with the member selected per output, took
  // 1.3-2.4 us per item beside the other workgroup's tiles.)
  constexpr int C4 = D / 4;
  const int G = a.G;
  for (int idx = threadIdx.x; idx < ncols * C4; idx += kNW * kWave) {
    const int c = idx / C4, d4 = idx - c * C4;
    const int j = (c >= G) + (c >= 2 * G) + (c >= 3 * G);  // member (at most four)
    const int h = c - j * G;
    const int s = j == 0 ? mem[0] : j == 1 ? mem[1] : j == 2 ? mem[2] : mem[3];
    const int nparts = j == 0 ? np[0] : j == 1 ? np[1] : j == 2 ? np[2] : np[3];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, s_ml[w][c][0]);
    float L = 0.f;
    f32x4 O = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float sc = exp2f(s_ml[w][c][0] - M);
      L += s_ml[w][c][1] * sc;
      O += *reinterpret_cast<const f32x4*>(&s_o[w][c][4 * d4]) * sc;
    }
    f32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = bad ? NAN : O[i] / L;
    const int hq = kvh * G + h;
    if (nparts == 1) {
      T* op = static_cast<T*>(a.out) + (static_cast<size_t>(s) * a.Hq + hq) * D + 4 * d4;
      if constexpr (sizeof(T) == 2) {
        const uint32_t lo = Elem<T>::from_f32(r[0]) | (uint32_t(Elem<T>::from_f32(r[1])) << 16);
        const uint32_t hi = Elem<T>::from_f32(r[2]) | (uint32_t(Elem<T>::from_f32(r[3])) << 16);
        *reinterpret_cast<uint2*>(op) = make_uint2(lo, hi);
      } else {
        *reinterpret_cast<f32x4*>(op) = r;
      }
    } else {
      // partials are written through to memory (agent scope): the workgroup that merges them
      // may run on another XCD, behind another L2
      const size_t row = (static_cast<size_t>(s) * a.Hq + hq) * a.Pmax + slot;
      st_agent2(a.part_o + row * D + 4 * d4, r[0], r[1]);
      st_agent2(a.part_o + row * D + 4 * d4 + 2, r[2], r[3]);
      if (d4 == 0) st_agent2(reinterpret_cast<float*>(a.part_ml + row), bad ? 0.f : M, bad ? NAN : L);
    }
  }
}

// ---------------------------------------------------------------------------------------
// Partition merge: m = max_p m_p; out = sum_p o_p l_p 2^(m_p - m) / sum_p l_p 2^(m_p - m).
// It runs in the decode kernel, in the workgroup that finishes the last partition of a
// (sequence, kv-head): each workgroup that stores a partial counts it in `done` once its
// stores are complete, and the one that brings the count to nparts merges.  Partials are
// stored and loaded with agent-scope accesses, which bypass the per-XCD L2s, so no cache
// write-back or invalidation is needed; the workgroups never wait on each other.
// The merging workgroup covers the G x D outputs, four consecutive dims per thread, summing
// partitions in index order (the result does not depend on which workgroup merges).
// ---------------------------------------------------------------------------------------
template <typename T, int D>
__device__ void merge_partials(const DecodeArgs& a, int s, int kvh, int nparts) {
  bool bad;
  (void)eff_len(a.ctx_lens[s], a.len_cap, bad);
  constexpr int C4 = D / 4;  // float4 chunks per head
  const size_t row0 = (static_cast<size_t>(s) * a.Hq + kvh * a.G) * a.Pmax;  // head 0, partition 0
  const int64_t o_bytes = static_cast<int64_t>(a.G) * a.Pmax * D * 4;
  if (o_bytes < (int64_t(1) << 31)) {
    // The partials are read with the device-scope cache bit an agent-scope atomic load carries
    // (sc1), but as plain buffer loads: the compiler issued the atomic loads one at a time,
    // each waiting for the previous, so a merge of many partitions became a serial tail
    // (32,768 tokens at batch 1: 128 partitions per head).  Buffer loads stay in flight
    // together, and an output chunk is one 16-byte load.
    constexpr int kSc1 = 16;  // cache-policy bit sc1 (gfx940+ encoding)
    const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
        a.part_ml + row0, 0, static_cast<int>(static_cast<int64_t>(a.G) * a.Pmax * 8), 0x00020000);
    const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
        a.part_o + row0 * D, 0, static_cast<int>(o_bytes), 0x00020000);
    for (int c = threadIdx.x; c < a.G * C4; c += kNW * kWave) {
      const int h = c / C4, d4 = c - h * C4;
      const int hr = h * a.Pmax;  // partition 0 of head h inside the (sequence, kv-head) block
      // groups of kGrp partitions: every load of a group is issued before any is used; the
      // indices of a short last group are clamped to the last partition and skipped
      constexpr int kGrp = 8;
      // up to kGrp partitions form one group: the max comes from the group's own loads below
      // (a separate pass of loads for the max cost one more round trip to memory per merge)
      const bool one_group = nparts <= kGrp;
      float M = -INFINITY;
      for (int p0 = 0; !one_group && p0 < nparts; p0 += kGrp) {
        float mv[kGrp];
#pragma unroll
        for (int k = 0; k < kGrp; ++k)
          mv[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                rm, (hr + min(p0 + k, nparts - 1)) * 8, 0, kSc1));
#pragma unroll
        for (int k = 0; k < kGrp; ++k) M = fmaxf(M, mv[k]);  // a clamped repeat changes nothing
      }
      float L = 0.f;
      float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int p0 = 0; p0 < nparts; p0 += kGrp) {
        decltype(__builtin_amdgcn_raw_buffer_load_b64(rm, 0, 0, 0)) mlv[kGrp];
        u32x4 ov[kGrp];
#pragma unroll
        for (int k = 0; k < kGrp; ++k) {
          const int r = hr + min(p0 + k, nparts - 1);
          mlv[k] = __builtin_amdgcn_raw_buffer_load_b64(rm, r * 8, 0, kSc1);
          ov[k] = __builtin_amdgcn_raw_buffer_load_b128(ro, (r * D + 4 * d4) * 4, 0, kSc1);
        }
        if (one_group) {
#pragma unroll
          for (int k = 0; k < kGrp; ++k) M = fmaxf(M, __uint_as_float(mlv[k][0]));
        }
#pragma unroll
        for (int k = 0; k < kGrp; ++k) {  // partitions in index order
          // a clamped repeat is dropped by selects (no branch, so the group's loads stay
          // together; no 0 * Inf either)
          const bool use = p0 + k < nparts;
          const float wgt = __uint_as_float(mlv[k][1]) * exp2f(__uint_as_float(mlv[k][0]) - M);
          L = use ? L + wgt : L;
          O.x = use ? fmaf(wgt, __uint_as_float(ov[k][0]), O.x) : O.x;
          O.y = use ? fmaf(wgt, __uint_as_float(ov[k][1]), O.y) : O.y;
          O.z = use ? fmaf(wgt, __uint_as_float(ov[k][2]), O.z) : O.z;
          O.w = use ? fmaf(wgt, __uint_as_float(ov[k][3]), O.w) : O.w;
        }
      }
      const float inv = bad ? NAN : 1.f / L;
      T* op = static_cast<T*>(a.out) + (static_cast<size_t>(s) * a.Hq + kvh * a.G + h) * D + 4 * d4;
      op[0] = Elem<T>::from_f32(O.x * inv);
      op[1] = Elem<T>::from_f32(O.y * inv);
      op[2] = Elem<T>::from_f32(O.z * inv);
      op[3] = Elem<T>::from_f32(O.w * inv);
    }
    return;
  }
  for (int c = threadIdx.x; c < a.G * C4; c += kNW * kWave) {
    const int h = c / C4, d4 = c - h * C4;
    const int hq = kvh * a.G + h;
    const size_t row = (static_cast<size_t>(s) * a.Hq + hq) * a.Pmax;
    const float* ml = reinterpret_cast<const float*>(a.part_ml + row);
    const float* po = a.part_o + row * D + 4 * d4;
    float M = -INFINITY;
    for (int p = 0; p < nparts; ++p) M = fmaxf(M, ld_agent(ml + 2 * p));
    float L = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int p = 0; p < nparts; ++p) {
      const float wgt = ld_agent(ml + 2 * p + 1) * exp2f(ld_agent(ml + 2 * p) - M);
      const float* v = po + static_cast<size_t>(p) * D;
      L += wgt;
      O.x = fmaf(wgt, ld_agent(v + 0), O.x);
      O.y = fmaf(wgt, ld_agent(v + 1), O.y);
      O.z = fmaf(wgt, ld_agent(v + 2), O.z);
      O.w = fmaf(wgt, ld_agent(v + 3), O.w);
    }
    const float inv = bad ? NAN : 1.f / L;
    T* op = static_cast<T*>(a.out) + (static_cast<size_t>(s) * a.Hq + hq) * D + 4 * d4;
    op[0] = Elem<T>::from_f32(O.x * inv);
    op[1] = Elem<T>::from_f32(O.y * inv);
    op[2] = Elem<T>::from_f32(O.z * inv);
    op[3] = Elem<T>::from_f32(O.w * inv);
  }
}

template <typename T, int D>
__device__ void merge_if_last(const DecodeArgs& a, int s, int kvh, int nparts) {
  __shared__ int s_last;
  if (nparts <= 1) return;
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(a.done + s * a.Hkv + kvh, 1) == nparts - 1;
  __syncthreads();
  if (s_last) merge_partials<T, D>(a, s, kvh, nparts);
}

// Start of a work item: its token range [t0, t1), partial slot and members come with the
// entry; read each member's number of partial results, the context length (for the bad-length
// check of a sequence's own item) and stage the slice of the block table the range needs in
// LDS.  The loads do not depend on each other, so they are in flight together.  A share-group
// item reads its first member's table: over the group's range the members hold the same K/V.
// Entries the range uses that lie outside the pool are replaced by block 0 (every load stays
// inside the pool) and flag the item as bad.
struct ItemRange {
  int t0, t1, b0, slot, nmem;
  int mem[kGroupMembers], np[kGroupMembers];
  int tail[kGroupMembers];  // fused tail of each member: its tokens [t1, t1 + tail)
  bool bad;
};

// Table entries staged for one member's fused tail (tokens t1 .. t1 + kFuseTail - 1).
template <int B>
constexpr int kTailTbl = kFuseTail / B + 1;

// The item's loads (all independent of each other, in flight together), kept in registers
// until begin_stage writes them to LDS.
template <int B>
struct ItemLoad {
  static constexpr int kTbl = kMaxPT / B + 1;  // a range may start inside a block
  static constexpr int kPer = (kTbl + kNW * kWave - 1) / (kNW * kWave);
  ItemRange it;
  int nb;         // table entries of the range
  int ent[kPer];  // thread's entries i = threadIdx.x + r * threads
  int tent;       // fused-tail entry (thread (tj, ti)); -1 past the table row: block 0, NaN out
  bool tneed, bad_len;
};

template <int B>
__device__ __forceinline__ ItemLoad<B> begin_load(const DecodeArgs& a, const int4 e0,
                                                  const int4 e1, bool tails) {
  using L = ItemLoad<B>;
  L ld;
  ItemRange& it = ld.it;
  it.t0 = e0.z;
  it.t1 = e0.w;
  it.slot = e0.y;
  // a member slot: the sequence in the low 16 bits, its fused tail length above (-1: none)
  const int c4[kGroupMembers] = {e1.x, e1.y, e1.z, e1.w};
#pragma unroll
  for (int k = 0; k < kGroupMembers; ++k) {
    it.mem[k] = c4[k] < 0 ? -1 : (c4[k] & 0xFFFF);
    it.tail[k] = c4[k] < 0 ? 0 : (c4[k] >> 16);
  }
  it.nmem = 1 + (e1.y >= 0) + (e1.z >= 0) + (e1.w >= 0);
  it.bad = false;
  const int s = it.mem[0];
  const bool own = e0.x >= 0;
  const int raw_n = own ? a.ctx_lens[s] : 1;
  it.b0 = it.t0 / B;
  int nb = it.t1 > it.t0 ? (it.t1 - 1) / B - it.b0 + 1 : 0;
  ld.nb = min(nb, a.max_blocks - it.b0);
  const int32_t* row = a.tables + static_cast<size_t>(s) * a.max_blocks + it.b0;
#pragma unroll
  for (int r = 0; r < L::kPer; ++r) {
    const int i = threadIdx.x + r * kNW * kWave;
    ld.ent[r] = i < ld.nb ? row[i] : 0;
  }
#pragma unroll
  for (int k = 0; k < kGroupMembers; ++k) it.np[k] = it.mem[k] >= 0 ? a.nparts[it.mem[k]] : 0;
  // fused tails: thread (j, i) loads entry i of member j's blocks from t1 on
  constexpr int kTT = kTailTbl<B>;
  const int tj = static_cast<int>(threadIdx.x) / kTT, ti = static_cast<int>(threadIdx.x) - tj * kTT;
  ld.tent = -1;
  ld.tneed = false;
  if (tails && tj < kGroupMembers) {
    const int tl = pick4(it.tail, tj);
    const int cnt = tl > 0 ? (it.t1 + tl - 1) / B - it.t1 / B + 1 : 0;
    ld.tneed = ti < cnt;
    if (ld.tneed && it.t1 / B + ti < a.max_blocks)
      ld.tent = a.tables[static_cast<size_t>(pick4(it.mem, tj)) * a.max_blocks + it.t1 / B + ti];
  }
  ld.bad_len = false;
  if (own) (void)eff_len(raw_n, a.len_cap, ld.bad_len);
  return ld;
}

// Write the loaded entries to LDS.  *s_bad must have been cleared before a barrier that
// precedes this call; after the next barrier it is 1 when an entry lay outside the pool.
template <int B>
__device__ __forceinline__ void begin_stage(const DecodeArgs& a, const ItemLoad<B>& ld,
                                            int* s_tbl, int* s_bad, int* s_tail) {
  using L = ItemLoad<B>;
  bool bad_ent = false;
#pragma unroll
  for (int r = 0; r < L::kPer; ++r) {
    const int i = threadIdx.x + r * kNW * kWave;
    if (i < ld.nb) {
      int p = ld.ent[r];
      if (p < 0 || p >= a.num_blocks) {
        bad_ent = true;
        p = 0;
      }
      s_tbl[i] = p;
    }
  }
  if (ld.tneed) {
    constexpr int kTT = kTailTbl<B>;
    const int tj = static_cast<int>(threadIdx.x) / kTT, ti = static_cast<int>(threadIdx.x) - tj * kTT;
    int tent = ld.tent;
    if (tent < 0 || tent >= a.num_blocks) {
      bad_ent = true;
      tent = 0;
    }
    s_tail[tj * kTT + ti] = tent;
  }
  if (bad_ent) *s_bad = 1;
}

template <int B>
__device__ __forceinline__ ItemRange begin_item(const DecodeArgs& a, const int4 e0, const int4 e1,
                                                int* s_tbl, int* s_bad, int* s_tail) {
  const ItemLoad<B> ld = begin_load<B>(a, e0, e1, s_tail != nullptr);
  if (threadIdx.x == 0) *s_bad = 0;
  __syncthreads();
  begin_stage<B>(a, ld, s_tbl, s_bad, s_tail);
  __syncthreads();
  ItemRange it = ld.it;
  it.bad = ld.bad_len || *s_bad;
  return it;
}

// Persistent work loop.  Workgroup g starts with item g; the next item is claimed near the
// end of the current one, so the atomic's latency hides behind its epilogue; every workgroup
// leaves once the claims pass the item count.  Two ways to claim, chosen by the planner (queue[1]):
//   * one global cursor (queue[10]): every workgroup takes the next item of the longest-first
//     list, so the XCDs balance among themselves;
//   * one queue per XCD (queue[2 + x]), for batches whose sequences share prefix blocks.  The
//     dispatcher deals workgroups round-robin to the kXcd XCDs, so workgroup g runs on XCD
//     g % kXcd; queue x holds the items i = c * kXcd + x, c = 0, 1, ... (every kXcd-th item of
//     the list).  With kXcd | Hkv those are exactly the items of the kv-heads h = x
//     (mod kXcd): a kv-head's blocks are read through one XCD's L2, where the shared prefix
//     blocks stay resident.
template <typename Body>
__device__ __forceinline__ void for_each_item(const DecodeArgs& a, int* s_next, Body&& body) {
  const int count = a.queue[0];
  const bool per_xcd = a.queue[1] != 0;
  const int x = static_cast<int>(blockIdx.x % kXcd);
  int i = blockIdx.x;
  while (i < count) {
    // The body calls claim() once it is nearly done (thread 0 takes the next item); a claim
    // taken a whole item ahead commits the workgroup to work that an idle one could run, and
    // with items of up to 2048 tokens that shows as a ragged end (1-5% of the decode).
    int nxt = 0;
    bool claimed = false;
    auto claim = [&] {
      if (threadIdx.x == 0 && !claimed) {
        nxt = per_xcd ? atomicAdd(&a.queue[2 + x], 1) * kXcd + x : atomicAdd(&a.queue[2 + kXcd], 1);
        claimed = true;
      }
    };
    const int e = i / a.Hkv;
    const int4 e0 = a.items[2 * e], e1 = a.items[2 * e + 1];
    body(e0, e1, i % a.Hkv, claim);
    claim();  // a body that had no tile for wave 0
    if (threadIdx.x == 0) *s_next = nxt;
    __syncthreads();
    i = __builtin_amdgcn_readfirstlane(*s_next);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------------------
// MFMA kernel: bf16, 1 <= G <= 16 query heads per kv-head, D in {64, 128}, B in {16, 32, 64}.
//
// A wave walks its partition in tiles of 32 tokens (tiles w, w + NW, ...).  Per tile a lane
// holds D/32 16-byte pieces of K as loaded (whole key rows, 1 KB contiguous per instruction)
// and D/16 pieces of V^T.  The K tile is re-laid out into the QK^T operand through the wave's
// LDS slot; V^T pieces are already in the PV operand layout.  The loads are staggered so that
// one register set keeps a full tile in flight: the next tile's K is issued as soon as the
// current K is staged, the next V as soon as PV has consumed the current V.  Two waves per SIMD
// (8 per CU): at three the register budget spills, measured slower.
// ---------------------------------------------------------------------------------------
constexpr float kLazyRescale = 8.f;  // log2 units: weights stay below 256
constexpr int kMfmaWaves = 2;  // waves per SIMD the register budget is cut for (256 VGPRs)

template <int D>
struct MfmaK {
  static constexpr int CH = D / 8;       // 16-byte chunks per key row
  static constexpr int TPI = kWave / CH;  // tokens per contiguous load instruction
  static constexpr int NI = 32 / TPI;     // load instructions per 32-token tile
  bf16x8 raw[NI];                         // the tile as loaded: 1 KB contiguous per instruction
};
template <int D>
struct MfmaV {
  bf16x8 v[D / 16];     // V^T rows (16 dims per tile) x 8 tokens of this lane group
};

// A segment of tokens [t0, t1) read through table entries tbl[] of logical blocks from b0 on:
// an item's range, or one member's fused tail.
struct Seg {
  int t0, t1, b0;
  const int* tbl;
};

// KEEP: K/V loaded without the non-temporal hint (the plan saw blocks shared by several
// sequences; their lines are read again by other items).
//
// K is loaded in whole rows (instruction i covers tokens TPI*i .. TPI*i + TPI-1 of the tile,
// 1 KB contiguous; the matrix-core layout would read 16 rows x 64 B per instruction, measured
// 5% slower) and re-laid out through the wave's LDS slot.  Tokens past the end repeat the
// last live token; their scores are masked.  Token indices are taken unsigned (they are never
// negative), so block and offset are a shift and a mask: the signed forms cost four more
// instructions per load (Mistral-7B-shaped batch 0.1091-0.1101 -> 0.1074-0.1079 ms).
template <int D, int B, bool KEEP>
__device__ __forceinline__ void load_k_tile(const DecodeArgs& a, MfmaK<D>& kt, const Seg& sg,
                                            int tile, int kvh) {
  using KT = MfmaK<D>;
  const int lane = threadIdx.x & (kWave - 1);
  const uint16_t* kc = static_cast<const uint16_t*>(a.kc);
  const size_t head_stride = static_cast<size_t>(B) * D;  // elements per (block, kv-head)
  const int tt = sg.t0 + 32 * tile;
  if ((tt & 31) == 0 && tt + 32 <= sg.t1) {  // uniform: a whole aligned tile, nothing to clamp
    // The tile's 32 tokens lie in NB consecutive blocks (B = 16: two; B >= 32: one), so one
    // table entry and one address per block serve its loads, which differ by constant offsets.
    constexpr int NB = B >= 32 ? 1 : 32 / B;
    constexpr int PER = KT::NI / NB;  // loads per block
    const size_t lane_off = static_cast<size_t>(lane / KT::CH) * D + 8 * (lane % KT::CH);
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
      const int p = sg.tbl[tt / B + bi - sg.b0];
      const uint16_t* bp = kc + (static_cast<size_t>(p) * a.Hkv + kvh) * head_stride +
                           static_cast<size_t>(tt % B) * D + lane_off;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const uint16_t* kp = bp + static_cast<size_t>(KT::TPI * i) * D;
        kt.raw[bi * PER + i] = KEEP ? ld_kv16_keep(kp) : ld_kv16(kp);
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < KT::NI; ++i) {
    const unsigned tok = static_cast<unsigned>(min(tt + KT::TPI * i + lane / KT::CH, sg.t1 - 1));
    const int p = sg.tbl[static_cast<int>(tok / B) - sg.b0];
    const uint16_t* kp = kc + (static_cast<size_t>(p) * a.Hkv + kvh) * head_stride +
                         static_cast<size_t>(tok % B) * D;
    kt.raw[i] = KEEP ? ld_kv16_keep(kp + 8 * (lane % KT::CH)) : ld_kv16(kp + 8 * (lane % KT::CH));
  }
}

// V^T rows: lane (gp, r16) reads dim 16*ni + r16 at tokens 8*gp .. 8*gp+7 of the tile
// (16 contiguous bytes of the transposed block).
template <int D, int B, bool KEEP>
__device__ __forceinline__ void load_v_tile(const DecodeArgs& a, MfmaV<D>& vt, const Seg& sg,
                                            int tile, int kvh) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r16 = lane & 15, gp = lane >> 4;
  const uint16_t* vc = static_cast<const uint16_t*>(a.vc);
  const size_t head_stride = static_cast<size_t>(B) * D;
  const unsigned tv = static_cast<unsigned>(min(sg.t0 + 32 * tile + 8 * gp, (sg.t1 - 1) & ~7));
  const int p = sg.tbl[static_cast<int>(tv / B) - sg.b0];
  const uint16_t* vp = vc + (static_cast<size_t>(p) * a.Hkv + kvh) * head_stride + (tv % B);
  // At B = 64 a V^T row is 128 bytes and a 32-token tile reads half of it; the other half is
  // another wave's tile, read at about the same time.  A non-temporal load lets the line go
  // before that second read (HBM reads were 27% above the algorithmic bytes), so these loads
  // are ordinary ones: 0.378 -> 0.325 ms on the Llama-3-70B-shaped batch at B = 64.  At
  // B <= 32 each line is used whole by one load instruction and non-temporal stays faster.
#pragma unroll
  for (int ni = 0; ni < D / 16; ++ni)
    vt.v[ni] = (KEEP || B == 64) ? ld_kv16_keep(vp + (16 * ni + r16) * B)
                                 : ld_kv16(vp + (16 * ni + r16) * B);
}

// Q^T operand: column r16 = head r16 % G of member r16 / G (zero past the item's members),
// k = 8 dims per step.  A sequence's own item has one member; a share-group item up to 16 / G.
template <int D>
__device__ __forceinline__ void load_qop(const DecodeArgs& a, const int4 e1, int kvh,
                                         bf16x8 (&qop)[D / 32]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int r16 = lane & 15, gp = lane >> 4;
  const int j = r16 / a.G, h = r16 - j * a.G;
  const int cj = j == 0 ? e1.x : j == 1 ? e1.y : j == 2 ? e1.z : j == 3 ? e1.w : -1;
  const bool live = cj >= 0;
  const int mj = live ? (cj & 0xFFFF) : (e1.x & 0xFFFF);  // low 16 bits: the sequence
  const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                       (static_cast<size_t>(mj) * a.Hq + kvh * a.G + (live ? h : 0)) * D;
#pragma unroll
  for (int st = 0; st < D / 32; ++st) {
    uint4 u = *reinterpret_cast<const uint4*>(qp + 8 * (4 * st + gp));
    if (!live) u = make_uint4(0, 0, 0, 0);
    qop[st] = __builtin_bit_cast(bf16x8, u);
  }
}

// A workgroup's current item and what was loaded for it before its tiles start: the entry, the
// range (table slice staged in LDS) and the Q^T operand; kt / vt are the wave's tile registers.
// (Loading this wave's first tile of the next item during the epilogue as well kept the tile
// registers live through the merge: 48-56 bytes of scratch per lane.)
template <int D>
struct MfmaCur {
  int4 e0, e1;
  int kvh;
  ItemRange rg;
  bf16x8 qop[D / 32];
  MfmaK<D> kt;
  MfmaV<D> vt;
};

// Shared state of the persistent loop.
template <int D>
struct MfmaShared {
  int* tbl;
  int* tail;
  int* bad;
  int* next;
  int* last;
  float (*ml)[16][2];
  float (*o)[16][D];
};

// One item: its tiles, then an epilogue that overlaps the item's completion with the next
// item's start.  Item start-up (entry, table slice, first tile: three dependent round trips to
// memory) and completion (partial stores, done counter, merge loads: three more) cost 8-9 us
// per item when run one after the other; a workgroup spent about a fifth of a Mistral-7B-shaped
// decode there.  The epilogue therefore issues the next item's entry load before the wave
// states are merged, the next item's table, context length and Q loads together with the
// partial stores, and its table staging together with the done counters, so the waits overlap.
// Returns the next item index.
template <int D, int B, bool KEEP>
__device__ __forceinline__ int mfma_item(const DecodeArgs& a, MfmaCur<D>& c,
                                         const MfmaShared<D>& sh, int count, bool per_xcd) {
  constexpr int NST = D / 32, NNT = D / 16;
  const int lane = threadIdx.x & (kWave - 1), w = wave_id();
  const int r16 = lane & 15, gp = lane >> 4;
  const ItemRange rg = c.rg;
  const int kvh = c.kvh;
  const int t0 = rg.t0, t1 = rg.t1, b0 = rg.b0;
  const Seg main_seg{t0, t1, b0, sh.tbl};

  float m_run = -INFINITY, l_run = 0.f;
  float m_use = 0.f;  // the reference the weights are taken against: m_run once finite
  f32x4 o[NNT];
#pragma unroll
  for (int i = 0; i < NNT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = t1 > t0 ? (t1 - t0 + 31) / 32 : 0;

  using KT = MfmaK<D>;
  unsigned char* kstage = reinterpret_cast<unsigned char*>(&sh.o[w][0][0]);
  static_assert(sizeof(sh.o[0]) >= 32 * D * 2, "the wave's output slot holds a K tile");
  // Stage the tile (row = token of the tile, chunks permuted by kswz) and read back the QK^T
  // operand: row r16 of row group m holds token 8*(r16/4) + 4*m + r16%4 of the tile, so that
  // after QK^T lane group gp owns tokens 8*gp .. 8*gp+7 (the PV operand layout).  The wave
  // reads back what it wrote (LDS operations of one wave complete in order).
  auto stage_k = [&](const KT& kt) {
#pragma unroll
    for (int i = 0; i < KT::NI; ++i) {
      const int row = KT::TPI * i + lane / KT::CH, ch = lane % KT::CH;
      *reinterpret_cast<bf16x8*>(kstage + row * (D * 2) + ((ch ^ kswz<D>(row)) << 4)) = kt.raw[i];
    }
  };
  auto k_operand = [&](int m, bf16x8 (&kop)[NST]) {
    const int row = 8 * (r16 >> 2) + 4 * m + (r16 & 3);
#pragma unroll
    for (int st = 0; st < NST; ++st)
      kop[st] = *reinterpret_cast<const bf16x8*>(
          kstage + row * (D * 2) + (((4 * st + gp) ^ kswz<D>(row)) << 4));
  };

  // One tile of segment sg: QK^T on kt, refill kt with tile `pf` of segment nsg (when `more`),
  // softmax, PV on vt, refill vt.  col_ok: this lane's column takes part (false for the other
  // members' columns while a member's fused tail is read).
  auto step = [&](MfmaK<D>& kt, MfmaV<D>& vt, const Seg& sg, int tile, bool col_ok,
                  const Seg& nsg, int pf, bool more) {
    const int tt = sg.t0 + 32 * tile;
    stage_k(kt);
    if (more) load_k_tile<D, B, KEEP>(a, kt, nsg, pf, kvh);  // the raw registers are free once staged
    f32x4 sacc[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      bf16x8 kop[NST];
      k_operand(m, kop);
      sacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NST; ++st)
        sacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[st], c.qop[st], sacc[m], 0, 0, 0);
    }

    // lane (gp, r16): scores of head r16 for tokens tt + 8*gp + j, j = 4*m + i
    const int valid = sg.t1 - (tt + 8 * gp);  // tokens of this lane's group that exist
    // raw scores; the scale (> 0, checked on the host) is applied inside the exponent
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = col_ok ? sacc[j >> 2][j & 3] : -INFINITY;
    if (sg.t1 - tt < 32) {  // uniform: the segment's last tile holds tokens past its end
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = j < valid ? x[j] : -INFINITY;
    }
    // column max over the 32 tokens: this lane's 8, then its xor-16 and xor-32 partners
    float mx = vmax(vmax3(x[0], x[1], x[2]), vmax3(x[3], x[4], vmax3(x[5], x[6], x[7])));
    mx = max_xor32(max_xor16(mx)) * a.scale_log2;
    // Lazy rescaling: a column's reference max m_run moves only when a score exceeds it by
    // more than kLazyRescale (log2 units), so its weights stay below 2^kLazyRescale and the
    // accumulators are rescaled on few tiles; the final division by the sum makes the result
    // the same softmax.  A column with no score yet (m_run = -inf: a masked member column of
    // a fused tail) keeps reference 0, so no -inf - -inf arises.
    if (__builtin_amdgcn_ballot_w64(mx > m_run + kLazyRescale)) {  // uniform
      const bool up = mx > m_run + kLazyRescale;
      const float alpha = up ? fast_exp2(m_run - mx) : 1.f;  // 0 on a column's first score
      m_run = up ? mx : m_run;
      m_use = up ? mx : m_use;
      l_run *= alpha;
#pragma unroll
      for (int ni = 0; ni < NNT; ++ni) o[ni] *= alpha;
    }
    bf16x8 pop;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      pop[j] = static_cast<__bf16>(fast_exp2(fmaf(x[j], a.scale_log2, -m_use)));
    // the sum takes the same bf16 weights the numerator uses
#pragma unroll
    for (int i = 0; i < 4; ++i)
      l_run = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pop[2 * i], pop[2 * i + 1]}, kOnes2, l_run,
                                              false);
    if (valid < 8) {  // tail: zero the V elements of tokens past the end (0 * NaN = NaN)
#pragma unroll
      for (int ni = 0; ni < NNT; ++ni) {
        uint16_t vv[8];
        __builtin_memcpy(vv, &vt.v[ni], 16);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j >= valid) vv[j] = 0;
        __builtin_memcpy(&vt.v[ni], vv, 16);
      }
    }
#pragma unroll
    for (int ni = 0; ni < NNT; ++ni)
      o[ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt.v[ni], pop, o[ni], 0, 0, 0);
    if (more) load_v_tile<D, B, KEEP>(a, vt, nsg, pf, kvh);
  };

  // The wave's tiles are w, w + NW, ...  (A second register set, two tiles in flight at two
  // waves per SIMD, measured no faster than one set at three waves per SIMD.)
  if (w < ntiles) {
    load_k_tile<D, B, KEEP>(a, c.kt, main_seg, w, kvh);
    load_v_tile<D, B, KEEP>(a, c.vt, main_seg, w, kvh);
    for (int tile = w; tile < ntiles; tile += kNW)
      step(c.kt, c.vt, main_seg, tile, true, main_seg, tile + kNW, tile + kNW < ntiles);
  }

  // Fused tails (a share-group item that ends its range): member j's own tokens [t1, t1 +
  // tail_j), read through its staged table entries, with only member j's columns live.  The
  // tail tiles of all members are numbered member after member; wave w takes g = w, w + NW, ...
  const int nt0 = (rg.tail[0] + 31) / 32, nt1 = (rg.tail[1] + 31) / 32;
  const int nt2 = (rg.tail[2] + 31) / 32, nt3 = (rg.tail[3] + 31) / 32;
  const int ntail = nt0 + nt1 + nt2 + nt3;  // uniform: 0 on every other item
  if (w < ntail) {
    constexpr int kTT = kTailTbl<B>;
    auto seg_of = [&](int g, Seg& sg, int& k, int& j) {
      j = g < nt0 ? 0 : g < nt0 + nt1 ? 1 : g < nt0 + nt1 + nt2 ? 2 : 3;
      k = g - (j == 0 ? 0 : j == 1 ? nt0 : j == 2 ? nt0 + nt1 : nt0 + nt1 + nt2);
      sg = Seg{t1, t1 + pick4(rg.tail, j), t1 / B, sh.tail + j * kTT};
    };
    // (the main range's tile registers are free again)
    Seg sg;
    int k, j;
    seg_of(w, sg, k, j);
    load_k_tile<D, B, KEEP>(a, c.kt, sg, k, kvh);
    load_v_tile<D, B, KEEP>(a, c.vt, sg, k, kvh);
    for (int g = w; g < ntail; g += kNW) {
      Seg ns;
      int nk, nj;
      seg_of(min(g + kNW, ntail - 1), ns, nk, nj);
      const bool col_ok = r16 >= j * a.G && r16 < (j + 1) * a.G;
      step(c.kt, c.vt, sg, k, col_ok, ns, nk, g + kNW < ntail);
      sg = ns;
      k = nk;
      j = nj;
    }
  }

  // Wave 0 is done with its tiles: claim the next item now (thread 0), so the atomic's latency
  // hides behind the wave-state merge.  A claim taken a whole item ahead commits the workgroup
  // to work that an idle one could run, and with items of up to 2048 tokens that shows as a
  // ragged end (claiming at the start of the item measured 1-5% slower; one or two tiles early,
  // the same or up to 1% slower on long contexts).
  int nxt = 0;
  if (threadIdx.x == 0) {
    const int x = static_cast<int>(blockIdx.x % kXcd);
    nxt = per_xcd ? atomicAdd(&a.queue[2 + x], 1) * kXcd + x : atomicAdd(&a.queue[2 + kXcd], 1);
  }
  // Wave state -> LDS.  l_run is per lane (its 8 tokens); sum the four lane groups.
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  if (gp == 0) {
    sh.ml[w][r16][0] = m_run;
    sh.ml[w][r16][1] = l_run;
  }
#pragma unroll
  for (int ni = 0; ni < NNT; ++ni)
#pragma unroll
    for (int i = 0; i < 4; ++i) sh.o[w][r16][16 * ni + 4 * gp + i] = o[ni][i];
  if (threadIdx.x == 0) *sh.next = nxt;
  __syncthreads();
  const int ni = __builtin_amdgcn_readfirstlane(*sh.next);
  const bool more = ni < count;
  int4 ne0 = make_int4(0, 0, 0, 0), ne1 = make_int4(0, 0, 0, 0);
  if (more) {
    const int e = ni / a.Hkv;
    ne0 = a.items[2 * e];
    ne1 = a.items[2 * e + 1];
  }
  finish_partition<uint16_t, D, 16>(a, rg.mem, rg.np, rg.nmem * a.G, kvh, rg.slot, rg.bad, sh.ml, sh.o);
  // members with partial results count them once this thread's stores have completed
  bool split = false;
#pragma unroll
  for (int k = 0; k < kGroupMembers; ++k) split = split || (rg.mem[k] >= 0 && rg.np[k] > 1);
  const int nkvh = more ? ni % a.Hkv : 0;
  ItemLoad<B> nl;
  bf16x8 nq[NST];
  if (more) {
    nl = begin_load<B>(a, ne0, ne1, true);
    load_qop<D>(a, ne1, nkvh, nq);
  }
  if (split) __builtin_amdgcn_s_waitcnt(0);
  if (threadIdx.x == 0) *sh.bad = 0;
  __syncthreads();  // partial stores complete; the wave states and the table slice are free
  int last = 0;
  if (split && threadIdx.x == 0) {
#pragma unroll
    for (int k = 0; k < kGroupMembers; ++k) {
      const int s = pick4(rg.mem, k), np = pick4(rg.np, k);
      if (s >= 0 && np > 1 && atomicAdd(a.done + s * a.Hkv + kvh, 1) == np - 1) last |= 1 << k;
    }
  }
  if (more) begin_stage<B>(a, nl, sh.tbl, sh.bad, sh.tail);
  if (threadIdx.x == 0) *sh.last = last;
  __syncthreads();
  last = __builtin_amdgcn_readfirstlane(*sh.last);
  if (more) {
    c.e0 = ne0;
    c.e1 = ne1;
    c.kvh = nkvh;
    c.rg = nl.it;
    c.rg.bad = nl.bad_len || *sh.bad;
#pragma unroll
    for (int st = 0; st < NST; ++st) c.qop[st] = nq[st];
  }
#pragma unroll
  for (int k = 0; k < kGroupMembers; ++k)
    if ((last >> k) & 1) merge_partials<uint16_t, D>(a, pick4(rg.mem, k), kvh, pick4(rg.np, k));
  return ni;
}

template <int D, int B>
__global__ __launch_bounds__(kNW * kWave) __attribute__((amdgpu_waves_per_eu(kMfmaWaves)))
void decode_mfma_kernel(DecodeArgs a) {
  a.PT = a.queue[kPtSlot];      // the plan's choice
  a.Pmax = a.queue[kPmaxSlot];  // partial results packed for it
  // s_o doubles as each wave's K staging slot, read and written in 16-byte vectors: keep it
  // (and the rest) 16-byte aligned whatever the table slice's size
  __shared__ __attribute__((aligned(16))) int s_tbl[kMaxPT / B + 1];
  __shared__ int s_tail[kGroupMembers * kTailTbl<B>];  // fused tails' table entries
  __shared__ int s_bad, s_next, s_last;
  __shared__ __attribute__((aligned(16))) float s_ml[kNW][16][2];
  __shared__ __attribute__((aligned(16))) float s_o[kNW][16][D];
  // A batch whose sequences share prefix blocks (the plan's sharing test, which also picks
  // the per-XCD queues) keeps K/V lines in cache: each shared line is read by many items of
  // the same kv-head on one XCD, and a non-temporal load marks it to leave first.  Shared-
  // prefix batches: 0.1975 -> 0.183 ms (B = 16), 0.205 -> 0.190 ms (B = 32); on a batch with
  // no sharing the hint is worth 11% (Llama-3-70B-shaped batch 0.296 vs 0.33 ms without it).
  // With share groups the re-read blocks are the groups' ranges: only share-group items keep
  // their lines; a sequence's own tokens are read once and stay non-temporal (shared-prefix
  // batch with groups: 0.1656 -> 0.1423 ms against keeping every item's lines).
  const bool keep = a.queue[1] != 0;
  const bool grouped = a.gmem > 0 && a.ngroups > 0;
  const int count = a.queue[0];
  // Persistent loop: workgroup g starts with item g and claims the next one near the end of
  // each item (see for_each_item for the two ways to claim); every workgroup leaves once the
  // claims pass the item count.
  int i = blockIdx.x;
  if (i >= count) return;
  const MfmaShared<D> sh{s_tbl, s_tail, &s_bad, &s_next, &s_last, s_ml, s_o};
  MfmaCur<D> c;
  {
    const int e = i / a.Hkv;
    c.e0 = a.items[2 * e];
    c.e1 = a.items[2 * e + 1];
    c.kvh = i % a.Hkv;
    load_qop<D>(a, c.e1, c.kvh, c.qop);
    c.rg = begin_item<B>(a, c.e0, c.e1, s_tbl, &s_bad, s_tail);
  }
  do {
    if (keep && (!grouped || c.e0.x < 0))
      i = mfma_item<D, B, true>(a, c, sh, count, keep);
    else
      i = mfma_item<D, B, false>(a, c, sh, count, keep);
  } while (i < count);
}

// ---------------------------------------------------------------------------------------
// VALU kernel: T in {float, bf16 bits}, G in {1, 2, 4, 8}; LPT lanes per token.
//
// A round covers TPR = 64 / LPT consecutive tokens (inside one block).  Lane (tk, pp) holds
// a 1/LPT slice of token tk's key row; the dot products are finished with xor-shuffles over
// the LPT lanes, the round max with xor-shuffles over the tokens.  For P.V each lane owns
// D / 64 dims and reads their V^T rows (TPR contiguous tokens); the TPR weights of the round
// are broadcast through a per-wave LDS slot.
// ---------------------------------------------------------------------------------------
template <typename T, int D, int B, int G, int LPT, int TPR>
__device__ __forceinline__ void valu_item(const DecodeArgs& a, const int4 e0, const int4 e1,
                                          int kvh, int* s_tbl, int* s_bad, float (*s_ml)[G][2],
                                          float (*s_o)[G][D], float (*s_p)[G][TPR]) {
  const int s = e1.x;  // no share groups on this kernel: always the sequence's own item
  constexpr int VEC = 16 / sizeof(T);   // elements per 16-byte load
  constexpr int CPL = D / LPT / VEC;    // 16-byte chunks of a key row per lane
  constexpr int DPL = CPL * VEC;        // dims per lane in QK
  constexpr int DV = D / kWave;         // dims per lane in PV
  constexpr int VPR = TPR * sizeof(T) / 16;  // 16-byte loads per V^T row piece
  static_assert(TPR == kWave / LPT, "tokens per round");
  static_assert(CPL >= 1, "head_dim too small for LPT");
  static_assert(B % TPR == 0, "a round must stay inside one block");
  static_assert(VPR >= 1 && TPR % 4 == 0, "V rows are read in 16-byte pieces");

  const int lane = threadIdx.x & (kWave - 1), w = wave_id();
  const int tk = lane / LPT, pp = lane % LPT;
  const T* kc = static_cast<const T*>(a.kc);
  const T* vc = static_cast<const T*>(a.vc);

  // q slice of this lane, pre-scaled into the log2 domain.
  float qr[G][DPL];
  {
    const T* qp = static_cast<const T*>(a.q) + (static_cast<size_t>(s) * a.Hq + kvh * G) * D;
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        const uint4 u = *reinterpret_cast<const uint4*>(qp + h * D + (pp + LPT * i) * VEC);
        T e[VEC];
        __builtin_memcpy(e, &u, 16);
#pragma unroll
        for (int j = 0; j < VEC; ++j) qr[h][i * VEC + j] = Elem<T>::to_f32(e[j]) * a.scale_log2;
      }
  }

  const ItemRange rg = begin_item<B>(a, e0, e1, s_tbl, s_bad, nullptr);
  const int t0 = rg.t0, t1 = rg.t1, b0 = rg.b0;

  float m_run[G], l_run[G], acc[G][DV];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DV; ++e) acc[h][e] = 0.f;
  }

  const size_t head_stride = static_cast<size_t>(B) * D;
  const int nrounds = t1 > t0 ? (t1 - t0 + TPR - 1) / TPR : 0;

  for (int r = w; r < nrounds; r += kNW) {
    const int tt = t0 + TPR * r;
    // ---- loads: this lane's key slice (clamped to a live token) and its V^T rows
    const unsigned tok = static_cast<unsigned>(min(tt + tk, t1 - 1));  // >= 0
    const int pk = s_tbl[static_cast<int>(tok / B) - b0];
    const T* kp = kc + (static_cast<size_t>(pk) * a.Hkv + kvh) * head_stride + static_cast<size_t>(tok % B) * D;
    uint4 kr[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) kr[i] = *reinterpret_cast<const uint4*>(kp + (pp + LPT * i) * VEC);
    const unsigned tu = static_cast<unsigned>(tt);
    const int pv = s_tbl[static_cast<int>(tu / B) - b0];
    const T* vp = vc + (static_cast<size_t>(pv) * a.Hkv + kvh) * head_stride + (tu % B);
    T vv[DV][TPR];
#pragma unroll
    for (int e = 0; e < DV; ++e)
#pragma unroll
      for (int c = 0; c < VPR; ++c) {
        const uint4 u = *reinterpret_cast<const uint4*>(vp + static_cast<size_t>(lane + kWave * e) * B + c * VEC);
        __builtin_memcpy(&vv[e][c * VEC], &u, 16);
      }

    // ---- scores of the round (log2 domain); tokens past the end get -inf
    const bool valid = tt + tk < t1;
    float x[G];
#pragma unroll
    for (int h = 0; h < G; ++h) x[h] = 0.f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      T e[VEC];
      __builtin_memcpy(e, &kr[i], 16);
#pragma unroll
      for (int j = 0; j < VEC; ++j) {
        const float kv = Elem<T>::to_f32(e[j]);
#pragma unroll
        for (int h = 0; h < G; ++h) x[h] = fmaf(qr[h][i * VEC + j], kv, x[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int off = 1; off < LPT; off <<= 1) x[h] += shfl_xor(x[h], off);
      if (!valid) x[h] = -INFINITY;
    }
    // V elements of tokens past the end may hold anything (even NaN): zero them.
    const int nv = t1 - tt;
    if (nv < TPR) {
#pragma unroll
      for (int e = 0; e < DV; ++e)
#pragma unroll
        for (int j = 0; j < TPR; ++j)
          if (j >= nv) vv[e][j] = T(0);
    }

    // ---- online softmax update and P.V
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = x[h];
#pragma unroll
      for (int off = LPT; off < kWave; off <<= 1) mx = fmaxf(mx, shfl_xor(mx, off));
      const float m_new = fmaxf(m_run[h], mx);  // finite: the round has a live token
      const float alpha = exp2f(m_run[h] - m_new);
      m_run[h] = m_new;
      const float p = exp2f(x[h] - m_new);
      l_run[h] = l_run[h] * alpha + (pp == 0 ? p : 0.f);
      if (pp == 0) s_p[w][h][tk] = p;
#pragma unroll
      for (int e = 0; e < DV; ++e) acc[h][e] *= alpha;
    }
    // The wave reads back what it just wrote (LDS ops of one wave complete in order).
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int j4 = 0; j4 < TPR / 4; ++j4) {
        const float4 p4 = *reinterpret_cast<const float4*>(&s_p[w][h][4 * j4]);
        const float pj[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < DV; ++e)
            acc[h][e] = fmaf(pj[q], Elem<T>::to_f32(vv[e][4 * j4 + q]), acc[h][e]);
      }
    }
  }

#pragma unroll
  for (int h = 0; h < G; ++h) {
    float l = l_run[h];
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) l += shfl_xor(l, off);
    if (lane == 0) {
      s_ml[w][h][0] = m_run[h];
      s_ml[w][h][1] = l;
    }
#pragma unroll
    for (int e = 0; e < DV; ++e) s_o[w][h][lane + kWave * e] = acc[h][e];
  }
  __syncthreads();
  finish_partition<T, D, G>(a, rg.mem, rg.np, G, kvh, rg.slot, rg.bad, s_ml, s_o);
  merge_if_last<T, D>(a, s, kvh, rg.np[0]);
}

template <typename T, int D, int B, int G, int LPT>
__global__ __launch_bounds__(kNW * kWave) void decode_valu_kernel(DecodeArgs a) {
  a.PT = a.queue[kPtSlot];      // the plan's choice
  a.Pmax = a.queue[kPmaxSlot];  // partial results packed for it
  constexpr int TPR = kWave / LPT;      // tokens per round
  __shared__ __attribute__((aligned(16))) int s_tbl[kMaxPT / B + 1];
  __shared__ int s_bad, s_next;
  __shared__ __attribute__((aligned(16))) float s_ml[kNW][G][2];
  __shared__ __attribute__((aligned(16))) float s_o[kNW][G][D];
  __shared__ __attribute__((aligned(16))) float s_p[kNW][G][TPR];  // weights of the round
  for_each_item(a, &s_next, [&](const int4 e0, const int4 e1, int kvh, auto&& claim) {
    claim();  // at the start: these items are short
    valu_item<T, D, B, G, LPT, TPR>(a, e0, e1, kvh, s_tbl, &s_bad, s_ml, s_o, s_p);
  });
}

// ---------------------------------------------------------------------------------------
// Planning: the work list, longest items first.  One workgroup reads every context length,
// places the full partitions first (positions by a prefix sum) and buckets the partial last
// partitions by their length in 32-token tiles, in decreasing order (an empty or invalid
// context gets one item, which writes NaN).  The list holds one (sequence, partition) entry
// per partition; item i is entry i / Hkv for kv-head i % Hkv, so the Hkv heads of a partition
// are consecutive items.  It also picks how the persistent kernel claims items (one global
// cursor, or one queue per XCD when sequences share prefix blocks) and sets the claim
// counters past the items the grid starts with (workgroup g starts with item g).  When
// partitions will be merged it zeroes the merge counters.  Positions inside a bucket are
// claimed with LDS atomics,
// so the order inside a bucket can change from call to call; results do not depend on it
// (each item's output has a fixed place).
// ---------------------------------------------------------------------------------------
// A range of R tokens in partitions: `full` of PT tokens, then a last one of `last` tokens (0:
// none).  A last partition of at most PT / 4 tokens joins the one before it (a partition of up
// to 1.25 PT tokens, within kMaxPT), so no item is a sliver that costs an item start-up, a
// partial result and a merge for a few tokens.
struct Split {
  int full, last;
};
__device__ __forceinline__ Split split_range(int R, int PT) {
  Split sp{R / PT, R % PT};
  if (sp.last > 0 && sp.full > 0 && 4 * sp.last <= PT && PT + sp.last <= kMaxPT) {
    sp.full -= 1;
    sp.last += PT;
  }
  return sp;
}
__device__ __forceinline__ int parts_of(int R, int PT) {
  const Split sp = split_range(R, PT);
  return sp.full + (sp.last > 0);
}

template <bool V> struct Flag { static constexpr bool value = V; };

__device__ __forceinline__ int wave_inclusive_sum(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int t = __shfl_up(v, off, kWave);
    if (lane >= off) v += t;
  }
  return v;
}

// lens_src: the lengths to plan with (system-scope loads when `sys`: page-locked host memory);
// lens_out: when not null, receives a copy of them for the decode kernel (a.ctx_lens).
//
// Share groups (a.gmem > 0, a.ngroups > 0, S <= kPlanKeep): group g names up to kGroupMembers
// sequences that hold the same K/V at positions [0, L).  The plan accepts a member only if its
// index is in range, its length is valid and no earlier group took it (first come, by an LDS
// claim); a group keeps L' = min(L, its members' lengths) rounded down to a multiple of 32, and
// is dropped (its members then plan alone) with fewer than two members or L' < 32.  Each
// accepted group's range is split into partitions of PT tokens, and each partition into items
// of a.gmem members; a member's own items cover [L', n) in partitions of PT from L', unless
// 0 < n - L' <= kFuseTail: then the group's item that ends at L' also reads those tokens of the
// member (its "fused tail": the member's slot in the entry carries the tail length in its upper
// 16 bits).  A member's partial results are the group's partitions first, then its own.
__device__ void plan_body(const DecodeArgs& a, int grid, const int32_t* lens_src,
                          int32_t* lens_out, bool sys) {
  constexpr int kPlanWaves = kPlanThreads / kWave;
  __shared__ int s_cnt[kMaxBuckets];   // partial partitions per bucket
  __shared__ int s_base[kMaxBuckets];  // first entry of each bucket (then a cursor)
  __shared__ int s_wave[kPlanWaves];
  __shared__ int s_full;               // full partitions (pass 1's count)
  __shared__ int s_fcur;               // next list position of a full partition (pass 2)
  __shared__ int s_len[kPlanKeep];     // pass 0's lengths of the first kPlanKeep sequences
  __shared__ int s_grp[kPlanKeep];     // group that took the sequence (claims), then its L'
  __shared__ int s_first[kShareSlots];  // open-addressing set of first blocks seen
  __shared__ int s_dups;                // sequences whose first block another one also has
  __shared__ unsigned long long s_total;  // tokens the items will read
  const bool groups_on = a.gmem > 0 && a.ngroups > 0 && a.S <= kPlanKeep;
  const int ngroups = groups_on ? a.ngroups : 0;
  // The first round's table entries and lengths are requested before the LDS set-up, so their
  // latency (device memory; the bus for page-locked lengths) overlaps it.  The table entry goes
  // first: it then travels with the length.
  int pre_blk = -1, pre_raw = 0;
  if (threadIdx.x < a.S) {
    pre_blk = a.tables[static_cast<size_t>(threadIdx.x) * a.max_blocks];
    pre_raw = ld_step(lens_src + threadIdx.x, sys);
  }
  for (int i = threadIdx.x; i < kShareSlots; i += kPlanThreads) s_first[i] = -1;
  if (groups_on)
    for (int i = threadIdx.x; i < kPlanKeep; i += kPlanThreads) s_grp[i] = -1;
  for (int b = threadIdx.x; b < kMaxBuckets; b += kPlanThreads) s_cnt[b] = 0;
  if (threadIdx.x == 0) {
    s_full = 0;
    s_fcur = 0;  // set by the scan (PT is a multiple of 32 in [32, kMaxPT]: bucket PT / 32 exists)
    s_dups = 0;
    s_total = 0;
  }
  const int w = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
  lds_barrier();
  // Pass 0, one sequence per thread per round: lengths (kept in LDS, copied to lens_out), the
  // sharing test, and without share groups the total of tokens the items read.
  unsigned long long my_total = 0;
  for (int s = threadIdx.x; s < a.S; s += kPlanThreads) {
    const bool first = s < kPlanThreads;
    const int blk = first ? pre_blk : a.tables[static_cast<size_t>(s) * a.max_blocks];
    const int raw = first ? pre_raw : ld_step(lens_src + s, sys);
    if (lens_out) lens_out[s] = raw;
    if (s < kPlanKeep) s_len[s] = raw;
    if (!groups_on) {
      bool bad;
      const int n = eff_len(raw, a.len_cap, bad);
      my_total += static_cast<unsigned long long>(bad ? 0 : n);
    }
    // Prefix sharing shows as one physical first block in several tables.  A set in LDS
    // (bounded probing, so a full set only undercounts) counts the repeats.
    if (blk >= 0) {
      int h = static_cast<int>((static_cast<uint32_t>(blk) * 2654435761u) >> (32 - kShareBits));
      for (int k = 0; k < kShareProbes; ++k) {
        const int old = atomicCAS(&s_first[h], -1, blk);
        if (old == -1) break;
        if (old == blk) {
          atomicAdd(&s_dups, 1);
          break;
        }
        h = (h + 1) & (kShareSlots - 1);
      }
    }
  }
  if (groups_on) {
  lds_barrier();
  // Share groups: claim members, then record each group as accepted (L' = 0: dropped).
  for (int g = threadIdx.x; g < ngroups; g += kPlanThreads) {
    const int32_t* rec = a.groups + static_cast<size_t>(g) * kGroupRec;
    const int L = rec[0];
    // accepted members, compacted (scalars: a runtime index into a local array would put it
    // in scratch memory)
    int m0 = -1, m1 = -1, m2 = -1, m3 = -1, nm = 0, nmin = INT_MAX;
#pragma unroll
    for (int k = 0; k < kGroupMembers; ++k) {
      const int m = rec[1 + k];
      if (m < 0 || m >= a.S) continue;
      bool bad;
      const int n = eff_len(s_len[m], a.len_cap, bad);
      if (bad || atomicCAS(&s_grp[m], -1, g) != -1) continue;
      if (nm == 0) m0 = m;
      else if (nm == 1) m1 = m;
      else if (nm == 2) m2 = m;
      else m3 = m;
      ++nm;
      nmin = min(nmin, n);
    }
    int Lg = nm >= 2 && L > 0 ? (min(L, nmin) & ~31) : 0;
    int* v = a.vgroups + static_cast<size_t>(g) * kVGroupRec;
    v[0] = Lg;
    v[1] = m0;
    v[2] = m1;
    v[3] = m2;
    v[4] = m3;
    v[1 + kGroupMembers] = nm;
  }
  __syncthreads();  // vgroups: global memory read by other threads
  // Each claimed sequence's range base: its group's L' (0 for a dropped group); the total of
  // tokens the items read (a group's range once per item of gmem members).
  for (int s = threadIdx.x; s < a.S; s += kPlanThreads) {
    bool bad;
    const int raw = s < kPlanKeep ? s_len[s] : lens_out ? lens_out[s] : ld_step(lens_src + s, sys);
    const int n = eff_len(raw, a.len_cap, bad);
    int base = 0;
    if (groups_on) {
      const int g = s_grp[s];
      base = g >= 0 ? a.vgroups[static_cast<size_t>(g) * kVGroupRec] : 0;
      s_grp[s] = base;
    }
    my_total += static_cast<unsigned long long>(bad ? 0 : n - base);
  }
  for (int g = threadIdx.x; g < ngroups; g += kPlanThreads) {
    const int* v = a.vgroups + static_cast<size_t>(g) * kVGroupRec;
    const int chunks = (v[1 + kGroupMembers] + a.gmem - 1) / a.gmem;
    my_total += static_cast<unsigned long long>(v[0]) * static_cast<unsigned long long>(chunks);
  }
  }
  // one LDS atomic per wave: 256 64-bit atomics on one word serialised (~2.5 us of the plan)
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) my_total += __shfl_xor(my_total, off, kWave);
  if (lane == 0 && my_total) atomicAdd(&s_total, my_total);
  lds_barrier();
  // Partition length: the caller's, or the longest multiple of kAutoPTStep in [kMinAutoPT,
  // kMaxAutoPT] that is at most 3/4 of one workgroup's share of the work (token-heads / grid).
  // Longer partitions mean fewer partial results and item start-ups; the bound keeps the
  // longest items short enough for the tail to even out.  (Powers of two only gave the
  // Mistral-7B-shaped batch 1,024 where 1,280-1,536 measured 1.4% faster.)  Every thread
  // derives it from the total itself (no barrier to publish it).
  int PT = a.PT;
  if (PT == 0) {
    const unsigned long long share = s_total * static_cast<unsigned long long>(a.Hkv) /
                                     static_cast<unsigned long long>(grid > 0 ? grid : 1);
    const unsigned long long lim = 3ull * share / 4ull / kAutoPTStep * kAutoPTStep;
    PT = static_cast<int>(lim < kMinAutoPT ? kMinAutoPT : lim > kMaxAutoPT ? kMaxAutoPT : lim);
  }
  // a member's group partitions and own partitions together are at most one more than an
  // unsplit range's
  const int pmax = (a.len_cap + PT - 1) / PT + (groups_on ? 1 : 0);
  // a last partition has 0 .. 1.25 PT tokens (see split_range): buckets 0 .. nbk
  const int nbk = (min(kMaxPT, PT + PT / 4) + 31) / 32;  // s_cnt was zeroed at the start
  // A group member's slot in the entry of the group's last item: its index, and in the upper 16
  // bits the number of its own tokens that item reads after the range (0 when it has none, or
  // more than kFuseTail, which get items of their own).
  auto fused_member = [&](int m, int Lg) {
    bool bad;
    const int tail = eff_len(s_len[m], a.len_cap, bad) - Lg;
    return m | ((tail > 0 && tail <= kFuseTail ? tail : 0) << 16);
  };
  // A sequence's length in passes 1 and 2: from LDS when pass 0 kept them all.  The loops then
  // hold no global load, so the wave never waits on the stores it issued before (on this ISA
  // the counter a load is waited on with also counts stores, and stores take ~1 us to retire).
  auto seq_len = [&](int s, auto all_kept) {
    if constexpr (decltype(all_kept)::value) return s_len[s];
    else return s < kPlanKeep ? s_len[s] : lens_out ? lens_out[s] : ld_step(lens_src + s, sys);
  };
  // The list, longest first: partial partitions longer than PT (a last partition that took in
  // a sliver), the full partitions (PT tokens each, in any order), then the shorter partial
  // ones, each group of partials by 32-token buckets in decreasing order.  Pass 1 counts, the
  // scan turns the counts into list positions, pass 2 writes the entries.
  // Pass 1: partial partitions per bucket, full partitions in total.
  int my_full = 0;
  auto pass1 = [&](auto all_kept) {
    for (int s = threadIdx.x; s < a.S; s += kPlanThreads) {
      bool bad;
      const int n = eff_len(seq_len(s, all_kept), a.len_cap, bad);
      const int base = groups_on ? s_grp[s] : 0;
      const bool fused = base > 0 && n - base <= kFuseTail;
      const Split sp = bad || fused ? Split{0, 0} : split_range(n - base, PT);
      a.nparts[s] = bad ? 1 : parts_of(base, PT) + sp.full + (sp.last > 0);  // fused: the group's alone
      if (bad || sp.last > 0) atomicAdd(&s_cnt[(sp.last + 31) / 32], 1);
      my_full += sp.full;
    }
  };
  if (a.S <= kPlanKeep) pass1(Flag<true>{});
  else pass1(Flag<false>{});
  for (int g = threadIdx.x; g < ngroups; g += kPlanThreads) {
    const int* v = a.vgroups + static_cast<size_t>(g) * kVGroupRec;
    const int Lg = v[0], nm = v[1 + kGroupMembers];
    if (Lg <= 0) continue;
    const int chunks = (nm + a.gmem - 1) / a.gmem;
    const Split sp = split_range(Lg, PT);
    if (sp.last > 0) atomicAdd(&s_cnt[(sp.last + 31) / 32], chunks);
    my_full += chunks * sp.full;
  }
  // one LDS atomic per wave (per-lane atomics of differing amounts are serialised over the lanes)
  {
    const int wsum = __shfl(wave_inclusive_sum(my_full), kWave - 1, kWave);
    if (lane == 0 && wsum > 0) atomicAdd(&s_full, wsum);
  }
  lds_barrier();
  // List positions by a block-wide scan over the buckets in decreasing order, thread t on bucket
  // nbk - t (a serial sum per thread took ~6 us at 160 buckets): base[b] = sum_{b' > b} cnt[b'],
  // plus the full partitions' count for buckets of at most PT tokens (b <= PT / 32); the full
  // partitions start after the longer buckets.  nbk <= kPlanThreads: only bucket 0 can be left
  // over, when nbk == kPlanThreads.
  {
    const int bb = PT / 32;
    const int b = nbk - static_cast<int>(threadIdx.x);
    const int c = b >= 0 ? s_cnt[b] : 0;
    const int incl = wave_inclusive_sum(c);  // sum of cnt over buckets b .. b + lane
    if (lane == kWave - 1) s_wave[w] = incl;
    lds_barrier();
    int above = 0;  // buckets above this wave's
    for (int u = 0; u < w; ++u) above += s_wave[u];
    const int excl = above + incl - c;
    if (b >= 0) s_base[b] = excl + (b <= bb ? s_full : 0);
    if (b == bb) s_fcur = excl;
    if (threadIdx.x == 0) {
      int all = 0;
      for (int u = 0; u < kPlanWaves; ++u) all += s_wave[u];
      if (nbk >= kPlanThreads) {  // bucket 0 had no thread
        s_base[0] = s_full + all;
        if (bb == 0) s_fcur = all;
        all += s_cnt[0];
      }
      a.queue[0] = (s_full + all) * a.Hkv;
      // per-XCD queues (kv-head affinity) when at least 1/8 of the sequences share their
      // first block and the kv-heads split evenly over the XCDs; else one global cursor
      a.queue[1] = (a.Hkv % kXcd == 0 && 8 * s_dups >= a.S) ? 1 : 0;
      for (int x = 0; x < kXcd; ++x) a.queue[2 + x] = (grid - x + kXcd - 1) / kXcd;
      a.queue[2 + kXcd] = grid;
      a.queue[kPtSlot] = PT;
      a.queue[kPmaxSlot] = pmax;
    }
  }
  lds_barrier();
  // Pass 2: the entries (each thread revisits the sequences and groups of pass 1).  A wave's
  // full partitions take one claim on the full cursor, placed by a wave prefix sum.
  auto pass2 = [&](auto all_kept) {
    for (int s0 = threadIdx.x - lane; s0 < a.S; s0 += kPlanThreads) {  // wave-uniform rounds
      const int s = s0 + lane;
      int full = 0, npre = 0, base = 0;
      if (s < a.S) {
        bool bad;
        const int n = eff_len(seq_len(s, all_kept), a.len_cap, bad);
        base = groups_on ? s_grp[s] : 0;
        npre = parts_of(base, PT);
        const bool fused = base > 0 && n - base <= kFuseTail;
        const Split sp = bad || fused ? Split{0, 0} : split_range(n - base, PT);
        if (bad || sp.last > 0) {
          const int e = atomicAdd(&s_base[(sp.last + 31) / 32], 1);
          const int t0 = bad ? 0 : base + sp.full * PT;
          a.items[2 * e] = make_int4(s, bad ? 0 : npre + sp.full, t0, bad ? 0 : n);
          a.items[2 * e + 1] = make_int4(s, -1, -1, -1);
        }
        full = sp.full;
      }
      const int incl = wave_inclusive_sum(full);
      const int wsum = __shfl(incl, kWave - 1, kWave);
      int wbase = 0;
      if (lane == kWave - 1 && wsum > 0) wbase = atomicAdd(&s_fcur, wsum);
      int e = __shfl(wbase, kWave - 1, kWave) + incl - full;
      for (int q = 0; q < full; ++q, ++e) {
        a.items[2 * e] = make_int4(s, npre + q, base + q * PT, base + (q + 1) * PT);
        a.items[2 * e + 1] = make_int4(s, -1, -1, -1);
      }
    }
  };
  if (a.S <= kPlanKeep) pass2(Flag<true>{});
  else pass2(Flag<false>{});
  for (int g = threadIdx.x; g < ngroups; g += kPlanThreads) {
    const int* v = a.vgroups + static_cast<size_t>(g) * kVGroupRec;
    const int Lg = v[0], nm = v[1 + kGroupMembers];
    if (Lg <= 0) continue;
    const Split sp = split_range(Lg, PT);
    const int full = sp.full;
    const int chunks = (nm + a.gmem - 1) / a.gmem;
    const bool ends_full = sp.last == 0;  // the last full entry ends at Lg
    int e = full > 0 ? atomicAdd(&s_fcur, chunks * full) : 0;
    for (int c = 0; c < chunks; ++c) {
      int mm[kGroupMembers], mt[kGroupMembers];
#pragma unroll
      for (int k = 0; k < kGroupMembers; ++k) {
        const int j = c * a.gmem + k;
        mm[k] = k < a.gmem && j < nm ? v[1 + j] : -1;
        mt[k] = mm[k] >= 0 ? fused_member(mm[k], Lg) : mm[k];
      }
      // a member's slot in the group's last item carries its fused tail (see fused_member)
      for (int p = 0; p < full; ++p, ++e) {
        a.items[2 * e] = make_int4(-1 - g, p, p * PT, (p + 1) * PT);
        if (ends_full && p == full - 1)
          a.items[2 * e + 1] = make_int4(mt[0], mt[1], mt[2], mt[3]);
        else
          a.items[2 * e + 1] = make_int4(mm[0], mm[1], mm[2], mm[3]);
      }
      if (sp.last > 0) {
        const int el = atomicAdd(&s_base[(sp.last + 31) / 32], 1);
        a.items[2 * el] = make_int4(-1 - g, full, full * PT, Lg);
        a.items[2 * el + 1] = make_int4(mt[0], mt[1], mt[2], mt[3]);
      }
    }
  }
  // The decode kernel's per-(sequence, kv-head) done counters, zeroed last: nothing here waits
  // for these stores.
  for (int i = threadIdx.x; i < a.S * a.Hkv; i += kPlanThreads) a.done[i] = 0;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(DecodeArgs a, int grid) {
  plan_body(a, grid, a.ctx_lens, nullptr, false);
}

// The prologue of a fused serving step: the step's cache write (and table patch) and the
// decode planning are independent, so one launch does both -- the first workgroup plans, the
// others scatter the new tokens.
static_assert(kPlanThreads == kWriteThreads, "one block size for both halves of the prologue");

// A step's slots and lengths carried in the prologue's kernel arguments: when the caller keeps
// them in page-locked host memory and the batch is small enough, the host copies them at the
// call, so the kernel reads them from device memory instead of across the bus (a bus round
// trip is ~1.4 us of the step's first kernel).
constexpr int kMetaMax = 384;  // entries of each array (3 KiB; kernel arguments stay < 4 KiB)
struct StepMeta {
  int32_t has_slots, has_lens;  // 0: read through the pointers in the write's arguments
  int32_t slots[kMetaMax];
  int32_t lens[kMetaMax];
};
static_assert(sizeof(CacheWriteArgs) + sizeof(DecodeArgs) + sizeof(StepMeta) + 16 <= 3584,
              "the prologue's kernel arguments (with the runtime's hidden ones) fit in 4 KiB");
static_assert(offsetof(StepMeta, has_slots) == 0 && offsetof(StepMeta, has_lens) == 4,
              "the kernel reads the flags as the segment's first two words");

// The plan reads the step's lengths from w.tp.ctx_lens (where the write's table patch reads
// them too) and, when lens_out is set, stores them for the decode kernel.
// m is the first argument, so it starts the kernel-argument segment; the kernel reads it there
// through the segment pointer (taking its address would copy 3 KiB into scratch memory).
template <typename T>
__global__ __launch_bounds__(kPlanThreads) void step_prologue_kernel(StepMeta m, CacheWriteArgs w,
                                                                     DecodeArgs a, int grid,
                                                                     int32_t* lens_out) {
  const int32_t* km = (const int32_t*)__builtin_amdgcn_kernarg_segment_ptr();
  // w.sys covers what is still read through host pointers
  CacheWriteArgs wl = w;
  if (km[0]) wl.slots = km + offsetof(StepMeta, slots) / 4;
  if (km[1]) wl.tp.ctx_lens = km + offsetof(StepMeta, lens) / 4;
  if (blockIdx.x == 0) {  // dispatched first: the plan is the longer chain
    plan_body(a, grid, wl.tp.ctx_lens, lens_out, wl.sys);
    return;
  }
  cache_write_wg<T>(wl, blockIdx.x - 1);
}

// ---------------------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------------------

// Workspace: [queue header | work list | merge counters | partial-result counts | accepted
// share groups | partition (m, l) | partition outputs].  Counters are sized for Hq heads (an
// upper bound of Hkv), so the size query needs no Hkv.  Pmax is the number of partial-result
// slots per (sequence, head): one more than an unsplit context needs, for the share groups.
struct WsLayout {
  size_t items, done, nparts, vgroups, ml, o, total;
};

static size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

static WsLayout ws_layout(int S, int Hq, int D, int Pmax) {
  WsLayout L{};
  size_t off = 256;
  L.items = off;  // at most S * Pmax entries of two int4
  off += round256(static_cast<size_t>(S) * Pmax * 2 * sizeof(int4));
  L.done = off;
  off += round256(static_cast<size_t>(S) * Hq * sizeof(int));
  L.nparts = off;
  off += round256(static_cast<size_t>(S) * sizeof(int));
  L.vgroups = off;
  off += round256(static_cast<size_t>(S) * kVGroupRec * sizeof(int));
  const size_t rows = static_cast<size_t>(S) * Hq * Pmax;
  L.ml = off;
  off += round256(rows * sizeof(float2));
  L.o = off;
  off += rows * D * sizeof(float);
  L.total = off;
  return L;
}

// Partial-result slots per (sequence, head) the workspace holds for contexts of at most
// max_ctx tokens in partitions of at least pt tokens (see WsLayout).
static int ws_pmax(int max_ctx, int pt) { return (max_ctx > 0 ? (max_ctx + pt - 1) / pt : 1) + 1; }

// Workgroups of kernel k that fit on the device at once (the persistent grid size).
static int resident_grid(const void* k, int threads, size_t lds_dynamic) {
  static std::mutex mu;
  static std::map<std::pair<const void*, int>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_pair(k, dev);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, threads, lds_dynamic) != hipSuccess)
    return 0;
  const int g = cus * (per_cu > 0 ? per_cu : 1);
  cache[key] = g;
  return g;
}

typedef void (*KernelFn)(DecodeArgs);

// Lanes per token: enough that the per-lane q slice stays small.
template <int D, int B>
static KernelFn pick_valu(int32_t dtype, int G) {
  if (dtype == PA_DTYPE_F32) {
    switch (G) {
      case 1: return decode_valu_kernel<float, D, B, 1, (D == 64 ? 4 : 8)>;
      case 2: return decode_valu_kernel<float, D, B, 2, (D == 64 ? 4 : 8)>;
      case 4: return decode_valu_kernel<float, D, B, 4, (D == 64 ? 8 : 16)>;
      case 8: return decode_valu_kernel<float, D, B, 8, 16>;
    }
  } else {
    switch (G) {
      case 1: return decode_valu_kernel<uint16_t, D, B, 1, (D == 64 ? 4 : 8)>;
      case 2: return decode_valu_kernel<uint16_t, D, B, 2, (D == 64 ? 4 : 8)>;
    }
  }
  return nullptr;
}

// Picks the kernel, the partition length and the grid, lays out the workspace and launches
// plan -> decode (which merges split partitions itself) on `stream`.  With a cache write (`wr`,
// pa_decode_step) the plan shares its launch with the write.
template <int D, int B>
static pa_status launch(DecodeArgs a, int32_t dtype, int partition_tokens, void* workspace,
                        size_t workspace_bytes_in, hipStream_t stream,
                        const CacheWriteArgs* wr = nullptr, int32_t* lens_out = nullptr,
                        const StepMeta* meta = nullptr) {
  KernelFn k = nullptr;
  if (dtype == PA_DTYPE_BF16 && a.G >= 3 && a.G <= 16)
    k = decode_mfma_kernel<D, B>;
  else
    k = pick_valu<D, B>(dtype, a.G);
  if (!k)
    return fail(PA_ERR_UNSUPPORTED,
                "pa_decode: %d query heads per kv-head not supported for dtype %d "
                "(bf16: 1..16, f32: 1, 2, 4, 8)", a.G, dtype);
  const int cap = resident_grid(reinterpret_cast<const void*>(k), kNW * kWave, 0);
  if (cap <= 0) return fail(PA_ERR_HIP, "pa_decode: cannot query the device's compute units");
  // Share groups run on the matrix-core kernel only: a group item puts 16 / G sequences' heads
  // in the 16 columns of the Q^T operand (at most kGroupMembers).
  a.gmem = (k == decode_mfma_kernel<D, B>) ? min(kGroupMembers, 16 / a.G) : 0;
  if (a.gmem <= 1) a.gmem = 0;
  // partition_tokens = 0: the plan picks the length from the batch (at least kMinAutoPT, which
  // bounds the partitions per sequence; the size query assumed the same).
  a.PT = partition_tokens;
  const int pt_min = partition_tokens ? partition_tokens : kMinAutoPT;
  a.Pmax = ws_pmax(a.len_cap, pt_min);
  if (static_cast<int64_t>(a.S) * a.Pmax * a.Hq >= (int64_t(1) << 31))
    return fail(PA_ERR_INVALID_ARG, "pa_decode: S * partitions * Hq too large");
  const WsLayout L = ws_layout(a.S, a.Hq, D, a.Pmax);  // fits: PT >= the size query's choice
  char* ws = static_cast<char*>(workspace);
  a.queue = reinterpret_cast<int*>(ws);
  a.items = reinterpret_cast<int4*>(ws + L.items);
  a.done = reinterpret_cast<int*>(ws + L.done);
  a.nparts = reinterpret_cast<int*>(ws + L.nparts);
  a.vgroups = reinterpret_cast<int*>(ws + L.vgroups);
  a.part_ml = reinterpret_cast<float2*>(ws + L.ml);
  a.part_o = reinterpret_cast<float*>(ws + L.o);

  const int64_t max_items = static_cast<int64_t>(a.S) * a.Pmax * a.Hkv;
  const int grid = static_cast<int>(max_items < cap ? max_items : cap);
  if (wr) {
    const unsigned nw = static_cast<unsigned>(cache_write_wgs(*wr));
    static const StepMeta none{};  // nothing carried: read through the pointers
    const StepMeta& m = meta ? *meta : none;
    if (dtype == PA_DTYPE_F32)
      hipLaunchKernelGGL(step_prologue_kernel<float>, dim3(nw + 1), dim3(kPlanThreads), 0, stream, m, *wr, a, grid, lens_out);
    else
      hipLaunchKernelGGL(step_prologue_kernel<uint16_t>, dim3(nw + 1), dim3(kPlanThreads), 0, stream, m, *wr, a, grid, lens_out);
    if (pa_status st = launch_status("pa_decode_step (cache write + plan)")) return st;
  } else {
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, a, grid);
    if (pa_status st = launch_status("pa_decode (plan)")) return st;
  }
  hipLaunchKernelGGL(k, dim3(grid), dim3(kNW * kWave), 0, stream, a);
  if (pa_status st = launch_status("pa_decode")) return st;
  return ok();
}

}  // namespace pa

using namespace pa;

extern "C" pa_status pa_decode_workspace_size(int32_t S, int32_t Hq, int32_t D, int32_t max_ctx_len,
                                              int32_t partition_tokens, size_t* bytes) {
  if (!bytes) return fail(PA_ERR_INVALID_ARG, "pa_decode_workspace_size: bytes is NULL");
  *bytes = 0;
  if (S < 0 || Hq <= 0 || D <= 0 || max_ctx_len < 0)
    return fail(PA_ERR_INVALID_ARG, "pa_decode_workspace_size: bad sizes");
  if (partition_tokens != 0 && (partition_tokens % 32 || partition_tokens < 32 || partition_tokens > kMaxPT))
    return fail(PA_ERR_INVALID_ARG, "pa_decode_workspace_size: partition_tokens %d", partition_tokens);
  const int pt = partition_tokens ? partition_tokens : kMinAutoPT;
  const int Pmax = ws_pmax(max_ctx_len, pt);
  if (static_cast<int64_t>(S) * Pmax * Hq >= (int64_t(1) << 31))
    return fail(PA_ERR_INVALID_ARG, "pa_decode_workspace_size: S * partitions * Hq too large");
  *bytes = ws_layout(S, Hq, D, Pmax).total;
  return ok();
}

// Argument checks and DecodeArgs of pa_decode / pa_decode_step (everything visible on the host
// is validated before any device work).
static pa_status decode_setup(const char* who, void* out, const void* q, const void* k_cache,
                              const void* v_cache, const int32_t* block_tables,
                              const int32_t* ctx_lens, int32_t S, int32_t Hq, int32_t Hkv,
                              int32_t D, int32_t B, int32_t num_blocks, int32_t max_blocks,
                              int32_t max_ctx_len, float scale, int32_t dtype,
                              int32_t partition_tokens, void* workspace, size_t workspace_bytes_in,
                              DecodeArgs* out_args) {
  if (elem_bytes(dtype) == 0) return fail(PA_ERR_UNSUPPORTED, "%s: dtype %d", who, dtype);
  if (D != 64 && D != 128) return fail(PA_ERR_UNSUPPORTED, "%s: head_dim %d not in {64, 128}", who, D);
  if (B != 16 && B != 32 && B != 64)
    return fail(PA_ERR_UNSUPPORTED, "%s: block size %d not in {16, 32, 64}", who, B);
  if (S < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv)
    return fail(PA_ERR_INVALID_ARG, "%s: S %d, Hq %d, Hkv %d (Hq must be a multiple of Hkv)", who, S, Hq, Hkv);
  if (S > 65535 || Hkv > 65535) return fail(PA_ERR_INVALID_ARG, "%s: S and Hkv must be <= 65535", who);
  if (num_blocks <= 0 || max_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "%s: num_blocks %d, max_blocks %d", who, num_blocks, max_blocks);
  if (max_ctx_len < 1 || static_cast<int64_t>(max_ctx_len) > static_cast<int64_t>(max_blocks) * B)
    return fail(PA_ERR_INVALID_ARG, "%s: max_ctx_len %d outside [1, max_blocks*B]", who, max_ctx_len);
  if (partition_tokens != 0 && (partition_tokens % 32 || partition_tokens < 32 || partition_tokens > kMaxPT))
    return fail(PA_ERR_INVALID_ARG, "%s: partition_tokens %d is not a multiple of 32 in [32, %d]",
                who, partition_tokens, kMaxPT);
  if (partition_tokens % B)  // a partition is made of whole blocks
    return fail(PA_ERR_INVALID_ARG, "%s: partition_tokens %d is not a multiple of the block size %d",
                who, partition_tokens, B);
  // the kernels take the row max of the raw scores and scale it afterwards
  if (!(scale > 0.f) || scale == INFINITY)
    return fail(PA_ERR_INVALID_ARG, "%s: scale must be positive and finite", who);
  if (S == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !ctx_lens)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARG, "%s: q, out and the pools must be 16-byte aligned", who);
  // The workspace must hold the layout for the shortest partition this call may pick (the
  // size pa_decode_workspace_size reports), checked before anything touches the device.
  const int pt_min = partition_tokens ? partition_tokens : kMinAutoPT;
  const int pmax_min = ws_pmax(max_ctx_len, pt_min);
  if (static_cast<int64_t>(S) * pmax_min * Hq >= (int64_t(1) << 31))
    return fail(PA_ERR_INVALID_ARG, "%s: S * partitions * Hq too large", who);
  const size_t need = ws_layout(S, Hq, D, pmax_min).total;
  if (!workspace || workspace_bytes_in < need)
    return fail(PA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", who, need,
                workspace ? workspace_bytes_in : size_t(0));
  if (!aligned16(workspace)) return fail(PA_ERR_INVALID_ARG, "%s: workspace must be 16-byte aligned", who);

  DecodeArgs& a = *out_args;
  a = DecodeArgs{};
  a.out = out;
  a.q = q;
  a.kc = k_cache;
  a.vc = v_cache;
  a.tables = block_tables;
  a.ctx_lens = ctx_lens;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.len_cap = max_ctx_len;  // validated above: max_ctx_len <= max_blocks * B
  a.scale_log2 = scale * kLog2e;
  return ok();
}

static pa_status dispatch(DecodeArgs a, int D, int B, int32_t dtype, int pt, void* w, size_t wb,
                          void* stream, const CacheWriteArgs* wr, int32_t* lens_out = nullptr,
                          const StepMeta* meta = nullptr) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (D == 64)
    return B == 16 ? launch<64, 16>(a, dtype, pt, w, wb, st, wr, lens_out, meta)
         : B == 32 ? launch<64, 32>(a, dtype, pt, w, wb, st, wr, lens_out, meta)
                   : launch<64, 64>(a, dtype, pt, w, wb, st, wr, lens_out, meta);
  return B == 16 ? launch<128, 16>(a, dtype, pt, w, wb, st, wr, lens_out, meta)
       : B == 32 ? launch<128, 32>(a, dtype, pt, w, wb, st, wr, lens_out, meta)
                 : launch<128, 64>(a, dtype, pt, w, wb, st, wr, lens_out, meta);
}

// Checks the share groups of pa_decode_shared / pa_decode_step_shared visible on the host and
// adds them to the arguments.
static pa_status set_groups(const char* who, DecodeArgs* a, const int32_t* groups,
                            int32_t n_groups) {
  if (n_groups < 0 || n_groups > a->S)
    return fail(PA_ERR_INVALID_ARG, "%s: n_groups %d outside [0, S = %d]", who, n_groups, a->S);
  if (n_groups == 0) return ok();
  if (!groups) return fail(PA_ERR_INVALID_ARG, "%s: groups is NULL", who);
  bool host = false;
  if (pa_status st = memory_kind(who, "groups", groups, &host)) return st;
  if (host) return fail(PA_ERR_INVALID_ARG, "%s: groups must be device memory", who);
  a->groups = groups;
  a->ngroups = n_groups;
  return ok();
}

static pa_status decode_call(const char* who, void* out, const void* q, const void* k_cache,
                             const void* v_cache, const int32_t* block_tables,
                             const int32_t* ctx_lens, int32_t S, int32_t Hq, int32_t Hkv,
                             int32_t D, int32_t B, int32_t num_blocks, int32_t max_blocks,
                             int32_t max_ctx_len, float scale, int32_t dtype,
                             int32_t partition_tokens, const int32_t* groups, int32_t n_groups,
                             void* workspace, size_t workspace_bytes_in, void* stream) {
  DecodeArgs a;
  if (pa_status st = decode_setup(who, out, q, k_cache, v_cache, block_tables, ctx_lens, S, Hq,
                                  Hkv, D, B, num_blocks, max_blocks, max_ctx_len, scale, dtype,
                                  partition_tokens, workspace, workspace_bytes_in, &a))
    return st;
  if (S == 0) return ok();
  if (pa_status st = set_groups(who, &a, groups, n_groups)) return st;
  return dispatch(a, D, B, dtype, partition_tokens, workspace, workspace_bytes_in, stream, nullptr);
}

static pa_status step_call(const char* who, void* out, const void* q, const void* key,
                           const void* value, void* k_cache, void* v_cache,
                           const int32_t* slot_mapping, int32_t* block_tables, int32_t* ctx_lens,
                           const int32_t* new_ctx_lens, int32_t S, int32_t Hq, int32_t Hkv,
                           int32_t D, int32_t B, int32_t num_blocks, int32_t max_blocks,
                           int32_t max_ctx_len, float scale, int32_t dtype,
                           int32_t partition_tokens, const int32_t* groups, int32_t n_groups,
                           void* workspace, size_t workspace_bytes_in, void* stream) {
  DecodeArgs a;
  if (pa_status st = decode_setup(who, out, q, k_cache, v_cache, block_tables, ctx_lens, S, Hq,
                                  Hkv, D, B, num_blocks, max_blocks, max_ctx_len, scale, dtype,
                                  partition_tokens, workspace, workspace_bytes_in, &a))
    return st;
  if (S == 0) return ok();
  if (!key || !value || !slot_mapping) return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (!aligned16(key) || !aligned16(value))
    return fail(PA_ERR_INVALID_ARG, "%s: key and value must be 16-byte aligned", who);
  if (pa_status st = set_groups(who, &a, groups, n_groups)) return st;
  if (new_ctx_lens == ctx_lens) new_ctx_lens = nullptr;
  bool host_slots = false, host_lens = false;
  if (pa_status st = memory_kind(who, "slot_mapping", slot_mapping, &host_slots)) return st;
  if (new_ctx_lens)
    if (pa_status st = memory_kind(who, "new_ctx_lens", new_ctx_lens, &host_lens)) return st;
  // The write's table patch and the plan read the step's lengths from their source; the decode
  // kernel reads the device copy the plan leaves in ctx_lens.
  CacheWriteArgs wr = make_cache_write_args(
      key, value, k_cache, v_cache, slot_mapping, S, Hkv, D, B, num_blocks, dtype,
      TablePatch{block_tables, new_ctx_lens ? new_ctx_lens : ctx_lens, 1, max_blocks});
  // Host-memory slots and lengths of a batch of at most kMetaMax sequences travel in the
  // first kernel's arguments (copied here, at the call); the rest is read across the bus.
  StepMeta meta;
  meta.has_slots = host_slots && S <= kMetaMax;
  meta.has_lens = host_lens && S <= kMetaMax;
  if (meta.has_slots) std::memcpy(meta.slots, slot_mapping, sizeof(int32_t) * S);
  if (meta.has_lens) std::memcpy(meta.lens, new_ctx_lens, sizeof(int32_t) * S);
  wr.sys = (host_slots && !meta.has_slots) || (host_lens && !meta.has_lens);
  return dispatch(a, D, B, dtype, partition_tokens, workspace, workspace_bytes_in, stream, &wr,
                  new_ctx_lens ? ctx_lens : nullptr, &meta);
}

extern "C" pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* ctx_lens, int32_t S,
                               int32_t Hq, int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks,
                               int32_t max_blocks, int32_t max_ctx_len, float scale, int32_t dtype,
                               int32_t partition_tokens, void* workspace, size_t workspace_bytes_in,
                               void* stream) {
  return decode_call("pa_decode", out, q, k_cache, v_cache, block_tables, ctx_lens, S, Hq, Hkv, D,
                     B, num_blocks, max_blocks, max_ctx_len, scale, dtype, partition_tokens,
                     nullptr, 0, workspace, workspace_bytes_in, stream);
}

extern "C" pa_status pa_decode_shared(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* ctx_lens, int32_t S, int32_t Hq, int32_t Hkv,
                                      int32_t D, int32_t B, int32_t num_blocks, int32_t max_blocks,
                                      int32_t max_ctx_len, float scale, int32_t dtype,
                                      int32_t partition_tokens, const int32_t* groups,
                                      int32_t n_groups, void* workspace,
                                      size_t workspace_bytes_in, void* stream) {
  return decode_call("pa_decode_shared", out, q, k_cache, v_cache, block_tables, ctx_lens, S, Hq,
                     Hkv, D, B, num_blocks, max_blocks, max_ctx_len, scale, dtype,
                     partition_tokens, groups, n_groups, workspace, workspace_bytes_in, stream);
}

extern "C" pa_status pa_decode_step(void* out, const void* q, const void* key, const void* value,
                                    void* k_cache, void* v_cache, const int32_t* slot_mapping,
                                    int32_t* block_tables, int32_t* ctx_lens,
                                    const int32_t* new_ctx_lens, int32_t S, int32_t Hq,
                                    int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks,
                                    int32_t max_blocks, int32_t max_ctx_len, float scale,
                                    int32_t dtype, int32_t partition_tokens, void* workspace,
                                    size_t workspace_bytes_in, void* stream) {
  return step_call("pa_decode_step", out, q, key, value, k_cache, v_cache, slot_mapping,
                   block_tables, ctx_lens, new_ctx_lens, S, Hq, Hkv, D, B, num_blocks, max_blocks,
                   max_ctx_len, scale, dtype, partition_tokens, nullptr, 0, workspace,
                   workspace_bytes_in, stream);
}

extern "C" pa_status pa_decode_step_shared(void* out, const void* q, const void* key,
                                           const void* value, void* k_cache, void* v_cache,
                                           const int32_t* slot_mapping, int32_t* block_tables,
                                           int32_t* ctx_lens, const int32_t* new_ctx_lens,
                                           int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                                           int32_t B, int32_t num_blocks, int32_t max_blocks,
                                           int32_t max_ctx_len, float scale, int32_t dtype,
                                           int32_t partition_tokens, const int32_t* groups,
                                           int32_t n_groups, void* workspace,
                                           size_t workspace_bytes_in, void* stream) {
  return step_call("pa_decode_step_shared", out, q, key, value, k_cache, v_cache, slot_mapping,
                   block_tables, ctx_lens, new_ctx_lens, S, Hq, Hkv, D, B, num_blocks, max_blocks,
                   max_ctx_len, scale, dtype, partition_tokens, groups, n_groups, workspace,
                   workspace_bytes_in, stream);
}

// ---------------------------------------------------------------------------------------
// pa_decode_step without a caller workspace, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
// The decode's scratch -- queue header, work list, merge counters, partial results -- lives
// in one file-scope device array of a fixed size; each GPU the library runs on holds its own
// copy until the process ends.  The plan kernel initialises everything the decode reads from
// it (the header, the list, and the merge counters when partitions are merged), so nothing
// has to be cleared between calls.  Every call on one GPU uses the same array: calls that
// overlap on one GPU (two streams, two threads) race on it.
// ---------------------------------------------------------------------------------------
namespace pa {
constexpr size_t kNoAllocScratchBytes = size_t(PA_NOALLOC_SCRATCH_MIB) << 20;
constexpr int kMaxDevices = 64;
}  // namespace pa

static __device__ __align__(256) unsigned char scratch[pa::kNoAllocScratchBytes];

namespace pa {

// Device address of `scratch` on the current device, taken once per device with
// hipGetSymbolAddress (in host code the array's name is only a host-side stand-in, never a
// device address).  No allocation: a fixed table indexed by device.
static pa_status noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return fail(PA_ERR_HIP, "pa_decode_step_noalloc: no current device below %d", kMaxDevices);
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(PA_ERR_HIP, "pa_decode_step_noalloc: hipGetSymbolAddress(scratch) failed: %s",
                  hipGetErrorString(e));
    }
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return ok();
}

}  // namespace pa

extern "C" pa_status pa_decode_step_noalloc(void* out, const void* q, const void* key,
                                            const void* value, void* k_cache, void* v_cache,
                                            const int32_t* slot_mapping, int32_t* block_tables,
                                            int32_t* ctx_lens, const int32_t* new_ctx_lens,
                                            int32_t S, int32_t Hq, int32_t Hkv, int32_t D,
                                            int32_t B, int32_t num_blocks, int32_t max_blocks,
                                            int32_t max_ctx_len, float scale, int32_t dtype,
                                            int32_t partition_tokens, void* stream) {
  // The scratch this call needs (the size pa_decode_workspace_size reports), checked against
  // the array before any HIP call.
  size_t need = 0;
  if (pa_status st = pa_decode_workspace_size(S, Hq, D, max_ctx_len, partition_tokens, &need))
    return st;
  if (need > kNoAllocScratchBytes)
    return fail(PA_ERR_WORKSPACE,
                "pa_decode_step_noalloc: this batch needs %zu bytes of scratch, the static scratch "
                "holds %zu (PA_NOALLOC_SCRATCH_MIB); use pa_decode_step with a workspace",
                need, kNoAllocScratchBytes);
  if (S == 0) return ok();
  void* ws = nullptr;
  if (pa_status st = noalloc_scratch(&ws)) return st;
  return pa_decode_step(out, q, key, value, k_cache, v_cache, slot_mapping, block_tables, ctx_lens,
                        new_ctx_lens, S, Hq, Hkv, D, B, num_blocks, max_blocks, max_ctx_len, scale,
                        dtype, partition_tokens, ws, kNoAllocScratchBytes, stream);
}
