// Chunked-query paged attention on the gfx950 matrix cores.
//
// What is computed: the prefill of the tokens past a cached prefix (KV-cache chapter,
// "RadixAttention": only the tokens after the point of divergence need a prefill pass, over
// the K/V blocks already in the pool).  Sequence s holds n = ctx_lens[s] tokens including its
// C new ones; query row i sits at position n - C + i and attends to positions 0 .. n - C + i
// (causal inside the chunk), with the same scores and softmax as dense attention (KV-cache
// chapter, "Common misconception").  The K/V of every position are reached through the block
// table ("Taming the Tail", "Under the Hood: The CUDA Kernel Engineering").
//
// Decomposition (CDNA4-specific):
//   * a unit of work = (sequence, kv-head, block of TQ chunk tokens); its rows are the
//     (token, query head) pairs of that kv-head's group, so every K/V tile loaded is used by
//     all g heads (GQA) -- 256 rows per unit, 32 per wave (8 waves): the accumulators of
//     32 rows fit in VGPRs (64 rows per wave spilled them to AGPRs and the loop moved them
//     back and forth).  A persistent grid of resident workgroups takes the units in rounds
//     (chunk_kernel);
//   * the query blocks of one (sequence, kv-head) run on one XCD, so they share its L2;
//   * K/V tiles of 64 keys go from HBM straight into LDS (global_load_lds_dwordx4, no
//     register staging), two stages: tile t+1 is requested before tile t is multiplied.  The
//     16-byte chunks of K rows and of V^T rows are XOR-swizzled by row (the lane-to-address
//     choice of the loads does it) so the 16-lane operand reads hit distinct banks;
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16_bf16 (32 keys x 32 rows per step):
//     keys on the MFMA rows put a query row's scores in one lane column, split over the two
//     lane halves, so the row max needs one cross-lane swap.  The K rows enter the QK^T
//     product in a permuted order that leaves the scores exactly where the PV product wants its
//     P^T operand, so the weights go from the score registers straight into the next product
//     (V is stored transposed per block in the pool);
//   * online softmax in the log2 domain, fp32 accumulation, P rounded to bf16 for the MFMA
//     and the row sum accumulated from the same rounded values (v_dot2c_f32_bf16 against
//     ones, each lane half summing its 16 keys; the halves are added once at the end).

#include <climits>
#include <cmath>
#include <map>
#include <mutex>

#include "device_common.h"

namespace pa {

namespace chunk {

constexpr int kWaves = 8;
constexpr int kRowsPerWave = 32;
constexpr int kRows = kWaves * kRowsPerWave;
constexpr int kKT = 64;                 // keys per LDS tile (one barrier per tile)
constexpr int kSub = 32;                // keys per compute step (two steps per tile)
constexpr int kTblWin = 512;            // block-table entries staged in LDS at a time
constexpr float kLazy = 8.f;            // lazy-rescale threshold (log2 units: weights < 256)
constexpr int kXcd = 8;                 // XCDs of an MI355X
constexpr float kLog2e = 1.4426950408889634f;

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Chunk permutation of the K tile in LDS: 16-byte chunk c of key row `key` sits at position
// c ^ kswz_chunk(key).  A matrix-core operand read has 16 lanes fetch the same chunk of 16
// consecutive keys (in kperm order); a K row of D = 128 fills the 64 banks once, one of
// D = 64 fills half of them, so the permutation takes key bits 0-3 (D = 128) or 1-3 (D = 64,
// where bit 0 already picks the bank half) and the 16 reads hit distinct banks.
template <int D>
__device__ __forceinline__ int kswz_chunk(int key) {
  return D == 128 ? (key & 15) : ((key >> 1) & 7);
}

// Sum over lane pairs (i, i ^ 32) with gfx950's 32-lane row swap.
__device__ __forceinline__ float add_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct Args {
  uint16_t* out;
  const uint16_t* q;
  const uint16_t* kc;
  const uint16_t* vc;
  const int32_t* tables;
  const int32_t* ctx_lens;
  int S, C, Hq, Hkv, G, TQ, NQB, max_blocks, num_blocks;
  int units;  // XCD-ordered query blocks: groups (padded to a multiple of kXcd) x NQB
  float scale_log2;
};

template <int D>
struct Smem {
  static constexpr int KROW = D * 2;           // bytes per key row of the K tile (swizzled)
  static constexpr int VROW = kKT * 2;         // bytes per dim row of the V^T tile (swizzled)
  static constexpr int KBYTES = kKT * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
};

// One unit of work: the query block `L` of the XCD-ordered list (see chunk_kernel), with the
// workgroup's two LDS stages and its table window.
template <int D, int B>
__device__ __forceinline__ void chunk_unit(const Args& a, int L, unsigned char* smem0,
                                           unsigned char* smem1, long long* s_tbl) {
  constexpr int NST = D / 16;  // QK contraction steps (16 dims each)
  constexpr int NDT = D / 32;  // PV tiles of 32 dims
  using SM = Smem<D>;

  // XCD-aware order: unit L runs on XCD L % kXcd (see chunk_kernel).  Every query block of one
  // (sequence, kv-head) group is placed on the same XCD, where they stream the same K/V
  // through one L2.
  const int xcd = L % kXcd, j = L / kXcd;
  const int grp = (j / a.NQB) * kXcd + xcd;
  if (grp >= a.S * a.Hkv) return;  // padding of the last round of groups
  const int qb = j % a.NQB, kvh = grp % a.Hkv, s = grp / a.Hkv;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), w = wave_id();
  const int G = a.G, C = a.C;

  const int n_raw = a.ctx_lens[s];
  const int cap = a.max_blocks * B;
  const bool bad = n_raw < C || n_raw > cap || C < 1;
  const int n = bad ? min(max(n_raw, 0), cap) : n_raw;
  const int base = n - C;               // position of chunk row 0 (may be < 0 if bad)
  const int i0 = qb * a.TQ;             // first chunk token of this workgroup
  const int i1 = min(C, i0 + a.TQ);
  // keys this workgroup needs: 0 .. base + i1 - 1
  const int kend = bad ? 0 : base + i1;
  const int ntiles = (kend + kKT - 1) / kKT;

  // ---- query operand: row rho = 32 w + lane % 32 -> (token i0 + rho / G, head rho % G).
  // The B operand of v_mfma_f32_32x32x16_bf16 has lane l hold B[8 (l / 32) + j][l % 32], so
  // lane half hf holds dims 16 st + 8 hf .. + 7 of the row for contraction step st.
  const int r32 = lane & 31, hf = lane >> 5;
  const int rho = kRowsPerWave * w + r32;
  const bool valid = rho < a.TQ * G && i0 + rho / G < i1;
  const int row_tok = valid ? i0 + rho / G : -1;  // chunk token of this lane's row (-1: padding)
  const int row_head = rho % G;
  bf16x8 qop[NST];
  {
    const uint16_t* qp = a.q + ((static_cast<size_t>(s) * C + (valid ? row_tok : 0)) * a.Hq +
                                kvh * G + (valid ? row_head : 0)) * D;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      uint4 u = *reinterpret_cast<const uint4*>(qp + 16 * st + 8 * hf);
      if (!valid) u = make_uint4(0, 0, 0, 0);
      qop[st] = __builtin_bit_cast(bf16x8, u);
    }
  }

  // ---- cooperative tile loads: the workgroup's 512 threads x 16 B per pass
  // K tile: kKT keys x D dims (row-major)  -> KTILE_VECS 16-byte pieces
  // V tile: D dims x kKT keys (transposed) -> VTILE_VECS 16-byte pieces
  constexpr int KV_PER_ROW = D * 2 / 16;           // 16-byte pieces per key row
  constexpr int KTILE_VECS = kKT * KV_PER_ROW;
  constexpr int VP_PER_ROW = kKT * 2 / 16;         // 16-byte pieces per dim row (8)
  constexpr int VTILE_VECS = D * VP_PER_ROW;
  constexpr int PASSES_K = KTILE_VECS / (kWaves * kWave);
  constexpr int PASSES_V = VTILE_VECS / (kWaves * kWave);
  static_assert(KTILE_VECS % (kWaves * kWave) == 0 && VTILE_VECS % (kWaves * kWave) == 0, "");
  const size_t head_stride = static_cast<size_t>(B) * D;
  const int32_t* trow = a.tables + static_cast<size_t>(s) * a.max_blocks;
  const int nblk_total = (kend + B - 1) / B;  // logical blocks this workgroup reads

  // The table slice is staged in LDS (a window of kTblWin entries, moved forward when the
  // tiles pass its end), so a tile's K/V loads never wait on a dependent table load.  Entries
  // outside the pool are replaced by block 0 and poison the workgroup's outputs.
  int bad_entry = 0;
  int win0 = 0;
  auto load_window = [&](int first) {
    const int cnt = min(kTblWin, nblk_total - first);
    for (int i = tid; i < cnt; i += kWaves * kWave) {
      int blk = trow[first + i];
      if (blk < 0 || blk >= a.num_blocks) {
        bad_entry = 1;
        blk = 0;
      }
      s_tbl[i] = (static_cast<long long>(blk) * a.Hkv + kvh) * static_cast<long long>(head_stride);
    }
  };
  load_window(0);
  __syncthreads();

  // Tiles go from HBM straight into LDS (global_load_lds_dwordx4: lane i of a wave's load
  // writes 16 bytes at the load's LDS base + 16 i), one stage ahead: tile t+1 is requested
  // before tile t is multiplied.  Which global 16 bytes a lane fetches implements the LDS
  // layout: K chunk c of key row k sits at position c ^ kswz(k); V^T chunk g (keys 8g..8g+7)
  // of dim row d sits at position g ^ vswz(d).
  auto vswz = [](int row) { return (row >> 1) & (VP_PER_ROW - 1); };

  auto dma = [&](unsigned char* kb, int t) {
    unsigned char* vb = kb + SM::KBYTES;
    const int k0 = t * kKT;
#pragma unroll
    for (int p = 0; p < PASSES_K; ++p) {
      const int u = w + kWaves * p;                    // this wave's 1 KiB piece of the tile
      const int e = u * kWave + lane;
      const int key = e / KV_PER_ROW, pos = e % KV_PER_ROW;
      const int piece = pos ^ kswz_chunk<D>(key);
      // clamp: never past the last needed key (kend >= 1 here, so j >= 0)
      const unsigned j = static_cast<unsigned>(min(k0 + key, kend - 1));
      const uint16_t* src = a.kc + s_tbl[static_cast<int>(j / B) - win0] + ((j % B) * D + piece * 8);
      pa::load16_to_lds(src, kb + u * (kWave * 16));
    }
#pragma unroll
    for (int p = 0; p < PASSES_V; ++p) {
      const int u = w + kWaves * p;
      const int e = u * kWave + lane;
      const int dim = e / VP_PER_ROW, pos = e % VP_PER_ROW;
      const int piece = pos ^ vswz(dim);               // 8 keys
      const unsigned j = static_cast<unsigned>(min(k0 + 8 * piece, (kend - 1) & ~7));
      const uint16_t* src = a.vc + s_tbl[static_cast<int>(j / B) - win0] + (dim * B + (j % B));
      pa::load16_to_lds(src, vb + u * (kWave * 16));
    }
  };
  // Keys at or past kend carry weight 0, but their slots may hold anything (even NaN, and
  // 0 * NaN = NaN inside the MFMA): once the last tile is in LDS, zero its V elements there.
  auto vfix = [&](unsigned char* base, int t) {
    unsigned char* vb = base + SM::KBYTES;
    const int k0 = t * kKT;
    for (int e = tid; e < VTILE_VECS; e += kWaves * kWave) {
      const int dim = e / VP_PER_ROW, pos = e % VP_PER_ROW;
      const int nvalid = kend - (k0 + 8 * (pos ^ vswz(dim)));
      if (nvalid >= 8) continue;
      u32x4* pv = reinterpret_cast<u32x4*>(vb + dim * SM::VROW + pos * 16);
      u32x4 vv = *pv;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd)
        vv[wd] &= (2 * wd < nvalid ? 0x0000FFFFu : 0u) | (2 * wd + 1 < nvalid ? 0xFFFF0000u : 0u);
      *pv = vv;
    }
  };

  float m_run = -INFINITY;  // the row's reference max (log2 units)
  float lpart = 0.f;        // this lane's half of the row sum (its 16 keys of every step)
  f32x16 o[NDT];            // O^T tiles: 32 dims x 32 rows
#pragma unroll
  for (int i = 0; i < NDT; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[i][e] = 0.f;

  // A tile is two 32-key steps (keys kSub*hs .. kSub*hs + 31 of the tile).  Per step: qk
  // issues S^T = K Q^T on the matrix cores; softmax turns the scores into bf16 weights; pv
  // accumulates O^T += V^T P^T.  A tile is issued as qk, qk, softmax, pv, softmax, pv, so the
  // second step's QK^T runs on the matrix cores while the first step's softmax runs on the VALU.
  //
  // The K rows are fed to the A operand in the order kperm, chosen so that the S^T result
  // lands where the P^T operand of the PV product needs it: the 32x32 result gives lane l
  // element e at row 8 (e / 4) + 4 (l / 32) + e % 4, and kperm of that row is key
  // 16 (e / 8) + 8 (l / 32) + e % 8, i.e. lane half hf holds keys 8 hf .. 8 hf + 7 of each
  // 16-key slice -- the B-operand layout of the product over that slice.
  auto kperm = [](int r) { return 16 * (r >> 4) + 8 * ((r >> 2) & 1) + 4 * ((r >> 3) & 1) + (r & 3); };
  using KOps = bf16x8[NST];
  using VOps = bf16x8[2 * NDT];
  auto read_k = [&](const unsigned char* kb, int hs, KOps& kop) {
    const int key = kSub * hs + kperm(r32);
#pragma unroll
    for (int st = 0; st < NST; ++st)
      kop[st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
          kb + key * SM::KROW + (((2 * st + hf) ^ kswz_chunk<D>(key)) << 4)));
  };
  auto read_v = [&](const unsigned char* vb, int hs, VOps& vop) {
#pragma unroll
    for (int i = 0; i < NDT; ++i) {
      const int dim = 32 * i + r32;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        vop[2 * i + ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(
            vb + dim * SM::VROW + (((4 * hs + 2 * ks + hf) ^ vswz(dim)) * 16)));
    }
  };
  auto qk = [&](const KOps& kop, f32x16& sacc) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sacc[e] = 0.f;
#pragma unroll
    for (int st = 0; st < NST; ++st)
      sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[st], qop[st], sacc, 0, 0, 0);
  };

  auto softmax = [&](int k0, const f32x16& sacc, bf16x8 (&pop)[2]) {
    // Online softmax; lane (hf, r32) owns keys k0 + 16 (e / 8) + 8 hf + e % 8 of row r32.
    // Masking is needed only on steps that reach past the causal limit of the workgroup's first
    // row (which also covers every key at or past kend); padding rows are never masked, their
    // outputs are dropped.
    const bool need_mask = k0 + kSub - 1 > base + i0;  // uniform
    // raw scores; the scale (> 0, checked on the host) is applied inside the exponent
    float x[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) x[e] = sacc[e];
    if (need_mask) {
      const int limit = row_tok < 0 ? INT32_MAX : base + row_tok;  // last visible key
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (k0 + 16 * (e >> 3) + 8 * hf + (e & 7) > limit) x[e] = -INFINITY;
    }
    float mx = vmax(vmax3(vmax3(x[0], x[1], x[2]), vmax3(x[3], x[4], x[5]), vmax3(x[6], x[7], x[8])),
                    vmax3(vmax3(x[9], x[10], x[11]), vmax3(x[12], x[13], x[14]), x[15]));
    mx = max_xor32(mx);
    mx *= a.scale_log2;  // row max in log2 units (the scale is positive)
    // Lazy rescaling: the row's reference max m_run moves only when a score exceeds it by
    // more than kLazy (log2 units).  Weights exp2(x - m_run) then stay below 2^kLazy, and
    // the rescale of the row's accumulators is rare.  After the final division by the
    // row sum the result is the same softmax.
    float alpha = 1.f;
    bool rescale = false;
    if (mx > m_run + kLazy) {
      alpha = fast_exp2(m_run - mx);  // 0 on the first visible key (m_run = -inf)
      m_run = mx;
      rescale = true;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      pop[e >> 3][e & 7] = static_cast<__bf16>(fast_exp2(fmaf(x[e], a.scale_log2, -m_use)));

    // O^T += V^T P^T over the 32 keys (V of keys past kend was zeroed when staged); the row
    // sum is taken from the same bf16 weights the numerator uses.
    if (__builtin_amdgcn_ballot_w64(rescale)) {  // uniform: some row of the wave rescales
      lpart *= alpha;
#pragma unroll
      for (int i = 0; i < NDT; ++i) o[i] *= alpha;
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bf16x2 pr = {pop[ks][2 * i], pop[ks][2 * i + 1]};
        lpart = __builtin_amdgcn_fdot2_f32_bf16(pr, kOnes2, lpart, false);
      }
  };
  auto pv = [&](const VOps& vop, const bf16x8 (&pop)[2]) {
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        o[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[2 * i + ks], pop[ks], o[i], 0, 0, 0);
  };

  // Iteration t: request tile t+1 into the other stage (free: tile t-1 used it and the last
  // barrier ended that), multiply tile t, then wait for the request and publish it.
  auto iteration = [&](int t, unsigned char* cur, unsigned char* nxt) {
    if (t + 1 < ntiles) {
      // keys of tile t+1: (t+1)*kKT .. min(kend, (t+2)*kKT) - 1
      const int last_blk = (min(kend, (t + 2) * kKT) - 1) / B;
      if (last_blk >= win0 + kTblWin) {  // uniform: move the window (no load reads it now)
        win0 = ((t + 1) * kKT) / B;
        load_window(win0);
        __syncthreads();
      }
      dma(nxt, t + 1);
    }
    const unsigned char* kb = cur;
    const unsigned char* vb = kb + SM::KBYTES;
    static_assert(kKT == 2 * kSub, "two steps per tile");
    const int k0 = t * kKT;
    // Both steps run unconditionally: on a last tile that ends in its first half, the second
    // step's keys are all past kend, masked to weight 0, and their V^T rows were zeroed.
    // The operand reads of a product are issued together, ahead of its matrix-core
    // instructions, so the wave waits for LDS once per group instead of once per product.
    f32x16 s0, s1;
    KOps ka, kc;
    read_k(kb, 0, ka);
    read_k(kb, 1, kc);
    qk(ka, s0);
    qk(kc, s1);
    bf16x8 p0[2], p1[2];
    VOps va, vc;
    read_v(vb, 0, va);
    softmax(k0, s0, p0);
    pv(va, p0);
    read_v(vb, 1, vc);
    softmax(k0 + kSub, s1, p1);
    pv(vc, p1);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's requests for tile t+1 have landed
    __syncthreads();
    if (t + 1 < ntiles && (t + 2) * kKT > kend) {  // uniform: tile t+1 is the last
      vfix(nxt, t + 1);
      __syncthreads();
    }
  };

  if (ntiles > 0) {
    dma(smem0, 0);
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();
  if (ntiles == 1) {
    vfix(smem0, 0);
    __syncthreads();
  }
  for (int t = 0; t < ntiles; t += 2) {
    iteration(t, smem0, smem1);
    if (t + 1 < ntiles) iteration(t + 1, smem1, smem0);
  }

  // bad table entries anywhere in the workgroup poison its outputs
  const int any_bad = __syncthreads_or(bad_entry);

  // ---- normalise and store: the two lane halves hold the row's two halves of the sum; lane
  // (hf, r32) holds row r32's dims 32 i + 8 g + 4 hf + 0..3 in o[i][4 g .. 4 g + 3].
  const float l = add_xor32(lpart);
  if (row_tok >= 0) {
    const float inv = (bad || any_bad) ? NAN : 1.f / l;
    uint16_t* op = a.out + ((static_cast<size_t>(s) * C + row_tok) * a.Hq + kvh * G + row_head) * D;
#pragma unroll
    for (int i = 0; i < NDT; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        uint2 pk2;
        pk2.x = static_cast<uint32_t>(f32_to_bf16(o[i][4 * g] * inv)) |
                (static_cast<uint32_t>(f32_to_bf16(o[i][4 * g + 1] * inv)) << 16);
        pk2.y = static_cast<uint32_t>(f32_to_bf16(o[i][4 * g + 2] * inv)) |
                (static_cast<uint32_t>(f32_to_bf16(o[i][4 * g + 3] * inv)) << 16);
        *reinterpret_cast<uint2*>(op + 32 * i + 8 * g + 4 * hf) = pk2;
      }
  }
}

// Persistent: a grid of as many workgroups as fit on the device at once (a multiple of kXcd),
// each running one unit per round of gridDim.x units.  The dispatcher deals workgroups
// round-robin to the kXcd XCDs, so workgroup g runs on XCD g % kXcd, and so does every unit it
// takes.  A workgroup per unit instead left each CU idle between one workgroup's end and the
// next one's first tile (dispatch, Q and table loads, the first tile's round trip) four times
// per kernel.
//
// In odd rounds a workgroup takes the unit mirrored within its XCD (g = 8 m + x -> 8 (M-1-m)
// + x for M = gridDim.x / 8).  Later query blocks of a group see more keys (the causal limit),
// and without the mirror a workgroup took the same block position in every round, so those
// holding the last blocks set the kernel's end; mirrored rounds pair long units with short.
template <int D, int B>
__global__ __launch_bounds__(kWaves * kWave) void chunk_kernel(Args a) {
  using SM = Smem<D>;
  __shared__ __attribute__((aligned(16))) unsigned char smem0[SM::STAGE];
  __shared__ __attribute__((aligned(16))) unsigned char smem1[SM::STAGE];
  // element offset of (physical block, kv-head) in the pools, for logical blocks win0 ..
  // win0 + kTblWin - 1 (K and V blocks share the stride B * D per head)
  __shared__ long long s_tbl[kTblWin];
  const int g = blockIdx.x, G = gridDim.x;
  const int mirrored = G - kXcd - g + 2 * (g % kXcd);
  for (int r = 0;; ++r) {
    const int L = ((r & 1) ? mirrored : g) + r * G;
    if (L >= a.units) break;
    chunk_unit<D, B>(a, L, smem0, smem1, s_tbl);
  }
}

}  // namespace chunk
}  // namespace pa

using namespace pa;

namespace {

// Workgroups of chunk_kernel<D, B> resident on the current device at once, rounded down to a
// multiple of kXcd (the persistent grid); cached per (kernel, device).
template <int D, int B>
int chunk_grid_cap() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, chunk::chunk_kernel<D, B>,
                                                   chunk::kWaves * kWave, 0) != hipSuccess)
    return 0;
  const int cap = cus * (per_cu > 0 ? per_cu : 1) / chunk::kXcd * chunk::kXcd;
  cache[dev] = cap < chunk::kXcd ? chunk::kXcd : cap;
  return cache[dev];
}

template <int D, int B>
pa_status launch_chunk(const chunk::Args& a, hipStream_t st) {
  const int cap = chunk_grid_cap<D, B>();
  if (cap <= 0) return fail(PA_ERR_HIP, "pa_chunk_attend: cannot query the device");
  const unsigned grid = static_cast<unsigned>(a.units < cap ? a.units : cap);
  hipLaunchKernelGGL((chunk::chunk_kernel<D, B>), dim3(grid), dim3(chunk::kWaves * kWave), 0, st, a);
  return launch_status("pa_chunk_attend");
}

}  // namespace

extern "C" pa_status pa_chunk_attend(void* out, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_tables,
                                     const int32_t* ctx_lens, int32_t S, int32_t C, int32_t Hq,
                                     int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks,
                                     int32_t max_blocks, float scale, int32_t dtype, void* stream) {
  if (dtype != PA_DTYPE_BF16) return fail(PA_ERR_UNSUPPORTED, "pa_chunk_attend: only bf16 is built");
  if (D != 64 && D != 128) return fail(PA_ERR_UNSUPPORTED, "pa_chunk_attend: head_dim %d not in {64, 128}", D);
  if (B != 16 && B != 32 && B != 64)
    return fail(PA_ERR_UNSUPPORTED, "pa_chunk_attend: block size %d not in {16, 32, 64}", B);
  if (S < 0 || C < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv)
    return fail(PA_ERR_INVALID_ARG, "pa_chunk_attend: S %d, C %d, Hq %d, Hkv %d", S, C, Hq, Hkv);
  const int G = Hq / Hkv;
  if (G > chunk::kRows) return fail(PA_ERR_UNSUPPORTED, "pa_chunk_attend: group of %d heads > %d", G, chunk::kRows);
  if (S > 65535 || Hkv > 65535) return fail(PA_ERR_INVALID_ARG, "pa_chunk_attend: S and Hkv must be <= 65535");
  if (num_blocks <= 0 || max_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "pa_chunk_attend: num_blocks %d, max_blocks %d", num_blocks, max_blocks);
  if (static_cast<int64_t>(C) > static_cast<int64_t>(max_blocks) * B)
    return fail(PA_ERR_INVALID_ARG, "pa_chunk_attend: chunk longer than a table row can hold");
  if (!(scale > 0.f) || scale == INFINITY)
    return fail(PA_ERR_INVALID_ARG, "pa_chunk_attend: scale must be positive and finite");
  if (S == 0 || C == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !ctx_lens)
    return fail(PA_ERR_INVALID_ARG, "pa_chunk_attend: NULL pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARG, "pa_chunk_attend: q, out and the pools must be 16-byte aligned");
  chunk::Args a{};
  a.out = static_cast<uint16_t*>(out);
  a.q = static_cast<const uint16_t*>(q);
  a.kc = static_cast<const uint16_t*>(k_cache);
  a.vc = static_cast<const uint16_t*>(v_cache);
  a.tables = block_tables;
  a.ctx_lens = ctx_lens;
  a.S = S;
  a.C = C;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = G;
  a.TQ = chunk::kRows / G;
  a.NQB = (C + a.TQ - 1) / a.TQ;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.scale_log2 = scale * chunk::kLog2e;
  const int64_t groups = (static_cast<int64_t>(S) * Hkv + chunk::kXcd - 1) / chunk::kXcd * chunk::kXcd;
  if (groups * a.NQB > INT_MAX) return fail(PA_ERR_INVALID_ARG, "pa_chunk_attend: grid too large");
  a.units = static_cast<int>(groups * a.NQB);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (D == 64) {
    if (B == 64) return launch_chunk<64, 64>(a, st);
    if (B == 16) return launch_chunk<64, 16>(a, st);
    return launch_chunk<64, 32>(a, st);
  }
  if (B == 64) return launch_chunk<128, 64>(a, st);
  if (B == 16) return launch_chunk<128, 16>(a, st);
  return launch_chunk<128, 32>(a, st);
}
