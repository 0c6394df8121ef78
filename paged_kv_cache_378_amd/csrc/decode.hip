// Paged decode attention on gfx950: split-K over context partitions, then a merge.
//
// What is computed ("vLLM PagedAttention" (tinycto), FAQ: mathematically identical to
// standard multi-head attention; KV-cache chapter, "Common misconception": the same scores and
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
//   * one workgroup per (sequence, kv-head, partition of PT tokens); NW = 4 waves split the
//     partition's 32-token tiles round-robin and each keeps its own online-softmax state
//     (running max m, running sum l, unnormalised output o), scores in the log2 domain;
//   * the partition's block-table slice is staged in LDS once, so tile loads never wait on a
//     dependent table load;
//   * the four wave states are merged through LDS; a single-partition sequence writes its
//     final output directly, otherwise the partition writes (m, l, o/l) and a merge kernel
//     combines the partitions (the FlashAttention-style tiling the KV-cache chapter mentions
//     in "Common misconception").
//   * GQA groups (bf16, g >= 3): QK^T and PV are real dense contractions of g heads against
//     the tile, done on the matrix cores (v_mfma_f32_16x16x32_bf16).  S^T = K Q^T puts 16
//     tokens on the rows and the (padded) 16 heads on the columns; O^T = V^T P^T contracts
//     over tokens.  Each lane loads 16-byte runs straight into its MFMA operand registers:
//     K rows are contiguous in the K pool, and the V pool is stored transposed per block so
//     8 consecutive tokens of one dim are contiguous too.  No LDS round trip for K/V.
//   * one query head per kv-head (g in {1, 2}) or fp32: a VALU kernel; LPT lanes share one
//     token's dot product (reduced with cross-lane shuffles), the round max uses shuffles, and
//     the PV update broadcasts the round's weights through a per-wave LDS slot.
//
// Tiles beyond the context are never formed; lanes whose token lies past ctx_len load a
// clamped in-range address and their score is set to -inf and their V elements to zero, so
// values past the end (even NaN) cannot reach the output.

#include <cmath>

#include "device_common.h"

namespace pa {

constexpr int kNW = 4;            // waves per workgroup
constexpr int kMaxPT = 8192;      // largest partition (tokens)
constexpr int kMinAutoPT = 256;   // smallest partition the automatic choice uses
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  void* out;
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* tables;
  const int32_t* ctx_lens;
  float* part_o;    // [S, Hq, Pmax, D]  partition outputs (normalised)
  float2* part_ml;  // [S, Hq, Pmax]     (max in log2 units, sum)
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

// ---------------------------------------------------------------------------------------
// Shared epilogue: merge the NW wave states held in LDS and store.
// s_ml[w][h] = (m, l); s_o[w][h][d] = unnormalised output of wave w relative to its own m.
// ---------------------------------------------------------------------------------------
template <typename T, int D, int HMAX>
__device__ void finish_partition(const DecodeArgs& a, int s, int kvh, int part, int nparts,
                                 bool bad, float (*s_ml)[HMAX][2], float (*s_o)[HMAX][D]) {
  const int G = a.G;
  for (int idx = threadIdx.x; idx < G * D; idx += kNW * kWave) {
    const int h = idx / D, d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kNW; ++w) M = fmaxf(M, s_ml[w][h][0]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int w = 0; w < kNW; ++w) {
      const float sc = exp2f(s_ml[w][h][0] - M);
      L += s_ml[w][h][1] * sc;
      O += s_o[w][h][d] * sc;
    }
    const int hq = kvh * G + h;
    const float r = bad ? NAN : O / L;
    if (nparts == 1) {
      static_cast<T*>(a.out)[(static_cast<size_t>(s) * a.Hq + hq) * D + d] = Elem<T>::from_f32(r);
    } else {
      const size_t row = (static_cast<size_t>(s) * a.Hq + hq) * a.Pmax + part;
      a.part_o[row * D + d] = r;
      if (d == 0) a.part_ml[row] = bad ? make_float2(0.f, NAN) : make_float2(M, L);
    }
  }
}

// Stage the partition's slice of the block table in LDS.  Entries outside the pool are
// replaced by block 0 (so every load stays inside the pool) and flag the partition as bad.
__device__ __forceinline__ void stage_table(const DecodeArgs& a, int s, int b0, int nb,
                                            int* s_tbl, int* s_bad) {
  if (threadIdx.x == 0) *s_bad = 0;
  __syncthreads();
  const int32_t* row = a.tables + static_cast<size_t>(s) * a.max_blocks + b0;
  for (int i = threadIdx.x; i < nb; i += kNW * kWave) {
    int p = row[i];
    if (p < 0 || p >= a.num_blocks) {
      *s_bad = 1;
      p = 0;
    }
    s_tbl[i] = p;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------------------
// MFMA kernel: bf16, 1 <= G <= 16 query heads per kv-head, D in {64, 128}, B in {16, 32}.
// ---------------------------------------------------------------------------------------
template <int D, int B>
struct MfmaTile {
  static constexpr int NST = D / 32;  // k-steps of QK^T (8 dims per lane per step)
  static constexpr int NNT = D / 16;  // 16-dim output tiles of PV
  bf16x8 k[2][NST];                   // two 16-token row groups
  bf16x8 v[NNT];                      // V^T rows (dims) x 8 tokens
};

template <int D, int B>
__global__ __launch_bounds__(kNW * kWave) void decode_mfma_kernel(DecodeArgs a) {
  using Tile = MfmaTile<D, B>;
  constexpr int NST = Tile::NST, NNT = Tile::NNT;
  __shared__ int s_tbl[kMaxPT / B];
  __shared__ int s_bad;
  __shared__ float s_ml[kNW][16][2];
  __shared__ float s_o[kNW][16][D];

  const int part = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
  bool bad_len;
  const int n = eff_len(a.ctx_lens[s], a.len_cap, bad_len);
  const int nparts = n > 0 ? (n + a.PT - 1) / a.PT : 1;
  const int t0 = part * a.PT;
  if (part >= nparts) return;
  const int t1 = min(n, t0 + a.PT);
  const int b0 = t0 / B;
  const int nb = (t1 + B - 1) / B - b0;

  const int lane = threadIdx.x & (kWave - 1), w = wave_id();
  const int r16 = lane & 15, gp = lane >> 4;
  const uint16_t* kc = static_cast<const uint16_t*>(a.kc);
  const uint16_t* vc = static_cast<const uint16_t*>(a.vc);

  stage_table(a, s, b0, nb > 0 ? nb : 0, s_tbl, &s_bad);

  // Q^T operand: column = head r16 (zero for padded heads), k = 8 dims per step.
  bf16x8 qop[NST];
  {
    const int h = r16 < a.G ? r16 : 0;
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<size_t>(s) * a.Hq + kvh * a.G + h) * D;
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      uint4 u = *reinterpret_cast<const uint4*>(qp + 8 * (4 * st + gp));
      if (r16 >= a.G) u = make_uint4(0, 0, 0, 0);
      qop[st] = __builtin_bit_cast(bf16x8, u);
    }
  }

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 o[NNT];
#pragma unroll
  for (int i = 0; i < NNT; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = n > 0 ? (t1 - t0 + 31) / 32 : 0;
  const size_t head_stride = static_cast<size_t>(B) * D;  // elements per (block, kv-head)

  // Issue the global loads of tile `tile` into `tl`.
  auto load = [&](Tile& tl, int tile) {
    const int tt = t0 + 32 * tile;
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      // row r16 of row group m holds token 8*(r16/4) + 4*m + r16%4 of the tile, so that after
      // QK^T lane group gp owns tokens 8*gp .. 8*gp+7 (the PV operand layout).
      int tok = tt + 8 * (r16 >> 2) + 4 * m + (r16 & 3);
      tok = min(tok, t1 - 1);
      const int p = s_tbl[tok / B - b0];
      const uint16_t* kp = kc + (static_cast<size_t>(p) * a.Hkv + kvh) * head_stride +
                           static_cast<size_t>(tok % B) * D;
#pragma unroll
      for (int st = 0; st < NST; ++st)
        tl.k[m][st] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(kp + 8 * (4 * st + gp)));
    }
    int tv = tt + 8 * gp;
    tv = min(tv, (t1 - 1) & ~7);
    const int p = s_tbl[tv / B - b0];
    const uint16_t* vp = vc + (static_cast<size_t>(p) * a.Hkv + kvh) * head_stride + (tv % B);
#pragma unroll
    for (int ni = 0; ni < NNT; ++ni)
      tl.v[ni] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(vp + (16 * ni + r16) * B));
  };

  auto compute = [&](Tile& tl, int tile) {
    const int tt = t0 + 32 * tile;
    f32x4 sacc[2];
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      sacc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < NST; ++st)
        sacc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl.k[m][st], qop[st], sacc[m], 0, 0, 0);
    }
    // lane (gp, r16): scores of head r16 for tokens tt + 8*gp + j, j = 4*m + i
    const int valid = t1 - (tt + 8 * gp);  // tokens of this lane's group that exist
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float v = sacc[j >> 2][j & 3] * a.scale_log2;
      x[j] = j < valid ? v : -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
    mx = fmaxf(mx, shfl_xor(mx, 16));
    mx = fmaxf(mx, shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    bf16x8 pop;
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const __bf16 pb = static_cast<__bf16>(exp2f(x[j] - m_new));
      pop[j] = pb;
      psum += static_cast<float>(pb);
    }
    l_run = l_run * alpha + psum;
    if (valid < 8) {  // tail: zero the V elements of tokens past the end
#pragma unroll
      for (int ni = 0; ni < NNT; ++ni) {
        uint16_t vv[8];
        __builtin_memcpy(vv, &tl.v[ni], 16);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j >= valid) vv[j] = 0;
        __builtin_memcpy(&tl.v[ni], vv, 16);
      }
    }
#pragma unroll
    for (int ni = 0; ni < NNT; ++ni) {
      o[ni] *= alpha;
      o[ni] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tl.v[ni], pop, o[ni], 0, 0, 0);
    }
  };

  // Two register sets: the next tile's loads are in flight while the current one computes.
  int tile = w;
  if (tile < ntiles) {
    Tile ta, tb;
    load(ta, tile);
    for (;;) {
      if (tile + kNW >= ntiles) { compute(ta, tile); break; }
      load(tb, tile + kNW);
      compute(ta, tile);
      tile += kNW;
      if (tile + kNW >= ntiles) { compute(tb, tile); break; }
      load(ta, tile + kNW);
      compute(tb, tile);
      tile += kNW;
    }
  }

  // Wave state -> LDS.  l_run is per lane (its 8 tokens); sum the four lane groups.
  l_run += shfl_xor(l_run, 16);
  l_run += shfl_xor(l_run, 32);
  if (gp == 0) {
    s_ml[w][r16][0] = m_run;
    s_ml[w][r16][1] = l_run;
  }
#pragma unroll
  for (int ni = 0; ni < NNT; ++ni)
#pragma unroll
    for (int i = 0; i < 4; ++i) s_o[w][r16][16 * ni + 4 * gp + i] = o[ni][i];
  __syncthreads();
  finish_partition<uint16_t, D, 16>(a, s, kvh, part, nparts, bad_len || s_bad, s_ml, s_o);
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
template <typename T, int D, int B, int G, int LPT>
__global__ __launch_bounds__(kNW * kWave) void decode_valu_kernel(DecodeArgs a) {
  constexpr int VEC = 16 / sizeof(T);   // elements per 16-byte load
  constexpr int TPR = kWave / LPT;      // tokens per round
  constexpr int CPL = D / LPT / VEC;    // 16-byte chunks of a key row per lane
  constexpr int DPL = CPL * VEC;        // dims per lane in QK
  constexpr int DV = D / kWave;         // dims per lane in PV
  constexpr int VPR = TPR * sizeof(T) / 16;  // 16-byte loads per V^T row piece
  static_assert(CPL >= 1, "head_dim too small for LPT");
  static_assert(B % TPR == 0, "a round must stay inside one block");
  static_assert(VPR >= 1 && TPR % 4 == 0, "V rows are read in 16-byte pieces");

  __shared__ int s_tbl[kMaxPT / B];
  __shared__ int s_bad;
  __shared__ float s_ml[kNW][G][2];
  __shared__ float s_o[kNW][G][D];
  __shared__ __attribute__((aligned(16))) float s_p[kNW][G][TPR];  // weights of the round

  const int part = blockIdx.x, kvh = blockIdx.y, s = blockIdx.z;
  bool bad_len;
  const int n = eff_len(a.ctx_lens[s], a.len_cap, bad_len);
  const int nparts = n > 0 ? (n + a.PT - 1) / a.PT : 1;
  const int t0 = part * a.PT;
  if (part >= nparts) return;
  const int t1 = min(n, t0 + a.PT);
  const int b0 = t0 / B;
  const int nb = (t1 + B - 1) / B - b0;

  const int lane = threadIdx.x & (kWave - 1), w = wave_id();
  const int tk = lane / LPT, pp = lane % LPT;
  const T* kc = static_cast<const T*>(a.kc);
  const T* vc = static_cast<const T*>(a.vc);

  stage_table(a, s, b0, nb > 0 ? nb : 0, s_tbl, &s_bad);

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

  float m_run[G], l_run[G], acc[G][DV];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int e = 0; e < DV; ++e) acc[h][e] = 0.f;
  }

  const size_t head_stride = static_cast<size_t>(B) * D;
  const int nrounds = n > 0 ? (t1 - t0 + TPR - 1) / TPR : 0;

  for (int r = w; r < nrounds; r += kNW) {
    const int tt = t0 + TPR * r;
    // ---- loads: this lane's key slice (clamped to a live token) and its V^T rows
    const int tok = min(tt + tk, t1 - 1);
    const T* kp = kc + (static_cast<size_t>(s_tbl[tok / B - b0]) * a.Hkv + kvh) * head_stride +
                  static_cast<size_t>(tok % B) * D;
    uint4 kr[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) kr[i] = *reinterpret_cast<const uint4*>(kp + (pp + LPT * i) * VEC);
    const T* vp = vc + (static_cast<size_t>(s_tbl[tt / B - b0]) * a.Hkv + kvh) * head_stride + (tt % B);
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
  finish_partition<T, D, G>(a, s, kvh, part, nparts, bad_len || s_bad, s_ml, s_o);
}

// ---------------------------------------------------------------------------------------
// Partition merge: m = max_p m_p; out = sum_p o_p l_p 2^(m_p - m) / sum_p l_p 2^(m_p - m).
// One workgroup per (head, sequence); sequences with one partition were finished already.
// ---------------------------------------------------------------------------------------
template <typename T, int D, int B>
__global__ __launch_bounds__(D) void merge_kernel(DecodeArgs a) {
  const int hq = blockIdx.x, s = blockIdx.y, d = threadIdx.x;
  bool bad;
  const int n = eff_len(a.ctx_lens[s], a.len_cap, bad);
  const int nparts = n > 0 ? (n + a.PT - 1) / a.PT : 1;
  if (nparts <= 1) return;
  const size_t row = (static_cast<size_t>(s) * a.Hq + hq) * a.Pmax;
  const float2* ml = a.part_ml + row;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[p].x);
  float L = 0.f, O = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float2 e = ml[p];
    const float wgt = e.y * exp2f(e.x - M);
    L += wgt;
    O = fmaf(wgt, a.part_o[(row + p) * D + d], O);
  }
  const float r = bad ? NAN : O / L;
  static_cast<T*>(a.out)[(static_cast<size_t>(s) * a.Hq + hq) * D + d] = Elem<T>::from_f32(r);
}

// ---------------------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------------------
static int auto_partition(int S, int Hkv, int max_ctx_len) {
  (void)S;
  (void)Hkv;
  (void)max_ctx_len;
  return 512;
}

static size_t workspace_bytes(int S, int Hq, int D, int Pmax) {
  if (Pmax <= 1) return 0;
  const size_t rows = static_cast<size_t>(S) * Hq * Pmax;
  const size_t ml = (rows * sizeof(float2) + 255) & ~size_t(255);
  return ml + rows * D * sizeof(float);
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

template <int D, int B>
static pa_status launch(const DecodeArgs& a, int32_t dtype, hipStream_t stream) {
  KernelFn k = nullptr;
  if (dtype == PA_DTYPE_BF16 && a.G >= 3 && a.G <= 16)
    k = decode_mfma_kernel<D, B>;
  else
    k = pick_valu<D, B>(dtype, a.G);
  if (!k)
    return fail(PA_ERR_UNSUPPORTED,
                "pa_decode: %d query heads per kv-head not supported for dtype %d "
                "(bf16: 1..16, f32: 1, 2, 4, 8)", a.G, dtype);
  hipLaunchKernelGGL(k, dim3(a.Pmax, a.Hkv, a.S), dim3(kNW * kWave), 0, stream, a);
  if (pa_status st = launch_status("pa_decode")) return st;
  if (a.Pmax > 1) {
    if (dtype == PA_DTYPE_F32)
      hipLaunchKernelGGL((merge_kernel<float, D, B>), dim3(a.Hq, a.S), dim3(D), 0, stream, a);
    else
      hipLaunchKernelGGL((merge_kernel<uint16_t, D, B>), dim3(a.Hq, a.S), dim3(D), 0, stream, a);
    return launch_status("pa_decode (merge)");
  }
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
  const int Pmax = max_ctx_len > 0 ? (max_ctx_len + pt - 1) / pt : 1;
  *bytes = workspace_bytes(S, Hq, D, Pmax);
  return ok();
}

extern "C" pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* ctx_lens, int32_t S,
                               int32_t Hq, int32_t Hkv, int32_t D, int32_t B, int32_t num_blocks,
                               int32_t max_blocks, int32_t max_ctx_len, float scale, int32_t dtype,
                               int32_t partition_tokens, void* workspace, size_t workspace_bytes_in,
                               void* stream) {
  if (elem_bytes(dtype) == 0) return fail(PA_ERR_UNSUPPORTED, "pa_decode: dtype %d", dtype);
  if (D != 64 && D != 128) return fail(PA_ERR_UNSUPPORTED, "pa_decode: head_dim %d not in {64, 128}", D);
  if (B != 16 && B != 32) return fail(PA_ERR_UNSUPPORTED, "pa_decode: block size %d not in {16, 32}", B);
  if (S < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv)
    return fail(PA_ERR_INVALID_ARG, "pa_decode: S %d, Hq %d, Hkv %d (Hq must be a multiple of Hkv)", S, Hq, Hkv);
  if (S > 65535 || Hkv > 65535) return fail(PA_ERR_INVALID_ARG, "pa_decode: S and Hkv must be <= 65535");
  if (num_blocks <= 0 || max_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "pa_decode: num_blocks %d, max_blocks %d", num_blocks, max_blocks);
  if (max_ctx_len < 1 || static_cast<int64_t>(max_ctx_len) > static_cast<int64_t>(max_blocks) * B)
    return fail(PA_ERR_INVALID_ARG, "pa_decode: max_ctx_len %d outside [1, max_blocks*B]", max_ctx_len);
  if (partition_tokens != 0 && (partition_tokens % 32 || partition_tokens < 32 || partition_tokens > kMaxPT))
    return fail(PA_ERR_INVALID_ARG, "pa_decode: partition_tokens %d is not a multiple of 32 in [32, %d]",
                partition_tokens, kMaxPT);
  if (!(scale == scale)) return fail(PA_ERR_INVALID_ARG, "pa_decode: scale is NaN");
  if (S == 0) return ok();
  if (!out || !q || !k_cache || !v_cache || !block_tables || !ctx_lens)
    return fail(PA_ERR_INVALID_ARG, "pa_decode: NULL pointer");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARG, "pa_decode: q, out and the pools must be 16-byte aligned");

  DecodeArgs a{};
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
  a.PT = partition_tokens ? partition_tokens : auto_partition(S, Hkv, max_ctx_len);
  a.Pmax = (max_ctx_len + a.PT - 1) / a.PT;
  a.len_cap = max_ctx_len;  // validated above: max_ctx_len <= max_blocks * B
  a.scale_log2 = scale * kLog2e;
  const size_t need = workspace_bytes(S, Hq, D, a.Pmax);
  if (need > 0) {
    if (!workspace || workspace_bytes_in < need)
      return fail(PA_ERR_WORKSPACE, "pa_decode: workspace of %zu bytes needed, %zu given", need,
                  workspace ? workspace_bytes_in : size_t(0));
    if (!aligned16(workspace)) return fail(PA_ERR_INVALID_ARG, "pa_decode: workspace must be 16-byte aligned");
    const size_t rows = static_cast<size_t>(S) * Hq * a.Pmax;
    const size_t ml = (rows * sizeof(float2) + 255) & ~size_t(255);
    a.part_ml = static_cast<float2*>(workspace);
    a.part_o = reinterpret_cast<float*>(static_cast<char*>(workspace) + ml);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (D == 64) return B == 16 ? launch<64, 16>(a, dtype, st) : launch<64, 32>(a, dtype, st);
  return B == 16 ? launch<128, 16>(a, dtype, st) : launch<128, 32>(a, dtype, st);
}
