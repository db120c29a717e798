// Multi-head sub-network FFN core of FlashFFN (FlashFFN README, "Overview":
// O_h = sum_e R_e ((SiLU(Q_h K_e^T) * (Q_h U_e^T)) V_e); "Model
// configurations": 16 heads of d_h = 128, 15 sub-networks, 5760 = 15 x 384
// neurons per head at 1.3B).  bf16 Q, K, U, V, O; fp32 R; fp32 accumulation.
//
// Forward: one workgroup per (head, 128 tokens).  The [128 tokens x 128] Q
// tile and the router weights of the tile stay in LDS; the [d_h x 128 tokens]
// fp32 output accumulator stays in registers for the whole sweep over
// sub-networks and their 96-neuron chunks -- with d_h = 128 it fits, which is
// the point of the multi-head split (a d_model-wide accumulator would not).
// Eight wavefronts, each owning 32 tokens.  Per chunk three 24 KB loads stream
// through a three-stage direct-to-LDS ring:
//   KU0, KU1  [K rows; U rows] of the chunk, K (= d_h) 0..63 and 64..127
//             (K-row tiles) -> [h1; h2]^T for the chunk
//   epilogue  a = R * SiLU(h1) * h2 -> bf16 LDS tile [token][neuron]
//   V         V rows of the chunk as an N-row tile (rows = neurons, d_h
//             contiguous) -> O^T += V^T a^T
// The intermediate never leaves the chip.
#include "esg_internal.hpp"
#include "esg_tiles.hpp"

namespace esg {
namespace {

using namespace tiles;

constexpr int MH_DH = 128;       // head width the kernel is built for
constexpr int MH_TM = 128;       // tokens per workgroup
constexpr int MH_NC = 96;        // neurons per chunk (the 1.3B width 384 is four chunks)
constexpr int MH_NT = 512;       // eight wavefronts: (neuron half) x (32-token quarter)
constexpr int MH_NW = MH_NT / 64;
constexpr int MH_STAGE = 2 * MH_NC * 128;      // ring stage: [K; U] 192 x 128 B, or V 96 x 256 B
constexpr int MH_L = MH_STAGE / 1024 / MH_NW;  // DMA instructions per lane per stage
constexpr int MH_SUB = MH_TM * 128;            // one 64-wide K-row sub-tile of 128 tokens
constexpr int MH_MAXE = 32;      // sub-networks per head the router table holds
static_assert(MH_STAGE % (1024 * MH_NW) == 0, "whole DMA instructions per wave");

__global__ __launch_bounds__(MH_NT, 1) void mhffn_fwd_kernel(const bf16_t* __restrict__ q, const float* __restrict__ r,
                                                             const bf16_t* __restrict__ kw,
                                                             const bf16_t* __restrict__ uw,
                                                             const bf16_t* __restrict__ vw, int tokens, int heads,
                                                             int subnets, int d_sub, bf16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char ring_[3 * MH_STAGE];
  __shared__ __attribute__((aligned(1024))) char qt_[2 * MH_SUB];   // Q [token][d_h], two 64-wide K sub-tiles
  __shared__ __attribute__((aligned(1024))) char act_[2 * MH_SUB];  // a [token][neuron], neurons 0..63 | 64..95
  __shared__ float rtab[MH_TM * MH_MAXE];                           // router weights [token][sub-network]
  ESG_LDS char* ring = (ESG_LDS char*)ring_;
  ESG_LDS char* qt = (ESG_LDS char*)qt_;
  ESG_LDS char* act = (ESG_LDS char*)act_;

  const int h = blockIdx.y;
  const int t0 = blockIdx.x * MH_TM;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int nchunks = (d_sub + MH_NC - 1) / MH_NC;
  const int nsteps = subnets * nchunks * 3;
  const uint32_t qrow = (uint32_t)heads * MH_DH * 2;       // bytes between tokens in Q and O
  const uint32_t wbytes_he = (uint32_t)d_sub * MH_DH * 2;  // one sub-network's K (or U, V)

  const DmaSrc rq = make_dma_src(q, (uint32_t)tokens * qrow);
  const uint32_t wtotal = (uint32_t)heads * subnets * wbytes_he;
  const DmaSrc rk = make_dma_src(kw, wtotal);
  const DmaSrc ru = make_dma_src(uw, wtotal);
  const DmaSrc rv = make_dma_src(vw, wtotal);
  const int c8 = (lane & 7) ^ (lane >> 3);

  // ---- router weights of the tile -> LDS (plain loads, before any ring load) ----
  for (int i = threadIdx.x; i < MH_TM * subnets; i += MH_NT) {
    const int t = t0 + i / subnets;
    rtab[i] = t < tokens ? r[((size_t)t * heads + h) * subnets + i % subnets] : 0.0f;
  }

  // ---- Q tile: K-row, two 64-wide sub-tiles [token][d_h] ----
#pragma unroll
  for (int i = 0; i < 32 / MH_NW; ++i) {
    const int ii = w * (32 / MH_NW) + i;  // 32 instructions: sub-tile ii/16, rows (ii%16)*8 + lane/8
    const int sb = ii >> 4, row = (ii & 15) * 8 + (lane >> 3);
    const int t = t0 + row;
    dma16(rq, qt + sb * MH_SUB + (ii & 15) * 1024,
          t < tokens ? (uint32_t)t * qrow + (uint32_t)h * MH_DH * 2 + sb * 128 + c8 * 16 : kOOB);
  }

  // lane-invariant parts of the ring addressing
  int kurow[MH_L], vrow[MH_L], vj[MH_L];
#pragma unroll
  for (int i = 0; i < MH_L; ++i) {
    const int ii = w * MH_L + i;
    kurow[i] = ii * 8 + (lane >> 3);  // row of [K; U] (0 .. 2*NC-1)
    vrow[i] = ii * 4 + (lane >> 4);   // neuron row of V (0 .. NC-1)
    vj[i] = (lane & 15) ^ mn_swz<16>(vrow[i]);
  }
  // ring step s: chunk s/3 = (sub-network e, neuron chunk), part s%3
  auto issue = [&](ESG_LDS char* st, int s) __attribute__((always_inline)) {
    const int part = s % 3, ch = s / 3;
    const int e = ch / nchunks, n0 = (ch % nchunks) * MH_NC;
    const uint32_t base = (uint32_t)(h * subnets + e) * wbytes_he;
    if (part < 2) {  // [K rows; U rows] of the chunk, K columns part*64 .. +63 (128-byte rows)
#pragma unroll
      for (int i = 0; i < MH_L; ++i) {
        const bool is_k = (w * MH_L + i) * 8 < MH_NC;  // wave-uniform
        const int n = n0 + (is_k ? kurow[i] : kurow[i] - MH_NC);
        const uint32_t off = n < d_sub ? base + (uint32_t)n * MH_DH * 2 + part * 128 + c8 * 16 : kOOB;
        dma16(is_k ? rk : ru, st + (w * MH_L + i) * 1024, off);
      }
    } else {  // V rows of the chunk, N-row (256-byte rows, swizzled chunks)
#pragma unroll
      for (int i = 0; i < MH_L; ++i) {
        const int n = n0 + vrow[i];
        dma16(rv, st + (w * MH_L + i) * 1024, n < d_sub ? base + (uint32_t)n * MH_DH * 2 + vj[i] * 16 : kOOB);
      }
    }
  };

  // phase 1: neurons [wm*48, +48) of K and of U; tokens [wn*32, +32)
  // phase 2: d_h [wm*64, +64); the same tokens
  const int wm = w & 1, wn = w >> 1;
  constexpr int FP = MH_NC / 2 / 16, FN = 2;
  int arow[2 * FP], brow[FN];
#pragma unroll
  for (int p = 0; p < FP; ++p) {
    arow[p] = wm * (MH_NC / 2) + p * 16 + (lane & 15);
    arow[FP + p] = MH_NC + arow[p];
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) brow[j] = wn * 32 + j * 16 + (lane & 15);
  f32x4 acc1[2 * FP][FN];  // [h1 ; h2] x token fragments
  f32x4 acc2[4][FN];       // O^T: d_h [wm*64, +64) x the wave's tokens
  zero_acc(acc2);

  auto compute = [&](const ESG_LDS char* st, int s) __attribute__((always_inline)) {
    const int part = s % 3;
    if (part < 2) {  // [h1; h2]^T += [K; U] . Q^T over d_h half `part`
      if (part == 0) zero_acc(acc1);
      const ESG_LDS char* qs = qt + part * MH_SUB;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int c = kb * 4 + (lane >> 4);
        uint4 a[2 * FP], b[FN];
#pragma unroll
        for (int i = 0; i < 2 * FP; ++i) a[i] = frag_krow(st, arow[i], c);
#pragma unroll
        for (int j = 0; j < FN; ++j) b[j] = frag_krow(qs, brow[j], c);
#pragma unroll
        for (int i = 0; i < 2 * FP; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) mma_bf16(acc1[i][j], a[i], b[j]);
      }
      if (part == 1) {  // epilogue: a = R * SiLU(h1) * h2 -> act tile [token][neuron]
        const int e = (s / 3) / nchunks;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int tl = brow[j];
          const float rw = rtab[tl * subnets + e];
#pragma unroll
          for (int p = 0; p < FP; ++p) {
            const int n = wm * (MH_NC / 2) + p * 16 + (lane >> 4) * 4;  // 4 consecutive neurons
            float a[4];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              const float h1 = acc1[p][j][x], h2 = acc1[FP + p][j][x];
              a[x] = rw * (h1 * sigmoid_f(h1)) * h2;
            }
            lds_write8(act + (n >> 6) * MH_SUB + krow_off(tl, (n & 63) >> 3) + (n & 7) * 2, pack_bf16x2(a[0], a[1]),
                       pack_bf16x2(a[2], a[3]));
          }
        }
      }
    } else {  // O^T += V^T a^T over the chunk's neurons
#pragma unroll
      for (int kb = 0; kb < MH_NC / 32; ++kb) {
        const int sb = kb >> 1, c = (kb & 1) * 4 + (lane >> 4);
        uint4 a[4], b[FN];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = frag_nrow<16>(st, kb, wm * 64 + i * 16, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) b[j] = frag_krow(act + sb * MH_SUB, brow[j], c);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) mma_bf16(acc2[i][j], a[i], b[j]);
      }
    }
  };
  // the Q tile's loads are older than the ring's: the first step's wait covers them
  kloop<3, MH_L, 0>(nsteps, ring, ring + MH_STAGE, ring + 2 * MH_STAGE, issue, compute);
  wait_lgkm0();
  barrier();

  // ---- O rows through LDS: [token][d_h] bf16, whole 256-byte rows ----
  using RS = RowStore<MH_DH>;  // staging layout (rows of 256 bytes, swizzled 16-byte chunks)
  ESG_LDS char* out0 = ring;
  ESG_LDS char* out1 = ring + 64 * RS::RB;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      float v[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) v[x] = acc2[i][j][x];
      RS::put(out0, out1, brow[j], wm * 64 + i * 16 + (lane >> 4) * 4, v);
    }
  wait_lgkm0();
  barrier();
  const rsrc_t ro = make_rsrc(out, (uint32_t)tokens * qrow);
#pragma unroll
  for (int it = 0; it < MH_TM * RS::NCHK / MH_NT; ++it) {
    const int qi = it * MH_NT + threadIdx.x;
    const int rr = qi / RS::NCHK, c = qi % RS::NCHK, t = t0 + rr;
    const u32x4_t val = *(const ESG_LDS u32x4_t*)((rr < 64 ? out0 : out1) + RS::off(rr & 63, c));
    const uint32_t o = t < tokens ? (uint32_t)t * qrow + (uint32_t)h * MH_DH * 2 + c * 16 : kOOB;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i32, val), ro, o, 0, 0);
  }
}

// ===========================================================================
// Backward.  Nothing [tokens, sub-networks, d_sub]-sized is kept by the
// forward, so both kernels recompute h1, h2 and g = dO . V^T per chunk of
// neurons (a chunk's [K; U; V] rows over all of d_h sit in one stage as two
// 64-column K-row sub-tiles):
//   per token:   a = SiLU(h1) h2;  dR[t,e] = sum_n a g;  da = R g;
//                dh2 = da SiLU(h1);  dh1 = da h2 SiLU'(h1)
//   dQ/dR kernel (per head and 128 tokens; eight wavefronts; chunks of 32
//                neurons, with the router column of their sub-network,
//                through a three-stage ring):
//                dQ^T += [K; U]^T [dh1 dh2]^T, the stage's K and U rows read
//                transposed (rows = neuron = the K index, columns = d_h),
//                each wave a 16-wide d_h slice for all 128 tokens; dQ
//                accumulates in registers over all chunks, each token's dR
//                over its sub-network's chunks
//   dW kernel    (per head, sub-network and 64-neuron chunk held in LDS, all tokens in
//                steps of 64): dK^T += Q^T dh1, dU^T += Q^T dh2,
//                dV^T += dO^T (R a), the Q / dO tiles and the per-step
//                [token][neuron] tiles read transposed
// ===========================================================================
constexpr int MB_TM = 64;                 // tokens per tile
constexpr int MB_TSUB = MB_TM * 128;      // one 64-wide K-row sub-tile of a 64-token tile (8 KB)
constexpr int MB_NW = 4;

// A chunk of NC neurons of one sub-network: its [K; U; V] rows over all of
// d_h as two 64-column K-row sub-tiles.
template <int NC, int NW = MB_NW>
struct Chunk {
  static constexpr int ROWS = 3 * NC;
  static constexpr int FR = ROWS / 16;           // 16-row fragments: K, U, V in turn
  static constexpr int HALF = ROWS * 128;        // one 64-column sub-tile
  static constexpr int STAGE = 2 * HALF;
  static constexpr int LW = STAGE / 1024 / NW;   // DMA instructions per lane (NW waves)
  static_assert(NC % 16 == 0 && STAGE % (1024 * NW) == 0, "whole fragments and DMA instructions");
};

// DMA of one chunk's [K; U; V] rows (neurons n0 .. n0+NC-1 of the sub-network
// at `base`): instruction ii covers sub-tile ii/(ROWS/8), rows (ii%(ROWS/8))*8 .. +7.
template <int NC, int NW = MB_NW>
__device__ __forceinline__ void issue_chunk(const DmaSrc& rk, const DmaSrc& ru, const DmaSrc& rv, ESG_LDS char* st,
                                            int w, int lane, uint32_t base, int n0, int d_sub) {
  using C = Chunk<NC, NW>;
  constexpr int PER = C::ROWS / 8;
  const int c8 = (lane & 7) ^ (lane >> 3);
#pragma unroll
  for (int i = 0; i < C::LW; ++i) {
    const int ii = w * C::LW + i;
    const int sub = ii / PER, rb = (ii % PER) * 8;
    const int mat = rb / NC;  // 0 K, 1 U, 2 V (wave-uniform: 8-row blocks never straddle)
    const int n = n0 + rb % NC + (lane >> 3);
    const uint32_t off = n < d_sub ? base + (uint32_t)n * MH_DH * 2 + sub * 128 + c8 * 16 : kOOB;
    dma16(mat == 0 ? rk : (mat == 1 ? ru : rv), st + sub * C::HALF + (ii % PER) * 1024, off);
  }
}

// DMA of a [TM tokens][128] bf16 head slice (Q or dO) into two K-row sub-tiles
// of TM * 128 bytes: TM/4 instructions, TM/4/NW per wave.  SWZ2: in the second
// swizzle (krow_swz2).
template <int NW = MB_NW, bool SWZ2 = false, int TM = MB_TM>
__device__ __forceinline__ void issue_tokens(const DmaSrc& src, ESG_LDS char* dst, int w, int lane, int t0,
                                             int tokens, uint32_t qrow, int h) {
  constexpr int PER = TM / 8;  // instructions per sub-tile
#pragma unroll
  for (int i = 0; i < TM / 4 / NW; ++i) {
    const int ii = w * (TM / 4 / NW) + i;
    const int sb = ii / PER, row = (ii % PER) * 8 + (lane >> 3);
    // position lane & 7 of the row takes chunk (lane & 7) ^ swizzle(row); row
    // bit 3 is ii & 1
    const int c8 = (lane & 7) ^ (lane >> 3) ^ (SWZ2 ? (ii & 1) * 5 : 0);
    const int t = t0 + row;
    dma16(src, dst + sb * (TM * 128) + (ii % PER) * 1024,
          t < tokens ? (uint32_t)t * qrow + (uint32_t)h * MH_DH * 2 + sb * 128 + c8 * 16 : kOOB);
  }
}

// Phase 1 of a chunk for the 16 tokens [tok0, +16): acc[f] (K, U, V row
// fragments in turn) = stage rows . [Q | Q | dO]^T over all of d_h.
template <int NC>
__device__ __forceinline__ void chunk_phase1(const ESG_LDS char* st, const ESG_LDS char* qt, const ESG_LDS char* dot,
                                             int tok0, int lane, f32x4 (&acc)[Chunk<NC>::FR]) {
  using C = Chunk<NC>;
  zero_acc(acc);
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int c = kb * 4 + (lane >> 4);
      const uint4 bq = frag_krow(qt + sub * MB_TSUB, tok0 + (lane & 15), c);
      const uint4 bo = frag_krow(dot + sub * MB_TSUB, tok0 + (lane & 15), c);
#pragma unroll
      for (int f = 0; f < C::FR; ++f) {
        const uint4 a = frag_krow(st + sub * C::HALF, f * 16 + (lane & 15), c);
        mma_bf16(acc[f], a, f < 2 * C::FR / 3 ? bq : bo);
      }
    }
}

// Phase 1 of 16 of a chunk's neurons (fragment p of each of K, U, V) for the
// 16 tokens [tok0, +16): acc = {h1, h2, g} of those neurons (the layout of a
// 16-neuron chunk, so chunk_grads<16> applies).
template <int NC, int TSUB = MB_TSUB>
__device__ __forceinline__ void chunk_phase1_part(const ESG_LDS char* st, const ESG_LDS char* qt,
                                                  const ESG_LDS char* dot, int tok0, int p, int lane,
                                                  f32x4 (&acc)[3]) {
  using C = Chunk<NC>;
  constexpr int F1 = NC / 16;
  zero_acc(acc);
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int c = kb * 4 + (lane >> 4);
      const uint4 bq = frag_krow(qt + sub * TSUB, tok0 + (lane & 15), c);
      const uint4 bo = frag_krow(dot + sub * TSUB, tok0 + (lane & 15), c);
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        const uint4 a = frag_krow(st + sub * C::HALF, (m * F1 + p) * 16 + (lane & 15), c);
        mma_bf16(acc[m], a, m < 2 ? bq : bo);
      }
    }
}

// The per-token chunk epilogue on one lane's 4 consecutive neurons (x) of
// fragment p: returns sum_x a*g and the bf16 pairs of dh1, dh2 and R*a.
struct ChunkGrads {
  float dr;
  uint32_t dh1[2], dh2[2], ra[2];
};
template <int NC>
__device__ __forceinline__ ChunkGrads chunk_grads(const f32x4 (&acc)[Chunk<NC>::FR], int p, float rw) {
  constexpr int F1 = NC / 16;
  ChunkGrads o;
  float d1[4], d2[4], ra[4];
  o.dr = 0.0f;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const float h1 = acc[p][x], h2 = acc[F1 + p][x], g = acc[2 * F1 + p][x];
    const float sg = sigmoid_f(h1);
    const float silu = h1 * sg;
    const float a = silu * h2;
    o.dr += a * g;
    const float da = rw * g;
    d2[x] = da * silu;
    d1[x] = da * h2 * (sg * (1.0f + h1 * (1.0f - sg)));
    ra[x] = rw * a;
  }
  o.dh1[0] = pack_bf16x2(d1[0], d1[1]);
  o.dh1[1] = pack_bf16x2(d1[2], d1[3]);
  o.dh2[0] = pack_bf16x2(d2[0], d2[1]);
  o.dh2[1] = pack_bf16x2(d2[2], d2[3]);
  o.ra[0] = pack_bf16x2(ra[0], ra[1]);
  o.ra[1] = pack_bf16x2(ra[2], ra[3]);
  return o;
}

// chunk widths: 32 neurons for the dQ/dR kernel (three 24 KB ring stages fit
// beside its resident tiles), 48 for the weight-gradient kernel (its chunk is
// resident; wider chunks mean fewer passes over the tokens)
constexpr int MBQ_NC = 32, MBW_NC = 64;

// Eight waves for the dQ/dR kernel.
constexpr int MBQ_NW = 8;

// dQ/dR over 128-token tiles (eight waves): phase 1 wave w takes tokens
// [(w%4)*32, +32) (two 16-token fragments) and neurons [(w/4)*16, +16) of the
// 32-neuron chunk; phase 2 d_h [w*16, +16) for all 128 tokens, so each
// barrier pair carries twice the MFMA work of a 64-token tile and each chunk's
// weights serve twice the tokens.  The router column of the chunk's
// sub-network rides in the ring stage (a 4-byte DMA per token), and each
// token's dR for the current sub-network accumulates in a register of its
// writer lane (the same chunk order as a per-tile table), stored after the
// sub-network's last chunk.
constexpr int MBQ2_TM = 128, MBQ2_TSUB = MBQ2_TM * 128;
__global__ __launch_bounds__(64 * MBQ_NW, 1) void mhffn_bwd_dq_kernel(
    const bf16_t* __restrict__ dout, const bf16_t* __restrict__ q, const float* __restrict__ r,
    const bf16_t* __restrict__ kw, const bf16_t* __restrict__ uw, const bf16_t* __restrict__ vw, int tokens,
    int heads, int subnets, int d_sub, bf16_t* __restrict__ dq, float* __restrict__ dr) {
  using C = Chunk<MBQ_NC, MBQ_NW>;
  static_assert(MBQ_NC == 32 && MBQ_NW == 8, "two neuron halves of 16 x four token groups of 32");
  // chunk rows, the router column (128 x 4 B), a sink for the other waves' empty router loads
  constexpr int R_OFF = C::STAGE, SINK_OFF = C::STAGE + 512, RSTAGE = C::STAGE + 1024;
  constexpr int L = C::LW + 1;  // loads per lane per stage
  __shared__ __attribute__((aligned(1024))) char ring_[3 * RSTAGE];
  __shared__ __attribute__((aligned(1024))) char qt_[2 * MBQ2_TSUB];
  __shared__ __attribute__((aligned(1024))) char dot_[2 * MBQ2_TSUB];
  __shared__ __attribute__((aligned(1024))) char dh_[MBQ2_TSUB];  // [token][dh1 (32) | dh2 (32)]
  __shared__ float drpart[2][MBQ2_TM];                            // the step's dR sums of each neuron half
  ESG_LDS char* ring = (ESG_LDS char*)ring_;
  ESG_LDS char* qt = (ESG_LDS char*)qt_;
  ESG_LDS char* dot = (ESG_LDS char*)dot_;
  ESG_LDS char* dh = (ESG_LDS char*)dh_;

  const int h = blockIdx.y, t0 = blockIdx.x * MBQ2_TM;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int nchunks = (d_sub + MBQ_NC - 1) / MBQ_NC;
  const uint32_t qrow = (uint32_t)heads * MH_DH * 2;
  const uint32_t wbytes_he = (uint32_t)d_sub * MH_DH * 2;
  const uint32_t wtotal = (uint32_t)heads * subnets * wbytes_he;
  const DmaSrc rk = make_dma_src(kw, wtotal), ru = make_dma_src(uw, wtotal), rv = make_dma_src(vw, wtotal);
  const DmaSrc rr = make_dma_src(r, (uint32_t)tokens * heads * subnets * 4);

  issue_tokens<MBQ_NW, false, MBQ2_TM>(make_dma_src(q, (uint32_t)tokens * qrow), qt, w, lane, t0, tokens, qrow, h);
  issue_tokens<MBQ_NW, false, MBQ2_TM>(make_dma_src(dout, (uint32_t)tokens * qrow), dot, w, lane, t0, tokens, qrow,
                                       h);

  const int nh = w >> 2;         // neuron half of phase 1
  const int tg = (w & 3) * 32;   // the wave's 32 tokens (two fragments)
  f32x4 acc1[2][3];
  f32x4 acc2[8];  // dQ^T: d_h [w*16, +16) x the tile's 8 token fragments
  zero_acc(acc2);
  float dracc[2] = {0.0f, 0.0f};  // writer lanes (nh == 0, lane < 16): tokens tg + i*16 + lane
  auto issue = [&](ESG_LDS char* st, int s) __attribute__((always_inline)) {
    const int e = s / nchunks, n0 = (s % nchunks) * MBQ_NC;
    issue_chunk<MBQ_NC, MBQ_NW>(rk, ru, rv, st, w, lane, (uint32_t)(h * subnets + e) * wbytes_he, n0, d_sub);
    // router column of sub-network e: waves 0 and 1 load tokens [w*64, +64),
    // the others an empty load into the sink (every wave counts L loads)
    const int t = t0 + w * 64 + lane;
    dma4(rr, st + (w < 2 ? R_OFF + w * 256 : SINK_OFF),
         (w < 2 && t < tokens) ? ((uint32_t)t * heads + h) * subnets * 4 + e * 4 : kOOB);
  };
  auto compute = [&](const ESG_LDS char* st, int s) __attribute__((always_inline)) {
    const int e = s / nchunks;
#pragma unroll
    for (int i = 0; i < 2; ++i) chunk_phase1_part<MBQ_NC, MBQ2_TSUB>(st, qt, dot, tg + i * 16, nh, lane, acc1[i]);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int tl = tg + i * 16 + (lane & 15);
      const float rw = *(const ESG_LDS float*)(st + R_OFF + tl * 4);
      const ChunkGrads cg = chunk_grads<16>(acc1[i], 0, rw);
      const int n = nh * 16 + (lane >> 4) * 4;  // dh1 column n, dh2 column 32 + n
      lds_write8(dh + krow_off(tl, n >> 3) + (n & 7) * 2, cg.dh1[0], cg.dh1[1]);
      const int n2 = MBQ_NC + n;
      lds_write8(dh + krow_off(tl, n2 >> 3) + (n2 & 7) * 2, cg.dh2[0], cg.dh2[1]);
      float drp = cg.dr;
      drp += __shfl_xor(drp, 16);
      drp += __shfl_xor(drp, 32);
      if (lane < 16) drpart[nh][tl] = drp;
    }
    wait_lgkm0();
    barrier();  // every wave's dh rows and dR halves are written
    if (nh == 0 && lane < 16) {  // one writer per token
      const bool last = s % nchunks == nchunks - 1;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int tl = tg + i * 16 + lane;
        dracc[i] += drpart[0][tl] + drpart[1][tl];
        if (last) {
          const int t = t0 + tl;
          if (t < tokens) dr[((size_t)t * heads + h) * subnets + e] = dracc[i];
          dracc[i] = 0.0f;
        }
      }
    }
    // dQ^T += [K; U]^T [dh1 dh2]^T  (K index = the 64 K and U neuron rows of the
    // stage); wave w takes d_h [w*16, +16) for all 128 tokens
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint4 a = frag_krow_t(st + (w >> 2) * C::HALF, kb, (w & 3) * 16, lane);
      uint4 b[8];
#pragma unroll
      for (int tf = 0; tf < 8; ++tf) b[tf] = frag_krow(dh, tf * 16 + (lane & 15), kb * 4 + (lane >> 4));
#pragma unroll
      for (int tf = 0; tf < 8; ++tf) mma_bf16(acc2[tf], a, b[tf]);
    }
  };
  // the Q and dO tiles' loads are older than the ring's: the first wait covers them
  kloop<3, L, 0>(subnets * nchunks, ring, ring + RSTAGE, ring + 2 * RSTAGE, issue, compute);
  wait_lgkm0();
  barrier();

#pragma unroll
  for (int tf = 0; tf < 8; ++tf) {
    const int t = t0 + tf * 16 + (lane & 15);
    if (t < tokens) {
      const int j = w * 16 + (lane >> 4) * 4;
      float v[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) v[x] = acc2[tf][x];
      Quad<bf16_t>::store(dq + ((size_t)t * heads + h) * MH_DH + j, v);
    }
  }
}

// Eight waves over a resident chunk of 64 neurons: for phase 1 wave w takes
// tokens [(w%4)*16, +16) and neurons [(w/4)*32, +32) (fragments of K, U, V in
// the layout of a 32-neuron chunk); for phase 2 it takes d_h [(w%4)*32, +32) x
// neurons [(w/4)*32, +32) of dK, dU and dV.  Two ring stages fit beside the
// 48 KB chunk and the three [token][neuron] tiles.
constexpr int MBW_NW = 8;
__global__ __launch_bounds__(64 * MBW_NW, 1) void mhffn_bwd_dw_kernel(
    const bf16_t* __restrict__ dout, const bf16_t* __restrict__ q, const float* __restrict__ r,
    const bf16_t* __restrict__ kw, const bf16_t* __restrict__ uw, const bf16_t* __restrict__ vw, int tokens,
    int heads, int subnets, int d_sub, bf16_t* __restrict__ dk, bf16_t* __restrict__ du, bf16_t* __restrict__ dv) {
  using C = Chunk<MBW_NC, MBW_NW>;
  static_assert(MBW_NC == 64 && MBW_NW == 8, "four token groups x two neuron halves of 32");
  // Q (2 sub-tiles), dO (2), router weights (4 x 256 B), and 1 KB where the
  // second neuron half's empty router loads land (an out-of-range load still
  // writes its zeros to LDS)
  constexpr int TSTAGE = 4 * MB_TSUB + 2048;
  constexpr int LT = 2 * (16 / MBW_NW) + 1;  // loads per lane per token stage
  __shared__ __attribute__((aligned(1024))) char wt_[C::STAGE];
  __shared__ __attribute__((aligned(1024))) char ring_[2 * TSTAGE];
  __shared__ __attribute__((aligned(1024))) char tiles_[3 * MB_TSUB];  // [token][64] dh1 | dh2 | R*a
  ESG_LDS char* wt = (ESG_LDS char*)wt_;
  ESG_LDS char* ring = (ESG_LDS char*)ring_;
  ESG_LDS char* t_dh1 = (ESG_LDS char*)tiles_;
  ESG_LDS char* t_dh2 = t_dh1 + MB_TSUB;
  ESG_LDS char* t_ra = t_dh2 + MB_TSUB;

  const int n0 = blockIdx.x * MBW_NC, e = blockIdx.y, h = blockIdx.z;
  const int lane = threadIdx.x & 63, w = wave_id();
  const uint32_t qrow = (uint32_t)heads * MH_DH * 2;
  const uint32_t wbytes_he = (uint32_t)d_sub * MH_DH * 2;
  const uint32_t wtotal = (uint32_t)heads * subnets * wbytes_he;
  const uint32_t base = (uint32_t)(h * subnets + e) * wbytes_he;
  issue_chunk<MBW_NC, MBW_NW>(make_dma_src(kw, wtotal), make_dma_src(uw, wtotal), make_dma_src(vw, wtotal), wt, w,
                              lane, base, n0, d_sub);
  const DmaSrc rq = make_dma_src(q, (uint32_t)tokens * qrow);
  const DmaSrc ro = make_dma_src(dout, (uint32_t)tokens * qrow);
  const DmaSrc rr = make_dma_src(r, (uint32_t)tokens * heads * subnets * 4);

  const int tg = w & 3, nh = w >> 2;
  const int tok0 = tg * 16, tl = tok0 + (lane & 15);
  auto issue = [&](ESG_LDS char* st, int s) __attribute__((always_inline)) {
    const int t0 = s * MB_TM;
    issue_tokens<MBW_NW, true>(rq, st, w, lane, t0, tokens, qrow, h);
    issue_tokens<MBW_NW, true>(ro, st + 2 * MB_TSUB, w, lane, t0, tokens, qrow, h);
    // router weights of token group tg: lanes 0..15 of the waves of the first
    // neuron half, 4 bytes each (the other waves issue an empty load into the
    // sink, so that every wave counts the same loads)
    const int t = t0 + tok0 + lane;
    dma4(rr, st + 4 * MB_TSUB + nh * 1024 + tg * 256,
         (nh == 0 && lane < 16 && t < tokens) ? ((uint32_t)t * heads + h) * subnets * 4 + e * 4 : kOOB);
  };
  // phase 2 wave tile: d_h [tg*32, +32) x neurons [nh*32, +32), for dK, dU, dV
  f32x4 acc2[3][2][2];
  zero_acc(acc2);
  f32x4 acc1[6];  // K0 K1 U0 U1 V0 V1 of the wave's 32 neurons
  // the resident chunk's phase-1 fragments of the wave's neurons, read from
  // LDS once (step 0) and kept in registers: [d_h sub-tile][32-wide K block][fragment]
  uint4 wf[2][2][6];
  auto compute = [&](const ESG_LDS char* st, int s) __attribute__((always_inline)) {
    const ESG_LDS char* qs = st;
    const ESG_LDS char* os = st + 2 * MB_TSUB;
    if (s == 0) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int f = 0; f < 6; ++f) {
            const int row = ((f >> 1) * (MBW_NC / 16) + nh * 2 + (f & 1)) * 16 + (lane & 15);  // mat f/2
            wf[sub][kb][f] = frag_krow(wt + sub * C::HALF, row, kb * 4 + (lane >> 4));
          }
    }
    zero_acc(acc1);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int c = kb * 4 + (lane >> 4);
        const uint4 bq = frag_krow2(qs + sub * MB_TSUB, tl, c);
        const uint4 bo = frag_krow2(os + sub * MB_TSUB, tl, c);
#pragma unroll
        for (int f = 0; f < 6; ++f) mma_bf16(acc1[f], wf[sub][kb][f], f < 4 ? bq : bo);
      }
    const float rw = *(const ESG_LDS float*)(st + 4 * MB_TSUB + tg * 256 + (lane & 15) * 4);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const ChunkGrads cg = chunk_grads<32>(acc1, p, rw);
      const int n = nh * 32 + p * 16 + (lane >> 4) * 4;
      const int o = krow_off2(tl, n >> 3) + (n & 7) * 2;
      lds_write8(t_dh1 + o, cg.dh1[0], cg.dh1[1]);
      lds_write8(t_dh2 + o, cg.dh2[0], cg.dh2[1]);
      lds_write8(t_ra + o, cg.ra[0], cg.ra[1]);
    }
    wait_lgkm0();
    barrier();  // every wave's part of the tiles is written
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {  // K = the tile's 64 tokens
      uint4 aq[2], ao[2], b1[2], b2[2], br[2];
#pragma unroll
      for (int jf = 0; jf < 2; ++jf) {
        const int j0 = tg * 32 + jf * 16;
        aq[jf] = frag_krow_t2(qs + (j0 >> 6) * MB_TSUB, kb, j0 & 63, lane);
        ao[jf] = frag_krow_t2(os + (j0 >> 6) * MB_TSUB, kb, j0 & 63, lane);
      }
#pragma unroll
      for (int nf = 0; nf < 2; ++nf) {
        const int c0 = nh * 32 + nf * 16;
        b1[nf] = frag_krow_t2(t_dh1, kb, c0, lane);
        b2[nf] = frag_krow_t2(t_dh2, kb, c0, lane);
        br[nf] = frag_krow_t2(t_ra, kb, c0, lane);
      }
#pragma unroll
      for (int jf = 0; jf < 2; ++jf)
#pragma unroll
        for (int nf = 0; nf < 2; ++nf) {
          mma_bf16(acc2[0][jf][nf], aq[jf], b1[nf]);
          mma_bf16(acc2[1][jf][nf], aq[jf], b2[nf]);
          mma_bf16(acc2[2][jf][nf], ao[jf], br[nf]);
        }
    }
  };
  // the resident chunk's loads are older than the ring's: the first wait covers them
  kloop<2, LT, 0>((tokens + MB_TM - 1) / MB_TM, ring, ring + TSTAGE, ring, issue, compute);
  wait_vmcnt<0>();  // with no tokens the resident chunk may still be landing

  bf16_t* outs[3] = {dk, du, dv};
#pragma unroll
  for (int m = 0; m < 3; ++m)
#pragma unroll
    for (int jf = 0; jf < 2; ++jf)
#pragma unroll
      for (int nf = 0; nf < 2; ++nf) {
        const int j = tg * 32 + jf * 16 + (lane >> 4) * 4;
        const int n = n0 + nh * 32 + nf * 16 + (lane & 15);
        if (n < d_sub) {
          float v[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) v[x] = acc2[m][jf][nf][x];
          Quad<bf16_t>::store(outs[m] + ((size_t)(h * subnets + e) * d_sub + n) * MH_DH + j, v);
        }
      }
}

}  // namespace

bool mhffn_supported(int tokens, int heads, int d_head, int subnets, int d_sub) {
  if (tokens < 0 || heads <= 0 || subnets <= 0 || d_sub <= 0) return false;
  if (d_head != MH_DH || d_sub % 8 || subnets > MH_MAXE) return false;
  const long long act = (long long)tokens * heads * d_head * 2;
  const long long w = (long long)heads * subnets * d_sub * d_head * 2;
  return act < (1ll << 31) && w < (1ll << 31);
}

hipError_t launch_mhffn_bwd(const void* dout, const void* q, const float* r, const void* k, const void* u,
                            const void* v, int tokens, int heads, int subnets, int d_sub, void* dq, float* dr,
                            void* dk, void* du, void* dv, hipStream_t stream) {
  if (tokens > 0) {
    LaunchTimer timer("mhffn_bwd_dq", stream);
    hipLaunchKernelGGL(mhffn_bwd_dq_kernel, dim3((tokens + MBQ2_TM - 1) / MBQ2_TM, heads), dim3(64 * MBQ_NW), 0,
                       stream, (const bf16_t*)dout, (const bf16_t*)q, r, (const bf16_t*)k, (const bf16_t*)u,
                       (const bf16_t*)v, tokens, heads, subnets, d_sub, (bf16_t*)dq, dr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  LaunchTimer timer("mhffn_bwd_dw", stream);
  hipLaunchKernelGGL(mhffn_bwd_dw_kernel, dim3((d_sub + MBW_NC - 1) / MBW_NC, subnets, heads), dim3(64 * MBW_NW), 0, stream,
                     (const bf16_t*)dout, (const bf16_t*)q, r, (const bf16_t*)k, (const bf16_t*)u, (const bf16_t*)v,
                     tokens, heads, subnets, d_sub, (bf16_t*)dk, (bf16_t*)du, (bf16_t*)dv);
  return hipGetLastError();
}

hipError_t launch_mhffn_fwd(const void* q, const float* r, const void* k, const void* u, const void* v, int tokens,
                            int heads, int subnets, int d_sub, void* out, hipStream_t stream) {
  if (tokens == 0) return hipSuccess;
  LaunchTimer timer("mhffn_fwd", stream);
  hipLaunchKernelGGL(mhffn_fwd_kernel, dim3((tokens + MH_TM - 1) / MH_TM, heads), dim3(MH_NT), 0, stream,
                     (const bf16_t*)q, r, (const bf16_t*)k, (const bf16_t*)u, (const bf16_t*)v, tokens, heads,
                     subnets, d_sub, (bf16_t*)out);
  return hipGetLastError();
}

}  // namespace esg
