// The dense limit of the layer: every group active (k = G), i.e. the plain
// SwiGLU feed-forward block y = (SiLU(x W_g^T) * (x W_u^T)) W_d^T and its
// gradients (eugen_sparse README, "What it does": the layer with all groups
// selected; the FlashFFN README, "Why", for the on-chip capacity limit of a
// one-pass fused FFN at d_model >= 2048).
//
// Forward (dense_fwd_kernel): token-stationary.  A workgroup owns 32 tokens
// and the whole fp32 [32, d] output accumulator in registers (d <= 2048: 128
// per lane over 8 wavefronts).  It sweeps d_ff in chunks of 128
// neurons: phase 1 computes [hg; hu] for the chunk (K = d), the gated
// activation goes bf16 into an LDS tile, phase 2 adds W_d[:, chunk] . a^T to
// the accumulator (K = 128).  The [tokens, d_ff] intermediate never exists in
// HBM; weights stream through a 4-stage direct-to-LDS ring and are shared
// through L2 by the workgroups that sweep the same chunk.
//
// Backward: over token chunks of at most 8192 tokens, with gate/up recomputed
// (nothing is saved by the forward):
//   dense_rec_kernel  per (128-token tile, 128-neuron block): hg, hu, dA
//                     (K = d), SiLU' epilogue -> dg, du, a in a chunk-sized
//                     workspace laid out [block][chunk rows][128];
//   dense_dx_kernel   dx = dg W_g + du W_u for the chunk's tokens (K = d_ff);
//   dense_dw_kernel   the weight-gradient tiles of the sparse path over the
//                     chunk's tokens, accumulated across chunks in fp32 in a
//                     fixed chunk order (deterministic).
#include "esg_internal.hpp"
#include "esg_tiles.hpp"

namespace esg {
namespace {

using namespace tiles;

// ===========================================================================
// Forward
// ===========================================================================
struct DFwd {
  static constexpr int NTD = 512;               // 8 wavefronts
  static constexpr int TM = 32;                 // tokens per workgroup
  static constexpr int FC = 128;                // neurons per chunk
  static constexpr int MAXDB = 16;              // 128-row d-blocks held (d <= 2048)
  static constexpr int A_BYTES = 2 * FC * 128;  // phase-1 weights: 256 rows x 64 K
  static constexpr int STAGE = A_BYTES + TM * 128;  // + x tile (32 rows x 64 K)
  static constexpr int NSTG = 4;
  static constexpr int L = 6;                   // DMA instructions per lane per stage
  static constexpr int ATILE = 2 * TM * 128;    // a tile: 32 tokens x 128 neurons (two K halves)
};

__global__ __launch_bounds__(DFwd::NTD, 1) void dense_fwd_kernel(const bf16_t* __restrict__ x,
                                                                 const bf16_t* __restrict__ wg,
                                                                 const bf16_t* __restrict__ wu,
                                                                 const bf16_t* __restrict__ wd, int tokens, int d,
                                                                 int F, bf16_t* __restrict__ y) {
  using C = DFwd;
  __shared__ __attribute__((aligned(1024))) char ring_[C::NSTG * C::STAGE];
  __shared__ __attribute__((aligned(1024))) char atile_[C::ATILE];
  ESG_LDS char* ring = (ESG_LDS char*)ring_;
  ESG_LDS char* atile = (ESG_LDS char*)atile_;

  const int lane = threadIdx.x & 63, w = wave_id();
  const int tok0 = blockIdx.x * C::TM;
  const uint32_t kbytes = (uint32_t)d * 2;
  const uint32_t fbytes = (uint32_t)F * 2;
  const int nk1 = (d + 63) / 64;            // phase-1 stages per chunk
  const int nd = (d + 127) / 128;           // phase-2 stages per chunk
  const int S = nk1 + nd;
  const int nchunks = (F + C::FC - 1) / C::FC;
  const int total = nchunks * S;

  const DmaSrc rx = make_dma_src(x, (uint32_t)tokens * kbytes);
  const DmaSrc rg = make_dma_src(wg, (uint32_t)F * kbytes);
  const DmaSrc ru = make_dma_src(wu, (uint32_t)F * kbytes);
  const DmaSrc rd = make_dma_src(wd, (uint32_t)d * fbytes);

  // 16-byte slots: chunk c_lane of row 8*k + lane/8 (K-row swizzle)
  const int c_lane = (lane & 7) ^ (lane >> 3);
  const int r8 = lane >> 3;
  // x tile by 4-byte slots: instruction m of wave w fills bytes (w*2 + m)*256 + 4*lane
  uint32_t xoff[2], xk[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int o = (w * 2 + m) * 256 + lane * 4;
    const int r = o >> 7, pch = (o & 127) >> 4, e = (o & 15) >> 2;
    xk[m] = ((pch ^ (r & 7)) << 4) + e * 4;  // byte of the row's 64-wide K slice
    xoff[m] = tok0 + r < tokens ? (uint32_t)(tok0 + r) * kbytes + xk[m] : kOOB;
  }

  auto issue = [&](int t, ESG_LDS char* st) __attribute__((always_inline)) {
    const int c = t / S, j = t - c * S;
    if (j < nk1) {
      // [W_g; W_u] rows of the chunk, 64 K from j*64; then the x tile
      const uint32_t kb = (uint32_t)j * 128;
      const bool kin = kb + c_lane * 16 < kbytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = w * 4 + i;              // 1 KB slot of the stage
        const int n = c * C::FC + ((g * 8 + r8) & (C::FC - 1));
        const bool ok = kin && n < F;
        dma16(g * 8 < C::FC ? rg : ru, st + g * 1024, ok ? (uint32_t)n * kbytes + kb + c_lane * 16 : kOOB);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)
        dma4(rx, st + C::A_BYTES + (w * 2 + m) * 256,
             (xoff[m] != kOOB && kb + xk[m] < kbytes) ? xoff[m] + kb : kOOB);
    } else {
      // W_d rows of d-block j - nk1, chunk columns in two 64-wide K halves
      const int db0 = (j - nk1) * 128;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int g = w * 4 + i;
        const int h = g >> 4, r = (g & 15) * 8 + r8;
        const int n = c * C::FC + h * 64 + c_lane * 8;
        const bool ok = db0 + r < d && n < F;
        dma16(rd, st + h * (128 * 128) + (g & 15) * 1024, ok ? (uint32_t)(db0 + r) * fbytes + (uint32_t)n * 2 : kOOB);
      }
#pragma unroll
      for (int m = 0; m < 2; ++m)  // keeps L uniform; lands in the unused x area
        dma4(rd, st + C::A_BYTES + (w * 2 + m) * 256, kOOB);
    }
  };

  // phase 1: wave w owns neurons [16w, 16w+16) of gate and of up, all 32 tokens
  const int arow0 = w * 16 + (lane & 15);
  int brow[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) brow[q] = q * 16 + (lane & 15);
  f32x4 acc1[2][2];
  // phase 2: wave w owns d rows db*128 + 16w + 0..15 of every d-block, all 32 tokens
  f32x4 acc2[C::MAXDB][2];
#pragma unroll
  for (int db = 0; db < C::MAXDB; ++db)
#pragma unroll
    for (int q = 0; q < 2; ++q) acc2[db][q] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 afr[4][2];  // a^T fragments of the chunk (K = 128 neurons)



  for (int t = 0; t < C::NSTG - 1 && t < total; ++t) issue(t, ring + t * C::STAGE);
  int t = 0, slot = 0;  // global stage index, t % NSTG
  // wait for stage t (the NSTG-2 younger stages may still be in flight), then
  // refill the stage every wave finished reading in step t-1
  auto head = [&]() __attribute__((always_inline)) {
    const int younger = total - 1 - t;
    if (younger >= 2)
      wait_vmcnt<2 * C::L>();
    else if (younger == 1)
      wait_vmcnt<C::L>();
    else
      wait_vmcnt<0>();
    wait_lgkm0();
    barrier();
    if (t + C::NSTG - 1 < total) issue(t + C::NSTG - 1, ring + (slot == 0 ? C::NSTG - 1 : slot - 1) * C::STAGE);
  };
  auto next = [&]() __attribute__((always_inline)) {
    ++t;
    slot = slot + 1 == C::NSTG ? 0 : slot + 1;
  };
  for (int c = 0; c < nchunks; ++c) {
    zero_acc(acc1);
    for (int j = 0; j < nk1; ++j) {
      head();
      const ESG_LDS char* st = ring + slot * C::STAGE;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int cc = kb * 4 + (lane >> 4);
        uint4 a[2], b[2];
        a[0] = frag_krow(st, arow0, cc);
        a[1] = frag_krow(st, C::FC + arow0, cc);
#pragma unroll
        for (int q = 0; q < 2; ++q) b[q] = frag_krow(st + C::A_BYTES, brow[q], cc);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int q = 0; q < 2; ++q) mma_bf16(acc1[i][q], a[i], b[q]);
      }
      next();
    }
    // a = SiLU(hg) * hu -> LDS a tile [token][neuron] (K-row, two 64-wide halves);
    // the previous chunk read its a tile before barriers every wave has passed
    {
      const int n = w * 16 + (lane >> 4) * 4;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        float a[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float hg = acc1[0][q][e], hu = acc1[1][q][e];
          a[e] = hg * sigmoid_f(hg) * hu;
        }
        lds_write8(atile + (n >> 6) * (C::TM * 128) + krow_off(brow[q], (n & 63) >> 3) + (n & 7) * 2,
                   pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
      }
    }
#pragma unroll
    for (int db = 0; db < C::MAXDB; ++db) {
      if (db < nd) {
        head();  // its barrier also publishes the a tile
        if (db == 0) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int q = 0; q < 2; ++q)
              afr[kb][q] = frag_krow(atile + (kb >> 1) * (C::TM * 128), brow[q], (kb & 1) * 4 + (lane >> 4));
        }
        const ESG_LDS char* st = ring + slot * C::STAGE;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const uint4 a = frag_krow(st + (kb >> 1) * (128 * 128), arow0, (kb & 1) * 4 + (lane >> 4));
#pragma unroll
          for (int q = 0; q < 2; ++q) mma_bf16(acc2[db][q], a, afr[kb][q]);
        }
        next();
      }
    }
  }
  // y rows: lane holds four consecutive d values of one token
#pragma unroll
  for (int db = 0; db < C::MAXDB; ++db) {
    if (db >= nd) continue;
    const int dd = db * 128 + w * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int tk = tok0 + brow[q];
      if (dd >= d || tk >= tokens) continue;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc2[db][q][e];
      Quad<bf16_t>::store(y + (size_t)tk * d + dd, v);
    }
  }
}

// ===========================================================================
// Backward
// ===========================================================================
constexpr int NB = 128;  // neurons per block
constexpr int DENSE_DW_XS = 2;  // 128-d sub-tiles per weight-gradient workgroup

// Token ids of a chunk's padded rows (-1 past the chunk's last token).
__global__ void dense_route_kernel(int t0, int tc, int tc_pad, int32_t* __restrict__ ptoken) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < tc_pad) ptoken[i] = i < tc ? t0 + i : -1;
}

// hg, hu, dA for one (128-token tile, 128-neuron block) of a chunk; writes
// dg, du, a rows to the packed layout [block][tc_pad][128].  Eight waves:
// the direct-to-LDS loads of the one workgroup per CU are issued by twice
// the waves of the 4-wave tile helpers' default.
constexpr int REC_NW = 8;
__global__ __launch_bounds__(64 * REC_NW, 1) void dense_rec_kernel(const bf16_t* __restrict__ x,
                                                          const bf16_t* __restrict__ dy,
                                                          const bf16_t* __restrict__ wg,
                                                          const bf16_t* __restrict__ wu,
                                                          const bf16_t* __restrict__ wd, int tokens, int d, int F,
                                                          const int32_t* __restrict__ ptoken, int tc_pad,
                                                          bf16_t* __restrict__ dg, bf16_t* __restrict__ du,
                                                          bf16_t* __restrict__ act) {
  using CF = Fwd2<NB, REC_NW>;
  using CD = Dh2<NB, REC_NW>;
  constexpr int NS = 3;
  constexpr int STG = CF::STAGE > CD::STAGE ? CF::STAGE : CD::STAGE;
  __shared__ __attribute__((aligned(1024))) char st0_[STG], st1_[STG], st2_[STG];
  ESG_LDS char* st0 = (ESG_LDS char*)st0_;
  ESG_LDS char* st1 = (ESG_LDS char*)st1_;
  ESG_LDS char* st2 = (ESG_LDS char*)st2_;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int tile = blockIdx.x, blk = blockIdx.y;
  const int nb0 = blk * NB;
  const uint32_t prow0 = (uint32_t)tile * BM;

  f32x4 gu[2 * CF::FMP][CF::FN];
  {
    ESG_LDS char* const st[NS] = {st0, st1, st2};
    gateup_tile<NB, NS, REC_NW>(x, wg, wu, tokens, d, F, nb0, ptoken, prow0, st, gu);
  }
  wait_lgkm0();
  barrier();  // the stages are reused
  f32x4 da[CD::FM][CD::FN];
  da_tile<NB, NS, REC_NW>(dy, wd, tokens, d, F, nb0, ptoken, prow0, st0, st1, st2, da);

  // both tiles use the same mapping: neurons wm*(NB/WM) + i*16 + (lane/16)*4 + e,
  // positions wn*64 + j*16 + lane%16
  static_assert(CF::WM == CD::WM && CF::FMP == CD::FM && CF::FN == CD::FN, "one wave mapping");
  const int wm = w % CD::WM, wn = w / CD::WM;
  // dg, du, a go out as whole rows, staged in st0, st1, st2
  using RE = RowStore<NB, 64 * REC_NW>;
  constexpr int EH = 128 * RE::RB;
  static_assert(EH <= STG, "one array per stage");
  wait_lgkm0();
  barrier();  // every wave is done with the stages
#pragma unroll
  for (int i = 0; i < CD::FM; ++i) {
    const int n = wm * (NB / CD::WM) + i * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < CD::FN; ++j) {
      const int r = wn * 64 + j * 16 + (lane & 15);
      float dgv[4], duv[4], av[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float hg = gu[i][j][e], hu = gu[CF::FMP + i][j][e], dA = da[i][j][e];
        const float sg = sigmoid_f(hg);
        const float silu = hg * sg;
        dgv[e] = dA * hu * (sg * (1.0f + hg * (1.0f - sg)));
        duv[e] = dA * silu;
        av[e] = silu * hu;
      }
      RE::put(st0, st0 + EH / 2, r, n, dgv);
      RE::put(st1, st1 + EH / 2, r, n, duv);
      RE::put(st2, st2 + EH / 2, r, n, av);
    }
  }
  uint32_t roffE[RE::IT];
#pragma unroll
  for (int it = 0; it < RE::IT; ++it) roffE[it] = (uint32_t)RE::row(it, threadIdx.x) * NB * 2;
  const size_t r0 = ((size_t)blk * tc_pad + prow0) * NB;
  wait_lgkm0();
  barrier();  // the rows are staged
  RE::template flush<0>(st0, st0 + EH / 2, make_rsrc(dg + r0, BM * NB * 2), roffE, 0, NB);
  RE::template flush<0>(st1, st1 + EH / 2, make_rsrc(du + r0, BM * NB * 2), roffE, 0, NB);
  RE::template flush<0>(st2, st2 + EH / 2, make_rsrc(act + r0, BM * NB * 2), roffE, 0, NB);
}

// dx[t0 + tile*128 + m, d-block] = sum over blocks of dg W_g + du W_u.
// C^T (d x tokens) = W^T (d x K) . [dg du]^T (K x tokens): the weights come in
// as N-row tiles (K = neuron rows, d contiguous), dg/du as K-row tiles.  A
// workgroup's block is 128 tokens x 256 d: the weight rows as two 128-d N-row
// sub-tiles, so each staged dg/du tile feeds twice the MFMAs of a 128-d block.
// Eight waves (one workgroup per CU): wave (wm, wn) owns d [wm*64, +64) x
// tokens [wn*64, +64) of the block; every wave issues IA + IB loads per stage.
struct DDx {
  static constexpr int NW = 8;
  static constexpr int DW = 256;                // d per block
  static constexpr int SUBA = 64 * 256;         // one sub-tile: 64 neuron rows x 128 d
  static constexpr int A_BYTES = (DW / 128) * SUBA;
  static constexpr int B_BYTES = BM * 128;      // 128 tokens x 64 neurons
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int IA = A_BYTES / 1024 / NW, IB = B_BYTES / 1024 / NW;
  static constexpr int L = IA + IB;
  static constexpr int WM = NW / 2, FM = DW / WM / 16, FN = 4;
  static_assert(IA * 1024 * NW == A_BYTES && IB * 1024 * NW == B_BYTES, "whole DMA instructions");
};

__global__ __launch_bounds__(64 * DDx::NW, 1) void dense_dx_kernel(const bf16_t* __restrict__ wg,
                                                         const bf16_t* __restrict__ wu, int d, int F, int t0,
                                                         int tc, int tc_pad, const bf16_t* __restrict__ dg,
                                                         const bf16_t* __restrict__ du, bf16_t* __restrict__ dx) {
  using C = DDx;
  __shared__ __attribute__((aligned(1024))) char st0_[C::STAGE], st1_[C::STAGE], st2_[C::STAGE];
  ESG_LDS char* st0 = (ESG_LDS char*)st0_;
  ESG_LDS char* st1 = (ESG_LDS char*)st1_;
  ESG_LDS char* st2 = (ESG_LDS char*)st2_;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int tile = blockIdx.x, db0 = blockIdx.y * C::DW;
  const int nblk = (F + NB - 1) / NB;
  const uint32_t kbytes = (uint32_t)d * 2;
  const DmaSrc rg = make_dma_src(wg, (uint32_t)F * kbytes);
  const DmaSrc ru = make_dma_src(wu, (uint32_t)F * kbytes);
  const uint32_t pbytes = (uint32_t)((size_t)nblk * tc_pad * NB * 2);
  const DmaSrc rdg = make_dma_src(dg, pbytes);
  const DmaSrc rdu = make_dma_src(du, pbytes);

  // A: instruction ii = w*IA + i fills sub-tile ii/16 (d from db0 + 128*(ii/16)),
  // neuron row kr = (ii%16)*4 + lane/16, 16-byte chunk jz
  int jz[C::IA];
#pragma unroll
  for (int i = 0; i < C::IA; ++i) jz[i] = (lane & 15) ^ mn_swz<16>(((w * C::IA + i) & 15) * 4 + (lane >> 4));
  // B: packed row (w*IB + i)*8 + lane/8, chunk c_lane
  const int c_lane = (lane & 7) ^ (lane >> 3);
  // stage kt: block kt/4, half (kt/2)&1 (0: dg with W_g, 1: du with W_u), 64-neuron sub-block kt&1
  auto issue = [&](ESG_LDS char* st, int kt) __attribute__((always_inline)) {
    const int blk = kt >> 2, h = (kt >> 1) & 1, sb = kt & 1;
    const int n0 = blk * NB + sb * 64;
#pragma unroll
    for (int i = 0; i < C::IA; ++i) {
      const int ii = w * C::IA + i;
      const int kr = (ii & 15) * 4 + (lane >> 4), dsub = db0 + (ii >> 4) * 128;
      const bool ok = n0 + kr < F && dsub + jz[i] * 8 < d;
      dma16(h ? ru : rg, st + ii * 1024, ok ? (uint32_t)(n0 + kr) * kbytes + (uint32_t)dsub * 2 + jz[i] * 16 : kOOB);
    }
    const uint32_t rbase = ((uint32_t)blk * tc_pad + (uint32_t)tile * BM) * (NB * 2) + sb * 128 + c_lane * 16;
#pragma unroll
    for (int i = 0; i < C::IB; ++i) {
      const int r = (w * C::IB + i) * 8 + (lane >> 3);
      dma16(h ? rdu : rdg, st + C::A_BYTES + (w * C::IB + i) * 1024, rbase + (uint32_t)r * (NB * 2));
    }
  };
  const int wm = w % C::WM, wn = w / C::WM;
  f32x4 acc[C::FM][C::FN];
  zero_acc(acc);
  auto compute = [&](const ESG_LDS char* st, int) __attribute__((always_inline)) {
    uint4 a[2][C::FM];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < C::FM; ++i) {
        const int dl = wm * (C::DW / C::WM) + i * 16;  // d within the block: sub-tile dl/128
        a[kb][i] = frag_nrow<16>(st + (dl >> 7) * C::SUBA, kb, dl & 127, lane);
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint4 b[C::FN];
#pragma unroll
      for (int j = 0; j < C::FN; ++j) b[j] = frag_krow(st + C::A_BYTES, wn * 64 + j * 16 + (lane & 15), kb * 4 + (lane >> 4));
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) mma_bf16(acc[i][j], a[kb][i], b[j]);
    }
  };
  kloop<3, C::L, 0>(nblk * 4, st0, st1, st2, issue, compute);
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int dd = db0 + wm * (C::DW / C::WM) + i * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int m = tile * BM + wn * 64 + j * 16 + (lane & 15);
      if (dd >= d || m >= tc) continue;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = acc[i][j][e];
      Quad<bf16_t>::store(dx + (size_t)(t0 + m) * d + dd, v);
    }
  }
}

// Weight gradients of one chunk: the sparse path's dW tiles with the chunk's
// tokens as the K positions of every neuron block.
constexpr int kDenseDwWaves = 8;  // two waves per SIMD, as the sparse 128-neuron weight gradients

template <int MODE>
__global__ __launch_bounds__(64 * kDenseDwWaves, 1) void dense_dw_kernel(const bf16_t* __restrict__ x,
                                                         const bf16_t* __restrict__ dy, int tokens, int d, int F,
                                                         const int32_t* __restrict__ ptoken, int tc_pad, int np,
                                                         const bf16_t* __restrict__ dg, const bf16_t* __restrict__ du,
                                                         const bf16_t* __restrict__ act, float* __restrict__ fg,
                                                         float* __restrict__ fu, float* __restrict__ fd,
                                                         bf16_t* __restrict__ dwg, bf16_t* __restrict__ dwu,
                                                         bf16_t* __restrict__ dwd) {
  // 256 d per workgroup (two 128-d sub-tiles, two 64 KB stages): the packed
  // dg/du/a rows are read d/256 times; items in the XCD-local order
  using C = Dw2<NB, DENSE_DW_XS, kDenseDwWaves>;
  __shared__ __attribute__((aligned(1024))) char st0_[C::STAGE], st1_[C::STAGE];
  ESG_LDS char* st0 = (ESG_LDS char*)st0_;
  ESG_LDS char* st1 = (ESG_LDS char*)st1_;
  const int nblk = (F + NB - 1) / NB;
  DwWork wk;
  if (!dw_work_xcd(blockIdx.x, 2 * nblk, (d + C::DW - 1) / C::DW, wk)) return;
  const int blk = wk.unit >> 1, db0 = wk.db * C::DW;
  const uint32_t pbytes = (uint32_t)((size_t)nblk * tc_pad * NB * 2);
  const int p0 = blk * tc_pad;
  if ((wk.unit & 1) == 0)
    dw2_body<NB, 0, 2, MODE, DENSE_DW_XS, kDenseDwWaves>(x, tokens, d, F, blk * NB, ptoken, 0, p0, np, 0, fg, fu,
                                                         dg, du, pbytes, dwg, dwu, db0, st0, st1, st1);
  else
    dw2_body<NB, 1, 2, MODE, DENSE_DW_XS, kDenseDwWaves>(dy, tokens, d, F, blk * NB, ptoken, 0, p0, np, 0, fd, fd,
                                                         act, act, pbytes, dwd, dwd, db0, st0, st1, st1);
}

}  // namespace

DenseBwdLayout dense_bwd_layout(int tokens, int d_model, int d_ff) {
  DenseBwdLayout L;
  const int tpad = (tokens + kTileRows - 1) / kTileRows * kTileRows;
  L.tc = tpad < kDenseChunkTokens ? tpad : kDenseChunkTokens;
  if (L.tc == 0) L.tc = kTileRows;
  L.chunks = (tokens + L.tc - 1) / L.tc;
  L.nblk = (d_ff + NB - 1) / NB;
  auto a256 = [](size_t v) { return (v + 255) & ~(size_t)255; };
  const size_t packed = (size_t)L.nblk * L.tc * NB * 2;
  size_t o = 0;
  L.ptoken = o;   o = a256(o + (size_t)L.tc * 4);
  L.dg = o;       o = a256(o + packed);
  L.du = o;       o = a256(o + packed);
  L.act = o;      o = a256(o + packed);
  if (L.chunks > 1) {
    const size_t w32 = (size_t)d_ff * d_model * 4;
    L.fg = o; o = a256(o + w32);
    L.fu = o; o = a256(o + w32);
    L.fd = o; o = a256(o + w32);
  }
  L.bytes = o;
  return L;
}

bool dense_supported(const FfnShape& s) {
  return s.dtype == 1 && s.d_model <= DFwd::MAXDB * 128 && s.k == s.groups() &&
         (unsigned long long)s.tokens * s.d_model * 2 < (1ull << 31) &&
         (unsigned long long)s.d_ff * s.d_model * 2 < (1ull << 31);
}

hipError_t launch_dense_fwd(const FfnShape& s, const void* x, const void* wg, const void* wu, const void* wd, void* y,
                            hipStream_t stream) {
  if (s.tokens == 0) return hipSuccess;
  LaunchTimer timer("dense_fwd", stream);
  hipLaunchKernelGGL(dense_fwd_kernel, dim3((s.tokens + DFwd::TM - 1) / DFwd::TM), dim3(DFwd::NTD), 0, stream,
                     (const bf16_t*)x, (const bf16_t*)wg, (const bf16_t*)wu, (const bf16_t*)wd, s.tokens, s.d_model,
                     s.d_ff, (bf16_t*)y);
  return hipGetLastError();
}

hipError_t launch_dense_bwd(const FfnShape& s, const void* dy, const void* x, const void* wg, const void* wu,
                            const void* wd, void* dx, void* dwg, void* dwu, void* dwd, void* scratch,
                            hipStream_t stream) {
  const DenseBwdLayout L = dense_bwd_layout(s.tokens, s.d_model, s.d_ff);
  char* base = (char*)scratch;
  int32_t* ptoken = (int32_t*)(base + L.ptoken);
  bf16_t* dg = (bf16_t*)(base + L.dg);
  bf16_t* du = (bf16_t*)(base + L.du);
  bf16_t* act = (bf16_t*)(base + L.act);
  float* fg = L.chunks > 1 ? (float*)(base + L.fg) : nullptr;
  float* fu = L.chunks > 1 ? (float*)(base + L.fu) : nullptr;
  float* fd = L.chunks > 1 ? (float*)(base + L.fd) : nullptr;
  const int d = s.d_model, F = s.d_ff;
  for (int c = 0; c < L.chunks; ++c) {
    const int t0 = c * L.tc;
    const int tc = s.tokens - t0 < L.tc ? s.tokens - t0 : L.tc;
    const int tiles = (tc + kTileRows - 1) / kTileRows;
    {
      LaunchTimer timer("dense_route", stream);
      hipLaunchKernelGGL(dense_route_kernel, dim3((L.tc + 255) / 256), dim3(256), 0, stream, t0, tc, L.tc, ptoken);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    {
      LaunchTimer timer("dense_rec", stream);
      hipLaunchKernelGGL(dense_rec_kernel, dim3(tiles, L.nblk), dim3(64 * REC_NW), 0, stream, (const bf16_t*)x,
                         (const bf16_t*)dy, (const bf16_t*)wg, (const bf16_t*)wu, (const bf16_t*)wd, s.tokens, d, F,
                         ptoken, L.tc, dg, du, act);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    {
      LaunchTimer timer("dense_dx", stream);
      hipLaunchKernelGGL(dense_dx_kernel, dim3(tiles, (d + DDx::DW - 1) / DDx::DW), dim3(64 * DDx::NW), 0, stream,
                         (const bf16_t*)wg,
                         (const bf16_t*)wu, d, F, t0, tc, L.tc, dg, du, (bf16_t*)dx);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    {
      LaunchTimer timer("dense_dw", stream);
      const dim3 grid(dw_grid_xcd(2 * L.nblk, (d + 128 * DENSE_DW_XS - 1) / (128 * DENSE_DW_XS)));  // order: dw_work_xcd
      const int mode = L.chunks == 1 ? 0 : (c == 0 ? 1 : (c == L.chunks - 1 ? 3 : 2));
#define ESG_DW(M)                                                                                                  \
  hipLaunchKernelGGL(dense_dw_kernel<M>, grid, dim3(64 * kDenseDwWaves), 0, stream, (const bf16_t*)x,            \
                     (const bf16_t*)dy, s.tokens,                                                                  \
                     d, F, ptoken, L.tc, tiles * kTileRows, dg, du, act, fg, fu, fd, (bf16_t*)dwg, (bf16_t*)dwu,   \
                     (bf16_t*)dwd)
      if (mode == 0)
        ESG_DW(0);
      else if (mode == 1)
        ESG_DW(1);
      else if (mode == 2)
        ESG_DW(2);
      else
        ESG_DW(3);
#undef ESG_DW
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace esg
