// Pipelined bf16 kernels of the sparse SwiGLU layer for group blocks of 64 or
// 128 neurons (eugen_sparse README, "What it does", sparse_swiglu_ffn; the
// math is the one of esg_ffn.hip, which also serves fp32 and narrow groups).
//
// Forward tile (one group sub-block g x 128 padded bucket positions):
//   phase 1  [Hg; Hu]^T = [W_gate rows; W_up rows] . X_tile^T   (K = d)
//            direct-to-LDS pipeline, K-row tiles for both operands;
//            epilogue: a = SiLU(hg)*hu into an LDS tile (the gated activation
//            never leaves the chip), hg and hu saved row-major [pos][gsb]
//   phase 2  P^T = W_down[d-block, group cols] . a^T  (K = group width),
//            double-buffered W_down tiles; per-position partial rows of y
//            written with buffer stores (rows of padding positions land past
//            the buffer and are dropped)
// Backward: dh with the SiLU' epilogue and dx partials in one kernel, weight
// gradients per (group, d-block) in another; see the comments at each.
//
// Orientation: the MFMA M side is the neuron or d index, so each lane's four
// accumulator rows are four consecutive neurons / d values and every epilogue
// store is one 8-byte write.
#include <algorithm>

#include "esg_internal.hpp"
#include "esg_tiles.hpp"

namespace esg {
namespace {

using namespace tiles;

// Partial rows beyond this many bytes per launch are stored nontemporally
// (buffer-store cache policy 2): they do not stay in the 256 MB last-level
// cache until the row sum reads them, and caching them only evicts other data.
// Measured: 100 MB of partial rows faster with cached stores, 168 MB and more
// faster with nontemporal ones.
constexpr unsigned long long kCachedPartialBytes = 128ull << 20;
constexpr int kCpolNontemporal = 2;

// Waves of the forward tile: 64-neuron blocks two 4-wave workgroups per CU,
// 128-neuron blocks one 8-wave workgroup (the loads of the one workgroup are
// issued by eight waves: direct-to-LDS throughput grows with the issuing waves).
template <int GSB>
constexpr int fwd_waves() {
  return GSB >= 128 ? 8 : 4;
}

// 128-d sub-tiles per weight-gradient workgroup: two for 128-neuron blocks
// (one workgroup per CU holds the 256 accumulator registers per wave; the
// packed dg/du/a rows are then read half as often), one for 64-neuron blocks.
template <int GSB>
constexpr int dw_subtiles() {
  return GSB >= 128 ? 2 : 1;
}

// NW: waves (fwd_waves<GSB>(); 8 for 64-neuron blocks when the grid leaves each
// workgroup alone on its CU).
// MODE 0: both phases.  With few tiles the two phases run as two launches, so
// that each spreads over more CUs than there are tiles:
//   MODE 1: phase 1 over the K stages of range blockIdx.z (gridDim.z ranges of
//           equal length), its fp32 [hg; hu] stored position-major
//           [BM][2*GSB] in part_buf[blockIdx.y][tile][blockIdx.z];
//   MODE 2: the kparts K ranges summed in range order, the epilogue (hg, hu
//           saved by range 0 of the d-blocks), then phase 2 over the d-blocks
//           of range blockIdx.z.
// The sum over K ranges rounds differently from one accumulation over all of
// K; every launch of a shape takes the same split, so results stay
// reproducible.
template <int GSB, int CPOL, int NW, int MODE = 0>
__global__ __launch_bounds__(64 * NW, GSB >= 128 || NW == 8 ? 1 : 2) void fwd2_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg, const bf16_t* __restrict__ wu,
    const bf16_t* __restrict__ wd, int tokens, int d, int F, int gs, const int32_t* __restrict__ tile_group,
    const int32_t* __restrict__ ptoken, uint32_t rows_total, bf16_t* __restrict__ hg_saved,
    bf16_t* __restrict__ hu_saved, bf16_t* __restrict__ partials, float* __restrict__ part_buf, int kparts) {
  using C = Fwd2<GSB, NW>;
  constexpr int NS = stages_for<GSB>();
  // with two stages a third W_down buffer follows them
  __shared__ __attribute__((aligned(1024))) char stages_[NS * C::STAGE + (NS == 2 ? C::W2_BYTES : 0)];
  ESG_LDS char* st[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) st[i] = (ESG_LDS char*)stages_ + i * C::STAGE;
  ESG_LDS char* const st0 = st[0];
  ESG_LDS char* const st1 = st[1];

  const int tile = blockIdx.x;
  const int g = tile_group[tile];
  if (g < 0) return;
  const int s = blockIdx.y;
  const int nb0 = g * gs + s * GSB;
  const int lane = threadIdx.x & 63, w = wave_id();
  const uint32_t prow0 = (uint32_t)tile * BM;

  // wave (wm, wn) owns neurons [wm*GSB/WM, +GSB/WM) of gate and up, positions [wn*64, +64)
  const int wm = w % C::WM, wn = w / C::WM;
  int brow[C::FN];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) brow[j] = wn * 64 + j * 16 + (lane & 15);
  // phase-2 output rows (read before phase 1, so the load latency hides behind it)
  using RS = RowStore<DB, C::NTH>;
  const uint32_t psub = (uint32_t)s * rows_total * d * 2;
  uint32_t row_off[RS::IT];
  if constexpr (MODE != 1) {
#pragma unroll
    for (int it = 0; it < RS::IT; ++it) {
      const int r = RS::row(it, threadIdx.x);
      row_off[it] = ptoken[prow0 + r] >= 0 ? psub + (prow0 + r) * (uint32_t)d * 2 : kOOB;
    }
  }
  ESG_LDS char* act = st0;
  const uint32_t sv_bytes = gridDim.y * rows_total * GSB * 2;
  const rsrc_t rsv_g = make_rsrc(hg_saved, sv_bytes);
  const rsrc_t rsv_u = make_rsrc(hu_saved, sv_bytes);
  const uint32_t sub_off = (uint32_t)s * rows_total * GSB * 2;
  constexpr int PART = BM * 2 * GSB;  // floats of one K range's [hg; hu]
  float* const part = MODE == 0 ? nullptr : part_buf + ((size_t)s * gridDim.x + tile) * kFwdSplitK * PART;
  if constexpr (MODE == 2) {
    // ---- K ranges summed, then the epilogue, 4 neurons of one position per step;
    // the ring's first barrier publishes the act tile ----
    for (int i = threadIdx.x; i < BM * GSB / 4; i += C::NTH) {
      const int r = i / (GSB / 4), n = (i % (GSB / 4)) * 4;
      f32x4 g4 = *(const f32x4*)(part + r * 2 * GSB + n);
      f32x4 u4 = *(const f32x4*)(part + r * 2 * GSB + GSB + n);
      for (int z = 1; z < kparts; ++z) {
        g4 += *(const f32x4*)(part + (size_t)z * PART + r * 2 * GSB + n);
        u4 += *(const f32x4*)(part + (size_t)z * PART + r * 2 * GSB + GSB + n);
      }
      float hg[4], hu[4], a[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hg[e] = g4[e];
        hu[e] = u4[e];
        a[e] = hg[e] * sigmoid_f(hg[e]) * hu[e];
      }
      if (hg_saved != nullptr && blockIdx.z == 0) {
        const uint32_t so = sub_off + ((prow0 + r) * GSB + n) * 2;
        store8(rsv_g, so, hg);
        store8(rsv_u, so, hu);
      }
      lds_write8(act + (n >> 6) * BM * 128 + krow_off(r, (n & 63) >> 3) + (n & 7) * 2, pack_bf16x2(a[0], a[1]),
                 pack_bf16x2(a[2], a[3]));
    }
  } else {
  f32x4 acc[2 * C::FMP][C::FN];
  if constexpr (MODE == 1) {
    const int nkt_all = (d + 63) / 64, per = (nkt_all + gridDim.z - 1) / gridDim.z;
    const int kt0 = blockIdx.z * per;
    gateup_tile<GSB, NS, NW>(x, wg, wu, tokens, d, F, nb0, ptoken, prow0, st, acc, kt0, min(per, nkt_all - kt0));
    float* const mine = part + (size_t)blockIdx.z * PART;
#pragma unroll
    for (int p = 0; p < 2 * C::FMP; ++p) {
      const int n = (p < C::FMP ? 0 : GSB) + wm * (GSB / C::WM) + (p % C::FMP) * 16 + (lane >> 4) * 4;
#pragma unroll
      for (int j = 0; j < C::FN; ++j) *(f32x4*)(mine + brow[j] * 2 * GSB + n) = acc[p][j];
    }
    return;
  }
  gateup_tile<GSB, NS, NW>(x, wg, wu, tokens, d, F, nb0, ptoken, prow0, st, acc);
  wait_lgkm0();
  barrier();  // every wave is done with the stages

  // ---- epilogue: hg, hu saved; a = SiLU(hg)*hu -> LDS K-row tile [position][neuron] ----
#pragma unroll
  for (int p = 0; p < C::FMP; ++p) {
    const int n = wm * (GSB / C::WM) + p * 16 + (lane >> 4) * 4;  // 4 consecutive neurons
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int r = brow[j];
      float hg[4], hu[4], a[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hg[e] = acc[p][j][e];
        hu[e] = acc[C::FMP + p][j][e];
        a[e] = hg[e] * sigmoid_f(hg[e]) * hu[e];
      }
      const uint32_t so = sub_off + ((prow0 + r) * GSB + n) * 2;
      if (hg_saved != nullptr) {  // NULL: inference, nothing kept for a backward
        store8(rsv_g, so, hg);
        store8(rsv_u, so, hu);
      }
      lds_write8(act + (n >> 6) * BM * 128 + krow_off(r, (n & 63) >> 3) + (n & 7) * 2, pack_bf16x2(a[0], a[1]),
                 pack_bf16x2(a[2], a[3]));
    }
  }
  }  // MODE 0

  // ---- phase 2: P^T = W_down[d-block, nb0 .. nb0+GSB) . a^T ----
  // d-blocks [blk0, blk0 + nblk): all of them, or range blockIdx.z (MODE 2)
  const int nblk_all = (d + DB - 1) / DB;
  const int per = MODE == 2 ? (nblk_all + gridDim.z - 1) / gridDim.z : nblk_all;
  const int blk0 = MODE == 2 ? blockIdx.z * per : 0;
  const int nblk = min(per, nblk_all - blk0);
  const int c_lane = (lane & 7) ^ (lane >> 3);
  const DmaSrc rd = make_dma_src(wd, (uint32_t)d * F * 2);
  const rsrc_t rp = make_rsrc(partials, gridDim.y * rows_total * (uint32_t)d * 2);
  uint32_t voffW[C::IW2];
#pragma unroll
  for (int i = 0; i < C::IW2; ++i) {
    const int r = (w * C::IW2 + i) * 8 + (lane >> 3);
    voffW[i] = (uint32_t)r * F * 2 + (uint32_t)nb0 * 2 + c_lane * 16;
  }
  auto issueW = [&](ESG_LDS char* st, int blk) __attribute__((always_inline)) {
    const int db0 = (blk0 + blk) * DB;
#pragma unroll
    for (int sb = 0; sb < C::KSUB; ++sb)
#pragma unroll
      for (int i = 0; i < C::IW2; ++i) {
        const int r = (w * C::IW2 + i) * 8 + (lane >> 3);
        const uint32_t off = db0 + r < d ? voffW[i] + (uint32_t)db0 * F * 2 + sb * 128 : kOOB;
        dma16(rd, st + sb * DB * 128 + (w * C::IW2 + i) * 1024, off);
      }
  };
  int arow2[C::FM2], brow2[C::FN2];
#pragma unroll
  for (int i = 0; i < C::FM2; ++i) arow2[i] = wm * (DB / C::WM) + i * 16 + (lane & 15);
#pragma unroll
  for (int j = 0; j < C::FN2; ++j) brow2[j] = wn * 64 + j * 16 + (lane & 15);
  // staging of the output block: stage tails the W_down tiles and the act tile leave free
  ESG_LDS char* out0 = NS == 3 ? st1 + C::W2_BYTES : st0 + C::ACT_BYTES;
  ESG_LDS char* out1 = NS == 3 ? st[NS - 1] + C::W2_BYTES : st1 + C::W2_BYTES;
  auto compute2 = [&](const ESG_LDS char* cur, int blk) __attribute__((always_inline)) {
    f32x4 acc2[C::FM2][C::FN2];
    zero_acc(acc2);
#pragma unroll
    for (int kb = 0; kb < GSB / 32; ++kb) {
      const int sb = kb >> 1, c = (kb & 1) * 4 + (lane >> 4);
      uint4 a[C::FM2], b[C::FN2];
#pragma unroll
      for (int i = 0; i < C::FM2; ++i) a[i] = frag_krow(cur + sb * DB * 128, arow2[i], c);
#pragma unroll
      for (int j = 0; j < C::FN2; ++j) b[j] = frag_krow(act + sb * BM * 128, brow2[j], c);
#pragma unroll
      for (int i = 0; i < C::FM2; ++i)
#pragma unroll
        for (int j = 0; j < C::FN2; ++j) mma_bf16(acc2[i][j], a[i], b[j]);
    }
#pragma unroll
    for (int i = 0; i < C::FM2; ++i)
#pragma unroll
      for (int j = 0; j < C::FN2; ++j) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc2[i][j][e];
        RS::put(out0, out1, brow2[j], wm * (DB / C::WM) + i * 16 + (lane >> 4) * 4, v);
      }
    wait_lgkm0();
    barrier();  // the whole block is staged
    RS::template flush<CPOL>(out0, out1, rp, row_off, (blk0 + blk) * DB, d);
  };
  // the stages after st0 are free (the barrier above); the first step's wait
  // covers the epilogue stores (they precede every W_down load), and its
  // barrier publishes the act tile.  The two W_down buffers: st1 and the last
  // stage (three stages) or the region after st1 (two)
  ESG_LDS char* const wbuf[2] = {st1, NS == 2 ? st1 + C::STAGE : st[NS - 1]};
  kloop_ring<2, C::KSUB * C::IW2, C::STORES2>(nblk, wbuf, issueW, compute2);
}

// ===========================================================================
// Backward dh (+ SiLU' epilogue) and dx partials (see da_tile for phase 1).
// ===========================================================================
template <int GSB, int CPOL>
__global__ __launch_bounds__(64 * fwd_waves<GSB>(), GSB >= 128 ? 1 : 2) void dhdx2_kernel(
    const bf16_t* __restrict__ dy, const bf16_t* __restrict__ wg, const bf16_t* __restrict__ wu,
    const bf16_t* __restrict__ wd, int tokens, int d, int F, int gs, const int32_t* __restrict__ tile_group,
    const int32_t* __restrict__ ptoken, uint32_t rows_total, const bf16_t* __restrict__ hg_saved,
    const bf16_t* __restrict__ hu_saved, bf16_t* __restrict__ dg_out, bf16_t* __restrict__ du_out,
    bf16_t* __restrict__ act_out, bf16_t* __restrict__ partials) {
  constexpr int NW = fwd_waves<GSB>();
  using C = Dh2<GSB, NW>;
  constexpr int NS = stages_for<GSB>();
  // NS stages in one array (with two stages nothing uses st2; no placeholder
  // array, so that two workgroups fit in a compute unit's LDS)
  __shared__ __attribute__((aligned(1024))) char stages_[NS * C::STAGE];
  __shared__ __attribute__((aligned(1024))) char dgu_[C::DGU_BYTES];
  ESG_LDS char* st0 = (ESG_LDS char*)stages_;
  ESG_LDS char* st1 = st0 + C::STAGE;
  ESG_LDS char* st2 = NS == 3 ? st1 + C::STAGE : st0;
  ESG_LDS char* dgu = (ESG_LDS char*)dgu_;

  const int tile = blockIdx.x;
  const int g = tile_group[tile];
  if (g < 0) return;
  const int s = blockIdx.y;
  const int nb0 = g * gs + s * GSB;
  const int lane = threadIdx.x & 63, w = wave_id();
  const uint32_t prow0 = (uint32_t)tile * BM;
  const uint32_t kbytes = (uint32_t)d * 2;

  const int wm = w % C::WM, wn = w / C::WM;
  int brow[C::FN];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) brow[j] = wn * 64 + j * 16 + (lane & 15);
  // the saved pre-activations of the wave's outputs, loaded before phase 1 so
  // that their latency hides behind it (plain loads, older than every DMA)
  const size_t sub_el = (size_t)s * rows_total * GSB;
  uint2 hgq[C::FM][C::FN], huq[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const size_t q = sub_el + (size_t)(prow0 + brow[j]) * GSB + wm * (GSB / C::WM) + i * 16 + (lane >> 4) * 4;
      hgq[i][j] = *(const uint2*)(hg_saved + q);
      huq[i][j] = *(const uint2*)(hu_saved + q);
    }
  f32x4 acc[C::FM][C::FN];
  da_tile<GSB, NS, NW>(dy, wd, tokens, d, F, nb0, ptoken, prow0, st0, st1, st2, acc);

  // ---- epilogue: SiLU' ----
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int n = wm * (GSB / C::WM) + i * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int r = brow[j];
      const size_t q = sub_el + (size_t)(prow0 + r) * GSB + n;
      float hg[4], hu[4], dgv[4], duv[4], av[4];
      unpack_bf16x4(hgq[i][j], hg);
      unpack_bf16x4(huq[i][j], hu);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float da = acc[i][j][e];
        const float sg = sigmoid_f(hg[e]);
        const float silu = hg[e] * sg;
        dgv[e] = da * hu[e] * (sg * (1.0f + hg[e] * (1.0f - sg)));
        duv[e] = da * silu;
        av[e] = silu * hu[e];
      }
      Quad<bf16_t>::store(dg_out + q, dgv);
      Quad<bf16_t>::store(du_out + q, duv);
      Quad<bf16_t>::store(act_out + q, av);
      const int n2 = GSB + n;
      lds_write8(dgu + (n >> 6) * BM * 128 + krow_off(r, (n & 63) >> 3) + (n & 7) * 2, pack_bf16x2(dgv[0], dgv[1]),
                 pack_bf16x2(dgv[2], dgv[3]));
      lds_write8(dgu + (n2 >> 6) * BM * 128 + krow_off(r, (n2 & 63) >> 3) + (n2 & 7) * 2,
                 pack_bf16x2(duv[0], duv[1]), pack_bf16x2(duv[2], duv[3]));
    }
  }

  // ---- phase 2: Q^T = [Wg; Wu]^T[d-block] . [dg du]^T ----
  const DmaSrc rg = make_dma_src(wg, (uint32_t)F * kbytes);
  const DmaSrc ru = make_dma_src(wu, (uint32_t)F * kbytes);
  const rsrc_t rp = make_rsrc(partials, gridDim.y * rows_total * (uint32_t)d * 2);
  const uint32_t psub = (uint32_t)s * rows_total * d * 2;
  uint32_t voffW[C::IW];
  int jW[C::IW];
#pragma unroll
  for (int i = 0; i < C::IW; ++i) {
    const int row = (w * C::IW + i) * 8 + (lane >> 3);  // neuron row of [Wg; Wu]
    const int j = (lane & 7) ^ mn_swz<8>(row);
    const int grow = nb0 + (row < GSB ? row : row - GSB);
    jW[i] = j;
    voffW[i] = (uint32_t)grow * kbytes + j * 16;
  }
  auto issueW = [&](ESG_LDS char* st, int blk) __attribute__((always_inline)) {
    const uint32_t db0 = (uint32_t)blk * C::DB2;
#pragma unroll
    for (int i = 0; i < C::IW; ++i) {
      const bool gate = (w * C::IW + i) * 8 < GSB;  // wave-uniform
      dma16(gate ? rg : ru, st + (w * C::IW + i) * 1024,
            db0 + jW[i] * 8 < (uint32_t)d ? voffW[i] + db0 * 2 : kOOB);
    }
  };
  using RS = RowStore<C::DB2, C::NTH>;
  // phase-2 wave tile: d half wm2 (32 d) x position slice wn2 (PW2 positions)
  const int wm2 = w & 1, wn2 = w >> 1;
  int brow2[C::FN2];
#pragma unroll
  for (int j = 0; j < C::FN2; ++j) brow2[j] = wn2 * C::PW2 + j * 16 + (lane & 15);
  uint32_t row_off[RS::IT];
#pragma unroll
  for (int it = 0; it < RS::IT; ++it) {
    const int r = RS::row(it, threadIdx.x);
    row_off[it] = ptoken[prow0 + r] >= 0 ? psub + (prow0 + r) * (uint32_t)d * 2 : kOOB;
  }
  // staging of the output block: st0 when the weight tiles use st1/st2, else the stage tails
  ESG_LDS char* out0 = NS == 3 ? st0 : st0 + C::W2_BYTES;
  ESG_LDS char* out1 = NS == 3 ? st0 + 64 * RS::RB : st1 + C::W2_BYTES;
  auto compute2 = [&](const ESG_LDS char* cur, int blk) __attribute__((always_inline)) {
    constexpr int KB = 2 * GSB / 32;
    uint4 a[KB][C::FM2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < C::FM2; ++i) a[kb][i] = frag_nrow<8>(cur, kb, wm2 * 32 + i * 16, lane);
    f32x4 acc2[C::FM2][C::FN2];
    zero_acc(acc2);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int c = (kb & 1) * 4 + (lane >> 4);
      uint4 b[C::FN2];
#pragma unroll
      for (int j = 0; j < C::FN2; ++j) b[j] = frag_krow(dgu + (kb >> 1) * BM * 128, brow2[j], c);
#pragma unroll
      for (int i = 0; i < C::FM2; ++i)
#pragma unroll
        for (int j = 0; j < C::FN2; ++j) mma_bf16(acc2[i][j], a[kb][i], b[j]);
    }
#pragma unroll
    for (int i = 0; i < C::FM2; ++i)
#pragma unroll
      for (int j = 0; j < C::FN2; ++j) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc2[i][j][e];
        RS::put(out0, out1, brow2[j], wm2 * 32 + i * 16 + (lane >> 4) * 4, v);
      }
    wait_lgkm0();
    barrier();  // the whole block is staged
    RS::template flush<CPOL>(out0, out1, rp, row_off, blk * C::DB2, d);
  };
  wait_lgkm0();
  barrier();  // all waves are done with the phase-1 stages
  kloop<2, 0, C::STORES2>((d + C::DB2 - 1) / C::DB2, st1, NS == 3 ? st2 : st0, st0, issueW, compute2);
}

// ===========================================================================
// Backward weight gradients (see dw2_body).
// ===========================================================================
template <int GSB>
__global__ __launch_bounds__(NT, GSB >= 128 ? 1 : 2) void dw2_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ dy, int tokens, int d, int F, int gs, int nsub,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ ptoken, uint32_t rows_total,
    const bf16_t* __restrict__ dg, const bf16_t* __restrict__ du, const bf16_t* __restrict__ act,
    bf16_t* __restrict__ dwg, bf16_t* __restrict__ dwu, bf16_t* __restrict__ dwd) {
  constexpr int XS = dw_subtiles<GSB>();
  using C = Dw2<GSB, XS>;
  constexpr int NS = XS == 2 ? 2 : stages_for<GSB>();
  __shared__ __attribute__((aligned(1024))) char stages_[NS * C::STAGE];  // no placeholder for a third stage
  DwWork wk;
  if (!dw_work(blockIdx.x, 2 * (F / gs) * nsub, (d + C::DW - 1) / C::DW, wk)) return;
  const int g = (wk.unit >> 1) / nsub, s = (wk.unit >> 1) % nsub;
  const int db0 = wk.db * C::DW;
  const int nb0 = g * gs + s * GSB;
  const int p0 = tile_off[g] * BM, p1 = tile_off[g + 1] * BM;
  const size_t sub_el = (size_t)s * rows_total * GSB;
  const uint32_t pbytes = (uint32_t)(nsub * rows_total * GSB * 2);
  ESG_LDS char* st0 = (ESG_LDS char*)stages_;
  ESG_LDS char* st1 = st0 + C::STAGE;
  ESG_LDS char* st2 = NS == 3 ? st1 + C::STAGE : st0;
  if ((wk.unit & 1) == 0)
    dw2_body<GSB, 0, NS, 0, XS>(x, tokens, d, F, nb0, ptoken, p0, p0, p1 - p0, sub_el, nullptr, nullptr, dg, du, pbytes,
                         dwg, dwu, db0, st0, st1, st2);
  else
    dw2_body<GSB, 1, NS, 0, XS>(dy, tokens, d, F, nb0, ptoken, p0, p0, p1 - p0, sub_el, nullptr, nullptr, act, act, pbytes,
                         dwd, dwd, db0, st0, st1, st2);
}

// ===========================================================================
// Launchers
// ===========================================================================
bool partials_nontemporal(const FfnShape& s, int ntiles_max) {
  return (unsigned long long)s.nsub() * ntiles_max * BM * s.d_model * 2 > kCachedPartialBytes;
}

template <int GSB>
hipError_t fwd2_t(const FfnShape& s, const void* x, const void* wg, const void* wu, const void* wd,
                  const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, void* hg, void* hu,
                  void* partials, void* act, hipStream_t stream) {
  LaunchTimer timer("fwd_grouped", stream);
  constexpr int NW = fwd_waves<GSB>();
  if constexpr (GSB == 64) {
    if (act != nullptr) {  // fwd_split: phase 1 over K ranges, then phase 2 over d-block ranges
      const int tiles = std::max(1, ntiles_max * s.nsub());
      // ranges of equal length, none empty (the kernels derive the same length)
      auto ranges = [](int n, int want) {
        want = std::max(1, std::min(n, want));
        const int per = (n + want - 1) / want;
        return (n + per - 1) / per;
      };
      const int kz = ranges((s.d_model + 63) / 64, std::min(kFwdSplitK, compute_units() / tiles));  // one per CU
      const int nz = ranges((s.d_model + DB - 1) / DB, 2 * compute_units() / tiles);              // two per CU
      hipLaunchKernelGGL((fwd2_kernel<GSB, 0, 8, 1>), dim3(ntiles_max, s.nsub(), kz), dim3(64 * 8), 0, stream,
                         (const bf16_t*)x, (const bf16_t*)wg, (const bf16_t*)wu, (const bf16_t*)wd, s.tokens,
                         s.d_model, s.d_ff, s.group_size, tile_group, ptoken, (uint32_t)ntiles_max * BM, (bf16_t*)hg,
                         (bf16_t*)hu, (bf16_t*)partials, (float*)act, kz);
      hipLaunchKernelGGL((fwd2_kernel<GSB, 0, NW, 2>), dim3(ntiles_max, s.nsub(), nz), dim3(64 * NW), 0, stream,
                         (const bf16_t*)x, (const bf16_t*)wg, (const bf16_t*)wu, (const bf16_t*)wd, s.tokens,
                         s.d_model, s.d_ff, s.group_size, tile_group, ptoken, (uint32_t)ntiles_max * BM, (bf16_t*)hg,
                         (bf16_t*)hu, (bf16_t*)partials, (float*)act, kz);
      return hipGetLastError();
    }
  }
  // a grid of at most one workgroup per CU: eight waves issue the loads
  const bool alone = NW == 4 && (long long)ntiles_max * s.nsub() <= compute_units();
  auto kern = partials_nontemporal(s, ntiles_max) ? fwd2_kernel<GSB, kCpolNontemporal, NW>
                                                  : (alone ? fwd2_kernel<GSB, 0, 8> : fwd2_kernel<GSB, 0, NW>);
  hipLaunchKernelGGL(kern, dim3(ntiles_max, s.nsub()), dim3(64 * (alone ? 8 : NW)), 0, stream, (const bf16_t*)x,
                     (const bf16_t*)wg, (const bf16_t*)wu, (const bf16_t*)wd, s.tokens, s.d_model, s.d_ff,
                     s.group_size, tile_group, ptoken, (uint32_t)ntiles_max * BM, (bf16_t*)hg, (bf16_t*)hu,
                     (bf16_t*)partials, nullptr, 0);
  return hipGetLastError();
}

template <int GSB>
hipError_t dhdx2_t(const FfnShape& s, const void* dy, const void* wg, const void* wu, const void* wd,
                   const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, const void* hg, const void* hu,
                   void* dg, void* du, void* act, void* partials, hipStream_t stream) {
  LaunchTimer timer("bwd_dh_dx", stream);
  auto kern = partials_nontemporal(s, ntiles_max) ? dhdx2_kernel<GSB, kCpolNontemporal> : dhdx2_kernel<GSB, 0>;
  hipLaunchKernelGGL(kern, dim3(ntiles_max, s.nsub()), dim3(64 * fwd_waves<GSB>()), 0, stream, (const bf16_t*)dy,
                     (const bf16_t*)wg, (const bf16_t*)wu, (const bf16_t*)wd, s.tokens, s.d_model, s.d_ff,
                     s.group_size, tile_group, ptoken, (uint32_t)ntiles_max * BM, (const bf16_t*)hg,
                     (const bf16_t*)hu, (bf16_t*)dg, (bf16_t*)du, (bf16_t*)act, (bf16_t*)partials);
  return hipGetLastError();
}

template <int GSB>
hipError_t dw2_t(const FfnShape& s, const void* x, const void* dy, const int32_t* tile_off, const int32_t* ptoken,
                 int rows_total, const void* dg, const void* du, const void* act, void* dwg, void* dwu, void* dwd,
                 hipStream_t stream) {
  LaunchTimer timer("bwd_dw", stream);
  const dim3 grid(dw_grid(2 * s.groups() * s.nsub(), (s.d_model + 128 * dw_subtiles<GSB>() - 1) /
                                                         (128 * dw_subtiles<GSB>())));  // order: dw_work
  hipLaunchKernelGGL((dw2_kernel<GSB>), grid, dim3(NT), 0, stream, (const bf16_t*)x, (const bf16_t*)dy, s.tokens,
                     s.d_model, s.d_ff, s.group_size, s.nsub(), tile_off, ptoken, (uint32_t)rows_total,
                     (const bf16_t*)dg, (const bf16_t*)du, (const bf16_t*)act, (bf16_t*)dwg, (bf16_t*)dwu,
                     (bf16_t*)dwd);
  return hipGetLastError();
}

}  // namespace

bool bf16_pipelined(const FfnShape& s, int ntiles_max) {
  if (s.dtype != 1 || (s.gsb() != 64 && s.gsb() != 128)) return false;
  const unsigned long long lim = 1ull << 31;
  const unsigned long long rows = (unsigned long long)ntiles_max * BM;
  return (unsigned long long)s.tokens * s.d_model * 2 < lim && (unsigned long long)s.d_ff * s.d_model * 2 < lim &&
         (unsigned long long)s.nsub() * rows * s.d_model * 2 < lim &&
         (unsigned long long)s.nsub() * rows * s.gsb() * 2 < lim;
}

bool fwd_split(const FfnShape& s, int ntiles_max) {
  return bf16_pipelined(s, ntiles_max) && s.gsb() == 64 && (long long)ntiles_max * s.nsub() <= kFwdSplitTiles &&
         !partials_nontemporal(s, ntiles_max);
}

hipError_t launch_fwd2(const FfnShape& s, const void* x, const void* wg, const void* wu, const void* wd,
                       const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, void* hg_saved,
                       void* hu_saved, void* partials, void* act, hipStream_t stream) {
  if (ntiles_max == 0) return hipSuccess;
  if (!fwd_split(s, ntiles_max)) act = nullptr;
  return s.gsb() == 64 ? fwd2_t<64>(s, x, wg, wu, wd, tile_group, ptoken, ntiles_max, hg_saved, hu_saved, partials,
                                    act, stream)
                       : fwd2_t<128>(s, x, wg, wu, wd, tile_group, ptoken, ntiles_max, hg_saved, hu_saved, partials,
                                     act, stream);
}

hipError_t launch_dhdx2(const FfnShape& s, const void* dy, const void* wg, const void* wu, const void* wd,
                        const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, const void* hg_saved,
                        const void* hu_saved, void* dg, void* du, void* act, void* partials, hipStream_t stream) {
  if (ntiles_max == 0) return hipSuccess;
  return s.gsb() == 64 ? dhdx2_t<64>(s, dy, wg, wu, wd, tile_group, ptoken, ntiles_max, hg_saved, hu_saved, dg, du,
                                     act, partials, stream)
                       : dhdx2_t<128>(s, dy, wg, wu, wd, tile_group, ptoken, ntiles_max, hg_saved, hu_saved, dg, du,
                                      act, partials, stream);
}

hipError_t launch_dw2(const FfnShape& s, const void* x, const void* dy, const int32_t* tile_off, const int32_t* ptoken,
                      int rows_total, const void* dg, const void* du, const void* act, void* dwg, void* dwu, void* dwd,
                      hipStream_t stream) {
  return s.gsb() == 64 ? dw2_t<64>(s, x, dy, tile_off, ptoken, rows_total, dg, du, act, dwg, dwu, dwd, stream)
                       : dw2_t<128>(s, x, dy, tile_off, ptoken, rows_total, dg, du, act, dwg, dwu, dwd, stream);
}

}  // namespace esg
