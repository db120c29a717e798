// Pipelined bf16 kernels of the sparse SwiGLU layer for group blocks of 32, 64
// or 128 neurons (eugen_sparse README, "What it does", sparse_swiglu_ffn; the
// math is the one of esg_ffn.hip, which also serves fp32 and 16-neuron groups).
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

// Phase 2 of a forward tile: the partial rows of 128 bucket positions,
// P^T = W_down[d-block, nb0 .. nb0+GSB) . a^T for the d-blocks [blk0, blk0 +
// nblk), K = the group block.  act: the LDS K-row tile a[position][neuron]
// (published by the first step's barrier); wbuf: two W_down buffers; out0 /
// out1: row staging; rp, row_off: the 128 partial rows (kOOB for padding).
// Every outstanding load or store of the caller is waited for at the first
// step.
template <int GSB, int NW, int CPOL>
__device__ __forceinline__ void fwd_down_blocks(const bf16_t* __restrict__ wd, int d, int F, int nb0, int blk0,
                                                int nblk, const ESG_LDS char* act, ESG_LDS char* const (&wbuf)[2],
                                                ESG_LDS char* out0, ESG_LDS char* out1, rsrc_t rp,
                                                const uint32_t (&row_off)[RowStore<DB, 64 * NW>::IT]) {
  using C = Fwd2<GSB, NW>;
  using RS = RowStore<DB, C::NTH>;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int wm = w % C::WM, wn = w / C::WM;
  const int c_lane = (lane & 7) ^ (lane >> 3);
  const DmaSrc rd = make_dma_src(wd, (uint32_t)d * F * 2);
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
  kloop_ring<2, C::KSUB * C::IW2, C::STORES2>(nblk, wbuf, issueW, compute2);
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
// K.  The split is a function of the shape alone (the tile bound and the
// nominal CU count), so every launch of a shape rounds the same way on every
// device; a token's y can still round differently in batches of other sizes,
// whose tile bounds choose another number of ranges (4 up to 64 tiles, then 3,
// 2, and one launch above 128 tiles).
template <int GSB, int CPOL, int NW, int MODE = 0>
__global__ __launch_bounds__(64 * NW, GSB >= 128 || NW == 8 ? 1 : 2) void fwd2_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg, const bf16_t* __restrict__ wu,
    const bf16_t* __restrict__ wd, int tokens, int d, int F, int gs, const int32_t* __restrict__ tile_group,
    const int32_t* __restrict__ ptoken, uint32_t rows_total, bf16_t* __restrict__ hg_saved,
    bf16_t* __restrict__ hu_saved, bf16_t* __restrict__ partials, float* __restrict__ part_buf, int kparts) {
  using C = Fwd2<GSB, NW>;
  constexpr int NS = stages_for<GSB>();
  // Phase 2 keeps the act tile in st0 and puts the W_down buffers and the row
  // staging into the stages (with two stages a second W_down buffer follows
  // them).  32-neuron stages are too small for that: phase 2 then lays act,
  // two W_down buffers and the staging out one after another.
  constexpr int RSB = 64 * RowStore<DB, C::NTH>::RB;  // half of the row staging
  constexpr bool FLAT = GSB < 64;
  constexpr int P1 = NS * C::STAGE + (NS == 2 ? C::W2_BYTES : 0);
  constexpr int P2 = C::ACT_BYTES + 2 * C::W2_BYTES + 2 * RSB;
  static_assert(FLAT || (C::ACT_BYTES + RSB <= C::STAGE && C::W2_BYTES + RSB <= C::STAGE), "stage tails");
  __shared__ __attribute__((aligned(1024))) char stages_[FLAT && P2 > P1 ? P2 : P1];
  ESG_LDS char* st[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) st[i] = (ESG_LDS char*)stages_ + i * C::STAGE;
  ESG_LDS char* const st0 = st[0];
  ESG_LDS char* const st1 = st[1];

  // XCD-local runs of tiles: workgroup L runs on XCD L % 8, which takes the
  // contiguous tiles [x*per, (x+1)*per) (gridDim.x is a multiple of 8)
  const int per_x = gridDim.x / 8;
  const int tile = (int)(blockIdx.x % 8) * per_x + (int)(blockIdx.x / 8);
  if (tile >= (int)(rows_total / BM)) return;
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
  // the tile's own partial rows, addressed from a per-tile buffer base (offsets
  // stay below BM*d*2 bytes however large the whole partial buffer is)
  uint32_t row_off[RS::IT];
  if constexpr (MODE != 1) {
#pragma unroll
    for (int it = 0; it < RS::IT; ++it) {
      const int r = RS::row(it, threadIdx.x);
      row_off[it] = ptoken[prow0 + r] >= 0 ? (uint32_t)r * d * 2 : kOOB;
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
  // hg and hu go out as whole rows, staged from st1 on as [array][128 rows]
  // (the act tile lies in st0); 32-neuron rows (64 bytes) keep the direct
  // 8-byte stores, which measured as fast
  constexpr bool ROWS = GSB >= 64;
  using RE = RowStore<GSB, C::NTH>;
  constexpr int EH = 128 * RE::RB;  // one array (GSB * 256 bytes)
  static_assert(2 * EH <= (FLAT ? (FLAT && P2 > P1 ? P2 : P1) - C::STAGE : (NS - 1) * C::STAGE),
                "hg and hu staging after st0");
  const bool keep = hg_saved != nullptr;  // NULL: inference, nothing kept for a backward
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
      if (keep) {
        if constexpr (ROWS) {
          RE::put(st1, st1 + EH / 2, r, n, hg);
          RE::put(st1 + EH, st1 + EH + EH / 2, r, n, hu);
        } else {
          const uint32_t so = sub_off + ((prow0 + r) * GSB + n) * 2;
          store8(rsv_g, so, hg);
          store8(rsv_u, so, hu);
        }
      }
      lds_write8(act + (n >> 6) * BM * 128 + krow_off(r, (n & 63) >> 3) + (n & 7) * 2, pack_bf16x2(a[0], a[1]),
                 pack_bf16x2(a[2], a[3]));
    }
  }
  if (ROWS && keep) {
    uint32_t roffE[RE::IT];
#pragma unroll
    for (int it = 0; it < RE::IT; ++it) roffE[it] = (uint32_t)RE::row(it, threadIdx.x) * GSB * 2;
    const size_t r0 = (size_t)s * rows_total * GSB + (size_t)prow0 * GSB;
    wait_lgkm0();
    barrier();  // hg and hu staged
    RE::template flush<0>(st1, st1 + EH / 2, make_rsrc(hg_saved + r0, BM * GSB * 2), roffE, 0, GSB);
    RE::template flush<0>(st1 + EH, st1 + EH + EH / 2, make_rsrc(hu_saved + r0, BM * GSB * 2), roffE, 0, GSB);
    wait_lgkm0();
    barrier();  // the staged rows are read before the W_down ring refills st1
  }
  }  // MODE 0

  // ---- phase 2: P^T = W_down[d-block, nb0 .. nb0+GSB) . a^T ----
  // d-blocks [blk0, blk0 + nblk): all of them, or range blockIdx.z (MODE 2)
  const int nblk_all = (d + DB - 1) / DB;
  const int per = MODE == 2 ? (nblk_all + gridDim.z - 1) / gridDim.z : nblk_all;
  const int blk0 = MODE == 2 ? blockIdx.z * per : 0;
  const int nblk = min(per, nblk_all - blk0);
  const rsrc_t rp = make_rsrc(partials + ((size_t)s * rows_total + prow0) * d, (uint32_t)BM * d * 2);
  // staging of the output block: stage tails the W_down tiles and the act tile leave free
  ESG_LDS char* out0 = FLAT ? st0 + C::ACT_BYTES + 2 * C::W2_BYTES
                            : (NS == 3 ? st1 + C::W2_BYTES : st0 + C::ACT_BYTES);
  ESG_LDS char* out1 = FLAT ? out0 + RSB : (NS == 3 ? st[NS - 1] + C::W2_BYTES : st1 + C::W2_BYTES);
  // the stages after st0 are free (the barrier above); the first step's wait
  // covers the epilogue stores (they precede every W_down load), and its
  // barrier publishes the act tile.  The two W_down buffers: st1 and the last
  // stage (three stages) or the region after st1 (two)
  ESG_LDS char* const wbuf[2] = {FLAT ? st0 + C::ACT_BYTES : st1,
                                 FLAT ? st0 + C::ACT_BYTES + C::W2_BYTES : (NS == 2 ? st1 + C::STAGE : st[NS - 1])};
  fwd_down_blocks<GSB, NW, CPOL>(wd, d, F, nb0, blk0, nblk, act, wbuf, out0, out1, rp, row_off);
}

// ===========================================================================
// Forward for 128-neuron blocks on a pair of tiles of one group (256 bucket
// positions; groups are padded to an even number of tiles for it).
// Phase 1 ([Hg; Hu]^T, K = d) runs over all 256 positions, so each staged
// 64-wide K slice of the gate/up rows feeds twice the MFMAs of a 128-position
// tile: a stage is 32 KB of weight rows and 32 KB of x rows for 8.4 MFLOP.
// The weight slices come from L2 (every tile of the group reads them), the x
// rows are gathered from HBM, so the x ring is one stage deeper: two weight
// buffers and three x buffers (160 KB), x slice t+2 and weight slice t+1
// issued while slice t is consumed.
// The epilogue saves hg, hu and keeps a = SiLU(hg)*hu packed in registers;
// phase 2 (partial rows) then runs on the two 128-position halves in turn,
// each half's act tile written into LDS by the four waves that hold it.
// ===========================================================================
template <int CPOL>
__global__ __launch_bounds__(512, 1) void fwd2_pair_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg, const bf16_t* __restrict__ wu,
    const bf16_t* __restrict__ wd, int tokens, int d, int F, int gs, const int32_t* __restrict__ tile_group,
    const int32_t* __restrict__ ptoken, uint32_t rows_total, bf16_t* __restrict__ hg_saved,
    bf16_t* __restrict__ hu_saved, bf16_t* __restrict__ partials) {
  constexpr int GSB = 128, NW = 8, BMT = 2 * BM;
  using C = Fwd2<GSB, NW>;  // phase-1 weight tile and the phase 2 of 128 positions
  using RS = RowStore<DB, C::NTH>;
  constexpr int A_BYTES = C::A_BYTES;  // 256 weight rows x 64 K
  constexpr int B_BYTES = BMT * 128;   // 256 positions x 64 K
  constexpr int IA = C::IA;            // DMA instructions per lane per weight slice
  constexpr int IB = BMT / (8 * NW);   // ... per x slice
  constexpr int FMP = C::FMP, FN = BMT / 2 / 16;  // wave tile: 2*FMP*16 rows x 128 positions
  static_assert(A_BYTES == 32768 && B_BYTES == 32768 && IA == 4 && IB == 4, "pair tile shape");
  // phase 1: weight buffers at 0 and 32 KB, x buffers at 64, 96 and 128 KB;
  // phase 2: act at 0, W_down buffers at 32 and 64 KB, row staging at 96 KB
  __shared__ __attribute__((aligned(1024))) char lds_[2 * A_BYTES + 3 * B_BYTES];
  ESG_LDS char* const base = (ESG_LDS char*)lds_;
  static_assert(C::ACT_BYTES + 2 * C::W2_BYTES + 128 * RS::RB <= 2 * A_BYTES + 3 * B_BYTES, "phase-2 LDS");

  // XCD-local runs of pair tiles: workgroup L runs on XCD L % 8, which takes
  // the contiguous pairs [x*per, (x+1)*per) (gridDim.x is a multiple of 8), so
  // the pairs in flight on an XCD share their group's weights in its L2
  const int npair = (int)(rows_total / (2 * BM));
  const int per = gridDim.x / 8;
  const int pr = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (pr >= npair) return;
  const int tile0 = 2 * pr;
  const int g = tile_group[tile0];
  if (g < 0) return;
  const int s = blockIdx.y;
  const int nb0 = g * gs + s * GSB;
  const int lane = threadIdx.x & 63, w = wave_id();
  const uint32_t prow0 = (uint32_t)tile0 * BM;
  const uint32_t kbytes = (uint32_t)d * 2;

  // partial-row offsets of both halves (loaded now: the latency hides behind phase 1)
  uint32_t row_off[2][RS::IT];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int it = 0; it < RS::IT; ++it) {
      const int r = RS::row(it, threadIdx.x);
      row_off[h][it] = ptoken[prow0 + h * BM + r] >= 0 ? (uint32_t)r * d * 2 : kOOB;
    }

  // ---- phase 1 DMA: lane (row = lane/8 of an 8-row group, slot = lane%8) ----
  const DmaSrc rx = make_dma_src(x, (uint32_t)tokens * kbytes);
  const DmaSrc rg = make_dma_src(wg, (uint32_t)F * kbytes);
  const DmaSrc ru = make_dma_src(wu, (uint32_t)F * kbytes);
  const int c_lane = (lane & 7) ^ (lane >> 3);
  uint32_t voffA[IA], voffB[IB];
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    const int r = (w * IA + i) * 8 + (lane >> 3);
    const int grow = nb0 + (r < GSB ? r : r - GSB);
    voffA[i] = grow < F ? (uint32_t)grow * kbytes + c_lane * 16 : kOOB;
  }
#pragma unroll
  for (int i = 0; i < IB; ++i) {
    const int r = (w * IB + i) * 8 + (lane >> 3);
    const int t = ptoken[prow0 + r];
    voffB[i] = t >= 0 ? (uint32_t)t * kbytes + c_lane * 16 : kOOB;
  }
  auto issueA = [&](int kt) __attribute__((always_inline)) {
    ESG_LDS char* st = base + (kt & 1) * A_BYTES;
    const uint32_t kb = (uint32_t)kt * 128;
    const bool kin = kb + c_lane * 16 < kbytes;
#pragma unroll
    for (int i = 0; i < IA; ++i) {
      const bool gate = (w * IA + i) * 8 < GSB;  // wave-uniform
      dma16(gate ? rg : ru, st + (w * IA + i) * 1024, (kin && voffA[i] != kOOB) ? voffA[i] + kb : kOOB);
    }
  };
  auto issueB = [&](int kt) __attribute__((always_inline)) {
    ESG_LDS char* st = base + 2 * A_BYTES + (kt % 3) * B_BYTES;
    const uint32_t kb = (uint32_t)kt * 128;
    const bool kin = kb + c_lane * 16 < kbytes;
#pragma unroll
    for (int i = 0; i < IB; ++i)
      dma16(rx, st + (w * IB + i) * 1024, (kin && voffB[i] != kOOB) ? voffB[i] + kb : kOOB);
  };

  // wave (wm, wn): gate and up neurons [wm*GSB/WM, +GSB/WM), positions [wn*128, +128)
  const int wm = w % C::WM, wn = w / C::WM;
  int arow[2 * FMP], brow[FN];
#pragma unroll
  for (int p = 0; p < FMP; ++p) {
    arow[p] = wm * (GSB / C::WM) + p * 16 + (lane & 15);
    arow[FMP + p] = GSB + arow[p];
  }
#pragma unroll
  for (int j = 0; j < FN; ++j) brow[j] = wn * BM + j * 16 + (lane & 15);
  f32x4 acc[2 * FMP][FN];
  zero_acc(acc);
  // Issue order: x0, w0, x1, then per step t: w(t+1), x(t+2).  At step t the
  // loads younger than weight slice t are those of x slice t+1 (if any), and
  // x slice t is older than weight slice t, so one vmcnt of IB (or 0) waits
  // for both operands of slice t.  The buffers a step refills were read at
  // step t-1, which the step's barrier closes.
  const int nk = (int)((kbytes + 127) / 128);
  issueB(0);
  issueA(0);
  if (nk > 1) issueB(1);
  for (int t = 0; t < nk; ++t) {
    if (t + 1 < nk) wait_vmcnt<IB>();
    else wait_vmcnt<0>();
    wait_lgkm0();
    barrier();
    if (t + 1 < nk) issueA(t + 1);
    if (t + 2 < nk) issueB(t + 2);
    const ESG_LDS char* sa = base + (t & 1) * A_BYTES;
    const ESG_LDS char* sb = base + 2 * A_BYTES + (t % 3) * B_BYTES;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int c = kb * 4 + (lane >> 4);
      uint4 a[2 * FMP], b[FN];
#pragma unroll
      for (int i = 0; i < 2 * FMP; ++i) a[i] = frag_krow(sa, arow[i], c);
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = frag_krow(sb, brow[j], c);
#pragma unroll
      for (int i = 0; i < 2 * FMP; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma_bf16(acc[i][j], a[i], b[j]);
    }
  }

  // ---- epilogue: hg, hu saved; a = SiLU(hg)*hu kept packed ----
  // hg and hu go out as whole 256-byte rows, staged in the (now idle) phase-1
  // LDS as [array][half][128 rows]
  using RE = RowStore<GSB, C::NTH>;
  constexpr int EH = 128 * RE::RB;  // one half of one array (32 KB)
  static_assert(4 * EH <= 2 * A_BYTES + 3 * B_BYTES, "hg and hu staging");
  const bool keep = hg_saved != nullptr;  // NULL: inference, nothing kept for a backward
  if (keep) {
    wait_lgkm0();
    barrier();  // every wave is done with the phase-1 stages
  }
  uint2 apk[FMP][FN];
#pragma unroll
  for (int p = 0; p < FMP; ++p) {
    const int n = wm * (GSB / C::WM) + p * 16 + (lane >> 4) * 4;  // 4 consecutive neurons
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      float hg[4], hu[4], a[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hg[e] = acc[p][j][e];
        hu[e] = acc[FMP + p][j][e];
        a[e] = hg[e] * sigmoid_f(hg[e]) * hu[e];
      }
      if (keep) {
        const int r = j * 16 + (lane & 15);  // row within the wave's half wn
        RE::put(base + wn * EH, base + wn * EH + EH / 2, r, n, hg);
        RE::put(base + (2 + wn) * EH, base + (2 + wn) * EH + EH / 2, r, n, hu);
      }
      apk[p][j] = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
    }
  }
  if (keep) {
    uint32_t roffE[RE::IT];
#pragma unroll
    for (int it = 0; it < RE::IT; ++it) roffE[it] = (uint32_t)RE::row(it, threadIdx.x) * GSB * 2;
    const size_t sub_el = (size_t)s * rows_total * GSB;
    wait_lgkm0();
    barrier();  // hg and hu staged
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const size_t r0 = sub_el + (size_t)(prow0 + h * BM) * GSB;
      RE::template flush<0>(base + h * EH, base + h * EH + EH / 2, make_rsrc(hg_saved + r0, BM * GSB * 2), roffE,
                            0, GSB);
      RE::template flush<0>(base + (2 + h) * EH, base + (2 + h) * EH + EH / 2,
                            make_rsrc(hu_saved + r0, BM * GSB * 2), roffE, 0, GSB);
    }
  }

  // ---- phase 2 per half: P^T = W_down[d-block, nb0 .. nb0+GSB) . a^T ----
  ESG_LDS char* const act = base;
  ESG_LDS char* wbuf[2];  // (not a const array: its initializer would become a global)
  wbuf[0] = base + C::ACT_BYTES;
  wbuf[1] = base + C::ACT_BYTES + C::W2_BYTES;
  ESG_LDS char* const out0 = base + C::ACT_BYTES + 2 * C::W2_BYTES;
  ESG_LDS char* const out1 = out0 + 64 * RS::RB;
  const int nblk = (d + DB - 1) / DB;
  for (int h = 0; h < 2; ++h) {
    wait_lgkm0();
    barrier();  // phase 1 (or the previous half's phase 2) is done with these bytes
    if (wn == h) {
#pragma unroll
      for (int p = 0; p < FMP; ++p) {
        const int n = wm * (GSB / C::WM) + p * 16 + (lane >> 4) * 4;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = j * 16 + (lane & 15);
          lds_write8(act + (n >> 6) * BM * 128 + krow_off(r, (n & 63) >> 3) + (n & 7) * 2, apk[p][j].x,
                     apk[p][j].y);
        }
      }
    }
    const rsrc_t rp = make_rsrc(partials + ((size_t)s * rows_total + prow0 + h * BM) * d, (uint32_t)BM * d * 2);
    fwd_down_blocks<GSB, NW, CPOL>(wd, d, F, nb0, 0, nblk, act, wbuf, out0, out1, rp, row_off[h]);
  }
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

  // XCD-local runs of tiles: workgroup L runs on XCD L % 8, which takes the
  // contiguous tiles [x*per, (x+1)*per) (gridDim.x is a multiple of 8)
  const int per_x = gridDim.x / 8;
  const int tile = (int)(blockIdx.x % 8) * per_x + (int)(blockIdx.x / 8);
  if (tile >= (int)(rows_total / BM)) return;
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
  // dg and du go to the LDS K-row tile phase 2 reads, a to a row staging in
  // st0; all three then go out as whole rows (32-neuron rows, 64 bytes, keep
  // the direct 8-byte stores, which measured as fast)
  constexpr bool ROWS = GSB >= 64;
  using RE = RowStore<GSB, C::NTH>;
  constexpr int EH = 128 * RE::RB;  // the a rows (GSB * 256 bytes)
  static_assert(EH <= C::STAGE, "a staging in st0");
  if constexpr (ROWS) {
    wait_lgkm0();
    barrier();  // every wave is done with the phase-1 stages
  }
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int n = wm * (GSB / C::WM) + i * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int r = brow[j];
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
      if constexpr (ROWS) {
        RE::put(st0, st0 + EH / 2, r, n, av);
      } else {
        const size_t q = sub_el + (size_t)(prow0 + r) * GSB + n;
        Quad<bf16_t>::store(dg_out + q, dgv);
        Quad<bf16_t>::store(du_out + q, duv);
        Quad<bf16_t>::store(act_out + q, av);
      }
      const int n2 = GSB + n;
      lds_write8(dgu + (n >> 6) * BM * 128 + krow_off(r, (n & 63) >> 3) + (n & 7) * 2, pack_bf16x2(dgv[0], dgv[1]),
                 pack_bf16x2(dgv[2], dgv[3]));
      lds_write8(dgu + (n2 >> 6) * BM * 128 + krow_off(r, (n2 & 63) >> 3) + (n2 & 7) * 2,
                 pack_bf16x2(duv[0], duv[1]), pack_bf16x2(duv[2], duv[3]));
    }
  }

  if constexpr (ROWS) {
    wait_lgkm0();
    barrier();  // dg, du and a staged
    // dg, du rows from the K-row tile: chunk c (8 neurons) of row r of an
    // array sits in sub-tile (c0 + c) / 8 at chunk (c0 + c) % 8, c0 = 0 (dg)
    // or GSB / 8 (du); lanes take consecutive chunks, so each store
    // instruction writes whole rows
    constexpr int CPR = GSB / 8;  // 16-byte chunks per row
    const size_t r0 = sub_el + (size_t)prow0 * GSB;
    const rsrc_t rdg = make_rsrc(dg_out + r0, BM * GSB * 2), rdu = make_rsrc(du_out + r0, BM * GSB * 2);
    for (int qq = threadIdx.x; qq < BM * CPR; qq += C::NTH) {
      const int r = qq / CPR, c = qq % CPR, cu = CPR + c;
      const u32x4_t vg = *(const ESG_LDS u32x4_t*)(dgu + (c >> 3) * BM * 128 + krow_off(r, c & 7));
      const u32x4_t vu = *(const ESG_LDS u32x4_t*)(dgu + (cu >> 3) * BM * 128 + krow_off(r, cu & 7));
      const uint32_t o = (uint32_t)r * GSB * 2 + c * 16;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i32, vg), rdg, o, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i32, vu), rdu, o, 0, 0);
    }
    uint32_t roffE[RE::IT];
#pragma unroll
    for (int it = 0; it < RE::IT; ++it) roffE[it] = (uint32_t)RE::row(it, threadIdx.x) * GSB * 2;
    RE::template flush<0>(st0, st0 + EH / 2, make_rsrc(act_out + r0, BM * GSB * 2), roffE, 0, GSB);
    wait_lgkm0();
    barrier();  // the a rows are read before phase 2 refills the stages
  }

  // ---- phase 2: Q^T = [Wg; Wu]^T[d-block] . [dg du]^T ----
  const DmaSrc rg = make_dma_src(wg, (uint32_t)F * kbytes);
  const DmaSrc ru = make_dma_src(wu, (uint32_t)F * kbytes);
  // the tile's own partial rows from a per-tile buffer base (see the forward)
  const rsrc_t rp = make_rsrc(partials + ((size_t)s * rows_total + prow0) * d, (uint32_t)BM * d * 2);
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
    row_off[it] = ptoken[prow0 + r] >= 0 ? (uint32_t)r * d * 2 : kOOB;
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
// Backward dh + dx for 128-neuron blocks on a pair of tiles of one group (256
// bucket positions; groups are padded to an even number of tiles for it).
// Wave w owns positions [32w, 32w+32) with all 128 neurons.
// Phase 1 (dA^T = W_down[:, block]^T . dY^T, K = d) runs over all 256
// positions, so each staged 64-row slice of W_down feeds twice the MFMAs of a
// 128-position tile.  The epilogue stores dg, du, a and keeps dg, du packed in
// registers, as accumulator fragments: lane l holds four consecutive neurons
// 16i + 4(l/16) .. of position 16j + l%16 of its wave's slice.
// Phase 2 (dx partials, Q^T = [W_g; W_u]^T[d-block] . [dg du]^T, K = 256)
// takes those registers as the B operand: a K step of 32 neurons pairs two
// stacked fragments, and the weight tile is read in the same neuron order
// (frag_nrow_acc8).  So [dg du] never goes through LDS, and one staged weight
// d-block serves all 256 positions (a quarter of the LDS the weights and the
// [dg du] tile took per 128 positions before): three 32 KB weight buffers
// and 32 KB of row staging for the two halves' partial rows.
// ===========================================================================
template <int CPOL>
__global__ __launch_bounds__(512, 1) void dhdx2_pair_kernel(
    const bf16_t* __restrict__ dy, const bf16_t* __restrict__ wg, const bf16_t* __restrict__ wu,
    const bf16_t* __restrict__ wd, int tokens, int d, int F, int gs, const int32_t* __restrict__ tile_group,
    const int32_t* __restrict__ ptoken, uint32_t rows_total, const bf16_t* __restrict__ hg_saved,
    const bf16_t* __restrict__ hu_saved, bf16_t* __restrict__ dg_out, bf16_t* __restrict__ du_out,
    bf16_t* __restrict__ act_out, bf16_t* __restrict__ partials) {
  constexpr int GSB = 128, NW = 8, BMT = 2 * BM;
  using C = Dh2<GSB, NW, BMT>;
  using WV = DaWave<GSB, NW, BMT, 1>;
  constexpr int FM = WV::FM, FN = WV::FN;  // 8 neuron fragments x 2 position fragments
  constexpr int NS = 3;
  constexpr int DB2 = 64;                  // d per phase-2 step
  constexpr int W2 = 2 * GSB * DB2 * 2;    // N-row: 256 neuron rows x 64 d
  constexpr int IW = 2 * GSB / (8 * NW);   // weight DMA instructions per lane per step
  constexpr int NWB = 3;                   // weight buffers
  using RS = RowStore<DB2, 64 * NW>;
  constexpr int LDS1 = NS * C::STAGE1;
  constexpr int LDS2 = NWB * W2 + 2 * 128 * RS::RB;
  static_assert(FM == 8 && FN == 2 && IW == 4 && W2 == 32768 && LDS2 <= LDS1, "pair tile shape");
  __shared__ __attribute__((aligned(1024))) char lds_[LDS1];
  ESG_LDS char* const base = (ESG_LDS char*)lds_;

  // XCD-local runs of pair tiles: workgroup L runs on XCD L % 8, which takes
  // the contiguous pairs [x*per, (x+1)*per) (gridDim.x is a multiple of 8), so
  // the pairs in flight on an XCD share their group's weights in its L2
  const int npair = (int)(rows_total / (2 * BM));
  const int per = gridDim.x / 8;
  const int pr = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (pr >= npair) return;
  const int tile0 = 2 * pr;
  const int g = tile_group[tile0];
  if (g < 0) return;
  const int s = blockIdx.y;
  const int nb0 = g * gs + s * GSB;
  const int lane = threadIdx.x & 63, w = wave_id();
  const uint32_t prow0 = (uint32_t)tile0 * BM;
  const uint32_t kbytes = (uint32_t)d * 2;
  const int p0 = WV::pos0(w);  // the wave's first position in the pair

  // partial-row offsets of both halves, and the saved hg, hu of the wave's
  // positions (loaded now: the latency hides behind phase 1)
  uint32_t row_off[2][RS::IT];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int it = 0; it < RS::IT; ++it) {
      const int r = RS::row(it, threadIdx.x);
      row_off[h][it] = ptoken[prow0 + h * BM + r] >= 0 ? (uint32_t)r * d * 2 : kOOB;
    }
  const size_t sub_el = (size_t)s * rows_total * GSB;
  uint2 hgq[FM][FN], huq[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const size_t q = sub_el + (size_t)(prow0 + p0 + j * 16 + (lane & 15)) * GSB + i * 16 + (lane >> 4) * 4;
      hgq[i][j] = *(const uint2*)(hg_saved + q);
      huq[i][j] = *(const uint2*)(hu_saved + q);
    }
  f32x4 acc[FM][FN];
  da_tile<GSB, NS, NW, BMT, 1>(dy, wd, tokens, d, F, nb0, ptoken, prow0, base, base + C::STAGE1,
                               base + 2 * C::STAGE1, acc);

  // ---- epilogue: SiLU'; dg, du kept packed as accumulator fragments ----
  // dg, du and a go out as whole 256-byte rows: staged in the (now idle)
  // phase-1 LDS as [array][half][128 rows], dg and du first, then a.
  using RE = RowStore<GSB, 64 * NW>;
  constexpr int EH = 128 * RE::RB;  // one half of one array (32 KB)
  static_assert(4 * EH <= LDS1, "dg and du staging");
  wait_lgkm0();
  barrier();  // every wave is done with the phase-1 stages
  const int eh = p0 / BM;  // the half the wave's positions lie in
  uint2 dgp[FM][FN], dup[FM][FN], apk[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int n = i * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
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
      const int r = (p0 % BM) + j * 16 + (lane & 15);
      RE::put(base + eh * EH, base + eh * EH + EH / 2, r, n, dgv);
      RE::put(base + (2 + eh) * EH, base + (2 + eh) * EH + EH / 2, r, n, duv);
      dgp[i][j] = make_uint2(pack_bf16x2(dgv[0], dgv[1]), pack_bf16x2(dgv[2], dgv[3]));
      dup[i][j] = make_uint2(pack_bf16x2(duv[0], duv[1]), pack_bf16x2(duv[2], duv[3]));
      apk[i][j] = make_uint2(pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3]));
    }
  }
  uint32_t roffE[RE::IT];
#pragma unroll
  for (int it = 0; it < RE::IT; ++it) roffE[it] = (uint32_t)RE::row(it, threadIdx.x) * GSB * 2;
  auto rsE = [&](bf16_t* arr, int h) __attribute__((always_inline)) {
    return make_rsrc(arr + sub_el + (size_t)(prow0 + h * BM) * GSB, (uint32_t)BM * GSB * 2);
  };
  wait_lgkm0();
  barrier();  // dg and du staged
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    RE::template flush<0>(base + h * EH, base + h * EH + EH / 2, rsE(dg_out, h), roffE, 0, GSB);
    RE::template flush<0>(base + (2 + h) * EH, base + (2 + h) * EH + EH / 2, rsE(du_out, h), roffE, 0, GSB);
  }
  wait_lgkm0();
  barrier();  // their rows are read: stage a
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = (p0 % BM) + j * 16 + (lane & 15);
      float av[4];
      unpack_bf16x4(apk[i][j], av);
      RE::put(base + eh * EH, base + eh * EH + EH / 2, r, i * 16 + (lane >> 4) * 4, av);
    }
  wait_lgkm0();
  barrier();
#pragma unroll
  for (int h = 0; h < 2; ++h)
    RE::template flush<0>(base + h * EH, base + h * EH + EH / 2, rsE(act_out, h), roffE, 0, GSB);

  // ---- phase 2: Q^T = [Wg; Wu]^T[d-block] . [dg du]^T over all 256 positions ----
  // LDS: NWB weight buffers, then the row staging of half 0 and of half 1
  ESG_LDS char* wbuf[NWB];  // (not a const array: its initializer would become a global)
#pragma unroll
  for (int i = 0; i < NWB; ++i) wbuf[i] = base + i * W2;
  ESG_LDS char* const stg = base + NWB * W2;  // half h: rows 0..63 at stg + h*128*RB, 64..127 after
  const int h = p0 / BM;                      // the half the wave's positions lie in (wave-uniform)
  ESG_LDS char* const out0 = stg + h * 128 * RS::RB;
  ESG_LDS char* const out1 = out0 + 64 * RS::RB;
  const rsrc_t rp0 = make_rsrc(partials + ((size_t)s * rows_total + prow0) * d, (uint32_t)BM * d * 2);
  const rsrc_t rp1 = make_rsrc(partials + ((size_t)s * rows_total + prow0 + BM) * d, (uint32_t)BM * d * 2);
  const DmaSrc rg = make_dma_src(wg, (uint32_t)F * kbytes);
  const DmaSrc ru = make_dma_src(wu, (uint32_t)F * kbytes);
  uint32_t voffW[IW];
  int jW[IW];
#pragma unroll
  for (int i = 0; i < IW; ++i) {
    const int row = (w * IW + i) * 8 + (lane >> 3);  // neuron row of [Wg; Wu]
    const int j = (lane & 7) ^ swz_acc8(row);  // the phase-2 tile's swizzle (frag_nrow_acc8)
    const int grow = nb0 + (row < GSB ? row : row - GSB);
    jW[i] = j;
    voffW[i] = (uint32_t)grow * kbytes + j * 16;
  }
  auto issueW = [&](ESG_LDS char* st, int blk) __attribute__((always_inline)) {
    const uint32_t db0 = (uint32_t)blk * DB2;
#pragma unroll
    for (int i = 0; i < IW; ++i) {
      const bool gate = (w * IW + i) * 8 < GSB;  // wave-uniform
      dma16(gate ? rg : ru, st + (w * IW + i) * 1024,
            db0 + jW[i] * 8 < (uint32_t)d ? voffW[i] + db0 * 2 : kOOB);
    }
  };
  auto compute2 = [&](const ESG_LDS char* cur, int blk) __attribute__((always_inline)) {
    constexpr int FMD = DB2 / 16;  // d fragments
    f32x4 acc2[FMD][FN];
    zero_acc(acc2);
#pragma unroll
    for (int kb = 0; kb < 2 * GSB / 32; ++kb) {
      // K step kb: neurons 32*kb .. of [dg du] (gate rows first), i.e. the
      // stacked fragments 2*(kb%4) and 2*(kb%4)+1 of dg (kb < 4) or du
      const int i0 = 2 * (kb % 4);
      uint4 b[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint2 lo = kb < 4 ? dgp[i0][j] : dup[i0][j];
        const uint2 hi = kb < 4 ? dgp[i0 + 1][j] : dup[i0 + 1][j];
        b[j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
      uint4 a[FMD];
#pragma unroll
      for (int m = 0; m < FMD; ++m) a[m] = frag_nrow_acc8(cur, kb, m * 16, lane);
#pragma unroll
      for (int m = 0; m < FMD; ++m)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma_bf16(acc2[m][j], a[m], b[j]);
    }
#pragma unroll
    for (int m = 0; m < FMD; ++m)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc2[m][j][e];
        RS::put(out0, out1, (p0 % BM) + j * 16 + (lane & 15), m * 16 + (lane >> 4) * 4, v);
      }
    wait_lgkm0();
    barrier();  // both halves' blocks are staged
    RS::template flush<CPOL>(stg, stg + 64 * RS::RB, rp0, row_off[0], blk * DB2, d);
    RS::template flush<CPOL>(stg + 128 * RS::RB, stg + 192 * RS::RB, rp1, row_off[1], blk * DB2, d);
  };
  wait_lgkm0();
  barrier();  // every wave is done with the phase-1 stages
  kloop_ring<NWB, IW, 2 * RS::IT>((d + DB2 - 1) / DB2, wbuf, issueW, compute2);
}

// ===========================================================================
// Backward weight gradients (see dw2_body).
// ===========================================================================
// Waves of the weight-gradient workgroup: eight for 128-neuron blocks (one
// workgroup per CU: two waves per SIMD, each holding an eighth of the output),
// four for narrower blocks (two workgroups per CU).
template <int GSB>
constexpr int dw_waves() {
  return GSB >= 128 ? 8 : 4;
}

template <int GSB>
__global__ __launch_bounds__(64 * dw_waves<GSB>(), GSB >= 128 ? 1 : 2) void dw2_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ dy, int tokens, int d, int F, int gs, int nsub,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ ptoken, uint32_t rows_total,
    const bf16_t* __restrict__ dg, const bf16_t* __restrict__ du, const bf16_t* __restrict__ act,
    bf16_t* __restrict__ dwg, bf16_t* __restrict__ dwu, bf16_t* __restrict__ dwd, int cht,
    float* __restrict__ slots) {
  constexpr int XS = dw_subtiles<GSB>();
  constexpr int NWD = dw_waves<GSB>();
  using C = Dw2<GSB, XS, NWD>;
  constexpr int NS = XS == 2 ? 2 : stages_for<GSB>();
  __shared__ __attribute__((aligned(1024))) char stages_[NS * C::STAGE];  // no placeholder for a third stage
  const int G = F / gs, units = 2 * G * nsub, ndb = (d + C::DW - 1) / C::DW;
  // eight waves: the chunked plan of dw_plan_xcd (with cht = 0 one item per
  // (unit, d-block)); four waves: dw_work
  DwItem it;
  if constexpr (NWD == 8) {
    if (!dw_plan_xcd(blockIdx.x, tile_off, G, 2 * nsub, ndb, cht, it)) return;
  } else {
    DwWork wk;
    if (!dw_work(blockIdx.x, units, ndb, wk)) return;
    const int g = (wk.unit >> 1) / nsub;
    it = DwItem{wk.unit, wk.db, tile_off[g], tile_off[g + 1] - tile_off[g], -1};
  }
  const int g = (it.unit >> 1) / nsub, s = (it.unit >> 1) % nsub;
  const int db0 = it.db * C::DW;
  const int nb0 = g * gs + s * GSB;
  const int p0 = it.t0 * BM, np = it.nt * BM;
  const size_t sub_el = (size_t)s * rows_total * GSB;
  const uint32_t pbytes = (uint32_t)(nsub * rows_total * GSB * 2);
  ESG_LDS char* st0 = (ESG_LDS char*)stages_;
  ESG_LDS char* st1 = st0 + C::STAGE;
  ESG_LDS char* st2 = NS == 3 ? st1 + C::STAGE : st0;
  if constexpr (NWD == 8) {
    if (it.slot >= 0) {  // a chunk of a split group: fp32 sums into its slot ([nsub][gate, up, down] blocks)
      float* sb = slots + (size_t)it.slot * 3 * gs * d + (size_t)s * 3 * GSB * d;
      if ((it.unit & 1) == 0)
        dw2_body<GSB, 0, NS, 4, XS, NWD>(x, tokens, d, F, nb0, ptoken, p0, p0, np, sub_el, sb,
                                         sb + (size_t)GSB * d, dg, du, pbytes, dwg, dwu, db0, st0, st1, st2);
      else
        dw2_body<GSB, 1, NS, 4, XS, NWD>(dy, tokens, d, F, nb0, ptoken, p0, p0, np, sub_el,
                                         sb + (size_t)2 * GSB * d, nullptr, act, act, pbytes, dwd, dwd, db0, st0,
                                         st1, st2);
      return;
    }
  }
  if ((it.unit & 1) == 0)
    dw2_body<GSB, 0, NS, 0, XS, NWD>(x, tokens, d, F, nb0, ptoken, p0, p0, np, sub_el, nullptr, nullptr, dg, du,
                                     pbytes, dwg, dwu, db0, st0, st1, st2);
  else
    dw2_body<GSB, 1, NS, 0, XS, NWD>(dy, tokens, d, F, nb0, ptoken, p0, p0, np, sub_el, nullptr, nullptr, act, act,
                                     pbytes, dwd, dwd, db0, st0, st1, st2);
}

// The slot sums of split groups (see dw_plan_xcd): workgroup (x, y) takes
// elements [x*E, (x+1)*E), E = 256 threads x 4 x kDwSumIt, of the split
// groups y, y + gridDim.y, ... (in group order), adds each one's c slots in
// chunk order in fp32 and stores bf16 like the one-item groups.  A slot holds,
// per 128-neuron sub-block, [gate: GSB][d], [up: GSB][d] and [down: d][GSB].
constexpr int kDwSumIt = 8;
__global__ __launch_bounds__(256) void dw_slot_sum_kernel(const int32_t* __restrict__ tile_off, int G, int cht,
                                                          int gs, int d, int F, const float* __restrict__ slots,
                                                          bf16_t* __restrict__ dwg, bf16_t* __restrict__ dwu,
                                                          bf16_t* __restrict__ dwd) {
  constexpr int GSB = 128;
  const int lane = threadIdx.x & 63;
  const size_t per_slot = (size_t)3 * gs * d;
  const size_t blk = (size_t)3 * GSB * d;
  const size_t e0 = (size_t)blockIdx.x * kDwSumIt * 1024 + threadIdx.x * 4;
  for (int j = blockIdx.y;; j += gridDim.y) {
    // the j-th group with more than one chunk: g, its chunk count c, first slot ps
    int seen = 0, g = -1, c = 0, ps = 0, sc = 0;
    for (int g0 = 0; g0 < G && g < 0; g0 += 64) {
      const int gg = g0 + lane;
      const int cc = gg < G ? dw_chunks(tile_off, gg, cht) : 1;
      const uint64_t split = __ballot(cc >= 2);
      const int inc = wave_incl_scan(cc >= 2 ? cc : 0) + sc;
      const int n = __popcll(split);
      if (j < seen + n) {
        uint64_t m = split;
        for (int i = 0; i < j - seen; ++i) m &= m - 1;  // drop the lower split groups
        const int src = __builtin_ctzll(m);
        g = g0 + src;
        c = __builtin_amdgcn_readfirstlane(__shfl(cc, src));
        ps = __builtin_amdgcn_readfirstlane(__shfl(inc, src)) - c;
      }
      seen += n;
      sc = __builtin_amdgcn_readfirstlane(__shfl(inc, 63));
    }
    if (g < 0) return;
    float v[kDwSumIt][4];
#pragma unroll
    for (int u = 0; u < kDwSumIt; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) v[u][i] = 0.0f;
    for (int q = 0; q < c; ++q) {  // chunk order
      const float* src = slots + (size_t)(ps + q) * per_slot;
#pragma unroll
      for (int u = 0; u < kDwSumIt; ++u) {
        const size_t e = e0 + (size_t)u * 1024;
        if (e < per_slot) {
          float o[4];
          Quad<float>::load(src + e, o);
#pragma unroll
          for (int i = 0; i < 4; ++i) v[u][i] += o[i];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kDwSumIt; ++u) {
      const size_t e = e0 + (size_t)u * 1024;
      if (e >= per_slot) break;
      const int sb = (int)(e / blk);
      const size_t r = e % blk;
      const int part = (int)(r / ((size_t)GSB * d));
      const int w = (int)(r % ((size_t)GSB * d));
      const int nb0 = g * gs + sb * GSB;
      if (part < 2) {
        const int n = w / d, dd = w % d;
        Quad<bf16_t>::store((part == 0 ? dwg : dwu) + (size_t)(nb0 + n) * d + dd, v[u]);
      } else {
        const int dd = w / GSB, n = w % GSB;
        Quad<bf16_t>::store(dwd + (size_t)dd * F + nb0 + n, v[u]);
      }
    }
  }
}

// ===========================================================================
// Launchers
// ===========================================================================
bool partials_nontemporal(const FfnShape& s, int ntiles_max) {
  return (unsigned long long)s.nsub() * ntiles_max * BM * s.d_model * 2 > kCachedPartialBytes;
}

// The split forward's range counts come from the shape and the fixed nominal
// compute-unit count kNominalCUs, not from the device, so a shape rounds the
// same way on every device and partition mode.
template <int GSB>
hipError_t fwd2_t(const FfnShape& s, const void* x, const void* wg, const void* wu, const void* wd,
                  const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, int pad, void* hg, void* hu,
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
      const int kz = ranges((s.d_model + 63) / 64, std::min(kFwdSplitK, kNominalCUs / tiles));  // one per CU
      const int nz = ranges((s.d_model + DB - 1) / DB, 2 * kNominalCUs / tiles);              // two per CU
      const unsigned gx = (ntiles_max + 7) / 8 * 8;  // a multiple of 8 (the tile order is XCD-local)
      hipLaunchKernelGGL((fwd2_kernel<GSB, 0, 8, 1>), dim3(gx, s.nsub(), kz), dim3(64 * 8), 0, stream,
                         (const bf16_t*)x, (const bf16_t*)wg, (const bf16_t*)wu, (const bf16_t*)wd, s.tokens,
                         s.d_model, s.d_ff, s.group_size, tile_group, ptoken, (uint32_t)ntiles_max * BM, (bf16_t*)hg,
                         (bf16_t*)hu, (bf16_t*)partials, (float*)act, kz);
      hipLaunchKernelGGL((fwd2_kernel<GSB, 0, NW, 2>), dim3(gx, s.nsub(), nz), dim3(64 * NW), 0, stream,
                         (const bf16_t*)x, (const bf16_t*)wg, (const bf16_t*)wu, (const bf16_t*)wd, s.tokens,
                         s.d_model, s.d_ff, s.group_size, tile_group, ptoken, (uint32_t)ntiles_max * BM, (bf16_t*)hg,
                         (bf16_t*)hu, (bf16_t*)partials, (float*)act, kz);
      return hipGetLastError();
    }
  }
  if constexpr (GSB == 128) {
    if (pad == 2 * BM) {  // pairs of tiles of one group (the bucketing padded groups to pairs)
      auto kp = partials_nontemporal(s, ntiles_max) ? fwd2_pair_kernel<kCpolNontemporal> : fwd2_pair_kernel<0>;
      hipLaunchKernelGGL(kp, dim3((ntiles_max / 2 + 7) / 8 * 8, s.nsub()), dim3(512), 0, stream, (const bf16_t*)x,
                         (const bf16_t*)wg, (const bf16_t*)wu, (const bf16_t*)wd, s.tokens, s.d_model, s.d_ff,
                         s.group_size, tile_group, ptoken, (uint32_t)ntiles_max * BM, (bf16_t*)hg, (bf16_t*)hu,
                         (bf16_t*)partials);
      return hipGetLastError();
    }
  }
  auto kern = partials_nontemporal(s, ntiles_max) ? fwd2_kernel<GSB, kCpolNontemporal, NW> : fwd2_kernel<GSB, 0, NW>;
  int waves = NW;
  if constexpr (NW == 4 && GSB >= 64) {
    // a grid of at most one workgroup per CU (cached partial rows): eight waves issue the loads
    if ((long long)ntiles_max * s.nsub() <= kNominalCUs && !partials_nontemporal(s, ntiles_max)) {
      kern = fwd2_kernel<GSB, 0, 8>;
      waves = 8;
    }
  }
  const unsigned gx = (ntiles_max + 7) / 8 * 8;  // a multiple of 8 (the tile order is XCD-local)
  hipLaunchKernelGGL(kern, dim3(gx, s.nsub()), dim3(64 * waves), 0, stream, (const bf16_t*)x,
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
  if constexpr (GSB == 128) {
    if (tile_pad(s) == 2 * BM) {  // pairs of tiles of one group (the bucketing padded groups to pairs)
      auto kp = partials_nontemporal(s, ntiles_max) ? dhdx2_pair_kernel<kCpolNontemporal> : dhdx2_pair_kernel<0>;
      hipLaunchKernelGGL(kp, dim3((ntiles_max / 2 + 7) / 8 * 8, s.nsub()), dim3(512), 0, stream, (const bf16_t*)dy,
                         (const bf16_t*)wg, (const bf16_t*)wu, (const bf16_t*)wd, s.tokens, s.d_model, s.d_ff,
                         s.group_size, tile_group, ptoken, (uint32_t)ntiles_max * BM, (const bf16_t*)hg,
                         (const bf16_t*)hu, (bf16_t*)dg, (bf16_t*)du, (bf16_t*)act, (bf16_t*)partials);
      return hipGetLastError();
    }
  }
  auto kern = partials_nontemporal(s, ntiles_max) ? dhdx2_kernel<GSB, kCpolNontemporal> : dhdx2_kernel<GSB, 0>;
  const unsigned gx = (ntiles_max + 7) / 8 * 8;  // a multiple of 8 (the tile order is XCD-local)
  hipLaunchKernelGGL(kern, dim3(gx, s.nsub()), dim3(64 * fwd_waves<GSB>()), 0, stream, (const bf16_t*)dy,
                     (const bf16_t*)wg, (const bf16_t*)wu, (const bf16_t*)wd, s.tokens, s.d_model, s.d_ff,
                     s.group_size, tile_group, ptoken, (uint32_t)ntiles_max * BM, (const bf16_t*)hg,
                     (const bf16_t*)hu, (bf16_t*)dg, (bf16_t*)du, (bf16_t*)act, (bf16_t*)partials);
  return hipGetLastError();
}

template <int GSB>
hipError_t dw2_t(const FfnShape& s, const void* x, const void* dy, const int32_t* tile_off, const int32_t* ptoken,
                 int rows_total, const void* dg, const void* du, const void* act, void* dwg, void* dwu, void* dwd,
                 int cht, void* slots, hipStream_t stream) {
  LaunchTimer timer("bwd_dw", stream);
  const int G = s.groups(), units = 2 * G * s.nsub();
  const int ndb = (s.d_model + 128 * dw_subtiles<GSB>() - 1) / (128 * dw_subtiles<GSB>());
  if (dw_waves<GSB>() != 8) cht = 0;
  // order: dw_plan_xcd (eight waves; sized for the most chunks the rows allow) or dw_work
  const dim3 grid(dw_waves<GSB>() == 8 ? dw_plan_grid(G, 2 * s.nsub(), ndb, rows_total, cht) : dw_grid(units, ndb));
  hipLaunchKernelGGL((dw2_kernel<GSB>), grid, dim3(64 * dw_waves<GSB>()), 0, stream, (const bf16_t*)x,
                     (const bf16_t*)dy, s.tokens,
                     s.d_model, s.d_ff, s.group_size, s.nsub(), tile_off, ptoken, (uint32_t)rows_total,
                     (const bf16_t*)dg, (const bf16_t*)du, (const bf16_t*)act, (bf16_t*)dwg, (bf16_t*)dwu,
                     (bf16_t*)dwd, cht, (float*)slots);
  hipError_t e = hipGetLastError();
  const int sg = std::min(G, dw_split_groups_max(rows_total, cht));
  if (e != hipSuccess || sg == 0) return e;
  const size_t per_slot = (size_t)3 * s.group_size * s.d_model;
  const dim3 sgrid((unsigned)((per_slot + 1024 * kDwSumIt - 1) / (1024 * kDwSumIt)), (unsigned)std::min(sg, 8));
  hipLaunchKernelGGL(dw_slot_sum_kernel, sgrid, dim3(256), 0, stream, tile_off, G, cht, s.group_size, s.d_model,
                     s.d_ff, (const float*)slots, (bf16_t*)dwg, (bf16_t*)dwu, (bf16_t*)dwd);
  return hipGetLastError();
}

}  // namespace

// Buffers the tile kernels address with 32-bit offsets from one base: x / dy
// (gathered rows), the weights and the compact activations.  The partial rows
// are addressed per tile, so their total size is not limited.
bool bf16_pipelined(const FfnShape& s, int ntiles_max) {
  if (s.dtype != 1 || (s.gsb() != 32 && s.gsb() != 64 && s.gsb() != 128)) return false;
  const unsigned long long lim = 1ull << 31;
  const unsigned long long rows = (unsigned long long)ntiles_max * BM;
  return (unsigned long long)s.tokens * s.d_model * 2 < lim && (unsigned long long)s.d_ff * s.d_model * 2 < lim &&
         (unsigned long long)s.nsub() * rows * s.gsb() * 2 < lim;
}

bool fwd_split(const FfnShape& s, int ntiles_max) {
  return bf16_pipelined(s, ntiles_max) && s.gsb() == 64 && (long long)ntiles_max * s.nsub() <= kFwdSplitTiles &&
         !partials_nontemporal(s, ntiles_max);
}

hipError_t launch_fwd2(const FfnShape& s, const void* x, const void* wg, const void* wu, const void* wd,
                       const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, int pad, void* hg_saved,
                       void* hu_saved, void* partials, void* act, hipStream_t stream) {
  if (ntiles_max == 0) return hipSuccess;
  if (!fwd_split(s, ntiles_max)) act = nullptr;
  switch (s.gsb()) {
    case 32: return fwd2_t<32>(s, x, wg, wu, wd, tile_group, ptoken, ntiles_max, pad, hg_saved, hu_saved, partials,
                               act, stream);
    case 64: return fwd2_t<64>(s, x, wg, wu, wd, tile_group, ptoken, ntiles_max, pad, hg_saved, hu_saved, partials,
                               act, stream);
    default: return fwd2_t<128>(s, x, wg, wu, wd, tile_group, ptoken, ntiles_max, pad, hg_saved, hu_saved, partials,
                                act, stream);
  }
}

hipError_t launch_dhdx2(const FfnShape& s, const void* dy, const void* wg, const void* wu, const void* wd,
                        const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, const void* hg_saved,
                        const void* hu_saved, void* dg, void* du, void* act, void* partials, hipStream_t stream) {
  if (ntiles_max == 0) return hipSuccess;
  switch (s.gsb()) {
    case 32: return dhdx2_t<32>(s, dy, wg, wu, wd, tile_group, ptoken, ntiles_max, hg_saved, hu_saved, dg, du, act,
                                partials, stream);
    case 64: return dhdx2_t<64>(s, dy, wg, wu, wd, tile_group, ptoken, ntiles_max, hg_saved, hu_saved, dg, du, act,
                                partials, stream);
    default: return dhdx2_t<128>(s, dy, wg, wu, wd, tile_group, ptoken, ntiles_max, hg_saved, hu_saved, dg, du, act,
                                 partials, stream);
  }
}

hipError_t launch_dw2(const FfnShape& s, const void* x, const void* dy, const int32_t* tile_off, const int32_t* ptoken,
                      int rows_total, const void* dg, const void* du, const void* act, void* dwg, void* dwu, void* dwd,
                      int cht, void* slots, hipStream_t stream) {
  switch (s.gsb()) {
    case 32: return dw2_t<32>(s, x, dy, tile_off, ptoken, rows_total, dg, du, act, dwg, dwu, dwd, 0, slots, stream);
    case 64: return dw2_t<64>(s, x, dy, tile_off, ptoken, rows_total, dg, du, act, dwg, dwu, dwd, 0, slots, stream);
    default:
      return dw2_t<128>(s, x, dy, tile_off, ptoken, rows_total, dg, du, act, dwg, dwu, dwd, cht, slots, stream);
  }
}

// From the shape alone: buckets above 1.5 times the mean (at least 16
// tiles) are cut, so an even load runs one item per (unit, d-block) and a hot
// group's chunks spread over the CUs.  A launch whose (unit, d-block) items
// number fewer than two per CU runs about one round, so its slowest item sets
// the time: there buckets above 1.125 times the mean are cut (an even load's
// largest bucket lies far below that: at the 370M shape 35 tiles against 31
// on average, about 10 standard deviations of the binomial counts).  (Cutting
// every bucket when the items underfill the CUs, e.g. 168 items at the 370M
// shape into 504, measured slower: weight gradients 145 -> 138 us, but the
// step 0.443 -> 0.506 ms, the fp32 slots' traffic slowing the kernels around
// them.)
int dw_chunk_tiles(const FfnShape& s, int ntiles_max, int pad) {
  if (!bf16_pipelined(s, ntiles_max) || s.gsb() != 128 || s.tokens <= 0) return 0;
  const long long mean_rows = ((long long)s.tokens * s.k + s.groups() - 1) / s.groups();
  const long long items = 2ll * s.groups() * s.nsub() * ((s.d_model + 128 * dw_subtiles<128>() - 1) /
                                                           (128 * dw_subtiles<128>()));
  const long long num = items >= 2ll * kNominalCUs ? 3 : 9, den = items >= 2ll * kNominalCUs ? 2 : 8;
  const long long cht = std::max(16ll, (num * mean_rows + den * BM - 1) / (den * BM));
  // a bucket holds at most one position per token, padded to the pad unit
  const long long most = ((long long)s.tokens + pad - 1) / pad * (pad / BM);
  return cht >= most ? 0 : (int)cht;
}

size_t dw_slot_bytes(const FfnShape& s, size_t rows, int cht) {
  return (size_t)dw_split_slots_max((long long)rows, cht) * 3 * s.group_size * s.d_model * 4;
}

}  // namespace esg
