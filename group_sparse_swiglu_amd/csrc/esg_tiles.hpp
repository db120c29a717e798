// Tile building blocks of the pipelined bf16 kernels (esg_ffn_bf16.hip,
// esg_dense.hip): the direct-to-LDS pipelines, the per-tile phase-1 loops of
// the forward (gate/up) and backward (dA) GEMMs, and the weight-gradient body.
#pragma once

#include "esg_internal.hpp"
#include "esg_pipe.hpp"

namespace esg {
namespace tiles {

constexpr int NT = 256;
constexpr int BM = kTileRows;  // bucket positions per tile
constexpr int DB = 128;        // d rows per forward phase-2 block

typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef int v4i32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store8(rsrc_t r, uint32_t voff, const float (&v)[4]) {
  const v2i32 q = {(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3])};
  __builtin_amdgcn_raw_buffer_store_b64(q, r, voff, 0, 0);
}

// A [128 positions][DW d] bf16 block held as MFMA accumulators (lane: four
// consecutive d of one position) is written to row-major partial rows through
// LDS, so that every store instruction writes whole rows (16 bytes per lane,
// DW*2 bytes per row) instead of 32-byte pieces of 16 rows.  Rows 0..63 are
// staged in lds0, rows 64..127 in lds1 (DW*2*64 bytes each); 16-byte chunks
// are XOR-swizzled by row.  row_off[it]: byte offset of the partial row this
// thread stores at iteration it (kOOB for padding rows).
template <int DW, int NTH = 256>
struct RowStore {
  static constexpr int RB = DW * 2;       // bytes per staged row
  static constexpr int NCHK = RB / 16;    // 16-byte chunks per row
  static constexpr int IT = 128 * NCHK / NTH;  // 16-byte stores per thread (NTH threads)
  static_assert(IT * NTH == 128 * NCHK, "whole rows per pass");
  static __device__ __forceinline__ int row(int it, int tid) { return (it * NTH + tid) / NCHK; }
  static __device__ __forceinline__ int chunk(int it, int tid) { return (it * NTH + tid) % NCHK; }
  static __device__ __forceinline__ int off(int rr, int c) { return rr * RB + ((c ^ (rr & (NCHK - 1))) << 4); }
  // acc value e of a lane: d = dl + e (dl % 4 == 0, dl < DW), position r (0..127)
  static __device__ __forceinline__ void put(ESG_LDS char* lds0, ESG_LDS char* lds1, int r, int dl,
                                             const float (&v)[4]) {
    ESG_LDS char* h = r < 64 ? lds0 : lds1;
    lds_write8(h + off(r & 63, dl >> 3) + (dl & 7) * 2, pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
  // after a barrier: every thread stores IT chunks of 16 bytes (CPOL: the
  // buffer store's cache policy, 2 = nontemporal)
  template <int CPOL = 0>
  static __device__ __forceinline__ void flush(const ESG_LDS char* lds0, const ESG_LDS char* lds1, rsrc_t rp,
                                               const uint32_t (&row_off)[IT], int db0, int d) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int it = 0; it < IT; ++it) {
      const int r = row(it, tid), c = chunk(it, tid);
      const u32x4_t q = *(const ESG_LDS u32x4_t*)((r < 64 ? lds0 : lds1) + off(r & 63, c));
      const int dd = db0 + c * 8;
      const uint32_t o = (row_off[it] != kOOB && dd < d) ? row_off[it] + dd * 2 : kOOB;
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(v4i32, q), rp, o, 0, CPOL);
    }
  }
};

// Pipeline depth: 3 stages for 128-neuron blocks (one workgroup per CU), 2 for
// 64-neuron blocks so that two workgroups share a CU.
template <int GSB>
constexpr int stages_for() {
  return GSB >= 128 ? 3 : 2;
}


// ---------------------------------------------------------------------------
// Direct-to-LDS K loop over a ring of NS stages (2 to 4): tile t lands in
// stage t % NS and NS-1 tiles are in flight ahead of the one consumed.
//   issue(stage, t)    enqueues tile t's loads (L per lane; called once per
//                      tile, in order);
//   compute(stage, t)  consumes a landed tile and may end with S global stores
//                      per lane.
// Step t waits for tile t with the exact vmcnt the issue order implies
// (vector loads and stores retire in order): younger than tile t are the
// loads of the min(NS-2, nk-1-t) tiles issued after it and the stores of the
// min(t, NS-1) steps computed since it was issued.  The direct-to-LDS loads
// are invisible to the compiler (esg_pipe.hpp), so these explicit waits are
// the only ones that order them, and the loop can stay a plain rolled loop:
// the accumulators then stay in place across steps.
// ---------------------------------------------------------------------------
template <int L, int S, int A, int B>
__device__ __forceinline__ void wait_tile(int a, int b) {
  // a in [0, A], b in [0, B], wave-uniform: one immediate wait per case
  if (a == A && b == B) {
    static_assert(A * L + B * S < 64, "vmcnt range");
    wait_vmcnt<A * L + B * S>();
  } else if constexpr (B > 0) {
    if (a == A) wait_tile<L, S, A, B - 1>(a, b);
    else if constexpr (A > 0) wait_tile<L, S, A - 1, B>(a, b);
  } else if constexpr (A > 0) {
    wait_tile<L, S, A - 1, B>(a, b);
  }
}

template <int NS, int L, int S, class Issue, class Compute>
__device__ __forceinline__ void kloop_ring(int nk, ESG_LDS char* const (&st)[NS], Issue&& issue,
                                           Compute&& compute) {
  static_assert(NS >= 2 && NS <= 4, "two to four stages");
  if (nk <= 0) return;
#pragma unroll
  for (int j = 0; j < NS - 1; ++j)
    if (j < nk) issue(st[j], j);
  int cur = 0;       // t % NS
  int nxt = NS - 1;  // (t + NS - 1) % NS
  for (int t = 0; t < nk; ++t) {
    wait_tile<L, S, NS - 2, (S > 0 ? NS - 1 : 0)>(min(NS - 2, nk - 1 - t), S > 0 ? min(t, NS - 1) : 0);
    wait_lgkm0();
    barrier();
    if (t + NS - 1 < nk) issue(st[nxt], t + NS - 1);
    compute(st[cur], t);
    cur = cur + 1 == NS ? 0 : cur + 1;
    nxt = nxt + 1 == NS ? 0 : nxt + 1;
  }
}

template <int NS, int L, int S, class Issue, class Compute>
__device__ __forceinline__ void kloop(int nk, ESG_LDS char* s0, ESG_LDS char* s1, ESG_LDS char* s2, Issue&& issue,
                                      Compute&& compute) {
  static_assert(NS == 2 || NS == 3, "two or three stages");
  if constexpr (NS == 2) {
    ESG_LDS char* const st[2] = {s0, s1};
    kloop_ring<2, L, S>(nk, st, issue, compute);
  } else {
    ESG_LDS char* const st[3] = {s0, s1, s2};
    kloop_ring<3, L, S>(nk, st, issue, compute);
  }
}


// ===========================================================================
// Forward
// ===========================================================================
// NW wavefronts: WM = NW/2 neuron slices x 2 position halves (64 each).
template <int GSB, int NW = 4>
struct Fwd2 {
  static constexpr int NTH = 64 * NW;
  static constexpr int WM = NW / 2;
  static constexpr int RA = 2 * GSB;           // weight rows per tile (gate, then up)
  static constexpr int A_BYTES = RA * 128;     // one 64-wide K stage
  static constexpr int B_BYTES = BM * 128;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int IA = RA / (8 * NW);     // DMA instructions per lane per stage (A)
  static constexpr int IB = BM / (8 * NW);     // (B)
  static constexpr int L = IA + IB;
  static constexpr int FMP = GSB / WM / 16;    // gate/up fragment pairs per wave
  static constexpr int FN = 4;                 // 64 positions per wave
  static constexpr int KSUB = GSB >= 64 ? GSB / 64 : 1;  // 64-wide K sub-tiles of the group width (32: half of one)
  static constexpr int ACT_BYTES = KSUB * BM * 128;
  static constexpr int W2_BYTES = KSUB * DB * 128;
  static constexpr int IW2 = DB / (8 * NW);    // W_down DMA instructions per lane per K sub-tile
  static constexpr int FM2 = DB / WM / 16, FN2 = 4;  // phase-2 wave tile DB/WM d x 64 positions
  static constexpr int STORES2 = RowStore<DB, NTH>::IT;  // buffer stores per lane per d-block
  static_assert(ACT_BYTES <= STAGE && W2_BYTES <= STAGE, "phase-2 tiles reuse the stages");
  static_assert(IA * 8 * NW == RA && IB * 8 * NW == BM && FMP >= 1, "whole DMA instructions and fragments");
};

// Phase 1 of a forward tile: [hg; hu]^T for the GSB neurons from nb0 (gate
// rows, then up rows) against the 128 bucket positions from prow0, whose token
// ids come from ptoken (-1 = padding, reads zeros).  K = d in 64-wide stages.
// acc[p][j] (p < FMP: gate, p >= FMP: up) follows the wave mapping below.
// kt0, nkt: the K stages [kt0, kt0 + nkt) only (nkt < 0: all of K).
template <int GSB, int NS, int NW = 4>
__device__ __forceinline__ void gateup_tile(const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg,
                                            const bf16_t* __restrict__ wu, int tokens, int d, int F, int nb0,
                                            const int32_t* __restrict__ ptoken, uint32_t prow0,
                                            ESG_LDS char* const (&st)[NS],
                                            f32x4 (&acc)[2 * Fwd2<GSB, NW>::FMP][Fwd2<GSB, NW>::FN],
                                            int kt0 = 0, int nkt = -1) {
  using C = Fwd2<GSB, NW>;
  const int lane = threadIdx.x & 63, w = wave_id();
  const uint32_t kbytes = (uint32_t)d * 2;
  const DmaSrc rx = make_dma_src(x, (uint32_t)tokens * kbytes);
  const DmaSrc rg = make_dma_src(wg, (uint32_t)F * kbytes);
  const DmaSrc ru = make_dma_src(wu, (uint32_t)F * kbytes);

  // ---- DMA addressing: lane (row = lane/8 of an 8-row group, slot = lane%8) ----
  const int c_lane = (lane & 7) ^ (lane >> 3);  // logical chunk this lane moves
  uint32_t voffA[C::IA];
#pragma unroll
  for (int i = 0; i < C::IA; ++i) {
    const int r = (w * C::IA + i) * 8 + (lane >> 3);
    const int grow = nb0 + (r < GSB ? r : r - GSB);
    voffA[i] = grow < F ? (uint32_t)grow * kbytes + c_lane * 16 : kOOB;
  }
  uint32_t voffB[C::IB];
#pragma unroll
  for (int i = 0; i < C::IB; ++i) {
    const int r = (w * C::IB + i) * 8 + (lane >> 3);
    const int t = ptoken[prow0 + r];
    voffB[i] = t >= 0 ? (uint32_t)t * kbytes + c_lane * 16 : kOOB;
  }
  auto issue = [&](ESG_LDS char* st, int kt) __attribute__((always_inline)) {
    const uint32_t kb = (uint32_t)(kt0 + kt) * 128;
    const bool kin = kb + c_lane * 16 < kbytes;
#pragma unroll
    for (int i = 0; i < C::IA; ++i) {
      const bool gate = (w * C::IA + i) * 8 < GSB;  // wave-uniform
      dma16(gate ? rg : ru, st + (w * C::IA + i) * 1024, (kin && voffA[i] != kOOB) ? voffA[i] + kb : kOOB);
    }
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
      dma16(rx, st + C::A_BYTES + (w * C::IB + i) * 1024, (kin && voffB[i] != kOOB) ? voffB[i] + kb : kOOB);
  };

  // MFMA: wave (wm, wn) owns neurons [wm*GSB/WM, +GSB/WM) of gate and up, positions [wn*64, +64) ----
  const int wm = w % C::WM, wn = w / C::WM;
  int arow[2 * C::FMP], brow[C::FN];
#pragma unroll
  for (int p = 0; p < C::FMP; ++p) {
    arow[p] = wm * (GSB / C::WM) + p * 16 + (lane & 15);
    arow[C::FMP + p] = GSB + arow[p];
  }
#pragma unroll
  for (int j = 0; j < C::FN; ++j) brow[j] = wn * 64 + j * 16 + (lane & 15);
  zero_acc(acc);
  auto compute = [&](const ESG_LDS char* st, int) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int c = kb * 4 + (lane >> 4);
      uint4 a[2 * C::FMP], b[C::FN];
#pragma unroll
      for (int i = 0; i < 2 * C::FMP; ++i) a[i] = frag_krow(st, arow[i], c);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) b[j] = frag_krow(st + C::A_BYTES, brow[j], c);
#pragma unroll
      for (int i = 0; i < 2 * C::FMP; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) mma_bf16(acc[i][j], a[i], b[j]);
    }
  };
  kloop_ring<NS, C::L, 0>(nkt < 0 ? (int)((kbytes + 127) / 128) : nkt, st, issue, compute);
}

// ===========================================================================
// Backward dh (+ SiLU' epilogue) and dx partials.
//   phase 1  dA^T = W_down[:, group cols]^T . dY_tile^T   (K = d); W_down comes
//            in as an N-row tile (rows = d, columns = neurons)
//   epilogue dg = dA*hu*SiLU'(hg), du = dA*SiLU(hg), a = SiLU(hg)*hu, stored
//            row-major [pos][gsb] for the dW kernel; [dg du] to an LDS K-row tile
//   phase 2  Q^T = [W_gate; W_up]^T[d-block] . [dg du]^T  (K = 2*gsb); the
//            weights come in as N-row tiles (rows = neurons, columns = d)
// ===========================================================================
// NW wavefronts: phase 1 WM = NW/2 neuron slices x 2 position halves;
// phase 2 two d halves (32 each) x NW/2 position slices.
// BMT: bucket positions of a phase-1 tile (128, or 256 for a pair of tiles of
// one group); phase 2 always works on 128 positions at a time.
template <int GSB, int NW = 4, int BMT = BM>
struct Dh2 {
  static constexpr int NTH = 64 * NW;
  static constexpr int WM = NW / 2;
  static constexpr int NCH = GSB / 8;            // 16-byte chunks per neuron row segment
  static constexpr int A_BYTES = 64 * GSB * 2;   // N-row: 64 d rows x GSB neurons
  static constexpr int B_BYTES = BMT * 128;      // K-row: BMT positions x 64 d
  static constexpr int STAGE1 = A_BYTES + B_BYTES;
  static constexpr int IA = NCH / NW;
  static constexpr int IB = BMT / (8 * NW);
  static constexpr int L = IA + IB;
  static constexpr int FM = GSB / WM / 16, FN = BMT / 32;  // wave tile GSB/WM neurons x BMT/2 positions
  static constexpr int KSUB2 = 2 * GSB / 64;
  static constexpr int DGU_BYTES = KSUB2 * BM * 128;
  static constexpr int DB2 = 64;
  static constexpr int W2_BYTES = 2 * GSB * DB2 * 2;  // N-row: 2*GSB neuron rows x 64 d
  static constexpr int IW = 2 * GSB / (8 * NW);
  static constexpr int PW2 = BM / (NW / 2);      // positions per wave in phase 2
  static constexpr int FM2 = 2, FN2 = PW2 / 16;  // wave tile 32 d x PW2 positions
  static constexpr int STORES2 = RowStore<DB2, NTH>::IT;
  static constexpr int STAGE = STAGE1 > W2_BYTES ? STAGE1 : W2_BYTES;
  static_assert(IA * NW == NCH && IB * 8 * NW == BMT && IW * 8 * NW == 2 * GSB && FM >= 1, "whole instructions");
};

// Wave tile of a backward phase 1.  WL = 0: wave w takes neuron slice w % WM
// (GSB/WM neurons) of position half w / WM (BMT/2 positions); WL = 1: wave w
// takes all GSB neurons of position slice w (BMT/NW positions).
template <int GSB, int NW, int BMT, int WL>
struct DaWave {
  static constexpr int FM = WL == 0 ? Dh2<GSB, NW, BMT>::FM : GSB / 16;
  static constexpr int FN = WL == 0 ? Dh2<GSB, NW, BMT>::FN : BMT / NW / 16;
  static __device__ __forceinline__ int neuron0(int w) { return WL == 0 ? (w % (NW / 2)) * (GSB / (NW / 2)) : 0; }
  static __device__ __forceinline__ int pos0(int w) { return WL == 0 ? (w / (NW / 2)) * (BMT / 2) : w * (BMT / NW); }
};

// Phase 1 of a backward tile: dA^T = W_down[:, nb0 .. nb0+GSB)^T . dY_tile^T
// (K = d) for the BMT bucket positions from prow0 (token ids from ptoken).
// acc[i][j]: neurons neuron0 + 16i.., positions pos0 + 16j.. (DaWave).
template <int GSB, int NS, int NW = 4, int BMT = BM, int WL = 0>
__device__ __forceinline__ void da_tile(const bf16_t* __restrict__ dy, const bf16_t* __restrict__ wd, int tokens,
                                        int d, int F, int nb0, const int32_t* __restrict__ ptoken, uint32_t prow0,
                                        ESG_LDS char* st0, ESG_LDS char* st1, ESG_LDS char* st2,
                                        f32x4 (&acc)[DaWave<GSB, NW, BMT, WL>::FM][DaWave<GSB, NW, BMT, WL>::FN]) {
  using C = Dh2<GSB, NW, BMT>;
  using WV = DaWave<GSB, NW, BMT, WL>;
  const int lane = threadIdx.x & 63, w = wave_id();
  const uint32_t kbytes = (uint32_t)d * 2;
  const DmaSrc ry = make_dma_src(dy, (uint32_t)tokens * kbytes);
  const DmaSrc rd = make_dma_src(wd, (uint32_t)d * F * 2);

  // phase-1 DMA: A = W_down N-row tile, B = dY K-row tile
  uint32_t voffA[C::IA];
  int rowA[C::IA];
#pragma unroll
  for (int i = 0; i < C::IA; ++i) {
    const int row = (w * C::IA + i) * (64 / C::NCH) + lane / C::NCH;
    const int j = (lane % C::NCH) ^ mn_swz<C::NCH>(row);
    rowA[i] = nb0 + j * 8 < F ? row : 0x40000000;  // columns past F: never in range
    voffA[i] = (uint32_t)row * F * 2 + (uint32_t)nb0 * 2 + j * 16;
  }
  const int c_lane = (lane & 7) ^ (lane >> 3);
  uint32_t voffB[C::IB];
#pragma unroll
  for (int i = 0; i < C::IB; ++i) {
    const int r = (w * C::IB + i) * 8 + (lane >> 3);
    const int t = ptoken[prow0 + r];
    voffB[i] = t >= 0 ? (uint32_t)t * kbytes + c_lane * 16 : kOOB;
  }
  auto issue = [&](ESG_LDS char* st, int kt) __attribute__((always_inline)) {
    const uint32_t k0 = (uint32_t)kt * 64;
#pragma unroll
    for (int i = 0; i < C::IA; ++i)
      dma16(rd, st + (w * C::IA + i) * 1024, k0 + rowA[i] < (uint32_t)d ? voffA[i] + k0 * F * 2 : kOOB);
    const uint32_t kb = k0 * 2;
    const bool kin = kb + c_lane * 16 < kbytes;
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
      dma16(ry, st + C::A_BYTES + (w * C::IB + i) * 1024, (kin && voffB[i] != kOOB) ? voffB[i] + kb : kOOB);
  };
  const int n0 = WV::neuron0(w);
  int brow[WV::FN];
#pragma unroll
  for (int j = 0; j < WV::FN; ++j) brow[j] = WV::pos0(w) + j * 16 + (lane & 15);
  zero_acc(acc);
  auto compute = [&](const ESG_LDS char* st, int) __attribute__((always_inline)) {
    uint4 a[2][WV::FM], b[2][WV::FN];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int c = kb * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < WV::FM; ++i) a[kb][i] = frag_nrow<C::NCH>(st, kb, n0 + i * 16, lane);
#pragma unroll
      for (int j = 0; j < WV::FN; ++j) b[kb][j] = frag_krow(st + C::A_BYTES, brow[j], c);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < WV::FM; ++i)
#pragma unroll
        for (int j = 0; j < WV::FN; ++j) mma_bf16(acc[i][j], a[kb][i], b[kb][j]);
  };
  kloop<NS, C::L, 0>((d + 63) / 64, st0, st1, st2, issue, compute);
}

// ===========================================================================
// Backward weight gradients, one workgroup per (group sub-block, 128-wide
// d-block, kind) with K = the group's padded positions:
//   kind 0: dW_gate|up[rows of g]^T[d-block] = X^T . [dg | du]
//   kind 1: dW_down[d-block, cols of g]^T   = a^T . dY
// Every operand comes in as an N-row tile (rows = positions).  Within a stage
// LDS row R holds position perm(R) (two 2-bit fields of R swapped) so each
// lane's four gathered rows are four consecutive positions whose token ids
// come from one 16-byte load; both operands use the same row order, which
// only permutes the K summation.
// ===========================================================================
// XS 128-d sub-tiles of the gathered operand per stage: a workgroup covers
// DW = 128*XS d of one neuron block, so the packed dg/du/a rows (which every
// d-block of the block reads again) are read ceil(d/DW) times.
// NWD wavefronts: 4 (one per SIMD, each holding a quarter of the output), or
// 8 (two per SIMD, an eighth each: kind 0 splits the d range in four, kind 1
// in four along d as well).
template <int GSB, int XS = 1, int NWD = 4>
struct Dw2 {
  static constexpr int NTH = 64 * NWD;
  static constexpr int DW = 128 * XS;
  static constexpr int NCHP = GSB / 8;           // chunks per position row of dg/du/a
  static constexpr int X_SUB = 64 * 256;         // N-row: 64 positions x 128 d
  static constexpr int X_BYTES = XS * X_SUB;
  static constexpr int P_BYTES = 64 * GSB * 2;   // N-row: 64 positions x GSB neurons
  static constexpr int STAGE = X_BYTES + 2 * P_BYTES;
  static constexpr int IXS = 16 / NWD;           // x DMA instructions per lane per 128-d sub-tile
  static constexpr int IX = IXS * XS;
  static constexpr int IP = NCHP * 4 / NWD / 4;  // packed-tile DMA instructions per lane
  static constexpr int L0 = IX + 2 * IP, L1 = IX + IP;
  static constexpr int WM0 = NWD / 2;            // kind 0: d slices x {gate, up}
  static constexpr int FM0 = 8 * XS / WM0, FN0 = GSB / 16;   // kind 0 wave tile: DW/WM0 d x GSB neurons
  static constexpr int WN1 = NWD / 2;            // kind 1: neuron halves x d slices
  static constexpr int FM1 = GSB / 32, FN1 = 8 * XS / WN1;   // kind 1 wave tile: GSB/2 neurons x DW/WN1 d
  static_assert(IXS >= 1 && IP >= 1 && FM0 >= 1 && FN1 >= 1, "whole instructions and fragments");
};

// Order of the weight-gradient workgroups.  A "unit" is one (neuron block,
// kind) pair; its ndb d-blocks read the same packed dg/du/a rows.
// dw_work: workgroup L takes neuron block L % GB, then d-block, then kind
// (GB = units / 2), so the workgroups in flight together spread over all
// neuron blocks (four-wave workgroups of 32- and 64-neuron blocks).
// dw_work_xcd: workgroups go to the 8 XCDs round-robin, so workgroup L runs
// on XCD L % 8; XCD x takes the flat items [x*per, (x+1)*per) in order (unit
// major, d-block minor), so a unit's d-blocks run together in one L2 and read
// its packed rows from there (the dense limit's eight-wave workgroups; for
// the routed 128-neuron blocks, measured at the 1.3B shape, 4.24 -> 3.26 GB
// of L2 misses; they now take dw_plan_xcd below).
// Both return false for workgroups past the last item.
struct DwWork {
  int unit, db;
};
__device__ __forceinline__ bool dw_work(int L, int units, int ndb, DwWork& w) {
  const int GB = units / 2;
  if (L >= units * ndb) return false;
  const int gb = L % GB, rest = L / GB;
  w.db = rest % ndb;
  w.unit = gb * 2 + rest / ndb;
  return true;
}
inline int dw_grid(int units, int ndb) { return units * ndb; }
__device__ __forceinline__ bool dw_work_xcd(int L, int units, int ndb, DwWork& w) {
  const int n = units * ndb, per = (n + 7) / 8;
  const int f = (L % 8) * per + L / 8;
  if (f >= n) return false;
  w.unit = f / ndb;  // neuron block unit / 2, kind unit % 2
  w.db = f % ndb;
  return true;
}
inline int dw_grid_xcd(int units, int ndb) { return (units * ndb + 7) / 8 * 8; }

// Weight-gradient work with heavy groups cut by positions.  Under uneven
// routing a popular group's (unit, d-block) workgroups sum many times the
// positions of the others and finish last.  A group whose bucket holds more
// than cht tiles is cut into c = ceil(tiles / cht) chunks of cht tiles (the
// last one shorter); each chunk is an item per (unit, d-block) that sums its
// positions into an fp32 slot, and a second launch adds a group's slots in
// chunk order.  Groups of at most cht tiles (every group when cht = 0) keep
// one item per (unit, d-block) that writes bf16 directly.  The (unit, chunk)
// pairs are numbered group-major, then chunk, then unit; workgroups go to the
// 8 XCDs round-robin (workgroup L runs on XCD L % 8), and the m-th pair of XCD
// x is j = 8m + (x + m) % 8, with all d-blocks of a pair in a row: a pair's
// d-blocks read its packed rows from one L2, the chunks of a hot group land on
// different XCDs, and every XCD gets both kinds (kind 0 does twice the work
// of kind 1, and with j = 8m + x the even XCDs would take every kind-0 pair).
// Every wave of the workgroup derives the same item from tile_off (a
// wave-wide scan of the per-group chunk counts).
struct DwItem {
  int unit, db;  // as in DwWork
  int t0, nt;    // the chunk's first tile and tile count
  int slot;      // the chunk's fp32 slot (group-major, chunk order), or -1
};
__device__ __forceinline__ int dw_chunks(const int32_t* __restrict__ tile_off, int g, int cht) {
  const int nt = tile_off[g + 1] - tile_off[g];
  return cht > 0 && nt > cht ? (nt + cht - 1) / cht : 1;
}
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}
// The group holding chunk-unit q (q counts chunks over the groups in order):
// g, its chunk count c, its first chunk index pc and its first slot ps (split
// groups only take slots).  False when q is past the last chunk.
struct DwGroupAt {
  int g, c, pc, ps;
};
__device__ __forceinline__ bool dw_group_at(const int32_t* __restrict__ tile_off, int G, int cht, int q,
                                            DwGroupAt& r) {
  const int lane = threadIdx.x & 63;
  int carry = 0, scarry = 0;
  for (int g0 = 0; g0 < G; g0 += 64) {
    const int g = g0 + lane;
    const int c = g < G ? dw_chunks(tile_off, g, cht) : 0;
    const int s = c >= 2 ? c : 0;
    const int inc = wave_incl_scan(c) + carry;
    const int sinc = wave_incl_scan(s) + scarry;
    const uint64_t hit = __ballot(inc > q);
    if (hit != 0) {  // (lane reads return vector registers: readfirstlane keeps the item scalar)
      const int src = __builtin_ctzll(hit);
      r.g = g0 + src;
      r.c = __builtin_amdgcn_readfirstlane(__shfl(c, src));
      r.pc = __builtin_amdgcn_readfirstlane(__shfl(inc, src)) - r.c;
      r.ps = __builtin_amdgcn_readfirstlane(__shfl(sinc, src) - __shfl(s, src));
      return true;
    }
    carry = __shfl(inc, 63);
    scarry = __shfl(sinc, 63);
  }
  return false;
}
// upg: units per group (2 * nsub).  Returns false past the last item (the
// grid is sized for the most chunks the rows allow).
__device__ __forceinline__ bool dw_plan_xcd(int L, const int32_t* __restrict__ tile_off, int G, int upg, int ndb,
                                            int cht, DwItem& it) {
  const int i = L / 8, m = i / ndb, j = 8 * m + ((L + m) & 7);
  DwGroupAt r;
  if (!dw_group_at(tile_off, G, cht, j / upg, r)) return false;  // past the last pair
  const int local = j - r.pc * upg;
  const int chunk = local / upg;
  it.unit = r.g * upg + local % upg;
  it.db = i % ndb;
  const int ta = __builtin_amdgcn_readfirstlane(tile_off[r.g]), tb = __builtin_amdgcn_readfirstlane(tile_off[r.g + 1]);
  it.t0 = ta + chunk * cht;
  it.nt = min(r.c == 1 ? tb - ta : cht, tb - it.t0);
  it.slot = r.c >= 2 ? r.ps + chunk : -1;
  return true;
}
// Upper bounds for a launch of `rows` bucket rows (padding included) and
// chunks of cht tiles: a split group holds more than cht tiles, so there are
// fewer than rows / (cht * 128) of them, and its c chunks number fewer than
// twice its tiles / cht.
inline int dw_split_groups_max(long long rows, int cht) { return cht > 0 ? (int)(rows / ((long long)BM * cht)) : 0; }
inline int dw_split_slots_max(long long rows, int cht) {
  return cht > 0 ? (int)(2 * rows / ((long long)BM * cht)) : 0;
}
inline int dw_plan_grid(int G, int upg, int ndb, long long rows, int cht) {
  const long long chunks = (long long)G + dw_split_groups_max(rows, cht);
  return (int)(8ll * ndb * ((chunks * upg + 7) / 8));
}

template <int MODE>
__device__ __forceinline__ void store_dw(bf16_t* out, float* acc32, float (&v)[4]) {
  if constexpr (MODE == 2 || MODE == 3) {
    float o[4];
    Quad<float>::load(acc32, o);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] += o[e];
  }
  if constexpr (MODE == 0 || MODE == 3)
    Quad<bf16_t>::store(out, v);
  else
    Quad<float>::store(acc32, v);
}

__device__ __forceinline__ int dw_perm(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

// MODE: 0 stores bf16; 1 stores the fp32 sums to f0/f1; 2 adds them to
// f0/f1; 3 adds f0/f1 and stores bf16 (K split over consecutive launches, in
// a fixed order); 4 stores the fp32 sums to f0/f1 laid out for this block
// alone (kind 0: [GSB][d], kind 1: [d][GSB]), a chunk's slot.  Ids of the K positions come from ptoken[pid0 ..], their
// packed dg/du/a rows start at row p0; np positions (a multiple of 64).
template <int GSB, int KIND, int NS, int MODE = 0, int XS = 1, int NWD = 4>
__device__ __forceinline__ void dw2_body(const bf16_t* __restrict__ src, int tokens, int d, int F, int nb0,
                                         const int32_t* __restrict__ ptoken, int pid0, int p0, int np,
                                         size_t sub_el, float* __restrict__ f0, float* __restrict__ f1,
                                         const bf16_t* __restrict__ pa, const bf16_t* __restrict__ pb,
                                         uint32_t pbytes, bf16_t* __restrict__ out0, bf16_t* __restrict__ out1,
                                         int db0, ESG_LDS char* st0, ESG_LDS char* st1, ESG_LDS char* st2) {
  using C = Dw2<GSB, XS, NWD>;
  constexpr int NP = KIND == 0 ? 2 : 1;  // packed operand tiles per stage
  constexpr int L = KIND == 0 ? C::L0 : C::L1;
  constexpr int IXS = C::IXS;
  // row order within a stage: four waves use perm (positions 16w + 4q + i in
  // the rows of instruction i); eight waves keep positions in row order
  constexpr bool PERM = NWD == 4;
  const int lane = threadIdx.x & 63, w = wave_id();
  const uint32_t kbytes = (uint32_t)d * 2;
  const DmaSrc rz = make_dma_src(src, (uint32_t)tokens * kbytes);
  const DmaSrc rpa = make_dma_src(pa, pbytes);
  const DmaSrc rpb = make_dma_src(pb, pbytes);
  const int nk = np / 64;

  // gathered tile (x or dY): instruction i of wave w fills LDS rows
  // (w*IXS + i)*4 + q, q = lane/16, holding positions 16w + 4q + i (four
  // waves) or the rows' own positions (eight)
  const int q = lane >> 4;
  int jz[IXS];
#pragma unroll
  for (int i = 0; i < IXS; ++i) jz[i] = (lane & 15) ^ mn_swz<16>((w * IXS + i) * 4 + q);
  // packed tiles (dg / du / a rows of positions)
  uint32_t voffP[C::IP];
#pragma unroll
  for (int i = 0; i < C::IP; ++i) {
    const int R = (w * C::IP + i) * (64 / C::NCHP) + lane / C::NCHP;
    const int j = (lane % C::NCHP) ^ mn_swz<C::NCHP>(R);
    voffP[i] = (uint32_t)((sub_el + (size_t)(p0 + (PERM ? dw_perm(R) : R)) * GSB) * 2) + j * 16;
  }
  // The wave's 16 token ids of a tile come through the scalar unit (constant
  // address space: ptoken is not written while this kernel runs), so that
  // their wait is an lgkmcnt one, which every pipeline step performs anyway;
  // a vector load would make the compiler wait for every load in flight.
  // Lane group q takes ids 4q .. 4q+3.
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  typedef const __attribute__((address_space(4))) i32x4 cint4;
  struct IdBlock {
    i32x4 v[4];
  };
  // the wave's 64/NWD ids of a tile
  auto load_ids = [&](int kt) __attribute__((always_inline)) {
    const cint4* src = (const cint4*)(ptoken + pid0 + kt * 64 + w * (64 / NWD));
    IdBlock r;
#pragma unroll
    for (int i = 0; i < 16 / NWD; ++i) r.v[i] = src[i];
    return r;
  };
  IdBlock next_ids;  // ids of the next tile to issue, loaded one issue ahead
  if (nk > 0) next_ids = load_ids(0);
  auto issue = [&](ESG_LDS char* st, int kt) __attribute__((always_inline)) {
    const IdBlock r = next_ids;
    if (kt + 1 < nk) next_ids = load_ids(kt + 1);
    int tk[IXS];
#pragma unroll
    for (int c = 0; c < IXS; ++c) {
      if constexpr (PERM) {  // branch-free pick of r.v[q][c]
        const int lo = __builtin_amdgcn_ubfe(q, 0, 1) ? r.v[1][c] : r.v[0][c];
        const int hi = __builtin_amdgcn_ubfe(q, 0, 1) ? r.v[3][c] : r.v[2][c];
        tk[c] = q >= 2 ? hi : lo;
      } else {  // row (w*IXS + c)*4 + q holds position 8w + 4c + q: r.v[c][q]
        const int lo = __builtin_amdgcn_ubfe(q, 0, 1) ? r.v[c][1] : r.v[c][0];
        const int hi = __builtin_amdgcn_ubfe(q, 0, 1) ? r.v[c][3] : r.v[c][2];
        tk[c] = q >= 2 ? hi : lo;
      }
    }
#pragma unroll
    for (int x = 0; x < XS; ++x)  // 128-d sub-tile x: d from db0 + 128x
#pragma unroll
      for (int i = 0; i < IXS; ++i) {
        const int dx = db0 + x * 128 + jz[i] * 8;
        const bool ok = tk[i] >= 0 && dx < d;
        dma16(rz, st + x * C::X_SUB + (w * IXS + i) * 1024,
              ok ? (uint32_t)tk[i] * kbytes + (uint32_t)dx * 2 : kOOB);
      }
    const uint32_t kofs = (uint32_t)kt * 64 * GSB * 2;
#pragma unroll
    for (int i = 0; i < C::IP; ++i) dma16(rpa, st + C::X_BYTES + (w * C::IP + i) * 1024, voffP[i] + kofs);
    if constexpr (NP == 2) {
#pragma unroll
      for (int i = 0; i < C::IP; ++i)
        dma16(rpb, st + C::X_BYTES + C::P_BYTES + (w * C::IP + i) * 1024, voffP[i] + kofs);
    }
  };

  // kind 0: wave (wm, wn) = (d slice of DW/WM0, gate or up);
  // kind 1: wave (wm, wn) = (neuron half, d slice of DW/WN1)
  const int wm = KIND == 0 ? w % C::WM0 : w & 1;
  const int wn = KIND == 0 ? w / C::WM0 : w >> 1;
  constexpr int FM = KIND == 0 ? C::FM0 : C::FM1;
  constexpr int FN = KIND == 0 ? C::FN0 : C::FN1;
  f32x4 acc[FM][FN];
  zero_acc(acc);
  auto compute = [&](const ESG_LDS char* st, int) __attribute__((always_inline)) {
    uint4 a[2][FM], b[2][FN];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (KIND == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int dl = wm * (C::DW / C::WM0) + i * 16;  // d within the workgroup's DW
          a[kb][i] = frag_nrow<16>(st + (dl >> 7) * C::X_SUB, kb, dl & 127, lane);
        }
        const ESG_LDS char* tb = st + C::X_BYTES + wn * C::P_BYTES;
#pragma unroll
        for (int j = 0; j < FN; ++j) b[kb][j] = frag_nrow<C::NCHP>(tb, kb, j * 16, lane);
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
          a[kb][i] = frag_nrow<C::NCHP>(st + C::X_BYTES, kb, wm * (GSB / 2) + i * 16, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int dl = wn * (C::DW / C::WN1) + j * 16;
          b[kb][j] = frag_nrow<16>(st + (dl >> 7) * C::X_SUB, kb, dl & 127, lane);
        }
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma_bf16(acc[i][j], a[kb][i], b[kb][j]);
  };
  kloop<NS, L, 0>(nk, st0, st1, st2, issue, compute);

  if constexpr (KIND == 0) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int dd = db0 + wm * (C::DW / C::WM0) + i * 16 + (lane >> 4) * 4;
      if (dd >= d) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = j * 16 + (lane & 15);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][e];
        if (nb0 + n >= F) continue;
        const size_t o = (size_t)(nb0 + n) * d + dd;
        const size_t of = MODE == 4 ? (size_t)n * d + dd : o;
        store_dw<MODE>((wn == 0 ? out0 : out1) + o, (wn == 0 ? f0 : f1) + of, v);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int n = wm * (GSB / 2) + i * 16 + (lane >> 4) * 4;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int dd = db0 + wn * (C::DW / C::WN1) + j * 16 + (lane & 15);
        if (dd >= d) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][e];
        if (nb0 + n >= F) continue;
        const size_t o = (size_t)dd * F + nb0 + n;
        const size_t of = MODE == 4 ? (size_t)dd * GSB + n : o;
        store_dw<MODE>(out0 + o, f0 + of, v);
      }
    }
  }
}

}  // namespace tiles
}  // namespace esg
