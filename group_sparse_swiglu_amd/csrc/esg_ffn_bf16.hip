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
#include "esg_internal.hpp"
#include "esg_pipe.hpp"

namespace esg {
namespace {

constexpr int NT = 256;
constexpr int BM = kTileRows;  // bucket positions per tile
constexpr int DB = 128;        // d rows per forward phase-2 block

typedef int v2i32 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void store8(rsrc_t r, uint32_t voff, const float (&v)[4]) {
  const v2i32 q = {(int)pack_bf16x2(v[0], v[1]), (int)pack_bf16x2(v[2], v[3])};
  __builtin_amdgcn_raw_buffer_store_b64(q, r, voff, 0, 0);
}

// Pipeline depth: 3 stages for 128-neuron blocks (one workgroup per CU), 2 for
// 64-neuron blocks so that two workgroups share a CU.
template <int GSB>
constexpr int stages_for() {
  return GSB >= 128 ? 3 : 2;
}

// ---------------------------------------------------------------------------
// Direct-to-LDS pipelines.  Tile t lands in buffer b = t % NS.
//   pre(b, t)              loads what issue(.., b, t) needs (E loads per
//                          lane), one step before tile t's loads are issued;
//   issue(stage, b, t)     enqueues tile t's loads (L per lane);
//   compute(stage, t, mid) consumes a landed tile and may end with S stores
//                          per lane; it calls mid() (the step's pre + issue)
//                          once, after issuing every LDS read of the stage
//                          that lacks alias information (the transposing
//                          reads), so the compiler never has to wait for the
//                          loads mid() starts before those reads.
// Each step waits for its own tile with the exact vmcnt the issue order
// implies (vector loads and stores retire in order).  The loop body has no
// branch around a wait: the steady state is an unrolled loop, first and last
// steps are peeled, and the buffer index handed to pre/issue is a constant at
// every call site.
// ---------------------------------------------------------------------------
#define ESG_MID(...) [&]() __attribute__((always_inline)) { __VA_ARGS__; }
#define ESG_HEAD(N) \
  wait_vmcnt<N>();  \
  wait_lgkm0();     \
  barrier()

// NS = 3, no stores in the loop: two tiles in flight ahead of the one
// consumed.  Step t: wait (tile t landed); barrier; compute(t) with
// mid = pre(t+3), issue(t+2).  Younger than tile t's loads are pre(t+2) and
// tile t+1's loads.
template <int L, int E, class Pre, class Issue, class Compute>
__device__ __forceinline__ void pipe3(int nk, ESG_LDS char* s0, ESG_LDS char* s1, ESG_LDS char* s2, Pre&& pre,
                                      Issue&& issue, Compute&& compute) {
  if (nk >= 6) {
    pre(0, 0);
    pre(1, 1);
    issue(s0, 0, 0);
    pre(2, 2);
    issue(s1, 1, 1);
    int t = 0;
    for (; t + 5 < nk; t += 3) {
      ESG_HEAD(L + E); compute(s0, t, ESG_MID(pre(0, t + 3); issue(s2, 2, t + 2)));
      ESG_HEAD(L + E); compute(s1, t + 1, ESG_MID(pre(1, t + 4); issue(s0, 0, t + 3)));
      ESG_HEAD(L + E); compute(s2, t + 2, ESG_MID(pre(2, t + 5); issue(s1, 1, t + 4)));
    }
    const int r = nk - t;  // 3, 4 or 5 steps left
    if (r == 3) {
      ESG_HEAD(L + E); compute(s0, t, ESG_MID(issue(s2, 2, t + 2)));
      ESG_HEAD(L); compute(s1, t + 1, ESG_MID());
      ESG_HEAD(0); compute(s2, t + 2, ESG_MID());
    } else if (r == 4) {
      ESG_HEAD(L + E); compute(s0, t, ESG_MID(pre(0, t + 3); issue(s2, 2, t + 2)));
      ESG_HEAD(L + E); compute(s1, t + 1, ESG_MID(issue(s0, 0, t + 3)));
      ESG_HEAD(L); compute(s2, t + 2, ESG_MID());
      ESG_HEAD(0); compute(s0, t + 3, ESG_MID());
    } else {
      ESG_HEAD(L + E); compute(s0, t, ESG_MID(pre(0, t + 3); issue(s2, 2, t + 2)));
      ESG_HEAD(L + E); compute(s1, t + 1, ESG_MID(pre(1, t + 4); issue(s0, 0, t + 3)));
      ESG_HEAD(L + E); compute(s2, t + 2, ESG_MID(issue(s1, 1, t + 4)));
      ESG_HEAD(L); compute(s0, t + 3, ESG_MID());
      ESG_HEAD(0); compute(s1, t + 4, ESG_MID());
    }
  } else {
    // short K: one tile at a time through buffers 0 and 1
    for (int t = 0; t < nk; ++t) {
      ESG_HEAD(0);
      if (t & 1) {
        pre(1, t);
        issue(s1, 1, t);
      } else {
        pre(0, t);
        issue(s0, 0, t);
      }
      ESG_HEAD(0);
      compute((t & 1) ? s1 : s0, t, ESG_MID());
    }
  }
}

// NS = 2: one tile in flight.  Step t: wait (tile t landed); barrier;
// compute(t) with mid = pre(t+2), issue(t+1), then its S stores.  pre(t+1)
// was issued before tile t's loads, so only the previous step's S stores are
// younger.
template <int S, class Pre, class Issue, class Compute>
__device__ __forceinline__ void pipe2(int nk, ESG_LDS char* s0, ESG_LDS char* s1, Pre&& pre, Issue&& issue,
                                      Compute&& compute) {
  if (nk >= 4) {
    pre(0, 0);
    pre(1, 1);
    issue(s0, 0, 0);
    ESG_HEAD(0); compute(s0, 0, ESG_MID(pre(0, 2); issue(s1, 1, 1)));
    int t = 1;
    for (; t + 3 < nk; t += 2) {
      ESG_HEAD(S); compute(s1, t, ESG_MID(pre(1, t + 2); issue(s0, 0, t + 1)));
      ESG_HEAD(S); compute(s0, t + 1, ESG_MID(pre(0, t + 3); issue(s1, 1, t + 2)));
    }
    const int r = nk - t;  // 2 or 3 steps left
    if (r == 2) {
      ESG_HEAD(S); compute(s1, t, ESG_MID(issue(s0, 0, t + 1)));
      ESG_HEAD(S); compute(s0, t + 1, ESG_MID());
    } else {
      ESG_HEAD(S); compute(s1, t, ESG_MID(pre(1, t + 2); issue(s0, 0, t + 1)));
      ESG_HEAD(S); compute(s0, t + 1, ESG_MID(issue(s1, 1, t + 2)));
      ESG_HEAD(S); compute(s1, t + 2, ESG_MID());
    }
  } else {
    for (int t = 0; t < nk; ++t) {
      ESG_HEAD(0);
      if (t & 1) {
        pre(1, t);
        issue(s1, 1, t);
      } else {
        pre(0, t);
        issue(s0, 0, t);
      }
      ESG_HEAD(0);
      compute((t & 1) ? s1 : s0, t, ESG_MID());
    }
  }
}

// K loop of a phase-1 GEMM (no stores inside) with NS stages.
template <int NS, int L, int E, class Pre, class Issue, class Compute>
__device__ __forceinline__ void run_kloop(int nk, ESG_LDS char* s0, ESG_LDS char* s1, ESG_LDS char* s2, Pre&& pre,
                                          Issue&& issue, Compute&& compute) {
  if constexpr (NS == 3)
    pipe3<L, E>(nk, s0, s1, s2, pre, issue, compute);
  else
    pipe2<0>(nk, s0, s1, pre, issue, compute);
}

struct NoPre {
  __device__ __forceinline__ void operator()(int, int) const {}
};

// ===========================================================================
// Forward
// ===========================================================================
template <int GSB>
struct Fwd2 {
  static constexpr int RA = 2 * GSB;           // weight rows per tile (gate, then up)
  static constexpr int A_BYTES = RA * 128;     // one 64-wide K stage
  static constexpr int B_BYTES = BM * 128;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int IA = RA / 32;           // DMA instructions per lane per stage (A)
  static constexpr int IB = BM / 32;           // (B)
  static constexpr int L = IA + IB;
  static constexpr int FMP = GSB / 32;         // gate/up fragment pairs per wave
  static constexpr int FN = 4;                 // 64 positions per wave
  static constexpr int KSUB = GSB / 64;        // 64-wide K sub-tiles of the group width
  static constexpr int ACT_BYTES = KSUB * BM * 128;
  static constexpr int W2_BYTES = KSUB * DB * 128;
  static constexpr int FM2 = 4, FN2 = 4;       // phase-2 wave tile 64 d x 64 positions
  static constexpr int STORES2 = FM2 * FN2;    // buffer stores per lane per d-block
  static_assert(ACT_BYTES <= STAGE && W2_BYTES <= STAGE, "phase-2 tiles reuse the stages");
};

template <int GSB>
__global__ __launch_bounds__(NT, GSB >= 128 ? 1 : 2) void fwd2_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wg, const bf16_t* __restrict__ wu,
    const bf16_t* __restrict__ wd, int tokens, int d, int F, int gs, const int32_t* __restrict__ tile_group,
    const int32_t* __restrict__ ptoken, uint32_t rows_total, bf16_t* __restrict__ hg_saved,
    bf16_t* __restrict__ hu_saved, bf16_t* __restrict__ partials) {
  using C = Fwd2<GSB>;
  constexpr int NS = stages_for<GSB>();
  // with two stages the third buffer only holds the second W_down tile
  __shared__ __attribute__((aligned(1024))) char st0_[C::STAGE], st1_[C::STAGE],
      st2_[NS == 3 ? C::STAGE : C::W2_BYTES];
  ESG_LDS char* st0 = (ESG_LDS char*)st0_;
  ESG_LDS char* st1 = (ESG_LDS char*)st1_;
  ESG_LDS char* st2 = (ESG_LDS char*)st2_;

  const int tile = blockIdx.x;
  const int g = tile_group[tile];
  if (g < 0) return;
  const int s = blockIdx.y;
  const int nb0 = g * gs + s * GSB;
  const int lane = threadIdx.x & 63, w = wave_id();
  const uint32_t prow0 = (uint32_t)tile * BM;
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
    voffA[i] = (uint32_t)grow * kbytes + c_lane * 16;
  }
  uint32_t voffB[C::IB];
#pragma unroll
  for (int i = 0; i < C::IB; ++i) {
    const int r = (w * C::IB + i) * 8 + (lane >> 3);
    const int t = ptoken[prow0 + r];
    voffB[i] = t >= 0 ? (uint32_t)t * kbytes + c_lane * 16 : kOOB;
  }
  auto issue = [&](ESG_LDS char* st, int, int kt) __attribute__((always_inline)) {
    const uint32_t kb = (uint32_t)kt * 128;
    const bool kin = kb + c_lane * 16 < kbytes;
#pragma unroll
    for (int i = 0; i < C::IA; ++i) {
      const bool gate = (w * C::IA + i) * 8 < GSB;  // wave-uniform
      dma16(gate ? rg : ru, st + (w * C::IA + i) * 1024, kin ? voffA[i] + kb : kOOB);
    }
#pragma unroll
    for (int i = 0; i < C::IB; ++i)
      dma16(rx, st + C::A_BYTES + (w * C::IB + i) * 1024, (kin && voffB[i] != kOOB) ? voffB[i] + kb : kOOB);
  };

  // ---- MFMA: wave (wm, wn) owns neurons [wm*GSB/2, +GSB/2) of gate and up, positions [wn*64, +64) ----
  const int wm = w & 1, wn = w >> 1;
  int arow[2 * C::FMP], brow[C::FN];
#pragma unroll
  for (int p = 0; p < C::FMP; ++p) {
    arow[p] = wm * (GSB / 2) + p * 16 + (lane & 15);
    arow[C::FMP + p] = GSB + arow[p];
  }
#pragma unroll
  for (int j = 0; j < C::FN; ++j) brow[j] = wn * 64 + j * 16 + (lane & 15);
  f32x4 acc[2 * C::FMP][C::FN];
  zero_acc(acc);
  auto compute = [&](const ESG_LDS char* st, int, auto&& mid) __attribute__((always_inline)) {
    mid();  // K-row reads only: the compiler tells the stages apart
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
  run_kloop<NS, C::L, 0>((int)((kbytes + 127) / 128), st0, st1, st2, NoPre{}, issue, compute);
  wait_lgkm0();
  barrier();  // every wave is done with the stages

  // ---- epilogue: hg, hu saved; a = SiLU(hg)*hu -> LDS K-row tile [position][neuron] ----
  ESG_LDS char* act = st0;
  const uint32_t sv_bytes = gridDim.y * rows_total * GSB * 2;
  const rsrc_t rsv_g = make_rsrc(hg_saved, sv_bytes);
  const rsrc_t rsv_u = make_rsrc(hu_saved, sv_bytes);
  const uint32_t sub_off = (uint32_t)s * rows_total * GSB * 2;
#pragma unroll
  for (int p = 0; p < C::FMP; ++p) {
    const int n = wm * (GSB / 2) + p * 16 + (lane >> 4) * 4;  // 4 consecutive neurons
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
      store8(rsv_g, so, hg);
      store8(rsv_u, so, hu);
      lds_write8(act + (n >> 6) * BM * 128 + krow_off(r, (n & 63) >> 3) + (n & 7) * 2, pack_bf16x2(a[0], a[1]),
                 pack_bf16x2(a[2], a[3]));
    }
  }

  // ---- phase 2: P^T = W_down[d-block, nb0 .. nb0+GSB) . a^T ----
  const DmaSrc rd = make_dma_src(wd, (uint32_t)d * F * 2);
  const rsrc_t rp = make_rsrc(partials, gridDim.y * rows_total * (uint32_t)d * 2);
  const uint32_t psub = (uint32_t)s * rows_total * d * 2;
  uint32_t voffW[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = (w * 4 + i) * 8 + (lane >> 3);
    voffW[i] = (uint32_t)r * F * 2 + (uint32_t)nb0 * 2 + c_lane * 16;
  }
  auto issueW = [&](ESG_LDS char* st, int, int blk) __attribute__((always_inline)) {
    const int db0 = blk * DB;
#pragma unroll
    for (int sb = 0; sb < C::KSUB; ++sb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (w * 4 + i) * 8 + (lane >> 3);
        const uint32_t off = db0 + r < d ? voffW[i] + (uint32_t)db0 * F * 2 + sb * 128 : kOOB;
        dma16(rd, st + sb * DB * 128 + (w * 4 + i) * 1024, off);
      }
  };
  int arow2[C::FM2], brow2[C::FN2];
  uint32_t pbase[C::FN2];
#pragma unroll
  for (int i = 0; i < C::FM2; ++i) arow2[i] = wm * 64 + i * 16 + (lane & 15);
#pragma unroll
  for (int j = 0; j < C::FN2; ++j) {
    brow2[j] = wn * 64 + j * 16 + (lane & 15);
    pbase[j] = ptoken[prow0 + brow2[j]] >= 0 ? psub + (prow0 + brow2[j]) * (uint32_t)d * 2 : kOOB;
  }
  auto compute2 = [&](const ESG_LDS char* cur, int blk, auto&& mid) __attribute__((always_inline)) {
    mid();
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
    const int db0 = blk * DB;
#pragma unroll
    for (int i = 0; i < C::FM2; ++i) {
      const int dd = db0 + wm * 64 + i * 16 + (lane >> 4) * 4;
#pragma unroll
      for (int j = 0; j < C::FN2; ++j) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc2[i][j][e];
        store8(rp, (pbase[j] != kOOB && dd < d) ? pbase[j] + dd * 2 : kOOB, v);
      }
    }
  };
  // st1 and st2 are free (the barrier above); the first step's full wait
  // covers the epilogue stores, and its barrier publishes the act tile
  pipe2<C::STORES2>((d + DB - 1) / DB, st1, st2, NoPre{}, issueW, compute2);
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
template <int GSB>
struct Dh2 {
  static constexpr int NCH = GSB / 8;            // 16-byte chunks per neuron row segment
  static constexpr int A_BYTES = 64 * GSB * 2;   // N-row: 64 d rows x GSB neurons
  static constexpr int B_BYTES = BM * 128;       // K-row: BM positions x 64 d
  static constexpr int STAGE1 = A_BYTES + B_BYTES;
  static constexpr int IA = NCH / 4;
  static constexpr int IB = BM / 32;
  static constexpr int L = IA + IB;
  static constexpr int FM = GSB / 32, FN = 4;    // wave tile GSB/2 neurons x 64 positions
  static constexpr int KSUB2 = 2 * GSB / 64;
  static constexpr int DGU_BYTES = KSUB2 * BM * 128;
  static constexpr int DB2 = 64;
  static constexpr int W2_BYTES = 2 * GSB * DB2 * 2;  // N-row: 2*GSB neuron rows x 64 d
  static constexpr int IW = 2 * GSB / 32;
  static constexpr int FM2 = 2, FN2 = 4;         // wave tile 32 d x 64 positions
  static constexpr int STORES2 = FM2 * FN2;
  static constexpr int STAGE = STAGE1 > W2_BYTES ? STAGE1 : W2_BYTES;
};

template <int GSB>
__global__ __launch_bounds__(NT, GSB >= 128 ? 1 : 2) void dhdx2_kernel(
    const bf16_t* __restrict__ dy, const bf16_t* __restrict__ wg, const bf16_t* __restrict__ wu,
    const bf16_t* __restrict__ wd, int tokens, int d, int F, int gs, const int32_t* __restrict__ tile_group,
    const int32_t* __restrict__ ptoken, uint32_t rows_total, const bf16_t* __restrict__ hg_saved,
    const bf16_t* __restrict__ hu_saved, bf16_t* __restrict__ dg_out, bf16_t* __restrict__ du_out,
    bf16_t* __restrict__ act_out, bf16_t* __restrict__ partials) {
  using C = Dh2<GSB>;
  constexpr int NS = stages_for<GSB>();
  __shared__ __attribute__((aligned(1024))) char st0_[C::STAGE], st1_[C::STAGE], st2_[NS == 3 ? C::STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char dgu_[C::DGU_BYTES];
  ESG_LDS char* st0 = (ESG_LDS char*)st0_;
  ESG_LDS char* st1 = (ESG_LDS char*)st1_;
  ESG_LDS char* st2 = (ESG_LDS char*)st2_;
  ESG_LDS char* dgu = (ESG_LDS char*)dgu_;

  const int tile = blockIdx.x;
  const int g = tile_group[tile];
  if (g < 0) return;
  const int s = blockIdx.y;
  const int nb0 = g * gs + s * GSB;
  const int lane = threadIdx.x & 63, w = wave_id();
  const uint32_t prow0 = (uint32_t)tile * BM;
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
    rowA[i] = row;
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
  auto issue = [&](ESG_LDS char* st, int, int kt) __attribute__((always_inline)) {
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
  const int wm = w & 1, wn = w >> 1;
  int brow[C::FN];
#pragma unroll
  for (int j = 0; j < C::FN; ++j) brow[j] = wn * 64 + j * 16 + (lane & 15);
  f32x4 acc[C::FM][C::FN];
  zero_acc(acc);
  auto compute = [&](const ESG_LDS char* st, int, auto&& mid) __attribute__((always_inline)) {
    uint4 a[2][C::FM], b[2][C::FN];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int c = kb * 4 + (lane >> 4);
#pragma unroll
      for (int i = 0; i < C::FM; ++i) a[kb][i] = frag_nrow<C::NCH>(st, kb, wm * (GSB / 2) + i * 16, lane);
#pragma unroll
      for (int j = 0; j < C::FN; ++j) b[kb][j] = frag_krow(st + C::A_BYTES, brow[j], c);
    }
    mid();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) mma_bf16(acc[i][j], a[kb][i], b[kb][j]);
  };
  run_kloop<NS, C::L, 0>((d + 63) / 64, st0, st1, st2, NoPre{}, issue, compute);

  // ---- epilogue: SiLU' ----
  const size_t sub_el = (size_t)s * rows_total * GSB;
#pragma unroll
  for (int i = 0; i < C::FM; ++i) {
    const int n = wm * (GSB / 2) + i * 16 + (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const int r = brow[j];
      const size_t q = sub_el + (size_t)(prow0 + r) * GSB + n;
      float hg[4], hu[4], dgv[4], duv[4], av[4];
      Quad<bf16_t>::load(hg_saved + q, hg);
      Quad<bf16_t>::load(hu_saved + q, hu);
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
  auto issueW = [&](ESG_LDS char* st, int, int blk) __attribute__((always_inline)) {
    const uint32_t db0 = (uint32_t)blk * C::DB2;
#pragma unroll
    for (int i = 0; i < C::IW; ++i) {
      const bool gate = (w * C::IW + i) * 8 < GSB;  // wave-uniform
      dma16(gate ? rg : ru, st + (w * C::IW + i) * 1024,
            db0 + jW[i] * 8 < (uint32_t)d ? voffW[i] + db0 * 2 : kOOB);
    }
  };
  uint32_t pbase[C::FN2];
#pragma unroll
  for (int j = 0; j < C::FN2; ++j)
    pbase[j] = ptoken[prow0 + brow[j]] >= 0 ? psub + (prow0 + brow[j]) * (uint32_t)d * 2 : kOOB;
  auto compute2 = [&](const ESG_LDS char* cur, int blk, auto&& mid) __attribute__((always_inline)) {
    constexpr int KB = 2 * GSB / 32;
    uint4 a[KB][C::FM2];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int i = 0; i < C::FM2; ++i) a[kb][i] = frag_nrow<8>(cur, kb, wm * 32 + i * 16, lane);
    mid();
    f32x4 acc2[C::FM2][C::FN2];
    zero_acc(acc2);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int c = (kb & 1) * 4 + (lane >> 4);
      uint4 b[C::FN2];
#pragma unroll
      for (int j = 0; j < C::FN2; ++j) b[j] = frag_krow(dgu + (kb >> 1) * BM * 128, brow[j], c);
#pragma unroll
      for (int i = 0; i < C::FM2; ++i)
#pragma unroll
        for (int j = 0; j < C::FN2; ++j) mma_bf16(acc2[i][j], a[kb][i], b[j]);
    }
    const int db0 = blk * C::DB2;
#pragma unroll
    for (int i = 0; i < C::FM2; ++i) {
      const int dd = db0 + wm * 32 + i * 16 + (lane >> 4) * 4;
#pragma unroll
      for (int j = 0; j < C::FN2; ++j) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc2[i][j][e];
        store8(rp, (pbase[j] != kOOB && dd < d) ? pbase[j] + dd * 2 : kOOB, v);
      }
    }
  };
  wait_lgkm0();
  barrier();  // all waves are done with the phase-1 stages
  pipe2<C::STORES2>((d + C::DB2 - 1) / C::DB2, st1, NS == 3 ? st2 : st0, NoPre{}, issueW, compute2);
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
template <int GSB>
struct Dw2 {
  static constexpr int NCHP = GSB / 8;           // chunks per position row of dg/du/a
  static constexpr int X_BYTES = 64 * 256;       // N-row: 64 positions x 128 d
  static constexpr int P_BYTES = 64 * GSB * 2;   // N-row: 64 positions x GSB neurons
  static constexpr int STAGE = X_BYTES + 2 * P_BYTES;
  static constexpr int IX = 4;
  static constexpr int IP = NCHP / 4;
  static constexpr int L0 = IX + 2 * IP, L1 = IX + IP;
  static constexpr int FM0 = 4, FN0 = GSB / 16;  // kind 0 wave tile: 64 d x GSB neurons
  static constexpr int FM1 = GSB / 32, FN1 = 4;  // kind 1 wave tile: GSB/2 neurons x 64 d
};

__device__ __forceinline__ int dw_perm(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

template <int GSB, int KIND, int NS>
__device__ __forceinline__ void dw2_body(const bf16_t* __restrict__ src, int tokens, int d, int F, int nb0,
                                         const int32_t* __restrict__ ptoken, int p0, int p1, size_t sub_el,
                                         const bf16_t* __restrict__ pa, const bf16_t* __restrict__ pb,
                                         uint32_t pbytes, bf16_t* __restrict__ out0, bf16_t* __restrict__ out1,
                                         int db0, ESG_LDS char* st0, ESG_LDS char* st1, ESG_LDS char* st2) {
  using C = Dw2<GSB>;
  constexpr int NP = KIND == 0 ? 2 : 1;  // packed operand tiles per stage
  constexpr int L = KIND == 0 ? C::L0 : C::L1;
  const int lane = threadIdx.x & 63, w = wave_id();
  const uint32_t kbytes = (uint32_t)d * 2;
  const DmaSrc rz = make_dma_src(src, (uint32_t)tokens * kbytes);
  const DmaSrc rpa = make_dma_src(pa, pbytes);
  const DmaSrc rpb = make_dma_src(pb, pbytes);
  const int nk = (p1 - p0) / 64;

  // gathered tile (x or dY): instruction i of wave w fills LDS rows
  // (w*4 + i)*4 + q, q = lane/16, holding positions 16w + 4q + i
  const int q = lane >> 4;
  int jz[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) jz[i] = (lane & 15) ^ mn_swz<16>((w * 4 + i) * 4 + q);
  // packed tiles (dg / du / a rows of positions)
  uint32_t voffP[C::IP];
#pragma unroll
  for (int i = 0; i < C::IP; ++i) {
    const int R = (w * C::IP + i) * (64 / C::NCHP) + lane / C::NCHP;
    const int j = (lane % C::NCHP) ^ mn_swz<C::NCHP>(R);
    voffP[i] = (uint32_t)((sub_el + (size_t)(p0 + dw_perm(R)) * GSB) * 2) + j * 16;
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
  IdBlock ib0, ib1, ib2;
  auto pre = [&](int b, int kt) __attribute__((always_inline)) {
    const cint4* src = (const cint4*)(ptoken + p0 + kt * 64 + w * 16);
    IdBlock r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = src[i];
    if (b == 0)
      ib0 = r;
    else if (b == 1)
      ib1 = r;
    else
      ib2 = r;
  };
  auto issue = [&](ESG_LDS char* st, int b, int kt) __attribute__((always_inline)) {
    const IdBlock& r = b == 0 ? ib0 : (b == 1 ? ib1 : ib2);
    int tk[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {  // branch-free pick of r.v[q][c]
      const int lo = __builtin_amdgcn_ubfe(q, 0, 1) ? r.v[1][c] : r.v[0][c];
      const int hi = __builtin_amdgcn_ubfe(q, 0, 1) ? r.v[3][c] : r.v[2][c];
      tk[c] = q >= 2 ? hi : lo;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bool ok = tk[i] >= 0 && db0 + jz[i] * 8 < d;
      dma16(rz, st + (w * 4 + i) * 1024, ok ? (uint32_t)tk[i] * kbytes + (uint32_t)db0 * 2 + jz[i] * 16 : kOOB);
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

  const int wm = w & 1, wn = w >> 1;
  constexpr int FM = KIND == 0 ? C::FM0 : C::FM1;
  constexpr int FN = KIND == 0 ? C::FN0 : C::FN1;
  f32x4 acc[FM][FN];
  zero_acc(acc);
  auto compute = [&](const ESG_LDS char* st, int, auto&& mid) __attribute__((always_inline)) {
    uint4 a[2][FM], b[2][FN];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (KIND == 0) {
#pragma unroll
        for (int i = 0; i < FM; ++i) a[kb][i] = frag_nrow<16>(st, kb, wm * 64 + i * 16, lane);
        const ESG_LDS char* tb = st + C::X_BYTES + wn * C::P_BYTES;
#pragma unroll
        for (int j = 0; j < FN; ++j) b[kb][j] = frag_nrow<C::NCHP>(tb, kb, j * 16, lane);
      } else {
#pragma unroll
        for (int i = 0; i < FM; ++i)
          a[kb][i] = frag_nrow<C::NCHP>(st + C::X_BYTES, kb, wm * (GSB / 2) + i * 16, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) b[kb][j] = frag_nrow<16>(st, kb, wn * 64 + j * 16, lane);
      }
    }
    mid();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma_bf16(acc[i][j], a[kb][i], b[kb][j]);
  };
  if (nk > 0) run_kloop<NS, L, 0>(nk, st0, st1, st2, pre, issue, compute);

  if constexpr (KIND == 0) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int dd = db0 + wm * 64 + i * 16 + (lane >> 4) * 4;
      if (dd >= d) continue;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = j * 16 + (lane & 15);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][e];
        Quad<bf16_t>::store((wn == 0 ? out0 : out1) + (size_t)(nb0 + n) * d + dd, v);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int n = wm * (GSB / 2) + i * 16 + (lane >> 4) * 4;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int dd = db0 + wn * 64 + j * 16 + (lane & 15);
        if (dd >= d) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][e];
        Quad<bf16_t>::store(out0 + (size_t)dd * F + nb0 + n, v);
      }
    }
  }
}

template <int GSB>
__global__ __launch_bounds__(NT, GSB >= 128 ? 1 : 2) void dw2_kernel(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ dy, int tokens, int d, int F, int gs, int nsub,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ ptoken, uint32_t rows_total,
    const bf16_t* __restrict__ dg, const bf16_t* __restrict__ du, const bf16_t* __restrict__ act,
    bf16_t* __restrict__ dwg, bf16_t* __restrict__ dwu, bf16_t* __restrict__ dwd) {
  using C = Dw2<GSB>;
  constexpr int NS = stages_for<GSB>();
  __shared__ __attribute__((aligned(1024))) char st0_[C::STAGE], st1_[C::STAGE], st2_[NS == 3 ? C::STAGE : 16];
  const int g = blockIdx.x / nsub, s = blockIdx.x % nsub;
  const int db0 = blockIdx.y * 128;
  const int nb0 = g * gs + s * GSB;
  const int p0 = tile_off[g] * BM, p1 = tile_off[g + 1] * BM;
  const size_t sub_el = (size_t)s * rows_total * GSB;
  const uint32_t pbytes = (uint32_t)(nsub * rows_total * GSB * 2);
  ESG_LDS char* st0 = (ESG_LDS char*)st0_;
  ESG_LDS char* st1 = (ESG_LDS char*)st1_;
  ESG_LDS char* st2 = (ESG_LDS char*)st2_;
  if (blockIdx.z == 0)
    dw2_body<GSB, 0, NS>(x, tokens, d, F, nb0, ptoken, p0, p1, sub_el, dg, du, pbytes, dwg, dwu, db0, st0, st1,
                         st2);
  else
    dw2_body<GSB, 1, NS>(dy, tokens, d, F, nb0, ptoken, p0, p1, sub_el, act, act, pbytes, dwd, dwd, db0, st0, st1,
                         st2);
}

// ===========================================================================
// Launchers
// ===========================================================================
template <int GSB>
hipError_t fwd2_t(const FfnShape& s, const void* x, const void* wg, const void* wu, const void* wd,
                  const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, void* hg, void* hu,
                  void* partials, hipStream_t stream) {
  LaunchTimer timer("fwd_grouped", stream);
  hipLaunchKernelGGL((fwd2_kernel<GSB>), dim3(ntiles_max, s.nsub()), dim3(NT), 0, stream, (const bf16_t*)x,
                     (const bf16_t*)wg, (const bf16_t*)wu, (const bf16_t*)wd, s.tokens, s.d_model, s.d_ff,
                     s.group_size, tile_group, ptoken, (uint32_t)ntiles_max * BM, (bf16_t*)hg, (bf16_t*)hu,
                     (bf16_t*)partials);
  return hipGetLastError();
}

template <int GSB>
hipError_t dhdx2_t(const FfnShape& s, const void* dy, const void* wg, const void* wu, const void* wd,
                   const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, const void* hg, const void* hu,
                   void* dg, void* du, void* act, void* partials, hipStream_t stream) {
  LaunchTimer timer("bwd_dh_dx", stream);
  hipLaunchKernelGGL((dhdx2_kernel<GSB>), dim3(ntiles_max, s.nsub()), dim3(NT), 0, stream, (const bf16_t*)dy,
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
  const dim3 grid(s.groups() * s.nsub(), (s.d_model + 127) / 128, 2);
  hipLaunchKernelGGL((dw2_kernel<GSB>), grid, dim3(NT), 0, stream, (const bf16_t*)x, (const bf16_t*)dy, s.tokens,
                     s.d_model, s.d_ff, s.group_size, s.nsub(), tile_off, ptoken, (uint32_t)rows_total,
                     (const bf16_t*)dg, (const bf16_t*)du, (const bf16_t*)act, (bf16_t*)dwg, (bf16_t*)dwu,
                     (bf16_t*)dwd);
  return hipGetLastError();
}

#undef ESG_MID
#undef ESG_HEAD

}  // namespace

bool bf16_pipelined(const FfnShape& s, int ntiles_max) {
  if (s.dtype != 1 || (s.gsb() != 64 && s.gsb() != 128)) return false;
  const unsigned long long lim = 1ull << 31;
  const unsigned long long rows = (unsigned long long)ntiles_max * BM;
  return (unsigned long long)s.tokens * s.d_model * 2 < lim && (unsigned long long)s.d_ff * s.d_model * 2 < lim &&
         (unsigned long long)s.nsub() * rows * s.d_model * 2 < lim &&
         (unsigned long long)s.nsub() * rows * s.gsb() * 2 < lim;
}

hipError_t launch_fwd2(const FfnShape& s, const void* x, const void* wg, const void* wu, const void* wd,
                       const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, void* hg_saved,
                       void* hu_saved, void* partials, hipStream_t stream) {
  if (ntiles_max == 0) return hipSuccess;
  return s.gsb() == 64 ? fwd2_t<64>(s, x, wg, wu, wd, tile_group, ptoken, ntiles_max, hg_saved, hu_saved, partials,
                                    stream)
                       : fwd2_t<128>(s, x, wg, wu, wd, tile_group, ptoken, ntiles_max, hg_saved, hu_saved, partials,
                                     stream);
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
