// LeakyReLU(0.5)-squared MLP with a stored activation gradient (parameter-golf
// pull request 1105, "1. Fused MLP Kernels": the forward fuses the up
// projection with the activation, the backward fuses (dy . W_down) with the
// product by the stored act_grad; A.7 gives d_model 512 and width 1792).
//
//   forward   pre = x . W_up^T (never stored); act_grad = pre > 0 ? 2 pre :
//             pre / 2; post = act_grad * pre / 2  -> post, act_grad (bf16)
//             y = post . W_down^T
//   backward  dpre = (dy . W_down) * act_grad       (product in the epilogue)
//             dx = dpre . W_up;  dW_up = dpre^T . x;  dW_down = dy^T . post
//
// Every product is one instance of a single MFMA tile: an output block of 256
// contiguous columns (q, the MFMA M side, so each lane's four accumulator rows
// are four consecutive output columns) by 128 rows (p, the MFMA N side), K in
// 64-wide steps through a three-stage direct-to-LDS pipeline.  Each operand
// comes in either as K-row tiles (K contiguous in memory: rows of x, W_up,
// W_down, post, dy, dpre) or as N-row tiles (q or p contiguous: W_down and
// W_up read along their other axis, and the token-major operands of the
// weight gradients).  Four waves each own 128 q x 64 p.  Output blocks are
// staged in LDS and written as whole rows of 16-byte stores.  The weight
// gradients contract over the tokens: the token range is split so that the
// grid fills the chip, each split writes an fp32 partial, and a second kernel
// adds the partials in split order (deterministic, no atomics).
#include <algorithm>

#include "esg_internal.hpp"
#include "esg_tiles.hpp"

namespace esg {
namespace {

using namespace tiles;

enum { KROW = 0, NROW = 1 };
enum { EPI_STORE = 0, EPI_ACT = 1, EPI_MUL = 2, EPI_PARTIAL = 3 };

constexpr int GP = 128, GK = 64;
constexpr int B_BYTES = GP * 128;  // 16 KB: K-row 128 x 128 B, or N-row 64 x 256 B

// Output tile TQ (256 or 128) columns x 128 rows.  256: three 48 KB stages,
// one 8-wave workgroup per compute unit, waves of 64 x 64.  128: two 32 KB
// stages, two 4-wave workgroups per compute unit (one's epilogue overlaps
// the other's loop), waves of 64 x 64.  Eight waves per CU either way: the
// direct-to-LDS loads of a CU go faster with more waves issuing them.
template <int TQ>
struct TileCfg {
  static constexpr int NS = TQ == 256 ? 3 : 2;
  static constexpr int OCC = TQ == 256 ? 1 : 2;
  static constexpr int NW = TQ == 256 ? 8 : 4;    // waves: NW/2 q slices x 2 p halves
  static constexpr int NTH = 64 * NW;
  static constexpr int A_BYTES = TQ * 128;  // K-row TQ x 128 B, or N-row TQ/128 x (64 x 256 B)
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int LDMA = STAGE / 1024 / NW;  // 1 KB DMA instructions per wave per stage
  static constexpr int HQ = TQ / (NW / 2);        // q columns per wave
  static constexpr int FM = HQ / 16;              // 16-wide q fragments per wave
};

struct GemmArgs {
  const bf16_t* a;  // KROW: [Q][K] (row stride lda); NROW: [K][Q]
  const bf16_t* b;  // KROW: [P][K]; NROW: [K][P]
  int lda, ldb;
  int Q, P, K;
  int k_split;      // K extent of one split (multiple of 64)
  int nq, np;       // q and p blocks
  int splits;       // K splits
  int nitems;       // work items of the persistent loop (tiles, plus empty ones for the XCD order)
  bf16_t* c0;       // [P][ldc] outputs (q contiguous)
  bf16_t* c1;
  int ldc;
  const bf16_t* aux;  // EPI_MUL: act_grad [P][ldc]
  float* part;        // EPI_PARTIAL: [splits][P][Q] fp32
};

// Direct-to-LDS addressing of one operand.  K-row: instruction covers 8 rows
// of 128 bytes, lane -> row lane/8, logical chunk (lane%8)^(row%8).  N-row:
// instruction covers 4 K rows of 256 bytes, lane -> row lane/16, logical
// chunk (lane%16)^swz(row).
template <int LAY, int ROWS, int NW>
struct OperandDma {
  static constexpr int NI = ROWS * 128 / 1024 / NW;  // instructions per wave per stage
  uint32_t base[NI];    // byte offset of this lane's chunk at K step 0 (kOOB: outside)
  uint32_t kstep;       // bytes to add per K step
  int koff[NI];         // K offset within a step: of the lane's chunk (K-row) or of its row (N-row)
  // r0: first tile row (K-row) or column (N-row); n: rows (K-row) or columns (N-row) of the operand
  __device__ __forceinline__ void init(int w, int lane, int r0, int n, int ld, int kbeg) {
    if constexpr (LAY == KROW) {
      const int c = (lane & 7) ^ (lane >> 3);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = r0 + (w * NI + i) * 8 + (lane >> 3);
        base[i] = r < n ? (uint32_t)r * ld * 2 + (uint32_t)(kbeg + c * 8) * 2 : kOOB;
        koff[i] = c * 8;
      }
      kstep = GK * 2;
    } else {
      // stage rows: ROWS/128 halves of 128 columns, 64 K rows each
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int ii = w * NI + i;           // 0 .. NW*NI-1
        const int half = ii / 16;            // 16 instructions per half (64 rows x 256 B)
        const int kr = (ii % 16) * 4 + (lane >> 4);
        const int j = (lane & 15) ^ mn_swz<16>(kr);
        const int col = r0 + half * 128 + j * 8;
        base[i] = col < n ? (uint32_t)(kbeg + kr) * ld * 2 + (uint32_t)col * 2 : kOOB;
        koff[i] = kr;
      }
      kstep = (uint32_t)GK * ld * 2;
    }
  }
  // lane offsets for K step kt; K positions at or past kend read zeros
  __device__ __forceinline__ void issue(const DmaSrc& src, ESG_LDS char* st, int w, int kt, int kbeg, int kend) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int k = kbeg + kt * GK + koff[i];
      const bool ok = base[i] != kOOB && k < kend;
      dma16(src, st + (w * NI + i) * 1024, ok ? base[i] + (uint32_t)kt * kstep : kOOB);
    }
  }
};

template <int LAY>
__device__ __forceinline__ uint4 frag(const ESG_LDS char* t, int rowbase, int kb, int lane) {
  if constexpr (LAY == KROW) {
    return frag_krow(t, rowbase + (lane & 15), kb * 4 + (lane >> 4));
  } else {
    return frag_nrow<16>(t + (rowbase >> 7) * (64 * 256), kb, rowbase & 127, lane);
  }
}

// One output tile (q block qb, p block pb, K split z).  Leaves the stages free
// for the next tile (all LDS reads done, every wave past a barrier).
template <int TQ, int AL, int BL, int EPI>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, int qb, int pb, int z, ESG_LDS char* st0,
                                          ESG_LDS char* st1, ESG_LDS char* st2) {
  using C = TileCfg<TQ>;
  const int lane = threadIdx.x & 63, w = wave_id();
  const int q0 = qb * TQ, p0 = pb * GP;
  const int kbeg = z * g.k_split;
  const int kend = min(g.K, kbeg + g.k_split);
  const int nk = (kend - kbeg + GK - 1) / GK;

  const DmaSrc ra = make_dma_src(g.a, AL == KROW ? (uint32_t)g.Q * g.lda * 2 : (uint32_t)g.K * g.lda * 2);
  const DmaSrc rb = make_dma_src(g.b, BL == KROW ? (uint32_t)g.P * g.ldb * 2 : (uint32_t)g.K * g.ldb * 2);
  OperandDma<AL, TQ, C::NW> da;
  OperandDma<BL, GP, C::NW> db;
  da.init(w, lane, q0, g.Q, g.lda, kbeg);
  db.init(w, lane, p0, g.P, g.ldb, kbeg);

  const int wm = w % (C::NW / 2), wn = w / (C::NW / 2);  // wave: q [wm*HQ, +HQ), p [wn*64, +64)
  constexpr int FM = C::FM, FN = 4, HQ = C::HQ;

  // EPI_MUL: the act_grad values of this lane's outputs, loaded before the K
  // loop (the first pipeline wait covers them)
  uint2 auxv[EPI == EPI_MUL ? FM : 1][EPI == EPI_MUL ? FN : 1];
  if constexpr (EPI == EPI_MUL) {
    const rsrc_t rx = make_rsrc(g.aux, (uint32_t)g.P * g.ldc * 2);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int q = q0 + wm * HQ + i * 16 + (lane >> 4) * 4;
        const int p = p0 + wn * 64 + j * 16 + (lane & 15);
        const uint32_t o = (q < g.Q && p < g.P) ? ((uint32_t)p * g.ldc + q) * 2 : kOOB;
        const v2i32 v = __builtin_amdgcn_raw_buffer_load_b64(rx, o, 0, 0);
        auxv[i][j] = make_uint2((uint32_t)v.x, (uint32_t)v.y);
      }
  }

  f32x4 acc[FM][FN];
  zero_acc(acc);
  auto issue = [&](ESG_LDS char* st, int kt) __attribute__((always_inline)) {
    da.issue(ra, st, w, kt, kbeg, kend);
    db.issue(rb, st + C::A_BYTES, w, kt, kbeg, kend);
  };
  auto compute = [&](const ESG_LDS char* st, int) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      uint4 a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = frag<AL>(st, wm * HQ + i * 16, kb, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = frag<BL>(st + C::A_BYTES, wn * 64 + j * 16, kb, lane);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) mma_bf16(acc[i][j], a[i], b[j]);
    }
  };
  kloop<C::NS, C::LDMA, 0>(nk, st0, st1, st2, issue, compute);
  wait_lgkm0();
  barrier();  // every wave is done with the stages

  if constexpr (EPI == EPI_PARTIAL) {
    float* out = g.part + (size_t)z * g.P * g.Q;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int q = q0 + wm * HQ + i * 16 + (lane >> 4) * 4;
        const int p = p0 + wn * 64 + j * 16 + (lane & 15);
        if (q < g.Q && p < g.P)
          *(float4*)(out + (size_t)p * g.Q + q) = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      }
  } else {
    using RS = RowStore<TQ, C::NTH>;
    const rsrc_t rc0 = make_rsrc(g.c0, (uint32_t)g.P * g.ldc * 2);
    uint32_t row_off[RS::IT];
#pragma unroll
    for (int it = 0; it < RS::IT; ++it) {
      const int p = p0 + RS::row(it, threadIdx.x);
      row_off[it] = p < g.P ? (uint32_t)p * g.ldc * 2 : kOOB;
    }
    ESG_LDS char* out0 = st0;  // rows 0..63 (TQ/4 KB)
    ESG_LDS char* out1 = st1;  // rows 64..127
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = acc[i][j][e];
          if constexpr (EPI == EPI_ACT) {
            const float ag = x > 0.0f ? 2.0f * x : 0.5f * x;
            v[e] = 0.5f * ag * x;  // post
          } else if constexpr (EPI == EPI_MUL) {
            const uint32_t word = e < 2 ? auxv[i][j].x : auxv[i][j].y;
            v[e] = x * bf16_to_f32((e & 1) ? (word >> 16) : (word & 0xffffu));
          } else {
            v[e] = x;
          }
        }
        RS::put(out0, out1, wn * 64 + j * 16 + (lane & 15), wm * HQ + i * 16 + (lane >> 4) * 4, v);
      }
    wait_lgkm0();
    barrier();
    RS::flush(out0, out1, rc0, row_off, q0, g.Q);
    if constexpr (EPI == EPI_ACT) {
      wait_lgkm0();
      barrier();  // the staged post block has been read
      const rsrc_t rc1 = make_rsrc(g.c1, (uint32_t)g.P * g.ldc * 2);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x = acc[i][j][e];
            v[e] = x > 0.0f ? 2.0f * x : 0.5f * x;  // act_grad
          }
          RS::put(out0, out1, wn * 64 + j * 16 + (lane & 15), wm * HQ + i * 16 + (lane >> 4) * 4, v);
        }
      wait_lgkm0();
      barrier();
      RS::flush(out0, out1, rc1, row_off, q0, g.Q);
    }
  }
  wait_lgkm0();
  barrier();  // staged output read by every wave: the stages are free again
}

// Persistent: each workgroup takes work items blockIdx.x, + gridDim.x, ... so
// that a tile's output stores drain while the next tile's operands stream in.
// Workgroups go to the 8 XCDs round-robin (and gridDim.x is a multiple of 8),
// so item t runs on XCD t % 8.  The order keeps operands that several tiles
// read in one XCD's L2: without splits, item t takes p block
// 8 * (t / 8 / nq) + t % 8 and q block (t / 8) % nq, so the nq tiles of one p
// block (same token rows) share an XCD; with splits, item t takes split
// t % splits, so with 8 splits each split's token range is read by one XCD.
template <int TQ, int AL, int BL, int EPI>
__global__ __launch_bounds__(TileCfg<TQ>::NTH, TileCfg<TQ>::OCC) void mlp_gemm_kernel(GemmArgs g) {
  using C = TileCfg<TQ>;
  __shared__ __attribute__((aligned(1024))) char stages_[C::NS * C::STAGE];
  for (int t = blockIdx.x; t < g.nitems; t += gridDim.x) {
    int qb, pb, z;
    if (g.splits > 1) {
      z = t % g.splits;
      const int r = t / g.splits;
      qb = r % g.nq;
      pb = r / g.nq;
    } else {
      z = 0;
      const int r = t >> 3;
      qb = r % g.nq;
      pb = (r / g.nq) * 8 + (t & 7);
      if (pb >= g.np) continue;
    }
    ESG_LDS char* st0 = (ESG_LDS char*)stages_;
    gemm_tile<TQ, AL, BL, EPI>(g, qb, pb, z, st0, st0 + C::STAGE, C::NS == 3 ? st0 + 2 * C::STAGE : st0);
  }
}

// out[p][q] = bf16(sum over splits s, in order, of part[s][p][q]); 4 per thread
__global__ void mlp_reduce_kernel(const float* __restrict__ part, int splits, size_t n4, bf16_t* __restrict__ out) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4; i += (size_t)gridDim.x * blockDim.x) {
    float4 s = ((const float4*)part)[i];
    for (int z = 1; z < splits; ++z) {
      const float4 v = ((const float4*)part)[(size_t)z * n4 + i];
      s.x += v.x;
      s.y += v.y;
      s.z += v.z;
      s.w += v.w;
    }
    ((uint2*)out)[i] = make_uint2(pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w));
  }
}

template <int TQ, int AL, int BL, int EPI>
hipError_t launch_gemm(const char* name, GemmArgs a, int splits, hipStream_t stream) {
  a.nq = (a.Q + TQ - 1) / TQ;
  a.np = (a.P + GP - 1) / GP;
  a.splits = splits;
  a.nitems = splits > 1 ? a.nq * a.np * splits : a.nq * 8 * ((a.np + 7) / 8);
  // TileCfg::OCC workgroups per compute unit, a multiple of 8
  const int slots = compute_units() * TileCfg<TQ>::OCC;
  const int blocks = std::min((a.nitems + 7) / 8 * 8, slots / 8 * 8);
  LaunchTimer timer(name, stream);
  hipLaunchKernelGGL((mlp_gemm_kernel<TQ, AL, BL, EPI>), dim3(blocks), dim3(TileCfg<TQ>::NTH), 0, stream, a);
  return hipGetLastError();
}

GemmArgs args(const bf16_t* A, int lda, const bf16_t* B, int ldb, int Q, int P, int K) {
  GemmArgs g{};
  g.a = A;
  g.b = B;
  g.lda = lda;
  g.ldb = ldb;
  g.Q = Q;
  g.P = P;
  g.K = K;
  g.k_split = K;
  return g;
}

// Token splits of a weight-gradient product: as many as keep every compute
// unit busy in one round of tiles (tiles * splits <= CUs, at most kMaxSplits),
// each split a whole number of 64-token steps.
constexpr int kMaxSplits = 16;
int dw_splits(int tokens, int tiles, int cus, int* k_split) {
  const int steps = (tokens + GK - 1) / GK;
  if (steps == 0) {  // no tokens: nothing to split
    *k_split = GK;
    return 1;
  }
  // one split per XCD when a split's tiles fit in one XCD, else fill the CUs
  int s = tiles <= cus / 8 ? 8 : std::min(kMaxSplits, std::max(1, cus / tiles));
  if (s > steps) s = steps;
  const int per = (steps + s - 1) / s;
  *k_split = per * GK;
  return (steps + per - 1) / per;
}

template <int TQ>
hipError_t weight_grad(const char* name, const bf16_t* A, int lda, const bf16_t* B, int ldb, int Q, int P,
                       int tokens, float* part, bf16_t* out, hipStream_t stream) {
  GemmArgs g = args(A, lda, B, ldb, Q, P, tokens);
  const int tiles = ((Q + TQ - 1) / TQ) * ((P + GP - 1) / GP);
  // the split count (and so the rounding of the sum) depends on the shape only
  const int splits = dw_splits(tokens, tiles, kNominalCUs * TileCfg<TQ>::OCC, &g.k_split);
  g.part = part;
  hipError_t e = launch_gemm<TQ, NROW, NROW, EPI_PARTIAL>(name, g, splits, stream);
  if (e != hipSuccess) return e;
  const size_t n4 = (size_t)P * Q / 4;
  LaunchTimer timer("mlp_dw_reduce", stream);
  const size_t blocks = std::min<size_t>((n4 + 255) / 256, 4096);
  hipLaunchKernelGGL(mlp_reduce_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, part, splits, n4, out);
  return hipGetLastError();
}

}  // namespace

// tile width per product (measured on the 86016 x 512 x 1792 workload)
constexpr int kUpTQ = 128, kDownTQ = 256, kDpreTQ = 128, kDxTQ = 256, kDwTQ = 128;

size_t mlp_partial_bytes(int tokens, int d_model, int d_ff) {
  // any device and tile width: at most kMaxSplits splits, each a whole 64-token step
  const size_t steps = ((size_t)tokens + GK - 1) / GK;
  const size_t splits = std::max<size_t>(1, std::min<size_t>(kMaxSplits, steps));
  return splits * d_model * d_ff * 4;
}

hipError_t launch_mlp_fwd(const void* xv, const void* w_upv, const void* w_downv, int tokens, int d, int F, void* yv,
                          void* postv, void* act_gradv, hipStream_t stream) {
  if (tokens == 0) return hipSuccess;
  const bf16_t *x = (const bf16_t*)xv, *w_up = (const bf16_t*)w_upv, *w_down = (const bf16_t*)w_downv;
  bf16_t *y = (bf16_t*)yv, *post = (bf16_t*)postv, *act_grad = (bf16_t*)act_gradv;
  // [post; act_grad]^T = epilogue(W_up . x^T): q = neuron, p = token, K = d
  GemmArgs g = args(w_up, d, x, d, F, tokens, d);
  g.c0 = post;
  g.c1 = act_grad;
  g.ldc = F;
  hipError_t e = launch_gemm<kUpTQ, KROW, KROW, EPI_ACT>("mlp_up_act", g, 1, stream);
  if (e != hipSuccess) return e;
  // y^T = W_down . post^T: q = d, p = token, K = F
  GemmArgs h = args(w_down, F, post, F, d, tokens, F);
  h.c0 = y;
  h.ldc = d;
  return launch_gemm<kDownTQ, KROW, KROW, EPI_STORE>("mlp_down", h, 1, stream);
}

hipError_t launch_mlp_bwd(const void* dyv, const void* xv, const void* w_upv, const void* w_downv, int tokens, int d,
                          int F, const void* postv, const void* act_gradv, void* dxv, void* dw_upv, void* dw_downv,
                          void* dprev, float* part, hipStream_t stream) {
  const bf16_t *dy = (const bf16_t*)dyv, *x = (const bf16_t*)xv, *w_up = (const bf16_t*)w_upv,
               *w_down = (const bf16_t*)w_downv, *post = (const bf16_t*)postv, *act_grad = (const bf16_t*)act_gradv;
  bf16_t *dx = (bf16_t*)dxv, *dw_up = (bf16_t*)dw_upv, *dw_down = (bf16_t*)dw_downv, *dpre = (bf16_t*)dprev;
  if (tokens > 0) {
    // dpre^T = (W_down^T . dy^T) * act_grad^T: q = neuron (W_down read along d), p = token, K = d
    GemmArgs g = args(w_down, F, dy, d, F, tokens, d);
    g.c0 = dpre;
    g.ldc = F;
    g.aux = act_grad;
    hipError_t e = launch_gemm<kDpreTQ, NROW, KROW, EPI_MUL>("mlp_dpre", g, 1, stream);
    if (e != hipSuccess) return e;
    // dx^T = W_up^T . dpre^T: q = d (W_up read along neurons), p = token, K = F
    GemmArgs h = args(w_up, d, dpre, F, d, tokens, F);
    h.c0 = dx;
    h.ldc = d;
    e = launch_gemm<kDxTQ, NROW, KROW, EPI_STORE>("mlp_dx", h, 1, stream);
    if (e != hipSuccess) return e;
  }
  // dW_down [d][F] = dy^T . post: q = neuron, p = d, K = tokens (both token-major)
  hipError_t e = weight_grad<kDwTQ>("mlp_dw_down", post, F, dy, d, F, d, tokens, part, dw_down, stream);
  if (e != hipSuccess) return e;
  // dW_up [F][d] = dpre^T . x: q = d, p = neuron, K = tokens
  return weight_grad<kDwTQ>("mlp_dw_up", x, d, dpre, F, d, F, tokens, part, dw_up, stream);
}

}  // namespace esg
