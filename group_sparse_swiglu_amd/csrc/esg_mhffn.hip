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

}  // namespace

bool mhffn_supported(int tokens, int heads, int d_head, int subnets, int d_sub) {
  if (tokens < 0 || heads <= 0 || subnets <= 0 || d_sub <= 0) return false;
  if (d_head != MH_DH || d_sub % 8 || subnets > MH_MAXE) return false;
  const long long act = (long long)tokens * heads * d_head * 2;
  const long long w = (long long)heads * subnets * d_sub * d_head * 2;
  return act < (1ll << 31) && w < (1ll << 31);
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
