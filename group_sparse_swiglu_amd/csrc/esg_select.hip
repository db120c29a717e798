// Grouped top-k selection (eugen_sparse README, "What it does",
// grouped_topk_select): per token, the k groups with the largest
// sum over sampled gate rows of |SiLU(x . w_gate_row)|, plus the bias.
//
// One workgroup owns BM tokens.  The gate contraction over the sampled rows
// runs on MFMA over super-chunks of sampled rows held in registers; each
// super-chunk's |SiLU| values are staged in LDS and summed per (token, group)
// in column order into an fp32 energy table E[BM][G] that starts at the bias.
// The top-k is a wavefront rank test: lane g counts the groups that beat group
// g (higher score, or equal score and lower id), reading the other scores as
// broadcast LDS reads, for all of a wavefront's tokens in one pass; the group
// is selected when fewer than k beat it, and its output slot is its rank among
// the selected ids (a ballot prefix).  Every token's result depends only on
// its own row: batch invariant and bitwise reproducible.
#include <algorithm>
#include <type_traits>

#include "esg_device.hpp"
#include "esg_internal.hpp"
#include "esg_tiles.hpp"

namespace esg {
namespace {

constexpr int NT = 256;
constexpr int KC = 4;  // chunks per K stage
constexpr size_t kSelLds = 160 * 1024;
constexpr int kSel128Waves = 8;

// BM tokens per workgroup; each wave owns FNW 16-column fragments of a
// super-chunk of 4*FNW*16 sampled rows, interleaved across the waves, so the
// x tile is read once per super-chunk.
// bf16 with BM = 32, 64 or 128 streams both operands by direct-to-LDS loads
// into K-row tiles (64 K per stage, DMA_NS stages); other cases stage through
// registers.  Every workgroup streams all sampled rows once per K step, so a
// larger BM divides that traffic over more tokens.
// Eight waves (NW = 8): 64- and 128-token blocks keep four column groups and
// split their rows in two halves; 32-token blocks take eight column groups (the x
// tile's four load instructions then come from four waves, the other four
// issue an empty load into a sink so that every wave counts the same loads).
template <typename T, int BM, int FNW, bool USE_DMA = true, int NW = 4>
struct SelCfg {
  static constexpr int NTH = 64 * NW;
  static constexpr int CG = NW == 8 && BM == 32 ? 8 : 4;  // column groups
  static constexpr int RH = NW / CG;                        // row parts
  static constexpr int NSC = CG * FNW * 16;  // sampled rows per super-chunk
  static constexpr int FM = BM / 16;
  static constexpr int FMW = FM / RH;        // row fragments per wave
  static constexpr bool DMA = USE_DMA && std::is_same<T, bf16_t>::value && (BM == 32 || BM == 64 || BM == 128) &&
                              FNW <= 4;
  static constexpr int IA = BM >= 8 * NW ? BM / (8 * NW) : 1;  // x load instructions per lane per stage
  static constexpr int IB = NSC / (8 * NW);
  static constexpr int SINK = BM < 8 * NW ? 1024 : 0;  // where the empty x loads land
  static_assert(NW == 4 || (DMA && IB * 8 * NW == NSC && (IA * 8 * NW == BM || (IA == 1 && BM % 8 == 0))),
                "eight waves: whole DMA loads");
  static constexpr int PA = Plane<BM>::BYTES;
  static constexpr int PB = Plane<NSC>::BYTES;
  static constexpr int A_BYTES = DMA ? BM * 128 : KC * PA;
  static constexpr int B_BYTES = DMA ? NSC * 128 : KC * PB;
  static constexpr int DMA_NS = 3 * (A_BYTES + B_BYTES + SINK) <= 120 * 1024 ? 3 : 2;
  static constexpr int DMA_L = IA + IB;  // loads per lane per stage
  static constexpr int STAGES = (DMA ? DMA_NS : 2) * (A_BYTES + B_BYTES + SINK);
  static constexpr int S_STRIDE = NSC + 1;  // odd float stride: conflict-free column walks
  static constexpr int S_BYTES = BM * S_STRIDE * 4;
  static constexpr int FIXED = STAGES > S_BYTES ? STAGES : S_BYTES;
};

// |SiLU| of one super-chunk's accumulators into S, then per (token, group)
// sums over the super-chunk's columns, in column order, added to E.
template <class C, int FMW, int FNW>
__device__ __forceinline__ void select_energy(const f32x4 (&acc)[FMW][FNW], float* S, float* E, int ES, int n0,
                                              int ncols, int rpg, int groups, int lane, const int (&brow)[FNW],
                                              int rh) {
  constexpr int BM = C::FM * 16;
#pragma unroll
  for (int i = 0; i < FMW; ++i)
#pragma unroll
    for (int j = 0; j < FNW; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = (rh * FMW + i) * 16 + (lane >> 4) * 4 + e;
        const float h = acc[i][j][e];
        S[r * C::S_STRIDE + brow[j]] = fabsf(h * sigmoid_f(h));
      }
  __syncthreads();
  const int g_lo = n0 / rpg;
  const int g_hi = min(groups - 1, (min(n0 + C::NSC, ncols) - 1) / rpg);
  const int ng = g_hi - g_lo + 1;
  for (int p = threadIdx.x; p < BM * ng; p += C::NTH) {
    const int r = p % BM, g = g_lo + p / BM;
    const int c0 = max(n0, g * rpg) - n0, c1 = min(n0 + C::NSC, (g + 1) * rpg) - n0;
    float sum = E[r * ES + g];
    for (int c = c0; c < c1; ++c) sum += S[r * C::S_STRIDE + c];
    E[r * ES + g] = sum;
  }
}

// Scores are compared through an order-preserving integer key: for every
// non-NaN pair of scores a > b exactly when key(a) > key(b), and -0 and +0 map
// to the same key; a NaN with its sign bit clear ranks above +inf.
__device__ __forceinline__ uint32_t score_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Top-k of the BM tokens whose scores are E[r * ES + g] (LDS, complete: the
// caller synchronised after writing them), written to idx_out in ascending
// group id; per-group counts through the LDS table cnt (zeroed by the caller)
// when counts is given.  NW waves.  E is turned into keys in place.
template <int BM, int NW = 4>
__device__ __forceinline__ void rank_topk(float* E, int ES, int* cnt, int t0, int tokens, int groups, int k,
                                          int32_t* __restrict__ idx_out, int32_t* __restrict__ counts) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* const Kt = (uint32_t*)E;
  for (int i = tid; i < BM * ES; i += 64 * NW) Kt[i] = score_key(E[i]);
  __syncthreads();
  // group g is selected when fewer than k groups beat it (higher score, or
  // equal score and lower id), i.e. it is among the k first in the order
  // (score descending, id ascending); its output slot is its rank among the
  // selected ids (a ballot prefix)
  const uint64_t lt = (1ull << lane) - 1ull;
  if (groups <= 32) {
    // the two half-waves rank two tokens at a time: lane l holds group l % 32
    // of token half l / 32; a token's other scores are broadcast reads
    constexpr int TPW = BM / (2 * NW);  // token pairs per wave
    const int hf = lane >> 5, g = lane & 31;
    uint32_t sg[TPW];
    int beat[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int r = wave + NW * (2 * i + hf);
      sg[i] = g < groups ? Kt[r * ES + g] : 0u;
      beat[i] = 0;
    }
    for (int q = 0; q < groups; ++q) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const uint32_t sq = Kt[(wave + NW * (2 * i + hf)) * ES + q];
        beat[i] += (sq > sg[i]) || (sq == sg[i] && q < g);
      }
    }
    const uint64_t half = hf ? 0xffffffff00000000ull : 0x00000000ffffffffull;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = t0 + wave + NW * (2 * i + hf);
      const bool sel = g < groups && beat[i] < k;
      const uint64_t m = __ballot(sel) & half;
      const int pos = __popcll(m & lt);
      if (t < tokens && sel && pos < k) {
        idx_out[(size_t)t * k + pos] = g;
        if (counts) atomicAdd(&cnt[g], 1);
      }
    }
  } else if (groups <= 64) {
    // lane g holds group g of the wave's BM/NW tokens at once; every other
    // group's score comes as a broadcast LDS read (same address in all lanes)
    constexpr int TPW = BM / NW;
    uint32_t sg[TPW];
    int beat[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      sg[i] = lane < groups ? Kt[(wave + NW * i) * ES + lane] : 0u;
      beat[i] = 0;
    }
    for (int q = 0; q < groups; ++q) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
        const uint32_t sq = Kt[(wave + NW * i) * ES + q];
        beat[i] += (sq > sg[i]) || (sq == sg[i] && q < lane);
      }
    }
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = t0 + wave + NW * i;
      const bool sel = lane < groups && beat[i] < k;
      const uint64_t m = __ballot(sel);
      const int pos = __popcll(m & lt);
      if (t < tokens && sel && pos < k) {
        idx_out[(size_t)t * k + pos] = lane;
        if (counts) atomicAdd(&cnt[lane], 1);
      }
    }
  } else if (groups <= 256) {
    // one token per wave at a time; lane l holds the keys of groups l, l+64,
    // l+128, l+192.  The key of the k-th group in the order is found bit by
    // bit from the top (a radix select: per bit, a ballot count of the keys
    // that match the bits found so far and have this bit set); the groups
    // above it are selected and, of the groups equal to it, the lowest ids
    // fill the remaining slots.
    for (int r = wave; r < BM; r += NW) {
      const int t = t0 + r;
      if (t >= tokens) break;
      const uint32_t* row = Kt + r * ES;
      uint32_t key[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) key[c] = c * 64 + lane < groups ? row[c * 64 + lane] : 0u;
      uint32_t pre = 0;  // the bits of the k-th key found so far
      int need = k;      // its position among the keys that match them
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t hi = ~0u << bit, cand = pre | (1u << bit);
        int n = 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          if (c * 64 >= groups) break;  // wave-uniform
          n += __popcll(__ballot(c * 64 + lane < groups && (key[c] & hi) == cand));
        }
        if (n >= need) pre = cand;
        else need -= n;
      }
      int base = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        if (c * 64 >= groups) break;  // wave-uniform
        const int g = c * 64 + lane;
        uint64_t eq = __ballot(g < groups && key[c] == pre), take = 0;
        for (; need > 0 && eq != 0; --need) {  // the lowest ids among the equal keys
          const uint64_t low = eq & (~eq + 1ull);
          take |= low;
          eq ^= low;
        }
        const bool sel = g < groups && (key[c] > pre || ((take >> lane) & 1ull));
        const uint64_t m = __ballot(sel);
        const int pos = base + __popcll(m & lt);
        if (sel) {
          idx_out[(size_t)t * k + pos] = g;
          if (counts) atomicAdd(&cnt[g], 1);
        }
        base += __popcll(m);
      }
    }
  } else {
    for (int r = wave; r < BM; r += NW) {
      const int t = t0 + r;
      if (t >= tokens) break;
      const uint32_t* row = Kt + r * ES;
      int base = 0;
      for (int g0 = 0; g0 < groups; g0 += 64) {
        const int g = g0 + lane;
        bool sel = false;
        if (g < groups) {
          const uint32_t sg = row[g];
          int beat = 0;
          for (int q = 0; q < groups; ++q) {
            const uint32_t sq = row[q];
            beat += (sq > sg) || (sq == sg && q < g);
          }
          sel = beat < k;
        }
        const uint64_t m = __ballot(sel);
        const int pos = base + __popcll(m & lt);
        if (sel && pos < k) {
          idx_out[(size_t)t * k + pos] = g;
          if (counts) atomicAdd(&cnt[g], 1);
        }
        base += __popcll(m);
      }
    }
  }
  if (counts) {
    __syncthreads();
    for (int g = tid; g < groups; g += 64 * NW)
      if (cnt[g]) atomicAdd(&counts[g], cnt[g]);
  }
}

template <typename T, int BM, int FNW, bool USE_DMA, int NW>
__global__ __launch_bounds__(64 * NW) void select_kernel(const T* __restrict__ x, const T* __restrict__ wg,
                                                     int tokens, int d_model, int d_ff, int groups, int k,
                                                     const int32_t* __restrict__ sub, int rpg,
                                                     const float* __restrict__ bias,
                                                     int32_t* __restrict__ idx_out,
                                                     int32_t* __restrict__ counts, int gpc,
                                                     float* __restrict__ e_out) {
  using C = SelCfg<T, BM, FNW, USE_DMA, NW>;
  static_assert(NW == 4 || C::DMA, "the register-staged path runs four waves");
  extern __shared__ __align__(16) char smem[];
  auto la = [&](int i_) -> char* { return smem + i_ * C::A_BYTES; };
  auto lb = [&](int i_) -> char* { return smem + 2 * C::A_BYTES + i_ * C::B_BYTES; };
  float* S = (float*)smem;                     // aliases the stage buffers after each K loop
  const int ES = groups | 1;                   // odd row stride of the energy table
  float* E = (float*)(smem + C::FIXED);        // [BM][ES]
  int* cnt = (int*)(E + BM * ES);              // [groups]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = blockIdx.x * BM;
  // this workgroup's groups [g_begin, g_end) and sampled columns [c_begin, ncols)
  const int g_begin = blockIdx.y * gpc, g_end = min(groups, g_begin + gpc);
  const int c_begin = g_begin * rpg, ncols = g_end * rpg;
  const int kbytes = d_model * (int)sizeof(T);
  const int nk = (kbytes + KC * 16 - 1) / (KC * 16);

  // every row of the score table starts at the bias: one load per column
  for (int g = tid; g < ES; g += C::NTH) {
    const float b = (bias != nullptr && g < groups) ? bias[g] : 0.0f;
#pragma unroll 8
    for (int r = 0; r < BM; ++r) E[r * ES + g] = b;
  }
  for (int i = tid; i < groups; i += C::NTH) cnt[i] = 0;

  // wave -> column group cg (FNW fragments interleaved over the CG groups)
  // and row part rh
  const int cg = wave % C::CG, rh = wave / C::CG;
  int arow[C::FMW], brow[FNW];
#pragma unroll
  for (int i = 0; i < C::FMW; ++i) arow[i] = (rh * C::FMW + i) * 16 + (lane & 15);
#pragma unroll
  for (int j = 0; j < FNW; ++j) brow[j] = (j * C::CG + cg) * 16 + (lane & 15);

  if constexpr (C::DMA) {
    ESG_LDS char* st0 = (ESG_LDS char*)smem;
    const DmaSrc rx = make_dma_src(x, (uint32_t)tokens * kbytes);
    const DmaSrc rwg = make_dma_src(wg, (uint32_t)d_ff * kbytes);
    const int w = wave_id();
    const int c_lane = (lane & 7) ^ (lane >> 3);
    uint32_t voffA[C::IA];
#pragma unroll
    for (int i = 0; i < C::IA; ++i) {
      const int xr = (w * C::IA + i) * 8 + (lane >> 3);  // rows >= BM: an empty load into the sink
      voffA[i] = xr < BM && t0 + xr < tokens ? (uint32_t)(t0 + xr) * kbytes + c_lane * 16 : kOOB;
    }
    constexpr int IB = C::IB;
    for (int n0 = c_begin; n0 < ncols; n0 += C::NSC) {
      uint32_t voffB[IB];
#pragma unroll
      for (int i = 0; i < IB; ++i) {
        const int col = n0 + (w * IB + i) * 8 + (lane >> 3);
        const int row = col < ncols ? (sub ? sub[col] : col) : -1;
        voffB[i] = row >= 0 ? (uint32_t)row * kbytes + c_lane * 16 : kOOB;
      }
      auto issue = [&](ESG_LDS char* st, int kt) __attribute__((always_inline)) {
        const uint32_t kb = (uint32_t)kt * 128;
        const bool kin = kb + c_lane * 16 < (uint32_t)kbytes;
#pragma unroll
        for (int i = 0; i < C::IA; ++i) {
          const bool real = (w * C::IA + i) * 8 < BM;  // wave-uniform
          dma16(rx, real ? st + (w * C::IA + i) * 1024 : st + C::A_BYTES + C::B_BYTES,
                (kin && voffA[i] != kOOB) ? voffA[i] + kb : kOOB);
        }
#pragma unroll
        for (int i = 0; i < IB; ++i)
          dma16(rwg, st + C::A_BYTES + (w * IB + i) * 1024, (kin && voffB[i] != kOOB) ? voffB[i] + kb : kOOB);
      };
      f32x4 acc[C::FMW][FNW];
      zero_acc(acc);
      auto compute = [&](const ESG_LDS char* st, int) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int cc = kb * 4 + (lane >> 4);
          uint4 a[C::FMW], b[FNW];
#pragma unroll
          for (int i = 0; i < C::FMW; ++i) a[i] = frag_krow(st, arow[i], cc);
#pragma unroll
          for (int j = 0; j < FNW; ++j) b[j] = frag_krow(st + C::A_BYTES, brow[j], cc);
#pragma unroll
          for (int i = 0; i < C::FMW; ++i)
#pragma unroll
            for (int j = 0; j < FNW; ++j) mma_bf16(acc[i][j], a[i], b[j]);
        }
      };
      wait_lgkm0();
      barrier();  // the previous super-chunk's S reads (S aliases the stages) are done
      constexpr int SB = C::A_BYTES + C::B_BYTES + C::SINK;
      tiles::kloop<C::DMA_NS, C::DMA_L, 0>((kbytes + 127) / 128, st0, st0 + SB, st0 + 2 * SB, issue, compute);
      wait_lgkm0();
      barrier();  // every wave is done with the stages before S overwrites them
      select_energy<C>(acc, S, E, ES, n0, ncols, rpg, groups, lane, brow, rh);
    }
  } else {
  RowKLoader<BM, KC, NT> ldA;
  ldA.init(tid, [&](int r) -> const char* {
    const int t = t0 + r;
    return t < tokens ? (const char*)(x + (size_t)t * d_model) : nullptr;
  });
  for (int n0 = c_begin; n0 < ncols; n0 += C::NSC) {
    RowKLoader<C::NSC, KC, NT> ldB;
    ldB.init(tid, [&](int r) -> const char* {
      const int col = n0 + r;
      if (col >= ncols) return nullptr;
      const int row = sub ? sub[col] : col;  // without a subsample the columns are all gate rows
      return (const char*)(wg + (size_t)row * d_model);
    });
    f32x4 acc[C::FM][FNW];
    zero_acc(acc);
    ldA.load(0, kbytes);
    ldB.load(0, kbytes);
    __syncthreads();  // previous super-chunk's S reads and the E init are done
    ldA.store(la(0));
    ldB.store(lb(0));
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) {
        ldA.load((kt + 1) * KC * 16, kbytes);
        ldB.load((kt + 1) * KC * 16, kbytes);
      }
      mma_lds<T, C::FM, FNW, KC, C::PA, C::PB>(acc, la(kt & 1), lb(kt & 1), arow, brow, lane);
      if (kt + 1 < nk) {
        ldA.store(la((kt + 1) & 1));
        ldB.store(lb((kt + 1) & 1));
      }
      __syncthreads();
    }
    select_energy<C>(acc, S, E, ES, n0, ncols, rpg, groups, lane, brow, rh);
    // the next super-chunk's first __syncthreads orders these before S is reused
  }
  }
  __syncthreads();

  // energies only: the ranking runs in select_rank_kernel over the whole table
  if (e_out != nullptr) {
    for (int p = tid; p < BM * (g_end - g_begin); p += C::NTH) {
      const int r = p / (g_end - g_begin), g = g_begin + p % (g_end - g_begin);
      if (t0 + r < tokens) e_out[(size_t)(t0 + r) * groups + g] = E[r * ES + g];
    }
    return;
  }
  rank_topk<BM, NW>(E, ES, cnt, t0, tokens, groups, k, idx_out, counts);
}

// Top-k from an energy table e_in [tokens, groups] (bias included) written by
// energy-only launches of select_kernel: BM tokens per workgroup.
template <int BM>
__global__ __launch_bounds__(NT) void select_rank_kernel(const float* __restrict__ e_in, int tokens, int groups,
                                                          int k, int32_t* __restrict__ idx_out,
                                                          int32_t* __restrict__ counts) {
  extern __shared__ __align__(16) char smem[];
  const int ES = groups | 1;
  float* E = (float*)smem;        // [BM][ES]
  int* cnt = (int*)(E + BM * ES);  // [groups]
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * BM;
  for (int i = tid; i < groups; i += NT) cnt[i] = 0;
  // the block's rows are one contiguous run of the table: all loads in flight
  // before the stores (8 per thread per batch)
  const int n = BM * groups;
  for (int p0 = 0; p0 < n; p0 += 8 * NT) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * NT + tid;
      v[u] = p < n && t0 + p / groups < tokens ? e_in[(size_t)t0 * groups + p] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * NT + tid;
      if (p < n) E[(p / groups) * ES + p % groups] = v[u];
    }
  }
  __syncthreads();
  rank_topk<BM>(E, ES, cnt, t0, tokens, groups, k, idx_out, counts);
}

struct SelArgs {
  const void* x;
  const void* wg;
  int tokens, d_model, d_ff, groups, k;
  const int32_t* sub;
  int rpg;
  const float* bias;
  int32_t* idx;
  int32_t* counts;
};

// gpc groups per workgroup along y; e_out != NULL: energies only (no ranking).
template <typename T, int BM, int FNW, bool USE_DMA, int NW>
hipError_t launch_select_v(const SelArgs& a, int gpc, float* e_out, hipStream_t stream) {
  using C = SelCfg<T, BM, FNW, USE_DMA, NW>;
  const size_t smem = C::FIXED + (size_t)BM * (a.groups | 1) * 4 + (size_t)a.groups * 4;
  static const hipError_t attr = hipFuncSetAttribute((const void*)select_kernel<T, BM, FNW, USE_DMA, NW>,
                                                     hipFuncAttributeMaxDynamicSharedMemorySize, kSelLds);
  if (attr != hipSuccess) return attr;
  const dim3 grid((a.tokens + BM - 1) / BM, (a.groups + gpc - 1) / gpc);
  LaunchTimer timer("select", stream);
  hipLaunchKernelGGL((select_kernel<T, BM, FNW, USE_DMA, NW>), grid, dim3(C::NTH), smem, stream, (const T*)a.x,
                     (const T*)a.wg, a.tokens, a.d_model, a.d_ff, a.groups, a.k, a.sub, a.rpg, a.bias,
                     e_out ? nullptr : a.idx, e_out ? nullptr : a.counts, gpc, e_out);
  return hipGetLastError();
}

// The direct-to-LDS path addresses x and w_gate through 32-bit buffer offsets.
// (the register-staged fallback keeps BM = 32 and four waves)
template <typename T, int BM, int FNW, int NW = 4>
hipError_t launch_select_t(const SelArgs& a, hipStream_t stream, int gpc = 0, float* e_out = nullptr) {
  if (gpc <= 0) gpc = a.groups;
  const unsigned long long kb = (unsigned long long)a.d_model * sizeof(T);
  if ((unsigned long long)a.tokens * kb < (1ull << 31) && (unsigned long long)a.d_ff * kb < (1ull << 31))
    return launch_select_v<T, BM, FNW, true, NW>(a, gpc, e_out, stream);
  return launch_select_v<T, (BM < 32 ? BM : 32), FNW, false, 4>(a, gpc, e_out, stream);
}

// Fragments per wave: the choice with the least padded MFMA work (ties: wider).
int pick_fnw(int ncols) {
  int best = 8;
  long long best_work = -1;
  for (int f : {8, 6, 4, 2}) {
    const long long nsc = 64LL * f;
    const long long work = (ncols + nsc - 1) / nsc * nsc;
    if (best_work < 0 || work < best_work) {
      best_work = work;
      best = f;
    }
  }
  return best;
}

// Batches of fewer 32-token blocks than CUs, given an energy table: the groups
// are split over workgroups (about two per CU), each writing its groups'
// energies, and a second launch ranks.  Every sampled column's dot product and
// every group's sum run in the same order as in the one-launch path, so the
// selection is bitwise the same.
template <typename T>
hipError_t select_split(const SelArgs& a, float* ews, hipStream_t st) {
  const int blocks = (a.tokens + 31) / 32;
  const int want = std::max(1, (2 * compute_units() + blocks - 1) / blocks);
  const int chunks0 = std::min(a.groups, want);
  // at most 128 sampled rows per workgroup (one super-chunk of the small-stage
  // configuration, two workgroups per CU)
  const int gpc = std::min((a.groups + chunks0 - 1) / chunks0, std::max(1, 128 / a.rpg));
  const int cols = gpc * a.rpg;  // sampled columns per workgroup
  hipError_t e;
  if (std::is_same<T, bf16_t>::value)
    e = cols > 128 && cols <= 256 ? launch_select_t<T, 32, 4>(a, st, gpc, ews)
        : cols <= 64              ? launch_select_t<T, 32, 1>(a, st, gpc, ews)  // fewer empty loads
                                  : launch_select_t<T, 32, 2>(a, st, gpc, ews);
  else
    switch (pick_fnw(cols)) {
      case 2: e = launch_select_t<T, 32, 2>(a, st, gpc, ews); break;
      case 4: e = launch_select_t<T, 32, 4>(a, st, gpc, ews); break;
      case 6: e = launch_select_t<T, 32, 6>(a, st, gpc, ews); break;
      default: e = launch_select_t<T, 32, 8>(a, st, gpc, ews); break;
    }
  if (e != hipSuccess) return e;
  // ranking in 8-token workgroups: four times the workgroups of the 32-token
  // blocks, two tokens (or one pair) per wave
  constexpr int RBM = 8;
  LaunchTimer timer("select_rank", st);
  const size_t smem = (size_t)RBM * (a.groups | 1) * 4 + (size_t)a.groups * 4;
  hipLaunchKernelGGL(select_rank_kernel<RBM>, dim3((a.tokens + RBM - 1) / RBM), dim3(NT), smem, st,
                     (const float*)ews, a.tokens, a.groups, a.k, a.idx, a.counts);
  return hipGetLastError();
}

template <typename T>
hipError_t select_d(const SelArgs& a, float* ews, hipStream_t st) {
  const int groups = a.groups, rpg = a.rpg;
  if (groups > 256) return launch_select_t<T, 16, 8>(a, st);
  if (ews != nullptr && (a.tokens + 31) / 32 < compute_units()) return select_split<T>(a, ews, st);
  if constexpr (std::is_same<T, bf16_t>::value) {
    // direct-to-LDS: up to 256 sampled rows in one super-chunk of 4 fragments
    // per wave; beyond, super-chunks of 128 rows, whose small stages let two
    // workgroups share a CU (more waves issuing loads; measured faster than
    // fewer, wider super-chunks).  From 128 tokens per CU on, 128-token
    // workgroups (if their LDS fits): each workgroup streams all sampled rows
    // once per K step, and the larger block divides that over more tokens
    // (measured faster there; at 64 tokens per CU slower, since a CU then
    // holds one workgroup instead of two)
    // (one 256-row super-chunk: eight waves in eight column groups, two waves
    // per SIMD at one workgroup per CU; 128M select 19 -> 16 us)
    if (groups * rpg > 128 && groups * rpg <= 256) return launch_select_t<T, 32, 2, 8>(a, st);
    // (128-token blocks run eight waves: one workgroup per CU, two waves per SIMD.
    // Each super-chunk streams the x tile again: at the 1.3B shape 688 sampled
    // rows in 128-row super-chunks took 6 passes (171 us), in 256-row ones 3
    // passes (162 us), whose 48 KB stages fit a 2-stage ring only, so one stage
    // was in flight per step and each step waited about a memory latency; 192-row
    // super-chunks take 4 passes with 40 KB stages in a 3-stage ring: 159 -> 147 us)
    // (64 to 128 tokens per CU: 64-token blocks of eight waves, one per CU, with
    // 192-row super-chunks: every workgroup streams all sampled rows, and 64
    // tokens divide that over twice the tokens of 32-token blocks: 370M select
    // 34 -> 29 us, README layer 72 -> 70 us)
    if (a.tokens >= 64 * compute_units() && a.tokens < 128 * compute_units() &&
        SelCfg<T, 64, 3, true, kSel128Waves>::FIXED + (size_t)64 * (groups | 1) * 4 + groups * 4 <= kSelLds)
      return launch_select_t<T, 64, 3, kSel128Waves>(a, st);
    if (a.tokens >= 128 * compute_units()) {
      if (SelCfg<T, 128, 3, true, kSel128Waves>::FIXED + (size_t)128 * (groups | 1) * 4 + groups * 4 <= kSelLds)
        return launch_select_t<T, 128, 3, kSel128Waves>(a, st);
      if (SelCfg<T, 128, 4, true, kSel128Waves>::FIXED + (size_t)128 * (groups | 1) * 4 + groups * 4 <= kSelLds)
        return launch_select_t<T, 128, 4, kSel128Waves>(a, st);
      if (SelCfg<T, 128, 2, true, kSel128Waves>::FIXED + (size_t)128 * (groups | 1) * 4 + groups * 4 <= kSelLds)
        return launch_select_t<T, 128, 2, kSel128Waves>(a, st);
    }
    return launch_select_t<T, 32, 2>(a, st);  // (eight waves measured slower here: 16 waves per CU)
  } else {
    switch (pick_fnw(groups * rpg)) {
      case 2: return launch_select_t<T, 32, 2>(a, st);
      case 4: return launch_select_t<T, 32, 4>(a, st);
      case 6: return launch_select_t<T, 32, 6>(a, st);
      default: return launch_select_t<T, 32, 8>(a, st);
    }
  }
}

}  // namespace

size_t select_energy_bytes(int tokens, int groups) { return (size_t)tokens * groups * sizeof(float); }

hipError_t launch_select(int dtype, const void* x, const void* w_gate, int tokens, int d_model,
                         int groups, int k, const int32_t* sub, int rows_per_group, int group_size,
                         const float* bias, int32_t* idx_out, int32_t* counts_out, float* energy_ws,
                         hipStream_t stream) {
  if (counts_out) {
    hipError_t e = launch_fill_i32(counts_out, 0, (size_t)groups, stream);
    if (e != hipSuccess) return e;
  }
  if (tokens == 0) return hipSuccess;
  const SelArgs a{x, w_gate, tokens, d_model, groups * group_size, groups, k, sub, rows_per_group, bias, idx_out,
                  counts_out};
  return dtype == 0 ? select_d<float>(a, energy_ws, stream) : select_d<bf16_t>(a, energy_ws, stream);
}

}  // namespace esg
