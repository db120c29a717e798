// Grouped top-k selection (eugen_sparse README, "What it does",
// grouped_topk_select): per token, the k groups with the largest
// sum over sampled gate rows of |SiLU(x . w_gate_row)|, plus the bias.
//
// One workgroup owns BM tokens.  The gate contraction over the sampled rows
// runs on MFMA in column chunks of 64 sampled rows; each chunk's |SiLU|
// values are staged in LDS and summed per (token, group) in column order into
// an fp32 energy table E[BM][G] that starts at the bias.  The top-k is then a
// wavefront rank test: lane g counts the groups that beat group g (higher
// score, or equal score and lower id); the group is selected when fewer than
// k beat it, and its output slot is its rank among the selected ids (a ballot
// prefix).  Every token's result depends only on its own row: batch
// invariant and bitwise reproducible.
#include "esg_device.hpp"
#include "esg_internal.hpp"

namespace esg {
namespace {

constexpr int NT = 256;
constexpr int BN = 64;  // sampled rows per column chunk
constexpr int KC = 8;   // chunks per K stage

template <typename T, int BM>
struct SelCfg {
  static constexpr int WAVES_M = BM >= 32 ? BM / 32 : 1;
  static constexpr int WAVES_N = 4 / WAVES_M;
  static constexpr int FM = BM / (16 * WAVES_M);
  static constexpr int FN = BN / (16 * WAVES_N);
  static constexpr int PA = Plane<BM>::BYTES;
  static constexpr int PB = Plane<BN>::BYTES;
  static constexpr int A_BYTES = KC * PA;
  static constexpr int B_BYTES = KC * PB;
  static constexpr int S_STRIDE = BN + 1;  // floats per staged row
  static constexpr int S_BYTES = BM * S_STRIDE * 4;
  static constexpr int FIXED = 2 * A_BYTES + 2 * B_BYTES + S_BYTES;
};

template <typename T, int BM>
__global__ __launch_bounds__(NT) void select_kernel(const T* __restrict__ x, const T* __restrict__ wg,
                                                     int tokens, int d_model, int groups, int k,
                                                     const int32_t* __restrict__ sub, int rpg,
                                                     const float* __restrict__ bias,
                                                     int32_t* __restrict__ idx_out,
                                                     int32_t* __restrict__ counts) {
  using C = SelCfg<T, BM>;
  extern __shared__ __align__(16) char smem[];
  auto la = [&](int i_) -> char* { return i_ ? (smem + C::A_BYTES) : (smem); };
  auto lb = [&](int i_) -> char* { return i_ ? (smem + 2 * C::A_BYTES + C::B_BYTES) : (smem + 2 * C::A_BYTES); };
  float* S = (float*)(smem + 2 * C::A_BYTES + 2 * C::B_BYTES);
  float* E = (float*)(smem + C::FIXED);  // [BM][groups]
  int* cnt = (int*)(E + BM * groups);    // [groups]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % C::WAVES_M, wn = wave / C::WAVES_M;
  const int t0 = blockIdx.x * BM;
  const int ncols = groups * rpg;
  const int kbytes = d_model * (int)sizeof(T);
  const int nk = (d_model * (int)sizeof(T) + KC * 16 - 1) / (KC * 16);

  for (int i = tid; i < BM * groups; i += NT) E[i] = bias ? bias[i % groups] : 0.0f;
  for (int i = tid; i < groups; i += NT) cnt[i] = 0;

  RowKLoader<BM, KC, NT> ldA;
  ldA.init(tid, [&](int r) -> const char* {
    const int t = t0 + r;
    return t < tokens ? (const char*)(x + (size_t)t * d_model) : nullptr;
  });

  int arow[C::FM], brow[C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i) arow[i] = wm * (C::FM * 16) + i * 16 + (lane & 15);
#pragma unroll
  for (int j = 0; j < C::FN; ++j) brow[j] = wn * (C::FN * 16) + j * 16 + (lane & 15);

  for (int n0 = 0; n0 < ncols; n0 += BN) {
    RowKLoader<BN, KC, NT> ldB;
    ldB.init(tid, [&](int r) -> const char* {
      const int col = n0 + r;
      if (col >= ncols) return nullptr;
      const int row = sub ? sub[col] : col;  // without a subsample the columns are all gate rows
      return (const char*)(wg + (size_t)row * d_model);
    });
    f32x4 acc[C::FM][C::FN];
    zero_acc(acc);
    ldA.load(0, kbytes);
    ldB.load(0, kbytes);
    __syncthreads();  // E init and previous chunk's S reads are done
    ldA.store(la(0));
    ldB.store(lb(0));
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
      if (kt + 1 < nk) {
        ldA.load((kt + 1) * KC * 16, kbytes);
        ldB.load((kt + 1) * KC * 16, kbytes);
      }
      mma_lds<T, C::FM, C::FN, KC, C::PA, C::PB>(acc, la(kt & 1), lb(kt & 1), arow, brow, lane);
      if (kt + 1 < nk) {
        ldA.store(la((kt + 1) & 1));
        ldB.store(lb((kt + 1) & 1));
      }
      __syncthreads();
    }
    // |SiLU| of the chunk into S
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = arow[i] - (lane & 15) + (lane >> 4) * 4 + e;
          const int c = brow[j];
          const float h = acc[i][j][e];
          S[r * C::S_STRIDE + c] = fabsf(h * sigmoid_f(h));
        }
    __syncthreads();
    // per (token, group) sums over this chunk's columns, in column order
    const int g_lo = n0 / rpg;
    const int g_hi = min(groups - 1, (min(n0 + BN, ncols) - 1) / rpg);
    const int ng = g_hi - g_lo + 1;
    for (int p = tid; p < BM * ng; p += NT) {
      const int r = p / ng, g = g_lo + p % ng;
      const int c0 = max(n0, g * rpg) - n0, c1 = min(n0 + BN, (g + 1) * rpg) - n0;
      float s = E[r * groups + g];
      for (int c = c0; c < c1; ++c) s += S[r * C::S_STRIDE + c];
      E[r * groups + g] = s;
    }
    // the next chunk's first __syncthreads orders these writes before reuse
  }
  __syncthreads();

  // rank top-k: one token per wave at a time, lanes over groups
  for (int r = wave; r < BM; r += 4) {
    const int t = t0 + r;
    if (t >= tokens) break;
    const float* row = E + r * groups;
    int base = 0;
    for (int g0 = 0; g0 < groups; g0 += 64) {
      const int g = g0 + lane;
      bool sel = false;
      if (g < groups) {
        const float sg = row[g];
        int beat = 0;
        for (int q = 0; q < groups; ++q) {
          const float sq = row[q];
          beat += (sq > sg) || (sq == sg && q < g);
        }
        sel = beat < k;
      }
      const uint64_t m = __ballot(sel);
      const int pos = base + __popcll(m & ((1ull << lane) - 1ull));
      if (sel && pos < k) {  // NaN scores could select more than k: never write past the row
        idx_out[(size_t)t * k + pos] = g;
        if (counts) atomicAdd(&cnt[g], 1);
      }
      base += __popcll(m);
    }
  }
  if (counts) {
    __syncthreads();
    for (int g = tid; g < groups; g += NT)
      if (cnt[g]) atomicAdd(&counts[g], cnt[g]);
  }
}

template <typename T, int BM>
hipError_t launch_select_t(const void* x, const void* wg, int tokens, int d_model, int groups, int k,
                           const int32_t* sub, int rpg, const float* bias, int32_t* idx,
                           int32_t* counts, hipStream_t stream) {
  using C = SelCfg<T, BM>;
  const size_t smem = C::FIXED + (size_t)BM * groups * 4 + (size_t)groups * 4;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)select_kernel<T, BM>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int blocks = (tokens + BM - 1) / BM;
  LaunchTimer timer("select", stream);
  hipLaunchKernelGGL((select_kernel<T, BM>), dim3(blocks), dim3(NT), smem, stream, (const T*)x,
                     (const T*)wg, tokens, d_model, groups, k, sub, rpg, bias, idx, counts);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(int dtype, const void* x, const void* w_gate, int tokens, int d_model,
                         int groups, int k, const int32_t* sub, int rows_per_group, int group_size,
                         const float* bias, int32_t* idx_out, int32_t* counts_out, hipStream_t stream) {
  (void)group_size;
  if (counts_out) {
    hipError_t e = launch_fill_i32(counts_out, 0, (size_t)groups, stream);
    if (e != hipSuccess) return e;
  }
  if (tokens == 0) return hipSuccess;
  const bool small_g = groups <= 256;
  if (dtype == 0) {
    return small_g ? launch_select_t<float, 64>(x, w_gate, tokens, d_model, groups, k, sub, rows_per_group,
                                                bias, idx_out, counts_out, stream)
                   : launch_select_t<float, 16>(x, w_gate, tokens, d_model, groups, k, sub, rows_per_group,
                                                bias, idx_out, counts_out, stream);
  }
  return small_g ? launch_select_t<bf16_t, 64>(x, w_gate, tokens, d_model, groups, k, sub, rows_per_group,
                                               bias, idx_out, counts_out, stream)
                 : launch_select_t<bf16_t, 16>(x, w_gate, tokens, d_model, groups, k, sub, rows_per_group,
                                               bias, idx_out, counts_out, stream);
}

}  // namespace esg
