// Sigmoid top-k routing with an expert bias (Megatron-Core developer guide,
// "core.inference.moe.sigmoid_topk": _sigmoid_topk_kernel and
// sigmoid_topk_routing).
//
// One wavefront per token row; lane l holds the C experts [l*C, l*C + C).
//   score   s_e = sigmoid(logit_e), evaluated in fp64 and rounded once to fp32
//   key     s_e + bias_e (one fp32 addition), mapped to a uint32 whose order
//           is the total order of fp32 values (negatives have every bit
//           flipped, the others only the sign bit, so -0.0 < +0.0)
//   filter  fp32 estimates of the scores bound every key from below and
//           above; experts whose upper bound lies under a lower bound of the
//           k-th largest lower bound cannot be selected.  The (usually few)
//           remaining candidates are compacted one per lane and only they get
//           the fp64 score; rows with more than 64 candidates (many equal
//           keys) take the exact score of every expert instead
//   select  the k-th largest key by a radix descent over the 32 key bits: a
//           step counts, with one ballot per held expert, the keys that match
//           the prefix found so far with the next bit set; the descent also
//           leaves how many keys equal to the k-th one the row takes.  The row
//           lists the experts above that key in ascending order, then the ones
//           equal to it in ascending order; lanes hold ascending expert
//           ranges, so an expert's slot is the number of flagged experts in
//           lower lanes (ballot under the lane mask) plus those before it in
//           its own lane
//   weights p_j = s_j / ((((s_0 + s_1) + s_2) + ...) + 1e-20) [* scaling],
//           the sum folded left in output order, every operation in fp32.
// Rows never interact and each row's arithmetic is the same whichever
// wavefront takes it, so a row's result does not depend on the batch.
#include "esg_internal.hpp"

namespace esg {
namespace {

constexpr int kRouteRows = 4;  // wavefronts (token rows) per workgroup
// Top ordered key bits the filter's descent resolves: sign, exponent and 3
// mantissa bits, so its bound is within 1/8 (relative) of the k-th lower bound.
constexpr int kFilterBits = 12;
// Margin of the candidate filter: a bound, with room to spare, on the error
// of the fp32 score estimate (below 2^-21 for every finite logit).
constexpr float kEstimateMargin = 1.0f / 65536.0f;

__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float exact_sigmoid(float z) { return (float)(1.0 / (1.0 + exp(-(double)z))); }

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)v, off);
    v = o < v ? o : v;
  }
  return v;
}

// Radix descent over the top NB key bits of the C keys per lane: returns the
// k-th largest key of the valid ones (its top NB bits; the rest zero) and
// leaves in `need` how many keys equal to it the row takes.  With NB = 32 the
// descent stops as soon as the class of keys sharing the prefix holds exactly
// `need` keys: they are all taken, the k-th largest is their minimum, and
// `need` is recounted against it.
template <int C, int NB>
__device__ __forceinline__ uint32_t kth_largest(const uint32_t (&u)[C], const bool (&valid)[C], int nvalid, int k,
                                                int& need) {
  uint32_t prefix = 0;
  int cls = nvalid;  // keys matching the prefix so far
  need = k;
  for (int bit = 31; bit >= 32 - NB; --bit) {
    const uint32_t m = ~0u << bit;
    const uint32_t cand = prefix | (1u << bit);
    int cnt = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) cnt += __popcll(__ballot(valid[c] && (u[c] & m) == cand));
    if (cnt >= need) {
      prefix = cand;
      cls = cnt;
    } else {
      need -= cnt;
      cls -= cnt;
    }
    if (NB == 32 && cls == need && bit > 0) {
      uint32_t mn = 0xffffffffu;
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (valid[c] && (u[c] & m) == prefix && u[c] < mn) mn = u[c];
      prefix = wave_min_u32(mn);
      int above = 0;
#pragma unroll
      for (int c = 0; c < C; ++c) above += __popcll(__ballot(valid[c] && u[c] > prefix));
      need = k - above;
      break;
    }
  }
  return prefix;
}

// Slots of the selected keys (C per lane, lanes in ascending expert order):
// keys above tau fill slots [0, k - need) in order, then the first `need` keys
// equal to tau fill the rest.  Writes score and expert of each to the row's
// LDS lists.
template <int C>
__device__ __forceinline__ void place(const uint32_t (&u)[C], const bool (&valid)[C], const float (&sc)[C],
                                      const int (&ex)[C], uint32_t tau, int k, int need, int lane, float* s_row,
                                      int* e_row) {
  const uint64_t lower = (1ull << lane) - 1ull;
  int ia = 0, ie = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    ia += __popcll(__ballot(valid[c] && u[c] > tau) & lower);
    ie += __popcll(__ballot(valid[c] && u[c] == tau) & lower);
  }
  const int n_above = k - need;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    int slot = -1;
    if (valid[c] && u[c] > tau) {
      slot = ia++;
    } else if (valid[c] && u[c] == tau) {
      if (ie < need) slot = n_above + ie;
      ++ie;
    }
    if (slot >= 0) {
      s_row[slot] = sc[c];
      e_row[slot] = ex[c];
    }
  }
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Logits of row t for the C experts from e0 (zeros past E).
template <int C>
__device__ __forceinline__ void load_row(const float* __restrict__ logits, int t, int E, int vec4, int e0,
                                         float (&lg)[C]) {
  const float* row = logits + (size_t)t * E;
  if constexpr (C % 4 == 0) {
    if (vec4) {
#pragma unroll
      for (int q = 0; q < C / 4; ++q) {
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e0 + 4 * q < E) v = *(const float4*)(row + e0 + 4 * q);  // E % 4 == 0: all four in range
        lg[4 * q] = v.x;
        lg[4 * q + 1] = v.y;
        lg[4 * q + 2] = v.z;
        lg[4 * q + 3] = v.w;
      }
      return;
    }
  }
#pragma unroll
  for (int c = 0; c < C; ++c) lg[c] = e0 + c < E ? row[e0 + c] : 0.f;
}

// One wavefront per token row (a grid-stride loop with the next row's logits
// prefetched measured slower: more registers, fewer wavefronts in flight, and
// the kernel is bound by the scalar issue of the radix counting).
template <int C>
__global__ __launch_bounds__(64 * kRouteRows) void sigmoid_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int bias_stride, int tokens, int E, int k,
    float scaling, int apply_scaling, int vec4, float* __restrict__ probs, int64_t* __restrict__ indices) {
#pragma clang fp contract(off)
  __shared__ float s_sel[kRouteRows][kRouteMaxK];
  __shared__ int e_sel[kRouteRows][kRouteMaxK];
  __shared__ float c_logit[kRouteRows][64];
  __shared__ float c_bias[kRouteRows][64];
  __shared__ int c_exp[kRouteRows][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t = blockIdx.x * kRouteRows + w;
  if (t >= tokens) return;  // whole wavefronts; nothing below synchronises the workgroup
  const int e0 = lane * C;
  bool valid[C];
  float bv[C];
  int ex[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    ex[c] = e0 + c;
    valid[c] = ex[c] < E;
    bv[c] = valid[c] ? bias[(size_t)ex[c] * bias_stride] : 0.f;
  }
  float lg[C];
  load_row<C>(logits, t, E, vec4, e0, lg);

  // ---- candidate filter: fp32 estimates bound every exact key ----
  // est = 1/(1 + e^-z) with the fast exponential and reciprocal is within
  // 2^-21 of sigmoid(z) (its error is ~s(1-s) times the exponential's
  // relative error, itself ~(2|z| + 2) 2^-24, plus two roundings of at most
  // 2^-24 s each, and s(1-s)|z| <= 0.23), so
  // s lies in [est - m, est + m] and, rounding being monotone, the exact key
  // fl(s + b) lies in [lo, hi] = [fl(fl(est - m) + b), fl(fl(est + m) + b)].
  // A lower bound L on the k-th largest lo (its top ordered bits) leaves
  // out only experts with hi < L: k experts have exact keys >= L above them.
  uint32_t ulo[C], uhi[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const float est = 1.0f / (1.0f + __expf(-lg[c]));
    ulo[c] = order_key((est - kEstimateMargin) + bv[c]);
    uhi[c] = order_key((est + kEstimateMargin) + bv[c]);
  }
  int need;
  const uint32_t L = kth_largest<C, kFilterBits>(ulo, valid, E, k, need);
  bool cand[C];
  int n_cand = 0;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    cand[c] = valid[c] && uhi[c] >= L;
    n_cand += __popcll(__ballot(cand[c]));
  }

  float* s_row = s_sel[w];
  int* e_row = e_sel[w];
  if (n_cand <= 64) {
    // compact the candidates in ascending expert order: lane i takes the i-th
    const uint64_t lower = (1ull << lane) - 1ull;
    int pos = 0;
#pragma unroll
    for (int c = 0; c < C; ++c) pos += __popcll(__ballot(cand[c]) & lower);
#pragma unroll
    for (int c = 0; c < C; ++c)
      if (cand[c]) {
        c_logit[w][pos] = lg[c];
        c_bias[w][pos] = bv[c];
        c_exp[w][pos] = ex[c];
        ++pos;
      }
    wave_lds_sync();
    bool v1[1] = {lane < n_cand};
    float s1[1] = {0.f};
    int e1[1] = {0};
    uint32_t u1[1] = {0};
    if (v1[0]) {
      e1[0] = c_exp[w][lane];
      s1[0] = exact_sigmoid(c_logit[w][lane]);
      u1[0] = order_key(s1[0] + c_bias[w][lane]);
    }
    const uint32_t tau = kth_largest<1, 32>(u1, v1, n_cand, k, need);
    place<1>(u1, v1, s1, e1, tau, k, need, lane, s_row, e_row);
  } else {
    // many near-equal keys (ties, saturated scores): exact keys for all experts
    float sc[C];
    uint32_t u[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      sc[c] = exact_sigmoid(lg[c]);
      u[c] = order_key(sc[c] + bv[c]);
    }
    const uint32_t tau = kth_largest<C, 32>(u, valid, E, k, need);
    place<C>(u, valid, sc, ex, tau, k, need, lane, s_row, e_row);
  }
  wave_lds_sync();  // the row's slots were written by other lanes of this wavefront

  float total = 0.0f;
  for (int i = 0; i < k; ++i) total = total + s_row[i];
  if (lane < k) {
    float p = s_row[lane] / (total + 1e-20f);
    if (apply_scaling) p = p * scaling;
    probs[(size_t)t * k + lane] = p;
    indices[(size_t)t * k + lane] = (int64_t)e_row[lane];
  }
}

template <int C>
void launch_c(const float* logits, const float* bias, int bias_stride, int tokens, int E, int k, float scaling,
              int apply_scaling, int vec4, float* probs, int64_t* indices, hipStream_t stream) {
  const int blocks = (tokens + kRouteRows - 1) / kRouteRows;
  hipLaunchKernelGGL(sigmoid_topk_kernel<C>, dim3(blocks), dim3(64 * kRouteRows), 0, stream, logits, bias,
                     bias_stride, tokens, E, k, scaling, apply_scaling, vec4, probs, indices);
}

}  // namespace

bool sigmoid_topk_supported(int num_experts, int topk) {
  return num_experts >= 1 && num_experts <= kRouteMaxExperts && topk >= 1 && topk <= kRouteMaxK &&
         topk <= num_experts;
}

hipError_t launch_sigmoid_topk(const float* logits, const float* bias, int bias_stride, int tokens, int E, int k,
                               float scaling, int apply_scaling, float* probs, int64_t* indices,
                               hipStream_t stream) {
  if (tokens == 0) return hipSuccess;
  const int vec4 = (E % 4 == 0) && ((uintptr_t)logits % 16 == 0);
  LaunchTimer timer("sigmoid_topk", stream);
  if (E <= 64)
    launch_c<1>(logits, bias, bias_stride, tokens, E, k, scaling, apply_scaling, vec4, probs, indices, stream);
  else if (E <= 128)
    launch_c<2>(logits, bias, bias_stride, tokens, E, k, scaling, apply_scaling, vec4, probs, indices, stream);
  else if (E <= 256)
    launch_c<4>(logits, bias, bias_stride, tokens, E, k, scaling, apply_scaling, vec4, probs, indices, stream);
  else if (E <= 512)
    launch_c<8>(logits, bias, bias_stride, tokens, E, k, scaling, apply_scaling, vec4, probs, indices, stream);
  else if (E <= 1024)
    launch_c<16>(logits, bias, bias_stride, tokens, E, k, scaling, apply_scaling, vec4, probs, indices, stream);
  else
    launch_c<32>(logits, bias, bias_stride, tokens, E, k, scaling, apply_scaling, vec4, probs, indices, stream);
  return hipGetLastError();
}

}  // namespace esg
