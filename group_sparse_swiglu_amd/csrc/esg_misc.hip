// Load-balance bias update (eugen_sparse README, "What it does",
// update_load_balance_bias; "Parameters and how to choose them" gives
// gamma 1e-3, bias_max 0.5, momentum 0.99 and target k/G) and small fills.
//
// Per group g, in float32 with every operation rounded separately (no fused
// multiply-add, so a float32 host implementation reproduces it bit for bit):
//   cur  = current_freq[g]            (or counts[g] / tokens)
//   ema  = ema + (1 - momentum) * (cur - ema)
//   bias = clamp(bias + gamma * sign(target - ema), -bias_max, bias_max)
#include "esg_internal.hpp"

namespace esg {
namespace {

// The current frequency of group g: freq[g], or counts[g] / tokens, or (from
// the CSR group offsets of a routing) (offsets[g+1] - offsets[g]) / tokens.
__global__ void bias_update_kernel(float* __restrict__ bias, float* __restrict__ ema,
                                   const float* __restrict__ freq, const int32_t* __restrict__ counts,
                                   const int32_t* __restrict__ offsets, int tokens, float target, float gamma,
                                   float bias_max, float momentum, int groups) {
#pragma clang fp contract(off)
  for (int g = blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += gridDim.x * blockDim.x) {
    const int n = counts ? counts[g] : (offsets ? offsets[g + 1] - offsets[g] : 0);
    const float cur = freq ? freq[g] : (float)n / (float)tokens;
    const float e = ema[g];
    const float om = 1.0f - momentum;
    const float ne = e + om * (cur - e);
    const float diff = target - ne;
    const float step = diff > 0.0f ? gamma : (diff < 0.0f ? -gamma : 0.0f);
    float nb = bias[g] + step;
    nb = fminf(fmaxf(nb, -bias_max), bias_max);
    ema[g] = ne;
    bias[g] = nb;
  }
}

// Rate probe of the bf16 matrix cores: every wave runs `iters` rounds of
// eight independent 16x16x32 bf16 MFMAs on register operands (no memory
// traffic in the loop) and writes one sum per lane, so the work stays.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* __restrict__ out) {
  typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
  typedef __attribute__((ext_vector_type(4))) float f32x4;
  const unsigned lane = threadIdx.x & 63;
  // small normal bf16 values (about 2^-7), different per lane
  const uint4 ua = make_uint4(0x3c003c00u + lane, 0x3c103c10u, 0x3c203c20u, 0x3c303c30u);
  const uint4 ub = make_uint4(0x3c083c08u, 0x3c183c18u + lane, 0x3c283c28u, 0x3c383c38u);
  const bf16x8 a = __builtin_bit_cast(bf16x8, ua), b = __builtin_bit_cast(bf16x8, ub);
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) sum += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int32_t v, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = v;
}

}  // namespace

hipError_t launch_bias_update(float* bias, float* ema, const float* freq, const int32_t* counts,
                              const int32_t* offsets, int tokens, float target, float gamma, float bias_max,
                              float momentum, int groups, hipStream_t stream) {
  if (groups == 0) return hipSuccess;
  const int threads = 256;
  const int blocks = (groups + threads - 1) / threads;
  LaunchTimer timer("bias_update", stream);
  hipLaunchKernelGGL(bias_update_kernel, dim3(blocks), dim3(threads), 0, stream, bias, ema, freq, counts, offsets,
                     tokens, target, gamma, bias_max, momentum, groups);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t value, size_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  LaunchTimer timer("fill", stream);
  hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, value, n);
  return hipGetLastError();
}

hipError_t launch_mfma_probe(int blocks, int iters, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, stream, iters, out);
  return hipGetLastError();
}

// Compute units of the current device (cached per device; 256 if the query fails).
int compute_units() {
  static int cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace esg
