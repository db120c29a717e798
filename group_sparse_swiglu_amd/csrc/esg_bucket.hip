// Deterministic CSR bucketing of routed (token, slot) pairs by group (the
// eugen_sparse README's "Pitfalls and limitations" states that the CSR
// bucketing is deterministic; the layout is this library's).
//
// Pairs are ordered by (group, token).  Three passes, no floating point and no
// order-dependent atomics:
//   count   one wavefront per 64 tokens: per-token group bitmask in LDS (marks
//           out-of-range ids and repeats as skipped), then a block histogram;
//   scan    one workgroup: group totals, offsets, per-block bases in token
//           order, tile bookkeeping for the grouped GEMMs;
//   scatter one wavefront per 64 tokens: for each group in id order a ballot
//           over the wavefront's tokens gives each token its rank among the
//           block's tokens that chose the group (ascending token), which plus
//           the block base is its bucket position.
//
// Besides the plain CSR (offsets, perm_token, inv) it can emit the padded
// layout the grouped GEMMs use: each group's positions are padded to whole
// tiles of `tile_rows`, groups laid out one after another.
#include "esg_internal.hpp"

namespace esg {
namespace {

constexpr int TB = 64;  // tokens per block (one wavefront)

__device__ __forceinline__ bool slot_valid(const int32_t* row, int j, int groups, uint32_t* mask,
                                           int* status_bits) {
  const int g = row[j];
  if (g < 0 || g >= groups) {
    *status_bits |= 1;
    return false;
  }
  const uint32_t bit = 1u << (g & 31);
  if (mask[g >> 5] & bit) {
    *status_bits |= 2;
    return false;
  }
  mask[g >> 5] |= bit;
  return true;
}

// Per-block group histogram -> bc[block][g].
__global__ __launch_bounds__(TB) void bucket_count_kernel(const int32_t* __restrict__ idx, int tokens,
                                                          int k, int groups, int32_t* __restrict__ bc,
                                                          int32_t* status) {
  extern __shared__ uint32_t sm[];
  const int gw = (groups + 31) >> 5;
  uint32_t* mask = sm + threadIdx.x * gw;
  int* hist = (int*)(sm + TB * gw);
  for (int i = threadIdx.x; i < groups; i += TB) hist[i] = 0;
  for (int i = 0; i < gw; ++i) mask[i] = 0;
  __syncthreads();
  const int t = blockIdx.x * TB + threadIdx.x;
  int bits = 0;
  if (t < tokens) {
    const int32_t* row = idx + (size_t)t * k;
    for (int j = 0; j < k; ++j)
      if (slot_valid(row, j, groups, mask, &bits)) atomicAdd(&hist[row[j]], 1);
  }
  if (bits && status) atomicOr(status, bits);
  __syncthreads();
  for (int g = threadIdx.x; g < groups; g += TB) bc[(size_t)blockIdx.x * groups + g] = hist[g];
}

// Block-wide exclusive scan of one int per thread (NTS threads).
template <int NTS>
__device__ int block_exclusive_scan(int v, int* buf, int* total) {
  const int tid = threadIdx.x;
  buf[tid] = v;
  __syncthreads();
  for (int off = 1; off < NTS; off <<= 1) {
    const int add = tid >= off ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += add;
    __syncthreads();
  }
  const int incl = buf[tid];
  *total = buf[NTS - 1];
  __syncthreads();
  return incl - v;
}

constexpr int SCAN_NT = 1024;

// bc[b][g] (counts) -> base[b][g] (CSR position of the block's first pair of
// group g) and pbase[b][g] (same in the padded layout).
__global__ __launch_bounds__(SCAN_NT) void bucket_scan_kernel(int nblocks, int groups, int tile_rows,
                                                              int max_tiles, const int32_t* __restrict__ bc,
                                                              int32_t* __restrict__ base,
                                                              int32_t* __restrict__ pbase,
                                                              int32_t* offsets, int32_t* tile_off,
                                                              int32_t* tile_group, int32_t* ptoken) {
  __shared__ int buf[SCAN_NT];
  const int g = threadIdx.x;
  int n = 0;
  if (g < groups)
    for (int b = 0; b < nblocks; ++b) n += bc[(size_t)b * groups + g];
  int total = 0, total_tiles = 0;
  const int off = block_exclusive_scan<SCAN_NT>(n, buf, &total);
  const int nt = (n + tile_rows - 1) / tile_rows;
  const int toff = block_exclusive_scan<SCAN_NT>(nt, buf, &total_tiles);
  if (g < groups) {
    if (offsets) offsets[g] = off;
    if (tile_off) tile_off[g] = toff;
    int run = 0;
    for (int b = 0; b < nblocks; ++b) {
      const size_t i = (size_t)b * groups + g;
      const int c = bc[i];
      base[i] = off + run;
      pbase[i] = toff * tile_rows + run;
      run += c;
    }
    if (tile_group)
      for (int tt = toff; tt < toff + nt; ++tt) tile_group[tt] = g;
    if (ptoken)
      for (int p = toff * tile_rows + n; p < (toff + nt) * tile_rows; ++p) ptoken[p] = -1;
  }
  if (g == 0) {
    if (offsets) offsets[groups] = total;
    if (tile_off) tile_off[groups] = total_tiles;
  }
  if (tile_group)
    for (int tt = total_tiles + g; tt < max_tiles; tt += SCAN_NT) tile_group[tt] = -1;
}

__global__ __launch_bounds__(TB) void bucket_scatter_kernel(const int32_t* __restrict__ idx, int tokens,
                                                            int k, int groups,
                                                            const int32_t* __restrict__ base,
                                                            const int32_t* __restrict__ pbase,
                                                            int32_t* perm_token, int32_t* inv,
                                                            int32_t* ptoken, int32_t* pinv) {
  extern __shared__ uint32_t sm[];
  const int gw = (groups + 31) >> 5;
  const int lane = threadIdx.x;
  uint32_t* mask = sm + lane * gw;
  int* rk = (int*)(sm + TB * gw) + lane * k;  // rank of this token among the block's
                                              // tokens of its i-th smallest group
  for (int i = 0; i < gw; ++i) mask[i] = 0;
  const int t = blockIdx.x * TB + lane;
  const int32_t* row = idx + (size_t)t * k;
  int bits = 0;
  if (t < tokens)
    for (int j = 0; j < k; ++j) slot_valid(row, j, groups, mask, &bits);
  // ranks, group by group in ascending id
  int hits = 0;
  const uint64_t lt = (1ull << lane) - 1ull;
  for (int g = 0; g < groups; ++g) {
    const bool has = (t < tokens) && ((mask[g >> 5] >> (g & 31)) & 1u);
    const uint64_t m = __ballot(has);
    if (has) rk[hits++] = __popcll(m & lt);
  }
  if (t >= tokens) return;
  // outputs per slot; a slot is valid when it is the first occurrence of an
  // in-range id (the same rule as the count pass)
  const size_t brow = (size_t)blockIdx.x * groups;
  for (int j = 0; j < k; ++j) {
    const int g = row[j];
    bool valid = g >= 0 && g < groups;
    for (int q = 0; valid && q < j; ++q) valid = row[q] != g;
    int order = 0;  // valid distinct ids of this token below g = mask bits below g
    if (valid) {
      for (int w = 0; w < (g >> 5); ++w) order += __popc(mask[w]);
      order += __popc(mask[g >> 5] & ((1u << (g & 31)) - 1u));
    }
    const size_t o = (size_t)t * k + j;
    if (!valid) {
      if (inv) inv[o] = -1;
      if (pinv) pinv[o] = -1;
      continue;
    }
    const int r = rk[order];
    const int pos = base[brow + g] + r;
    const int ppos = pbase[brow + g] + r;
    if (perm_token) perm_token[pos] = t;
    if (inv) inv[o] = pos;
    if (ptoken) ptoken[ppos] = t;
    if (pinv) pinv[o] = ppos;
  }
}

}  // namespace

size_t bucket_scratch_bytes(int tokens, int groups) {
  const size_t nb = (size_t)(tokens + TB - 1) / TB;
  return 3 * nb * (size_t)groups * sizeof(int32_t) + 256;
}

int max_tiles(int tokens, int k, int groups, int tile_rows) {
  const long long tk = (long long)tokens * k;
  return (int)((tk + (long long)groups * (tile_rows - 1)) / tile_rows);
}

hipError_t launch_bucket(const int32_t* idx, int tokens, int k, int groups, int tile_rows,
                         const BucketOut& out, void* scratch, hipStream_t stream) {
  const int nb = (tokens + TB - 1) / TB;
  int32_t* bc = (int32_t*)scratch;
  int32_t* base = bc + (size_t)nb * groups;
  int32_t* pbase = base + (size_t)nb * groups;
  const int gw = (groups + 31) / 32;
  const int mt = max_tiles(tokens, k, groups, tile_rows);
  if (nb > 0) {
    LaunchTimer timer("bucket_count", stream);
    const size_t smem = (size_t)TB * gw * 4 + (size_t)groups * 4;
    hipLaunchKernelGGL(bucket_count_kernel, dim3(nb), dim3(TB), smem, stream, idx, tokens, k, groups, bc,
                       out.status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    LaunchTimer timer("bucket_scan", stream);
    hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(SCAN_NT), 0, stream, nb, groups, tile_rows, mt, bc,
                       base, pbase, out.offsets, out.tile_off, out.tile_group, out.ptoken);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (nb > 0) {
    LaunchTimer timer("bucket_scatter", stream);
    const size_t smem = (size_t)TB * gw * 4 + (size_t)TB * k * 4;
    hipLaunchKernelGGL(bucket_scatter_kernel, dim3(nb), dim3(TB), smem, stream, idx, tokens, k, groups, base,
                       pbase, out.perm_token, out.inv, out.ptoken, out.pinv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace esg
