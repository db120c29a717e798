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

// Inclusive prefix sum across a wavefront (64 lanes).
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Block-wide exclusive scans of two ints per thread (NTS threads, a multiple
// of 64): wavefront scans, then a scan of the wavefront totals by wavefront 0.
// Two barriers.
template <int NTS>
__device__ void block_exclusive_scan2(int a, int b, int& ea, int& eb, int& ta, int& tb, int* wsum) {
  constexpr int NW = NTS / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ia = wave_inclusive_scan(a, lane), ib = wave_inclusive_scan(b, lane);
  if (lane == 63) {
    wsum[w] = ia;
    wsum[NW + w] = ib;
  }
  __syncthreads();
  if (w == 0) {
    const int va = lane < NW ? wsum[lane] : 0, vb = lane < NW ? wsum[NW + lane] : 0;
    const int sa = wave_inclusive_scan(va, lane), sb = wave_inclusive_scan(vb, lane);
    if (lane < NW) {
      wsum[2 * NW + lane] = sa - va;  // exclusive wavefront bases
      wsum[3 * NW + lane] = sb - vb;
    }
    if (lane == NW - 1) {
      wsum[4 * NW] = sa;
      wsum[4 * NW + 1] = sb;
    }
  }
  __syncthreads();
  ea = wsum[2 * NW + w] + ia - a;
  eb = wsum[3 * NW + w] + ib - b;
  ta = wsum[4 * NW];
  tb = wsum[4 * NW + 1];
}

constexpr int SCAN_NT = 1024;

// bc[b][g] (counts) -> base[b][g] (CSR position of the block's first pair of
// group g) and pbase[b][g] (same in the padded layout).  One workgroup: thread
// t owns group g = t % G and a contiguous slice of the blocks; slice sums are
// scanned per group in LDS, group totals are scanned across groups.
__global__ __launch_bounds__(SCAN_NT) void bucket_scan_kernel(int nblocks, int groups, int tile_rows,
                                                              int max_tiles, const int32_t* __restrict__ bc,
                                                              int32_t* __restrict__ base,
                                                              int32_t* __restrict__ pbase,
                                                              int32_t* offsets, int32_t* tile_off,
                                                              int32_t* tile_group, int32_t* ptoken) {
  __shared__ int wsum[4 * (SCAN_NT / 64) + 2];
  __shared__ int part[SCAN_NT];     // [slice][group] sums, then exclusive prefix over slices
  __shared__ int g_off[SCAN_NT + 1], g_toff[SCAN_NT + 1];
  const int tid = threadIdx.x;
  const int slices = max(1, SCAN_NT / groups);
  const int per = (nblocks + slices - 1) / slices;
  const int g = tid % groups, sl = tid / groups;
  const bool active = sl < slices;
  const int b0 = min(nblocks, sl * per), b1 = min(nblocks, b0 + per);
  int sum = 0;
  if (active)
    for (int b = b0; b < b1; ++b) sum += bc[(size_t)b * groups + g];
  if (active) part[sl * groups + g] = sum;
  __syncthreads();
  int n = 0;  // total of group `tid`
  if (tid < groups) {
    for (int q = 0; q < slices; ++q) {
      const int v = part[q * groups + tid];
      part[q * groups + tid] = n;
      n += v;
    }
  }
  __syncthreads();
  int total = 0, total_tiles = 0, off = 0, toff = 0;
  const int nt = tid < groups ? (n + tile_rows - 1) / tile_rows : 0;
  block_exclusive_scan2<SCAN_NT>(tid < groups ? n : 0, nt, off, toff, total, total_tiles, wsum);
  if (tid < groups) {
    g_off[tid] = off;
    g_toff[tid] = toff;
    if (offsets) offsets[tid] = off;
    if (tile_off) tile_off[tid] = toff;
  }
  if (tid == 0) {
    g_off[groups] = total;
    g_toff[groups] = total_tiles;
    if (offsets) offsets[groups] = total;
    if (tile_off) tile_off[groups] = total_tiles;
  }
  __syncthreads();
  if (active) {
    int run = part[sl * groups + g];
    const int o = g_off[g], po = g_toff[g] * tile_rows;
    for (int b = b0; b < b1; ++b) {
      const size_t i = (size_t)b * groups + g;
      const int c = bc[i];
      base[i] = o + run;
      pbase[i] = po + run;
      run += c;
    }
  }
  // tile -> group by binary search over the tile offsets; -1 past the end
  if (tile_group) {
    for (int tt = tid; tt < max_tiles; tt += SCAN_NT) {
      int grp = -1;
      if (tt < total_tiles) {
        int lo = 0, hi = groups - 1;  // last group with g_toff[grp] <= tt
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (g_toff[mid] <= tt) lo = mid; else hi = mid - 1;
        }
        grp = lo;
      }
      tile_group[tt] = grp;
    }
  }
  // padding rows of each group's last tile
  if (ptoken) {
    for (int i = tid; i < groups * tile_rows; i += SCAN_NT) {
      const int gg = i / tile_rows;
      const int p = g_toff[gg] * tile_rows + (g_off[gg + 1] - g_off[gg]) + i % tile_rows;
      if (p < g_toff[gg + 1] * tile_rows) ptoken[p] = -1;
    }
  }
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
  int* sbase = (int*)(sm + TB * gw) + TB * k;  // the block's bases: [G] CSR, then [G] padded
  for (int i = 0; i < gw; ++i) mask[i] = 0;
  const size_t brow = (size_t)blockIdx.x * groups;
  for (int g = lane; g < groups; g += TB) {
    sbase[g] = base[brow + g];
    sbase[groups + g] = pbase[brow + g];
  }
  __syncthreads();
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
    const int pos = sbase[g] + r;
    const int ppos = sbase[groups + g] + r;
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
    const size_t smem = (size_t)TB * gw * 4 + (size_t)TB * k * 4 + (size_t)groups * 8;
    hipLaunchKernelGGL(bucket_scatter_kernel, dim3(nb), dim3(TB), smem, stream, idx, tokens, k, groups, base,
                       pbase, out.perm_token, out.inv, out.ptoken, out.pinv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace esg
