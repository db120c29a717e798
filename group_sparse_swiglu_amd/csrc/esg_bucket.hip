// Deterministic CSR bucketing of routed (token, slot) pairs by group (the
// eugen_sparse README's "Pitfalls and limitations" states that the CSR
// bucketing is deterministic; the layout is this library's).
//
// Pairs are ordered by (group, token).  Three passes, no floating point and no
// order-dependent atomics:
//   count   one wavefront per 64 tokens: the block's ids are staged in LDS,
//           each lane walks its token's slots (marking out-of-range ids and
//           repeats as skipped) into a per-token group bitmask and the block
//           histogram;
//   scan    one workgroup: group totals, offsets, per-block bases in token
//           order, tile bookkeeping for the grouped GEMMs;
//   scatter one wavefront per 64 tokens: for each group the block uses, in id
//           order, a ballot over the wavefront's tokens gives each token its
//           rank among the block's tokens that chose the group (ascending
//           token), which plus the block base is its bucket position.
// Up to 64 tokens (one block) a single workgroup does all three in one launch;
// while the [blocks, G] count table is small, scan and scatter share a launch
// (each workgroup reads the whole table).
//
// All loads of a pass are issued together (the ids of a block are one
// contiguous slab of 64*k ints, read coalesced), so a pass costs a couple of
// memory round trips whatever k is.
//
// Besides the plain CSR (offsets, perm_token, inv) it can emit the padded
// layout the grouped GEMMs use: each group's positions are padded to whole
// tiles of `tile_rows`, groups laid out one after another.
#include "esg_internal.hpp"

namespace esg {
namespace {

constexpr int TB = 64;  // tokens per block (one wavefront)
constexpr int LU = 16;  // id loads in flight per lane

// LDS strides with an odd number of dwords per token, so that lanes walking
// their own token's row hit distinct banks: ids as int16, masks as uint32.
__host__ __device__ inline int row_stride(int k) { return 2 * (((k + 1) >> 1) | 1); }
__host__ __device__ inline int mask_stride(int groups) { return ((groups + 31) >> 5) | 1; }

// Inclusive prefix sum across a wavefront (64 lanes).
__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) v |= (uint32_t)__shfl_xor((int)v, o);
  return v;
}

// Ids of the block's nt tokens (the slab idx[t0*k, (t0+nt)*k)) -> srow[token][slot]
// as int16, -1 for an id outside [0, groups) (status bit 1).  NT threads, thread
// `tid` taking elements tid, tid + NT, ...
template <int NT>
__device__ void stage_ids(const int32_t* __restrict__ idx, size_t t0, int nt, int k, int groups,
                          int16_t* srow, int rs, int tid, int& bits) {
  const int n = nt * k;
  const int32_t* src = idx + t0 * k;
  const int q = NT / k, rr = NT % k;  // step of (token, slot) per NT elements
  int tl = tid / k, j = tid - (tid / k) * k;
  for (int o0 = 0; o0 < n; o0 += LU * NT) {
    int v[LU];
#pragma unroll
    for (int u = 0; u < LU; ++u) {
      const int o = o0 + u * NT + tid;
      v[u] = o < n ? src[o] : 0;
    }
#pragma unroll
    for (int u = 0; u < LU; ++u) {
      if (o0 + u * NT + tid < n) {
        const int g = v[u];
        const bool ok = g >= 0 && g < groups;
        if (!ok) bits |= 1;
        srow[tl * rs + j] = ok ? (int16_t)g : (int16_t)-1;
      }
      tl += q;
      j += rr;
      if (j >= k) {
        j -= k;
        ++tl;
      }
    }
  }
}

// One lane walks its token's ids in slot order: the first occurrence of an id
// sets its bit in the token's group mask (and counts it in `hist` if given);
// a repeat is rewritten to -1 (status bit 2).  Up to 64 groups the mask lives
// in two registers and the ids are read 16 at a time (no dependent LDS round
// trip per slot); beyond, the mask is updated in LDS.
__device__ void mark_slots(int16_t* r, int k, uint32_t* m, int gw, int* hist, int& bits) {
  if (gw <= 2) {
    uint32_t m0 = 0, m1 = 0;
    for (int j0 = 0; j0 < k; j0 += 16) {
      int v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = j0 + u < k ? r[j0 + u] : -1;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int g = v[u];
        if (g < 0) continue;
        const uint32_t bit = 1u << (g & 31);
        const uint32_t mw = g >= 32 ? m1 : m0;
        if (mw & bit) {
          r[j0 + u] = -1;
          bits |= 2;
        } else {
          if (g >= 32) m1 |= bit; else m0 |= bit;
          if (hist) atomicAdd(&hist[g], 1);
        }
      }
    }
    m[0] = m0;
    if (gw > 1) m[1] = m1;
    return;
  }
  for (int i = 0; i < gw; ++i) m[i] = 0;
  for (int j = 0; j < k; ++j) {
    const int g = r[j];
    if (g < 0) continue;
    const uint32_t bit = 1u << (g & 31);
    if (m[g >> 5] & bit) {
      r[j] = -1;
      bits |= 2;
    } else {
      m[g >> 5] |= bit;
      if (hist) atomicAdd(&hist[g], 1);
    }
  }
}

// rk[token][i] = rank of the token among the block's tokens holding its i-th
// smallest group.  Only the groups some token of the block holds are visited.
__device__ void block_ranks(const uint32_t* masks, int ms, int gw, int k, uint8_t* rk, int lane) {
  const uint64_t lt = (1ull << lane) - 1ull;
  int hits = 0;
  for (int wi = 0; wi < gw; ++wi) {
    const uint32_t mw = masks[lane * ms + wi];
    uint32_t any = wave_or(mw);
    while (any) {
      const int b = __ffs(any) - 1;
      any &= any - 1u;
      const bool has = (mw >> b) & 1u;
      const uint64_t bal = __ballot(has);
      if (has) rk[lane * k + hits++] = (uint8_t)__popcll(bal & lt);
    }
  }
}

// Per-pair outputs of the block, written coalesced in (token, slot) order by NT
// threads: pos = cbase[g] + rank, ppos = pbase[g] * pmul + rank.
template <int NT>
__device__ void block_outputs(const int16_t* srow, int rs, const uint32_t* masks, int ms, const uint8_t* rk,
                              size_t t0, int nt, int k, const int* cbase, const int* pbase, int pmul,
                              int32_t* perm_token, int32_t* inv, int32_t* ptoken, int32_t* pinv, int tid) {
  const int n = nt * k;
  const int q = NT / k, rr = NT % k;
  int tl = tid / k, j = tid - (tid / k) * k;
  for (int o = tid; o < n; o += NT) {
    const int g = srow[tl * rs + j];
    const size_t out = t0 * k + o;
    if (g < 0) {
      if (inv) inv[out] = -1;
      if (pinv) pinv[out] = -1;
    } else {
      const uint32_t* m = masks + tl * ms;
      int order = __popc(m[g >> 5] & ((1u << (g & 31)) - 1u));
      for (int w = 0; w < (g >> 5); ++w) order += __popc(m[w]);
      const int r = rk[tl * k + order];
      const int tok = (int)t0 + tl;
      const int pos = cbase[g] + r, ppos = pbase[g] * pmul + r;
      if (perm_token) perm_token[pos] = tok;
      if (inv) inv[out] = pos;
      if (ptoken) ptoken[ppos] = tok;
      if (pinv) pinv[out] = ppos;
    }
    tl += q;
    j += rr;
    if (j >= k) {
      j -= k;
      ++tl;
    }
  }
}

// tile -> group by binary search over the tile offsets; -1 past the end.
__device__ void write_tile_groups(const int* g_toff, int groups, int max_tiles, int32_t* tile_group, int tid,
                                  int nthreads) {
  const int total_tiles = g_toff[groups];
  for (int tt = tid; tt < max_tiles; tt += nthreads) {
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

// Padding rows after each group's positions (to the end of its last tile, or
// of its last pair of tiles with a pad of two tiles) -> -1: one wavefront per
// group, its lanes over the group's (contiguous) padding rows.
__device__ void write_padding(const int* g_off, const int* g_toff, int groups, int tile_rows, int32_t* ptoken,
                              int wave, int nwaves, int lane) {
  for (int gg = wave; gg < groups; gg += nwaves) {
    const int end = g_toff[gg + 1] * tile_rows;
    for (int p = g_toff[gg] * tile_rows + (g_off[gg + 1] - g_off[gg]) + lane; p < end; p += 64) ptoken[p] = -1;
  }
}

// Per-block group histogram -> bc[block][g].
__global__ __launch_bounds__(TB) void bucket_count_kernel(const int32_t* __restrict__ idx, int tokens, int k,
                                                          int groups, int32_t* __restrict__ bc, int32_t* status) {
  extern __shared__ uint32_t sm[];
  const int lane = threadIdx.x;
  const int gw = (groups + 31) >> 5, ms = mask_stride(groups), rs = row_stride(k);
  uint32_t* masks = sm;                             // [TB][ms]
  int* hist = (int*)(masks + TB * ms);              // [groups]
  int16_t* srow = (int16_t*)(hist + groups);        // [TB][rs]
  const size_t t0 = (size_t)blockIdx.x * TB;
  const int nt = min(TB, tokens - (int)t0);
  int bits = 0;
  for (int g = lane; g < groups; g += TB) hist[g] = 0;
  stage_ids<TB>(idx, t0, nt, k, groups, srow, rs, lane, bits);
  __syncthreads();
  mark_slots(srow + lane * rs, lane < nt ? k : 0, masks + lane * ms, gw, hist, bits);
  if (bits && status) atomicOr(status, bits);
  __syncthreads();
  for (int g = lane; g < groups; g += TB) bc[(size_t)blockIdx.x * groups + g] = hist[g];
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
constexpr int SU = 8;  // block counts loaded per batch

// bc[b][g] (counts) -> base[b][g] (CSR position of the block's first pair of
// group g) and pbase[b][g] (same in the padded layout).  One workgroup: thread
// t owns group g = t % G and a contiguous slice of the blocks; slice sums are
// scanned per group in LDS, group totals are scanned across groups.
__global__ __launch_bounds__(SCAN_NT) void bucket_scan_kernel(int nblocks, int groups, int tile_rows,
                                                              int max_tiles, const int32_t* __restrict__ bc,
                                                              int32_t* __restrict__ base,
                                                              int32_t* __restrict__ pbase,
                                                              int32_t* offsets, int32_t* tile_off,
                                                              int32_t* tile_group, int32_t* ptoken, int tile_pad) {
  __shared__ int wsum[4 * (SCAN_NT / 64) + 2];
  __shared__ int part[SCAN_NT];     // [slice][group] sums, then exclusive prefix over slices
  __shared__ int g_off[SCAN_NT + 1], g_toff[SCAN_NT + 1];
  const int tid = threadIdx.x;
  const int slices = max(1, SCAN_NT / groups);
  const int per = (nblocks + slices - 1) / slices;
  const int g = tid % groups, sl = tid / groups;
  const bool active = sl < slices;
  const int b0 = min(nblocks, sl * per), b1 = active ? min(nblocks, b0 + per) : b0;
  int sum = 0;
  for (int b = b0; b < b1; b += SU) {
    int v[SU];
#pragma unroll
    for (int u = 0; u < SU; ++u) v[u] = b + u < b1 ? bc[(size_t)(b + u) * groups + g] : 0;
#pragma unroll
    for (int u = 0; u < SU; ++u) sum += v[u];
  }
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
  const int nt = tid < groups ? (n + tile_pad - 1) / tile_pad * (tile_pad / tile_rows) : 0;
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
    for (int b = b0; b < b1; b += SU) {
      int v[SU];
#pragma unroll
      for (int u = 0; u < SU; ++u) v[u] = b + u < b1 ? bc[(size_t)(b + u) * groups + g] : 0;
#pragma unroll
      for (int u = 0; u < SU; ++u) {
        if (b + u < b1) {
          const size_t i = (size_t)(b + u) * groups + g;
          base[i] = o + run;
          pbase[i] = po + run;
        }
        run += v[u];
      }
    }
  }
  if (tile_group) write_tile_groups(g_toff, groups, max_tiles, tile_group, tid, SCAN_NT);
  if (ptoken) write_padding(g_off, g_toff, groups, tile_rows, ptoken, tid >> 6, SCAN_NT / 64, tid & 63);
}

__global__ __launch_bounds__(TB) void bucket_scatter_kernel(const int32_t* __restrict__ idx, int tokens, int k,
                                                            int groups, const int32_t* __restrict__ base,
                                                            const int32_t* __restrict__ pbase,
                                                            int32_t* perm_token, int32_t* inv, int32_t* ptoken,
                                                            int32_t* pinv) {
  extern __shared__ uint32_t sm[];
  const int lane = threadIdx.x;
  const int gw = (groups + 31) >> 5, ms = mask_stride(groups), rs = row_stride(k);
  uint32_t* masks = sm;                            // [TB][ms]
  int* sbase = (int*)(masks + TB * ms);            // the block's bases: [G] CSR, then [G] padded
  int16_t* srow = (int16_t*)(sbase + 2 * groups);  // [TB][rs]
  uint8_t* rk = (uint8_t*)(srow + TB * rs);        // [TB][k]
  const size_t t0 = (size_t)blockIdx.x * TB;
  const int nt = min(TB, tokens - (int)t0);
  const size_t brow = (size_t)blockIdx.x * groups;
  for (int g0 = 0; g0 < groups; g0 += 4 * TB) {
    int v[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = g0 + u * TB + lane;
      v[2 * u] = g < groups ? base[brow + g] : 0;
      v[2 * u + 1] = g < groups ? pbase[brow + g] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int g = g0 + u * TB + lane;
      if (g < groups) {
        sbase[g] = v[2 * u];
        sbase[groups + g] = v[2 * u + 1];
      }
    }
  }
  int bits = 0;  // reported by the count pass
  stage_ids<TB>(idx, t0, nt, k, groups, srow, rs, lane, bits);
  __syncthreads();
  mark_slots(srow + lane * rs, lane < nt ? k : 0, masks + lane * ms, gw, nullptr, bits);
  __syncthreads();
  block_ranks(masks, ms, gw, k, rk, lane);
  __syncthreads();
  block_outputs<TB>(srow, rs, masks, ms, rk, t0, nt, k, sbase, sbase + groups, 1, perm_token, inv, ptoken, pinv,
                    lane);
}

constexpr int PW = 4;          // blocks (wavefronts) per placement workgroup
constexpr int PNT = PW * TB;   // 256 threads
constexpr int PU = 16;         // block counts loaded per batch
constexpr int kPlaceMaxTable = 32768;  // count-table entries a placement workgroup reads whole

// Scan and scatter in one pass, for count tables small enough that every
// workgroup reads the whole of bc[nblocks][groups]: workgroup p places blocks
// [PW*p, PW*p + PW), one wavefront each.  Per group it sums the total and the
// prefix over the blocks before its own (integer sums: any order gives the same
// result), scans the totals into group and tile offsets (wavefront 0), and
// wavefront w adds the counts of the workgroup's blocks before its own; then
// the scatter above.  Workgroup 0 also writes offsets, tile_off, tile_group
// and the padding rows.
__global__ __launch_bounds__(PNT) void bucket_place_kernel(const int32_t* __restrict__ idx, int tokens, int k,
                                                           int groups, int tile_rows, int max_tiles, int nblocks,
                                                           const int32_t* __restrict__ bc, BucketOut out,
                                                           int tile_pad) {
  extern __shared__ uint32_t sm[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int gw = (groups + 31) >> 5, ms = mask_stride(groups), rs = row_stride(k);
  const int slices = groups >= PNT ? 1 : PNT / groups;
  int* tot = (int*)sm;                    // [groups]
  int* pre = tot + groups;                // [groups]
  int* g_off = pre + groups;              // [groups + 1]
  int* g_toff = g_off + groups + 1;       // [groups + 1]
  int* part = g_toff + groups + 1;        // [2][slices][groups]
  const int fixed_words = 2 * groups + 2 * (groups + 1) + 2 * slices * groups;
  char* wbase = (char*)sm + (((size_t)fixed_words * 4 + 15) & ~(size_t)15);  // per-wavefront regions
  const size_t wbytes = ((size_t)2 * groups * 4 + (size_t)TB * ms * 4 + (size_t)TB * rs * 2 + (size_t)TB * k + 15) &
                        ~(size_t)15;
  char* mine = wbase + w * wbytes;
  int* sbase = (int*)mine;                             // [2][groups]: CSR, padded
  uint32_t* masks = (uint32_t*)(sbase + 2 * groups);   // [TB][ms]
  int16_t* srow = (int16_t*)(masks + TB * ms);         // [TB][rs]
  uint8_t* rk = (uint8_t*)(srow + TB * rs);            // [TB][k]

  const int b0 = blockIdx.x * PW;
  const int per = (nblocks + slices - 1) / slices;
  for (int i = tid; i < slices * groups; i += PNT) {
    const int g = i % groups, sl = i / groups;
    const int lo = min(nblocks, sl * per), hi = min(nblocks, lo + per);
    int sp = 0, st = 0;
    for (int b = lo; b < hi; b += PU) {
      int v[PU];
#pragma unroll
      for (int u = 0; u < PU; ++u) v[u] = b + u < hi ? bc[(size_t)(b + u) * groups + g] : 0;
#pragma unroll
      for (int u = 0; u < PU; ++u) {
        st += v[u];
        if (b + u < b0) sp += v[u];
      }
    }
    part[sl * groups + g] = sp;
    part[(slices + sl) * groups + g] = st;
  }
  __syncthreads();
  for (int g = tid; g < groups; g += PNT) {
    int sp = 0, st = 0;
    for (int sl = 0; sl < slices; ++sl) {
      sp += part[sl * groups + g];
      st += part[(slices + sl) * groups + g];
    }
    pre[g] = sp;
    tot[g] = st;
  }
  __syncthreads();
  if (w == 0) {
    int carry = 0, tcarry = 0;
    for (int c = 0; c < groups; c += TB) {
      const int g = c + lane;
      const int n = g < groups ? tot[g] : 0;
      const int ntl = (n + tile_pad - 1) / tile_pad * (tile_pad / tile_rows);
      const int io = wave_inclusive_scan(n, lane), it = wave_inclusive_scan(ntl, lane);
      if (g < groups) {
        g_off[g] = carry + io - n;
        g_toff[g] = tcarry + it - ntl;
      }
      carry += __shfl(io, 63);
      tcarry += __shfl(it, 63);
    }
    if (lane == 0) {
      g_off[groups] = carry;
      g_toff[groups] = tcarry;
    }
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    for (int g = tid; g <= groups; g += PNT) {
      if (out.offsets) out.offsets[g] = g_off[g];
      if (out.tile_off) out.tile_off[g] = g_toff[g];
    }
    if (out.tile_group) write_tile_groups(g_toff, groups, max_tiles, out.tile_group, tid, PNT);
    if (out.ptoken) write_padding(g_off, g_toff, groups, tile_rows, out.ptoken, w, PW, lane);
  }
  // this wavefront's block: its bases, then the scatter
  const int b = b0 + w;
  const bool active = b < nblocks;
  const size_t t0 = (size_t)b * TB;
  const int nt = active ? min(TB, tokens - (int)t0) : 0;
  if (active)
    for (int g = lane; g < groups; g += TB) {
      int run = pre[g];
      for (int j = 0; j < w; ++j) run += bc[(size_t)(b0 + j) * groups + g];
      sbase[g] = g_off[g] + run;
      sbase[groups + g] = g_toff[g] * tile_rows + run;
    }
  int bits = 0;  // reported by the count pass
  if (active) stage_ids<TB>(idx, t0, nt, k, groups, srow, rs, lane, bits);
  __syncthreads();
  mark_slots(srow + lane * rs, lane < nt ? k : 0, masks + lane * ms, gw, nullptr, bits);
  __syncthreads();
  block_ranks(masks, ms, gw, k, rk, lane);
  __syncthreads();
  block_outputs<TB>(srow, rs, masks, ms, rk, t0, nt, k, sbase, sbase + groups, 1, out.perm_token, out.inv,
                    out.ptoken, out.pinv, lane);
}

size_t place_smem(int groups, int k) {
  const int slices = groups >= PNT ? 1 : PNT / groups;
  const size_t fixed = (size_t)(2 * groups + 2 * (groups + 1) + 2 * slices * groups) * 4;
  const size_t wbytes = ((size_t)2 * groups * 4 + (size_t)TB * mask_stride(groups) * 4 +
                         (size_t)TB * row_stride(k) * 2 + (size_t)TB * k + 15) & ~(size_t)15;
  return ((fixed + 15) & ~(size_t)15) + PW * wbytes;
}

constexpr int SINGLE_NT = 1024;

// All three passes for at most 64 tokens in one workgroup: every thread loads
// ids and writes outputs and tile bookkeeping; wavefront 0 (a lane per token)
// builds the masks, the ranks and the group scan.
__global__ __launch_bounds__(SINGLE_NT) void bucket_single_kernel(const int32_t* __restrict__ idx, int tokens,
                                                                  int k, int groups, int tile_rows, int max_tiles,
                                                                  BucketOut out, int tile_pad) {
  extern __shared__ uint32_t sm[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int gw = (groups + 31) >> 5, ms = mask_stride(groups), rs = row_stride(k);
  uint32_t* masks = sm;                             // [TB][ms]
  int* hist = (int*)(masks + TB * ms);              // [groups]
  int* g_off = hist + groups;                       // [groups + 1]
  int* g_toff = g_off + groups + 1;                 // [groups + 1]
  int16_t* srow = (int16_t*)(g_toff + groups + 1);  // [TB][rs]
  uint8_t* rk = (uint8_t*)(srow + TB * rs);         // [TB][k]
  const int nt = tokens;
  int bits = 0;
  for (int g = tid; g < groups; g += SINGLE_NT) hist[g] = 0;
  stage_ids<SINGLE_NT>(idx, 0, nt, k, groups, srow, rs, tid, bits);
  __syncthreads();
  if (w == 0) mark_slots(srow + lane * rs, lane < nt ? k : 0, masks + lane * ms, gw, hist, bits);
  if (bits && out.status) atomicOr(out.status, bits);
  __syncthreads();
  if (w == 0) {
    int carry = 0, tcarry = 0;
    for (int c = 0; c < groups; c += TB) {
      const int g = c + lane;
      const int n = g < groups ? hist[g] : 0;
      const int ntl = (n + tile_pad - 1) / tile_pad * (tile_pad / tile_rows);
      const int io = wave_inclusive_scan(n, lane), it = wave_inclusive_scan(ntl, lane);
      if (g < groups) {
        g_off[g] = carry + io - n;
        g_toff[g] = tcarry + it - ntl;
        if (out.offsets) out.offsets[g] = carry + io - n;
        if (out.tile_off) out.tile_off[g] = tcarry + it - ntl;
      }
      carry += __shfl(io, 63);
      tcarry += __shfl(it, 63);
    }
    if (lane == 0) {
      g_off[groups] = carry;
      g_toff[groups] = tcarry;
      if (out.offsets) out.offsets[groups] = carry;
      if (out.tile_off) out.tile_off[groups] = tcarry;
    }
  }
  __syncthreads();
  if (w == 0) block_ranks(masks, ms, gw, k, rk, lane);
  if (out.tile_group) write_tile_groups(g_toff, groups, max_tiles, out.tile_group, tid, SINGLE_NT);
  if (out.ptoken) write_padding(g_off, g_toff, groups, tile_rows, out.ptoken, w, SINGLE_NT / 64, lane);
  __syncthreads();
  block_outputs<SINGLE_NT>(srow, rs, masks, ms, rk, 0, nt, k, g_off, g_toff, tile_rows, out.perm_token, out.inv,
                           out.ptoken, out.pinv, tid);
}

}  // namespace

size_t bucket_scratch_bytes(int tokens, int groups) {
  const size_t nb = (size_t)(tokens + TB - 1) / TB;
  return 3 * nb * (size_t)groups * sizeof(int32_t) + 256;
}

int max_tiles(int tokens, int k, int groups, int tile_rows, int tile_pad) {
  // sum over groups of ceil(n_g / tile_pad) * (tile_pad / tile_rows) tiles,
  // at most (T*k + G*(tile_pad - 1)) / tile_rows; rounded up to whole pads
  const long long tk = (long long)tokens * k;
  const long long per = tile_pad / tile_rows;
  const long long bound = (tk + (long long)groups * (tile_pad - 1)) / tile_rows;
  return (int)((bound + per - 1) / per * per);
}

hipError_t launch_bucket(const int32_t* idx, int tokens, int k, int groups, int tile_rows,
                         const BucketOut& out, void* scratch, hipStream_t stream, int tile_pad) {
  if (tile_pad <= 0) tile_pad = tile_rows;
  const int nb = (tokens + TB - 1) / TB;
  const int mt = max_tiles(tokens, k, groups, tile_rows, tile_pad);
  const size_t masks = (size_t)TB * mask_stride(groups) * 4, rows = (size_t)TB * row_stride(k) * 2,
               ranks = (size_t)TB * k;
  if (nb <= 1) {
    LaunchTimer timer("bucket_single", stream);
    const size_t smem = masks + (size_t)(3 * groups + 2) * 4 + rows + ranks;
    hipLaunchKernelGGL(bucket_single_kernel, dim3(1), dim3(SINGLE_NT), smem, stream, idx, tokens, k, groups,
                       tile_rows, mt, out, tile_pad);
    return hipGetLastError();
  }
  int32_t* bc = (int32_t*)scratch;
  int32_t* base = bc + (size_t)nb * groups;
  int32_t* pbase = base + (size_t)nb * groups;
  {
    LaunchTimer timer("bucket_count", stream);
    const size_t smem = masks + (size_t)groups * 4 + rows;
    hipLaunchKernelGGL(bucket_count_kernel, dim3(nb), dim3(TB), smem, stream, idx, tokens, k, groups, bc,
                       out.status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // a count table every workgroup can read whole: scan and scatter in one pass
  const size_t psmem = place_smem(groups, k);
  if ((size_t)nb * groups <= (size_t)kPlaceMaxTable && psmem <= 64 * 1024) {
    LaunchTimer timer("bucket_place", stream);
    hipLaunchKernelGGL(bucket_place_kernel, dim3((nb + PW - 1) / PW), dim3(PNT), psmem, stream, idx, tokens, k,
                       groups, tile_rows, mt, nb, (const int32_t*)bc, out, tile_pad);
    return hipGetLastError();
  }
  {
    LaunchTimer timer("bucket_scan", stream);
    hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(SCAN_NT), 0, stream, nb, groups, tile_rows, mt, bc,
                       base, pbase, out.offsets, out.tile_off, out.tile_group, out.ptoken, tile_pad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    LaunchTimer timer("bucket_scatter", stream);
    const size_t smem = masks + (size_t)groups * 8 + rows + ranks;
    hipLaunchKernelGGL(bucket_scatter_kernel, dim3(nb), dim3(TB), smem, stream, idx, tokens, k, groups, base,
                       pbase, out.perm_token, out.inv, out.ptoken, out.pinv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace esg
