// Sparse SwiGLU forward and backward over CSR buckets (eugen_sparse README,
// "What it does", sparse_swiglu_ffn):
//   y[t] = sum over selected g of (SiLU(x W_gate[g]^T) * (x W_up[g]^T)) W_down[:, g]^T
//
// Work is organised by tiles of kTileRows bucket positions of one group
// (padded layout, see esg_bucket.hip).  A group wider than GSB neurons is
// processed as group_size/GSB sub-blocks; every sub-block yields its own
// per-position partial, and partials are summed per token in a fixed order
// (slot, then sub-block) without atomics.
//
// Forward tile (fwd_grouped_kernel):
//   phase 1  H = X_tile [BM x d] . [W_gate rows ; W_up rows]^T   (MFMA, K = d)
//            epilogue in registers: a = SiLU(hg) * hu; hg, hu saved compact
//            for the backward; a goes to LDS only -- never to HBM
//   phase 2  P^T = W_down[d-block, group cols] . a^T  (MFMA, K = group width),
//            written as per-position partial rows of y
//   rowsum   y[t] = sum_j P[pinv[t, j]]
//
// Backward tile (bwd_dh_dx_kernel):
//   phase 1  dA = dY_tile . W_down[:, group cols]        (MFMA, K = d)
//            epilogue: dg = dA*hu*SiLU'(hg), du = dA*SiLU(hg), a = SiLU(hg)*hu
//            (compact, for dW) and [dg du] to LDS
//   phase 2  Q^T = [W_gate; W_up]^T[d-block] . [dg du]^T (MFMA, K = 2*width),
//            per-position partial rows of dx; then rowsum as above
// dW (bwd_dw_kernel), one workgroup per (group, d-block, kind):
//   dW_gate|up[g] = [dg du]^T X_g, dW_down[:, g] = dY_g^T a_g, K = the
//   group's padded positions; a group nobody chose runs zero iterations and
//   writes exact zeros.
//
// Compact per-position activations use the layout [sub][pos/EPC][GSB][EPC]:
// 16-byte chunks of EPC consecutive positions of one neuron, which is both the
// MFMA result layout of phase 1 and the K-packed operand layout of the dW
// contraction over positions.
#include "esg_device.hpp"
#include "esg_internal.hpp"

namespace esg {
namespace {

constexpr int NT = 256;
constexpr int BM = kTileRows;
constexpr int DB = 128;  // d-block rows in the phase-2 / dW contractions
constexpr int KC = 8;    // chunks per K stage

constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int round4(int a) { return (a + 3) / 4 * 4; }

template <typename T>
__device__ __forceinline__ size_t packed_index(size_t pos, int n, int gsb) {
  constexpr int EPC = Elem<T>::EPC;
  return ((pos / EPC) * gsb + n) * EPC + pos % EPC;
}

// ===========================================================================
// Forward
// ===========================================================================
template <typename T, int GSB>
struct FwdCfg {
  static constexpr int EPC = Elem<T>::EPC;
  static constexpr int WN1 = GSB >= 32 ? 2 : 1;
  static constexpr int WM1 = 4 / WN1;
  static constexpr int FM1 = BM / (16 * WM1);
  static constexpr int FP1 = GSB / (16 * WN1);  // gate/up fragment pairs per wave
  static constexpr int PA1 = Plane<BM>::BYTES;
  static constexpr int PB1 = Plane<2 * GSB>::BYTES;
  static constexpr int A1 = KC * PA1, B1 = KC * PB1;
  static constexpr int P1_BYTES = 2 * (A1 + B1);
  static constexpr int KC2 = round4(GSB / EPC);
  static constexpr int FM2 = DB / 32, FN2 = BM / 32;  // 2 x 2 waves
  static constexpr int PW = Plane<DB>::BYTES;
  static constexpr int PACT = Plane<BM>::BYTES;
  static constexpr int ACT = KC2 * PACT;
  static constexpr int W2 = KC2 * PW;
  static constexpr int P2_BYTES = ACT + 2 * W2;
  static constexpr int SMEM = cmax(P1_BYTES, P2_BYTES);
};

template <typename T, int GSB>
__global__ __launch_bounds__(NT) void fwd_grouped_kernel(
    const T* __restrict__ x, const T* __restrict__ wg, const T* __restrict__ wu, const T* __restrict__ wd,
    int d, int F, int gs, const int32_t* __restrict__ tile_group, const int32_t* __restrict__ ptoken,
    size_t rows_total, T* __restrict__ hg_saved, T* __restrict__ hu_saved, T* __restrict__ partials) {
  using C = FwdCfg<T, GSB>;
  constexpr int EPC = C::EPC;
  extern __shared__ __align__(16) char smem[];
  const int tile = blockIdx.x;
  const int g = tile_group[tile];
  if (g < 0) return;
  const int s = blockIdx.y;
  const int nb0 = g * gs + s * GSB;  // first neuron of this sub-block
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t prow0 = (size_t)tile * BM;
  const int32_t* tok = ptoken + prow0;

  // ---------------- phase 1: [hg hu] = X . [Wg; Wu]^T ----------------
  auto la = [&](int i_) -> char* { return i_ ? (smem + C::A1) : (smem); };
  auto lb = [&](int i_) -> char* { return i_ ? (smem + 2 * C::A1 + C::B1) : (smem + 2 * C::A1); };
  const int wm = wave % C::WM1, wn = wave / C::WM1;
  RowKLoader<BM, KC, NT> ldA;
  ldA.init(tid, [&](int r) -> const char* {
    const int t = tok[r];
    return t >= 0 ? (const char*)(x + (size_t)t * d) : nullptr;
  });
  RowKLoader<2 * GSB, KC, NT> ldB;
  ldB.init(tid, [&](int r) -> const char* {
    return r < GSB ? (const char*)(wg + (size_t)(nb0 + r) * d) : (const char*)(wu + (size_t)(nb0 + r - GSB) * d);
  });
  int arow[C::FM1], brow[2 * C::FP1];
#pragma unroll
  for (int i = 0; i < C::FM1; ++i) arow[i] = wm * (C::FM1 * 16) + i * 16 + (lane & 15);
#pragma unroll
  for (int p = 0; p < C::FP1; ++p) {
    brow[p] = wn * (GSB / C::WN1) + p * 16 + (lane & 15);
    brow[C::FP1 + p] = GSB + brow[p];
  }
  f32x4 acc[C::FM1][2 * C::FP1];
  zero_acc(acc);
  const int kbytes = d * (int)sizeof(T);
  const int nk = (kbytes + KC * 16 - 1) / (KC * 16);
  ldA.load(0, kbytes);
  ldB.load(0, kbytes);
  ldA.store(la(0));
  ldB.store(lb(0));
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) {
      ldA.load((kt + 1) * KC * 16, kbytes);
      ldB.load((kt + 1) * KC * 16, kbytes);
    }
    mma_lds<T, C::FM1, 2 * C::FP1, KC, C::PA1, C::PB1>(acc, la(kt & 1), lb(kt & 1), arow, brow, lane);
    if (kt + 1 < nk) {
      ldA.store(la((kt + 1) & 1));
      ldB.store(lb((kt + 1) & 1));
    }
    __syncthreads();
  }

  // ---------------- epilogue: save hg, hu; a -> LDS ----------------
  char* act = smem;  // phase-1 buffers are dead now
  if constexpr (C::KC2 * EPC > GSB) {
    for (int i = tid; i < (C::KC2 - GSB / EPC) * BM; i += NT) {
      const int c = GSB / EPC + i / BM, r = i % BM;
      *(uint4*)(act + c * C::PACT + r * 16) = make_uint4(0, 0, 0, 0);
    }
  }
  const size_t sub_off = (size_t)s * rows_total * GSB;
#pragma unroll
  for (int i = 0; i < C::FM1; ++i) {
    const int r0 = arow[i] - (lane & 15) + (lane >> 4) * 4;
#pragma unroll
    for (int p = 0; p < C::FP1; ++p) {
      const int n = brow[p];
      float hg[4], hu[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        hg[e] = acc[i][p][e];
        hu[e] = acc[i][C::FP1 + p][e];
      }
      const size_t q = sub_off + packed_index<T>(prow0 + r0, n, GSB);
      if (hg_saved != nullptr) {  // NULL: inference, nothing kept for a backward
        Quad<T>::store(hg_saved + q, hg);
        Quad<T>::store(hu_saved + q, hu);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = hg[e] * sigmoid_f(hg[e]) * hu[e];
        store_elem<T>((T*)(act + (n / EPC) * C::PACT + (r0 + e) * 16) + (n % EPC), a);
      }
    }
  }
  __syncthreads();

  // ---------------- phase 2: P^T = Wd[d-block, group] . a^T ----------------
  auto lw = [&](int i_) -> char* { return i_ ? (smem + C::ACT + C::W2) : (smem + C::ACT); };
  const int wm2 = wave & 1, wn2 = wave >> 1;
  int arow2[C::FM2], brow2[C::FN2];
  bool valid[C::FN2];
#pragma unroll
  for (int i = 0; i < C::FM2; ++i) arow2[i] = wm2 * (C::FM2 * 16) + i * 16 + (lane & 15);
#pragma unroll
  for (int j = 0; j < C::FN2; ++j) {
    brow2[j] = wn2 * (C::FN2 * 16) + j * 16 + (lane & 15);
    valid[j] = tok[brow2[j]] >= 0;
  }
  const int kbytes2 = GSB * (int)sizeof(T);
  const int nblk = (d + DB - 1) / DB;
  RowKLoader<DB, C::KC2, NT> ldW;
  auto wrow = [&](int db0) {
    return [=](int r) -> const char* {
      return db0 + r < d ? (const char*)(wd + (size_t)(db0 + r) * F + nb0) : nullptr;
    };
  };
  ldW.init(tid, wrow(0));
  ldW.load(0, kbytes2);
  ldW.store(lw(0));
  __syncthreads();
  T* out = partials + (size_t)s * rows_total * d;
  for (int blk = 0; blk < nblk; ++blk) {
    if (blk + 1 < nblk) {
      ldW.init(tid, wrow((blk + 1) * DB));
      ldW.load(0, kbytes2);
    }
    f32x4 acc2[C::FM2][C::FN2];
    zero_acc(acc2);
    mma_lds<T, C::FM2, C::FN2, C::KC2, C::PW, C::PACT>(acc2, lw(blk & 1), act, arow2, brow2, lane);
#pragma unroll
    for (int i = 0; i < C::FM2; ++i) {
      const int dd = blk * DB + arow2[i] - (lane & 15) + (lane >> 4) * 4;
      if (dd >= d) continue;
#pragma unroll
      for (int j = 0; j < C::FN2; ++j) {
        if (!valid[j]) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc2[i][j][e];
        Quad<T>::store(out + (prow0 + brow2[j]) * d + dd, v);
      }
    }
    if (blk + 1 < nblk) ldW.store(lw((blk + 1) & 1));
    __syncthreads();
  }
}

template <typename T>
__global__ __launch_bounds__(256) void rowsum_kernel(const T* __restrict__ partials, size_t sub_stride,
                                                     int nsub, const int32_t* __restrict__ pinv, int tokens,
                                                     int k, int d, T* __restrict__ out) {
  rowsum_range<T>(partials, sub_stride, nsub, pinv, tokens, k, d, out, blockIdx.x, gridDim.x);
}

// ===========================================================================
// Backward: dh (+ SiLU' epilogue) and dx partials
// ===========================================================================
template <typename T, int GSB>
struct BwdCfg {
  static constexpr int EPC = Elem<T>::EPC;
  static constexpr int WN1 = GSB >= 32 ? 2 : 1;
  static constexpr int WM1 = 4 / WN1;
  static constexpr int FM1 = BM / (16 * WM1);
  static constexpr int FN1 = GSB / (16 * WN1);
  static constexpr int PA1 = Plane<BM>::BYTES;
  static constexpr int PB1 = Plane<GSB>::BYTES;
  static constexpr int A1 = KC * PA1, B1 = KC * PB1;
  static constexpr int P1_BYTES = 2 * (A1 + B1);
  static constexpr int KDG = (2 * GSB / EPC + KC - 1) / KC * KC;  // chunks of [dg du] along K
  static constexpr int PDG = Plane<BM>::BYTES;
  static constexpr int DGU = KDG * PDG;
  static constexpr int PW = Plane<DB>::BYTES;
  static constexpr int W2 = KC * PW;
  static constexpr int NKS = (KDG + KC - 1) / KC;  // K stages per d-block
  static constexpr int FM2 = DB / 32, FN2 = BM / 32;
  static constexpr int SMEM = cmax(P1_BYTES, DGU + 2 * W2);
};

template <typename T, int GSB>
__global__ __launch_bounds__(NT) void bwd_dh_dx_kernel(
    const T* __restrict__ dy, const T* __restrict__ wg, const T* __restrict__ wu, const T* __restrict__ wd,
    int d, int F, int gs, const int32_t* __restrict__ tile_group, const int32_t* __restrict__ ptoken,
    size_t rows_total, const T* __restrict__ hg_saved, const T* __restrict__ hu_saved, T* __restrict__ dg_out,
    T* __restrict__ du_out, T* __restrict__ act_out, T* __restrict__ partials) {
  using C = BwdCfg<T, GSB>;
  constexpr int EPC = C::EPC;
  extern __shared__ __align__(16) char smem[];
  const int tile = blockIdx.x;
  const int g = tile_group[tile];
  if (g < 0) return;
  const int s = blockIdx.y;
  const int nb0 = g * gs + s * GSB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t prow0 = (size_t)tile * BM;
  const int32_t* tok = ptoken + prow0;

  // ---------------- phase 1: dA = dY . Wd[:, group] ----------------
  auto la = [&](int i_) -> char* { return i_ ? (smem + C::A1) : (smem); };
  auto lb = [&](int i_) -> char* { return i_ ? (smem + 2 * C::A1 + C::B1) : (smem + 2 * C::A1); };
  const int wm = wave % C::WM1, wn = wave / C::WM1;
  RowKLoader<BM, KC, NT> ldA;
  ldA.init(tid, [&](int r) -> const char* {
    const int t = tok[r];
    return t >= 0 ? (const char*)(dy + (size_t)t * d) : nullptr;
  });
  TransLoader<T, GSB, KC, NT> ldB;
  ldB.init(tid);
  auto wdrow = [&](int k) -> const char* { return (const char*)(wd + (size_t)k * F + nb0); };
  int arow[C::FM1], brow[C::FN1];
#pragma unroll
  for (int i = 0; i < C::FM1; ++i) arow[i] = wm * (C::FM1 * 16) + i * 16 + (lane & 15);
#pragma unroll
  for (int j = 0; j < C::FN1; ++j) brow[j] = wn * (C::FN1 * 16) + j * 16 + (lane & 15);
  f32x4 acc[C::FM1][C::FN1];
  zero_acc(acc);
  const int kbytes = d * (int)sizeof(T);
  const int kstep = KC * EPC;
  const int nk = (d + kstep - 1) / kstep;
  ldA.load(0, kbytes);
  ldB.load(0, d, GSB, wdrow);
  ldA.store(la(0));
  ldB.store(lb(0));
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) {
      ldA.load((kt + 1) * KC * 16, kbytes);
      ldB.load((kt + 1) * kstep, d, GSB, wdrow);
    }
    mma_lds<T, C::FM1, C::FN1, KC, C::PA1, C::PB1>(acc, la(kt & 1), lb(kt & 1), arow, brow, lane);
    if (kt + 1 < nk) {
      ldA.store(la((kt + 1) & 1));
      ldB.store(lb((kt + 1) & 1));
    }
    __syncthreads();
  }

  // ---------------- epilogue: SiLU' ----------------
  char* dgu = smem;
  if constexpr (C::KDG * EPC > 2 * GSB) {
    for (int i = tid; i < (C::KDG - 2 * GSB / EPC) * BM; i += NT) {
      const int c = 2 * GSB / EPC + i / BM, r = i % BM;
      *(uint4*)(dgu + c * C::PDG + r * 16) = make_uint4(0, 0, 0, 0);
    }
  }
  const size_t sub_off = (size_t)s * rows_total * GSB;
#pragma unroll
  for (int i = 0; i < C::FM1; ++i) {
    const int r0 = arow[i] - (lane & 15) + (lane >> 4) * 4;
#pragma unroll
    for (int j = 0; j < C::FN1; ++j) {
      const int n = brow[j];
      const size_t q = sub_off + packed_index<T>(prow0 + r0, n, GSB);
      float hg[4], hu[4], dgv[4], duv[4], av[4];
      Quad<T>::load(hg_saved + q, hg);
      Quad<T>::load(hu_saved + q, hu);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float da = acc[i][j][e];
        const float sg = sigmoid_f(hg[e]);
        const float silu = hg[e] * sg;
        const float dsilu = sg * (1.0f + hg[e] * (1.0f - sg));
        dgv[e] = da * hu[e] * dsilu;
        duv[e] = da * silu;
        av[e] = silu * hu[e];
      }
      Quad<T>::store(dg_out + q, dgv);
      Quad<T>::store(du_out + q, duv);
      Quad<T>::store(act_out + q, av);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        store_elem<T>((T*)(dgu + (n / EPC) * C::PDG + (r0 + e) * 16) + (n % EPC), dgv[e]);
        const int n2 = GSB + n;
        store_elem<T>((T*)(dgu + (n2 / EPC) * C::PDG + (r0 + e) * 16) + (n2 % EPC), duv[e]);
      }
    }
  }
  __syncthreads();

  // ---------------- phase 2: Q^T = [Wg; Wu]^T[d-block] . [dg du]^T ----------------
  auto lw = [&](int i_) -> char* { return i_ ? (smem + C::DGU + C::W2) : (smem + C::DGU); };
  const int wm2 = wave & 1, wn2 = wave >> 1;
  int arow2[C::FM2], brow2[C::FN2];
  bool valid[C::FN2];
#pragma unroll
  for (int i = 0; i < C::FM2; ++i) arow2[i] = wm2 * (C::FM2 * 16) + i * 16 + (lane & 15);
#pragma unroll
  for (int j = 0; j < C::FN2; ++j) {
    brow2[j] = wn2 * (C::FN2 * 16) + j * 16 + (lane & 15);
    valid[j] = tok[brow2[j]] >= 0;
  }
  TransLoader<T, DB, KC, NT> ldW;
  ldW.init(tid);
  const int nblk = (d + DB - 1) / DB;
  const int niter = nblk * C::NKS;
  auto wload = [&](int it) {
    const int db0 = (it / C::NKS) * DB, ks = it % C::NKS;
    ldW.load(ks * KC * EPC, 2 * GSB, d - db0, [&](int kk) -> const char* {
      return kk < GSB ? (const char*)(wg + (size_t)(nb0 + kk) * d + db0)
                      : (const char*)(wu + (size_t)(nb0 + kk - GSB) * d + db0);
    });
  };
  wload(0);
  ldW.store(lw(0));
  __syncthreads();
  T* out = partials + (size_t)s * rows_total * d;
  f32x4 acc2[C::FM2][C::FN2];
  for (int it = 0; it < niter; ++it) {
    const int ks = it % C::NKS;
    if (ks == 0) zero_acc(acc2);
    if (it + 1 < niter) wload(it + 1);
    mma_lds<T, C::FM2, C::FN2, KC, C::PW, C::PDG>(acc2, lw(it & 1), dgu + ks * KC * C::PDG, arow2, brow2, lane);
    if (ks == C::NKS - 1) {
      const int db0 = (it / C::NKS) * DB;
#pragma unroll
      for (int i = 0; i < C::FM2; ++i) {
        const int dd = db0 + arow2[i] - (lane & 15) + (lane >> 4) * 4;
        if (dd >= d) continue;
#pragma unroll
        for (int j = 0; j < C::FN2; ++j) {
          if (!valid[j]) continue;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] = acc2[i][j][e];
          Quad<T>::store(out + (prow0 + brow2[j]) * d + dd, v);
        }
      }
    }
    if (it + 1 < niter) ldW.store(lw((it + 1) & 1));
    __syncthreads();
  }
}

// ===========================================================================
// Backward: per-group weight gradients
// ===========================================================================
template <typename T, int GSB>
struct DwCfg {
  static constexpr int EPC = Elem<T>::EPC;
  // kind 0: out[DB x 2GSB] = X^T . [dg du];  kind 1: out[GSB x DB] = a^T . dY
  static constexpr int PX = Plane<DB>::BYTES;
  static constexpr int PGU = Plane<2 * GSB>::BYTES;
  static constexpr int PACT = Plane<GSB>::BYTES;
  static constexpr int SMEM0 = 2 * KC * (PX + PGU);
  static constexpr int SMEM1 = 2 * KC * (PACT + PX);
  static constexpr int SMEM = cmax(SMEM0, SMEM1);
  // kind 0 waves 2 x 2: 64 d-rows x GSB neurons each
  static constexpr int FM0 = DB / 32, FN0 = 2 * GSB / 32;
  // kind 1: GSB >= 32: 2 x 2 waves of (GSB/2) x 64; GSB = 16: 1 x 4 of 16 x 32
  static constexpr int WM1 = GSB >= 32 ? 2 : 1;
  static constexpr int WN1 = 4 / WM1;
  static constexpr int FM1 = GSB / (16 * WM1), FN1 = DB / (16 * WN1);
};

template <typename T, int GSB>
__global__ __launch_bounds__(NT) void bwd_dw_kernel(const T* __restrict__ x, const T* __restrict__ dy, int d,
                                                    int F, int gs, int nsub, const int32_t* __restrict__ tile_off,
                                                    const int32_t* __restrict__ ptoken, size_t rows_total,
                                                    const T* __restrict__ dg, const T* __restrict__ du,
                                                    const T* __restrict__ act, T* __restrict__ dwg,
                                                    T* __restrict__ dwu, T* __restrict__ dwd) {
  using C = DwCfg<T, GSB>;
  constexpr int EPC = C::EPC;
  extern __shared__ __align__(16) char smem[];
  const int g = blockIdx.x / nsub, s = blockIdx.x % nsub;
  const int db0 = blockIdx.y * DB;
  const int kind = blockIdx.z;
  const int nb0 = g * gs + s * GSB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int p0 = tile_off[g] * BM, p1 = tile_off[g + 1] * BM;  // padded positions of the group
  const int kstep = KC * EPC;
  const int nk = (p1 - p0) / kstep;  // BM is a multiple of kstep
  const size_t sub_off = (size_t)s * rows_total * GSB;
  const int kc_base = p0 / EPC;
  const int kc_end = p1 / EPC;
  const T* src = kind == 0 ? x : dy;
  auto tokrow = [&](int p) -> const char* {
    const int t = ptoken[p];
    return t >= 0 ? (const char*)(src + (size_t)t * d + db0) : nullptr;
  };

  if (kind == 0) {
    auto lx = [&](int i_) -> char* { return i_ ? (smem + KC * C::PX) : (smem); };
    auto lg = [&](int i_) -> char* { return i_ ? (smem + 2 * KC * C::PX + KC * C::PGU) : (smem + 2 * KC * C::PX); };
    TransLoader<T, DB, KC, NT> ldX;
    ldX.init(tid);
    PackedLoader<GSB, KC, NT, 2 * GSB> ldG, ldU;
    ldG.init(tid, (const char*)(dg + sub_off), GSB);
    ldU.init(tid, (const char*)(du + sub_off), GSB);
    const int wm = wave & 1, wn = wave >> 1;
    int arow[C::FM0], brow[C::FN0];
#pragma unroll
    for (int i = 0; i < C::FM0; ++i) arow[i] = wm * (C::FM0 * 16) + i * 16 + (lane & 15);
#pragma unroll
    for (int j = 0; j < C::FN0; ++j) brow[j] = wn * (C::FN0 * 16) + j * 16 + (lane & 15);
    f32x4 acc[C::FM0][C::FN0];
    zero_acc(acc);
    if (nk > 0) {
      ldX.load(p0, p1, d - db0, tokrow);
      ldG.load(kc_base, kc_end);
      ldU.load(kc_base, kc_end);
      ldX.store(lx(0));
      ldG.store(lg(0), 0);
      ldU.store(lg(0), GSB);
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) {
          ldX.load(p0 + (kt + 1) * kstep, p1, d - db0, tokrow);
          ldG.load(kc_base + (kt + 1) * KC, kc_end);
          ldU.load(kc_base + (kt + 1) * KC, kc_end);
        }
        mma_lds<T, C::FM0, C::FN0, KC, C::PX, C::PGU>(acc, lx(kt & 1), lg(kt & 1), arow, brow, lane);
        if (kt + 1 < nk) {
          ldX.store(lx((kt + 1) & 1));
          ldG.store(lg((kt + 1) & 1), 0);
          ldU.store(lg((kt + 1) & 1), GSB);
        }
        __syncthreads();
      }
    }
    // lane: out[d = db0 + row][neuron col] rows (lane>>4)*4+e
#pragma unroll
    for (int i = 0; i < C::FM0; ++i) {
      const int dd = db0 + arow[i] - (lane & 15) + (lane >> 4) * 4;
      if (dd >= d) continue;
#pragma unroll
      for (int j = 0; j < C::FN0; ++j) {
        const int n = brow[j];
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][e];
        T* dst = n < GSB ? dwg + (size_t)(nb0 + n) * d + dd : dwu + (size_t)(nb0 + n - GSB) * d + dd;
        Quad<T>::store(dst, v);
      }
    }
  } else {
    auto la = [&](int i_) -> char* { return i_ ? (smem + KC * C::PACT) : (smem); };
    auto ly = [&](int i_) -> char* { return i_ ? (smem + 2 * KC * C::PACT + KC * C::PX) : (smem + 2 * KC * C::PACT); };
    PackedLoader<GSB, KC, NT> ldA;
    ldA.init(tid, (const char*)(act + sub_off), GSB);
    TransLoader<T, DB, KC, NT> ldY;
    ldY.init(tid);
    const int wm = wave % C::WM1, wn = wave / C::WM1;
    int arow[C::FM1], brow[C::FN1];
#pragma unroll
    for (int i = 0; i < C::FM1; ++i) arow[i] = wm * (C::FM1 * 16) + i * 16 + (lane & 15);
#pragma unroll
    for (int j = 0; j < C::FN1; ++j) brow[j] = wn * (C::FN1 * 16) + j * 16 + (lane & 15);
    f32x4 acc[C::FM1][C::FN1];
    zero_acc(acc);
    if (nk > 0) {
      ldA.load(kc_base, kc_end);
      ldY.load(p0, p1, d - db0, tokrow);
      ldA.store(la(0));
      ldY.store(ly(0));
      __syncthreads();
      for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) {
          ldA.load(kc_base + (kt + 1) * KC, kc_end);
          ldY.load(p0 + (kt + 1) * kstep, p1, d - db0, tokrow);
        }
        mma_lds<T, C::FM1, C::FN1, KC, C::PACT, C::PX>(acc, la(kt & 1), ly(kt & 1), arow, brow, lane);
        if (kt + 1 < nk) {
          ldA.store(la((kt + 1) & 1));
          ldY.store(ly((kt + 1) & 1));
        }
        __syncthreads();
      }
    }
    // lane: out[neuron row][d col]; rows (lane>>4)*4+e are consecutive neurons
#pragma unroll
    for (int i = 0; i < C::FM1; ++i) {
      const int n = arow[i] - (lane & 15) + (lane >> 4) * 4;
#pragma unroll
      for (int j = 0; j < C::FN1; ++j) {
        const int dd = db0 + brow[j];
        if (dd >= d) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][e];
        Quad<T>::store(dwd + (size_t)dd * F + nb0 + n, v);
      }
    }
  }
}

// ===========================================================================
// Launchers
// ===========================================================================
template <auto Kernel>
hipError_t set_smem(int bytes) {
  // once per kernel instantiation
  static const hipError_t err =
      hipFuncSetAttribute((const void*)Kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  return err;
}

template <typename T, int GSB>
hipError_t fwd_t(const FfnShape& s, const void* x, const void* wg, const void* wu, const void* wd,
                 const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, void* hg, void* hu,
                 void* partials, hipStream_t stream) {
  using C = FwdCfg<T, GSB>;
  hipError_t e = set_smem<fwd_grouped_kernel<T, GSB>>(C::SMEM);
  if (e != hipSuccess) return e;
  LaunchTimer timer("fwd_grouped", stream);
  hipLaunchKernelGGL((fwd_grouped_kernel<T, GSB>), dim3(ntiles_max, s.nsub()), dim3(NT), C::SMEM, stream,
                     (const T*)x, (const T*)wg, (const T*)wu, (const T*)wd, s.d_model, s.d_ff, s.group_size,
                     tile_group, ptoken, (size_t)ntiles_max * BM, (T*)hg, (T*)hu, (T*)partials);
  return hipGetLastError();
}

template <typename T, int GSB>
hipError_t dhdx_t(const FfnShape& s, const void* dy, const void* wg, const void* wu, const void* wd,
                  const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, const void* hg,
                  const void* hu, void* dg, void* du, void* act, void* partials, hipStream_t stream) {
  using C = BwdCfg<T, GSB>;
  hipError_t e = set_smem<bwd_dh_dx_kernel<T, GSB>>(C::SMEM);
  if (e != hipSuccess) return e;
  LaunchTimer timer("bwd_dh_dx", stream);
  hipLaunchKernelGGL((bwd_dh_dx_kernel<T, GSB>), dim3(ntiles_max, s.nsub()), dim3(NT), C::SMEM, stream,
                     (const T*)dy, (const T*)wg, (const T*)wu, (const T*)wd, s.d_model, s.d_ff, s.group_size,
                     tile_group, ptoken, (size_t)ntiles_max * BM, (const T*)hg, (const T*)hu, (T*)dg, (T*)du,
                     (T*)act, (T*)partials);
  return hipGetLastError();
}

template <typename T, int GSB>
hipError_t dw_t(const FfnShape& s, const void* x, const void* dy, const int32_t* tile_off,
                const int32_t* ptoken, int rows_total, const void* dg, const void* du, const void* act,
                void* dwg, void* dwu, void* dwd, hipStream_t stream) {
  using C = DwCfg<T, GSB>;
  hipError_t e = set_smem<bwd_dw_kernel<T, GSB>>(C::SMEM);
  if (e != hipSuccess) return e;
  LaunchTimer timer("bwd_dw", stream);
  const dim3 grid(s.groups() * s.nsub(), (s.d_model + DB - 1) / DB, 2);
  hipLaunchKernelGGL((bwd_dw_kernel<T, GSB>), grid, dim3(NT), C::SMEM, stream, (const T*)x, (const T*)dy,
                     s.d_model, s.d_ff, s.group_size, s.nsub(), tile_off, ptoken, (size_t)rows_total,
                     (const T*)dg, (const T*)du, (const T*)act, (T*)dwg, (T*)dwu, (T*)dwd);
  return hipGetLastError();
}

#define ESG_DISPATCH_GSB(T, FN, ...)                        \
  switch (s.gsb()) {                                        \
    case 16: return FN<T, 16>(__VA_ARGS__);                 \
    case 32: return FN<T, 32>(__VA_ARGS__);                 \
    case 64: return FN<T, 64>(__VA_ARGS__);                 \
    case 128:                                               \
      if constexpr (sizeof(T) == 2) return FN<T, 128>(__VA_ARGS__); \
      break;                                                \
    default: break;                                         \
  }                                                         \
  return hipErrorInvalidValue;

template <typename T>
hipError_t fwd_d(const FfnShape& s, const void* x, const void* wg, const void* wu, const void* wd,
                 const int32_t* tg, const int32_t* pt, int nt, void* hg, void* hu, void* part, hipStream_t st) {
  ESG_DISPATCH_GSB(T, fwd_t, s, x, wg, wu, wd, tg, pt, nt, hg, hu, part, st)
}
template <typename T>
hipError_t dhdx_d(const FfnShape& s, const void* dy, const void* wg, const void* wu, const void* wd,
                  const int32_t* tg, const int32_t* pt, int nt, const void* hg, const void* hu, void* dg,
                  void* du, void* act, void* part, hipStream_t st) {
  ESG_DISPATCH_GSB(T, dhdx_t, s, dy, wg, wu, wd, tg, pt, nt, hg, hu, dg, du, act, part, st)
}
template <typename T>
hipError_t dw_d(const FfnShape& s, const void* x, const void* dy, const int32_t* to, const int32_t* pt, int rows,
                const void* dg, const void* du, const void* act, void* dwg, void* dwu, void* dwd, hipStream_t st) {
  ESG_DISPATCH_GSB(T, dw_t, s, x, dy, to, pt, rows, dg, du, act, dwg, dwu, dwd, st)
}

}  // namespace

hipError_t launch_fwd_grouped(const FfnShape& s, const void* x, const void* wg, const void* wu, const void* wd,
                              const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, void* hg_saved,
                              void* hu_saved, void* partials, hipStream_t stream) {
  if (ntiles_max == 0) return hipSuccess;
  return s.dtype == 0 ? fwd_d<float>(s, x, wg, wu, wd, tile_group, ptoken, ntiles_max, hg_saved, hu_saved,
                                     partials, stream)
                      : fwd_d<bf16_t>(s, x, wg, wu, wd, tile_group, ptoken, ntiles_max, hg_saved, hu_saved,
                                      partials, stream);
}

hipError_t launch_rowsum(const FfnShape& s, const void* partials, size_t sub_stride_rows, const int32_t* pinv,
                         void* out, hipStream_t stream) {
  if (s.tokens == 0) return hipSuccess;
  const int epc = s.dtype == 0 ? 4 : 8;
  const size_t vecs = (size_t)s.tokens * (s.d_model / epc);
  // one vector per thread (measured faster than fewer workgroups looping)
  const int blocks = (int)((vecs + 255) / 256 < (1u << 20) ? (vecs + 255) / 256 : (1u << 20));
  LaunchTimer timer("rowsum", stream);
  if (s.dtype == 0)
    hipLaunchKernelGGL(rowsum_kernel<float>, dim3(blocks), dim3(256), 0, stream, (const float*)partials,
                       sub_stride_rows * s.d_model, s.nsub(), pinv, s.tokens, s.k, s.d_model, (float*)out);
  else
    hipLaunchKernelGGL(rowsum_kernel<bf16_t>, dim3(blocks), dim3(256), 0, stream, (const bf16_t*)partials,
                       sub_stride_rows * s.d_model, s.nsub(), pinv, s.tokens, s.k, s.d_model, (bf16_t*)out);
  return hipGetLastError();
}

hipError_t launch_bwd_dh_dx(const FfnShape& s, const void* dy, const void* wg, const void* wu, const void* wd,
                            const int32_t* tile_group, const int32_t* ptoken, int ntiles_max, const void* hg_saved,
                            const void* hu_saved, void* dg, void* du, void* act, void* partials,
                            hipStream_t stream) {
  if (ntiles_max == 0) return hipSuccess;
  return s.dtype == 0 ? dhdx_d<float>(s, dy, wg, wu, wd, tile_group, ptoken, ntiles_max, hg_saved, hu_saved, dg,
                                      du, act, partials, stream)
                      : dhdx_d<bf16_t>(s, dy, wg, wu, wd, tile_group, ptoken, ntiles_max, hg_saved, hu_saved, dg,
                                       du, act, partials, stream);
}

hipError_t launch_bwd_dw(const FfnShape& s, const void* x, const void* dy, const int32_t* tile_off,
                         const int32_t* ptoken, int rows_total, const void* dg, const void* du, const void* act,
                         void* dwg, void* dwu, void* dwd, hipStream_t stream) {
  return s.dtype == 0 ? dw_d<float>(s, x, dy, tile_off, ptoken, rows_total, dg, du, act, dwg, dwu, dwd, stream)
                      : dw_d<bf16_t>(s, x, dy, tile_off, ptoken, rows_total, dg, du, act, dwg, dwu, dwd, stream);
}

}  // namespace esg
