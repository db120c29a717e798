// Device building blocks shared by the esg kernels (gfx950 / CDNA4).
//
// Operand tiles live in LDS in a "K-packed" layout: a tile of R rows (the M or
// N side of a contraction) and KC chunks along K, where one chunk is 16 bytes
// = EPC consecutive K elements of one row (EPC = 8 for bf16, 4 for fp32).
// Chunk (c, r) sits at byte c*PLANE + r*16 with PLANE = R*16 + 16; the extra
// 16 bytes per plane shift consecutive planes by four banks.
//
// The MFMA used is 16x16 with K = 32 (bf16) or 4 (fp32).  Lane l of a wave
// reads chunk (kblock*4 + l/16) of row (fragment_row0 + l%16) for both
// operands, so both see the same K permutation and the product is exact up
// to summation order.  The 16x16 fp32 result sits in the wave as: lane l
// holds rows (l/16)*4 + i, i = 0..3, of column l%16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace esg {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// bf16 storage type (raw bits)
struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct Elem;
template <>
struct Elem<bf16_t> {
  static constexpr int EPC = 8;  // elements per 16-byte chunk
  static constexpr int BYTES = 2;
};
template <>
struct Elem<float> {
  static constexpr int EPC = 4;
  static constexpr int BYTES = 4;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Two floats -> two bf16 packed in one dword (low = a), round to nearest even
// by the hardware convert.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2_t v = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// float -> bf16 bits, round to nearest even.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

template <typename T>
__device__ __forceinline__ float load_elem(const T* p);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p) {
  return *p;
}
template <>
__device__ __forceinline__ float load_elem<bf16_t>(const bf16_t* p) {
  return bf16_to_f32(p->bits);
}

template <typename T>
__device__ __forceinline__ void store_elem(T* p, float v);
template <>
__device__ __forceinline__ void store_elem<float>(float* p, float v) {
  *p = v;
}
template <>
__device__ __forceinline__ void store_elem<bf16_t>(bf16_t* p, float v) {
  p->bits = (uint16_t)f32_to_bf16(v);
}

// Four consecutive elements <-> four floats.
template <typename T>
struct Quad;
template <>
struct Quad<float> {
  static __device__ __forceinline__ void load(const void* p, float (&v)[4]) {
    const float4 q = *(const float4*)p;
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  }
  static __device__ __forceinline__ void store(void* p, const float (&v)[4]) {
    *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
  }
};
// four bf16 values (8 bytes) to fp32
__device__ __forceinline__ void unpack_bf16x4(uint2 q, float (&v)[4]) {
  v[0] = __uint_as_float(q.x << 16);
  v[1] = __uint_as_float(q.x & 0xffff0000u);
  v[2] = __uint_as_float(q.y << 16);
  v[3] = __uint_as_float(q.y & 0xffff0000u);
}

template <>
struct Quad<bf16_t> {
  static __device__ __forceinline__ void load(const void* p, float (&v)[4]) {
    const uint2 q = *(const uint2*)p;
    v[0] = __uint_as_float(q.x << 16);
    v[1] = __uint_as_float(q.x & 0xffff0000u);
    v[2] = __uint_as_float(q.y << 16);
    v[3] = __uint_as_float(q.y & 0xffff0000u);
  }
  static __device__ __forceinline__ void store(void* p, const float (&v)[4]) {
    *(uint2*)p = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
};

// ---------------------------------------------------------------------------
// MFMA: acc += A(16 x K) * B(K x 16) for one K-block of 4 chunks per lane
// group (64 bytes of K per row).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void mma_chunk(f32x4& acc, const uint4& a, const uint4& b, bf16_t) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                               __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_chunk(f32x4& acc, const uint4& a, const uint4& b, float) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

template <int R>
struct Plane {
  static constexpr int BYTES = R * 16 + 16;
};

// Accumulate KC chunks (KC % 4 == 0) of A-rows arow[] x B-rows brow[] held in
// LDS.  arow/brow are the row indices this lane reads (fragment row0 + l%16).
template <typename T, int FM, int FN, int KC, int PA, int PB>
__device__ __forceinline__ void mma_lds(f32x4 (&acc)[FM][FN], const char* la, const char* lb,
                                        const int (&arow)[FM], const int (&brow)[FN], int lane) {
  static_assert(KC % 4 == 0, "K-block is four chunks");
#pragma unroll
  for (int kb = 0; kb < KC / 4; ++kb) {
    const int c = kb * 4 + (lane >> 4);
    uint4 a[FM], b[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) a[i] = *(const uint4*)(la + c * PA + arow[i] * 16);
#pragma unroll
    for (int j = 0; j < FN; ++j) b[j] = *(const uint4*)(lb + c * PB + brow[j] * 16);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) mma_chunk(acc[i][j], a[i], b[j], T{});
  }
}

template <int FM, int FN>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
}
template <int N>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}
template <int A, int B, int C>
__device__ __forceinline__ void zero_acc(f32x4 (&acc)[A][B][C]) {
#pragma unroll
  for (int i = 0; i < A; ++i) zero_acc(acc[i]);
}

// ---------------------------------------------------------------------------
// Loaders: global -> registers (load) -> LDS (store), for one K-stage of KC
// chunks of an R-row operand tile, with NT threads.
// ---------------------------------------------------------------------------

// Rows contiguous along K; each row has its own base pointer (NULL = a row of
// zeros).  Thread t always moves chunk column t % KC.
template <int R, int KC, int NT>
struct RowKLoader {
  static_assert(NT % KC == 0, "threads must cover whole rows");
  static constexpr int RPP = NT / KC;  // rows per pass
  static constexpr int N = (R + RPP - 1) / RPP;
  const char* base[N];
  uint4 v[N];
  int c, r0;

  template <typename RowFn>
  __device__ __forceinline__ void init(int tid, RowFn rowptr) {
    c = tid % KC;
    r0 = tid / KC;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = r0 + i * RPP;
      base[i] = (r < R) ? rowptr(r) : nullptr;
    }
  }
  // kbyte: byte offset of the stage's first chunk; kbytes: row length in bytes
  __device__ __forceinline__ void load(int kbyte, int kbytes) {
    const int off = kbyte + c * 16;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      v[i] = make_uint4(0, 0, 0, 0);
      if (base[i] != nullptr && off < kbytes) v[i] = *(const uint4*)(base[i] + off);
    }
  }
  __device__ __forceinline__ void store(char* lds) const {
    constexpr int P = Plane<R>::BYTES;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int r = r0 + i * RPP;
      if (r < R) *(uint4*)(lds + c * P + r * 16) = v[i];
    }
  }
};

// Source already K-packed in global memory: chunk (kc, r) of a buffer with
// `rows_total` rows at base + (kc*rows_total + r)*16.  Consecutive threads take
// consecutive rows of one chunk plane.  The R rows land at rows
// [row_off, row_off + R) of an LDS tile whose planes hold RT rows.
template <int R, int KC, int NT, int RT = R>
struct PackedLoader {
  static constexpr int TOTAL = R * KC;
  static constexpr int N = (TOTAL + NT - 1) / NT;
  const char* base;
  int rows_total;
  uint4 v[N];
  int tid;

  __device__ __forceinline__ void init(int t, const char* b, int rtot) {
    tid = t;
    base = b;
    rows_total = rtot;
  }
  // kc0: first chunk plane of the stage; kc_end: planes available
  __device__ __forceinline__ void load(int kc0, int kc_end) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + i * NT;
      const int r = idx % R, c = idx / R;
      v[i] = make_uint4(0, 0, 0, 0);
      if (idx < TOTAL && kc0 + c < kc_end)
        v[i] = *(const uint4*)(base + ((size_t)(kc0 + c) * rows_total + r) * 16);
    }
  }
  __device__ __forceinline__ void store(char* lds, int row_off = 0) const {
    constexpr int P = Plane<RT>::BYTES;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int idx = tid + i * NT;
      if (idx < TOTAL) {
        const int r = idx % R, c = idx / R;
        *(uint4*)(lds + c * P + (row_off + r) * 16) = v[i];
      }
    }
  }
};

// Source contiguous along the R side: global row k (one per K element) holds
// the R values of that k contiguously.  A unit is an EPC x EPC block: EPC
// global rows x 16 bytes, transposed in registers into EPC chunks.
template <typename T, int R, int KC, int NT>
struct TransLoader {
  static constexpr int EPC = Elem<T>::EPC;
  static constexpr int RG = R / EPC;  // 16-byte column groups
  static constexpr int UNITS = RG * KC;
  static constexpr int N = (UNITS + NT - 1) / NT;
  static_assert(R % EPC == 0, "rows must fill whole chunks");
  uint4 v[N][EPC];
  int tid;

  __device__ __forceinline__ void init(int t) { tid = t; }

  // kptr(k) -> byte pointer of global row k at R-offset 0, or NULL (zeros);
  // k0: first K element of the stage; kend: K elements available; rlim: R
  // values available in each row (a multiple of EPC).
  template <typename KFn>
  __device__ __forceinline__ void load(int k0, int kend, int rlim, KFn kptr) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int u = tid + i * NT;
      const int rg = u % RG, c = u / RG;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        v[i][e] = make_uint4(0, 0, 0, 0);
        const int k = k0 + c * EPC + e;
        if (u < UNITS && k < kend && rg * EPC < rlim) {
          const char* p = kptr(k);
          if (p != nullptr) v[i][e] = *(const uint4*)(p + rg * 16);
        }
      }
    }
  }

  __device__ __forceinline__ void store(char* lds) const {
    constexpr int P = Plane<R>::BYTES;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int u = tid + i * NT;
      if (u >= UNITS) continue;
      const int rg = u % RG, c = u / RG;
      char* dst = lds + c * P + rg * EPC * 16;
      if constexpr (EPC == 8) {
        // 8x8 transpose of 16-bit values: out chunk j, dword m pairs element j
        // of rows 2m and 2m+1.
        const uint32_t* w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = (const uint32_t*)&v[i][e];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int q = j >> 1;
          uint32_t o[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const uint32_t lo = w[2 * m][q], hi = w[2 * m + 1][q];
            o[m] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
          }
          *(uint4*)(dst + j * 16) = make_uint4(o[0], o[1], o[2], o[3]);
        }
      } else {
        const uint32_t* w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (const uint32_t*)&v[i][e];
#pragma unroll
        for (int j = 0; j < 4; ++j) *(uint4*)(dst + j * 16) = make_uint4(w[0][j], w[1][j], w[2][j], w[3][j]);
      }
    }
  }
};

// Logistic function with the hardware exponential and reciprocal (about one
// ulp each); SiLU(z) = z * sigmoid(z).
__device__ __forceinline__ float sigmoid_f(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// y[t] = sum of the token's partial rows in a fixed order: sub-block by
// sub-block, slots in order within each.  A thread owns one 16-byte vector of one token's output row; the partial
// rows' positions are read for up to KB slots at a time and all their vectors
// are requested before the first is summed, so the k loads overlap.
template <typename T>
__device__ __forceinline__ void add_vec(float (&acc)[Elem<T>::EPC], const uint4& q) {
  if constexpr (Elem<T>::EPC == 8) {
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc[2 * m] += __uint_as_float(w[m] << 16);
      acc[2 * m + 1] += __uint_as_float(w[m] & 0xffff0000u);
    }
  } else {
    acc[0] += __uint_as_float(q.x);
    acc[1] += __uint_as_float(q.y);
    acc[2] += __uint_as_float(q.z);
    acc[3] += __uint_as_float(q.w);
  }
}

// 16-byte load marked nontemporal: the line is not kept in the caches (for data
// read exactly once, such as the partial rows of a row sum).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t w = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(w.x, w.y, w.z, w.w);
}

// Workgroup `bid` of `nblk` (256 threads each) takes every nblk-th run of 256
// vectors.  The partial rows are read once, with nontemporal loads (measured
// about 20% faster than cached loads right after the kernel that wrote them).
template <typename T>
__device__ __forceinline__ void rowsum_range(const T* __restrict__ partials, size_t sub_stride, int nsub,
                                             const int32_t* __restrict__ pinv, int tokens, int k, int d,
                                             T* __restrict__ out, int bid, int nblk) {
  constexpr int EPC = Elem<T>::EPC;
  constexpr int KB = 16;
  const int vpr = d / EPC;  // 16-byte vectors per row
  const size_t total = (size_t)tokens * vpr;
  for (size_t i = (size_t)bid * 256 + threadIdx.x; i < total; i += (size_t)nblk * 256) {
    const int t = (int)(i / vpr), v = (int)(i % vpr);
    float acc[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] = 0.f;
    const int32_t* prow = pinv + (size_t)t * k;
    for (int sb = 0; sb < nsub; ++sb) {
      const T* base = partials + sb * sub_stride + v * EPC;
      for (int j0 = 0; j0 < k; j0 += KB) {
        int p[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) p[j] = j0 + j < k ? prow[j0 + j] : -1;
        uint4 q[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j)
          q[j] = p[j] >= 0 ? load_nt16(base + (size_t)p[j] * d) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < KB; ++j)
          if (p[j] >= 0) add_vec<T>(acc, q[j]);
      }
    }
    T* o = out + (size_t)t * d + v * EPC;
    if constexpr (EPC == 8) {
      *(uint4*)o = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                              pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
    } else {
      *(float4*)o = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

}  // namespace esg
