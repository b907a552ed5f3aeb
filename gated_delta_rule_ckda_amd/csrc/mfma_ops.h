// Device building blocks shared by the chunked-forward kernels: MFMA tile
// products on LDS operands, register-fragment products, raw buffer loads and
// wave reductions.  gfx950 only.
#pragma once

#include "ckda_internal.h"

namespace ckda {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int align16(int x) { return (x + 15) & ~15; }
constexpr int align256(int x) { return (x + 255) & ~255; }
constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// Row stride (in elements of `es` bytes) for LDS operands whose rows are read
// as MFMA fragments (16 rows at a time, four 16-byte pieces of each row's
// first 64 bytes per K slice): the smallest stride of at least n elements
// that is 32 bytes past a multiple of 128.  Measured on gfx950 with the LDS
// bank-conflict counter, that is the stride family with no conflicts for this
// access shape (272- or 144-byte strides cost 25% more LDS cycles).
constexpr int frag_stride(int n, int es) { return ((n * es + 95) / 128 * 128 + 32) / es; }

// ---- MFMA operand types ----------------------------------------------------
// 16x16 output tiles.  The fp32 result of a tile holds, in lane l, rows
// 4*(l/16)+i (i = 0..3) of column l%16.
//
// mmaK: both operands in LDS as [rows][K] with K contiguous (A as [M][K], B as
// B^T = [N][K]); lane l reads row l%16 and the K-slice selected by l/16.
//
// Register-fragment products ("perm" forms): one operand comes straight from
// fp32 accumulators of earlier products.  A lane holding rows 4*lq+i of column
// l16 of a 16-row tile supplies those rows as its K-values, so the contraction
// runs over K in the order (tile, lq, i) instead of the natural order; the LDS
// operand is read in the same permuted order (row fragments at 4*lq and, for
// bf16, 16 + 4*lq within each 32-wide K slice), which leaves the sum unchanged.
// Storage order of rows that are read as permuted-order fragments (bf16 rows
// whose length K is a multiple of 32): logical index 32s + 16h + 4q + i is
// stored at 32s + 8q + 4h + i, so the 8 values lane group q needs for slice s
// are contiguous (one 16-byte LDS read).  Rows of length 16 keep their order.
__host__ __device__ constexpr int perm32(int k) {
  return (k & ~31) | (((k & 15) >> 2) << 3) | (((k & 31) >> 4) << 2) | (k & 3);
}

struct OpBF16 {
  using T = __bf16;
  using Frag = bf16x8;                 // K-slice of 32 per MFMA
  static constexpr int KS = 32;
  static __device__ __forceinline__ T cvt(float x) { return static_cast<__bf16>(x); }
  // storage position of logical index k in a row of length K
  template <int K>
  static __device__ __forceinline__ int pos(int k) { return K % 32 == 0 ? perm32(k) : k; }

  // acc += A[16 x K] * B[16 x K]^T, K a multiple of 16.  A K remainder of 16
  // runs as one more 16x16x32 MFMA whose upper half of K is zero (lanes 32..63
  // supply zeros), so every MFMA accumulating into a tile has the same shape
  // and dependent MFMAs never mix pass counts.
  template <int K>
  static __device__ __forceinline__ void mmaK(f32x4& acc, const T* a, int lda, const T* b, int ldb,
                                              int lane) {
    const int r = lane & 15, kq = lane >> 4;
    const T* pa = a + r * lda;
    const T* pb = b + r * ldb;
    constexpr int N32 = K / 32;
    bf16x8 fa[N32 > 0 ? N32 : 1], fb[N32 > 0 ? N32 : 1];
#pragma unroll
    for (int s = 0; s < N32; ++s) {
      fa[s] = *reinterpret_cast<const bf16x8*>(pa + 32 * s + 8 * kq);
      fb[s] = *reinterpret_cast<const bf16x8*>(pb + 32 * s + 8 * kq);
    }
    bf16x8 ta, tb;
    if constexpr (K % 32 != 0) {
      const bf16x8 z = {};
      ta = kq < 2 ? *reinterpret_cast<const bf16x8*>(pa + 32 * N32 + 8 * kq) : z;
      tb = kq < 2 ? *reinterpret_cast<const bf16x8*>(pb + 32 * N32 + 8 * kq) : z;
    }
#pragma unroll
    for (int s = 0; s < N32; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[s], fb[s], acc, 0, 0, 0);
    if constexpr (K % 32 != 0) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ta, tb, acc, 0, 0, 0);
  }

  // Register fragments of a K-deep contraction from fp32 accumulator tiles
  // t[0 .. K/16): slice s packs tiles 2s and 2s+1 (zeros for a missing 2s+1).
  template <int K>
  static __device__ __forceinline__ void frags(Frag* f, const f32x4* t) {
#pragma unroll
    for (int s = 0; s < (K + 31) / 32; ++s) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[s][i] = cvt(t[2 * s][i]);
        f[s][4 + i] = (2 * s + 1 < K / 16) ? cvt(t[2 * s + 1][i]) : cvt(0.f);
      }
    }
  }
  // Row fragment of an LDS operand in the permuted K order (row = this lane's
  // row, stored in pos<K> order): 16 contiguous bytes, or 8 bytes and zeros
  // for a row of length 16.
  template <int K>
  static __device__ __forceinline__ Frag row_frag(const T* row, int s, int lq) {
    if constexpr (K % 32 == 0) {
      return *reinterpret_cast<const bf16x8*>(row + 32 * s + 8 * lq);
    } else {
      static_assert(K == 16, "row length");
      Frag f;
      const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row + 4 * lq);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f[i] = lo[i];
        f[4 + i] = cvt(0.f);
      }
      return f;
    }
  }
  // acc += A * B over one K-slice, both operands as fragments in the same K order
  static __device__ __forceinline__ void mma(f32x4& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
  // Store 4 (or 2, or 1) consecutive values at p.
  static __device__ __forceinline__ void store4(T* p, f32x4 x) {
    bf16x4 y;
    y[0] = cvt(x[0]); y[1] = cvt(x[1]); y[2] = cvt(x[2]); y[3] = cvt(x[3]);
    *reinterpret_cast<bf16x4*>(p) = y;
  }
  static __device__ __forceinline__ void store2(T* p, float x0, float x1) {
    bf16x2 y;
    y[0] = cvt(x0); y[1] = cvt(x1);
    *reinterpret_cast<bf16x2*>(p) = y;
  }
  static __device__ __forceinline__ void store1(T* p, float x0) { p[0] = cvt(x0); }
};

struct OpF32 {
  using T = float;
  using Frag = f32x4;                  // K-slice of 16 = 4 MFMAs of depth 4
  static constexpr int KS = 16;
  static __device__ __forceinline__ T cvt(float x) { return x; }
  // the permuted fragment order is already contiguous for fp32
  template <int K>
  static __device__ __forceinline__ int pos(int k) { return k; }

  template <int K>
  static __device__ __forceinline__ void mmaK(f32x4& acc, const T* a, int lda, const T* b, int ldb,
                                              int lane) {
    const int r = lane & 15, kq = lane >> 4;
    const T* pa = a + r * lda + kq;
    const T* pb = b + r * ldb + kq;
    float fa[K / 4], fb[K / 4];
#pragma unroll
    for (int s = 0; s < K / 4; ++s) {
      fa[s] = pa[4 * s];
      fb[s] = pb[4 * s];
    }
#pragma unroll
    for (int s = 0; s < K / 4; ++s) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(fa[s], fb[s], acc, 0, 0, 0);
  }

  template <int K>
  static __device__ __forceinline__ void frags(Frag* f, const f32x4* t) {
#pragma unroll
    for (int s = 0; s < K / 16; ++s) f[s] = t[s];
  }
  template <int K>
  static __device__ __forceinline__ Frag row_frag(const T* row, int s, int lq) {
    return *reinterpret_cast<const f32x4*>(row + 16 * s + 4 * lq);
  }
  // MFMA i of a slice contracts over K-value 16s + 4*lq + i in every lane.
  static __device__ __forceinline__ void mma(f32x4& acc, const Frag& a, const Frag& b) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[i], acc, 0, 0, 0);
  }
  static __device__ __forceinline__ void store4(T* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
  static __device__ __forceinline__ void store2(T* p, float x0, float x1) {
    *reinterpret_cast<float2*>(p) = make_float2(x0, x1);
  }
  static __device__ __forceinline__ void store1(T* p, float x0) { p[0] = x0; }
};

// N consecutive values v[0..N) at p (N = 1, 2, 4 or a multiple of 4)
template <class Op, int N>
__device__ __forceinline__ void store_run(typename Op::T* p, const float* v) {
  if constexpr (N == 1) {
    Op::store1(p, v[0]);
  } else if constexpr (N == 2) {
    Op::store2(p, v[0], v[1]);
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4) Op::store4(p + i, f32x4{v[i], v[i + 1], v[i + 2], v[i + 3]});
  }
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---- buffer loads ----------------------------------------------------------
// A raw buffer resource covers a byte range; callers keep every offset inside
// it (rows are clamped to the last valid row), whatever the range-check rules
// for the offset operands are.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           num_bytes, kRsrcWord3);
}

// Cache policy of a buffer load: kStream marks data read once (the gfx950
// "nt" bit), so streamed inputs do not displace lines that are read again
// soon (the workspace blocks the transform pass hands to the state pass).
constexpr int kCached = 0, kStream = 2;

template <int BYTES, int CPOL = kCached>
__device__ __forceinline__ void ldraw(rsrc_t r, int voff, uint32_t* d) {
  if constexpr (BYTES == 2) {
    d[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, CPOL);
  } else if constexpr (BYTES == 4) {
    d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, CPOL);
  } else if constexpr (BYTES == 8) {
    const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, CPOL);
    d[0] = u[0];
    d[1] = u[1];
  } else {
    static_assert(BYTES == 16, "load width");
    const auto u = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, CPOL);
    d[0] = u[0]; d[1] = u[1]; d[2] = u[2]; d[3] = u[3];
  }
}

// element e of a raw row fragment, widened to fp32
template <class IO>
__device__ __forceinline__ float dec(const uint32_t* d, int e) {
  if constexpr (sizeof(typename IO::storage) == 2)
    return __uint_as_float((e & 1) ? (d[e >> 1] & 0xFFFF0000u) : (d[e >> 1] << 16));
  else
    return __uint_as_float(d[e]);
}

__device__ __forceinline__ int iclamp(int x, int hi) { return x < hi ? x : hi; }

// a value known to be equal in all lanes, moved to scalar registers
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint64_t u = static_cast<uint64_t>(x);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ int uniform32(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Row sums over the 64 lanes of a wave of N per-lane values (N = rows, a power
// of two <= 8): a butterfly that halves the values per step.  Returns the sum
// for row (lane >> (6 - log2 N)), the same in all 64/N lanes of that row.
template <int N>
__device__ __forceinline__ float wave_row_sums(float (&v)[N], int lane) {
  int m = 32;
#pragma unroll
  for (int half = N / 2; half >= 1; half /= 2) {
    const bool up = (lane & m) != 0;
    // both rows are reduced with the partner and the lane keeps one: a select
    // between two computed values (selecting between array elements would
    // make the compiler index the array dynamically)
#pragma unroll
    for (int i = 0; i < half; ++i) {
      const float lo = v[i] + __shfl_xor(v[i], m, 64);
      const float hi = v[i + half] + __shfl_xor(v[i + half], m, 64);
      v[i] = up ? hi : lo;
    }
    m >>= 1;
  }
  float s = v[0];
#pragma unroll
  for (int mm = 32 >> ilog2(N); mm >= 1; mm >>= 1) s += __shfl_xor(s, mm, 64);
  return s;
}

// Barrier among the lanes of one wave with LDS visibility (lanes of a wave
// exchange data through LDS between the two sides).
// One tile staged in LDS out to memory as 16-byte pieces, by NTH threads
// (this one is thread t): R rows of ROWB bytes from `st` (row stride LD
// bytes) to rows at `g` + r * gstride bytes; rows >= rmax are not written.
template <int R, int ROWB, int LD, int NTH>
__device__ __forceinline__ void flush_rows(const unsigned char* st, unsigned char* g, int64_t gstride,
                                           int rmax, int t) {
  static_assert(ROWB % 16 == 0 && LD % 16 == 0, "rows in 16-byte pieces");
  constexpr int PPR = ROWB / 16, NP = R * PPR;
#pragma unroll
  for (int u = 0; u < (NP + NTH - 1) / NTH; ++u) {
    const int pc = t + NTH * u;
    if (NP % NTH == 0 || pc < NP) {
      const int r = pc / PPR, c = pc % PPR;
      if (r < rmax)
        *reinterpret_cast<uint4*>(g + r * gstride + 16 * c) =
            *reinterpret_cast<const uint4*>(st + r * LD + 16 * c);
    }
  }
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace ckda
