// Chunked forward of the (Complex) Kimi Delta Attention recurrence, fused into
// one kernel: one workgroup owns one (sequence, head, dv-tile) chain, walks the
// sequence chunk by chunk and keeps the fp32 state tile on chip, so every
// input byte is read from HBM once and every output byte written once.
//
// The recurrence (picx.dev summary of the Complex KDA paper, section
// "Background": transition A_t = (I - beta_t k_t k_t^T) Diag(alpha_t), completed
// with the delta-rule write beta_t k_t v_t^T and the read-out o_t = S_t^T q_t).
// Within a chunk of C tokens with entry state S0, with the per-channel decay
// D(r<-j) = prod_{j<s<=r} alpha_s:
//
//   (I + A) U = Diag(beta) (V - Kt S0),     A_rj = beta_r <k_r . D(r<-j), k_j>   (j < r)
//   O  = Qt S0 + P U,                       P_rj = <q_r . D(r<-j), k_j>          (j <= r)
//   S' = Diag(g) S0 + Kh^T U
//
// with Kt_r = D(r<-start) . k_r, Qt_r = D(r<-start) . q_r, Kh_j = D(end<-j) . k_j
// and g = D(end<-start).
//
// Gate prefix.  The chunk's running product Ft_r = prod_{s<=r} alpha_s (per
// channel, fp32) carries the sign and the magnitude of the decay together:
// signs are exact under multiplication, and an exact zero gate makes every
// later product exactly zero.  When every |Ft_r| of the chunk lies in
// [2^-100, 2^10] (the chunk is "regular"), D(r<-j) = Ft_r * (1 / Ft_j) with no
// factor able to overflow, and the chunk runs in the ratio form:
//
//   Lk = k . Ft (= Kt),  Lq = q . Ft (= Qt),  Rk = k / Ft,  Kh = g . Rk,
//   A = tril(Diag(beta rk) Lk Rk^T Diag(rk), -1),  P = tril(Lq Rk^T).
//
// q and k enter raw; the in-op L2 normalisation (dormouse review "RoPE into the
// KDA q/k path", section 2) is applied as row scales rq, rk: A gets
// beta_r rk_r rk_j, Kt's rows get beta rk, U's rows get rk (U' = Diag(rk) U is
// what P and Kh^T multiply), and O's rows get rq.
//
// Chunks that are not regular (an exact zero gate, gates so small that the
// running product underflows the range, or non-finite values) run token by
// token on an LDS copy of the fp32 state instead: exact, slower, and absent
// from realistic gate distributions.
//
// Per regular chunk, on one workgroup of eight waves (wave w owns rows
// w*C/8 .. of the chunk in the element-wise phases):
//   1  decode the prefetched inputs, issue the next chunk's loads, running
//      products within the wave's rows, row norms
//   2  chunk-level products Ft, regularity vote, operands Lk, Lq, Rk
//   3  A and P^T on MFMA (bf16 -> fp32; fp32 MFMA for fp32 inputs)
//   4  Kt^T, Kh^T (transposed);  X = (I + A)^{-1}: 16x16 diagonal blocks by
//      forward substitution, then the off-diagonal blocks on fp32 MFMA
//   5  W^T = (Diag(beta rk) Kt)^T X^T,  Ubar = X (Diag(beta) V)    (MFMA)
//   6  U = Ubar - W S0                                             (MFMA)
//   7  O^T = S0^T Qt^T + U'^T P^T,  S' = Diag(g) S0 + Kh^T U'       (MFMA)
#include "ckda_internal.h"

namespace ckda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr float kRegularMin = 0x1p-100f;
constexpr float kRegularMax = 0x1p+10f;

constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int align16(int x) { return (x + 15) & ~15; }
constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// ---- MFMA operand types ----------------------------------------------------
// Both operands of every product are stored in LDS as [rows][K] with K (the
// contraction index) contiguous: A as [M][K], B as B^T = [N][K].  Lane l of a
// 16x16 tile reads row l%16 and a K-slice selected by l/16; the fp32 result
// holds rows 4*(l/16)+i, column l%16 (i = 0..3).
struct OpBF16 {
  using T = __bf16;
  static __device__ __forceinline__ T cvt(float x) { return static_cast<__bf16>(x); }
  // acc += A[16 x K] * B[16 x K]^T, K a compile-time multiple of 16: all
  // fragments are read before the MFMAs issue.  A K remainder of 16 runs as
  // one more 16x16x32 MFMA whose upper half of K is zero (lanes 32..63 supply
  // zeros), so every MFMA accumulating into a tile has the same shape and
  // dependent MFMAs never mix pass counts.
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
  static __device__ __forceinline__ T cvt(float x) { return x; }
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

// N (1 or 2) consecutive values x[i] at p
template <class Op, int N>
__device__ __forceinline__ void store_pair(typename Op::T* p, const float (&x)[N]) {
  if constexpr (N == 2)
    Op::store2(p, x[0], x[1]);
  else
    Op::store1(p, x[0]);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---- buffer loads ----------------------------------------------------------
// A raw buffer resource covers one chunk's rows of one head.  Callers clamp
// every row offset to the chunk's last valid row, so each access lies inside
// the tensor whatever the range-check rules for the offset operands are.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           num_bytes, kRsrcWord3);
}

template <int BYTES>
__device__ __forceinline__ void ldraw(rsrc_t r, int voff, uint32_t* d) {
  if constexpr (BYTES == 2) {
    d[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0);
  } else if constexpr (BYTES == 4) {
    d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0);
  } else if constexpr (BYTES == 8) {
    const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0);
    d[0] = u[0];
    d[1] = u[1];
  } else {
    static_assert(BYTES == 16, "load width");
    const auto u = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
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

// ---- compile-time configuration and LDS map ---------------------------------
template <class OpT, class IOT, int C_, int DK_, int DV_, int DVT_>
struct Cfg {
  using Op = OpT;
  using IO = IOT;
  using T = typename Op::T;
  static constexpr int NW = 8, NT = 64 * NW;          // waves, threads
  static constexpr int C = C_, DK = DK_, DV = DV_, DVT = DVT_;
  static constexpr int NSPLIT = DV / DVT;
  static constexpr int NB = C / 16;                  // 16-row MFMA blocks per chunk
  static constexpr int RPW = C / NW;                 // rows per wave in the element-wise phases
  static constexpr int CPT = DK >= 64 ? DK / 64 : 1; // channels per lane
  static constexpr int NCG = DK / CPT;               // active lanes per wave
  static constexpr int ES = static_cast<int>(sizeof(T));
  static constexpr int IOES = static_cast<int>(sizeof(typename IO::storage));
  static constexpr int PAD = 16 / ES;
  static constexpr int LDK = DK + PAD;               // stride of [*][DK] operands
  static constexpr int LDC = C + PAD;                // stride of [*][C] operands
  static constexpr int LDF = C + 4;                  // stride of fp32 [C][C] buffers
  static constexpr int TSCR = 16 * 20;               // per-wave fp32 scratch (16x16 + pad)

  static constexpr int NST = (DK / 16) * (DVT / 16); // state tiles
  static constexpr int NSW = (NST + NW - 1) / NW;
  static constexpr int NUT = (C / 16) * (DVT / 16);  // U tiles
  static constexpr int NUW = (NUT + NW - 1) / NW;
  static constexpr int NCP = DVT / 2;                // v column pairs
  static constexpr int RPL = (C * NCP + NT - 1) / NT; // v rows per thread
  static constexpr int VW = (2 * IOES) / 4;          // dwords per v column pair
  static constexpr int QB = CPT * IOES;              // bytes of q (or k) per row and lane
  static constexpr int QW = (QB + 3) / 4;

  // token-by-token path: float4 column groups x row groups
  static constexpr int FCG = DVT / 4;
  static constexpr int FRG = DK < NT / FCG ? DK : NT / FCG;
  static constexpr int FRPT = DK / FRG;
  static constexpr int FACT = FRG * FCG;

  // byte offsets
  static constexpr int O_S = 0;                                   // S^T   [DVT][LDK] T
  static constexpr int O_LQ = align16(O_S + DVT * LDK * ES);      // Lq = Qt [C][LDK]
  static constexpr int O_X = align16(O_LQ + C * LDK * ES);        // region X
  static constexpr int O_LK = O_X;                                //   Lk   [C][LDK]
  static constexpr int O_RK = O_LK + C * LDK * ES;                //   Rk   [C][LDK]
  static constexpr int O_KTT = O_X;                               //   Kt^T [DK][LDC] (after A, P)
  static constexpr int O_KHT = O_KTT + DK * LDC * ES;             //   Kh^T [DK][LDC]
  static constexpr int SZ_X = align16(cmax(cmax(2 * C * LDK * ES, 2 * DK * LDC * ES),
                                           DK * DVT * 4));        //   | fp32 state (token path)
  static constexpr int O_TS = O_X + SZ_X;                         // fp32 scratch [NB][TSCR]
  static constexpr int O_VT = align16(O_TS + NB * TSCR * 4);      // (beta V)^T [DVT][LDC]
  static constexpr int O_AT = align16(O_VT + DVT * LDC * ES);     // A^T fp32 | -W | partials
  static constexpr int SZ_AT = align16(cmax(cmax(C * LDF * 4, C * LDK * ES),
                                            (2 * FRG * DVT + FRG) * 4));
  static constexpr int O_XF = O_AT + SZ_AT;                       // X fp32 [C][LDF] | U'^T
  static constexpr int SZ_XF = align16(cmax(C * LDF * 4, DVT * LDC * ES));
  static constexpr int O_XB = O_XF + SZ_XF;                       // X operand copy [C][LDC]
  static constexpr int O_P = align16(O_XB + C * LDC * ES);        // P     [C][LDC]
  static constexpr int O_G = align16(O_P + C * LDC * ES);         // wave-row products [NW][DK]
  static constexpr int O_GC = O_G + NW * DK * 4;                  // g     [DK] fp32
  static constexpr int O_RQ = O_GC + DK * 4;                      // rq    [C]
  static constexpr int O_RK2 = O_RQ + C * 4;                      // rk    [C]
  static constexpr int O_BETA = O_RK2 + C * 4;                    // beta  [C]
  static constexpr int O_FLAG = O_BETA + C * 4;                   // regularity votes [NW]
  static constexpr int LDS_BYTES = align16(O_FLAG + NW * 4);

  static_assert(C % 16 == 0 && DK % 16 == 0 && DVT % 16 == 0 && DV % DVT == 0, "tile sizes");
  static_assert(NB <= NW && RPW >= 1 && (RPW & (RPW - 1)) == 0 && RPW <= 8, "row split");
  static_assert(DK <= 128 && NCG <= 64, "two channels per lane at most");
  static_assert(NT % NCP == 0 && (NT / NCP) * RPL >= C, "v tile mapping");
  static_assert(DK % FRG == 0 && FACT <= NT, "token path mapping");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// ---- chunk input prefetch ---------------------------------------------------
// Raw (undecoded) registers of one chunk's inputs for this thread.  The next
// chunk's loads are issued into them right after the current chunk has been
// decoded, so HBM latency hides behind a whole chunk of compute.  Row offsets
// are clamped to the chunk's last valid row; padded rows are replaced after
// the load (q = k = v = 0, alpha = 1, beta = 0: identity tokens).
template <class Cfg>
struct Prefetch {
  uint32_t q[Cfg::RPW][Cfg::QW], k[Cfg::RPW][Cfg::QW], al[Cfg::RPW][Cfg::CPT];
  uint32_t v[Cfg::RPL][Cfg::VW];
  uint32_t vb[Cfg::RPL];
  uint32_t bt;
};

template <class Cfg>
__device__ __forceinline__ void issue_loads(Prefetch<Cfg>& pf, const FwdArgs& a, int64_t t,
                                            int Ln, int h, int dv0, int tid, int r0,
                                            bool scan_on, int c0ch) {
  constexpr int DK = Cfg::DK, ES = Cfg::IOES;
  const int H = a.H;
  const int krow = H * DK * ES;   // bytes per token in q / k
  const int arow = H * DK * 4;    // bytes per token in alpha
  const int vrow = H * a.dv * ES; // bytes per token in v
  const int64_t qk_off = (t * H + h) * static_cast<int64_t>(DK);
  if (scan_on) {
    const rsrc_t rq = make_rsrc(static_cast<const char*>(a.q) + qk_off * ES, Ln * krow);
    const rsrc_t rk = make_rsrc(static_cast<const char*>(a.k) + qk_off * ES, Ln * krow);
    const rsrc_t ra = make_rsrc(a.alpha + qk_off, Ln * arow);
#pragma unroll
    for (int i = 0; i < Cfg::RPW; ++i) {
      const int row = iclamp(r0 + i, Ln - 1);
      ldraw<Cfg::QB>(rq, c0ch * ES + row * krow, pf.q[i]);
      ldraw<Cfg::QB>(rk, c0ch * ES + row * krow, pf.k[i]);
      ldraw<Cfg::CPT * 4>(ra, c0ch * 4 + row * arow, pf.al[i]);
    }
  }
  // v tile: column pair cp, rows rg * RPL + i
  const rsrc_t rv = make_rsrc(static_cast<const char*>(a.v) +
                                  ((t * H + h) * static_cast<int64_t>(a.dv) + dv0) * ES,
                              Ln * vrow);
  const rsrc_t rb = make_rsrc(a.beta + t * H + h, Ln * H * 4);
  const int cp = tid % Cfg::NCP, rg = tid / Cfg::NCP;
#pragma unroll
  for (int i = 0; i < Cfg::RPL; ++i) {
    const int j = iclamp(rg * Cfg::RPL + i, Ln - 1);
    ldraw<Cfg::VW * 4>(rv, 2 * cp * ES + j * vrow, pf.v[i]);
    pf.vb[i] = __builtin_amdgcn_raw_buffer_load_b32(rb, j * H * 4, 0, 0);
  }
  pf.bt = __builtin_amdgcn_raw_buffer_load_b32(rb, iclamp(tid, Ln - 1) * H * 4, 0, 0);
}

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

// ---- token-by-token path for irregular chunks ---------------------------------
// The state tile moves to LDS as fp32 [DK][DVT]; each token then applies
// S <- Diag(alpha) S; w = S^T k_hat; S += beta k_hat (v - w)^T;
// o = scale S^T q_hat (computed as y + beta (k_hat.q_hat)(v - w) with
// y = S~^T q_hat), with two column reductions over row groups per token.
// The pointers and sizes come as scalar arguments: a reference to the kernel's
// argument block would force a private copy of it, and values loaded from
// private memory count as lane-varying (every buffer load built from them would
// then run in a loop over distinct descriptors).
template <class Cfg>
__device__ __forceinline__ void token_path(const void* gq_, const void* gk_, const float* galpha,
                                        const void* gv_, const float* gbeta, void* go_, int H,
                                        int dv, float scale, int64_t t0, int L, int h, int dv0,
                                        f32x4* sacc, unsigned char* smem, int tid) {
  using IO = typename Cfg::IO;
  using ST = typename IO::storage;
  constexpr int DK = Cfg::DK, DVT = Cfg::DVT, NW = Cfg::NW;
  constexpr int FCG = Cfg::FCG, FRG = Cfg::FRG, FRPT = Cfg::FRPT, ES = Cfg::IOES;
  constexpr int NTN = DVT / 16;
  float* sSt = reinterpret_cast<float*>(smem + Cfg::O_X);
  f32x4* sPw = reinterpret_cast<f32x4*>(smem + Cfg::O_AT);
  f32x4* sPy = sPw + FRG * FCG;
  float* sKQ = reinterpret_cast<float*>(sPy + FRG * FCG);
  const float* srq = reinterpret_cast<const float*>(smem + Cfg::O_RQ);
  const float* srk = reinterpret_cast<const float*>(smem + Cfg::O_RK2);
  const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, lq = lane >> 4;

#pragma unroll
  for (int u = 0; u < Cfg::NSW; ++u) {
    const int t = wave + NW * u;
    if (t < Cfg::NST) {
      const int c = 16 * (t / NTN) + 4 * lq, dv = 16 * (t % NTN) + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) sSt[(c + i) * DVT + dv] = sacc[u][i];
    }
  }
  __syncthreads();

  const bool act = tid < Cfg::FACT;
  const int fcg = tid % FCG, frg = tid / FCG;
  const int c0 = frg * FRPT;
  const int krow = H * DK;  // elements per token in q / k / alpha
  const int64_t base = (t0 * H + h) * static_cast<int64_t>(DK);
  const rsrc_t rq = make_rsrc(static_cast<const char*>(gq_) + base * ES, L * krow * ES);
  const rsrc_t rk = make_rsrc(static_cast<const char*>(gk_) + base * ES, L * krow * ES);
  const rsrc_t ra = make_rsrc(galpha + base, L * krow * 4);
  const ST* gv = static_cast<const ST*>(gv_);
  ST* go = static_cast<ST*>(go_);

  for (int r = 0; r < L; ++r) {
    float kh[FRPT];
    f32x4 s[FRPT];
    float bt = 0.f;
    if (act) {
      const float rqr = srq[r], rkr = srk[r];
      float qh[FRPT], al[FRPT];
#pragma unroll
      for (int i = 0; i < FRPT; ++i) {
        uint32_t tq[1], tk[1], ta[1];
        ldraw<ES>(rq, ((r * krow) + c0 + i) * ES, tq);
        ldraw<ES>(rk, ((r * krow) + c0 + i) * ES, tk);
        ldraw<4>(ra, ((r * krow) + c0 + i) * 4, ta);
        qh[i] = dec<IO>(tq, 0) * rqr;
        kh[i] = dec<IO>(tk, 0) * rkr;
        al[i] = __uint_as_float(ta[0]);
      }
      bt = gbeta[(t0 + r) * H + h];
      f32x4 pw = {0.f, 0.f, 0.f, 0.f}, py = pw;
      float pkq = 0.f;
#pragma unroll
      for (int i = 0; i < FRPT; ++i) {
        s[i] = *reinterpret_cast<const f32x4*>(sSt + (c0 + i) * DVT + 4 * fcg) * al[i];
        pw += s[i] * kh[i];
        py += s[i] * qh[i];
        pkq += kh[i] * qh[i];
      }
      sPw[frg * FCG + fcg] = pw;
      sPy[frg * FCG + fcg] = py;
      if (fcg == 0) sKQ[frg] = pkq;
    }
    __syncthreads();
    if (act) {
      f32x4 w = {0.f, 0.f, 0.f, 0.f}, y = w;
      float kq = 0.f;
#pragma unroll 4
      for (int g = 0; g < FRG; ++g) {
        w += sPw[g * FCG + fcg];
        y += sPy[g * FCG + fcg];
        kq += sKQ[g];
      }
      const int64_t vo = ((t0 + r) * H + h) * static_cast<int64_t>(dv) + dv0 + 4 * fcg;
      const f32x4 vv = {IO::load(gv, vo), IO::load(gv, vo + 1), IO::load(gv, vo + 2),
                        IO::load(gv, vo + 3)};
      const f32x4 d = vv - w;
#pragma unroll
      for (int i = 0; i < FRPT; ++i)
        *reinterpret_cast<f32x4*>(sSt + (c0 + i) * DVT + 4 * fcg) = s[i] + (bt * kh[i]) * d;
      if (frg == 0) IO::store4(go + vo, (y + (bt * kq) * d) * scale);
    }
    __syncthreads();
  }

#pragma unroll
  for (int u = 0; u < Cfg::NSW; ++u) {
    const int t = wave + NW * u;
    if (t < Cfg::NST) {
      const int c = 16 * (t / NTN) + 4 * lq, dv = 16 * (t % NTN) + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[u][i] = sSt[(c + i) * DVT + dv];
    }
  }
}

template <class Cfg>
__global__ __launch_bounds__(Cfg::NT, 1) void fwd_kernel(FwdArgs a) {
  using Op = typename Cfg::Op;
  using IO = typename Cfg::IO;
  using T = typename Cfg::T;
  using ST = typename IO::storage;
  constexpr int C = Cfg::C, DK = Cfg::DK, DVT = Cfg::DVT, NB = Cfg::NB, NW = Cfg::NW;
  constexpr int NT = Cfg::NT, RPW = Cfg::RPW, CPT = Cfg::CPT, NCG = Cfg::NCG;
  constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC, LDF = Cfg::LDF;
  constexpr int NTN = DVT / 16;

  extern __shared__ __align__(16) unsigned char smem[];
  T* sS = reinterpret_cast<T*>(smem + Cfg::O_S);
  T* sLq = reinterpret_cast<T*>(smem + Cfg::O_LQ);
  T* sLk = reinterpret_cast<T*>(smem + Cfg::O_LK);
  T* sRk = reinterpret_cast<T*>(smem + Cfg::O_RK);
  T* sKtT = reinterpret_cast<T*>(smem + Cfg::O_KTT);
  T* sKhT = reinterpret_cast<T*>(smem + Cfg::O_KHT);
  float* sTS = reinterpret_cast<float*>(smem + Cfg::O_TS);
  T* sVT = reinterpret_cast<T*>(smem + Cfg::O_VT);
  float* sAT = reinterpret_cast<float*>(smem + Cfg::O_AT);
  T* sWn = reinterpret_cast<T*>(smem + Cfg::O_AT);
  float* sXf = reinterpret_cast<float*>(smem + Cfg::O_XF);
  T* sUn = reinterpret_cast<T*>(smem + Cfg::O_XF);
  T* sXb = reinterpret_cast<T*>(smem + Cfg::O_XB);
  T* sP = reinterpret_cast<T*>(smem + Cfg::O_P);
  float* sG = reinterpret_cast<float*>(smem + Cfg::O_G);
  float* sg = reinterpret_cast<float*>(smem + Cfg::O_GC);
  float* srq = reinterpret_cast<float*>(smem + Cfg::O_RQ);
  float* srk = reinterpret_cast<float*>(smem + Cfg::O_RK2);
  float* sbeta = reinterpret_cast<float*>(smem + Cfg::O_BETA);
  int* sFlag = reinterpret_cast<int*>(smem + Cfg::O_FLAG);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15, lq = lane >> 4;

  // ---- which chain: (sequence, head) pairs of one dv-split sit 8 workgroups
  // apart so that both tiles of a pair land on the same XCD (their shared
  // q/k/alpha reads then hit one L2).
  const int64_t nblk = gridDim.x;
  const int64_t b = blockIdx.x;
  int64_t pair;
  int split;
  if (Cfg::NSPLIT > 1 && nblk % (8 * Cfg::NSPLIT) == 0) {
    const int64_t xcd = b % 8, slot = b / 8;
    pair = (slot / Cfg::NSPLIT) * 8 + xcd;
    split = static_cast<int>(slot % Cfg::NSPLIT);
  } else {
    pair = b / Cfg::NSPLIT;
    split = static_cast<int>(b % Cfg::NSPLIT);
  }
  const int H = a.H;
  const int64_t n = pair / H;
  const int h = static_cast<int>(pair % H);
  int64_t bos, eos;
  if (a.cu_seqlens) {
    // the same for every lane; said so, the loop bounds and the buffer
    // descriptors built from them stay in scalar registers
    bos = uniform64(a.cu_seqlens[n]);
    eos = uniform64(a.cu_seqlens[n + 1]);
  } else {
    bos = n * a.T;
    eos = bos + a.T;
  }
  const int dv0 = split * DVT;
  ST* go = static_cast<ST*>(a.o);

  // ---- state tile in accumulator layout: tile t = wave + NW*u covers rows
  // c = 16*(t / NTN) + 4*lq + i, columns dv = 16*(t % NTN) + l16.
  f32x4 sacc[Cfg::NSW];
  const int64_t st_base = (n * H + h) * static_cast<int64_t>(DK) * a.dv + dv0;
#pragma unroll
  for (int u = 0; u < Cfg::NSW; ++u) {
    const int t = wave + NW * u;
    sacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (t < Cfg::NST && a.h0) {
      const int c = 16 * (t / NTN) + 4 * lq, dv = 16 * (t % NTN) + l16;
#pragma unroll
      for (int i = 0; i < 4; ++i) sacc[u][i] = a.h0[st_base + static_cast<int64_t>(c + i) * a.dv + dv];
    }
  }
#pragma unroll
  for (int u = 0; u < Cfg::NSW; ++u) {
    const int t = wave + NW * u;
    if (t < Cfg::NST) {
      const int c = 16 * (t / NTN) + 4 * lq, dv = 16 * (t % NTN) + l16;
      Op::store4(sS + dv * LDK + c, sacc[u]);
    }
  }
  // The blocks above the diagonal of P and of X's operand copy are never
  // written later: zero both buffers once.
  for (int e = tid; e < C * LDC; e += NT) {
    sP[e] = Op::cvt(0.f);
    sXb[e] = Op::cvt(0.f);
  }

  const bool use_l2 = a.use_l2norm != 0;
  const bool scan_on = lane < NCG;
  const int c0ch = lane * CPT;       // first channel of this lane
  const int r0 = wave * RPW;         // first chunk row of this wave
  const int vcp = tid % Cfg::NCP, vrg = tid / Cfg::NCP;

  Prefetch<Cfg> pf;
  if (bos < eos)
    issue_loads<Cfg>(pf, a, bos, static_cast<int>((eos - bos) < C ? (eos - bos) : C), h, dv0, tid,
                     r0, scan_on, c0ch);

  for (int64_t t0 = bos; t0 < eos; t0 += C) {
    const int L = static_cast<int>((eos - t0) < C ? (eos - t0) : C);

    // ================= 1: decode, next loads, running products, norms =======
    float xq[RPW][CPT], xk[RPW][CPT], F[RPW][CPT];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const bool in = scan_on && (r0 + i < L);
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        xq[i][c] = in ? dec<IO>(pf.q[i], c) : 0.f;
        xk[i][c] = in ? dec<IO>(pf.k[i], c) : 0.f;
        F[i][c] = in ? __uint_as_float(pf.al[i][c]) : 1.f;
      }
    }
    // (beta V)^T tile: this thread's column pair over RPL rows
#pragma unroll
    for (int i = 0; i < Cfg::RPL; ++i) {
      const int j = vrg * Cfg::RPL + i;
      if (j < C) {
        const float bj = (j < L) ? __uint_as_float(pf.vb[i]) : 0.f;
        sVT[(2 * vcp) * LDC + j] = Op::cvt(dec<IO>(pf.v[i], 0) * bj);
        sVT[(2 * vcp + 1) * LDC + j] = Op::cvt(dec<IO>(pf.v[i], 1) * bj);
      }
    }
    if (tid < C) sbeta[tid] = (tid < L) ? __uint_as_float(pf.bt) : 0.f;
    // the next chunk's inputs stream in while this chunk is processed
    if (t0 + C < eos)
      issue_loads<Cfg>(pf, a, t0 + C, static_cast<int>((eos - t0 - C) < C ? (eos - t0 - C) : C), h,
                       dv0, tid, r0, scan_on, c0ch);

    // running products over this wave's rows; their totals go to sG
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      float f = 1.f;
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        f *= F[i][c];
        F[i][c] = f;
      }
      if (scan_on) sG[wave * DK + c0ch + c] = f;
    }
    // row norms over all channels of the wave's rows
    {
      float pq[RPW], pk[RPW];
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        pq[i] = 0.f;
        pk[i] = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          pq[i] += xq[i][c] * xq[i][c];
          pk[i] += xk[i][c] * xk[i][c];
        }
      }
      const float sq = wave_row_sums<RPW>(pq, lane);
      const float sk = wave_row_sums<RPW>(pk, lane);
      constexpr int LPR = 64 / RPW;  // lanes per row
      if ((lane & (LPR - 1)) == 0) {
        const int row = r0 + lane / LPR;
        srq[row] = use_l2 ? __fdiv_rn(1.f, __fsqrt_rn(sq + kL2Eps)) : 1.f;
        srk[row] = use_l2 ? __fdiv_rn(1.f, __fsqrt_rn(sk + kL2Eps)) : 1.f;
      }
    }
    __syncthreads();  // B1

    // ================= 2: chunk products, regularity, operands ===============
    float kt[RPW][CPT], kh[RPW][CPT];
    {
      bool ok = true;
      if (scan_on) {
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          float gpre = 1.f, g = 1.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            const float gw = sG[w * DK + c0ch + c];
            if (w < wave) gpre *= gw;
            g *= gw;
          }
          if (wave == 0) sg[c0ch + c] = g;
#pragma unroll
          for (int i = 0; i < RPW; ++i) {
            const float ft = gpre * F[i][c];
            const float mag = fabsf(ft);
            ok = ok && (mag >= kRegularMin) && (mag <= kRegularMax);
            const float rinv = __builtin_amdgcn_rcpf(ft);
            kt[i][c] = xk[i][c] * ft;    // Lk = Kt
            xq[i][c] = xq[i][c] * ft;    // Lq = Qt
            xk[i][c] = xk[i][c] * rinv;  // Rk
            kh[i][c] = xk[i][c] * g;     // Kh
          }
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          const int r = r0 + i;
          store_pair<Op, CPT>(sLk + r * LDK + c0ch, kt[i]);
          store_pair<Op, CPT>(sLq + r * LDK + c0ch, xq[i]);
          store_pair<Op, CPT>(sRk + r * LDK + c0ch, xk[i]);
        }
      }
      const bool wave_ok = __all(ok);
      if (lane == 0) sFlag[wave] = wave_ok ? 1 : 0;
    }
    __syncthreads();  // B2
    int votes = 1;
#pragma unroll
    for (int w = 0; w < NW; ++w) votes &= sFlag[w];
    const bool regular = __builtin_amdgcn_readfirstlane(votes) != 0;  // the same in every lane

    if (!regular) {
      token_path<Cfg>(a.q, a.k, a.alpha, a.v, a.beta, a.o, H, a.dv, a.scale, t0, L, h, dv0, sacc,
                      smem, tid);
    } else {
      // ================= 3: A and P^T on MFMA ===============================
      {
        constexpr int NPT = NB * (NB + 1) / 2;  // lower 16x16 blocks per matrix
        constexpr int NU = (2 * NPT + NW - 1) / NW;
#pragma unroll 1
        for (int u = 0; u < NU; ++u) {
          const int tt = wave + NW * u;
          if (tt < 2 * NPT) {
            const bool isA = tt < NPT;
            int idx = isA ? tt : tt - NPT;
            int I = 0;
            while (idx > I) {
              idx -= I + 1;
              ++I;
            }
            const int J = idx;  // 0..I
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            if (isA) {
              Op::template mmaK<DK>(acc, sLk + 16 * I * LDK, LDK, sRk + 16 * J * LDK, LDK, lane);
              // rows r = 16I + 4lq + i, column j = 16J + l16; store A^T[j][r]
              const int j = 16 * J + l16;
              const float sj = srk[j];
              f32x4 out;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int r = 16 * I + 4 * lq + i;
                const float v = acc[i] * sbeta[r] * srk[r] * sj;
                out[i] = (I == J && j >= r) ? 0.f : v;
              }
              *reinterpret_cast<f32x4*>(sAT + j * LDF + 16 * I + 4 * lq) = out;
              if (I == J) {
                // the diagonal block also goes row-major into the diagonal
                // block of X's buffer, where the substitution reads it and then
                // overwrites it with X_II
#pragma unroll
                for (int i = 0; i < 4; ++i) sXf[(16 * I + 4 * lq + i) * LDF + 16 * I + l16] = out[i];
              }
            } else {
              Op::template mmaK<DK>(acc, sRk + 16 * J * LDK, LDK, sLq + 16 * I * LDK, LDK, lane);
              // rows j = 16J + 4lq + i, column r = 16I + l16; store P[r][j]
              const int r = 16 * I + l16;
              f32x4 out;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int j = 16 * J + 4 * lq + i;
                out[i] = (I == J && j > r) ? 0.f : acc[i];
              }
              Op::store4(sP + r * LDC + 16 * J + 4 * lq, out);
            }
          }
        }
      }
      __syncthreads();  // B3

      // ================= 4: Kt^T, Kh^T; X = (I + A)^{-1} ======================
      if (scan_on) {
        float wsc[RPW];  // beta_j rk_j folded into Kt's rows
#pragma unroll
        for (int i = 0; i < RPW; ++i) wsc[i] = sbeta[r0 + i] * srk[r0 + i];
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          float ktv[RPW], khv[RPW];
#pragma unroll
          for (int i = 0; i < RPW; ++i) {
            ktv[i] = kt[i][c] * wsc[i];
            khv[i] = kh[i][c];
          }
          store_run<Op, RPW>(sKtT + (c0ch + c) * LDC + r0, ktv);
          store_run<Op, RPW>(sKhT + (c0ch + c) * LDC + r0, khv);
        }
      }
      if (wave < NB && lane < 16) {
        // forward substitution for column j of the diagonal block (I, I):
        // x_i = delta_ij - sum_{m<i} A(i, m) x_m.  Every lane reads the same
        // row of A (a broadcast); X overwrites A only after the last read.
        const int I = wave, j = lane;
        const float* arow = sXf + 16 * I * LDF + 16 * I;  // A(16I + i, 16I + m) at [i * LDF + m]
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
          for (int g = 0; 4 * g < i; ++g) {
            const f32x4 ar = *reinterpret_cast<const f32x4*>(arow + i * LDF + 4 * g);
#pragma unroll
            for (int mm = 0; mm < 4; ++mm)
              if (4 * g + mm < i) acc -= ar[mm] * x[4 * g + mm];
          }
          x[i] = acc;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int i = 0; i < 16; ++i) sXf[(16 * I + i) * LDF + 16 * I + j] = x[i];
      }
      __syncthreads();  // B4
      // off-diagonal blocks: X_IJ = -X_II sum_{J<=M<I} A_IM X_MJ, level d = I - J
      for (int d = 1; d < NB; ++d) {
        for (int J = wave; J + d < NB; J += NW) {
          const int I = J + d;
          f32x4 tacc = {0.f, 0.f, 0.f, 0.f};
          for (int M = J; M < I; ++M) {
            float av[4], xv[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
              const int m = 16 * M + 4 * kk + lq;
              av[kk] = sAT[m * LDF + 16 * I + l16];
              xv[kk] = sXf[m * LDF + 16 * J + l16];
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) tacc = mfma_f32(av[kk], xv[kk], tacc);
          }
          float* ts = sTS + wave * Cfg::TSCR;
#pragma unroll
          for (int i = 0; i < 4; ++i) ts[(4 * lq + i) * 20 + l16] = tacc[i];
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          float xa[4], tb[4];
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const int m = 4 * kk + lq;
            xa[kk] = sXf[(16 * I + l16) * LDF + 16 * I + m];
            tb[kk] = ts[m * 20 + l16];
          }
          f32x4 xacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) xacc = mfma_f32(xa[kk], tb[kk], xacc);
#pragma unroll
          for (int i = 0; i < 4; ++i) sXf[(16 * I + 4 * lq + i) * LDF + 16 * J + l16] = -xacc[i];
        }
        __syncthreads();
      }
      // X (lower blocks; zeros above the diagonal inside the diagonal blocks)
      // as an MFMA operand.  Blocks above the diagonal stay zero from the start.
      {
        constexpr int NQ = NB * (NB + 1) / 2 * 64;  // 4-element groups of the lower blocks
        for (int e = tid; e < NQ; e += NT) {
          int blk = e / 64;
          const int w = e % 64;
          int I = 0;
          while (blk > I) {
            blk -= I + 1;
            ++I;
          }
          const int r = 16 * I + w / 4, j = 16 * blk + 4 * (w % 4);
          Op::store4(sXb + r * LDC + j, *reinterpret_cast<const f32x4*>(sXf + r * LDF + j));
        }
      }
      __syncthreads();

      // ================= 5: W and Ubar ==================================
      {
        // W^T tiles (channel block mc, row block nr): -W stored row-major
        constexpr int NWT = (DK / 16) * (C / 16);
        constexpr int NU = (NWT + NW - 1) / NW;
#pragma unroll 1
        for (int u = 0; u < NU; ++u) {
          const int tt = wave + NW * u;
          if (tt < NWT) {
            const int mc = tt / (C / 16), nr = tt % (C / 16);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            Op::template mmaK<C>(acc, sKtT + 16 * mc * LDC, LDC, sXb + 16 * nr * LDC, LDC, lane);
            // rows c = 16mc + 4lq + i, column r = 16nr + l16
            Op::store4(sWn + (16 * nr + l16) * LDK + 16 * mc + 4 * lq, -acc);
          }
        }
      }
      f32x4 uacc[Cfg::NUW];
#pragma unroll
      for (int u = 0; u < Cfg::NUW; ++u) {
        const int tt = wave + NW * u;
        uacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tt < Cfg::NUT) {
          const int rb = tt / NTN, db = tt % NTN;
          Op::template mmaK<C>(uacc[u], sXb + 16 * rb * LDC, LDC, sVT + 16 * db * LDC, LDC, lane);
        }
      }
      __syncthreads();

      // ================= 6: U = Ubar - W S0; store U' = Diag(rk) U ======
#pragma unroll
      for (int u = 0; u < Cfg::NUW; ++u) {
        const int tt = wave + NW * u;
        if (tt < Cfg::NUT) {
          const int rb = tt / NTN, db = tt % NTN;
          Op::template mmaK<DK>(uacc[u], sWn + 16 * rb * LDK, LDK, sS + 16 * db * LDK, LDK, lane);
          // rows j = 16rb + 4lq + i, column dv = 16db + l16 -> U'^T[dv][j]
          f32x4 un;
#pragma unroll
          for (int i = 0; i < 4; ++i) un[i] = uacc[u][i] * srk[16 * rb + 4 * lq + i];
          Op::store4(sUn + (16 * db + l16) * LDC + 16 * rb + 4 * lq, un);
        }
      }
      __syncthreads();

      // ================= 7: outputs and state update ====================
      {
        constexpr int NOT = NTN * (C / 16);
        constexpr int NU = (NOT + NW - 1) / NW;
#pragma unroll 1
        for (int u = 0; u < NU; ++u) {
          const int tt = wave + NW * u;
          if (tt < NOT) {
            const int db = tt / (C / 16), rb = tt % (C / 16);
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            Op::template mmaK<DK>(acc, sS + 16 * db * LDK, LDK, sLq + 16 * rb * LDK, LDK, lane);
            Op::template mmaK<C>(acc, sUn + 16 * db * LDC, LDC, sP + 16 * rb * LDC, LDC, lane);
            // rows dv = 16db + 4lq + i, column r = 16rb + l16
            const int r = 16 * rb + l16;
            if (r < L) {
              const float sc = a.scale * srq[r];
              const int64_t off =
                  ((t0 + r) * H + h) * static_cast<int64_t>(a.dv) + dv0 + 16 * db + 4 * lq;
              IO::store4(go + off, acc * sc);
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < Cfg::NSW; ++u) {
        const int t = wave + NW * u;
        if (t < Cfg::NST) {
          const int mc = t / NTN, db = t % NTN;
          const f32x4 gv = *reinterpret_cast<const f32x4*>(sg + 16 * mc + 4 * lq);
          sacc[u] *= gv;
          Op::template mmaK<C>(sacc[u], sKhT + 16 * mc * LDC, LDC, sUn + 16 * db * LDC, LDC, lane);
        }
      }
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < Cfg::NSW; ++u) {
      const int t = wave + NW * u;
      if (t < Cfg::NST) {
        const int c = 16 * (t / NTN) + 4 * lq, dv = 16 * (t % NTN) + l16;
        Op::store4(sS + dv * LDK + c, sacc[u]);
      }
    }
    // the next chunk's first shared-memory writes that readers of sS could
    // race with come after its barrier B1
  }

  if (a.ht) {
#pragma unroll
    for (int u = 0; u < Cfg::NSW; ++u) {
      const int t = wave + NW * u;
      if (t < Cfg::NST) {
        const int c = 16 * (t / NTN) + 4 * lq, dv = 16 * (t % NTN) + l16;
#pragma unroll
        for (int i = 0; i < 4; ++i) a.ht[st_base + static_cast<int64_t>(c + i) * a.dv + dv] = sacc[u][i];
      }
    }
  }
}

template <class Cfg>
launch_result launch_cfg(const FwdArgs& a, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&fwd_kernel<Cfg>), hipFuncAttributeMaxDynamicSharedMemorySize,
      Cfg::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  const int64_t blocks = static_cast<int64_t>(a.num_seqs) * a.H * Cfg::NSPLIT;
  hipLaunchKernelGGL(fwd_kernel<Cfg>, dim3(static_cast<unsigned>(blocks)), dim3(Cfg::NT),
                     Cfg::LDS_BYTES, stream, a);
  return hipGetLastError();
}

// The instantiated shapes.  Each entry: chunk, dk, dv, dtype -> launcher.
struct Entry {
  int chunk, dk, dv, dtype;
  launch_result (*fn)(const FwdArgs&, hipStream_t);
};

template <class Op, class IO, int C, int D, int DVT>
constexpr Entry entry(int dtype) {
  return Entry{C, D, D, dtype, &launch_cfg<Cfg<Op, IO, C, D, D, DVT>>};
}

const Entry kEntries[] = {
    entry<OpBF16, io_bf16, 64, 128, 64>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 32, 128, 64>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 16, 128, 64>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 64, 64, 32>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 32, 64, 32>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 16, 64, 32>(CKDA_DTYPE_BF16),
    entry<OpF32, io_f32, 16, 16, 16>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 32, 16, 16>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 64, 16, 16>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 16, 32, 32>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 32, 32, 32>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 64, 32, 32>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 16, 64, 32>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 32, 64, 32>(CKDA_DTYPE_F32),
};

const Entry* find(int32_t chunk, int32_t dk, int32_t dv, int32_t dtype) {
  for (const Entry& e : kEntries)
    if (e.chunk == chunk && e.dk == dk && e.dv == dv && e.dtype == dtype) return &e;
  return nullptr;
}

}  // namespace

bool fwd_supported(int32_t chunk, int32_t dk, int32_t dv, int32_t io_dtype) {
  return find(chunk, dk, dv, io_dtype) != nullptr;
}

launch_result launch_fwd(const FwdArgs& a, int32_t io_dtype, hipStream_t stream) {
  const Entry* e = find(a.chunk, a.dk, a.dv, io_dtype);
  if (!e) return hipErrorInvalidValue;
  if (static_cast<int64_t>(a.num_seqs) * a.H == 0) return hipSuccess;
  return e->fn(a, stream);
}

}  // namespace ckda
