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
// and g = D(end<-start).  q and k enter raw; the in-op L2 normalisation
// (dormouse review "RoPE into the KDA q/k path", section 2) is applied as row
// scales rq, rk: A gets beta_r rk_r rk_j, U's rows get rk (U' = Diag(rk) U is
// what P and Kh^T multiply), W = X Diag(beta rk) Kt, and O's rows get rq.
//
// Gate prefix: per 16-token sub-block I and channel, running products of
// alpha give F_r (block start .. r), B_r (after r .. block end) and the block
// total G_I.  Signs and exact zeros propagate through the products, so
// signed and zero gates are exact (the CKDA range of the summary's section
// "CKDA Definition"; the sign-magnitude split of its Proposition 2 is carried
// by the fp32 sign bit and exponent of each product).  For r in block I and j
// in an earlier block J, D(r<-j) = F_r (prod_{J<M<I} G_M) B_j: every factor has
// modulus <= 1, so the off-diagonal blocks of A and P are MFMA products of
// bounded operands.  Inside a block, D(r<-j) = F_r / F_j when no |F| of the
// block is below 2^-100 (then 1/F_j cannot overflow); channels that fail this
// test are left out of the MFMA and added back by a direct product of alpha.
//
// Per chunk, all on one workgroup of four waves:
//   1  load q, k, alpha (16-row block per wave, two channels per lane) and the
//      v tile; running products; operands Lk = k.F, Lq = q.F, Rdiag = k/F
//   2  block totals -> R panels k.B.G, Qt, Kt, Kh; row norms
//   3  A and P^T panels on MFMA (bf16 -> fp32; fp32 MFMA for fp32 inputs)
//   4  rare direct-product fix-ups for small-gate channels
//   5  X = (I + A)^{-1}: 16x16 diagonal blocks by forward substitution, then
//      the off-diagonal blocks level by level on fp32 MFMA
//   6  W^T = (Diag(beta rk) Kt)^T X^T,  Ubar = X (Diag(beta) V)    (MFMA)
//   7  U = Ubar - W S0                                             (MFMA)
//   8  O^T = S0^T Qt^T + U'^T P^T,  S' = Diag(g) S0 + Kh^T U'       (MFMA)
#include "ckda_internal.h"

namespace ckda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;  // threads per workgroup
constexpr int NW = 4;    // waves per workgroup
constexpr float kSafeMin = 0x1p-100f;

constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int align16(int x) { return (x + 15) & ~15; }

// ---- MFMA operand types ----------------------------------------------------
// Both operands of every product are stored in LDS as [rows][K] with K (the
// contraction index) contiguous: A as [M][K], B as B^T = [N][K].  Lane l of a
// 16x16 tile reads row l%16 and a K-slice selected by l/16; the fp32 result
// holds rows 4*(l/16)+i, column l%16 (i = 0..3).
struct OpBF16 {
  using T = __bf16;
  static __device__ __forceinline__ T cvt(float x) { return static_cast<__bf16>(x); }
  // acc += A[16 x K] * B[16 x K]^T for K a multiple of 16.
  static __device__ __forceinline__ void mma(f32x4& acc, const T* a, int lda, const T* b,
                                             int ldb, int K, int lane) {
    const int r = lane & 15, kq = lane >> 4;
    const T* pa = a + r * lda;
    const T* pb = b + r * ldb;
    int k0 = 0;
    for (; k0 + 32 <= K; k0 += 32) {
      const bf16x8 fa = *reinterpret_cast<const bf16x8*>(pa + k0 + 8 * kq);
      const bf16x8 fb = *reinterpret_cast<const bf16x8*>(pb + k0 + 8 * kq);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc, 0, 0, 0);
    }
    if (k0 < K) {
      const bf16x4 fa = *reinterpret_cast<const bf16x4*>(pa + k0 + 4 * kq);
      const bf16x4 fb = *reinterpret_cast<const bf16x4*>(pb + k0 + 4 * kq);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(fa, fb, acc, 0, 0, 0);
    }
  }
  // Store 4 consecutive values (one accumulator) at p.
  static __device__ __forceinline__ void store4(T* p, f32x4 x) {
    bf16x4 y;
    y[0] = cvt(x[0]); y[1] = cvt(x[1]); y[2] = cvt(x[2]); y[3] = cvt(x[3]);
    *reinterpret_cast<bf16x4*>(p) = y;
  }
};

struct OpF32 {
  using T = float;
  static __device__ __forceinline__ T cvt(float x) { return x; }
  static __device__ __forceinline__ void mma(f32x4& acc, const T* a, int lda, const T* b,
                                             int ldb, int K, int lane) {
    const int r = lane & 15, kq = lane >> 4;
    const T* pa = a + r * lda + kq;
    const T* pb = b + r * ldb + kq;
    for (int k0 = 0; k0 < K; k0 += 4)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k0], pb[k0], acc, 0, 0, 0);
  }
  static __device__ __forceinline__ void store4(T* p, f32x4 x) {
    *reinterpret_cast<f32x4*>(p) = x;
  }
};

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---- buffer loads ----------------------------------------------------------
// A raw buffer resource covers one chunk's rows of one head; rows are reached
// through the scalar offset, lanes through a 32-bit vector offset, and the
// hardware range check returns zero past num_bytes.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(num_bytes), kRsrcWord3);
}

// N consecutive io elements at (voff + soff) bytes, widened to fp32.
template <class IO, int N>
__device__ __forceinline__ void buf_load(rsrc_t r, int voff, int soff, float (&out)[N]);

template <>
__device__ __forceinline__ void buf_load<io_bf16, 1>(rsrc_t r, int voff, int soff, float (&out)[1]) {
  const uint32_t u = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
  out[0] = __uint_as_float(u << 16);
}
template <>
__device__ __forceinline__ void buf_load<io_bf16, 2>(rsrc_t r, int voff, int soff, float (&out)[2]) {
  const uint32_t u = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
  out[0] = __uint_as_float(u << 16);
  out[1] = __uint_as_float(u & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ void buf_load<io_f32, 1>(rsrc_t r, int voff, int soff, float (&out)[1]) {
  out[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
template <>
__device__ __forceinline__ void buf_load<io_f32, 2>(rsrc_t r, int voff, int soff, float (&out)[2]) {
  const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  out[0] = __uint_as_float(u[0]);
  out[1] = __uint_as_float(u[1]);
}
// 16 bytes: 8 bf16 or 4 fp32
template <class IO>
__device__ __forceinline__ void buf_load16(rsrc_t r, int voff, int soff, float* out);
template <>
__device__ __forceinline__ void buf_load16<io_bf16>(rsrc_t r, int voff, int soff, float* out) {
  const auto u = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(u[i] << 16);
    out[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
  }
}
template <>
__device__ __forceinline__ void buf_load16<io_f32>(rsrc_t r, int voff, int soff, float* out) {
  const auto u = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(u[i]);
}

// ---- compile-time configuration and LDS map ---------------------------------
template <class OpT, class IOT, int C_, int DK_, int DV_, int DVT_>
struct Cfg {
  using Op = OpT;
  using IO = IOT;
  using T = typename Op::T;
  static constexpr int C = C_, DK = DK_, DV = DV_, DVT = DVT_;
  static constexpr int NSPLIT = DV / DVT;
  static constexpr int NB = C / 16;                  // 16-token sub-blocks per chunk
  static constexpr int CPT = DK >= 64 ? DK / 64 : 1; // channels per lane in the scan
  static constexpr int NCG = DK / CPT;               // active lanes per scan wave
  static constexpr int PAD = 16 / static_cast<int>(sizeof(T));
  static constexpr int LDK = DK + PAD;               // stride of [*][DK] operands
  static constexpr int LDC = C + PAD;                // stride of [*][C] operands
  static constexpr int LDF = C + 4;                  // stride of fp32 [C][C] buffers
  static constexpr int RROWS = 16 * NB * (NB + 1) / 2;
  static constexpr int ES = static_cast<int>(sizeof(T));
  static constexpr int TSCR = 16 * 20;               // per-wave fp32 scratch (16x16 + pad)
  static constexpr int PART = 64 * 17;               // per-wave fp32 norm partials

  static constexpr int NST = (DK / 16) * (DVT / 16); // state tiles
  static constexpr int NSW = (NST + NW - 1) / NW;
  static constexpr int NUT = (C / 16) * (DVT / 16);  // U tiles
  static constexpr int NUW = (NUT + NW - 1) / NW;
  static constexpr int IOES = static_cast<int>(sizeof(typename IO::storage));
  static constexpr int VEC = 16 / IOES;              // v elements per 16-byte load
  static constexpr int TPR = DVT / VEC;              // threads per v row
  static constexpr int RPP = NT / TPR;               // v rows per pass

  // byte offsets
  static constexpr int O_S = 0;                                   // S^T   [DVT][LDK] T
  static constexpr int O_X = align16(O_S + DVT * LDK * ES);       // region X
  // phase a (inside X)
  static constexpr int O_LK = O_X;                                // Lk    [C][LDK]
  static constexpr int O_LQ = O_LK + C * LDK * ES;                // Lq    [C][LDK]
  static constexpr int O_R = O_LQ + C * LDK * ES;                 // R     [RROWS][LDK]
  static constexpr int END_XA = O_R + RROWS * LDK * ES;
  // phase b (inside X)
  static constexpr int O_QT = O_X;                                // Qt    [C][LDK]
  static constexpr int O_KTT = O_QT + C * LDK * ES;               // Kt^T  [DK][LDC] (rows scaled by beta rk)
  static constexpr int O_KHT = O_KTT + DK * LDC * ES;             // Kh^T  [DK][LDC]
  static constexpr int O_TS = align16(O_KHT + DK * LDC * ES);     // T scratch fp32 [NW][TSCR]
  static constexpr int END_XB = O_TS + NW * TSCR * 4;
  static constexpr int O_VT = align16(cmax(END_XA, END_XB));      // (beta V)^T [DVT][LDC]
  static constexpr int O_AT = align16(O_VT + DVT * LDC * ES);     // A^T fp32 [C][LDF] | -W [C][LDK] | k partials
  static constexpr int SZ_AT = align16(cmax(cmax(C * LDF * 4, C * LDK * ES), NB * PART * 4));
  static constexpr int O_XF = O_AT + SZ_AT;                       // X fp32 [C][LDF] | U'^T [DVT][LDC] | q partials
  static constexpr int SZ_XF = align16(cmax(cmax(C * LDF * 4, DVT * LDC * ES), NB * PART * 4));
  static constexpr int O_XB = O_XF + SZ_XF;                       // X (operand copy) [C][LDC]
  static constexpr int O_P = align16(O_XB + C * LDC * ES);        // P     [C][LDC]
  static constexpr int O_G = align16(O_P + C * LDC * ES);         // G     [NB][DK] fp32
  static constexpr int O_GC = O_G + NB * DK * 4;                  // g     [DK] fp32
  static constexpr int O_RQ = O_GC + DK * 4;                      // rq    [C]
  static constexpr int O_RK = O_RQ + C * 4;                       // rk    [C]
  static constexpr int O_BETA = O_RK + C * 4;                     // beta  [C]
  static constexpr int O_SAFE = O_BETA + C * 4;                   // safe  [NB][DK] bytes
  static constexpr int LDS_BYTES = align16(O_SAFE + NB * DK);

  static_assert(C % 16 == 0 && DK % 16 == 0 && DVT % 16 == 0 && DV % DVT == 0, "tile sizes");
  static_assert(NB <= NW, "one wave per sub-block");
  static_assert(DK <= 128 && NCG <= 64, "two channels per lane at most");
  static_assert(DVT % VEC == 0 && NT % TPR == 0, "v tile mapping");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <class Cfg>
__global__ __launch_bounds__(NT, 1) void fwd_kernel(FwdArgs a) {
  using Op = typename Cfg::Op;
  using IO = typename Cfg::IO;
  using T = typename Cfg::T;
  using ST = typename IO::storage;
  constexpr int C = Cfg::C, DK = Cfg::DK, DVT = Cfg::DVT, NB = Cfg::NB;
  constexpr int CPT = Cfg::CPT, NCG = Cfg::NCG;
  constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC, LDF = Cfg::LDF;

  extern __shared__ __align__(16) unsigned char smem[];
  T* sS = reinterpret_cast<T*>(smem + Cfg::O_S);
  T* sLk = reinterpret_cast<T*>(smem + Cfg::O_LK);
  T* sLq = reinterpret_cast<T*>(smem + Cfg::O_LQ);
  T* sR = reinterpret_cast<T*>(smem + Cfg::O_R);
  T* sQt = reinterpret_cast<T*>(smem + Cfg::O_QT);
  T* sKtT = reinterpret_cast<T*>(smem + Cfg::O_KTT);
  T* sKhT = reinterpret_cast<T*>(smem + Cfg::O_KHT);
  T* sVT = reinterpret_cast<T*>(smem + Cfg::O_VT);
  float* sTS = reinterpret_cast<float*>(smem + Cfg::O_TS);
  float* sAT = reinterpret_cast<float*>(smem + Cfg::O_AT);
  T* sWn = reinterpret_cast<T*>(smem + Cfg::O_AT);
  float* sKpart = reinterpret_cast<float*>(smem + Cfg::O_AT);
  float* sXf = reinterpret_cast<float*>(smem + Cfg::O_XF);
  T* sUn = reinterpret_cast<T*>(smem + Cfg::O_XF);
  float* sQpart = reinterpret_cast<float*>(smem + Cfg::O_XF);
  T* sXb = reinterpret_cast<T*>(smem + Cfg::O_XB);
  T* sP = reinterpret_cast<T*>(smem + Cfg::O_P);
  float* sG = reinterpret_cast<float*>(smem + Cfg::O_G);
  float* sg = reinterpret_cast<float*>(smem + Cfg::O_GC);
  float* srq = reinterpret_cast<float*>(smem + Cfg::O_RQ);
  float* srk = reinterpret_cast<float*>(smem + Cfg::O_RK);
  float* sbeta = reinterpret_cast<float*>(smem + Cfg::O_BETA);
  unsigned char* sSafe = smem + Cfg::O_SAFE;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l16 = lane & 15, lq = lane >> 4;

  // ---- which chain: (sequence, head) pairs of one dv-split sit 8 workgroups
  // apart so that both tiles of a pair land on the same XCD (shared q/k/alpha
  // reads hit one L2).
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
    bos = a.cu_seqlens[n];
    eos = a.cu_seqlens[n + 1];
  } else {
    bos = n * a.T;
    eos = bos + a.T;
  }
  const int dv0 = split * DVT;

  const ST* gq = static_cast<const ST*>(a.q);
  const ST* gk = static_cast<const ST*>(a.k);
  const ST* gv = static_cast<const ST*>(a.v);
  ST* go = static_cast<ST*>(a.o);

  // ---- state tile in accumulator layout: tile t = wave + NW*u covers rows
  // c = 16*(t / (DVT/16)) + 4*lq + i, columns dv = 16*(t % (DVT/16)) + l16.
  constexpr int NTN = DVT / 16;
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
  // bf16 (or fp32) operand copy S^T[dv][c]
#pragma unroll
  for (int u = 0; u < Cfg::NSW; ++u) {
    const int t = wave + NW * u;
    if (t < Cfg::NST) {
      const int c = 16 * (t / NTN) + 4 * lq, dv = 16 * (t % NTN) + l16;
      Op::store4(sS + dv * LDK + c, sacc[u]);
    }
  }

  const float use_l2 = static_cast<float>(a.use_l2norm);
  const int scan_I = wave;                 // sub-block handled by this wave in the scan
  const bool scan_on = (scan_I < NB) && (lane < NCG);
  const int c0ch = lane * CPT;             // first channel of this lane

  for (int64_t t0 = bos; t0 < eos; t0 += C) {
    const int L = static_cast<int>((eos - t0) < C ? (eos - t0) : C);

    // ================= phase 1: loads, running products, operands ==========
    // q/k/alpha of this lane's channels over the 16 rows of its sub-block.
    // Registers are reused in place as the phases go: alpha -> F -> Kt,
    // B -> Kh, q -> Qt.
    float xq[16][CPT], xk[16][CPT], F[16][CPT], Bk[16][CPT];
    {
      // (beta V)^T tile: thread loads 16 bytes (VEC columns) of one row per pass
      const int64_t vrow = static_cast<int64_t>(H) * a.dv * Cfg::IOES;  // bytes per token
      const rsrc_t rv = make_rsrc(reinterpret_cast<const char*>(gv) +
                                      ((t0 * H + h) * static_cast<int64_t>(a.dv) + dv0) * Cfg::IOES,
                                  static_cast<uint32_t>((L - 1) * vrow + DVT * Cfg::IOES));
      const int vc = (tid % Cfg::TPR) * Cfg::VEC, vr0 = tid / Cfg::TPR;
#pragma unroll
      for (int p = 0; p < (C + Cfg::RPP - 1) / Cfg::RPP; ++p) {
        const int j = vr0 + p * Cfg::RPP;
        if (j < C) {
          float x[Cfg::VEC];
          buf_load16<IO>(rv, vc * Cfg::IOES, static_cast<int>(j * vrow), x);
          const float bj = (j < L) ? a.beta[(t0 + j) * H + h] : 0.f;
#pragma unroll
          for (int e = 0; e < Cfg::VEC; ++e) sVT[(vc + e) * LDC + j] = Op::cvt(x[e] * bj);
        }
      }
    }
    if (scan_on) {
      const int64_t krow = static_cast<int64_t>(H) * DK * Cfg::IOES;  // bytes per token
      const int64_t base = (t0 * H + h) * static_cast<int64_t>(DK);
      const uint32_t nb = static_cast<uint32_t>((L - 1) * krow + DK * Cfg::IOES);
      const rsrc_t rq = make_rsrc(reinterpret_cast<const char*>(gq) + base * Cfg::IOES, nb);
      const rsrc_t rk = make_rsrc(reinterpret_cast<const char*>(gk) + base * Cfg::IOES, nb);
      const rsrc_t ra = make_rsrc(a.alpha + base,
                                  static_cast<uint32_t>((L - 1) * H * DK * 4 + DK * 4));
      const int sI = __builtin_amdgcn_readfirstlane(scan_I);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * sI + i;
        float tq[CPT], tk[CPT], ta[CPT];
        buf_load<IO, CPT>(rq, c0ch * Cfg::IOES, static_cast<int>(r * krow), tq);
        buf_load<IO, CPT>(rk, c0ch * Cfg::IOES, static_cast<int>(r * krow), tk);
        buf_load<io_f32, CPT>(ra, c0ch * 4, r * H * DK * 4, ta);
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          xq[i][c] = tq[c];
          xk[i][c] = tk[c];
          F[i][c] = (r < L) ? ta[c] : 1.f;
        }
      }
      float mn[CPT];
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        float bb = 1.f;
#pragma unroll
        for (int i = 15; i >= 0; --i) {
          Bk[i][c] = bb;
          bb *= F[i][c];
        }
        float f = 1.f;
        mn[c] = 1.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          f *= F[i][c];
          F[i][c] = f;
          mn[c] = fminf(mn[c], fabsf(f));
        }
        sG[scan_I * DK + c0ch + c] = F[15][c];
        sSafe[scan_I * DK + c0ch + c] = mn[c] >= kSafeMin ? 1 : 0;
      }
      // Lk, Lq and the diagonal panel slot of R
      T* rdiag = sR + (8 * scan_I * (scan_I + 1) + 16 * scan_I) * LDK;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * scan_I + i;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          sLk[r * LDK + c0ch + c] = Op::cvt(xk[i][c] * F[i][c]);
          sLq[r * LDK + c0ch + c] = Op::cvt(xq[i][c] * F[i][c]);
          rdiag[i * LDK + c0ch + c] = Op::cvt(mn[c] >= kSafeMin ? xk[i][c] / F[i][c] : 0.f);
        }
      }
      // per-row partial sums of squares (this lane's channels)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pq = 0.f, pk = 0.f;
#pragma unroll
        for (int c = 0; c < CPT; ++c) {
          pq += xq[i][c] * xq[i][c];
          pk += xk[i][c] * xk[i][c];
        }
        sQpart[scan_I * Cfg::PART + lane * 17 + i] = pq;
        sKpart[scan_I * Cfg::PART + lane * 17 + i] = pk;
      }
    } else if (scan_I < NB) {
      // idle lanes of an active scan wave contribute zero partials
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sQpart[scan_I * Cfg::PART + lane * 17 + i] = 0.f;
        sKpart[scan_I * Cfg::PART + lane * 17 + i] = 0.f;
      }
    }
    if (tid < C) sbeta[tid] = (tid < L) ? a.beta[(t0 + tid) * H + h] : 0.f;
    __syncthreads();  // B1

    // ================= phase 2: block products, panels, norms ==============
    if (scan_on) {
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        float gm[NW];
#pragma unroll
        for (int M = 0; M < NB; ++M) gm[M] = sG[M * DK + c0ch + c];
        float gpre = 1.f, gpost = 1.f;
#pragma unroll
        for (int M = 0; M < NB; ++M) {
          if (M < scan_I) gpre *= gm[M];
          if (M > scan_I) gpost *= gm[M];
        }
        if (scan_I == 0) {
          float g = 1.f;
#pragma unroll
          for (int M = 0; M < NB; ++M) g *= gm[M];
          sg[c0ch + c] = g;
        }
        // R panels of the later blocks: rows of this block, anchor at I2's start
        float mid = 1.f;
#pragma unroll
        for (int I2 = 1; I2 < NB; ++I2) {
          if (I2 > scan_I) {
            if (I2 > scan_I + 1) mid *= gm[I2 - 1];
            T* pan = sR + (8 * I2 * (I2 + 1) + 16 * scan_I) * LDK;
#pragma unroll
            for (int i = 0; i < 16; ++i) pan[i * LDK + c0ch + c] = Op::cvt(xk[i][c] * Bk[i][c] * mid);
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          xq[i][c] = xq[i][c] * F[i][c] * gpre;   // Qt
          F[i][c] = xk[i][c] * F[i][c] * gpre;    // Kt (unscaled)
          Bk[i][c] = xk[i][c] * Bk[i][c] * gpost; // Kh
        }
      }
    }
    if (scan_I < NB) {
      // row norms: lane (row r = lane/4, quarter g = lane%4) sums 16 lanes' partials
      const int r = lane >> 2, g = lane & 3;
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        sq += sQpart[scan_I * Cfg::PART + (16 * g + m) * 17 + r];
        sk += sKpart[scan_I * Cfg::PART + (16 * g + m) * 17 + r];
      }
      sq += __shfl_xor(sq, 1, 64);
      sk += __shfl_xor(sk, 1, 64);
      sq += __shfl_xor(sq, 2, 64);
      sk += __shfl_xor(sk, 2, 64);
      if (g == 0) {
        const int row = 16 * scan_I + r;
        srq[row] = use_l2 != 0.f ? __fdiv_rn(1.f, __fsqrt_rn(sq + kL2Eps)) : 1.f;
        srk[row] = use_l2 != 0.f ? __fdiv_rn(1.f, __fsqrt_rn(sk + kL2Eps)) : 1.f;
      }
    }
    __syncthreads();  // B2

    // ================= phase 3: A and P^T panels on MFMA ====================
    {
      constexpr int NPT = NB * (NB + 1) / 2;  // tiles per matrix
      for (int tt = wave; tt < 2 * NPT; tt += NW) {
        const bool isA = tt < NPT;
        int idx = isA ? tt : tt - NPT;
        int I = 0;
        while (idx > I) {
          idx -= I + 1;
          ++I;
        }
        const int J = idx;  // 0..I
        const T* pan = sR + (8 * I * (I + 1) + 16 * J) * LDK;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (isA) {
          Op::mma(acc, sLk + 16 * I * LDK, LDK, pan, LDK, DK, lane);
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
        } else {
          Op::mma(acc, pan, LDK, sLq + 16 * I * LDK, LDK, DK, lane);
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
    __syncthreads();  // B3

    // ================= phase 4: operands for later phases; fix-ups ==========
    if (scan_on) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * scan_I + i;
#pragma unroll
        for (int c = 0; c < CPT; ++c) sQt[r * LDK + c0ch + c] = Op::cvt(xq[i][c]);
      }
      float wsc[16];  // beta_j rk_j folded into Kt's rows
#pragma unroll
      for (int i = 0; i < 16; ++i) wsc[i] = sbeta[16 * scan_I + i] * srk[16 * scan_I + i];
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        T* ktrow = sKtT + (c0ch + c) * LDC + 16 * scan_I;
        T* khrow = sKhT + (c0ch + c) * LDC + 16 * scan_I;
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          Op::store4(ktrow + i, f32x4{F[i][c] * wsc[i], F[i + 1][c] * wsc[i + 1],
                                      F[i + 2][c] * wsc[i + 2], F[i + 3][c] * wsc[i + 3]});
          Op::store4(khrow + i, f32x4{Bk[i][c], Bk[i + 1][c], Bk[i + 2][c], Bk[i + 3][c]});
        }
      }
    }
    if (scan_I < NB) {
      // Direct products for channels whose block prefix got too small to
      // invert (exact zeros, or |F| < 2^-100).  Lane (j = l16, part = lq)
      // accumulates column j of the diagonal blocks of A and P over the
      // unsafe channels c with c % 4 == part, in increasing c; the four parts
      // are then summed in a fixed order, so the result is deterministic.
      const int I = scan_I;
      bool any = false;
      for (int c = lane; c < DK; c += 64) any |= sSafe[I * DK + c] == 0;
      if (__any(any)) {
        const int j = l16;
        float accA[16], accP[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) accA[r] = accP[r] = 0.f;
        const int64_t krow = static_cast<int64_t>(H) * DK;  // elements per token
        const int64_t base = (t0 * H + h) * static_cast<int64_t>(DK);
        const uint32_t nb = static_cast<uint32_t>(((L - 1) * krow + DK) * Cfg::IOES);
        const rsrc_t rq = make_rsrc(reinterpret_cast<const char*>(gq) + base * Cfg::IOES, nb);
        const rsrc_t rk = make_rsrc(reinterpret_cast<const char*>(gk) + base * Cfg::IOES, nb);
        const rsrc_t ra = make_rsrc(a.alpha + base, static_cast<uint32_t>(((L - 1) * krow + DK) * 4));
        const int sI = __builtin_amdgcn_readfirstlane(I);
        for (int c = lq; c < DK; c += 4) {
          if (sSafe[I * DK + c]) continue;
          float kj = 0.f, qr[16], kr[16], ar[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 16 * sI + r;
            float t1[1], t2[1], t3[1];
            buf_load<IO, 1>(rq, c * Cfg::IOES, static_cast<int>(row * krow * Cfg::IOES), t1);
            buf_load<IO, 1>(rk, c * Cfg::IOES, static_cast<int>(row * krow * Cfg::IOES), t2);
            buf_load<io_f32, 1>(ra, c * 4, static_cast<int>(row * krow * 4), t3);
            qr[r] = t1[0];
            kr[r] = t2[0];
            ar[r] = (row < L) ? t3[0] : 1.f;
            if (r == j) kj = kr[r];
          }
          float d = 1.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            if (r > j) {
              d *= ar[r];
              accA[r] += kr[r] * kj * d;
            }
            if (r >= j) accP[r] += qr[r] * kj * d;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          accA[r] += __shfl_xor(accA[r], 16, 64);
          accP[r] += __shfl_xor(accP[r], 16, 64);
          accA[r] += __shfl_xor(accA[r], 32, 64);
          accP[r] += __shfl_xor(accP[r], 32, 64);
        }
        if (lq == 0) {
          const int jj = 16 * I + j;
          const float sj = srk[jj];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rr = 16 * I + r;
            if (r > j) sAT[jj * LDF + rr] += accA[r] * sbeta[rr] * srk[rr] * sj;
            if (r >= j) {
              const float p = static_cast<float>(sP[rr * LDC + jj]) + accP[r];
              sP[rr * LDC + jj] = Op::cvt(p);
            }
          }
        }
      }
    }
    __syncthreads();  // B4

    // ================= phase 5: X = (I + A)^{-1} ============================
    if (wave < NB && lane < 16) {
      // forward substitution for column j of the diagonal block (I, I)
      const int I = wave, j = lane;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = (i == j) ? 1.f : 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const float* acol = sAT + (16 * I + m) * LDF + 16 * I;  // A(16I + i, 16I + m)
#pragma unroll
        for (int i = m + 1; i < 16; ++i) x[i] -= acol[i] * x[m];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sXf[(16 * I + i) * LDF + 16 * I + j] = x[i];
    }
    __syncthreads();
    // off-diagonal blocks: X_IJ = -X_II sum_{J<=M<I} A_IM X_MJ, level d = I - J
    for (int d = 1; d < NB; ++d) {
      for (int J = wave; J + d < NB; J += NW) {
        const int I = J + d;
        f32x4 tacc = {0.f, 0.f, 0.f, 0.f};
        for (int M = J; M < I; ++M) {
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const int m = 16 * M + 4 * kk + lq;
            tacc = mfma_f32(sAT[m * LDF + 16 * I + l16], sXf[m * LDF + 16 * J + l16], tacc);
          }
        }
        float* ts = sTS + wave * Cfg::TSCR;
#pragma unroll
        for (int i = 0; i < 4; ++i) ts[(4 * lq + i) * 20 + l16] = tacc[i];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        f32x4 xacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int m = 4 * kk + lq;
          xacc = mfma_f32(sXf[(16 * I + l16) * LDF + 16 * I + m], ts[m * 20 + l16], xacc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sXf[(16 * I + 4 * lq + i) * LDF + 16 * J + l16] = -xacc[i];
      }
      __syncthreads();
    }
    // X (lower triangle) as an MFMA operand
    for (int e = tid; e < C * C; e += NT) {
      const int r = e / C, j = e % C;
      sXb[r * LDC + j] = Op::cvt((j <= r) ? sXf[r * LDF + j] : 0.f);
    }
    __syncthreads();

    // ================= phase 6: W and Ubar ==================================
    {
      // W^T tiles (channel block mc, row block nr): -W stored row-major
      constexpr int NWT = (DK / 16) * (C / 16);
      for (int tt = wave; tt < NWT; tt += NW) {
        const int mc = tt / (C / 16), nr = tt % (C / 16);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        Op::mma(acc, sKtT + 16 * mc * LDC, LDC, sXb + 16 * nr * LDC, LDC, 16 * (nr + 1), lane);
        // rows c = 16mc + 4lq + i, column r = 16nr + l16
        Op::store4(sWn + (16 * nr + l16) * LDK + 16 * mc + 4 * lq, -acc);
      }
    }
    f32x4 uacc[Cfg::NUW];
#pragma unroll
    for (int u = 0; u < Cfg::NUW; ++u) {
      const int tt = wave + NW * u;
      uacc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (tt < Cfg::NUT) {
        const int rb = tt / NTN, db = tt % NTN;
        Op::mma(uacc[u], sXb + 16 * rb * LDC, LDC, sVT + 16 * db * LDC, LDC, 16 * (rb + 1), lane);
      }
    }
    __syncthreads();

    // ================= phase 7: U = Ubar - W S0; store U' = Diag(rk) U ======
#pragma unroll
    for (int u = 0; u < Cfg::NUW; ++u) {
      const int tt = wave + NW * u;
      if (tt < Cfg::NUT) {
        const int rb = tt / NTN, db = tt % NTN;
        Op::mma(uacc[u], sWn + 16 * rb * LDK, LDK, sS + 16 * db * LDK, LDK, DK, lane);
        // rows j = 16rb + 4lq + i, column dv = 16db + l16 -> U'^T[dv][j]
        f32x4 un;
#pragma unroll
        for (int i = 0; i < 4; ++i) un[i] = uacc[u][i] * srk[16 * rb + 4 * lq + i];
        Op::store4(sUn + (16 * db + l16) * LDC + 16 * rb + 4 * lq, un);
      }
    }
    __syncthreads();

    // ================= phase 8: outputs and state update ====================
    {
      constexpr int NOT = NTN * (C / 16);
      for (int tt = wave; tt < NOT; tt += NW) {
        const int db = tt / (C / 16), rb = tt % (C / 16);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        Op::mma(acc, sS + 16 * db * LDK, LDK, sQt + 16 * rb * LDK, LDK, DK, lane);
        Op::mma(acc, sUn + 16 * db * LDC, LDC, sP + 16 * rb * LDC, LDC, 16 * (rb + 1), lane);
        // rows dv = 16db + 4lq + i, column r = 16rb + l16
        const int r = 16 * rb + l16;
        if (r < L) {
          const float sc = a.scale * srq[r];
          const int64_t off = ((t0 + r) * H + h) * static_cast<int64_t>(a.dv) + dv0 + 16 * db + 4 * lq;
#pragma unroll
          for (int i = 0; i < 4; ++i) IO::store(go, off + i, acc[i] * sc);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < Cfg::NSW; ++u) {
      const int t = wave + NW * u;
      if (t < Cfg::NST) {
        const int mc = t / NTN, db = t % NTN;
#pragma unroll
        for (int i = 0; i < 4; ++i) sacc[u][i] *= sg[16 * mc + 4 * lq + i];
        Op::mma(sacc[u], sKhT + 16 * mc * LDC, LDC, sUn + 16 * db * LDC, LDC, C, lane);
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
    // the next chunk's first write to shared memory that sS readers could see
    // comes after its barrier B1
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
  hipLaunchKernelGGL(fwd_kernel<Cfg>, dim3(static_cast<unsigned>(blocks)), dim3(NT),
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
