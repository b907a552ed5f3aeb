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
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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
  // acc += A[16 x K] * B[16 x K]^T, K a compile-time multiple of 16: all
  // fragments are read before the MFMAs issue.
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
    // A K remainder of 16 runs as one more 16x16x32 MFMA whose upper half of
    // K is zero (lanes 32..63 supply zeros): every MFMA accumulating into one
    // tile then has the same shape, so dependent MFMAs never mix pass counts.
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
  // Store 4 consecutive values (one accumulator) at p.
  static __device__ __forceinline__ void store4(T* p, f32x4 x) {
    bf16x4 y;
    y[0] = cvt(x[0]); y[1] = cvt(x[1]); y[2] = cvt(x[2]); y[3] = cvt(x[3]);
    *reinterpret_cast<bf16x4*>(p) = y;
  }
  // Store N (1 or 2) consecutive values x[i] (times f[i]) at p.
  template <int N>
  static __device__ __forceinline__ void storeN(T* p, const float (&x)[N]) {
    if constexpr (N == 2) {
      bf16x2 y;
      y[0] = cvt(x[0]); y[1] = cvt(x[1]);
      *reinterpret_cast<bf16x2*>(p) = y;
    } else {
      p[0] = cvt(x[0]);
    }
  }
  template <int N>
  static __device__ __forceinline__ void storeN(T* p, const float (&x)[N], const float (&f)[N]) {
    float y[N];
#pragma unroll
    for (int i = 0; i < N; ++i) y[i] = x[i] * f[i];
    storeN<N>(p, y);
  }
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
  static __device__ __forceinline__ void store4(T* p, f32x4 x) {
    *reinterpret_cast<f32x4*>(p) = x;
  }
  template <int N>
  static __device__ __forceinline__ void storeN(T* p, const float (&x)[N]) {
    if constexpr (N == 2)
      *reinterpret_cast<float2*>(p) = make_float2(x[0], x[1]);
    else
      p[0] = x[0];
  }
  template <int N>
  static __device__ __forceinline__ void storeN(T* p, const float (&x)[N], const float (&f)[N]) {
    float y[N];
#pragma unroll
    for (int i = 0; i < N; ++i) y[i] = x[i] * f[i];
    storeN<N>(p, y);
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
  static constexpr int NCP = DVT / 2;                // v column pairs
  static constexpr int RPL = (C * NCP + NT - 1) / NT; // v rows per thread
  static constexpr int VW = (2 * IOES) / 4;          // dwords per column pair

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
  static_assert(NT % NCP == 0 && (NT / NCP) * RPL >= C, "v tile mapping");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// ---- chunk input prefetch ---------------------------------------------------
// Raw (undecoded) registers of one chunk's inputs for this thread.  The next
// chunk's loads are issued into them right after the current chunk has been
// decoded, so HBM latency hides behind a whole chunk of compute.  Row offsets
// are clamped to the chunk's last valid row, so every access stays inside the
// tensors; padded rows are replaced after the load (q = k = v = 0, alpha = 1,
// beta = 0: identity tokens).
template <class Cfg>
struct Prefetch {
  static constexpr int QB = Cfg::CPT * Cfg::IOES;  // bytes of q (or k) per row and lane
  static constexpr int QW = (QB + 3) / 4;
  uint32_t q[16][QW], k[16][QW], al[16][Cfg::CPT];
  uint32_t v[Cfg::RPL][Cfg::VW];
  uint32_t vb[Cfg::RPL];
  uint32_t bt;
};

template <int BYTES>
__device__ __forceinline__ void ldraw(rsrc_t r, int voff, int soff, uint32_t* d) {
  if constexpr (BYTES == 2) {
    d[0] = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
  } else if constexpr (BYTES == 4) {
    d[0] = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
  } else if constexpr (BYTES == 8) {
    const auto u = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
    d[0] = u[0];
    d[1] = u[1];
  } else {
    static_assert(BYTES == 16, "load width");
    const auto u = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
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

__device__ __forceinline__ int sclamp(int x, int hi) { return x < hi ? x : hi; }

template <class Cfg>
__device__ __forceinline__ void issue_loads(Prefetch<Cfg>& pf, const FwdArgs& a, int64_t t,
                                            int Ln, int h, int dv0, int tid, int scan_I,
                                            bool scan_on, int c0ch) {
  using IO = typename Cfg::IO;
  constexpr int DK = Cfg::DK, ES = Cfg::IOES;
  const int H = a.H;
  const int krow = H * DK * ES;       // bytes per token in q / k
  const int arow = H * DK * 4;        // bytes per token in alpha
  const int vrow = H * a.dv * ES;     // bytes per token in v
  const int64_t qk_off = (t * H + h) * static_cast<int64_t>(DK);
  if (scan_on) {
    const rsrc_t rq = make_rsrc(static_cast<const char*>(a.q) + qk_off * ES, Ln * krow);
    const rsrc_t rk = make_rsrc(static_cast<const char*>(a.k) + qk_off * ES, Ln * krow);
    const rsrc_t ra = make_rsrc(a.alpha + qk_off, Ln * arow);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = sclamp(16 * scan_I + i, Ln - 1);
      ldraw<Prefetch<Cfg>::QB>(rq, c0ch * ES + row * krow, 0, pf.q[i]);
      ldraw<Prefetch<Cfg>::QB>(rk, c0ch * ES + row * krow, 0, pf.k[i]);
      ldraw<Cfg::CPT * 4>(ra, c0ch * 4 + row * arow, 0, pf.al[i]);
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
    const int j = sclamp(rg * Cfg::RPL + i, Ln - 1);
    ldraw<Cfg::VW * 4>(rv, 2 * cp * ES + j * vrow, 0, pf.v[i]);
    pf.vb[i] = __builtin_amdgcn_raw_buffer_load_b32(rb, j * H * 4, 0, 0);
  }
  pf.bt = __builtin_amdgcn_raw_buffer_load_b32(rb, sclamp(tid, Ln - 1) * H * 4, 0, 0);
}

template <class Cfg>
__global__ __launch_bounds__(NT, 1) void fwd_kernel(FwdArgs a) {
  using Op = typename Cfg::Op;
  using IO = typename Cfg::IO;
  using T = typename Cfg::T;
  using ST = typename IO::storage;
  constexpr int C = Cfg::C, DK = Cfg::DK, DVT = Cfg::DVT, NB = Cfg::NB;
  constexpr int CPT = Cfg::CPT, NCG = Cfg::NCG;
  constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC, LDF = Cfg::LDF;
  constexpr int NTN = DVT / 16;

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
    bos = a.cu_seqlens[n];
    eos = a.cu_seqlens[n + 1];
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

  const float use_l2 = static_cast<float>(a.use_l2norm);
  const int scan_I = wave;                 // sub-block handled by this wave in the scan
  const bool scan_on = (scan_I < NB) && (lane < NCG);
  const int c0ch = lane * CPT;             // first channel of this lane
  const int vcp = tid % Cfg::NCP, vrg = tid / Cfg::NCP;

  Prefetch<Cfg> pf;
  if (bos < eos)
    issue_loads<Cfg>(pf, a, bos, static_cast<int>((eos - bos) < C ? (eos - bos) : C), h, dv0, tid,
                     scan_I, scan_on, c0ch);

  for (int64_t t0 = bos; t0 < eos; t0 += C) {
    const int L = static_cast<int>((eos - t0) < C ? (eos - t0) : C);

    // ================= phase 1: decode, running products, operands =========
    // q/k/alpha of this lane's channels over the 16 rows of its sub-block.
    // Registers are reused in place as the phases go: alpha -> F -> Kt,
    // B -> Kh, q -> Qt.
    float xq[16][CPT], xk[16][CPT], F[16][CPT], Bk[16][CPT];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool in = 16 * scan_I + i < L;
#pragma unroll
      for (int c = 0; c < CPT; ++c) {
        xq[i][c] = in ? dec<IO>(pf.q[i], c) : 0.f;
        xk[i][c] = in ? dec<IO>(pf.k[i], c) : 0.f;
        F[i][c] = in ? __uint_as_float(pf.al[i][c]) : 1.f;
      }
    }
    // (beta V)^T tile: this thread's column pair over RPL rows
    {
#pragma unroll
      for (int i = 0; i < Cfg::RPL; ++i) {
        const int j = vrg * Cfg::RPL + i;
        if (j < C) {
          const float bj = (j < L) ? __uint_as_float(pf.vb[i]) : 0.f;
          sVT[(2 * vcp) * LDC + j] = Op::cvt(dec<IO>(pf.v[i], 0) * bj);
          sVT[(2 * vcp + 1) * LDC + j] = Op::cvt(dec<IO>(pf.v[i], 1) * bj);
        }
      }
    }
    if (tid < C) sbeta[tid] = (tid < L) ? __uint_as_float(pf.bt) : 0.f;
    // the next chunk's inputs stream in while this chunk is processed
    if (t0 + C < eos)
      issue_loads<Cfg>(pf, a, t0 + C, static_cast<int>((eos - t0 - C) < C ? (eos - t0 - C) : C), h,
                       dv0, tid, scan_I, scan_on, c0ch);

    if (scan_on) {
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
      // Lk, Lq and the diagonal panel slot of R (k / F on safe channels)
      T* rdiag = sR + (8 * scan_I * (scan_I + 1) + 16 * scan_I) * LDK;
      float rinv[16][CPT];
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int c = 0; c < CPT; ++c)
          rinv[i][c] = mn[c] >= kSafeMin ? xk[i][c] * __builtin_amdgcn_rcpf(F[i][c]) : 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * scan_I + i;
        Op::template storeN<CPT>(sLk + r * LDK + c0ch, xk[i], F[i]);
        Op::template storeN<CPT>(sLq + r * LDK + c0ch, xq[i], F[i]);
        Op::template storeN<CPT>(rdiag + i * LDK + c0ch, rinv[i]);
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
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          xq[i][c] = xq[i][c] * F[i][c] * gpre;    // Qt
          F[i][c] = xk[i][c] * F[i][c] * gpre;     // Kt (unscaled)
          Bk[i][c] = xk[i][c] * Bk[i][c];          // k B (the anchor factor of the R panels)
        }
        // R panels of the later blocks: rows of this block, anchor at I2's start
        float mid = 1.f;
#pragma unroll
        for (int I2 = 1; I2 < NB; ++I2) {
          if (I2 > scan_I) {
            if (I2 > scan_I + 1) mid *= gm[I2 - 1];
            T* pan = sR + (8 * I2 * (I2 + 1) + 16 * scan_I) * LDK + c0ch + c;
#pragma unroll
            for (int i = 0; i < 16; ++i) pan[i * LDK] = Op::cvt(Bk[i][c] * mid);
          }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) Bk[i][c] *= gpost;  // Kh
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
          const T* pan = sR + (8 * I * (I + 1) + 16 * J) * LDK;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          if (isA) {
            Op::template mmaK<DK>(acc, sLk + 16 * I * LDK, LDK, pan, LDK, lane);
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
              // the diagonal block also goes row-major into the diagonal block
              // of X's buffer, where the substitution reads it and then
              // overwrites it with X_II (sXf is not in use during this phase)
#pragma unroll
              for (int i = 0; i < 4; ++i) sXf[(16 * I + 4 * lq + i) * LDF + 16 * I + l16] = out[i];
            }
          } else {
            Op::template mmaK<DK>(acc, pan, LDK, sLq + 16 * I * LDK, LDK, lane);
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

    // ================= phase 4: operands for later phases; fix-ups ==========
    if (scan_on) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * scan_I + i;
        Op::template storeN<CPT>(sQt + r * LDK + c0ch, xq[i]);
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
        const int krow = H * DK;  // elements per token
        const int64_t base = (t0 * H + h) * static_cast<int64_t>(DK);
        const rsrc_t rq = make_rsrc(static_cast<const char*>(a.q) + base * Cfg::IOES,
                                    L * krow * Cfg::IOES);
        const rsrc_t rk = make_rsrc(static_cast<const char*>(a.k) + base * Cfg::IOES,
                                    L * krow * Cfg::IOES);
        const rsrc_t ra = make_rsrc(a.alpha + base, L * krow * 4);
        const int sI = __builtin_amdgcn_readfirstlane(I);
        for (int c = lq; c < DK; c += 4) {
          if (sSafe[I * DK + c]) continue;
          float kj = 0.f, qr[16], kr[16], ar[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int row = 16 * sI + r;
            const int crow = sclamp(row, L - 1);
            uint32_t t1[1], t2[1], t3[1];
            ldraw<Cfg::IOES>(rq, c * Cfg::IOES, crow * krow * Cfg::IOES, t1);
            ldraw<Cfg::IOES>(rk, c * Cfg::IOES, crow * krow * Cfg::IOES, t2);
            ldraw<4>(ra, c * 4, crow * krow * 4, t3);
            qr[r] = (row < L) ? dec<IO>(t1, 0) : 0.f;
            kr[r] = (row < L) ? dec<IO>(t2, 0) : 0.f;
            ar[r] = (row < L) ? __uint_as_float(t3[0]) : 1.f;
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
            if (r > j) {
              const float add = accA[r] * sbeta[rr] * srk[rr] * sj;
              sAT[jj * LDF + rr] += add;
              sXf[rr * LDF + jj] += add;
            }
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
      // forward substitution for column j of the diagonal block (I, I):
      // x_i = delta_ij - sum_{m<i} A(i, m) x_m, with A's rows read in one batch
      const int I = wave, j = lane;
      const float* arow = sXf + 16 * I * LDF + 16 * I;  // A(16I + i, 16I + m) at [i * LDF + m]
      f32x4 av[16][4];
#pragma unroll
      for (int i = 1; i < 16; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if (4 * g < i) av[i][g] = *reinterpret_cast<const f32x4*>(arow + i * LDF + 4 * g);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < i; ++m) acc -= av[i][m >> 2][m & 3] * x[m];
        x[i] = acc;
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
    // X (lower blocks; zeros above the diagonal inside the diagonal blocks) as
    // an MFMA operand.  Blocks above the diagonal stay zero from the start.
    {
      constexpr int NLB = NB * (NB + 1) / 2;   // lower 16x16 blocks
      constexpr int NQ = NLB * 16 * 4;         // 4-element groups
      for (int e = tid; e < NQ; e += NT) {
        int blk = e / 64, w = e % 64;
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

    // ================= phase 6: W and Ubar ==================================
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

    // ================= phase 7: U = Ubar - W S0; store U' = Diag(rk) U ======
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

    // ================= phase 8: outputs and state update ====================
    {
      constexpr int NOT = NTN * (C / 16);
      constexpr int NU = (NOT + NW - 1) / NW;
#pragma unroll 1
      for (int u = 0; u < NU; ++u) {
        const int tt = wave + NW * u;
        if (tt < NOT) {
          const int db = tt / (C / 16), rb = tt % (C / 16);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          Op::template mmaK<DK>(acc, sS + 16 * db * LDK, LDK, sQt + 16 * rb * LDK, LDK, lane);
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
