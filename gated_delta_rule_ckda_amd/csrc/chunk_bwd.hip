// Backward of the chunked forward: gradients of o and of the final state
// with respect to q, k, v, alpha, beta and h0.
//
// The forward of one chunk (transform pass, chunk_prep.hip) with entry state
// S0, Y = X Diag(beta), Z = V - Kt S0, U = Y Z:
//   O  = scale (Qt S0 + P U),   S1 = Diag(g) S0 + Kh^T U
// (Kt = k^ F, Qt = q^ F, Rk = k^ / F with F the running gate product of the
// chunk, Kh = g Rk, P = tril(Qt Rk^T), G = tril(Kt Rk^T, -1), A = Diag(beta) G,
// X = (I + A)^{-1}; picx.dev summary of the Complex KDA paper, section
// "Background", for the recurrence these factor).  Reverse mode through it,
// given dO and the adjoint dS1 of the chunk's exit state:
//   dU  = scale P^T dO + Kh dS1
//   dS0 = scale Qt^T dO + Diag(g) dS1 - Kt^T Y^T dU,    dV = Y^T dU
// (the state adjoint runs backwards over the chunks of a sequence), and,
// chunk by chunk and independently,
//   dQt = scale dO S0^T + dP Rk,   dP = tril(scale dO U^T)
//   dKt = -(Y^T dU) S0^T + dG Rk,  dKh = U dS1^T,  dg = rowsum(dS1 * S0)
//   dY = dU Z^T,  dX = dY Diag(beta),  dbeta_j = sum_r X_rj dY_rj
//   dA = -X^T dX X^T (strictly lower),  dbeta_r += sum_j dA_rj G_rj,
//   dG = Diag(beta) dA,  dRk = dG^T Kt + dP^T Qt + g * dKh
//   dk^ = dKt F + dRk / F,  dq^ = dQt F,
//   Lam = dKt Kt + dQt Qt - dRk Rk  (+ (dg + sum_j dKh_j Rk_j) g on the last row)
//   dalpha_s = (sum_{r >= s} Lam_r) / alpha_s
// and through each L2 norm dx = r (dx^ - x^ (x^ . dx^)).  The ratio form
// needs every |F| of the chunk in [2^-100, 2^10]; other chunks (exact zero
// gates, gates that decay fast) are redone token by token from the chunk's
// entry state, with no division.
//
// Launches (all on the caller's stream):
//   1. the forward's two passes, also recording X (fp32) and every chunk's
//      entry state, and writing no output (skipped when the caller kept
//      these records from a forward of its own)
//   2. bwd_state_kernel: per (sequence, head, dv tile), chunks in reverse:
//      dU and dS1 of every chunk to the workspace, dv, dh0
//   3. per (chunk, head), the ratio form: dq, dk, dalpha, dbeta; flags the
//      chunks it cannot take.  bf16 inputs: bwd_chunk_kernel on the matrix
//      cores (a dP/dG part, then a dq/dk part on what the first left in
//      LDS); fp32 inputs: bwd_intra_kernel
//   4. bwd_token_kernel: the flagged chunks, token by token
// All arithmetic is fp32 (gradients are fp32 buffers); the forward's blocks
// are read in their storage type.
#include "mfma_ops.h"

namespace ckda {


namespace {

constexpr float kRegMin = 0x1p-100f, kRegMax = 0x1p+10f;
constexpr int kNT = 256;
// workgroups of the intra-chunk kernel: two per CU, all resident at once, so
// that the scratch they cycle through stays in the last-level caches
constexpr int64_t kGrid3 = 512;

// tokens of chunk slot c: first token t0, length L (n < 0: unused slot).
// Every caller passes a c that is the same across its workgroup.  The chunk
// map is read through generic pointers, whose loads the compiler takes as
// per-lane, so the values are made uniform explicitly: buffer descriptors
// formed from t0 and L then stay in scalar registers (a descriptor the
// compiler takes as per-lane costs a loop around every store that uses it).
struct Geo {
  int64_t t0;
  int L, n;  // n: 0 for a used slot, -1 for an unused one
};
__device__ __forceinline__ Geo geo_of(const FwdArgs& a, int c) {
  Geo g{0, 0, -1};
  const int C = a.chunk;
  if (a.cu_seqlens) {
    const int2 gc = a.chunk_geo[c];  // one load: the chunk's first token and length
    const int L = uniform32(gc.y);
    if (L == 0) return g;
    g.n = 0;
    g.t0 = uniform32(gc.x);
    g.L = L;
  } else {
    const int n = c / a.nc, i = c % a.nc;
    g.n = n;
    g.t0 = static_cast<int64_t>(n) * a.T + static_cast<int64_t>(i) * C;
    g.L = (a.T - i * C) < C ? (a.T - i * C) : C;
  }
  return g;
}

// element (row, col) of a block row-major matrix with rows of length K, in
// the block's storage order (perm32 for bf16 rows whose length is a
// multiple of 32)
template <class IO>
__device__ __forceinline__ float blk_at(const typename IO::storage* m, int row, int col, int K) {
  constexpr bool bf = sizeof(typename IO::storage) == 2;
  const int p = (bf && K % 32 == 0) ? perm32(col) : col;
  return IO::load(m, static_cast<int64_t>(row) * K + p);
}

__device__ __forceinline__ float block_sum(float v, float* red) {
  // sum over the workgroup (kNT threads); red holds kNT / 64 floats
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < kNT / 64; ++i) s += red[i];
  return s;
}

// out(m, n) = alpha * sum_k A(m, k) B(k, n) (+ out(m, n) when acc), fp32, for
// M <= 64, N <= 128, by the kNT threads of the workgroup on the fp32 matrix
// cores (16x16x4 MFMA): wave w owns the 32 x 64 quarter of rows 32 (w & 1)
// and columns 64 (w >> 1), as 2 x 4 tiles of 16 x 16.  la(m, k) and
// lb(k, n) load the operands (any storage); out(m, n) = O[m om + n on] (any
// address space).  K is walked in slices of 16 staged in LDS (`stage`,
// kGStage floats); a_mfast / b_nfast say which index of the operand is the
// contiguous one, so that consecutive threads stage consecutive elements.
// Ends with a barrier.
constexpr int kGM = 4, kGN = 8;
// staging floats for K slices of ks
constexpr int gstage(int ks) { return ks * (16 * kGM + 1) + ks * (16 * kGN + 1); }
constexpr int kGStage = gstage(16);
template <bool PREFETCH = true, int KS = 16, class LA, class LB>
__device__ __forceinline__ void gemm(int M, int N, int K, float alpha, bool acc, LA la,
                                     bool a_mfast, LB lb, bool b_nfast, float* O, int om, int on,
                                     float* stage) {
  constexpr int MP = 16 * kGM, NP = 16 * kGN;
  // threadIdx.x through an opaque move, so that each product forms its
  // lane-dependent addresses here instead of having them hoisted out of the
  // kernel's loops for every product at once (which only costs spills)
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(static_cast<int>(threadIdx.x)));
  const int lane = tid & 63, w = tid >> 6, l16 = lane & 15, lq = lane >> 4;
  const int m0 = 32 * (w & 1), n0 = 64 * (w >> 1);
  float* sA = stage;                   // [KS][MP + 1]
  float* sB = stage + KS * (MP + 1);   // [KS][NP + 1]
  f32x4 c[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) c[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // this thread's staging elements of one K slice, loaded one slice ahead
  constexpr int NA = KS * MP / kNT, NB2 = KS * NP / kNT;
  float ra[NA], rb[NB2];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      const int e = tid + u * kNT;
      int kk, m;
      if (a_mfast) { m = e % MP; kk = e / MP; } else { kk = e % KS; m = e / KS; }
      ra[u] = (m < M && k0 + kk < K) ? la(m, k0 + kk) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < NB2; ++u) {
      const int e = tid + u * kNT;
      int kk, n;
      if (b_nfast) { n = e % NP; kk = e / NP; } else { kk = e % KS; n = e / KS; }
      rb[u] = (n < N && k0 + kk < K) ? lb(k0 + kk, n) : 0.f;
    }
  };
  // tiles wholly outside M x N are skipped (the same for the whole wave)
  const bool live_m1 = m0 + 16 < M, live_n = n0 < N;
  if (PREFETCH) fetch(0);
  for (int k0 = 0; k0 < K; k0 += KS) {
    if (!PREFETCH) fetch(k0);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NA; ++u) {
      const int e = tid + u * kNT;
      int kk, m;
      if (a_mfast) { m = e % MP; kk = e / MP; } else { kk = e % KS; m = e / KS; }
      sA[kk * (MP + 1) + m] = ra[u];
    }
#pragma unroll
    for (int u = 0; u < NB2; ++u) {
      const int e = tid + u * kNT;
      int kk, n;
      if (b_nfast) { n = e % NP; kk = e / NP; } else { kk = e % KS; n = e / KS; }
      sB[kk * (NP + 1) + n] = rb[u];
    }
    __syncthreads();
    if (PREFETCH && k0 + KS < K) fetch(k0 + KS);  // in flight while this slice is multiplied
    if (live_n) {
#pragma unroll
      for (int k4 = 0; k4 < KS; k4 += 4) {
        const int kr = k4 + lq;
        float av[2], bv[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) av[i] = sA[kr * (MP + 1) + m0 + 16 * i + l16];
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = sB[kr * (NP + 1) + n0 + 16 * j + l16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          c[0][j] = mfma_f32(av[0], bv[j], c[0][j]);
          if (live_m1) c[1][j] = mfma_f32(av[1], bv[j], c[1][j]);
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 16 * i + 4 * lq + r, n = n0 + 16 * j + l16;
        if (m < M && n < N) {
          float* o = O + m * om + n * on;
          *o = acc ? *o + alpha * c[i][j][r] : alpha * c[i][j][r];
        }
      }
  __syncthreads();
}
// the same with both operands strided fp32 arrays: A(m, k) = A[m am + k ak],
// B(k, n) = B[k bk + n bn]; no slice prefetch (a kernel with many products
// inlined would run out of registers)
__device__ __forceinline__ void gemm(int M, int N, int K, float alpha, bool acc, const float* A,
                                     int am, int ak, const float* B, int bk, int bn, float* O,
                                     int om, int on, float* stage) {
  gemm<true>(M, N, K, alpha, acc, [=](int m, int k) { return A[m * am + k * ak]; }, am == 1,
       [=](int k, int n) { return B[k * bk + n * bn]; }, bn == 1, O, om, on, stage);
}

// ---------------------------------------------------------------- 2: state
// The state adjoint on the matrix cores: one workgroup per (sequence, head,
// dv tile), over the sequence's chunks in reverse.  Per chunk, with dS1 the
// adjoint at the chunk's end and the block's operands as the transform pass
// stored them (P' = scale P, X' = Y, W' = -W, Qt' = scale Qt, Kh' = Kh):
//   dU  = P'^T dO + Kh' dS1
//   dV  = X'^T dU
//   dS0 = Diag(g) dS1 + W'^T dU + Qt'^T dO
// The step has the forward state pass's shape with every block operand
// transposed, and the same division of labour: state waves own 16 columns of
// the tile each (the adjoint in fp32 accumulators, dU in registers), loader
// waves stream the blocks and the dO rows two chunks ahead.  The loaders
// write the transposes into LDS: a unit is one 16-byte piece of two adjacent
// source rows, so that each LDS write is a pair of adjacent elements of a
// transposed row, in the order the state waves read as fragments.
struct TSec {
  int g0, R, Kc, l0, ldd;  // R source rows of Kc elements at block byte g0 -> LDS [Kc][ldd] at byte l0
  bool tri;                // X' or P' (packed rows when the block is packed)
};

template <class OpT, class IOT, int C_, int DK_, int DV_, int DVT_>
struct BCfg {
  using Op = OpT;
  using IO = IOT;
  using T = typename Op::T;
  using Frag = typename Op::Frag;
  static constexpr int C = C_, DK = DK_, DV = DV_, DVT = DVT_;
  static constexpr int NSPLIT = DV / DVT;
  static constexpr int NSW = DVT / 16, NLW = 8;
  static constexpr int NT = 64 * (NSW + NLW), NLT = 64 * NLW;
  static constexpr int NB = C / 16, NMC = DK / 16;
  static constexpr int ES = static_cast<int>(sizeof(T));
  static constexpr int IOES = static_cast<int>(sizeof(typename IO::storage));
  static constexpr int LDK = frag_stride(DK, ES), LDC = frag_stride(C, ES);
  static constexpr int KS = Op::KS;
  static constexpr int NFK = (DK + KS - 1) / KS, NFC = (C + KS - 1) / KS;
  // P'^T and X'^T are upper triangular: K fragment s of row block rb holds a
  // nonzero only if its last column is at or right of the block's first row
  static constexpr bool up_live(int rb, int s) { return KS * s + KS - 1 >= 16 * rb; }
  // the block (bytes); X' and P' packed when TRI (first C/2 rows half long)
  static constexpr bool TRI = tri_packed(C, ES);
  static constexpr int TRIB = static_cast<int>(tri_elems(C, ES)) * ES;
  static constexpr int GB_X = 0, GB_W = TRIB, GB_Q = GB_W + C * DK * ES,
                       GB_P = GB_Q + C * DK * ES, GB_K = GB_P + TRIB,
                       GB_G = GB_K + DK * C * ES, GB_END = GB_G + DK * 4;
  // LDS (bytes)
  static constexpr int O_PT = 0;                                  // P'^T  [C][LDC]
  static constexpr int O_KH = align16(O_PT + C * LDC * ES);       // Kh'   [C][LDK]
  static constexpr int O_OT = align16(O_KH + C * LDK * ES);       // dO^T  [DVT][LDC]
  static constexpr int O_YT = align16(O_OT + DVT * LDC * ES);     // X'^T  [C][LDC]
  static constexpr int O_WT = align16(O_YT + C * LDC * ES);       // W'^T  [DK][LDC]
  static constexpr int O_QT = align16(O_WT + DK * LDC * ES);      // Qt'^T [DK][LDC]
  static constexpr int O_G = align16(O_QT + DK * LDC * ES);       // g [DK] fp32
  // the step's outputs, staged for whole-row stores by the loader waves:
  // dS1 [DK][DVT] and dU [C][DVT] in the io type, dV [C][DVT] fp32; rows
  // padded so that the four rows a state-wave store touches fall in
  // different banks
  static constexpr int SROW = DVT * IOES, LDS_S = SROW + 16, LDS_V = DVT * 4 + (DVT * 4 >= 64 ? 64 : 16);
  static constexpr int O_SS = align16(O_G + DK * 4);
  static constexpr int O_SU = O_SS + DK * LDS_S;
  static constexpr int O_SV = O_SU + C * LDS_S;
  static constexpr int LDS_BYTES = align16(O_SV + C * LDS_V);
  static_assert(SROW % 16 == 0 && (DVT * 4) % 16 == 0, "staged rows in 16-byte pieces");
  static_assert(GB_G == blk_g_byte(C, DK, ES), "block layout");
  static_assert(DV % DVT == 0 && DVT % 16 == 0 && NSW >= 1 && NSW <= 4, "dv tiling");
  static_assert((C * ES) % 16 == 0 && (DK * ES) % 16 == 0 && (DVT * IOES) % 16 == 0, "rows in pieces");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// logical index of storage position p in a perm32-ordered row (inverse of perm32)
__host__ __device__ constexpr int unperm32(int p) {
  return (p & ~31) | (((p >> 2) & 1) << 4) | (((p & 31) >> 3) << 2) | (p & 3);
}

// One loader thread's share of one chunk's group: A = {P'^T, Kh', dO^T} (what
// dU needs), B = {X'^T, W'^T, Qt'^T, g}.  Loads are issued for clamped
// indices whatever the thread's share, so every group has the same number of
// loads; duplicates are dropped at the store.
template <class Cfg, bool A>
struct BGroup {
  static constexpr int C = Cfg::C, DK = Cfg::DK, ES = Cfg::ES, NLT = Cfg::NLT;
  static constexpr int NS = A ? 2 : 3;
  static constexpr TSec sec(int k) {
    return A ? (k == 0 ? TSec{Cfg::GB_P, C, C, Cfg::O_PT, Cfg::LDC, true}
                       : TSec{Cfg::GB_K, DK, C, Cfg::O_KH, Cfg::LDK, false})
             : (k == 0   ? TSec{Cfg::GB_X, C, C, Cfg::O_YT, Cfg::LDC, true}
                : k == 1 ? TSec{Cfg::GB_W, C, DK, Cfg::O_WT, Cfg::LDC, false}
                         : TSec{Cfg::GB_Q, C, DK, Cfg::O_QT, Cfg::LDC, false});
  }
  // unit (row pair jp, piece cp) of a packed X' or P' that is not stored
  // (rows below C/2, pieces past the half row); its load reads the live
  // piece cp - C/2 * ES / 16 of the same rows instead, and it is not stored
  static constexpr int HP = C / 2 * ES / 16;
  static __device__ __forceinline__ bool dead(const TSec& s, int jp, int cp) {
    return Cfg::TRI && s.tri && 2 * jp < C / 2 && cp >= HP;
  }
  // byte offset of row r of a section
  static __device__ __forceinline__ int row_off(const TSec& s, int r) {
    return (Cfg::TRI && s.tri) ? static_cast<int>(tri_row(C, ES, r)) * ES : r * s.Kc * ES;
  }
  static constexpr int units(int k) { return sec(k).R / 2 * (sec(k).Kc * ES / 16); }
  static constexpr int per(int k) { return (units(k) + NLT - 1) / NLT; }
  static constexpr int first(int k) { return k == 0 ? 0 : first(k - 1) + per(k - 1); }
  static constexpr int NU = first(NS);
  static constexpr int NVU = A ? (C / 2) * (Cfg::DVT * Cfg::IOES / 16) : 0;  // dO units
  static constexpr int NV = (NVU + NLT - 1) / NLT;
  static constexpr int NGP = DK * 4 / 16;                                 // g pieces
  static constexpr int NG = A ? 0 : (NGP + NLT - 1) / NLT;
  uint32_t d[2 * NU + 2 * NV + NG][4];

  __device__ __forceinline__ void issue(const unsigned char* blk, const void* dout, int64_t t0, int L,
                                        int H, int h, int dv0, int lt) {
    using ST = typename Cfg::IO::storage;
    const rsrc_t rb = make_rsrc(blk, Cfg::GB_END);
#pragma unroll
    for (int k = 0; k < NS; ++k) {
#pragma unroll
      for (int u = 0; u < per(k); ++u) {
        const TSec s = sec(k);
        const int uu = iclamp(lt + NLT * u, units(k) - 1);
        const int jp = uu % (s.R / 2), cp0 = uu / (s.R / 2);
        const int cp = dead(s, jp, cp0) ? cp0 - HP : cp0;
        ldraw<16>(rb, s.g0 + row_off(s, 2 * jp) + 16 * cp, d[2 * (first(k) + u)]);
        ldraw<16>(rb, s.g0 + row_off(s, 2 * jp + 1) + 16 * cp, d[2 * (first(k) + u) + 1]);
      }
    }
    if constexpr (A) {
      const int vrow = H * Cfg::DV * Cfg::IOES;
      const rsrc_t rv = make_rsrc(
          static_cast<const ST*>(dout) + (t0 * H + h) * static_cast<int64_t>(Cfg::DV) + dv0, L * vrow);
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int uv = iclamp(lt + NLT * u, NVU - 1);
        const int jp = uv % (C / 2), cp = uv / (C / 2);
        ldraw<16>(rv, iclamp(2 * jp, L - 1) * vrow + 16 * cp, d[2 * NU + 2 * u]);
        ldraw<16>(rv, iclamp(2 * jp + 1, L - 1) * vrow + 16 * cp, d[2 * NU + 2 * u + 1]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < NG; ++u)
        ldraw<16>(rb, Cfg::GB_G + 16 * iclamp(lt + NLT * u, NGP - 1), d[2 * NU + u]);
    }
  }

  __device__ __forceinline__ void store(unsigned char* smem, int L, int lt) const {
    using Op = typename Cfg::Op;
    using T = typename Cfg::T;
    constexpr int NE = 16 / ES;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
#pragma unroll
      for (int u = 0; u < per(k); ++u) {
        const TSec s = sec(k);
        const int uu = lt + NLT * u;
        const int jp = uu % (s.R / 2), cp = uu / (s.R / 2);
        if ((units(k) % NLT == 0 || uu < units(k)) && !dead(s, jp, cp)) {
          const bool sp = ES == 2 && s.Kc % 32 == 0, dp = ES == 2 && s.R % 32 == 0;
          const int q = dp ? perm32(2 * jp) : 2 * jp;
          T* dst = reinterpret_cast<T*>(smem + s.l0);
          const uint32_t* r0 = d[2 * (first(k) + u)];
          const uint32_t* r1 = d[2 * (first(k) + u) + 1];
#pragma unroll
          for (int e = 0; e < NE; ++e) {
            const int p = NE * cp + e, c = sp ? unperm32(p) : p;
            Op::store2(dst + c * s.ldd + q, dec<typename Cfg::IO>(r0, e), dec<typename Cfg::IO>(r1, e));
          }
        }
      }
    }
    if constexpr (A) {
      constexpr int NEV = 16 / Cfg::IOES;
      T* ot = reinterpret_cast<T*>(smem + Cfg::O_OT);
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const int uv = lt + NLT * u;
        if (NVU % NLT == 0 || uv < NVU) {
          const int jp = uv % (C / 2), c0 = (uv / (C / 2)) * NEV;
          const bool in0 = 2 * jp < L, in1 = 2 * jp + 1 < L;
          const int q = Op::template pos<C>(2 * jp);
#pragma unroll
          for (int e = 0; e < NEV; ++e) {
            const float x0 = in0 ? dec<typename Cfg::IO>(d[2 * NU + 2 * u], e) : 0.f;
            const float x1 = in1 ? dec<typename Cfg::IO>(d[2 * NU + 2 * u + 1], e) : 0.f;
            Op::store2(ot + (c0 + e) * Cfg::LDC + q, x0, x1);
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < NG; ++u) {
        const int p = lt + NLT * u;
        if (p < NGP) {
          const uint32_t* r = d[2 * NU + u];
          *reinterpret_cast<uint4*>(smem + Cfg::O_G + 16 * p) = make_uint4(r[0], r[1], r[2], r[3]);
        }
      }
    }
  }
};

template <class Cfg>
__global__ __launch_bounds__(Cfg::NT, 1) void bwd_state_kernel(BwdArgs b) {
  using Op = typename Cfg::Op;
  using IO = typename Cfg::IO;
  using ST = typename IO::storage;
  using T = typename Cfg::T;
  using Frag = typename Cfg::Frag;
  constexpr int C = Cfg::C, DK = Cfg::DK, NB = Cfg::NB, NMC = Cfg::NMC;
  constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC, NFC = Cfg::NFC, NFK = Cfg::NFK;
  const FwdArgs& a = b.f;
  extern __shared__ __align__(16) unsigned char smem[];
  const T* sPT = reinterpret_cast<const T*>(smem + Cfg::O_PT);
  const T* sKH = reinterpret_cast<const T*>(smem + Cfg::O_KH);
  const T* sOT = reinterpret_cast<const T*>(smem + Cfg::O_OT);
  const T* sYT = reinterpret_cast<const T*>(smem + Cfg::O_YT);
  const T* sWT = reinterpret_cast<const T*>(smem + Cfg::O_WT);
  const T* sQT = reinterpret_cast<const T*>(smem + Cfg::O_QT);
  const float* sg = reinterpret_cast<const float*>(smem + Cfg::O_G);

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const bool is_state = wave < Cfg::NSW;
  const int lt = tid - 64 * Cfg::NSW;

  // the dv tiles of one (sequence, head) 8 workgroups apart: same XCD, so
  // they share its L2 for the blocks
  const int64_t nblk = gridDim.x, bi = blockIdx.x;
  int64_t pair;
  int split;
  if (Cfg::NSPLIT > 1 && nblk % (8 * Cfg::NSPLIT) == 0) {
    const int64_t xcd = bi % 8, slot = bi / 8;
    pair = (slot / Cfg::NSPLIT) * 8 + xcd;
    split = static_cast<int>(slot % Cfg::NSPLIT);
  } else {
    pair = bi / Cfg::NSPLIT;
    split = static_cast<int>(bi % Cfg::NSPLIT);
  }
  const int H = a.H, dv = a.dv;
  // packed sequences longest first, as in the forward's state pass
  const int n = a.cu_seqlens ? uniform32(a.seq_order[pair / H]) : static_cast<int>(pair / H);
  const int h = static_cast<int>(pair % H);
  int64_t s0;
  int c_begin, nch;
  if (a.cu_seqlens) {
    s0 = uniform64(a.cu_seqlens[n]);
    c_begin = uniform32(a.first[n]);
    nch = uniform32(a.first[n + 1]) - c_begin;
  } else {
    s0 = static_cast<int64_t>(n) * a.T;
    c_begin = n * a.nc;
    nch = a.nc;
  }
  const int64_t s1 = a.cu_seqlens ? uniform64(a.cu_seqlens[n + 1]) : s0 + a.T;
  const int dv0 = split * Cfg::DVT;
  const unsigned char* blocks = a.blocks + static_cast<int64_t>(h) * a.maxc * a.blk_bytes;
  auto chunk_t0 = [&](int i) { return s0 + static_cast<int64_t>(i) * C; };
  auto chunk_len = [&](int i) {
    const int64_t rem = s1 - chunk_t0(i);
    return static_cast<int>(rem < C ? rem : C);
  };

  // adjoint slab: tile mc holds rows 16mc + 4lq + i, column dv0 + 16 wave + l16
  f32x4 sacc[NMC];
  const int col = dv0 + 16 * wave + l16;
  const int64_t st_base = (static_cast<int64_t>(n) * H + h) * DK * dv + col;
  if (is_state) {
#pragma unroll
    for (int mc = 0; mc < NMC; ++mc)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sacc[mc][i] = b.dht ? b.dht[st_base + static_cast<int64_t>(16 * mc + 4 * lq + i) * dv] : 0.f;

    for (int k = 0; k < nch; ++k) {  // chunk nch - 1 - k; the loaders store its outputs
      {  // the adjoint at the chunk's end, for the intra-chunk pass (staged;
         // the loaders store it)
        ST* ds = reinterpret_cast<ST*>(smem + Cfg::O_SS) + 16 * wave + l16;
#pragma unroll
        for (int mc = 0; mc < NMC; ++mc)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            IO::store(ds, (16 * mc + 4 * lq + ii) * (Cfg::LDS_S / Cfg::IOES), sacc[mc][ii]);
      }
      __syncthreads();  // group A of this chunk is in LDS
      Frag sf[NFK], of[NFC];
      Op::template frags<DK>(sf, sacc);
      // dU tiles: P'^T dO + Kh' dS1 (all fragments read first, then the MFMAs)
      f32x4 uacc[NB];
      {
        Frag pf[NB][NFC], kf[NB][NFK];
        const T* orow = sOT + (16 * wave + l16) * LDC;
#pragma unroll
        for (int s = 0; s < NFC; ++s) of[s] = Op::template row_frag<C>(orow, s, lq);
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
#pragma unroll
          for (int s = 0; s < NFC; ++s)
            if (Cfg::up_live(rb, s)) pf[rb][s] = Op::template row_frag<C>(sPT + (16 * rb + l16) * LDC, s, lq);
#pragma unroll
          for (int s = 0; s < NFK; ++s) kf[rb][s] = Op::template row_frag<DK>(sKH + (16 * rb + l16) * LDK, s, lq);
        }
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
          uacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NFC; ++s)
            if (Cfg::up_live(rb, s)) Op::mma(uacc[rb], pf[rb][s], of[s]);
#pragma unroll
          for (int s = 0; s < NFK; ++s) Op::mma(uacc[rb], kf[rb][s], sf[s]);
        }
      }
      {
        ST* du = reinterpret_cast<ST*>(smem + Cfg::O_SU) + 16 * wave + l16;
#pragma unroll
        for (int rb = 0; rb < NB; ++rb)
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            IO::store(du, (16 * rb + 4 * lq + ii) * (Cfg::LDS_S / Cfg::IOES), uacc[rb][ii]);
      }
      Frag uf[NFC];
      Op::template frags<C>(uf, uacc);
      __syncthreads();  // group B of this chunk is in LDS
      {  // dV = X'^T dU (staged; the loaders store rows < L one step later)
        float* dvo = reinterpret_cast<float*>(smem + Cfg::O_SV) + 16 * wave + l16;
        Frag yf[NB][NFC];
#pragma unroll
        for (int rb = 0; rb < NB; ++rb)
#pragma unroll
          for (int s = 0; s < NFC; ++s)
            if (Cfg::up_live(rb, s)) yf[rb][s] = Op::template row_frag<C>(sYT + (16 * rb + l16) * LDC, s, lq);
#pragma unroll
        for (int rb = 0; rb < NB; ++rb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < NFC; ++s)
            if (Cfg::up_live(rb, s)) Op::mma(acc, yf[rb][s], uf[s]);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) dvo[(16 * rb + 4 * lq + ii) * (Cfg::LDS_V / 4)] = acc[ii];
        }
      }
      // dS0 = Diag(g) dS1 + W'^T dU + Qt'^T dO, in two halves of the rows
      constexpr int NH = NMC >= 2 ? 2 : 1, MH = NMC / NH;
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        Frag wf[MH][NFC], qf[MH][NFC];
        f32x4 gv[MH];
#pragma unroll
        for (int m = 0; m < MH; ++m) {
          const int mc = hf * MH + m;
          gv[m] = *reinterpret_cast<const f32x4*>(sg + 16 * mc + 4 * lq);
#pragma unroll
          for (int s = 0; s < NFC; ++s) {
            wf[m][s] = Op::template row_frag<C>(sWT + (16 * mc + l16) * LDC, s, lq);
            qf[m][s] = Op::template row_frag<C>(sQT + (16 * mc + l16) * LDC, s, lq);
          }
        }
#pragma unroll
        for (int m = 0; m < MH; ++m) {
          const int mc = hf * MH + m;
          sacc[mc] *= gv[m];
#pragma unroll
          for (int s = 0; s < NFC; ++s) {
            Op::mma(sacc[mc], wf[m][s], uf[s]);
            Op::mma(sacc[mc], qf[m][s], of[s]);
          }
        }
      }
    }
    __syncthreads();  // the loaders store the last chunk's dV
    if (b.dh0) {
#pragma unroll
      for (int mc = 0; mc < NMC; ++mc)
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
          b.dh0[st_base + static_cast<int64_t>(16 * mc + 4 * lq + ii) * dv] = sacc[mc][ii];
    }
  } else {
    using GA = BGroup<Cfg, true>;
    using GB = BGroup<Cfg, false>;
    // step k works on chunk nch - 1 - k; loads past the last step repeat it
    auto chunk_of = [&](int k) { return nch - 1 - (k < nch - 1 ? k : nch - 1); };
    auto blk = [&](int i) { return blocks + static_cast<int64_t>(c_begin + i) * a.blk_bytes; };
    auto issueA = [&](GA& g, int k) {
      const int i = chunk_of(k);
      g.issue(blk(i), b.dout, chunk_t0(i), chunk_len(i), H, h, dv0, lt);
    };
    auto issueB = [&](GB& g, int k) { g.issue(blk(chunk_of(k)), nullptr, 0, 1, H, h, dv0, lt); };
    GA sa0, sa1;
    GB sb0, sb1;
    if (nch > 0) {
      issueA(sa0, 0);
      issueB(sb0, 0);
      issueA(sa1, 1);
      issueB(sb1, 1);
      sa0.store(smem, chunk_len(chunk_of(0)), lt);
      issueA(sa0, 2);
    }
    // the state waves' staged outputs of step k, as whole rows
    constexpr int NLT = Cfg::NLT, IOES = Cfg::IOES;
    auto slot_of = [&](int k) { return static_cast<int64_t>(h) * a.maxc + c_begin + chunk_of(k); };
    auto flush_dS = [&](int k) {
      flush_rows<DK, Cfg::SROW, Cfg::LDS_S, NLT>(
          smem + Cfg::O_SS, static_cast<unsigned char*>(b.dS) + (slot_of(k) * DK * dv + dv0) * IOES,
          static_cast<int64_t>(dv) * IOES, DK, lt);
    };
    auto flush_dU = [&](int k) {
      flush_rows<C, Cfg::SROW, Cfg::LDS_S, NLT>(
          smem + Cfg::O_SU, static_cast<unsigned char*>(b.dU) + (slot_of(k) * C * dv + dv0) * IOES,
          static_cast<int64_t>(dv) * IOES, C, lt);
    };
    auto flush_dV = [&](int k) {
      const int i = chunk_of(k);
      flush_rows<C, Cfg::DVT * 4, Cfg::LDS_V, NLT>(
          smem + Cfg::O_SV, reinterpret_cast<unsigned char*>(b.dv + (chunk_t0(i) * H + h) * dv + dv0),
          static_cast<int64_t>(H) * dv * 4, chunk_len(i), lt);
    };
    // step k: B(k) (in gb) goes to LDS while dU(k) runs, then A(k+1) (in ga)
    // while dV(k) and dS0(k) run; gb then takes B(k+2) and ga takes A(k+3).
    // dS1(k) and dV(k-1) were staged before the first barrier of step k, dU(k)
    // before the second; each is read here before the state waves stage the
    // next one (after the other barrier).
    auto step = [&](int k, GB& gb, GA& ga) {
      __syncthreads();
      gb.store(smem, 0, lt);
      issueB(gb, k + 2);
      flush_dS(k);
      if (k > 0) flush_dV(k - 1);
      __syncthreads();
      ga.store(smem, chunk_len(chunk_of(k + 1)), lt);
      issueA(ga, k + 3);
      flush_dU(k);
    };
    int k = 0;
    for (; k + 1 < nch; k += 2) {
      step(k, sb0, sa1);
      step(k + 1, sb1, sa0);
    }
    if (k < nch) step(k, sb0, sa1);
    __syncthreads();  // the last chunk's dV is staged
    if (nch > 0) flush_dV(nch - 1);
  }
}

// ---------------------------------------------------------------- 3: intra
// One (chunk, head) at a time per workgroup, items b, b + grid, ...  The
// products run through gemm(); C x C matrices in LDS where they fit, the rest
// in the workgroup's slice of the scratch.
template <class IO>
__global__ __launch_bounds__(kNT, 2) void bwd_intra_kernel(BwdArgs b) {
  using ST = typename IO::storage;
  const FwdArgs& a = b.f;
  const int C = a.chunk, dk = a.dk, dv = a.dv, H = a.H;
  const int total = a.maxc * H;
  const bool l2 = a.use_l2norm != 0;
  const float scale = a.scale;
  const int SC = C * cmax(cmax(dk, dv), C);
  float* ws = b.scratch + static_cast<int64_t>(blockIdx.x) * 14 * SC;
  // scratch slices: C x dk (stride dk) or C x dv (stride dv) or C x C
  float *sF = ws, *sKt = ws + SC, *sQt = ws + 2 * SC, *sRk = ws + 3 * SC, *sZ = ws + 4 * SC,
        *sU = ws + 5 * SC, *sT1 = ws + 6 * SC, *sV = ws + 7 * SC, *sdO = ws + 8 * SC,
        *sG = ws + 9 * SC, *sdP = ws + 10 * SC, *sdQ = ws + 11 * SC, *sdK = ws + 12 * SC,
        *sdR = ws + 13 * SC;
  extern __shared__ float sm[];
  float* lY = sm;               // [C][C] Y = X Diag(beta)
  float* ldX = lY + C * C;      // [C][C] dY -> dX
  float* lT = ldX + C * C;      // [C][C] dX X^T
  float* ldA = lT + C * C;      // [C][C] dA -> dG
  float* stage = ldA + C * C;   // gemm staging
  float* lbeta = stage + kGStage;  // [C]
  float* lrq = lbeta + C;       // [C]
  float* lrk = lrq + C;         // [C]
  float* ldb = lrk + C;         // [C]
  float* lg = ldb + C;          // [dk]
  float* ldg = lg + dk;         // [dk]
  int* lflag = reinterpret_cast<int*>(ldg + dk);
  const int tid = threadIdx.x;
  const ST* q = static_cast<const ST*>(a.q);
  const ST* k = static_cast<const ST*>(a.k);
  const ST* v = static_cast<const ST*>(a.v);
  const ST* dO = static_cast<const ST*>(b.dout);
  const float* alpha = static_cast<const float*>(a.alpha);
  const float* beta = static_cast<const float*>(a.beta);

  for (int idx = blockIdx.x; idx < total; idx += gridDim.x) {
    const int c = idx / H, h = idx % H;
    const Geo g = geo_of(a, c);
    const int64_t slot = static_cast<int64_t>(h) * a.maxc + c;
    __syncthreads();  // the previous item is done with LDS and scratch
    if (g.n < 0) {
      if (tid == 0) b.bflag[slot] = 0;
      continue;
    }
    const int64_t t0 = g.t0;
    const int L = g.L;
    static_assert(sizeof(ST) == 4, "fp32 inputs only (bf16 inputs take bwd_chunk_kernel)");
    const float* S0 = static_cast<const float*>(a.hc) + slot * dk * dv;
    const float* dS1 = static_cast<const float*>(b.dS) + slot * dk * dv;
    const float* dU = static_cast<const float*>(b.dU) + slot * C * dv;
    const float* X = a.xout + slot * C * C;
    // norms (TPR threads per row, lane groups of a wave), beta
    if (tid == 0) *lflag = 0;
    {
      const int TPR = kNT / C, r = tid / TPR, sub = tid % TPR;
      float sq = 0.f, sk = 0.f;
      if (r < L) {
        const int64_t base = ((t0 + r) * H + h) * dk;
        for (int c0 = sub; c0 < dk; c0 += 8 * TPR) {
          float xs[8], ys[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int cc = c0 + u * TPR;
            xs[u] = cc < dk ? IO::load(q, base + cc) : 0.f;
            ys[u] = cc < dk ? IO::load(k, base + cc) : 0.f;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            sq += xs[u] * xs[u];
            sk += ys[u] * ys[u];
          }
        }
      }
      for (int o = 1; o < TPR; o <<= 1) {
        sq += __shfl_xor(sq, o);
        sk += __shfl_xor(sk, o);
      }
      if (sub == 0) {
        lrq[r] = l2 ? __fdiv_rn(1.f, __fsqrt_rn(sq + kL2Eps)) : 1.f;
        lrk[r] = l2 ? __fdiv_rn(1.f, __fsqrt_rn(sk + kL2Eps)) : 1.f;
        lbeta[r] = r < L ? beta[(t0 + r) * H + h] : 0.f;
      }
    }
    // gate products per channel, 16 loads in flight at a time; regularity
    for (int cc = tid; cc < dk; cc += kNT) {
      float f = 1.f;
      bool ok = true;
      for (int r0 = 0; r0 < C; r0 += 16) {
        float al[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const int r = r0 + u;
          al[u] = r < L ? alpha[((t0 + r) * H + h) * dk + cc] : 1.f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          f *= al[u];
          sF[(r0 + u) * dk + cc] = f;
          const float m = fabsf(f);
          ok = ok && m >= kRegMin && m <= kRegMax;
        }
      }
      lg[cc] = f;
      if (!ok) *lflag = 1;
    }
    __syncthreads();
    const bool irregular = *lflag != 0;
    if (tid == 0) b.bflag[slot] = irregular ? 1 : 0;
    if (irregular) continue;
    // operands: Kt, Qt, Rk; V, dO as fp32 (rows >= L zero); Y.  Loads of 8
    // elements go out before any of them is used.
    for (int e0 = tid; e0 < C * dk; e0 += 8 * kNT) {
      float xq[8], xk[8], xf[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kNT, r = e / dk, cc = e % dk;
        const int64_t i = ((t0 + r) * H + h) * dk + cc;
        const bool in = e < C * dk && r < L;
        xq[u] = in ? IO::load(q, i) : 0.f;
        xk[u] = in ? IO::load(k, i) : 0.f;
        xf[u] = e < C * dk ? sF[e] : 1.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kNT, r = e / dk;
        if (e < C * dk) {
          const float qh = xq[u] * lrq[r], kh = xk[u] * lrk[r];
          sKt[e] = kh * xf[u];
          sQt[e] = qh * xf[u];
          sRk[e] = kh / xf[u];
        }
      }
    }
    for (int e0 = tid; e0 < C * dv; e0 += 8 * kNT) {
      float xv[8], xo[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kNT, r = e / dv, j = e % dv;
        const int64_t i = ((t0 + r) * H + h) * dv + j;
        const bool in = e < C * dv && r < L;
        xv[u] = in ? IO::load(v, i) : 0.f;
        xo[u] = in ? IO::load(dO, i) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int e = e0 + u * kNT;
        if (e < C * dv) {
          sV[e] = xv[u];
          sZ[e] = xv[u];
          sdO[e] = xo[u];
        }
      }
    }
    for (int e = tid; e < C * C; e += kNT) lY[e] = X[e] * lbeta[e % C];
    __syncthreads();
    // Z = V - Kt S0;  U = Y Z;  T1 = Y^T dU
    gemm(C, dv, dk, -1.f, true, sKt, dk, 1, S0, dv, 1, sZ, dv, 1, stage);
    gemm(C, dv, C, 1.f, false, lY, C, 1, sZ, dv, 1, sU, dv, 1, stage);
    gemm(C, dv, C, 1.f, false, lY, 1, C, dU, dv, 1, sT1, dv, 1, stage);
    // dY = dU Z^T;  dP = scale dO U^T (both lower with the diagonal);  G = Kt Rk^T
    gemm(C, C, dv, 1.f, false, dU, dv, 1, sZ, 1, dv, ldX, C, 1, stage);
    gemm(C, C, dv, scale, false, sdO, dv, 1, sU, 1, dv, sdP, C, 1, stage);
    gemm(C, C, dk, 1.f, false, sKt, dk, 1, sRk, 1, dk, sG, C, 1, stage);
    // dbeta_j = sum_r X_rj dY_rj;  dX = dY Diag(beta), masked
    for (int j = tid; j < C; j += kNT) {
      float s = 0.f;
#pragma unroll 8
      for (int r = j; r < C; ++r) s += X[r * C + j] * ldX[r * C + j];
      ldb[j] = s;
    }
    __syncthreads();
    for (int e = tid; e < C * C; e += kNT) {
      const int r = e / C, m = e % C;
      ldX[e] = m <= r ? ldX[e] * lbeta[m] : 0.f;
      if (m > r) sdP[e] = 0.f;
    }
    __syncthreads();
    // T = dX X^T;  dA = -X^T T (strictly lower)
    gemm(C, C, C, 1.f, false, ldX, C, 1, X, 1, C, lT, C, 1, stage);
    gemm(C, C, C, -1.f, false, X, 1, C, lT, C, 1, ldA, C, 1, stage);
    // dbeta_r += sum_{j<r} dA_rj G_rj;  dG = Diag(beta) dA
    for (int r = tid; r < C; r += kNT) {
      float s = 0.f;
      for (int j = 0; j < r; ++j) s += ldA[r * C + j] * sG[r * C + j];
      ldb[r] += s;
    }
    __syncthreads();
    for (int e = tid; e < C * C; e += kNT) {
      const int r = e / C, j = e % C;
      ldA[e] = j < r ? ldA[e] * lbeta[r] : 0.f;
    }
    __syncthreads();
    // dQt = scale dO S0^T + dP Rk;  dKt = -T1 S0^T + dG Rk;
    // dRk = dG^T Kt + dP^T Qt + g dKh with dKh = U dS1^T
    // (the start terms scale dO S0^T and -T1 S0^T are also kept, in the
    // slices of V and G, which are no longer read: dalpha needs them apart)
    gemm(C, dk, dv, scale, false, sdO, dv, 1, S0, 1, dv, sdQ, dk, 1, stage);
    gemm(C, dk, dv, -1.f, false, sT1, dv, 1, S0, 1, dv, sdK, dk, 1, stage);
    float* sQ0 = sV;
    float* sK0 = sG;
    for (int e = tid; e < C * dk; e += kNT) {
      sQ0[e] = sdQ[e];
      sK0[e] = sdK[e];
    }
    __syncthreads();
    gemm(C, dk, C, 1.f, true, sdP, C, 1, sRk, dk, 1, sdQ, dk, 1, stage);
    gemm(C, dk, C, 1.f, true, ldA, C, 1, sRk, dk, 1, sdK, dk, 1, stage);
    gemm(C, dk, dv, 1.f, false, sU, dv, 1, dS1, 1, dv, sZ, dk, 1, stage);  // dKh -> Z's slice
    gemm(C, dk, C, 1.f, false, ldA, 1, C, sKt, dk, 1, sdR, dk, 1, stage);
    gemm(C, dk, C, 1.f, true, sdP, 1, C, sQt, dk, 1, sdR, dk, 1, stage);
    // dg = rowsum(dS1 * S0) (TPC threads per channel), the adjoint of the
    // pair (chunk end, chunk start); the end's pairs with the rows (Kh) are
    // counted where dalpha sums pairs
    {
      const int TPC = kNT / dk >= 1 ? kNT / dk : 1, cc = tid / TPC, sub = tid % TPC;
      float sacc = 0.f;
      if (cc < dk) {
        for (int j0 = sub; j0 < dv; j0 += 8 * TPC) {
          float x[8], y[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int j = j0 + u * TPC;
            x[u] = j < dv ? dS1[cc * dv + j] : 0.f;
            y[u] = j < dv ? S0[cc * dv + j] : 0.f;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) sacc += x[u] * y[u];
        }
      }
      for (int o = 1; o < TPC; o <<= 1) sacc += __shfl_xor(sacc, o);
      if (cc < dk && sub == 0) ldg[cc] = sacc;
    }
    __syncthreads();
    // dalpha per channel (one thread each), with no division by a gate: the
    // sum over the pairs (r, j) of positions that straddle s (j < s <= r;
    // chunk rows, start j = -1, end r = C) of the pair's adjoint times
    // D(r<-s) D(s-1<-j), split by 16-row tiles as in the bf16 pass: rows of
    // the tile with columns before it (rho, suffix recurrence), columns of
    // the tile with rows after it (kappa, prefix recurrence), rows after
    // with columns before (Gamma), and the tile's own pairs.  Runs before
    // dk^ and dq^ overwrite nothing it reads (F, Kt, Qt, Rk, the start terms,
    // dKh, dG, dP).
#pragma unroll 1
    for (int cc = tid; cc < dk; cc += kNT) {
      const float gg = lg[cc], gdg = gg * ldg[cc];
      auto at = [&](int r) { return r < L ? alpha[((t0 + r) * H + h) * dk + cc] : 1.f; };
      auto khat = [&](int r) { return r < L ? IO::load(k, ((t0 + r) * H + h) * dk + cc) * lrk[r] : 0.f; };
      auto qhat = [&](int r) { return r < L ? IO::load(q, ((t0 + r) * H + h) * dk + cc) * lrq[r] : 0.f; };
      const int nb = C / 16;
#pragma unroll 1
      for (int tb = 0; tb < nb; ++tb) {
        const int lo = 16 * tb, hi = lo + 16;
        const float Fa = tb == 0 ? 1.f : sF[(lo - 1) * dk + cc], Fe = sF[(hi - 1) * dk + cc];
        // Gamma: rows after the tile and the end, columns before it and the start
        float Z = gdg;
#pragma unroll 1
        for (int j = 0; j < lo; ++j) Z += gg * sZ[j * dk + cc] * sRk[j * dk + cc];
#pragma unroll 1
        for (int r = hi; r < C; ++r) {
          float xk = sK0[r * dk + cc], xq = sQ0[r * dk + cc];
#pragma unroll 1
          for (int j = 0; j < lo; ++j) {
            const float rk = sRk[j * dk + cc];
            xk += ldA[r * C + j] * rk;
            xq += sdP[r * C + j] * rk;
          }
          Z += sKt[r * dk + cc] * xk + sQt[r * dk + cc] * xq;
        }
        const float gam = Z * (Fa / Fe);
        float a[16], kh[16], rho[16], kap[16];
#pragma unroll 1
        for (int i = 0; i < 16; ++i) {
          const int r = lo + i;
          a[i] = at(r);
          kh[i] = khat(r);
          // rho_r: row r with the columns before the tile and the start
          float xk = sK0[r * dk + cc], xq = sQ0[r * dk + cc];
#pragma unroll 1
          for (int j = 0; j < lo; ++j) {
            const float rk = sRk[j * dk + cc];
            xk += ldA[r * C + j] * rk;
            xq += sdP[r * C + j] * rk;
          }
          rho[i] = Fa * (kh[i] * xk + qhat(r) * xq);
          // kappa_r: column r with the rows after the tile and the end
          float y = gg * sZ[r * dk + cc];
#pragma unroll 1
          for (int m = hi; m < C; ++m) y += ldA[m * C + r] * sKt[m * dk + cc] + sdP[m * C + r] * sQt[m * dk + cc];
          kap[i] = kh[i] / Fe * y;
        }
        float sig[16], pi[16], pre[16], suf[16], psi[16];
        sig[15] = rho[15];
#pragma unroll 1
        for (int i = 14; i >= 0; --i) sig[i] = rho[i] + a[i + 1] * sig[i + 1];
        pi[0] = 0.f;
#pragma unroll 1
        for (int i = 1; i < 16; ++i) pi[i] = a[i - 1] * pi[i - 1] + kap[i - 1];
        pre[0] = 1.f;
#pragma unroll 1
        for (int i = 1; i < 16; ++i) pre[i] = pre[i - 1] * a[i - 1];
        suf[15] = 1.f;
#pragma unroll 1
        for (int i = 14; i >= 0; --i) suf[i] = suf[i + 1] * a[i + 1];
#pragma unroll 1
        for (int i = 0; i < 16; ++i) psi[i] = 0.f;
        // the tile's own pairs: Phi_r(s) = sum_{j<s} adj_rj D(s-1<-j) for
        // each row r, then D(r<-s) Phi_r(s) into s
#pragma unroll 1
        for (int ri = 1; ri < 16; ++ri) {
          const int r = lo + ri;
          const float kr = kh[ri], qr = qhat(r);
          float phis[16], phi = 0.f;
#pragma unroll 1
          for (int si = 1; si <= ri; ++si) {
            const int j = si - 1;
            phi = a[j] * phi + (ldA[r * C + lo + j] * kr + sdP[r * C + lo + j] * qr) * kh[j];
            phis[si] = phi;
          }
          float d = 1.f;
#pragma unroll 1
          for (int si = ri; si >= 1; --si) {
            psi[si] += d * phis[si];
            d *= a[si];
          }
        }
#pragma unroll 1
        for (int i = 0; i < 16; ++i) {
          const int r = lo + i;
          if (r < L)
            b.dalpha[((t0 + r) * H + h) * dk + cc] =
                pre[i] * sig[i] + suf[i] * pi[i] + pre[i] * suf[i] * gam + psi[i];
        }
      }
    }
    __syncthreads();  // dalpha has read F, Kt, Qt, Rk
    // elementwise: dk^, dq^ in place
    for (int e0 = tid; e0 < C * dk; e0 += 4 * kNT) {
      float f[4], dqt[4], dkt[4], drk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kNT;
        const bool in = e < C * dk;
        f[u] = in ? sF[e] : 1.f;
        dqt[u] = in ? sdQ[e] : 0.f;
        dkt[u] = in ? sdK[e] : 0.f;
        drk[u] = in ? sdR[e] + lg[e % dk] * sZ[e] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int e = e0 + u * kNT;
        if (e < C * dk) {
          sdK[e] = dkt[u] * f[u] + drk[u] / f[u];
          sdQ[e] = dqt[u] * f[u];
        }
      }
    }
    __syncthreads();
    // dq, dk through the norms (TPR threads per row); dbeta
    {
      const int TPR = kNT / C, r = tid / TPR, sub = tid % TPR;
      const int64_t base = ((t0 + r) * H + h) * dk;
      float pq = 0.f, pk = 0.f;
      if (r < L) {
        for (int c0 = sub; c0 < dk; c0 += 8 * TPR) {
          float xq[8], xk[8], gq[8], gk[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int cc = c0 + u * TPR;
            const bool in = cc < dk;
            xq[u] = in ? IO::load(q, base + cc) : 0.f;
            xk[u] = in ? IO::load(k, base + cc) : 0.f;
            gq[u] = in ? sdQ[r * dk + cc] : 0.f;
            gk[u] = in ? sdK[r * dk + cc] : 0.f;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            pq += xq[u] * gq[u];
            pk += xk[u] * gk[u];
          }
        }
      }
      for (int o = 1; o < TPR; o <<= 1) {
        pq += __shfl_xor(pq, o);
        pk += __shfl_xor(pk, o);
      }
      if (r < L) {
        pq *= lrq[r];
        pk *= lrk[r];
        for (int c0 = sub; c0 < dk; c0 += 8 * TPR) {
          float xq[8], xk[8], gq[8], gk[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int cc = c0 + u * TPR;
            const bool in = cc < dk;
            xq[u] = in ? IO::load(q, base + cc) : 0.f;
            xk[u] = in ? IO::load(k, base + cc) : 0.f;
            gq[u] = in ? sdQ[r * dk + cc] : 0.f;
            gk[u] = in ? sdK[r * dk + cc] : 0.f;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int cc = c0 + u * TPR;
            if (cc < dk) {
              const float qh = xq[u] * lrq[r], kh = xk[u] * lrk[r];
              b.dq[base + cc] = l2 ? lrq[r] * (gq[u] - qh * pq) : gq[u];
              b.dk[base + cc] = l2 ? lrk[r] * (gk[u] - kh * pk) : gk[u];
            }
          }
        }
        if (sub == 0) b.dbeta[(t0 + r) * H + h] = ldb[r];
      }
    }
  }
}

// bits of bf16(x), rounded as the matrix-core operands are
__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

__device__ __forceinline__ bf16x8 to_bf16x8(float4 x, float4 y) {
  bf16x8 r;
  r[0] = static_cast<__bf16>(x.x); r[1] = static_cast<__bf16>(x.y);
  r[2] = static_cast<__bf16>(x.z); r[3] = static_cast<__bf16>(x.w);
  r[4] = static_cast<__bf16>(y.x); r[5] = static_cast<__bf16>(y.y);
  r[6] = static_cast<__bf16>(y.z); r[7] = static_cast<__bf16>(y.w);
  return r;
}

// ---------------------------------------------------------------- 3a: dP, dG
// bf16 inputs: the intra-chunk products up to dP and dG, on the matrix
// cores.  One workgroup per (chunk, head), NW = d / 16 waves (dk = dv = d).
// Wave w owns channel (and value column) 16w + l16 of the lane, rows
// 16t + 4lq + i, for everything that lives along d: q, k, the gate products
// F, Kt, Rk, and the columns of Z and U.  The C x C products (dY, dP, G, T,
// dA) are spread over the waves tile by tile and read their operands from
// LDS as rows:
//   Z  = V - Kt S0           (S0 columns straight from memory)
//   U  = Y Z                 (Y = X Diag(beta) from LDS, Z from registers)
//   dY = dU Z^T,  dP = scale tril(dO U^T),  G = Kt Rk^T
//   dbeta_j = sum_r X_rj dY_rj,  dX = tril(dY) Diag(beta)
//   T  = dX X^T,  dA = -X^T T (strictly lower),  dbeta_r += sum_j dA_rj G_rj
//   dG = Diag(beta) dA
// Out: dbeta and the chunk flag (chunks whose gate products leave
// [2^-100, 2^10] go to the token-level kernel) to memory; dP, dG, their
// transposes, U, dO and the reciprocal row norms left in LDS for the dq/dk
// part.
// The dq/dk part's first loads (its dV rows, the lane's rows of S0 and
// dS1), issued by the dP/dG part during its last products so that they are
// in flight while those run, and the chunk's first token and length (for a
// packed batch, three dependent loads of the chunk map the dq/dk part need
// not repeat).  Rows >= L of dV are read from row L - 1 (no branch around a
// load) and replaced by zeros when they go to LDS.
template <class QC>
struct QLoads {
  static constexpr int PR = QC::DV / 8, NIT = (QC::C * PR + QC::NT - 1) / QC::NT;
  float4 xv[NIT][2];
  uint4 xs[QC::NFV], xd[QC::NFV];
  int64_t t0;
  int L;
};
template <class QC>
__device__ __forceinline__ void issue_qloads(const BwdArgs& b, QLoads<QC>& ql, int64_t t0, int L, int h,
                                             int64_t slot, int tid, int ch, int lq) {
  constexpr int C = QC::C, DK = QC::DK, DV = QC::DV, NT = QC::NT, NFV = QC::NFV;
  constexpr int PR = QLoads<QC>::PR, NIT = QLoads<QC>::NIT;
  const int H = b.f.H;
  ql.t0 = t0;
  ql.L = L;
  const float* dvo = b.dv;
#pragma unroll
  for (int u = 0; u < NIT; ++u) {
    const int p = iclamp(tid + NT * u, C * PR - 1), r = p / PR, cp = p % PR;
    const int64_t row = (t0 + (r < L ? r : L - 1)) * H + h;
    ql.xv[u][0] = *reinterpret_cast<const float4*>(dvo + row * DV + 8 * cp);
    ql.xv[u][1] = *reinterpret_cast<const float4*>(dvo + row * DV + 8 * cp + 4);
  }
  const uint16_t* S0 = static_cast<const uint16_t*>(b.f.hc) + slot * DK * DV + static_cast<int64_t>(ch) * DV + 8 * lq;
  const uint16_t* D1 = static_cast<const uint16_t*>(b.dS) + slot * DK * DV + static_cast<int64_t>(ch) * DV + 8 * lq;
#pragma unroll
  for (int s = 0; s < NFV; ++s) {
    ql.xs[s] = *reinterpret_cast<const uint4*>(S0 + 32 * s);
    ql.xd[s] = *reinterpret_cast<const uint4*>(D1 + 32 * s);
  }
}

template <int C_, int D_>
struct PCfg {
  static constexpr int C = C_, D = D_;
  static constexpr int NW = D / 16, NT = 64 * NW, NB = C / 16, NBC = C / 16;
  static constexpr int LDV = frag_stride(D, 2), LDC = frag_stride(C, 2);
  static constexpr int NFD = D / 32, NFC = (C + 31) / 32;
  static constexpr int NL = NBC * (NBC + 1) / 2;     // tiles on or below the diagonal
  static constexpr int NTL = (NL + NW - 1) / NW;     // ... per wave
  static constexpr int NA = NBC * NBC;               // all tiles
  static constexpr int NTA = (NA + NW - 1) / NW;
  static constexpr int MV = align16(C * LDV * 2), MC = align16(C * LDC * 2);
  // LDS (bytes); dX and T^T reuse the regions of Kt and Rk once G and Z are done
  static constexpr int O_KT = 0, O_RK = MV, O_Z = 2 * MV, O_U = 3 * MV, O_DU = 4 * MV, O_DO = 5 * MV;
  static constexpr int O_DX = O_KT, O_TT = O_RK;
  static constexpr int O_Y = 6 * MV, O_X = O_Y + MC, O_XT = O_X + MC;
  // floats: [2][C] row sums of squares, [NW][2][C] their per-wave parts,
  // [NBC][C] dbeta parts from the dY tiles (by tile row) and [NBC][C] from
  // the dA tiles (by tile column), then the int flag
  static constexpr int O_RED = O_XT + MC;
  static constexpr int NRED = 2 * C + 2 * NW * C + 2 * NBC * C;
  static constexpr int LDS_BYTES = align16(O_RED + (NRED + 4) * 4);
  // Y lower: K fragment s of row tile t is live if it starts at or left of
  // the tile's last row
  static constexpr bool lo_live(int t, int s) { return 32 * s <= 16 * t + 15; }
  // lower tile q -> (tr, tc), row by row
  static constexpr int ltr(int q) { int tr = 0; while ((tr + 1) * (tr + 2) / 2 <= q) ++tr; return tr; }
  static constexpr int ltc(int q) { return q - ltr(q) * (ltr(q) + 1) / 2; }
  static_assert(D % 32 == 0 && C % 16 == 0 && C <= D && MC <= MV, "shapes");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// The dq/dk part follows in the same workgroup, so dP, dG, U and the row
// norms stay in LDS (in the dq/dk part's layout, in regions this part is
// done with) instead of going through memory.  Returns whether the chunk
// goes on to the dq/dk part (false: an unused slot, or left to the
// token-level kernel).
template <class Cfg, class QC>
__device__ __forceinline__ bool dpg_part(const BwdArgs& b, QLoads<QC>& ql) {
  using Op = OpBF16;
  using Frag = Op::Frag;
  constexpr int C = Cfg::C, D = Cfg::D, NB = Cfg::NB, NW = Cfg::NW, NT = Cfg::NT, NBC = Cfg::NBC;
  constexpr int LDV = Cfg::LDV, LDC = Cfg::LDC, NFD = Cfg::NFD, NFC = Cfg::NFC;
  const FwdArgs& a = b.f;
  const int H = a.H;
  const int c = static_cast<int>(blockIdx.x / H), h = static_cast<int>(blockIdx.x % H);
  const int64_t slot = static_cast<int64_t>(h) * a.maxc + c;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, lq = lane >> 4;
  const Geo g = geo_of(a, c);
  if (g.n < 0) {
    if (tid == 0) b.bflag[slot] = 0;
    return false;
  }
  const int64_t t0 = g.t0;
  const int L = g.L;
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* sKT = reinterpret_cast<__bf16*>(smem + Cfg::O_KT);
  __bf16* sRK = reinterpret_cast<__bf16*>(smem + Cfg::O_RK);
  __bf16* sZ = reinterpret_cast<__bf16*>(smem + Cfg::O_Z);
  __bf16* sU = reinterpret_cast<__bf16*>(smem + Cfg::O_U);
  __bf16* sDU = reinterpret_cast<__bf16*>(smem + Cfg::O_DU);
  __bf16* sDO = reinterpret_cast<__bf16*>(smem + Cfg::O_DO);
  __bf16* sDX = reinterpret_cast<__bf16*>(smem + Cfg::O_DX);
  __bf16* sTT = reinterpret_cast<__bf16*>(smem + Cfg::O_TT);
  __bf16* sY = reinterpret_cast<__bf16*>(smem + Cfg::O_Y);
  __bf16* sX = reinterpret_cast<__bf16*>(smem + Cfg::O_X);
  __bf16* sXT = reinterpret_cast<__bf16*>(smem + Cfg::O_XT);
  float* nrm = reinterpret_cast<float*>(smem + Cfg::O_RED);  // [2][C] reciprocal row norms
  float* nrw = nrm + 2 * C;                                    // [NW][2][C]
  float* dbp = nrw + 2 * NW * C;                               // [NBC][C]
  float* dba = dbp + NBC * C;                                  // [NBC][C]
  int* flag = reinterpret_cast<int*>(dba + NBC * C);
  const int ch = 16 * w + l16;  // this lane's channel / value column
  typedef const __attribute__((address_space(1))) uint16_t gu16;
  typedef const __attribute__((address_space(1))) float gf32;
  // dbeta parts of tiles that hold none stay zero; the flag too (nothing
  // reads or adds to them before the norms' first barrier)
  for (int i = tid; i < 2 * NBC * C + 1; i += NT) dbp[i] = 0.f;

  // ---- the loads go out in three batches (rows >= L read from row L - 1,
  // no branch around a load; replaced afterwards): q, k, the dO, dU, X rows
  // and beta first; alpha and v once those rows are in LDS; the S0 columns
  // (first needed for Z) after the norms' first barrier.  All
  // at once they would be more loads than a wave can have in flight, and
  // their issue would stall for a whole memory latency.
  constexpr int PR = D / 8;
  constexpr int NIT = (C * PR + NT - 1) / NT;
  constexpr int NU = (C / 2) * (C / 4);
  constexpr int NUI = (NU + NT - 1) / NT;
  uint16_t xq[NB][4], xk[NB][4], xv[NB][4];
  float xa[NB][4];
  uint16_t xs[NFD][8];
  uint4 xo[NIT];
  float4 xu[NIT];  // 8 bf16 values each
  float4 xx[NUI][2];
  float xb[NUI][4];  // beta of the unit's 4 columns
  {
    gu16* qg = (gu16*)a.q;
    gu16* kg = (gu16*)a.k;
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * t + 4 * lq + i;
        const int64_t row = (t0 + (r < L ? r : L - 1)) * H + h;
        xq[t][i] = qg[row * D + ch];
        xk[t][i] = kg[row * D + ch];
      }
    const uint16_t* o = static_cast<const uint16_t*>(b.dout);
    const uint16_t* dU = static_cast<const uint16_t*>(b.dU) + slot * C * D;
#pragma unroll
    for (int u = 0; u < NIT; ++u) {
      const int p = iclamp(tid + NT * u, C * PR - 1), r = p / PR, cp = p % PR;
      const int64_t row = (t0 + (r < L ? r : L - 1)) * H + h;
      xo[u] = *reinterpret_cast<const uint4*>(o + row * D + 8 * cp);
      xu[u] = *reinterpret_cast<const float4*>(dU + r * D + 8 * cp);
    }
    const float* X = a.xout + slot * C * C;
#pragma unroll
    for (int u = 0; u < NUI; ++u) {
      const int uu = iclamp(tid + NT * u, NU - 1);
      const int r = 2 * (uu % (C / 2)), j0 = 4 * (uu / (C / 2));
      xx[u][0] = *reinterpret_cast<const float4*>(X + r * C + j0);
      xx[u][1] = *reinterpret_cast<const float4*>(X + (r + 1) * C + j0);
    }
    gf32* beta = (gf32*)a.beta;
#pragma unroll
    for (int u = 0; u < NUI; ++u) {
      const int j0 = 4 * (iclamp(tid + NT * u, NU - 1) / (C / 2));
#pragma unroll
      for (int e = 0; e < 4; ++e) xb[u][e] = beta[(t0 + (j0 + e < L ? j0 + e : L - 1)) * H + h];
    }
  }

  // ---- to LDS: dU, dO rows (rows >= L of dO as zeros); X, X^T (natural
  // order) and Y = X Diag(beta) (permuted order)
#pragma unroll
  for (int u = 0; u < NIT; ++u) {
    const int p = tid + NT * u, r = p / PR, cp = p % PR;
    if ((C * PR) % NT == 0 || p < C * PR) {
      uint4 vo = xo[u];
      if (r >= L) vo = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(sDO + r * LDV + 8 * cp) = vo;
      *reinterpret_cast<float4*>(sDU + r * LDV + 8 * cp) = xu[u];
    }
  }
  {
#pragma unroll
    for (int u = 0; u < NUI; ++u) {
      const int uu = tid + NT * u;
      if (NU % NT == 0 || uu < NU) {
        const int r = 2 * (uu % (C / 2)), j0 = 4 * (uu / (C / 2));
        float bj[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) bj[e] = j0 + e < L ? xb[u][e] : 0.f;
        const int qj = Op::pos<C>(j0);
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
          const float4 x = xx[u][rr];
          Op::store4(sX + (r + rr) * LDC + j0, f32x4{x.x, x.y, x.z, x.w});
          Op::store4(sY + (r + rr) * LDC + qj, f32x4{x.x * bj[0], x.y * bj[1], x.z * bj[2], x.w * bj[3]});
        }
        const float4 x0 = xx[u][0], x1 = xx[u][1];
        Op::store2(sXT + (j0 + 0) * LDC + r, x0.x, x1.x);
        Op::store2(sXT + (j0 + 1) * LDC + r, x0.y, x1.y);
        Op::store2(sXT + (j0 + 2) * LDC + r, x0.z, x1.z);
        Op::store2(sXT + (j0 + 3) * LDC + r, x0.w, x1.w);
      }
    }
  }
  {  // the second batch of loads
    gu16* vg = (gu16*)a.v;
    gf32* alpha = (gf32*)a.alpha;
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * t + 4 * lq + i;
        xa[t][i] = alpha[((t0 + (r < L ? r : L - 1)) * H + h) * D + ch];
        xv[t][i] = vg[((t0 + (r < L ? r : L - 1)) * H + h) * D + ch];
      }
  }
  // ---- row norms: sums of squares over the wave's channels by a butterfly
  // (lane l16 ends with value l16 >> (4 - log2 4NB)), then over the waves in
  // wave order (a fixed order: the sums are the same on every run)
  const bool l2 = a.use_l2norm != 0;
  {
    constexpr int NV = 4 * NB, LG = ilog2(NV);
    float vq[NV], vk[NV];
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool in = 16 * t + 4 * lq + i < L;
        const float x = in ? bf16_to_f32(xq[t][i]) : 0.f, y = in ? bf16_to_f32(xk[t][i]) : 0.f;
        vq[4 * t + i] = x * x;
        vk[4 * t + i] = y * y;
      }
    int m = 8;
#pragma unroll
    for (int half = NV / 2; half >= 1; half /= 2) {
      const bool up = (l16 & m) != 0;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const float ql = vq[i] + __shfl_xor(vq[i], m, 64), qu = vq[i + half] + __shfl_xor(vq[i + half], m, 64);
        const float kl = vk[i] + __shfl_xor(vk[i], m, 64), ku = vk[i + half] + __shfl_xor(vk[i + half], m, 64);
        vq[i] = up ? qu : ql;
        vk[i] = up ? ku : kl;
      }
      m >>= 1;
    }
#pragma unroll
    for (int mm = 8 >> LG; mm >= 1; mm >>= 1) {
      vq[0] += __shfl_xor(vq[0], mm, 64);
      vk[0] += __shfl_xor(vk[0], mm, 64);
    }
    const int v = l16 >> (4 - LG), r = 16 * (v >> 2) + 4 * lq + (v & 3);
    if ((l16 & ((1 << (4 - LG)) - 1)) == 0) {
      nrw[(2 * w) * C + r] = vq[0];
      nrw[(2 * w + 1) * C + r] = vk[0];
    }
  }
  __syncthreads();  // LDS operands and the per-wave sums of squares
  {  // the third batch of loads
    gu16* S0 = (gu16*)a.hc + slot * D * D + ch;
#pragma unroll
    for (int s = 0; s < NFD; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[s][e] = S0[(32 * s + 8 * lq + e) * D];
  }

  if (tid < 2 * C) {
    // the reciprocal norm of one row of q or k, once per row
    const int x = tid / C, r = tid % C;
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) sum += nrw[(2 * v + x) * C + r];
    const float rn = l2 ? __fdiv_rn(1.f, __fsqrt_rn(sum + kL2Eps)) : 1.f;
    nrm[tid] = rn;
  }
  __syncthreads();  // the reciprocal norms

  // ---- gate products (scan down the rows as in the dq/dk pass);
  // regularity; Kt, Rk to LDS rows; Z starts as V
  f32x4 rkv[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) rkv[t] = *reinterpret_cast<const f32x4*>(nrm + C + 16 * t + 4 * lq);
  f32x4 zacc[NB];
  {
    bool ok = true;
    float carry = 1.f;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) al[i] = 16 * t + 4 * lq + i < L ? xa[t][i] : 1.f;
      float loc[4];
      loc[0] = al[0];
      loc[1] = loc[0] * al[1];
      loc[2] = loc[1] * al[2];
      loc[3] = loc[2] * al[3];
      float inc = loc[3];
      float y = __shfl_up(inc, 16);
      if (lq >= 1) inc *= y;
      y = __shfl_up(inc, 32);
      if (lq >= 2) inc *= y;
      float exc = __shfl_up(inc, 16);
      if (lq == 0) exc = 1.f;
      const float tot = __shfl(inc, 48 + l16);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * t + 4 * lq + i;
        const bool in = r < L;
        const float f = carry * exc * loc[i], mf = fabsf(f);
        ok = ok && mf >= kRegMin && mf <= kRegMax;
        const float kh = in ? bf16_to_f32(xk[t][i]) * rkv[t][i] : 0.f;
        sKT[r * LDV + ch] = static_cast<__bf16>(kh * f);
        sRK[r * LDV + ch] = static_cast<__bf16>(kh * __builtin_amdgcn_rcpf(f));  // f in range below
        zacc[t][i] = in ? bf16_to_f32(xv[t][i]) : 0.f;
      }
      carry *= tot;
    }
    if (!ok) *flag = 1;
  }
  __syncthreads();  // Kt, Rk rows; the flag
  if (*flag != 0) {
    if (tid == 0) b.bflag[slot] = 1;
    return false;
  }
  if (tid == 0) b.bflag[slot] = 0;

  // ---- Z = V - Kt S0 (S0 columns negated: the bf16 sign bit flipped), U = Y Z
  {
    Frag sf[NFD];
#pragma unroll
    for (int s = 0; s < NFD; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) sf[s][e] = __builtin_bit_cast(__bf16, static_cast<uint16_t>(xs[s][e] ^ 0x8000u));
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int s = 0; s < NFD; ++s)
        Op::mma(zacc[t], *reinterpret_cast<const bf16x8*>(sKT + (16 * t + l16) * LDV + 32 * s + 8 * lq), sf[s]);
  }
  f32x4 uacc[NB];
  {
    Frag zf[NFC];
    Op::frags<C>(zf, zacc);
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      uacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NFC; ++s)
        if (Cfg::lo_live(t, s)) Op::mma(uacc[t], Op::row_frag<C>(sY + (16 * t + l16) * LDC, s, lq), zf[s]);
    }
  }
  // Z and U to LDS rows (bf16)
  {
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * t + 4 * lq + i;
        sZ[r * LDV + ch] = static_cast<__bf16>(zacc[t][i]);
        sU[r * LDV + ch] = static_cast<__bf16>(uacc[t][i]);
      }
  }
  // G = Kt Rk^T on this wave's lower tiles (kept for dbeta)
  f32x4 gacc[Cfg::NTL];
#pragma unroll
  for (int k = 0; k < Cfg::NTL; ++k) {
    const int q = w + NW * k;
    gacc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (q < Cfg::NL) {
      const int tr = Cfg::ltr(q), tc = Cfg::ltc(q);
      Op::mmaK<D>(gacc[k], sKT + 16 * tr * LDV, LDV, sRK + 16 * tc * LDV, LDV, lane);
    }
  }
  __syncthreads();  // Z, U rows; Kt and Rk no longer read

  // ---- dY, dP on the lower tiles; dbeta (Y part); dX to LDS rows
  const float scale = a.scale;
  gf32* Xg = (gf32*)(a.xout + slot * C * C);
  const float* beta = static_cast<const float*>(a.beta);
  float dpk[Cfg::NTL][4], dgk[Cfg::NTL][4];  // this wave's dP, dG tiles, to LDS at the end
#pragma unroll
  for (int k = 0; k < Cfg::NTL; ++k) {
    const int q = w + NW * k;
    if (q < Cfg::NL) {
      const int tr = Cfg::ltr(q), tc = Cfg::ltc(q);
      f32x4 dy = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
      Op::mmaK<D>(dy, sDU + 16 * tr * LDV, LDV, sZ + 16 * tc * LDV, LDV, lane);
      Op::mmaK<D>(dp, sDO + 16 * tr * LDV, LDV, sU + 16 * tc * LDV, LDV, lane);
      const int j = 16 * tc + l16;
      const float bj = beta[(t0 + (j < L ? j : L - 1)) * H + h];
      float xr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) xr[i] = Xg[(16 * tr + 4 * lq + i) * C + j];
      float colsum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * tr + 4 * lq + i;
        const bool low = j <= r;
        colsum += xr[i] * dy[i];
        dpk[k][i] = low ? scale * dp[i] : 0.f;
        sDX[r * LDC + j] = static_cast<__bf16>(low && j < L ? dy[i] * bj : 0.f);
      }
      colsum += __shfl_xor(colsum, 16);
      colsum += __shfl_xor(colsum, 32);
      if (lq == 0) dbp[tr * C + j] = colsum;
    }
  }
  // the upper tiles of dX: zero
  for (int e = tid; e < C * C; e += NT) {
    const int r = e / C, j = e % C;
    if (j / 16 > r / 16) sDX[r * LDC + j] = static_cast<__bf16>(0.f);
  }
  __syncthreads();  // dX rows

  // ---- T = dX X^T on all tiles, to LDS as T^T rows
#pragma unroll
  for (int k = 0; k < Cfg::NTA; ++k) {
    const int q = w + NW * k;
    if (q < Cfg::NA) {
      const int tr = q / NBC, tc = q % NBC;
      f32x4 tacc = {0.f, 0.f, 0.f, 0.f};
      Op::mmaK<C>(tacc, sDX + 16 * tr * LDC, LDC, sX + 16 * tc * LDC, LDC, lane);
      // T[m][j] (m = 16tr + 4lq + i, j = 16tc + l16) -> T^T[j][m .. m+3]
      Op::store4(sTT + (16 * tc + l16) * LDC + 16 * tr + 4 * lq, tacc);
    }
  }
  __syncthreads();  // T^T rows
  issue_qloads<QC>(b, ql, t0, L, h, slot, tid, ch, lq);  // for the dq/dk part

  // ---- dA = -X^T T on the lower tiles (strictly lower); dbeta (A part); dG
#pragma unroll
  for (int k = 0; k < Cfg::NTL; ++k) {
    const int q = w + NW * k;
    if (q < Cfg::NL) {
      const int tr = Cfg::ltr(q), tc = Cfg::ltc(q);
      f32x4 da = {0.f, 0.f, 0.f, 0.f};
      Op::mmaK<C>(da, sXT + 16 * tr * LDC, LDC, sTT + 16 * tc * LDC, LDC, lane);
      const int j = 16 * tc + l16;
      float rs[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * tr + 4 * lq + i;
        const float v = j < r ? -da[i] : 0.f;
        rs[i] = v * gacc[k][i];
        const float br = beta[(t0 + (r < L ? r : L - 1)) * H + h];
        dgk[k][i] = r < L ? v * br : 0.f;
      }
#pragma unroll
      for (int o = 1; o < 16; o <<= 1)
#pragma unroll
        for (int i = 0; i < 4; ++i) rs[i] += __shfl_xor(rs[i], o, 64);
      if (l16 == 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) dba[tc * C + 16 * tr + 4 * lq + i] = rs[i];
    }
  }
  __syncthreads();  // dbeta parts
  if (tid < L) {
    // the tiles' parts in a fixed order
    float db = 0.f;
#pragma unroll
    for (int u = 0; u < NBC; ++u) db += dbp[u * C + tid];
#pragma unroll
    for (int u = 0; u < NBC; ++u) db += dba[u * C + tid];
    b.dbeta[(t0 + tid) * H + h] = db;
  }
  {
    // dP and dG for the dq/dk part, as rows (permuted column order) and as
    // transposed rows, in the regions of Y, X, X^T and dU (none read any
    // more): the lower tiles from this wave's registers, zeros elsewhere
    uint16_t* hP = reinterpret_cast<uint16_t*>(smem + Cfg::O_Y);
    uint16_t* hPT = reinterpret_cast<uint16_t*>(smem + Cfg::O_X);
    uint16_t* hG = reinterpret_cast<uint16_t*>(smem + Cfg::O_XT);
    uint16_t* hGT = reinterpret_cast<uint16_t*>(smem + Cfg::O_DU);
#pragma unroll
    for (int k = 0; k < Cfg::NTL; ++k) {
      const int q = w + NW * k;
      if (q < Cfg::NL) {
        const int tr = Cfg::ltr(q), tc = Cfg::ltc(q);
        const int j = 16 * tc + l16, qj = Op::pos<C>(j), qr = Op::pos<C>(16 * tr + 4 * lq);
        uint16_t pb[4], gb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * tr + 4 * lq + i;
          pb[i] = bf16_bits(dpk[k][i]);
          gb[i] = bf16_bits(dgk[k][i]);
          hP[r * LDC + qj] = pb[i];
          hG[r * LDC + qj] = gb[i];
        }
        // rows 16tr + 4lq .. + 3 are adjacent in the permuted order
        *reinterpret_cast<uint2*>(hPT + j * LDC + qr) =
            make_uint2(pb[0] | (static_cast<uint32_t>(pb[1]) << 16), pb[2] | (static_cast<uint32_t>(pb[3]) << 16));
        *reinterpret_cast<uint2*>(hGT + j * LDC + qr) =
            make_uint2(gb[0] | (static_cast<uint32_t>(gb[1]) << 16), gb[2] | (static_cast<uint32_t>(gb[3]) << 16));
      }
    }
    for (int e = tid; e < C * C; e += NT) {
      const int r = e / C, j = e % C;
      if (j / 16 > r / 16) {  // above the diagonal tiles: zero, and below them in the transposes
        hP[r * LDC + Op::pos<C>(j)] = 0;
        hG[r * LDC + Op::pos<C>(j)] = 0;
        hPT[j * LDC + Op::pos<C>(r)] = 0;
        hGT[j * LDC + Op::pos<C>(r)] = 0;
      }
    }
  }
  return true;
}

// ---------------------------------------------------------------- 3b: dq, dk
// bf16 inputs: dq, dk and dalpha of the chunks the dP/dG part kept, on the
// matrix cores, in the same workgroup right after it.  Wave w owns the 16
// channels 16w .. 16w + 15, and lane (l16, lq) holds rows 16t + 4lq + i of
// channel 16w + l16 (the layout of an MFMA result tile), so every
// per-channel quantity (the gate products F, Kt, Qt, Rk, the reverse sums of
// dalpha) stays in one wave's registers.  The products
//   dQt = scale dO S0^T + dP Rk       dKt = -dV S0^T + dG Rk
//   dKh = U dS1^T                     dRk = dG^T Kt + dP^T Qt
// read the chunk-wide operands (dO, dV, U over dv; dP, dG and their
// transposes over the chunk rows) from LDS as row fragments, and the
// per-channel ones from registers: the lane's rows of S0 and dS1 straight
// from memory, Rk, Kt and Qt from its own tiles in the permuted order.
// The four products over the chunk rows carry the pair terms that cancel in
// the reverse sums of dalpha (a pair (r, j) inside [s, C) enters Lam at r
// and at j with opposite signs, through dG Rk at r and dG^T Kt at j, or dP Rk
// and dP^T Qt).  Both products of a pair read the same bf16 dG_rj (dP_rj),
// and the register operands run in split bf16, x = hi + lo with hi = bf16(x)
// and lo = bf16(x - hi), so each pair term is formed to about 16 significant
// bits on both sides and the cancellation holds to that precision.
template <int C_, int DK_>
struct QCfg {
  static constexpr int C = C_, DK = DK_, DV = DK_;
  static constexpr int NW = DK / 16, NT = 64 * NW, NB = C / 16;
  static constexpr int LDV = frag_stride(DV, 2), LDC = frag_stride(C, 2);
  static constexpr int NFV = DV / 32, NFC = (C + 31) / 32;
  // dP, dG lower: K fragment s of row tile t is live if it starts at or left
  // of the tile's last row; their transposes are upper
  static constexpr bool lo_live(int t, int s) { return 32 * s <= 16 * t + 15; }
  static constexpr bool up_live(int t, int s) { return 32 * s + 31 >= 16 * t; }
  static_assert(DV % 32 == 0 && C % 16 == 0, "shapes");
};

// Where the dq/dk part finds its LDS operands, in the dP/dG part's regions:
// dO and U are already there, dP, dG and their transposes were written by
// that part, the row norms are its reciprocal norms; dV, the reductions and
// dalpha's transposes go where nothing is read any more.
template <class QC, class PC>
struct QMap {
  static constexpr int DO = PC::O_DO;
  static constexpr int DV = PC::O_Z;
  static constexpr int U = PC::O_U;
  static constexpr int P = PC::O_Y;
  static constexpr int PT = PC::O_X;
  static constexpr int G = PC::O_XT;
  static constexpr int GT = PC::O_DU;
  static constexpr int RN = PC::O_RED;  // the reciprocal row norms [2][C]
  static constexpr int RED = align16(PC::LDS_BYTES);
  // dalpha's transposes: after the products over dv, over the Kt, Rk (dX,
  // T^T) and dV rows
  static constexpr int TB = PC::O_KT;
  static constexpr int TB_END = PC::O_U;
  static constexpr int LDS_BYTES = align16(RED + 2 * (QC::NW + 1) * QC::C * 4);
  static_assert(QC::LDV == PC::LDV && QC::LDC == PC::LDC && QC::NT == PC::NT, "shared strides");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

template <class Cfg, class PC>
__device__ __forceinline__ void dqk_part(const BwdArgs& b, const QLoads<Cfg>& ql) {
  using Op = OpBF16;
  using Frag = Op::Frag;
  using M = QMap<Cfg, PC>;
  constexpr int C = Cfg::C, DK = Cfg::DK, DV = Cfg::DV, NB = Cfg::NB, NW = Cfg::NW, NT = Cfg::NT;
  constexpr int LDV = Cfg::LDV, LDC = Cfg::LDC, NFV = Cfg::NFV;
  const FwdArgs& a = b.f;
  const int H = a.H;
  const int c = static_cast<int>(blockIdx.x / H), h = static_cast<int>(blockIdx.x % H);
  // a used slot, not flagged (the dP/dG part returned true)
  const int64_t slot = static_cast<int64_t>(h) * a.maxc + c;
  const int64_t t0 = ql.t0;
  const int L = ql.L;
  extern __shared__ __align__(16) unsigned char smem[];
  __bf16* sdO = reinterpret_cast<__bf16*>(smem + M::DO);
  __bf16* sdV = reinterpret_cast<__bf16*>(smem + M::DV);
  __bf16* sU = reinterpret_cast<__bf16*>(smem + M::U);
  __bf16* sP = reinterpret_cast<__bf16*>(smem + M::P);
  __bf16* sPT = reinterpret_cast<__bf16*>(smem + M::PT);
  __bf16* sG = reinterpret_cast<__bf16*>(smem + M::G);
  __bf16* sGT = reinterpret_cast<__bf16*>(smem + M::GT);
  float* red = reinterpret_cast<float*>(smem + M::RED);
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l16 = lane & 15, lq = lane >> 4;
  const int ch = 16 * w + l16;  // this lane's channel
  // global address space (plain global loads rather than flat ones)
  typedef const __attribute__((address_space(1))) uint16_t gu16;
  typedef const __attribute__((address_space(1))) float gf32;

  // ---- the loads this part adds to the dP/dG part's LDS operands (dV
  // rows, the lane's rows of S0 and dS1) were issued by that part
  constexpr int PR = QLoads<Cfg>::PR;              // 8-element pieces per row of dv
  constexpr int NIT = QLoads<Cfg>::NIT;            // pieces per thread
  const auto& xv = ql.xv;
  const auto& xs = ql.xs;
  const auto& xd = ql.xd;
  // dV to LDS as bf16 (rows >= L as zeros)
#pragma unroll
  for (int u = 0; u < NIT; ++u) {
    const int p = tid + NT * u, r = p / PR, cp = p % PR;
    if ((C * PR) % NT == 0 || p < C * PR) {
      const bool in = r < L;
      const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<bf16x8*>(sdV + r * LDV + 8 * cp) = to_bf16x8(in ? xv[u][0] : z, in ? xv[u][1] : z);
    }
  }
  // the lane's rows of S0 and dS1 as fragments over dv (natural order, as
  // the LDS rows), and their row dot product
  Frag s0f[NFV], d1f[NFV];
  float dg = 0.f;
#pragma unroll
  for (int s = 0; s < NFV; ++s) {
    const uint32_t xw[4] = {xs[s].x, xs[s].y, xs[s].z, xs[s].w}, yw[4] = {xd[s].x, xd[s].y, xd[s].z, xd[s].w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      dg += __uint_as_float(xw[e] << 16) * __uint_as_float(yw[e] << 16) +
            __uint_as_float(xw[e] & 0xFFFF0000u) * __uint_as_float(yw[e] & 0xFFFF0000u);
    s0f[s] = __builtin_bit_cast(bf16x8, xs[s]);
    d1f[s] = __builtin_bit_cast(bf16x8, xd[s]);
  }
  // the lane's q, k, alpha (in flight over the barrier and the first products)
  const float* rn = reinterpret_cast<const float*>(smem + M::RN);
  float xa[NB][4];
  uint16_t xq[NB][4], xk[NB][4];
  f32x4 nq[NB], nk[NB];
  {
    gu16* qg = (gu16*)a.q;
    gu16* kg = (gu16*)a.k;
    gf32* alpha = (gf32*)a.alpha;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      nq[t] = *reinterpret_cast<const f32x4*>(rn + 16 * t + 4 * lq);
      nk[t] = *reinterpret_cast<const f32x4*>(rn + C + 16 * t + 4 * lq);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * t + 4 * lq + i;
        const int64_t e = ((t0 + (r < L ? r : L - 1)) * H + h) * DK + ch;
        xa[t][i] = alpha[e];
        xq[t][i] = qg[e];
        xk[t][i] = kg[e];
      }
    }
  }
  __syncthreads();  // LDS operands ready

  const float scale = a.scale;
  // ---- products over dv
  f32x4 dKh[NB], dQt[NB], dKt[NB], dRk[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const int ro = 16 * t + l16;
    dKh[t] = dQt[t] = dKt[t] = dRk[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NFV; ++s) {
      const int o = ro * LDV + 32 * s + 8 * lq;
      Op::mma(dKh[t], *reinterpret_cast<const bf16x8*>(sU + o), d1f[s]);
      Op::mma(dQt[t], *reinterpret_cast<const bf16x8*>(sdO + o), s0f[s]);
      Op::mma(dKt[t], *reinterpret_cast<const bf16x8*>(sdV + o), s0f[s]);
    }
    dQt[t] *= scale;
    dKt[t] = -dKt[t];
  }

  // ---- normalised q, k; the gate products F, a scan down the rows: within
  // the lane's 4 rows, across the 4 lane groups of the tile, tile to tile
  f32x4 qh[NB], kh[NB], F[NB];
  {
    float carry = 1.f;
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      float al[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool in = 16 * t + 4 * lq + i < L;
        al[i] = in ? xa[t][i] : 1.f;
        qh[t][i] = in ? bf16_to_f32(xq[t][i]) * nq[t][i] : 0.f;
        kh[t][i] = in ? bf16_to_f32(xk[t][i]) * nk[t][i] : 0.f;
      }
      float loc[4];
      loc[0] = al[0];
      loc[1] = loc[0] * al[1];
      loc[2] = loc[1] * al[2];
      loc[3] = loc[2] * al[3];
      float inc = loc[3];
      float y = __shfl_up(inc, 16);
      if (lq >= 1) inc *= y;
      y = __shfl_up(inc, 32);
      if (lq >= 2) inc *= y;
      float exc = __shfl_up(inc, 16);
      if (lq == 0) exc = 1.f;
      const float tot = __shfl(inc, 48 + l16);
#pragma unroll
      for (int i = 0; i < 4; ++i) F[t][i] = carry * exc * loc[i];
      carry *= tot;
    }
  }
  const float gch = __shfl(F[NB - 1][3], 48 + l16);  // the chunk's total product, row C - 1

  // ---- products over the chunk rows, one MFMA per (row tile, column tile).
  // The register operand of column tile u holds only that tile's rows (its
  // half of the 32-wide K slice, the other half zero), so the accumulators
  // can be read at every tile boundary: dalpha needs the partial sums over
  // the columns before each tile (see the dalpha block below).
  auto tile_frag = [](const f32x4& x, int u) {
    Frag f;
    const bool hi = (u & 1) != 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = static_cast<__bf16>(hi ? 0.f : x[i]);
      f[4 + i] = static_cast<__bf16>(hi ? x[i] : 0.f);
    }
    return f;
  };
  // the chunk-anchored operands, formed where they are used
  auto Kt = [&](int t) { return kh[t] * F[t]; };
  auto Qt = [&](int t) { return qh[t] * F[t]; };
  auto Rk = [&](int t) {
    f32x4 x;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = kh[t][i] * __builtin_amdgcn_rcpf(F[t][i]);
    return x;
  };
  // F at the last row of each tile (e_t) and at the row before it (a_t)
  float Fe[NB], Fa[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    Fe[t] = __shfl(F[t][3], 48 + l16);
    Fa[t] = t == 0 ? 1.f : Fe[t - 1];
  }
  // rows: dKt += dG Rk, dQt += dP Rk over column tiles u <= t.  Before column
  // tile u the accumulators hold the pair terms of the row with the columns
  // before u (and the chunk start); for u < t their sum over the tile's rows
  // goes to the corner of tile u (zp), for u = t it is rho.
  f32x4 rho[NB];
  float zp[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) zp[t] = 0.f;
  {
    Frag rkm[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) rkm[u] = tile_frag(Rk(u), u);
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const int ro = (16 * t + l16) * LDC;
#pragma unroll
      for (int sl = 0; sl <= t / 2; ++sl) {
        const Frag gA = Op::row_frag<C>(sG + ro, sl, lq), pA = Op::row_frag<C>(sP + ro, sl, lq);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int u = 2 * sl + hh;
          if (u > t) continue;
          if (u < t) {
            const f32x4 kt = Kt(t), qt = Qt(t);
            float x = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) x += kt[i] * dKt[t][i] + qt[i] * dQt[t][i];
            zp[u] += x;
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) rho[t][i] = Fa[t] * (kh[t][i] * dKt[t][i] + qh[t][i] * dQt[t][i]);
          }
          Op::mma(dKt[t], gA, rkm[u]);
          Op::mma(dQt[t], pA, rkm[u]);
        }
      }
    }
  }
  // columns: dRk = g dKh + dG^T Kt + dP^T Qt over row tiles u >= t, last
  // first.  Before row tile t the accumulator holds the pair terms of the
  // column with the rows after its tile (and the chunk end): kappa.
  f32x4 kap[NB];
  {
    Frag ktm[NB], qtm[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      ktm[u] = tile_frag(Kt(u), u);
      qtm[u] = tile_frag(Qt(u), u);
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      const int ro = (16 * t + l16) * LDC;
      dRk[t] = gch * dKh[t];
#pragma unroll
      for (int sl = (NB - 1) / 2; sl >= t / 2; --sl) {
        const Frag gA = Op::row_frag<C>(sGT + ro, sl, lq), pA = Op::row_frag<C>(sPT + ro, sl, lq);
#pragma unroll
        for (int hh = 1; hh >= 0; --hh) {
          const int u = 2 * sl + hh;
          if (u < t || u >= NB) continue;
          if (u == t) {
            const float re = __builtin_amdgcn_rcpf(Fe[t]);
#pragma unroll
            for (int i = 0; i < 4; ++i) kap[t][i] = kh[t][i] * re * dRk[t][i];
          }
          Op::mma(dRk[t], gA, ktm[u]);
          Op::mma(dRk[t], pA, qtm[u]);
        }
      }
    }
  }

  // ---- per element
  f32x4 dqh[NB], dkh[NB];
  float ep[NB];  // the chunk end's pair terms with this lane's rows, per tile
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    ep[t] = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f = F[t][i], rf = __builtin_amdgcn_rcpf(f);  // F in [2^-100, 2^10]
      dkh[t][i] = dKt[t][i] * f + dRk[t][i] * rf;
      dqh[t][i] = dQt[t][i] * f;
      ep[t] += gch * dKh[t][i] * (kh[t][i] * rf);
    }
  }
  // over the four lane groups (the tile's 16 rows): the chunk end's pair with
  // the chunk start (dg), the corner sums and the end pairs per tile
  dg += __shfl_xor(dg, 16);
  dg += __shfl_xor(dg, 32);
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    zp[t] += __shfl_xor(zp[t], 16);
    zp[t] += __shfl_xor(zp[t], 32);
    ep[t] += __shfl_xor(ep[t], 16);
    ep[t] += __shfl_xor(ep[t], 32);
  }

  // outputs through buffer stores whose range ends at row L: the stores of
  // rows >= L are dropped by the range check, with no branch around them
  const int64_t obase = (t0 * H + h) * DK;
  const int orange = L * H * DK * 4;
  const int ooff = (4 * lq * H * DK + ch) * 4;  // row 4lq, this lane's channel (bytes)
  auto ostore = [&](float* out, int t, int i, float x) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), make_rsrc(out + obase, orange),
                                          ooff + (16 * t + i) * H * DK * 4, 0, 0);
  };

  // ---- through the norms: row sums q^ . dq^ and k^ . dk^ over the
  // channels.  Over the wave's 16 lanes by a butterfly that halves the
  // values per step (lane l16 ends with value l16 >> (4 - log2 4NB)), then
  // over the waves in LDS, one thread per (row, q or k), read back by rows.
  const bool l2 = a.use_l2norm != 0;
  {
    constexpr int NV = 4 * NB, LG = ilog2(NV);
    float vq[NV], vk[NV];
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vq[4 * t + i] = qh[t][i] * dqh[t][i];
        vk[4 * t + i] = kh[t][i] * dkh[t][i];
      }
    int m = 8;
#pragma unroll
    for (int half = NV / 2; half >= 1; half /= 2) {
      const bool up = (l16 & m) != 0;
#pragma unroll
      for (int i = 0; i < half; ++i) {
        const float ql = vq[i] + __shfl_xor(vq[i], m, 64), qu = vq[i + half] + __shfl_xor(vq[i + half], m, 64);
        const float kl = vk[i] + __shfl_xor(vk[i], m, 64), ku = vk[i + half] + __shfl_xor(vk[i + half], m, 64);
        vq[i] = up ? qu : ql;
        vk[i] = up ? ku : kl;
      }
      m >>= 1;
    }
#pragma unroll
    for (int mm = 8 >> LG; mm >= 1; mm >>= 1) {
      vq[0] += __shfl_xor(vq[0], mm, 64);
      vk[0] += __shfl_xor(vk[0], mm, 64);
    }
    const int v = l16 >> (4 - LG), r = 16 * (v >> 2) + 4 * lq + (v & 3);
    if ((l16 & ((1 << (4 - LG)) - 1)) == 0) {
      red[w * C + r] = vq[0];
      red[(NW + w) * C + r] = vk[0];
    }
  }
  __syncthreads();
  float* fin = red + 2 * NW * C;  // [2][C]
  if (tid < 2 * C) {
    const int x = tid / C, r = tid % C;
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) sum += red[(x * NW + v) * C + r];
    fin[tid] = sum;
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const f32x4 pq = *reinterpret_cast<const f32x4*>(fin + 16 * t + 4 * lq);
    // the row scales, read again here rather than held through the products
    const f32x4 rq4 = *reinterpret_cast<const f32x4*>(rn + 16 * t + 4 * lq);
    const f32x4 rk4 = *reinterpret_cast<const f32x4*>(rn + C + 16 * t + 4 * lq);
    const f32x4 pk = *reinterpret_cast<const f32x4*>(fin + C + 16 * t + 4 * lq);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ostore(b.dq, t, i, l2 ? rq4[i] * (dqh[t][i] - qh[t][i] * pq[i]) : dqh[t][i]);
      ostore(b.dk, t, i, l2 ? rk4[i] * (dkh[t][i] - kh[t][i] * pk[i]) : dkh[t][i]);
    }
  }
  // ---- dalpha, with no division by a gate.  dL/dalpha_s sums, over the
  // pairs (r, j) of positions with j < s <= r (rows of the chunk, its start
  // and its end), the pair's adjoint times D(r<-s) D(s-1<-j), the partial
  // gate products on either side of s.  For s in tile b (a_b, e_b the rows
  // before and at its ends), split by where r and j lie:
  //   r in b, j before b:      Pre_s * sum_{r>=s in b} D(r<-s) rho_r
  //   r after b, j in b:       Suf_s * sum_{j<s in b} D(s-1<-j) kappa_j
  //   r after b, j before b:   Pre_s * Suf_s * Gamma_b
  //   both in b:               Psi_s, pairwise (below)
  // Pre_s = D(s-1<-a_b), Suf_s = D(e_b<-s) are products inside the tile;
  // rho, kappa and Gamma_b are the pair terms anchored at the tile's edges,
  // formed above from the chunk-anchored operands (ratios of running
  // products within [2^-100, 2^10], so bounded and accurate).  The sums run
  // down the rows of a tile, so each tile goes to one lane: through a
  // per-wave LDS buffer (in the dO, dV, U rows, which no wave reads any
  // more), lane (l16, lq) takes the 16 rows of tile lq of its channel.  All
  // lanes of the wave then take the same row at the same step: the pairwise
  // loop runs the 120 (r, j) pairs of a tile with no masked steps, and the
  // recurrences need no carries between lanes.
  {
    constexpr int LDT = C + 4;  // floats per channel in the buffer (a 16-byte pad)
    static_assert(NW * 16 * LDT * 4 <= M::TB_END - M::TB, "transpose buffer");
    float* tbuf = reinterpret_cast<float*>(smem + M::TB) + w * 16 * LDT;
    const bool own = lq < NB;  // with fewer than 4 tiles the other lane groups only help move data
    const int T = own ? lq : 0;
    // rows 16t + 4lq + i held by lane (l16, lq) -> rows 16T + m of this lane
    auto to_tile = [&](const f32x4(&x)[NB], float(&y)[16]) {
      wave_lds_sync();  // this wave's earlier reads of the buffer are done
#pragma unroll
      for (int t = 0; t < NB; ++t) *reinterpret_cast<f32x4*>(tbuf + l16 * LDT + 16 * t + 4 * lq) = x[t];
      wave_lds_sync();
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(tbuf + l16 * LDT + 16 * T + 4 * g4);
#pragma unroll
        for (int i = 0; i < 4; ++i) y[4 * g4 + i] = v[i];
      }
    };
    // Gamma of this lane's tile: the end's pair with the start (adjoint dg,
    // D = g), the end's pairs with the columns before the tile and the
    // tile's corner, moved to the tile's edges
    float gam = 0.f;
    {
      const float gdg = gch * dg;
      float ecum = 0.f;
#pragma unroll
      for (int tb = 0; tb < NB; ++tb) {
        const float gt = (gdg + ecum + zp[tb]) * (Fa[tb] * __builtin_amdgcn_rcpf(Fe[tb]));
        ecum += ep[tb];
        gam = tb == T ? gt : gam;
      }
    }
    float al[16], kt[16], qt[16];  // the tile's gates (1 past the chunk), k^, q^
    {
      f32x4 alx[NB];
#pragma unroll
      for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) alx[t][i] = 16 * t + 4 * lq + i < L ? xa[t][i] : 1.f;
      to_tile(alx, al);
    }
    to_tile(kh, kt);
    to_tile(qh, qt);
    float suf[16];  // Suf_m: the tile's gates after row m
    suf[15] = 1.f;
#pragma unroll
    for (int m = 14; m >= 0; --m) suf[m] = suf[m + 1] * al[m + 1];
    // pairs inside the tile.  With Suf_r = D(e_b<-r), D(r<-s) = Suf_s / Suf_r
    // (a ratio of gates after s), so for each row r one pass
    //   phi = alpha_j phi + adj_rj / Suf_r  (j < r),  ps_{j+1} += phi
    // over its columns leaves Psi_s = Suf_s * ps_s, ps_s summed over the rows
    // r >= s.  adj_rj = (dG_rj k^_r + dP_rj q^_r) k^_j.
    float ps[16];
#pragma unroll
    for (int m = 0; m < 16; ++m) ps[m] = 0.f;
    {
      // columns 4 q2 .. 4 q2 + 3 of tile T sit together in the storage order
      const int tcol = C % 32 == 0 ? 32 * (T >> 1) + 4 * (T & 1) : 0;
#pragma unroll
      for (int r = 1; r < 16; ++r) {
        const __bf16* gr = sG + (16 * T + r) * LDC + tcol;
        const __bf16* pr = sP + (16 * T + r) * LDC + tcol;
        const float is = __builtin_amdgcn_rcpf(suf[r]);  // suf in [2^-110, 1]: a normal float
        const float kr = kt[r] * is, qr = qt[r] * is;
        float phi = 0.f;
#pragma unroll
        for (int q2 = 0; 4 * q2 < r; ++q2) {
          const bf16x4 g4 = *reinterpret_cast<const bf16x4*>(gr + (C % 32 == 0 ? 8 : 4) * q2);
          const bf16x4 p4 = *reinterpret_cast<const bf16x4*>(pr + (C % 32 == 0 ? 8 : 4) * q2);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int j = 4 * q2 + e;
            if (j < r) {
              phi = al[j] * phi + (static_cast<float>(g4[e]) * kr + static_cast<float>(p4[e]) * qr) * kt[j];
              ps[j + 1] += phi;
            }
          }
        }
      }
    }
    // sigma_m = rho_m + alpha_{m+1} sigma_{m+1} from the bottom (into rt),
    // then down the rows with Pre (running) and pi_{m+1} = alpha_m pi_m +
    // kappa_m:  dalpha_m = Pre_m sigma_m + Suf_m (pi_m + Pre_m Gamma + ps_m)
    float rt[16];
    to_tile(rho, rt);
#pragma unroll
    for (int m = 14; m >= 0; --m) rt[m] += al[m + 1] * rt[m + 1];
    to_tile(kap, kt);  // k^ is no longer needed: kappa in its place
    float pre = 1.f, pi = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const float x = pre * rt[m] + suf[m] * (pi + pre * gam + ps[m]);
      // rows >= L fall outside the buffer range and are dropped; the
      // descriptor is formed here from uniform values, so that it stays in
      // scalar registers
      if (own)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), make_rsrc(b.dalpha + obase, orange),
                                              ((16 * T + m) * H * DK + ch) * 4, 0, 0);
      pi = al[m] * pi + kt[m];
      pre *= al[m];
    }
  }
}

// Both chunk passes in one workgroup per (chunk, head): the dP/dG part,
// then (unless the chunk is left to the token-level kernel) the dq/dk part
// on the operands the first part left in LDS.
template <class PC, class QC>
__global__ __launch_bounds__(PC::NT, 1) void bwd_chunk_kernel(BwdArgs b) {
  QLoads<QC> ql;
  if (!dpg_part<PC, QC>(b, ql)) return;
  dqk_part<QC, PC>(b, ql);
}

// ---------------------------------------------------------------- 4: token
// Chunks the ratio form cannot take, token by token from the chunk's entry
// state: for token t (in reverse) the state before it is rebuilt from S0
// (t forward steps), then one reverse step of the recurrence's adjoint.
template <class IO>
__global__ __launch_bounds__(kNT) void bwd_token_kernel(BwdArgs b) {
  using ST = typename IO::storage;
  const FwdArgs& a = b.f;
  const int dk = a.dk, dv = a.dv, H = a.H;
  const int total = a.maxc * H;
  const bool l2 = a.use_l2norm != 0;
  const float scale = a.scale;
  const int LD = dv + 1;  // padded rows: column and row sweeps both conflict-free
  extern __shared__ float sm[];
  float* sS = sm;              // [dk][LD] state before the token
  float* sG = sS + dk * LD;    // [dk][LD] adjoint of the state after the token
  float* xq = sG + dk * LD;    // [dk]
  float* xk = xq + dk;         // [dk]
  float* al = xk + dk;         // [dk]
  float* dxq = al + dk;        // [dk]
  float* dxk = dxq + dk;       // [dk]
  float* vv = dxk + dk;        // [dv]
  float* w = vv + dv;          // [dv]
  float* go = w + dv;          // [dv]
  float* e = go + dv;          // [dv]
  float* red = e + dv;         // [kNT / 64]
  const int tid = threadIdx.x;
  const ST* q = static_cast<const ST*>(a.q);
  const ST* k = static_cast<const ST*>(a.k);
  const ST* v = static_cast<const ST*>(a.v);
  const ST* dO = static_cast<const ST*>(b.dout);
  const float* alpha = static_cast<const float*>(a.alpha);
  const float* beta = static_cast<const float*>(a.beta);

  // token t of the chunk: normalised q, k into xq, xk; alpha into al; v into vv
  auto load_token = [&](int64_t t, int h) {
    const int64_t base = (t * H + h) * dk;
    float sq = 0.f, sk = 0.f;
    for (int cc = tid; cc < dk; cc += kNT) {
      const float x = IO::load(q, base + cc), y = IO::load(k, base + cc);
      xq[cc] = x;
      xk[cc] = y;
      al[cc] = alpha[base + cc];
      sq += x * x;
      sk += y * y;
    }
    for (int j = tid; j < dv; j += kNT) vv[j] = IO::load(v, (t * H + h) * dv + j);
    sq = block_sum(sq, red);
    sk = block_sum(sk, red);
    const float rq = l2 ? __fdiv_rn(1.f, __fsqrt_rn(sq + kL2Eps)) : 1.f;
    const float rk = l2 ? __fdiv_rn(1.f, __fsqrt_rn(sk + kL2Eps)) : 1.f;
    for (int cc = tid; cc < dk; cc += kNT) {
      xq[cc] *= rq;
      xk[cc] *= rk;
    }
    __syncthreads();
    return make_float2(rq, rk);
  };
  // w = (Diag(al) S)^T xk
  auto erase = [&]() {
    for (int j = tid; j < dv; j += kNT) {
      float s = 0.f;
      for (int cc = 0; cc < dk; ++cc) s += al[cc] * sS[cc * LD + j] * xk[cc];
      w[j] = s;
    }
    __syncthreads();
  };

  for (int idx = blockIdx.x; idx < total; idx += gridDim.x) {
    const int c = idx / H, h = idx % H;
    const int64_t slot = static_cast<int64_t>(h) * a.maxc + c;
    if (b.bflag[slot] == 0) continue;
    const Geo g = geo_of(a, c);
    const ST* S0 = static_cast<const ST*>(a.hc) + slot * dk * dv;
    const ST* dS1 = static_cast<const ST*>(b.dS) + slot * dk * dv;
    __syncthreads();
    for (int i = tid; i < dk * dv; i += kNT) sG[(i / dv) * LD + i % dv] = IO::load(dS1, i);
    for (int t = g.L - 1; t >= 0; --t) {
      // the state before token t
      __syncthreads();
      for (int i = tid; i < dk * dv; i += kNT) sS[(i / dv) * LD + i % dv] = IO::load(S0, i);
      __syncthreads();
      for (int tt = 0; tt < t; ++tt) {
        load_token(g.t0 + tt, h);
        erase();
        const float bt = beta[(g.t0 + tt) * H + h];
        for (int i = tid; i < dk * dv; i += kNT) {
          const int cc = i / dv, j = i % dv;
          float& s = sS[cc * LD + j];
          s = al[cc] * s + bt * xk[cc] * (vv[j] - w[j]);
        }
        __syncthreads();
      }
      // reverse step of token t
      const float2 r = load_token(g.t0 + t, h);
      const int64_t tok = g.t0 + t;
      const float bt = beta[tok * H + h];
      for (int j = tid; j < dv; j += kNT) go[j] = IO::load(dO, (tok * H + h) * dv + j);
      erase();
      // u = v - w (into vv); G += scale xq dO^T
      for (int j = tid; j < dv; j += kNT) vv[j] -= w[j];
      for (int i = tid; i < dk * dv; i += kNT) {
        const int cc = i / dv, j = i % dv;
        sG[cc * LD + j] += scale * xq[cc] * go[j];
      }
      __syncthreads();
      // u . dO, e = G^T xk
      float ud = 0.f;
      for (int j = tid; j < dv; j += kNT) ud += vv[j] * go[j];
      ud = block_sum(ud, red);
      for (int j = tid; j < dv; j += kNT) {
        float s = 0.f;
        for (int cc = 0; cc < dk; ++cc) s += sG[cc * LD + j] * xk[cc];
        e[j] = s;
      }
      __syncthreads();
      float db = 0.f;
      for (int j = tid; j < dv; j += kNT) db += e[j] * vv[j];
      db = block_sum(db, red);
      // dxq = scale S_t dO with S_t = X + beta xk u^T; dxk = beta G u - X (beta e)
      for (int cc = tid; cc < dk; cc += kNT) {
        float sdo = 0.f, gu = 0.f, xe = 0.f;
        for (int j = 0; j < dv; ++j) {
          const float x = al[cc] * sS[cc * LD + j];
          sdo += x * go[j];
          gu += sG[cc * LD + j] * vv[j];
          xe += x * e[j];
        }
        dxq[cc] = scale * (sdo + bt * xk[cc] * ud);
        dxk[cc] = bt * gu - bt * xe;
      }
      __syncthreads();
      // dX = G - xk (beta e)^T; dalpha; G <- Diag(alpha) dX
      for (int cc = tid; cc < dk; cc += kNT) {
        float da = 0.f;
        for (int j = 0; j < dv; ++j) {
          const float dX = sG[cc * LD + j] - xk[cc] * bt * e[j];
          da += dX * sS[cc * LD + j];
          sG[cc * LD + j] = al[cc] * dX;
        }
        b.dalpha[(tok * H + h) * dk + cc] = da;
      }
      // through the norms
      float pq = 0.f, pk = 0.f;
      for (int cc = tid; cc < dk; cc += kNT) {
        pq += xq[cc] * dxq[cc];
        pk += xk[cc] * dxk[cc];
      }
      pq = block_sum(pq, red);
      pk = block_sum(pk, red);
      for (int cc = tid; cc < dk; cc += kNT) {
        const int64_t i = (tok * H + h) * dk + cc;
        b.dq[i] = l2 ? r.x * (dxq[cc] - xq[cc] * pq) : dxq[cc];
        b.dk[i] = l2 ? r.y * (dxk[cc] - xk[cc] * pk) : dxk[cc];
      }
      if (tid == 0) b.dbeta[tok * H + h] = db;
    }
  }
}

template <class Cfg>
launch_result launch_state(const BwdArgs& b, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&bwd_state_kernel<Cfg>), hipFuncAttributeMaxDynamicSharedMemorySize,
      Cfg::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  const int64_t blocks = static_cast<int64_t>(b.f.num_seqs) * b.f.H * Cfg::NSPLIT;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_state_kernel<Cfg>, dim3(static_cast<unsigned>(blocks)), dim3(Cfg::NT),
                     Cfg::LDS_BYTES, stream, b);
  return hipGetLastError();
}

template <class PC, class QC>
launch_result launch_chunk(const BwdArgs& b, hipStream_t stream) {
  using M = QMap<QC, PC>;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&bwd_chunk_kernel<PC, QC>), hipFuncAttributeMaxDynamicSharedMemorySize,
      M::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  const int64_t items = static_cast<int64_t>(b.f.maxc) * b.f.H;
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL((bwd_chunk_kernel<PC, QC>), dim3(static_cast<unsigned>(items)), dim3(PC::NT),
                     M::LDS_BYTES, stream, b);
  return hipGetLastError();
}

struct BEntry {
  int chunk, dk, dv;
  launch_result (*fn)(const BwdArgs&, hipStream_t);
};
template <class Op, class IO, int C, int D, int DVT>
constexpr BEntry bentry() {
  return BEntry{C, D, D, &launch_state<BCfg<Op, IO, C, D, D, DVT>>};
}
// the shapes the forward takes, with the same dv tiles
const BEntry kStateBF16[] = {
    bentry<OpBF16, io_bf16, 64, 128, 64>(), bentry<OpBF16, io_bf16, 32, 128, 64>(),
    bentry<OpBF16, io_bf16, 16, 128, 64>(), bentry<OpBF16, io_bf16, 64, 64, 32>(),
    bentry<OpBF16, io_bf16, 32, 64, 32>(),  bentry<OpBF16, io_bf16, 16, 64, 32>(),
};
const BEntry kStateF32[] = {
    bentry<OpF32, io_f32, 16, 16, 16>(), bentry<OpF32, io_f32, 32, 16, 16>(),
    bentry<OpF32, io_f32, 64, 16, 16>(), bentry<OpF32, io_f32, 16, 32, 32>(),
    bentry<OpF32, io_f32, 32, 32, 32>(), bentry<OpF32, io_f32, 64, 32, 32>(),
    bentry<OpF32, io_f32, 16, 64, 32>(), bentry<OpF32, io_f32, 32, 64, 32>(),
};

template <class IO>
launch_result launch_io(const BwdArgs& b, hipStream_t stream) {
  const FwdArgs& a = b.f;
  const int C = a.chunk, dk = a.dk, dv = a.dv;
  constexpr bool bf = sizeof(typename IO::storage) == 2;
  const BEntry* e2 = nullptr;
  {
    const BEntry* first = bf ? kStateBF16 : kStateF32;
    const int count = bf ? static_cast<int>(sizeof(kStateBF16) / sizeof(BEntry))
                         : static_cast<int>(sizeof(kStateF32) / sizeof(BEntry));
    for (int i = 0; i < count; ++i)
      if (first[i].chunk == C && first[i].dk == dk && first[i].dv == dv) e2 = &first[i];
  }
  if (!e2) return hipErrorInvalidValue;
  {
    const launch_result r = e2->fn(b, stream);
    if (r != hipSuccess) return r;
  }
  const int64_t total = static_cast<int64_t>(a.maxc) * a.H;
  if (total == 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if constexpr (bf) {
    // bf16 inputs: the intra-chunk work on the matrix cores, both passes in
    // one workgroup per (chunk, head)
    launch_result (*fc)(const BwdArgs&, hipStream_t) = nullptr;
    if (dk == dv) {
      if (C == 64 && dk == 128) fc = &launch_chunk<PCfg<64, 128>, QCfg<64, 128>>;
      if (C == 64 && dk == 64) fc = &launch_chunk<PCfg<64, 64>, QCfg<64, 64>>;
      if (C == 32 && dk == 128) fc = &launch_chunk<PCfg<32, 128>, QCfg<32, 128>>;
      if (C == 32 && dk == 64) fc = &launch_chunk<PCfg<32, 64>, QCfg<32, 64>>;
      if (C == 16 && dk == 128) fc = &launch_chunk<PCfg<16, 128>, QCfg<16, 128>>;
      if (C == 16 && dk == 64) fc = &launch_chunk<PCfg<16, 64>, QCfg<16, 64>>;
    }
    if (!fc) return hipErrorInvalidValue;
    e = fc(b, stream);
    if (e != hipSuccess) return e;
  } else {
    const size_t lds3 = sizeof(float) * (4 * C * C + kGStage + 4 * C + 2 * dk) + sizeof(int);
    static const hipError_t attr3 = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&bwd_intra_kernel<IO>), hipFuncAttributeMaxDynamicSharedMemorySize, 80 * 1024);
    if (attr3 != hipSuccess) return attr3;
    hipLaunchKernelGGL((bwd_intra_kernel<IO>), dim3(static_cast<unsigned>(b.grid3)), dim3(kNT), lds3, stream, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t lds4 = sizeof(float) * (2 * dk * (dv + 1) + 5 * dk + 4 * dv + kNT / 64);
  static const hipError_t attr4 = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&bwd_token_kernel<IO>), hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr4 != hipSuccess) return attr4;
  const int64_t g4 = total < 256 ? total : 256;
  hipLaunchKernelGGL((bwd_token_kernel<IO>), dim3(static_cast<unsigned>(g4)), dim3(kNT), lds4, stream, b);
  return hipGetLastError();
}

}  // namespace

int32_t bwd_grid3(int64_t total) { return static_cast<int32_t>(total < kGrid3 ? (total > 0 ? total : 1) : kGrid3); }

int64_t bwd_extra_bytes(int32_t H, int64_t maxc, int32_t C, int32_t dk, int32_t dv, int32_t io_dtype) {
  auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
  const int64_t hm = static_cast<int64_t>(H) * maxc;
  const bool bf = io_dtype == CKDA_DTYPE_BF16;
  const int64_t es = bf ? 2 : 4;  // records in the io type
  const int64_t common = up(4 * hm * C * C) + 2 * up(es * hm * dk * dv) + up(es * hm * C * dv) + up(4 * hm);
  if (bf) return common;
  const int64_t SC = static_cast<int64_t>(C) * cmax(cmax(dk, dv), C);
  return common + up(4 * static_cast<int64_t>(bwd_grid3(hm)) * 14 * SC);  // the intra kernel's scratch
}

void bwd_layout(BwdArgs& b, unsigned char* base, int32_t io_dtype) {
  const FwdArgs& a = b.f;
  auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
  const int64_t hm = static_cast<int64_t>(a.H) * a.maxc;
  const int C = a.chunk, dk = a.dk, dv = a.dv;
  const bool bf = io_dtype == CKDA_DTYPE_BF16;
  const int64_t es = bf ? 2 : 4;
  b.f.xout = reinterpret_cast<float*>(base);
  base += up(4 * hm * C * C);
  b.f.hc = base;
  base += up(es * hm * dk * dv);
  b.dS = base;
  base += up(es * hm * dk * dv);
  b.dU = base;
  base += up(es * hm * C * dv);
  b.bflag = reinterpret_cast<int32_t*>(base);
  base += up(4 * hm);
  b.scratch = nullptr;
  b.grid3 = bwd_grid3(hm);
  if (!bf) b.scratch = reinterpret_cast<float*>(base);  // the intra kernel's scratch
}

launch_result launch_bwd_passes(const BwdArgs& b, int32_t io_dtype, hipStream_t stream) {
  return io_dtype == CKDA_DTYPE_BF16 ? launch_io<io_bf16>(b, stream) : launch_io<io_f32>(b, stream);
}

}  // namespace ckda
