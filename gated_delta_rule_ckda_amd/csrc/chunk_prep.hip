// Transform pass of the chunked forward: one workgroup per (chunk, head),
// all chunks independent.  It computes the chunk's gate prefix, the in-op
// L2 norms, the strictly lower matrix A and its unit-lower inverse
// X = (I + A)^{-1}, and writes everything the sequential state pass needs as
// one block of the workspace (layout in ckda_internal.h).
//
// Algebra (picx.dev summary of the Complex KDA paper, section "Background":
// transition A_t = (I - beta_t k_t k_t^T) Diag(alpha_t), with the write
// beta_t k_t v_t^T and the read-out o_t = S_t^T q_t).  Within a chunk of C
// tokens entered with state S0, with the per-channel decay
// D(r<-j) = prod_{j<s<=r} alpha_s:
//
//   (I + A) U = Diag(beta) (V - Kt S0),     A_rj = beta_r <k^_r . D(r<-j), k^_j>   (j < r)
//   O  = scale (Qt S0 + P U),               P_rj = <q^_r . D(r<-j), k^_j>          (j <= r)
//   S' = Diag(g) S0 + Kh^T U
//
// with Kt_r = D(r<-start) . k^_r, Qt_r = D(r<-start) . q^_r,
// Kh_j = D(end<-j) . k^_j, g = D(end<-start).  Hence U = X' V - W S0 with
// X' = X Diag(beta) and W = X Diag(beta) Kt, which is what the state pass runs.
//
// Gate prefix.  Running products of the gates (per channel, fp32) carry sign
// and magnitude together: signs are exact under multiplication and an exact
// zero gate makes every later product exactly zero.  Ft_r = prod_{s<=r}
// alpha_s from the chunk start gives Kt = k . Ft, Qt = q . Ft and g, all
// plain products.  A and P use ratios of products anchored either at the
// chunk start or at the start of every 16-row block (the MFMA tile height):
// with Fb_r the product over block(r)'s rows up to r and T_b the total of
// block b, for r in block I and j in block J <= I
//   D(r<-j) = Fb_r * E_IJ * (1 / Fb_j),   E_IJ = prod_{J <= b < I} T_b
// (E_II = 1), so with Lk = k . Fb, Lq = q . Fb, Rk = k / Fb every tile is one
// MFMA whose right operand is scaled per channel by E_IJ on its way in:
//   A_IJ = Diag(beta rk) Lk_I (Rk_J . E_IJ)^T Diag(rk),
//   P_IJ = Diag(rq) Lq_I (Rk_J . E_IJ)^T Diag(rk),   Kh = rk . Rk . prod_{b>=J} T_b.
// E_IJ and Kt are products, so gates that decay fast over the chunk only make
// them small, never wrong.  When every |Ft_r| of the chunk lies in
// [2^-100, 2^10] (the usual case) the anchor is the chunk start instead
// (Fb = Ft, every E_IJ = 1, no scaling); otherwise, when every |Fb_r| lies in
// that range (a condition on 16 consecutive gates), the block anchors are
// used.  Chunks that pass neither test (exact zero gates among them: a zero
// makes every later plain product zero; products that underflow over 16
// tokens; non-finite values) are flagged and left to a second launch.  It
// restarts the products after each zero gate and masks the MFMA operands per
// (row, channel) with a map of the zero rows, so the pairs that straddle a
// zero drop out of A, P and Kh exactly (sign, magnitude and zero kept apart,
// as in Proposition 2 of the picx.dev summary, "Theoretical Framework").
// Chunks with two zeros in one (16-row block, channel), or with restarted
// products still out of range, get A, P and Kh from direct products of the
// gates staged in LDS.  Keeping both forms out of the first launch keeps its
// registers to what the other chunks need.
//
// Gates arrive as float32 values or as logits (float32 or bf16) activated on
// load (ckda_internal.h).
//
// q and k enter raw; the in-op L2 normalisation (dormouse review "RoPE into
// the KDA q/k path", section 2) is applied as the row scales rq, rk above.
//
// Phases (eight waves; wave w owns rows w*C/8 .. in the element-wise phases):
//   1  loads, running products within the wave's rows, row norms
//   2  chunk-level products Ft, anchor choice, regularity vote, operands Lk,
//      Lq, Rk (and E_IJ for block anchors); Qt', g out
//   3  A and P on MFMA (masked in the second launch, or direct products); P' out
//   4  Kt'^T to LDS, Kh'^T out; 16x16 diagonal blocks of X by forward substitution
//   5  off-diagonal blocks X_IJ = -X_II sum_{J<=M<I} A_IM X_MJ on fp32 MFMA
//   6  X' out, -W = -X Kt' on MFMA, out
// Rows of the block are written in the fragment storage order of
// mfma_ops.h (perm32 for bf16 rows whose length is a multiple of 32).
#include "mfma_ops.h"

namespace ckda {
namespace {

constexpr float kRegularMin = 0x1p-100f;
constexpr int64_t kRedoGrid = 256;  // workgroups of the second transform launch (one per CU)
constexpr float kRegularMax = 0x1p+10f;

// N consecutive logical entries start .. start+N-1 of a row of length K in
// the handoff storage order (start a multiple of 4, or of 2 for N == 2).
template <class Op, int N, int K>
__device__ __forceinline__ void store_run_pos(typename Op::T* row, int start, const float* v) {
  if constexpr (N <= 2) {
    store_run<Op, N>(row + Op::template pos<K>(start), v);
  } else {
#pragma unroll
    for (int g = 0; g < N; g += 4)
      Op::store4(row + Op::template pos<K>(start + g), f32x4{v[g], v[g + 1], v[g + 2], v[g + 3]});
  }
}

template <class OpT, class IOT, int C_, int DK_>
struct PrepCfg {
  using Op = OpT;
  using IO = IOT;
  using T = typename Op::T;
  static constexpr int NW = 8, NT = 64 * NW;
  static constexpr int C = C_, DK = DK_;
  static constexpr int NB = C / 16;
  static constexpr int RPW = C / NW;                 // rows per wave, element-wise phases
  static constexpr int CPT = DK >= 64 ? DK / 64 : 1; // channels per lane
  static constexpr int NCG = DK / CPT;               // lanes holding channels
  static constexpr int ES = static_cast<int>(sizeof(T));
  static constexpr int IOES = static_cast<int>(sizeof(typename IO::storage));
  static constexpr int LDK = frag_stride(DK, ES);
  static constexpr int LDC = frag_stride(C, ES);
  static constexpr int LDA = 20;                     // fp32 16x16 block stride (conflict-free)
  static constexpr int BLKF = 16 * LDA;              // floats per 16x16 block
  static constexpr int NBA = NB * (NB - 1) / 2;      // strictly lower blocks of A
  static constexpr int NBX = NB * (NB + 1) / 2;      // lower blocks of X (with the diagonal)
  static constexpr int QB = CPT * IOES;              // bytes of q (or k) per row and lane
  static constexpr int QW = (QB + 3) / 4;
  // direct path for irregular chunks: G threads per column, DG channels each
  static constexpr int DG = (NT / C) < DK ? (NT / C) : DK;
  static constexpr int DCH = DK / DG;

  // byte offsets
  static constexpr int O_LQ = 0;                                        // Lq [C][LDK] | Kh'^T [DK][LDH] | Xb [C][LDC]
  static constexpr int SZ_LQ = align16(cmax(C * LDK, C * LDC) * ES);
  // Kh'^T staged for row-wise stores: rows of C in storage order, padded by
  // 16 bytes where that fits (spreads the column writes over the banks)
  static constexpr int LDH = (DK * (C * ES + 16) <= SZ_LQ) ? C + 16 / ES : C;
  static constexpr int O_LK = O_LQ + SZ_LQ;                             // Lk [C][LDK] | Kt'^T [DK][LDC]
  static constexpr int O_RK = O_LK + C * LDK * ES;                      // Rk [C][LDK]
  static constexpr int O_TS = O_LK + align16(DK * LDC * ES);            // level scratch (after Rk dies)
  static constexpr int SZ_R = align16(cmax(2 * C * LDK * ES, DK * LDC * ES + NB * BLKF * 4));
  static constexpr int O_A = O_LK + SZ_R;                               // A blocks (I > J), fp32
  static constexpr int O_XF = O_A + (NBA > 0 ? NBA : 1) * BLKF * 4;     // X blocks (I >= J), fp32
  static constexpr int O_G = O_XF + NBX * BLKF * 4;                     // wave-row products [NW][DK]
  static constexpr int O_RQ = O_G + NW * DK * 4;                        // rq [C]
  static constexpr int O_RK2 = O_RQ + C * 4;                            // rk [C]
  static constexpr int O_BETA = O_RK2 + C * 4;                          // beta [C]
  static constexpr int O_FLAG = O_BETA + C * 4;                         // votes [3][NW]
  // rows whose gate is exactly zero: one byte per (wave, channel), bit i for
  // the wave's row i, laid out [block][channel][wave in block] so that a
  // channel's 16-row mask is WPB adjacent bytes
  static constexpr int WPB = 16 / RPW;                                  // waves per 16-row block
  static constexpr int O_ZB = O_FLAG + 3 * NW * 4;
  static constexpr int O_BC = O_ZB + NW * DK;                           // second launch: the next slot
  static constexpr int LDS_BYTES = align16(O_BC + 4);
  // direct path staging, inside the operand region it leaves unused
  static constexpr int O_DGATE = 0;                                     // gates [C][DK] fp32
  static constexpr int O_DROW = C * DK * 4;                             // q or k rows [C][DK]

  static_assert(C % 16 == 0 && DK % 16 == 0 && C <= 64 && DK <= 128, "tile sizes");
  static_assert(NB <= NW && RPW >= 2 && (RPW & (RPW - 1)) == 0 && RPW <= 8, "row split");
  static_assert(DG * C <= NT && DK % DG == 0 && (DG & (DG - 1)) == 0 && DG <= 64, "direct path");
  static_assert(LDS_BYTES <= 80 * 1024, "two workgroups per CU");
  static_assert(DK * LDH * ES <= SZ_LQ && (C * ES) % 16 == 0 && (LDH * ES) % 16 == 0, "Kh staging");
  static_assert(O_DROW + C * DK * IOES <= O_A, "direct path staging fits the operand region");
};

template <class Cfg>
__device__ __forceinline__ float* a_blk(unsigned char* smem, int I, int M) {
  return reinterpret_cast<float*>(smem + Cfg::O_A) + (I * (I - 1) / 2 + M) * Cfg::BLKF;
}
template <class Cfg>
__device__ __forceinline__ float* x_blk(unsigned char* smem, int I, int J) {
  return reinterpret_cast<float*>(smem + Cfg::O_XF) + (I * (I + 1) / 2 + J) * Cfg::BLKF;
}

// I, J of the idx-th lower block (J <= I) in row order
__device__ __forceinline__ void lower_block(int idx, int& I, int& J) {
  I = 0;
  while (idx > I) {
    idx -= I + 1;
    ++I;
  }
  J = idx;
}

// One lower 16x16 tile (I, J) of A and of P^T from the same right operand:
// acc_a += Lk_I (Rk_J . E)^T and acc_p += (Rk_J . E) Lq_I^T over K = DK, where
// the fp32 vector e[0..DK) (the gate product between the blocks) scales the K
// index of Rk on its way into the MFMA; e == nullptr (a diagonal tile) leaves
// it unscaled.  Operand rows are [16][LDK] in LDS.
template <class Cfg>
__device__ __forceinline__ void tile_ap(f32x4& acc_a, f32x4& acc_p, const typename Cfg::T* lk,
                                        const typename Cfg::T* lq, const typename Cfg::T* rk,
                                        const float* e, int lane) {
  using Op = typename Cfg::Op;
  constexpr int DK = Cfg::DK, LDK = Cfg::LDK;
  const int r = lane & 15, kq = lane >> 4;
  if constexpr (sizeof(typename Op::T) == 2) {
    static_assert(DK % 32 == 0, "bf16 operand rows");
    constexpr int NS = DK / 32;
    // one K slice at a time: three fragments live, not 3 * NS
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 fa = *reinterpret_cast<const bf16x8*>(lk + r * LDK + 32 * s + 8 * kq);
      const bf16x8 fq = *reinterpret_cast<const bf16x8*>(lq + r * LDK + 32 * s + 8 * kq);
      bf16x8 fb = *reinterpret_cast<const bf16x8*>(rk + r * LDK + 32 * s + 8 * kq);
      if (e) {
        const f32x4 e0 = *reinterpret_cast<const f32x4*>(e + 32 * s + 8 * kq);
        const f32x4 e1 = *reinterpret_cast<const f32x4*>(e + 32 * s + 8 * kq + 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          fb[i] = Op::cvt(static_cast<float>(fb[i]) * e0[i]);
          fb[4 + i] = Op::cvt(static_cast<float>(fb[4 + i]) * e1[i]);
        }
      }
      acc_a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc_a, 0, 0, 0);
      acc_p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, fq, acc_p, 0, 0, 0);
    }
  } else {
    constexpr int NS = DK / 4;
    float fa[NS], fq[NS], fb[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      fa[s] = lk[r * LDK + kq + 4 * s];
      fq[s] = lq[r * LDK + kq + 4 * s];
      fb[s] = rk[r * LDK + kq + 4 * s];
    }
    if (e) {
#pragma unroll
      for (int s = 0; s < NS; ++s) fb[s] *= e[kq + 4 * s];
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      acc_a = mfma_f32(fa[s], fb[s], acc_a);
      acc_p = mfma_f32(fb[s], fq[s], acc_p);
    }
  }
}

// The zero rows of a 16-row block for one channel as a 16-bit mask (bit r for
// the block's row r), from the block's bytes of the zero map.
template <class Cfg>
__device__ __forceinline__ uint32_t zmask16(const uint8_t* zb, int ch) {
  uint32_t m = 0;
#pragma unroll
  for (int w = 0; w < Cfg::WPB; ++w) m |= static_cast<uint32_t>(zb[ch * Cfg::WPB + w]) << (w * Cfg::RPW);
  return m;
}

// tile_ap for a chunk with exact zero gates (block anchors; the operands
// Lk, Lq, Rk use the products restarted after a zero: D(r<-j) is their ratio
// for r, j on the same side of every zero, and 0 across one).  zi, zj: the
// zero map of the row block I and of the column block J.
//   mode 0, off-diagonal tile: row r of I keeps channel c while no zero of
//     c lies at or before r in I (the prefix D(r<-a_I)); row j of J keeps it
//     while no zero lies after j in J (the suffix D(e_J<-j)); e scales the
//     right operand by the products between the blocks;
//   mode 1, diagonal tile: the pairs before the block's zero of c;
//   mode 2, diagonal tile: the pairs at or after it (one zero per block and
//     channel; more take the direct path).
template <class Cfg>
__device__ __forceinline__ void tile_ap_z(f32x4& acc_a, f32x4& acc_p,
                                                    const typename Cfg::T* lk,
                                                    const typename Cfg::T* lq,
                                                    const typename Cfg::T* rk, const float* e,
                                                    const uint8_t* zi, const uint8_t* zj,
                                                    int mode, int lane) {
  using Op = typename Cfg::Op;
  constexpr int DK = Cfg::DK, LDK = Cfg::LDK;
  const int r = lane & 15, kq = lane >> 4;
  const uint32_t upto = (2u << r) - 1u;  // rows 0..r
  // left: mode 2 keeps rows with a zero at or before them, modes 0 and 1
  // those without; right: mode 0 keeps rows with no zero after them, mode 1
  // rows with no zero at or before them, mode 2 rows with one
  const uint32_t lsel = mode == 2 ? 1u : 0u;
  auto keep_left = [&](uint32_t m) { return ((m & upto) != 0u ? 1u : 0u) == lsel; };
  auto keep_right = [&](uint32_t m) {
    return mode == 0 ? (m >> (r + 1)) == 0u : (((m & upto) != 0u ? 1u : 0u) == lsel);
  };
  if constexpr (sizeof(typename Op::T) == 2) {
    static_assert(DK % 32 == 0, "bf16 operand rows");
    constexpr int NS = DK / 32;
#pragma unroll 1
    for (int s = 0; s < NS; ++s) {
      const int c0 = 32 * s + 8 * kq;
      bf16x8 fa = *reinterpret_cast<const bf16x8*>(lk + r * LDK + c0);
      bf16x8 fq = *reinterpret_cast<const bf16x8*>(lq + r * LDK + c0);
      bf16x8 fb = *reinterpret_cast<const bf16x8*>(rk + r * LDK + c0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const bool kl = keep_left(zmask16<Cfg>(zi, c0 + i)), kr = keep_right(zmask16<Cfg>(zj, c0 + i));
        const float ev = e ? e[c0 + i] : 1.f;
        fa[i] = kl ? fa[i] : Op::cvt(0.f);
        fq[i] = kl ? fq[i] : Op::cvt(0.f);
        fb[i] = kr ? Op::cvt(static_cast<float>(fb[i]) * ev) : Op::cvt(0.f);
      }
      acc_a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa, fb, acc_a, 0, 0, 0);
      acc_p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb, fq, acc_p, 0, 0, 0);
    }
  } else {
    constexpr int NS = DK / 4;
#pragma unroll 1
    for (int s = 0; s < NS; ++s) {
      const int ch = kq + 4 * s;
      const bool kl = keep_left(zmask16<Cfg>(zi, ch)), kr = keep_right(zmask16<Cfg>(zj, ch));
      const float fa = kl ? lk[r * LDK + ch] : 0.f;
      const float fq = kl ? lq[r * LDK + ch] : 0.f;
      const float fb = kr ? rk[r * LDK + ch] * (e ? e[ch] : 1.f) : 0.f;
      acc_a = mfma_f32(fa, fb, acc_a);
      acc_p = mfma_f32(fb, fq, acc_p);
    }
  }
}

// Chunk rows 0..C-1 of a q/k/alpha-shaped tensor (row r at element
// base + r * rowstride) copied into LDS as [C][DK], with 16-byte loads that
// are all issued before the first store.  Gates are widened (and activated)
// to float32 and rows past L read as 1; q and k rows keep their io type and
// rows past L read as 0.
template <class Cfg, class G>
__device__ __forceinline__ void stage_gates(float* sgate, const void* galpha, bool ckda,
                                            int64_t base, int rowstride, int L, int tid) {
  using GS = typename G::storage;
  constexpr int C = Cfg::C, DK = Cfg::DK, NT = Cfg::NT;
  constexpr int ES = static_cast<int>(sizeof(GS)), VE = 16 / ES, NV = C * DK / VE;
  constexpr int PER = (NV + NT - 1) / NT;
  const rsrc_t rs = make_rsrc(static_cast<const GS*>(galpha) + base, ((L - 1) * rowstride + DK) * ES);
  uint32_t raw[PER][4];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = iclamp(u * NT + tid, NV - 1) * VE;
    ldraw<16>(rs, (iclamp(e / DK, L - 1) * rowstride + e % DK) * ES, raw[u]);
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int v = u * NT + tid;
    if (v < NV) {
      const int e = v * VE;
      const bool in = e / DK < L;
      float x[VE];
#pragma unroll
      for (int i = 0; i < VE; ++i) {
        float g = dec<G>(raw[u], i);
        if constexpr (G::logits) g = alpha_from_logit(g, ckda);
        x[i] = in ? g : 1.f;
      }
#pragma unroll
      for (int i = 0; i < VE; i += 4)
        *reinterpret_cast<f32x4*>(sgate + e + i) = f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]};
    }
  }
}

template <class Cfg>
__device__ __forceinline__ void stage_io(typename Cfg::IO::storage* srow, const void* gsrc,
                                         int64_t base, int rowstride, int L, int tid) {
  using ST = typename Cfg::IO::storage;
  constexpr int C = Cfg::C, DK = Cfg::DK, NT = Cfg::NT;
  constexpr int ES = static_cast<int>(sizeof(ST)), VE = 16 / ES, NV = C * DK / VE;
  constexpr int PER = (NV + NT - 1) / NT;
  const rsrc_t rs = make_rsrc(static_cast<const ST*>(gsrc) + base, ((L - 1) * rowstride + DK) * ES);
  uint32_t raw[PER][4];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int e = iclamp(u * NT + tid, NV - 1) * VE;
    ldraw<16>(rs, (iclamp(e / DK, L - 1) * rowstride + e % DK) * ES, raw[u]);
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int v = u * NT + tid;
    if (v < NV) {
      const int e = v * VE;
      const uint32_t m = (e / DK < L) ? 0xFFFFFFFFu : 0u;
      *reinterpret_cast<uint4*>(srow + e) =
          make_uint4(raw[u][0] & m, raw[u][1] & m, raw[u][2] & m, raw[u][3] & m);
    }
  }
}

// One pass of the direct products over the staged rows: for column j (DG
// lanes, DCH channels each) and every row r, the sum over channels of
// row_r . D(r<-j) . k_j, with D built one gate at a time (d *= alpha_r for
// r > j).  Several rows per step, so that their LDS reads and lane
// reductions overlap.  emit(r, sum) runs in the column's first lane.
template <class Cfg, class Emit>
__device__ __forceinline__ void direct_pass(const float* sgate, const typename Cfg::IO::storage* srow,
                                            const float (&kj)[Cfg::DCH], int j, int c0, bool col,
                                            Emit emit) {
  using IO = typename Cfg::IO;
  constexpr int C = Cfg::C, DK = Cfg::DK, DG = Cfg::DG, DCH = Cfg::DCH;
  constexpr int RS = DCH > 8 ? 2 : 4;  // rows per step
  float d[DCH];
#pragma unroll
  for (int e = 0; e < DCH; ++e) d[e] = 1.f;
#pragma unroll 1
  for (int r0 = 0; r0 < C; r0 += RS) {
    float p[RS];
#pragma unroll
    for (int u = 0; u < RS; ++u) {
      const int r = r0 + u;
      const float* gr = sgate + r * DK + c0;
      const typename IO::storage* xr = srow + r * DK + c0;
      p[u] = 0.f;
#pragma unroll
      for (int e = 0; e < DCH; ++e) {
        d[e] *= (r > j) ? gr[e] : 1.f;
        p[u] += IO::load(xr, e) * (d[e] * kj[e]);
      }
      p[u] = (col && r >= j) ? p[u] : 0.f;
    }
#pragma unroll
    for (int m = 1; m < DG; m <<= 1)
#pragma unroll
      for (int u = 0; u < RS; ++u) p[u] += __shfl_xor(p[u], m, 64);
#pragma unroll
    for (int u = 0; u < RS; ++u) emit(r0 + u, p[u]);
  }
}

// Direct products for a chunk that is not regular (a zero gate, or running
// gate products outside [2^-100, 2^10]): A and P from D(r<-j) built one gate
// at a time, over the chunk's rows staged in LDS (the MFMA operand region,
// which this path leaves unused): the gates stay, the k rows (A pass) and
// then the q rows (P pass) take turns in the second slot.  DG lanes per
// column j, DCH channels each.  Row r of the chunk starts at element
// qbase + r * qstride of q and k and at abase + r * astride of alpha.  Every
// thread of the workgroup calls
// this (it holds barriers).
template <class Cfg, class G>
__device__ __forceinline__ void direct_ap(const void* gq, const void* gk, const void* galpha,
                                       bool ckda, int64_t qbase, int qstride, int64_t abase,
                                       int astride, int L, float scale,
                                       typename Cfg::T* gP, unsigned char* smem, int tid) {
  using IO = typename Cfg::IO;
  using ST = typename IO::storage;
  using Op = typename Cfg::Op;
  constexpr int C = Cfg::C, DK = Cfg::DK, DG = Cfg::DG, DCH = Cfg::DCH, LDA = Cfg::LDA;
  const float* srq = reinterpret_cast<const float*>(smem + Cfg::O_RQ);
  const float* srk = reinterpret_cast<const float*>(smem + Cfg::O_RK2);
  const float* sbeta = reinterpret_cast<const float*>(smem + Cfg::O_BETA);
  float* sgate = reinterpret_cast<float*>(smem + Cfg::O_DGATE);
  ST* srow = reinterpret_cast<ST*>(smem + Cfg::O_DROW);

  stage_gates<Cfg, G>(sgate, galpha, ckda, abase, astride, L, tid);
  stage_io<Cfg>(srow, gk, qbase, qstride, L, tid);
  __syncthreads();
  const bool act = tid < DG * C;
  const int j = act ? tid / DG : 0, cg = tid % DG, c0 = cg * DCH;
  const int J = j / 16;
  const bool col = act && j < L;
  const bool lead = act && cg == 0;
  float kj[DCH];
#pragma unroll
  for (int e = 0; e < DCH; ++e) kj[e] = IO::load(srow, j * DK + c0 + e);
  const float rkj = srk[j];

  // A_rj = beta_r rk_r rk_j <k_r . D(r<-j), k_j>, j < r (lower blocks of A,
  // strict lower part of the diagonal blocks, which hold X's diagonal blocks)
  direct_pass<Cfg>(sgate, srow, kj, j, c0, col, [&](int r, float s) {
    const int I = r / 16;
    if (lead && I >= J) {
      const float av = (r > j) ? s * sbeta[r] * srk[r] * rkj : 0.f;
      float* blk = (I > J) ? a_blk<Cfg>(smem, I, J) : x_blk<Cfg>(smem, I, I);
      blk[(r % 16) * LDA + j % 16] = av;
    }
  });
  __syncthreads();
  stage_io<Cfg>(srow, gq, qbase, qstride, L, tid);
  __syncthreads();
  // P_rj = scale rq_r rk_j <q_r . D(r<-j), k_j>, j <= r, zero above
  direct_pass<Cfg>(sgate, srow, kj, j, c0, col, [&](int r, float s) {
    constexpr int TES = static_cast<int>(sizeof(typename Cfg::T));
    const int pj = Op::template pos<C>(j);
    if (lead && !tri_dead(C, TES, r, pj))
      gP[tri_row(C, TES, r) + pj] = Op::cvt((r >= j) ? s * scale * srq[r] * rkj : 0.f);
  });
}

// Flags of the transform pass's first launch, per (head, chunk slot)
constexpr int kFlagRegular = 0;  // done by the first launch
constexpr int kFlagRedo = 1;     // left to the second launch

// One (chunk, head) of the transform pass.  MODE = kFlagRegular (the first
// launch): the MFMA form for chunks whose plain running products are in
// range (so none with a zero gate); any other chunk gets its flag set and is
// left to the second launch.  MODE = kFlagRedo (the second launch): products
// restarted after zero gates; in range with one zero per (block, channel) at
// most, the masked MFMA form (tile_ap_z); anything else, A and P from direct
// products.
template <class Cfg, class G, int MODE>
__device__ __forceinline__ void prep_chunk(const FwdArgs& a, int c, int h, unsigned char* smem,
                                           int tid = static_cast<int>(threadIdx.x)) {
  using Op = typename Cfg::Op;
  using IO = typename Cfg::IO;
  using T = typename Cfg::T;
  constexpr int C = Cfg::C, DK = Cfg::DK, NB = Cfg::NB, NW = Cfg::NW, NT = Cfg::NT;
  constexpr int RPW = Cfg::RPW, CPT = Cfg::CPT, NCG = Cfg::NCG, ES = Cfg::IOES;
  constexpr int LDK = Cfg::LDK, LDC = Cfg::LDC, LDA = Cfg::LDA;

  T* sLq = reinterpret_cast<T*>(smem + Cfg::O_LQ);
  T* sXb = reinterpret_cast<T*>(smem + Cfg::O_LQ);
  T* sKhT = reinterpret_cast<T*>(smem + Cfg::O_LQ);
  T* sLk = reinterpret_cast<T*>(smem + Cfg::O_LK);
  T* sRk = reinterpret_cast<T*>(smem + Cfg::O_RK);
  T* sKtT = reinterpret_cast<T*>(smem + Cfg::O_LK);
  float* sTS = reinterpret_cast<float*>(smem + Cfg::O_TS);
  float* sG = reinterpret_cast<float*>(smem + Cfg::O_G);
  float* srq = reinterpret_cast<float*>(smem + Cfg::O_RQ);
  float* srk = reinterpret_cast<float*>(smem + Cfg::O_RK2);
  float* sbeta = reinterpret_cast<float*>(smem + Cfg::O_BETA);
  int* sFlag = reinterpret_cast<int*>(smem + Cfg::O_FLAG);

  const int wave = tid >> 6, lane = tid & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int H = a.H, Hk = a.Hk;
  const int hk = h / (H / Hk);  // query/key head of value head h

  int64_t t0;
  int L;
  if (a.cu_seqlens) {
    const int2 gc = a.chunk_geo[c];  // one load: the chunk's first token and length
    L = uniform32(gc.y);
    if (L == 0) {  // unused chunk slot
      if (MODE == kFlagRegular && tid == 0) a.irregular[h * a.maxc + c] = kFlagRegular;
      return;
    }
    t0 = uniform32(gc.x);
  } else {
    const int n = c / a.nc, i = c % a.nc;
    t0 = static_cast<int64_t>(n) * a.T + static_cast<int64_t>(i) * C;
    L = (a.T - i * C) < C ? (a.T - i * C) : C;
  }
  T* blk = reinterpret_cast<T*>(a.blocks + (static_cast<int64_t>(h) * a.maxc + c) * a.blk_bytes);
  T* gX = blk;
  constexpr int TES = static_cast<int>(sizeof(T));  // handoff element size
  T* gW = blk + blk_off_W(C, DK, TES);
  T* gQ = blk + blk_off_Q(C, DK, TES);
  T* gP = blk + blk_off_P(C, DK, TES);
  T* gK = blk + blk_off_K(C, DK, TES);
  float* gg = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(blk) + blk_g_byte(C, DK, sizeof(T)));

  const bool use_l2 = a.use_l2norm != 0;
  const bool ckda = a.gate_range == CKDA_GATE_CKDA;
  const bool scan_on = lane < NCG;
  const int c0ch = lane * CPT;
  const int r0 = wave * RPW;

  // ================= 1: loads, running products, norms ======================
  float xq[RPW][CPT], xk[RPW][CPT], F[RPW][CPT];
  {
    constexpr int GES = static_cast<int>(sizeof(typename G::storage));
    constexpr int GB = CPT * GES, GW = (GB + 3) / 4;  // gate bytes (words) per row and lane
    const int krow = Hk * DK * ES, arow = H * DK * GES;
    const int64_t qk_off = (t0 * Hk + hk) * static_cast<int64_t>(DK);
    const int64_t a_off = (t0 * H + h) * static_cast<int64_t>(DK);
    uint32_t rqv[RPW][Cfg::QW], rkv[RPW][Cfg::QW], rav[RPW][GW];
    if (scan_on) {
      const rsrc_t rq = make_rsrc(static_cast<const char*>(a.q) + qk_off * ES, L * krow);
      const rsrc_t rk = make_rsrc(static_cast<const char*>(a.k) + qk_off * ES, L * krow);
      const rsrc_t ra = make_rsrc(static_cast<const char*>(a.alpha) + a_off * GES, L * arow);
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int row = iclamp(r0 + i, L - 1);
        ldraw<Cfg::QB, kStream>(rq, c0ch * ES + row * krow, rqv[i]);
        ldraw<Cfg::QB, kStream>(rk, c0ch * ES + row * krow, rkv[i]);
        ldraw<GB, kStream>(ra, c0ch * GES + row * arow, rav[i]);
      }
    }
    if (tid < C) sbeta[tid] = (tid < L) ? load_beta<G>(a.beta, (t0 + tid) * H + h, ckda) : 0.f;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const bool in = scan_on && (r0 + i < L);
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) {
        xq[i][cc] = in ? dec<IO>(rqv[i], cc) : 0.f;
        xk[i][cc] = in ? dec<IO>(rkv[i], cc) : 0.f;
        float g = dec<G>(rav[i], cc);
        if constexpr (G::logits) g = alpha_from_logit(g, ckda);
        F[i][cc] = in ? g : 1.f;
      }
    }
  }
  // running products over this wave's rows, restarted after a gate that is
  // exactly zero (the zero's row takes 1, the empty product of the gates
  // after it); their totals go to sG and the zero rows to the zero map
  // (the first launch keeps plain products: a zero gate makes its chunk
  // irregular there, and the later launches take it)
  constexpr bool ZL = MODE != kFlagRegular;
  uint32_t zbits[CPT];
  if constexpr (!ZL) {
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      float f = 1.f;
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        f *= F[i][cc];
        F[i][cc] = f;
      }
      zbits[cc] = 0u;
      if (scan_on) sG[wave * DK + c0ch + cc] = f;
    }
  } else {
    uint8_t* zmap = reinterpret_cast<uint8_t*>(smem + Cfg::O_ZB);
    constexpr int WPB = Cfg::WPB;
    const int blk = wave / WPB, wib = wave % WPB;
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      float f = 1.f;
      uint32_t zb = 0;
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const bool z = F[i][cc] == 0.f;
        zb |= z ? (1u << i) : 0u;
        f = z ? 1.f : f * F[i][cc];
        F[i][cc] = f;
      }
      zbits[cc] = zb;
      if (scan_on) {
        sG[wave * DK + c0ch + cc] = f;
        zmap[(blk * DK + c0ch + cc) * WPB + wib] = static_cast<uint8_t>(zb);
      }
    }
  }
  {
    float pq[RPW], pk[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      pq[i] = 0.f;
      pk[i] = 0.f;
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) {
        pq[i] += xq[i][cc] * xq[i][cc];
        pk[i] += xk[i][cc] * xk[i][cc];
      }
    }
    const float sq = wave_row_sums<RPW>(pq, lane);
    const float sk = wave_row_sums<RPW>(pk, lane);
    constexpr int LPR = 64 / RPW;
    if ((lane & (LPR - 1)) == 0) {
      const int row = r0 + lane / LPR;
      srq[row] = use_l2 ? __fdiv_rn(1.f, __fsqrt_rn(sq + kL2Eps)) : 1.f;
      srk[row] = use_l2 ? __fdiv_rn(1.f, __fsqrt_rn(sk + kL2Eps)) : 1.f;
    }
  }
  __syncthreads();  // B1

  // ================= 2: chunk products, regularity, operands =================
  float kt[RPW][CPT], kh[RPW][CPT], gch[CPT], gsuf[CPT];
  bool canchor = false;  // operands anchored at the chunk start (no E_IJ)
  const uint8_t* zmap = reinterpret_cast<const uint8_t*>(smem + Cfg::O_ZB);
  {
    constexpr int WPB = Cfg::WPB;       // waves per 16-row block
    const int wb0 = wave - wave % WPB;  // first wave of this wave's block
    bool ok = true;
    // products of the wave totals.  Plain products (exactly zero across a
    // zero gate): before this wave from the chunk start (gpre), after this
    // wave (gsuf), all (gch).  Restarted after the block's zeros: from the
    // block start before this wave (bpre, the block anchor); the block's
    // total after its last zero times the plain totals of the later blocks
    // (gbs, for Kh).  Every (block, channel) may hold one zero gate at most.
    float gpre[CPT], bpre[CPT], gbs[CPT];
    uint32_t bz[CPT];  // this wave's block: the channel's zero rows
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      float gp = 1.f, bp = 1.f, g = 1.f, gs = 1.f, bt = 1.f, later = 1.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float tw = scan_on ? sG[w * DK + c0ch + cc] : 1.f;
        const bool zw = ZL && scan_on && zmap[((w / WPB) * DK + c0ch + cc) * WPB + w % WPB] != 0;
        const float pw = zw ? 0.f : tw;  // the plain total
        if (w < wave) gp *= pw;
        if (w > wave) gs *= pw;
        g *= pw;
        if (w >= wb0 && w < wave) bp = zw ? tw : bp * tw;
        if (w >= wb0 && w < wb0 + WPB) bt = zw ? tw : bt * tw;
        if (w >= wb0 + WPB) later *= pw;
      }
      gpre[cc] = gp;
      bpre[cc] = bp;
      gbs[cc] = bt * later;
      gch[cc] = g;
      gsuf[cc] = gs;
      bz[cc] = (ZL && scan_on) ? zmask16<Cfg>(zmap + (wave / WPB) * DK * WPB, c0ch + cc) : 0u;
      ok = ok && (bz[cc] & (bz[cc] - 1u)) == 0;  // one zero per block and channel at most
    }
    if (scan_on && wave == 0) {
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) gg[c0ch + cc] = gch[cc];
    }
    // chunk anchors when every |Ft| of the chunk is in range (then E_IJ = 1
    // factors out of every tile), else block anchors
    if constexpr (MODE == kFlagRegular) {
      // (a zero gate anywhere rules them out: F restarts after it)
      bool okc = true;
#pragma unroll
      for (int i = 0; i < RPW; ++i)
#pragma unroll
        for (int cc = 0; cc < CPT; ++cc) {
          const float mag = fabsf(gpre[cc] * F[i][cc]);
          okc = okc && (!scan_on || ((mag >= kRegularMin) && (mag <= kRegularMax) && zbits[cc] == 0u));
        }
      const bool wave_okc = __all(okc);
      if (lane == 0) sFlag[NW + wave] = wave_okc ? 1 : 0;
      __syncthreads();  // B1b
      int cv = 1;
#pragma unroll
      for (int w = 0; w < NW; ++w) cv &= sFlag[NW + w];
      canchor = uniform32(cv) != 0;
    }
    if (canchor) {
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) {
        bpre[cc] = gpre[cc];
        gbs[cc] = gch[cc];
      }
    }
    const int rb0 = r0 % 16;  // this wave's first row inside its block
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int r = r0 + i;
      const float rq = a.scale * srq[r];
      float qv[CPT], lq[CPT], lk[CPT];
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) {
        // a zero at or before row i among this wave's rows
        const bool zb = (zbits[cc] & ((2u << i) - 1u)) != 0;
        const float ft = gpre[cc] * (zb ? 0.f : F[i][cc]);  // D(r <- chunk start)
        const float fb = zb ? F[i][cc] : bpre[cc] * F[i][cc];  // restarted, from the anchor
        const float mag = fabsf(fb);
        ok = ok && (!scan_on || ((mag >= kRegularMin) && (mag <= kRegularMax)));
        const float rinv = __builtin_amdgcn_rcpf(fb);
        qv[cc] = xq[i][cc] * ft * rq;     // Qt'
        lq[cc] = xq[i][cc] * fb;          // Lq
        lk[cc] = xk[i][cc] * fb;          // Lk
        kt[i][cc] = xk[i][cc] * ft;       // Kt / rk
        xk[i][cc] = xk[i][cc] * rinv;     // Rk
        // Kh / rk (regular chunks): zero while a zero of the block follows
        kh[i][cc] = (bz[cc] >> (rb0 + i + 1)) != 0 ? 0.f : xk[i][cc] * gbs[cc];
      }
      if (scan_on) {
        store_run<Op, CPT>(gQ + r * DK + Op::template pos<DK>(c0ch), qv);
        store_run<Op, CPT>(sLk + r * LDK + c0ch, lk);
        store_run<Op, CPT>(sLq + r * LDK + c0ch, lq);
        store_run<Op, CPT>(sRk + r * LDK + c0ch, xk[i]);
      }
    }
    // E_IJ = T'_J prod_{J < b < I} T_b for every off-diagonal tile: block
    // J's total after its last zero (the suffix products of its rows are
    // taken relative to that) times the plain totals of the blocks between
    // (zero if one holds a zero gate); from the wave totals of waves
    // WPB*J .. WPB*I-1.  Into the X block (I, J), which holds nothing until
    // the off-diagonal levels of X are formed.
    if (NB > 1 && !canchor) {
      constexpr int NPR = NB * (NB - 1) / 2;
      for (int e = tid; e < NPR * DK; e += NT) {
        const int pr = e / DK, ch = e % DK;
        int I = 1;
        while (I * (I + 1) / 2 <= pr) ++I;
        const int J = pr - I * (I - 1) / 2;
        float v = 1.f;
        for (int w = WPB * J; w < WPB * I; ++w) {
          const float tw = sG[w * DK + ch];
          const bool zw = ZL && zmap[((w / WPB) * DK + ch) * WPB + w % WPB] != 0;
          v = (w < WPB * (J + 1)) ? (zw ? tw : v * tw) : (zw ? 0.f : v * tw);
        }
        x_blk<Cfg>(smem, I, J)[ch] = v;
      }
    }
    const bool wave_ok = __all(ok);
    bool anyz = false;
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) anyz = anyz || (ZL && scan_on && zbits[cc] != 0u);
    const bool wave_z = ZL && __any(anyz);
    if (lane == 0) {
      sFlag[wave] = wave_ok ? 1 : 0;
      sFlag[2 * NW + wave] = wave_z ? 1 : 0;
    }
  }
  __syncthreads();  // B2
  int votes = 1, zvotes = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    votes &= sFlag[w];
    zvotes |= sFlag[2 * NW + w];
  }
  const bool haszero = uniform32(zvotes) != 0;  // some gate of the chunk is exactly zero
  // in range with at most one zero per (block, channel): the MFMA form
  // applies (with the zero masks of tile_ap_z when a gate is exactly zero)
  const bool in_range = uniform32(votes) != 0;
  if constexpr (MODE == kFlagRegular) {
    // plain products: a chunk with a zero gate is out of range here
    if (tid == 0) a.irregular[h * a.maxc + c] = in_range ? kFlagRegular : kFlagRedo;
    if (!in_range) return;
  }
  (void)haszero;

  // ================= 3: A and P ================================================
  if (MODE == kFlagRegular || in_range) {
    // A tile (I, J) from its accumulator: rows r = 16I + 4lq + i, column
    // j = 16J + l16; the diagonal tile goes to the X block it seeds
    auto a_out = [&](const f32x4& acc_a, int I, int J) {
      const int j = 16 * J + l16;
      const float sj = srk[j];
      float* dst = (I == J) ? x_blk<Cfg>(smem, I, I) : a_blk<Cfg>(smem, I, J);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * I + 4 * lq + i;
        const float v = acc_a[i] * sbeta[r] * srk[r] * sj;
        dst[(4 * lq + i) * LDA + l16] = (I == J && j >= r) ? 0.f : v;
      }
    };
    // P' tile (I, J) from its accumulator: rows j = 16J + 4lq + i, column
    // r = 16I + l16, as P'[r][j]; zero above the diagonal
    auto p_vals = [&](const f32x4& acc_p, int I, int J) {
      const int r = 16 * I + l16;
      const float sr = a.scale * srq[r];
      f32x4 out;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = 16 * J + 4 * lq + i;
        out[i] = (J > I || (I == J && j > r)) ? 0.f : acc_p[i] * sr * srk[j];
      }
      return out;
    };
    auto tile = [&](f32x4& acc_a, f32x4& acc_p, int I, int J) {
      if constexpr (MODE == kFlagRedo) {
        const uint8_t* zi = zmap + I * DK * Cfg::WPB;
        const uint8_t* zj = zmap + J * DK * Cfg::WPB;
        if (I > J) {
          tile_ap_z<Cfg>(acc_a, acc_p, sLk + 16 * I * LDK, sLq + 16 * I * LDK, sRk + 16 * J * LDK,
                         x_blk<Cfg>(smem, I, J), zi, zj, 0, lane);
        } else {
          tile_ap_z<Cfg>(acc_a, acc_p, sLk + 16 * I * LDK, sLq + 16 * I * LDK, sRk + 16 * J * LDK,
                         nullptr, zi, zj, 1, lane);
          tile_ap_z<Cfg>(acc_a, acc_p, sLk + 16 * I * LDK, sLq + 16 * I * LDK, sRk + 16 * J * LDK,
                         nullptr, zi, zj, 2, lane);
        }
        return;
      }
      tile_ap<Cfg>(acc_a, acc_p, sLk + 16 * I * LDK, sLq + 16 * I * LDK, sRk + 16 * J * LDK,
                   (I > J && !canchor) ? x_blk<Cfg>(smem, I, J) : nullptr, lane);
    };
    if constexpr (ES == 2 && NB % 2 == 0) {
      // one task per (I, column pair J = 2p, 2p+1): in storage order the two
      // tiles' P' values of a lane are adjacent (16 bytes, 64 per row)
      constexpr int NPAIR = NB * NB / 2;
      constexpr int NU = (NPAIR + NW - 1) / NW;
#pragma unroll 1
      for (int u = 0; u < NU; ++u) {
        int tt = wave + NW * u;
        if (tt < NPAIR) {
          // C = 64: tasks ordered so that each SIMD (waves w, w + 4) gets 2 or 3 tiles
          if constexpr (NB == 4) tt = (0x31507642u >> (4 * tt)) & 7u;
          const int I = tt / (NB / 2), J0 = 2 * (tt % (NB / 2)), J1 = J0 + 1;
          f32x4 ap0 = {0.f, 0.f, 0.f, 0.f}, ap1 = {0.f, 0.f, 0.f, 0.f};
          if (J0 <= I) {
            f32x4 aa = {0.f, 0.f, 0.f, 0.f};
            tile(aa, ap0, I, J0);
            a_out(aa, I, J0);
          }
          if (J1 <= I) {
            f32x4 aa = {0.f, 0.f, 0.f, 0.f};
            tile(aa, ap1, I, J1);
            a_out(aa, I, J1);
          }
          const f32x4 o0 = p_vals(ap0, I, J0), o1 = p_vals(ap1, I, J1);
          bf16x8 y;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            y[i] = Op::cvt(o0[i]);
            y[4 + i] = Op::cvt(o1[i]);
          }
          const int pr = 16 * I + l16, pp = Op::template pos<C>(16 * J0 + 4 * lq);
          if (!tri_dead(C, TES, pr, pp)) *reinterpret_cast<bf16x8*>(gP + tri_row(C, TES, pr) + pp) = y;
        }
      }
    } else {
      constexpr int NPT = NB * (NB + 1) / 2;  // lower blocks (A and P together)
      constexpr int NZ = NB * (NB - 1) / 2;   // zero blocks of P above the diagonal
      constexpr int NTILE = NPT + NZ;
      constexpr int NU = (NTILE + NW - 1) / NW;
#pragma unroll 1
      for (int u = 0; u < NU; ++u) {
        const int tt = wave + NW * u;
        if (tt < NPT) {
          int I, J;
          lower_block(tt, I, J);
          f32x4 acc_a = {0.f, 0.f, 0.f, 0.f}, acc_p = {0.f, 0.f, 0.f, 0.f};
          tile(acc_a, acc_p, I, J);
          a_out(acc_a, I, J);
          const int pr = 16 * I + l16, pp = Op::template pos<C>(16 * J + 4 * lq);
          if (!tri_dead(C, TES, pr, pp)) Op::store4(gP + tri_row(C, TES, pr) + pp, p_vals(acc_p, I, J));
        } else if (tt < NTILE) {
          int I, J;
          lower_block(tt - NPT, J, I);  // J > I: a block above the diagonal
          J += 1;
          const int pr = 16 * I + l16, pp = Op::template pos<C>(16 * J + 4 * lq);
          if (!tri_dead(C, TES, pr, pp)) Op::store4(gP + tri_row(C, TES, pr) + pp, f32x4{0.f, 0.f, 0.f, 0.f});
        }
      }
    }
  } else {
    direct_ap<Cfg, G>(a.q, a.k, a.alpha, ckda, (t0 * Hk + hk) * static_cast<int64_t>(DK), Hk * DK,
                      (t0 * H + h) * static_cast<int64_t>(DK), H * DK, L, a.scale, gP, smem, tid);
    // Kh from suffix products of the gates (no division)
    if (scan_on) {
      // the direct path left the gates in LDS (1 past the end)
      const int64_t qk_off = (t0 * Hk + hk) * static_cast<int64_t>(DK);
      const float* sgate = reinterpret_cast<const float*>(smem + Cfg::O_DGATE);
#pragma unroll
      for (int cc = 0; cc < CPT; ++cc) {
        float suf = gsuf[cc];
#pragma unroll
        for (int i = RPW - 1; i >= 0; --i) {
          const int r = r0 + i;
          // kh = k * prod_{s>r} alpha_s ; xk was overwritten by Rk, so reload k
          const float kr = (r < L) ? IO::load(static_cast<const typename IO::storage*>(a.k),
                                              qk_off + static_cast<int64_t>(r) * Hk * DK + c0ch + cc)
                                   : 0.f;
          kh[i][cc] = kr * suf;
          suf *= sgate[r * DK + c0ch + cc];
        }
      }
    }
  }
  __syncthreads();  // B3

  // ================= 4: Kt'^T, Kh'^T; diagonal blocks of X ======================
  if (scan_on) {
    float wsc[RPW], rks[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      rks[i] = srk[r0 + i];
      wsc[i] = sbeta[r0 + i] * rks[i];
    }
#pragma unroll
    for (int cc = 0; cc < CPT; ++cc) {
      float ktv[RPW], khv[RPW];
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        ktv[i] = kt[i][cc] * wsc[i];
        khv[i] = kh[i][cc] * rks[i];
      }
      store_run<Op, RPW>(sKtT + (c0ch + cc) * LDC + r0, ktv);
      store_run_pos<Op, RPW, C>(sKhT + (c0ch + cc) * Cfg::LDH, r0, khv);
    }
  }
  if (wave < NB && lane < 16) {
    // forward substitution for column j of the diagonal block (I, I):
    // x_i = delta_ij - sum_{m<i} A(i, m) x_m.  Every lane reads the same row
    // of A (a broadcast); X overwrites A only after the last read.
    const int j = lane;
    float* blkI = x_blk<Cfg>(smem, wave, wave);
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
      for (int g = 0; 4 * g < i; ++g) {
        const f32x4 ar = *reinterpret_cast<const f32x4*>(blkI + i * LDA + 4 * g);
#pragma unroll
        for (int mm = 0; mm < 4; ++mm)
          if (4 * g + mm < i) acc -= ar[mm] * x[4 * g + mm];
      }
      x[i] = acc;
    }
    wave_lds_sync();
#pragma unroll
    for (int i = 0; i < 16; ++i) blkI[i * LDA + j] = x[i];
  }
  __syncthreads();  // B4
  {
    // Kh'^T out row by row, 16 bytes per thread: whole lines per wave
    // instead of a few bytes in each of 64 rows
    constexpr int VE = 16 / ES, RV = C / VE, NV = DK * RV;
    for (int e = tid; e < NV; e += NT) {
      const int row = e / RV, col = (e % RV) * VE;
      *reinterpret_cast<uint4*>(gK + row * C + col) =
          *reinterpret_cast<const uint4*>(sKhT + row * Cfg::LDH + col);
    }
  }

  // ================= 5: off-diagonal blocks of X ===============================
  for (int d = 1; d < NB; ++d) {
    for (int J = wave; J + d < NB; J += NW) {
      const int I = J + d;
      f32x4 tacc = {0.f, 0.f, 0.f, 0.f};
      for (int M = J; M < I; ++M) {
        const float* am = a_blk<Cfg>(smem, I, M);
        const float* xm = x_blk<Cfg>(smem, M, J);
        float av[4], xv[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          av[kk] = am[l16 * LDA + 4 * kk + lq];
          xv[kk] = xm[(4 * kk + lq) * LDA + l16];
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) tacc = mfma_f32(av[kk], xv[kk], tacc);
      }
      float* ts = sTS + wave * Cfg::BLKF;
#pragma unroll
      for (int i = 0; i < 4; ++i) ts[(4 * lq + i) * LDA + l16] = tacc[i];
      wave_lds_sync();
      const float* xi = x_blk<Cfg>(smem, I, I);
      float xa[4], tb[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        xa[kk] = xi[l16 * LDA + 4 * kk + lq];
        tb[kk] = ts[(4 * kk + lq) * LDA + l16];
      }
      f32x4 xacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) xacc = mfma_f32(xa[kk], tb[kk], xacc);
      float* xo = x_blk<Cfg>(smem, I, J);
#pragma unroll
      for (int i = 0; i < 4; ++i) xo[(4 * lq + i) * LDA + l16] = -xacc[i];
    }
    __syncthreads();
  }

  // ================= 6: X' out, X operand copy, -W out ==========================
  {
    // 4-element groups of the full C x C matrix (zeros above the block diagonal)
    constexpr int NQ = C * C / 4;
    for (int e = tid; e < NQ; e += NT) {
      const int r = e / (C / 4), j = 4 * (e % (C / 4));
      const int I = r / 16, J = j / 16;
      f32x4 xv = {0.f, 0.f, 0.f, 0.f};
      if (J <= I) xv = *reinterpret_cast<const f32x4*>(x_blk<Cfg>(smem, I, J) + (r % 16) * LDA + j % 16);
      Op::store4(sXb + r * LDC + j, xv);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(sbeta + j);
      const int xp = Op::template pos<C>(j);
      if (!tri_dead(C, TES, r, xp)) Op::store4(gX + tri_row(C, TES, r) + xp, xv * bv);
      if (a.xout)  // X itself in fp32, for the backward
        *reinterpret_cast<f32x4*>(a.xout + ((static_cast<int64_t>(h) * a.maxc + c) * C + r) * C + j) = xv;
    }
  }
  __syncthreads();
  {
    constexpr int NWT = (DK / 16) * (C / 16);
    if constexpr (ES == 2 && DK % 32 == 0) {
      // tiles mc = 2s, 2s+1 of one row block together: in storage order their
      // four values per lane are adjacent (16 bytes), 64 bytes per row
      constexpr int NWP = NWT / 2;
      constexpr int NU = (NWP + NW - 1) / NW;
#pragma unroll 1
      for (int u = 0; u < NU; ++u) {
        const int tt = wave + NW * u;
        if (tt < NWP) {
          const int sp = tt / (C / 16), nr = tt % (C / 16);
          f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
          Op::template mmaK<C>(acc0, sKtT + 32 * sp * LDC, LDC, sXb + 16 * nr * LDC, LDC, lane);
          Op::template mmaK<C>(acc1, sKtT + (32 * sp + 16) * LDC, LDC, sXb + 16 * nr * LDC, LDC, lane);
          // rows c = 32sp + 16h + 4lq + i, column r = 16nr + l16: W[r][c]
          bf16x8 y;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            y[i] = Op::cvt(-acc0[i]);
            y[4 + i] = Op::cvt(-acc1[i]);
          }
          *reinterpret_cast<bf16x8*>(gW + (16 * nr + l16) * DK + Op::template pos<DK>(32 * sp + 4 * lq)) = y;
        }
      }
    } else {
      constexpr int NU = (NWT + NW - 1) / NW;
#pragma unroll 1
      for (int u = 0; u < NU; ++u) {
        const int tt = wave + NW * u;
        if (tt < NWT) {
          const int mc = tt / (C / 16), nr = tt % (C / 16);
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          Op::template mmaK<C>(acc, sKtT + 16 * mc * LDC, LDC, sXb + 16 * nr * LDC, LDC, lane);
          // rows c = 16mc + 4lq + i, column r = 16nr + l16: W[r][c]
          Op::store4(gW + (16 * nr + l16) * DK + Op::template pos<DK>(16 * mc + 4 * lq), -acc);
        }
      }
    }
  }
}

// The transform pass: one workgroup per (chunk, head); workgroups of one
// chunk and consecutive heads are adjacent.  In a batch the chunks go by
// position in their sequence from last to first (every sequence and head of
// one position together), so the blocks written last, which the last-level
// cache still holds when the state pass starts, are the first chunks of
// every chain: the ones the state pass reads first.  Packed sequences keep
// the order of their chunk slots.
template <class Cfg, class G>
__global__ __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(4))) void prep_kernel(FwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int H = a.H;
  const int b = static_cast<int>(blockIdx.x);
  if (a.cu_seqlens) {
    prep_chunk<Cfg, G, kFlagRegular>(a, b / H, b % H, smem);
  } else {
    const int per = a.B * H;  // workgroups per chunk position
    const int i = a.nc - 1 - b / per, n = (b % per) / H;
    prep_chunk<Cfg, G, kFlagRegular>(a, n * a.nc + i, b % H, smem);
  }
}

// The chunks the first launch flagged (exact zero gates, running products
// outside [2^-100, 2^10]), redone in the masked MFMA form or by direct
// products.  The flagged slots are dealt out evenly: each workgroup scans
// every flag (16 per thread and step; prefix sums over the lanes and the
// waves give each flagged slot its rank among them) and takes the slots of
// rank b, b + G, b + 2G, ... (G workgroups), which it then redoes in turn;
// with no flag set it ends after the scan.  The launcher sizes G so that no workgroup gets
// more than NT slots.
template <class Cfg, class G>
__global__ __launch_bounds__(Cfg::NT) __attribute__((amdgpu_waves_per_eu(2))) void prep_redo_kernel(
    FwdArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int NW = Cfg::NW, NT = Cfg::NT;
  const int total = a.maxc * a.H;
  const int grid = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  int* list = reinterpret_cast<int*>(smem);  // [NT] this workgroup's slots (scan only)
  int* wcnt = list + NT;                     // [NW] flagged slots per wave, this step
  constexpr int SPT = 16;                    // flags per thread and step (four 16-byte loads)
  int seen = 0;                              // flagged slots before this step
  for (int s0 = 0; s0 < total; s0 += NT * SPT) {
    const int base = s0 + SPT * tid;
    int fl[SPT];
#pragma unroll
    for (int u = 0; u < SPT / 4; ++u) {
      // the flag array is padded to 256 bytes, so a load that starts below
      // `total` stays inside it
      const int4 v = base + 4 * u < total ? *reinterpret_cast<const int4*>(a.irregular + base + 4 * u)
                                          : make_int4(0, 0, 0, 0);
      fl[4 * u] = v.x;
      fl[4 * u + 1] = v.y;
      fl[4 * u + 2] = v.z;
      fl[4 * u + 3] = v.w;
    }
    int cnt = 0;
#pragma unroll
    for (int u = 0; u < SPT; ++u) cnt += (base + u < total && fl[u] != kFlagRegular) ? 1 : 0;
    // ranks: prefix of the counts over the lanes, then over the waves
    int x = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wcnt[wave] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int cw = wcnt[w];
      before += w < wave ? cw : 0;
      all += cw;
    }
    int rank = seen + before + x - cnt;
#pragma unroll
    for (int u = 0; u < SPT; ++u) {
      if (base + u < total && fl[u] != kFlagRegular) {
        if (rank % grid == b && rank / grid < NT) list[rank / grid] = base + u;
        ++rank;
      }
    }
    seen += uniform32(all);
    __syncthreads();
  }
  const int items = seen > b ? (seen - b + grid - 1) / grid : 0;
  const int mine = tid < items ? list[tid] : 0;
  __syncthreads();  // the list is read; LDS goes to the chunks
  int* bcast = reinterpret_cast<int*>(smem + Cfg::O_BC);
  for (int i = 0; i < items && i < NT; ++i) {
    if (tid == i) *bcast = mine;
    __syncthreads();
    const int idx = uniform32(*bcast);
    // threadIdx.x through an opaque move: the chunk's lane-dependent
    // addresses are then formed here, not hoisted into the kernel's
    // prologue, where with no chunk flagged they would only cost spills
    int tid_o;
    asm volatile("v_mov_b32 %0, %1" : "=v"(tid_o) : "v"(static_cast<int>(threadIdx.x)));
    prep_chunk<Cfg, G, kFlagRedo>(a, idx % a.maxc, idx / a.maxc, smem, tid_o);
    __syncthreads();
  }
}


// Chunk map of a packed batch: first[n] = sum over m < n of ceil(len_m / C),
// first[N] = the chunk count, chunk_seq[c] = the sequence owning chunk c (or
// -1 for c >= first[N]), seq_order = the sequences by chunk count, most
// first (the order the state pass starts their chains in).  One workgroup; a
// block-wide scan per 1024 sequences.
__global__ __launch_bounds__(1024) void chunk_map_kernel(const int32_t* cu, int32_t N, int32_t C,
                                                         int32_t maxc, int32_t* first,
                                                         int32_t* chunk_seq, int32_t* seq_order,
                                                         int2* geo) {
  __shared__ int32_t part[1024];
  __shared__ int32_t carry_s;
  const int tid = threadIdx.x;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  for (int base = 0; base < N; base += 1024) {
    const int n = base + tid;
    int cnt = 0;
    if (n < N) {
      const int len = cu[n + 1] - cu[n];
      cnt = len > 0 ? (len + C - 1) / C : 0;
    }
    part[tid] = cnt;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
      const int add = tid >= off ? part[tid - off] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    const int carry = carry_s;
    if (n < N) first[n] = carry + part[tid] - cnt;
    __syncthreads();
    if (tid == 1023) carry_s = carry + part[1023];
    __syncthreads();
  }
  if (tid == 0) first[N] = carry_s;
  __syncthreads();  // first[] complete and visible to the workgroup
  const int total = carry_s;
  for (int c = tid; c < maxc; c += 1024) {
    int owner = -1;
    if (c < total) {
      int lo = 0, hi = N - 1;  // last n with first[n] <= c
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (first[mid] <= c) lo = mid; else hi = mid - 1;
      }
      owner = lo;
    }
    chunk_seq[c] = owner;
    int2 gc = make_int2(0, 0);
    if (owner >= 0) {
      gc.x = cu[owner] + (c - first[owner]) * C;
      gc.y = cu[owner + 1] - gc.x < C ? cu[owner + 1] - gc.x : C;
    }
    geo[c] = gc;
  }
  // sequences by chunk count, most first (ties by index): rank of n among
  // all sequences.  Past kOrderMax sequences the quadratic ranking is not
  // worth its time and the order stays the identity.
  constexpr int kOrderMax = 4096;
  for (int n = tid; n < N; n += 1024) {
    if (N > kOrderMax) {
      seq_order[n] = n;
      continue;
    }
    const int cn = first[n + 1] - first[n];
    int rank = 0;
    for (int j = 0; j < N; ++j) {
      const int cj = first[j + 1] - first[j];
      rank += (cj > cn) || (cj == cn && j < n);
    }
    seq_order[rank] = n;
  }
}

template <class Cfg, class G>
launch_result launch_cfg(const FwdArgs& a, hipStream_t stream) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&prep_kernel<Cfg, G>),
      hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS_BYTES);
  static const hipError_t attr_d = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&prep_redo_kernel<Cfg, G>),
      hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS_BYTES);
  if (attr != hipSuccess) return attr;
  if (attr_d != hipSuccess) return attr_d;
  const int64_t blocks = static_cast<int64_t>(a.maxc) * a.H;
  hipLaunchKernelGGL((prep_kernel<Cfg, G>), dim3(static_cast<unsigned>(blocks)), dim3(Cfg::NT),
                     Cfg::LDS_BYTES, stream, a);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one workgroup per CU, more when that would leave one more than NT slots
  int64_t grid = (blocks + Cfg::NT - 1) / Cfg::NT;
  if (grid < kRedoGrid) grid = blocks < kRedoGrid ? blocks : kRedoGrid;
  hipLaunchKernelGGL((prep_redo_kernel<Cfg, G>), dim3(static_cast<unsigned>(grid)), dim3(Cfg::NT),
                     Cfg::LDS_BYTES, stream, a);
  return hipGetLastError();
}

using launch_fn = launch_result (*)(const FwdArgs&, hipStream_t);

struct Entry {
  int chunk, dk, dtype;
  launch_fn fn[3];  // by ckda_gate_input_t
};

template <class Op, class IO, int C, int D>
constexpr Entry entry(int dtype) {
  using Cfg = PrepCfg<Op, IO, C, D>;
  return Entry{C, D, dtype,
               {&launch_cfg<Cfg, gate_f32>, &launch_cfg<Cfg, gate_logit_f32>,
                &launch_cfg<Cfg, gate_logit_bf16>}};
}

const Entry kEntries[] = {
    entry<OpBF16, io_bf16, 64, 128>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 32, 128>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 16, 128>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 64, 64>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 32, 64>(CKDA_DTYPE_BF16),
    entry<OpBF16, io_bf16, 16, 64>(CKDA_DTYPE_BF16),
    entry<OpF32, io_f32, 16, 16>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 32, 16>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 64, 16>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 16, 32>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 32, 32>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 64, 32>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 16, 64>(CKDA_DTYPE_F32),
    entry<OpF32, io_f32, 32, 64>(CKDA_DTYPE_F32),
};

const Entry* find(int32_t chunk, int32_t dk, int32_t dtype) {
  for (const Entry& e : kEntries)
    if (e.chunk == chunk && e.dk == dk && e.dtype == dtype) return &e;
  return nullptr;
}

}  // namespace

bool prep_supported(int32_t chunk, int32_t dk, int32_t io_dtype) {
  return find(chunk, dk, io_dtype) != nullptr;
}

launch_result launch_prep(const FwdArgs& a, int32_t io_dtype, hipStream_t stream) {
  const Entry* e = find(a.chunk, a.dk, io_dtype);
  if (!e) return hipErrorInvalidValue;
  if (a.gate_input < 0 || a.gate_input > 2) return hipErrorInvalidValue;
  if (static_cast<int64_t>(a.maxc) * a.H == 0) return hipSuccess;
  return e->fn[a.gate_input](a, stream);
}

launch_result launch_chunk_map(const FwdArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(1024), 0, stream, a.cu_seqlens, a.num_seqs,
                     a.chunk, a.maxc, a.first, a.chunk_seq, a.seq_order, a.chunk_geo);
  return hipGetLastError();
}

}  // namespace ckda
