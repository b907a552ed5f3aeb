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
//      entry state, and writing no output
//   2. bwd_state_kernel: per (sequence, head, dv tile), chunks in reverse:
//      dU and dS1 of every chunk to the workspace, dv, dh0
//   3. bwd_intra_kernel: per (chunk, head), the ratio form: dq, dk, dalpha,
//      dbeta; flags chunks it cannot take
//   4. bwd_token_kernel: the flagged chunks, token by token
// All arithmetic is fp32 (gradients are fp32 buffers); the forward's blocks
// are read in their storage type.
#include "mfma_ops.h"

namespace ckda {


namespace {

constexpr float kRegMin = 0x1p-100f, kRegMax = 0x1p+10f;
constexpr int kNT = 256;

// tokens of chunk slot c: sequence n, first token t0, length L (n < 0: unused)
struct Geo {
  int64_t t0;
  int L, n;
};
__device__ __forceinline__ Geo geo_of(const FwdArgs& a, int c) {
  Geo g{0, 0, -1};
  const int C = a.chunk;
  if (a.cu_seqlens) {
    const int n = a.chunk_seq[c];
    if (n < 0) return g;
    const int i = c - a.first[n];
    const int64_t s0 = a.cu_seqlens[n], s1 = a.cu_seqlens[n + 1];
    g.n = n;
    g.t0 = s0 + static_cast<int64_t>(i) * C;
    g.L = static_cast<int>((s1 - g.t0) < C ? (s1 - g.t0) : C);
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

// ---------------------------------------------------------------- 2: state
// One workgroup per (sequence, head, tile of DVB value columns); the columns
// of the state adjoint are independent, so no tile needs another's.
template <class IO>
__global__ __launch_bounds__(kNT) void bwd_state_kernel(BwdArgs b) {
  using ST = typename IO::storage;
  const FwdArgs& a = b.f;
  const int C = a.chunk, dk = a.dk, dv = a.dv, H = a.H;
  const int DVB = dv < 32 ? dv : 32, ntile = dv / DVB;
  const int64_t wg = blockIdx.x;
  const int tile = static_cast<int>(wg % ntile);
  const int64_t pair = wg / ntile;
  const int n = static_cast<int>(pair / H), h = static_cast<int>(pair % H);
  const int dv0 = tile * DVB;
  int64_t s0, s1;
  int c_begin, nch;
  if (a.cu_seqlens) {
    s0 = a.cu_seqlens[n];
    s1 = a.cu_seqlens[n + 1];
    c_begin = a.first[n];
    nch = a.first[n + 1] - c_begin;
  } else {
    s0 = static_cast<int64_t>(n) * a.T;
    s1 = s0 + a.T;
    c_begin = n * a.nc;
    nch = a.nc;
  }
  extern __shared__ float sm[];
  float* sdO = sm;               // [C][DVB]
  float* sdS = sdO + C * DVB;    // [dk][DVB] adjoint at the chunk's exit
  float* sdU = sdS + dk * DVB;   // [C][DVB]
  float* sdS0 = sdU + C * DVB;   // [dk][DVB]
  const int tid = threadIdx.x;
  const int64_t st = (static_cast<int64_t>(n) * H + h) * dk * dv + dv0;
  for (int e = tid; e < dk * DVB; e += kNT)
    sdS[e] = b.dht ? b.dht[st + static_cast<int64_t>(e / DVB) * dv + e % DVB] : 0.f;
  const int es = static_cast<int>(sizeof(ST));
  for (int i = nch - 1; i >= 0; --i) {
    const int c = c_begin + i;
    const int64_t t0 = s0 + static_cast<int64_t>(i) * C;
    const int L = static_cast<int>((s1 - t0) < C ? (s1 - t0) : C);
    const int64_t slot = static_cast<int64_t>(h) * a.maxc + c;
    const unsigned char* blk = a.blocks + slot * a.blk_bytes;
    const ST* bX = reinterpret_cast<const ST*>(blk);
    const ST* bW = bX + C * C;
    const ST* bQ = bW + C * dk;
    const ST* bP = bQ + C * dk;
    const ST* bK = bP + C * C;
    const float* bg = reinterpret_cast<const float*>(blk + blk_g_byte(C, dk, es));
    __syncthreads();
    for (int e = tid; e < C * DVB; e += kNT) {
      const int r = e / DVB, j = e % DVB;
      sdO[e] = r < L ? IO::load(static_cast<const ST*>(b.dout), ((t0 + r) * H + h) * dv + dv0 + j) : 0.f;
    }
    for (int e = tid; e < dk * DVB; e += kNT)
      b.dS[(slot * dk + e / DVB) * dv + dv0 + e % DVB] = sdS[e];
    __syncthreads();
    // dU = P'^T dO + Kh' dS1   (P' = scale P, lower; Kh' = Kh)
    for (int e = tid; e < C * DVB; e += kNT) {
      const int r = e / DVB, j = e % DVB;
      float acc = 0.f;
      for (int rr = r; rr < C; ++rr) acc += blk_at<IO>(bP, rr, r, C) * sdO[rr * DVB + j];
      for (int cc = 0; cc < dk; ++cc) acc += blk_at<IO>(bK, cc, r, C) * sdS[cc * DVB + j];
      sdU[e] = acc;
    }
    __syncthreads();
    for (int e = tid; e < C * DVB; e += kNT) {
      const int r = e / DVB, j = e % DVB;
      b.dU[(slot * C + r) * dv + dv0 + j] = sdU[e];
      if (r < L) {  // dV = X'^T dU   (X' = Y, lower)
        float acc = 0.f;
        for (int rr = r; rr < C; ++rr) acc += blk_at<IO>(bX, rr, r, C) * sdU[rr * DVB + j];
        b.dv[((t0 + r) * H + h) * dv + dv0 + j] = acc;
      }
    }
    // dS0 = Qt'^T dO + Diag(g) dS1 + W'^T dU   (W' = -W as stored)
    for (int e = tid; e < dk * DVB; e += kNT) {
      const int cc = e / DVB, j = e % DVB;
      float acc = bg[cc] * sdS[e];
      for (int r = 0; r < C; ++r)
        acc += blk_at<IO>(bQ, r, cc, dk) * sdO[r * DVB + j] + blk_at<IO>(bW, r, cc, dk) * sdU[r * DVB + j];
      sdS0[e] = acc;
    }
    __syncthreads();
    for (int e = tid; e < dk * DVB; e += kNT) sdS[e] = sdS0[e];
  }
  __syncthreads();
  if (b.dh0)
    for (int e = tid; e < dk * DVB; e += kNT) b.dh0[st + static_cast<int64_t>(e / DVB) * dv + e % DVB] = sdS[e];
}

// ---------------------------------------------------------------- 3: intra
// One (chunk, head) at a time per workgroup, items b, b + grid, ...
// C x C matrices in LDS; C x dk and C x dv intermediates in the workgroup's
// slice of the scratch.
template <class IO>
__global__ __launch_bounds__(kNT) void bwd_intra_kernel(BwdArgs b) {
  using ST = typename IO::storage;
  const FwdArgs& a = b.f;
  const int C = a.chunk, dk = a.dk, dv = a.dv, H = a.H;
  const int total = a.maxc * H;
  const bool l2 = a.use_l2norm != 0;
  const float scale = a.scale;
  const int SC = C * (dk > dv ? dk : dv);
  float* ws = b.scratch + static_cast<int64_t>(blockIdx.x) * 10 * SC;
  float *sF = ws, *sKt = ws + SC, *sQt = ws + 2 * SC, *sRk = ws + 3 * SC, *sZ = ws + 4 * SC,
        *sU = ws + 5 * SC, *sT1 = ws + 6 * SC, *sdq = ws + 7 * SC, *sdk = ws + 8 * SC,
        *sLam = ws + 9 * SC;
  extern __shared__ float sm[];
  float* lX = sm;               // [C][C] X
  float* ldY = lX + C * C;      // [C][C] dY -> dX -> dA -> dG
  float* lT = ldY + C * C;      // [C][C] dX X^T
  float* ldP = lT + C * C;      // [C][C] dP
  float* lbeta = ldP + C * C;   // [C]
  float* lrq = lbeta + C;       // [C]
  float* lrk = lrq + C;         // [C]
  float* ldb = lrk + C;         // [C]
  float* lg = ldb + C;          // [dk]
  int* lflag = reinterpret_cast<int*>(lg + dk);
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
    const float* S0 = a.hc + slot * dk * dv;
    const float* dS1 = b.dS + slot * dk * dv;
    const float* dU = b.dU + slot * C * dv;
    const float* X = a.xout + slot * C * C;
    // A: norms, beta, gate products, regularity
    if (tid == 0) *lflag = 0;
    for (int r = tid; r < C; r += kNT) {
      float sq = 0.f, sk = 0.f;
      if (r < L) {
        for (int cc = 0; cc < dk; ++cc) {
          const int64_t i = ((t0 + r) * H + h) * dk + cc;
          const float x = IO::load(q, i), y = IO::load(k, i);
          sq += x * x;
          sk += y * y;
        }
      }
      lrq[r] = l2 ? __fdiv_rn(1.f, __fsqrt_rn(sq + kL2Eps)) : 1.f;
      lrk[r] = l2 ? __fdiv_rn(1.f, __fsqrt_rn(sk + kL2Eps)) : 1.f;
      lbeta[r] = r < L ? beta[(t0 + r) * H + h] : 0.f;
      ldb[r] = 0.f;
    }
    __syncthreads();
    for (int cc = tid; cc < dk; cc += kNT) {
      float f = 1.f;
      bool ok = true;
      for (int r = 0; r < C; ++r) {
        f *= r < L ? alpha[((t0 + r) * H + h) * dk + cc] : 1.f;
        sF[r * dk + cc] = f;
        const float m = fabsf(f);
        ok = ok && m >= kRegMin && m <= kRegMax;
      }
      lg[cc] = f;
      if (!ok) *lflag = 1;
    }
    __syncthreads();
    const bool irregular = *lflag != 0;
    if (tid == 0) b.bflag[slot] = irregular ? 1 : 0;
    if (irregular) continue;
    // B: Kt, Qt, Rk; X to LDS
    for (int e = tid; e < C * dk; e += kNT) {
      const int r = e / dk, cc = e % dk;
      const int64_t i = ((t0 + r) * H + h) * dk + cc;
      const float qh = r < L ? IO::load(q, i) * lrq[r] : 0.f;
      const float kh = r < L ? IO::load(k, i) * lrk[r] : 0.f;
      const float f = sF[e];
      sKt[e] = kh * f;
      sQt[e] = qh * f;
      sRk[e] = kh / f;
    }
    for (int e = tid; e < C * C; e += kNT) lX[e] = X[e];
    __syncthreads();
    // C: Z = V - Kt S0
    for (int e = tid; e < C * dv; e += kNT) {
      const int r = e / dv, j = e % dv;
      float acc = r < L ? IO::load(v, ((t0 + r) * H + h) * dv + j) : 0.f;
      for (int cc = 0; cc < dk; ++cc) acc -= sKt[r * dk + cc] * S0[cc * dv + j];
      sZ[e] = acc;
    }
    __syncthreads();
    // D: U = Y Z (Y = X Diag(beta), lower), T1 = Y^T dU
    for (int e = tid; e < C * dv; e += kNT) {
      const int r = e / dv, j = e % dv;
      float u = 0.f, t = 0.f;
      for (int m = 0; m <= r; ++m) u += lX[r * C + m] * lbeta[m] * sZ[m * dv + j];
      for (int m = r; m < C; ++m) t += lX[m * C + r] * lbeta[r] * dU[m * dv + j];
      sU[e] = u;
      sT1[e] = t;
    }
    __syncthreads();
    // E: dY = dU Z^T (lower with the diagonal), dP = tril(scale dO U^T)
    for (int e = tid; e < C * C; e += kNT) {
      const int r = e / C, m = e % C;
      float y = 0.f, p = 0.f;
      if (m <= r) {
        for (int j = 0; j < dv; ++j) y += dU[r * dv + j] * sZ[m * dv + j];
        if (r < L)
          for (int j = 0; j < dv; ++j) p += IO::load(dO, ((t0 + r) * H + h) * dv + j) * sU[m * dv + j];
      }
      ldY[e] = y;
      ldP[e] = scale * p;
    }
    __syncthreads();
    // F: dbeta_j = sum_r X_rj dY_rj; dX = dY Diag(beta)
    for (int j = tid; j < C; j += kNT) {
      float s = 0.f;
      for (int r = j; r < C; ++r) s += lX[r * C + j] * ldY[r * C + j];
      ldb[j] = s;
    }
    __syncthreads();
    for (int e = tid; e < C * C; e += kNT) ldY[e] *= lbeta[e % C];
    __syncthreads();
    // G: T = dX X^T
    for (int e = tid; e < C * C; e += kNT) {
      const int r = e / C, j = e % C;
      float s = 0.f;
      for (int m = 0; m < C; ++m) s += ldY[r * C + m] * lX[j * C + m];
      lT[e] = s;
    }
    __syncthreads();
    // H: dA = -X^T T, strictly lower
    for (int e = tid; e < C * C; e += kNT) {
      const int r = e / C, j = e % C;
      float s = 0.f;
      if (j < r)
        for (int m = 0; m < C; ++m) s -= lX[m * C + r] * lT[m * C + j];
      ldY[e] = s;
    }
    __syncthreads();
    // I: dbeta_r += sum_j dA_rj G_rj (G = Kt Rk^T); dG = Diag(beta) dA
    for (int r = tid; r < C; r += kNT) {
      float s = 0.f;
      for (int j = 0; j < r; ++j) {
        float gg = 0.f;
        for (int cc = 0; cc < dk; ++cc) gg += sKt[r * dk + cc] * sRk[j * dk + cc];
        s += ldY[r * C + j] * gg;
        ldY[r * C + j] *= lbeta[r];
      }
      ldb[r] += s;
    }
    __syncthreads();
    // J: per element (r, cc)
    for (int e = tid; e < C * dk; e += kNT) {
      const int r = e / dk, cc = e % dk;
      float dqt = 0.f, dkt = 0.f, dkh = 0.f, drk = 0.f;
      for (int j = 0; j < dv; ++j) {
        const float s0 = S0[cc * dv + j];
        if (r < L) dqt += IO::load(dO, ((t0 + r) * H + h) * dv + j) * s0;
        dkt -= sT1[r * dv + j] * s0;
        dkh += sU[r * dv + j] * dS1[cc * dv + j];
      }
      dqt *= scale;
      for (int m = 0; m <= r; ++m) dqt += ldP[r * C + m] * sRk[m * dk + cc];
      for (int m = 0; m < r; ++m) dkt += ldY[r * C + m] * sRk[m * dk + cc];
      for (int m = r + 1; m < C; ++m) drk += ldY[m * C + r] * sKt[m * dk + cc];
      for (int m = r; m < C; ++m) drk += ldP[m * C + r] * sQt[m * dk + cc];
      drk += lg[cc] * dkh;
      const float f = sF[e];
      sdk[e] = dkt * f + drk / f;
      sdq[e] = dqt * f;
      sLam[e] = dkt * sKt[e] + dqt * sQt[e] - drk * sRk[e];
      sZ[e] = dkh * sRk[e];  // Z is no longer needed: dg terms per row
    }
    __syncthreads();
    // K: dalpha per channel (reverse running sums of Lam, divided by alpha)
    for (int cc = tid; cc < dk; cc += kNT) {
      float dg = 0.f;
      for (int j = 0; j < dv; ++j) dg += dS1[cc * dv + j] * S0[cc * dv + j];
      for (int r = 0; r < C; ++r) dg += sZ[r * dk + cc];
      float acc = dg * lg[cc];
      for (int r = C - 1; r >= 0; --r) {
        acc += sLam[r * dk + cc];
        if (r < L) {
          const int64_t i = ((t0 + r) * H + h) * dk + cc;
          b.dalpha[i] = acc / alpha[i];
        }
      }
    }
    // L: dq, dk through the norms; dbeta
    for (int r = tid; r < L; r += kNT) {
      float pq = 0.f, pk = 0.f;
      const int64_t base = ((t0 + r) * H + h) * dk;
      for (int cc = 0; cc < dk; ++cc) {
        pq += IO::load(q, base + cc) * lrq[r] * sdq[r * dk + cc];
        pk += IO::load(k, base + cc) * lrk[r] * sdk[r * dk + cc];
      }
      for (int cc = 0; cc < dk; ++cc) {
        const float qh = IO::load(q, base + cc) * lrq[r], kh = IO::load(k, base + cc) * lrk[r];
        b.dq[base + cc] = l2 ? lrq[r] * (sdq[r * dk + cc] - qh * pq) : sdq[r * dk + cc];
        b.dk[base + cc] = l2 ? lrk[r] * (sdk[r * dk + cc] - kh * pk) : sdk[r * dk + cc];
      }
      b.dbeta[(t0 + r) * H + h] = ldb[r];
    }
  }
}

// ---------------------------------------------------------------- 4: token
// Chunks the ratio form cannot take, token by token from the chunk's entry
// state: for token t (in reverse) the state before it is rebuilt from S0
// (t forward steps), then one reverse step of the recurrence's adjoint.
template <class IO>
__global__ __launch_bounds__(kNT) void bwd_token_kernel(BwdArgs b) {
  using ST = typename IO::storage;
  const FwdArgs& a = b.f;
  const int C = a.chunk, dk = a.dk, dv = a.dv, H = a.H;
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
    const float* S0 = a.hc + slot * dk * dv;
    __syncthreads();
    for (int i = tid; i < dk * dv; i += kNT) sG[(i / dv) * LD + i % dv] = b.dS[slot * dk * dv + i];
    for (int t = g.L - 1; t >= 0; --t) {
      // the state before token t
      __syncthreads();
      for (int i = tid; i < dk * dv; i += kNT) sS[(i / dv) * LD + i % dv] = S0[i];
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

template <class IO>
launch_result launch_io(const BwdArgs& b, hipStream_t stream) {
  const FwdArgs& a = b.f;
  const int C = a.chunk, dk = a.dk, dv = a.dv;
  const int DVB = dv < 32 ? dv : 32;
  const int64_t g2 = static_cast<int64_t>(a.num_seqs) * a.H * (dv / DVB);
  const size_t lds2 = sizeof(float) * (2 * C * DVB + 2 * dk * DVB);
  if (g2 > 0) {
    hipLaunchKernelGGL((bwd_state_kernel<IO>), dim3(static_cast<unsigned>(g2)), dim3(kNT), lds2, stream, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t total = static_cast<int64_t>(a.maxc) * a.H;
  if (total == 0) return hipSuccess;
  const size_t lds3 = sizeof(float) * (4 * C * C + 4 * C + dk) + sizeof(int);
  static const hipError_t attr3 = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&bwd_intra_kernel<IO>), hipFuncAttributeMaxDynamicSharedMemorySize, 64 * 1024 + 4096);
  if (attr3 != hipSuccess) return attr3;
  hipLaunchKernelGGL((bwd_intra_kernel<IO>), dim3(static_cast<unsigned>(b.grid3)), dim3(kNT), lds3, stream, b);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t lds4 = sizeof(float) * (2 * dk * (dv + 1) + 5 * dk + 4 * dv + kNT / 64);
  static const hipError_t attr4 = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&bwd_token_kernel<IO>), hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr4 != hipSuccess) return attr4;
  const int64_t g4 = total < 256 ? total : 256;
  hipLaunchKernelGGL((bwd_token_kernel<IO>), dim3(static_cast<unsigned>(g4)), dim3(kNT), lds4, stream, b);
  return hipGetLastError();
}

}  // namespace

int32_t bwd_grid3(int64_t total) { return static_cast<int32_t>(total < 1024 ? (total > 0 ? total : 1) : 1024); }

int64_t bwd_extra_bytes(int32_t H, int64_t maxc, int32_t C, int32_t dk, int32_t dv) {
  auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
  const int64_t hm = static_cast<int64_t>(H) * maxc;
  const int64_t SC = static_cast<int64_t>(C) * (dk > dv ? dk : dv);
  return up(4 * hm * C * C) + 2 * up(4 * hm * dk * dv) + up(4 * hm * C * dv) + up(4 * hm) +
         up(4 * static_cast<int64_t>(bwd_grid3(hm)) * 10 * SC);
}

void bwd_layout(BwdArgs& b, unsigned char* base) {
  const FwdArgs& a = b.f;
  auto up = [](int64_t x) { return (x + 255) & ~int64_t(255); };
  const int64_t hm = static_cast<int64_t>(a.H) * a.maxc;
  const int C = a.chunk, dk = a.dk, dv = a.dv;
  b.f.xout = reinterpret_cast<float*>(base);
  base += up(4 * hm * C * C);
  b.f.hc = reinterpret_cast<float*>(base);
  base += up(4 * hm * dk * dv);
  b.dS = reinterpret_cast<float*>(base);
  base += up(4 * hm * dk * dv);
  b.dU = reinterpret_cast<float*>(base);
  base += up(4 * hm * C * dv);
  b.bflag = reinterpret_cast<int32_t*>(base);
  base += up(4 * hm);
  b.scratch = reinterpret_cast<float*>(base);
  b.grid3 = bwd_grid3(hm);
}

launch_result launch_bwd_passes(const BwdArgs& b, int32_t io_dtype, hipStream_t stream) {
  return io_dtype == CKDA_DTYPE_BF16 ? launch_io<io_bf16>(b, stream) : launch_io<io_f32>(b, stream);
}

}  // namespace ckda
