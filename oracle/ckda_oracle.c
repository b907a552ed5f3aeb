/*
 * ckda_oracle.c -- fp64 sequential reference for the (Complex) Kimi Delta
 * Attention recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file.  Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg may use it.  It shares no code, header,
 * table or helper with the HIP library: it includes only the C standard
 * library and OpenMP.
 *
 * What it computes (written from the method's definition, not from any
 * kernel design):
 *
 *   The transition of a gated delta-rule layer is
 *       A_t = (I - beta_t k_t k_t^T) Diag(alpha_t)
 *   (picx.dev summary of the Complex KDA paper, section "Background",
 *   transition-matrix equation).  The state S is dk x dv; Diag(alpha_t)
 *   scales its rows, so alpha carries one gate per key channel.  The full
 *   update adds the rank-one write beta_t k_t v_t^T and the read-out uses
 *   the updated state:
 *       S_t = A_t S_{t-1} + beta_t k_t v_t^T,      o_t = scale * S_t^T q_t.
 *   (The summary prints only A_t; the write term and the read-out are the
 *   plainest reading consistent with it: a delta-rule write scaled by the
 *   same beta.)
 *
 *   CKDA allows alpha in [-1,1]^dk and beta in [0,2]; KDA keeps alpha
 *   positive (same summary, section "CKDA Definition").  The oracle does
 *   not check ranges: it computes the formula as written for any values.
 *
 *   Optional query/key L2 normalisation happens inside the op, before the
 *   recurrence, per (token, head) over the dk channels (dormouse review
 *   "RoPE into the KDA q/k path", section 2 "Where the L2 norm lives"):
 *       x_hat = x / sqrt(sum_c x_c^2 + eps).
 *
 * Evaluation order per token (the rank-one expansion of A_t S + beta k v^T):
 *   1. S[c,:] *= alpha[c]                  (Diag(alpha) S)
 *   2. w = S^T k                           (dv-vector)
 *   3. S += beta * k (v - w)^T             ((I - beta k k^T) X + beta k v^T)
 *   4. o = scale * S^T q
 * Expanding 3 with X = Diag(alpha) S_{t-1} gives X - beta k k^T X + beta k v^T,
 * which is exactly A_t S_{t-1} + beta k v^T.
 *
 * Layout (all row-major, last index fastest; tokens of all sequences packed):
 *   q, k, alpha : [T_total][H][dk]     v, o : [T_total][H][dv]
 *   beta        : [T_total][H]         h0, ht : [N][H][dk][dv]
 *   seq_start   : [N+1], sequence n owns tokens seq_start[n] .. seq_start[n+1]-1
 * A dense batch [B,T,H,...] is the packed layout with seq_start[n] = n*T.
 * Sequences and heads are independent; OpenMP runs them in parallel.  Each
 * (sequence, head) pair is computed by one thread in token order, so the
 * result does not depend on the thread count.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <omp.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1
#define ORACLE_NO_MEMORY 2

int32_t ckda_oracle_version(void) { return 1; }

void ckda_oracle_set_num_threads(int32_t n) {
  if (n > 0) omp_set_num_threads(n);
}

int32_t ckda_oracle_max_threads(void) { return (int32_t)omp_get_max_threads(); }

/* x_hat = x / sqrt(sum x^2 + eps), in place, over d values. */
static void l2_normalise(double* x, int32_t d, double eps) {
  double ss = 0.0;
  for (int32_t c = 0; c < d; ++c) ss += x[c] * x[c];
  const double n = sqrt(ss + eps);
  for (int32_t c = 0; c < d; ++c) x[c] /= n;
}

/* Row-wise L2 normalisation of a [rows][d] array (exported so the tests can
 * pin the normalisation step on its own). */
int32_t ckda_oracle_l2norm(int64_t rows, int32_t d, const double* x, double* y,
                           double eps) {
  if (rows < 0 || d <= 0 || (rows > 0 && (!x || !y))) return ORACLE_BAD_ARG;
  for (int64_t r = 0; r < rows; ++r) {
    memcpy(y + r * d, x + r * d, sizeof(double) * (size_t)d);
    l2_normalise(y + r * d, d, eps);
  }
  return ORACLE_OK;
}

/* Logistic sigmoid 1 / (1 + e^-x). */
static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

/*
 * Gates from pre-activation logits (picx.dev summary, section "CKDA
 * Definition": the implementation forms beta = 2 sigmoid(b) and the signed
 * gate 2 sigmoid(a) - 1).  ckda_range = 0 (KDA) takes the sigmoid itself for
 * both, the reading that keeps alpha in (0,1) and beta in (0,1).  alpha and a
 * hold n_alpha values, beta and b n_beta.
 */
int32_t ckda_oracle_gates(int64_t n_alpha, const double* a, int64_t n_beta,
                          const double* b, int32_t ckda_range, double* alpha,
                          double* beta) {
  if (n_alpha < 0 || n_beta < 0) return ORACLE_BAD_ARG;
  if ((n_alpha > 0 && (!a || !alpha)) || (n_beta > 0 && (!b || !beta)))
    return ORACLE_BAD_ARG;
  for (int64_t i = 0; i < n_alpha; ++i)
    alpha[i] = ckda_range ? 2.0 * sigmoid(a[i]) - 1.0 : sigmoid(a[i]);
  for (int64_t i = 0; i < n_beta; ++i)
    beta[i] = ckda_range ? 2.0 * sigmoid(b[i]) : sigmoid(b[i]);
  return ORACLE_OK;
}

/*
 * Gradients through the gate activation above: given dL/dalpha and dL/dbeta
 * (the gates' gradients, e.g. from ckda_oracle_bwd), dL/da = dL/dalpha *
 * dalpha/da and dL/db = dL/dbeta * dbeta/db, with the derivative of the
 * sigmoid s(x) = 1 / (1 + e^-x) being s(x) (1 - s(x)); the CKDA range doubles
 * it for both gates (alpha = 2 s(a) - 1, beta = 2 s(b)).
 */
int32_t ckda_oracle_gates_bwd(int64_t n_alpha, const double* a, const double* dalpha,
                              int64_t n_beta, const double* b, const double* dbeta,
                              int32_t ckda_range, double* da, double* db) {
  if (n_alpha < 0 || n_beta < 0) return ORACLE_BAD_ARG;
  if ((n_alpha > 0 && (!a || !dalpha || !da)) || (n_beta > 0 && (!b || !dbeta || !db)))
    return ORACLE_BAD_ARG;
  const double f = ckda_range ? 2.0 : 1.0;
  for (int64_t i = 0; i < n_alpha; ++i) {
    const double s = sigmoid(a[i]);
    da[i] = dalpha[i] * f * s * (1.0 - s);
  }
  for (int64_t i = 0; i < n_beta; ++i) {
    const double s = sigmoid(b[i]);
    db[i] = dbeta[i] * f * s * (1.0 - s);
  }
  return ORACLE_OK;
}

/* One sequence, one head: runs tokens [t0, t1) in order on the state S. */
static void run_head(int64_t t0, int64_t t1, int32_t h, int32_t H, int32_t dk,
                     int32_t dv, const double* q, const double* k,
                     const double* v, const double* alpha, const double* beta,
                     double* S, double* o, int32_t use_l2norm, double scale,
                     double eps, double* xq, double* xk, double* w) {
  for (int64_t t = t0; t < t1; ++t) {
    const int64_t qk_off = (t * H + h) * (int64_t)dk;
    const int64_t v_off = (t * H + h) * (int64_t)dv;
    memcpy(xq, q + qk_off, sizeof(double) * (size_t)dk);
    memcpy(xk, k + qk_off, sizeof(double) * (size_t)dk);
    if (use_l2norm) {
      l2_normalise(xq, dk, eps);
      l2_normalise(xk, dk, eps);
    }
    const double* a = alpha + qk_off;
    const double b = beta[t * H + h];
    const double* vt = v + v_off;

    /* 1. Diag(alpha) S: channel c of the key space scales row c. */
    for (int32_t c = 0; c < dk; ++c)
      for (int32_t j = 0; j < dv; ++j) S[c * dv + j] *= a[c];

    /* 2. w = S^T k. */
    for (int32_t j = 0; j < dv; ++j) w[j] = 0.0;
    for (int32_t c = 0; c < dk; ++c)
      for (int32_t j = 0; j < dv; ++j) w[j] += S[c * dv + j] * xk[c];

    /* 3. S += beta k (v - w)^T. */
    for (int32_t c = 0; c < dk; ++c) {
      const double bk = b * xk[c];
      for (int32_t j = 0; j < dv; ++j) S[c * dv + j] += bk * (vt[j] - w[j]);
    }

    /* 4. o = scale S^T q (read-out after the update). */
    double* ot = o + v_off;
    for (int32_t j = 0; j < dv; ++j) ot[j] = 0.0;
    for (int32_t c = 0; c < dk; ++c)
      for (int32_t j = 0; j < dv; ++j) ot[j] += S[c * dv + j] * xq[c];
    for (int32_t j = 0; j < dv; ++j) ot[j] *= scale;
  }
}

/*
 * Full forward over N packed sequences.  h0 may be NULL (zero initial
 * state); ht may be NULL (final state not returned).  o must hold
 * seq_start[N] * H * dv values.
 */
int32_t ckda_oracle_fwd(int32_t N, const int64_t* seq_start, int32_t H,
                        int32_t dk, int32_t dv, const double* q,
                        const double* k, const double* v, const double* alpha,
                        const double* beta, const double* h0, double* o,
                        double* ht, int32_t use_l2norm, double scale,
                        double eps) {
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !seq_start) return ORACLE_BAD_ARG;
  if (seq_start[0] != 0) return ORACLE_BAD_ARG;
  for (int32_t n = 0; n < N; ++n)
    if (seq_start[n + 1] < seq_start[n]) return ORACLE_BAD_ARG;
  if (seq_start[N] > 0 && (!q || !k || !v || !alpha || !beta || !o))
    return ORACLE_BAD_ARG;

  int32_t failed = 0;
  const int64_t pairs = (int64_t)N * H;
#pragma omp parallel
  {
    double* S = (double*)malloc(sizeof(double) * (size_t)dk * (size_t)dv);
    double* xq = (double*)malloc(sizeof(double) * (size_t)dk);
    double* xk = (double*)malloc(sizeof(double) * (size_t)dk);
    double* w = (double*)malloc(sizeof(double) * (size_t)dv);
    const int ok = S && xq && xk && w;
    if (!ok) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
      if (!ok) continue;
      const int32_t n = (int32_t)(p / H);
      const int32_t h = (int32_t)(p % H);
      const size_t sz = (size_t)dk * (size_t)dv;
      const int64_t st_off = ((int64_t)n * H + h) * (int64_t)sz;
      if (h0)
        memcpy(S, h0 + st_off, sizeof(double) * sz);
      else
        memset(S, 0, sizeof(double) * sz);
      run_head(seq_start[n], seq_start[n + 1], h, H, dk, dv, q, k, v, alpha,
               beta, S, o, use_l2norm, scale, eps, xq, xk, w);
      if (ht) memcpy(ht + st_off, S, sizeof(double) * sz);
    }
    free(S);
    free(xq);
    free(xk);
    free(w);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * Gradients of the forward above (reverse mode through the same per-token
 * steps, in the reverse token order).  Given dL/do (dout, shaped like o) and
 * dL/dht (dht [N][H][dk][dv], or NULL for zero), returns dL/dq, dL/dk,
 * dL/dv, dL/dalpha, dL/dbeta and dL/dh0 (dh0 may be NULL).
 *
 * Per token the forward computes, with x_q, x_k the (normalised) q and k:
 *   X = Diag(alpha) S_prev;  w = X^T x_k;  u = v - w;
 *   S = X + beta x_k u^T;    o = scale S^T x_q.
 * The adjoints follow step by step (G = dL/dS accumulated from later
 * tokens and this token's read-out):
 *   G += scale x_q dout^T               dx_q = scale S dout
 *   e = G^T x_k;  du = beta e           dbeta = e . u
 *   dx_k = beta G u - X du              dv = du
 *   dX = G - x_k du^T
 *   dalpha[c] = sum_j dX[c,j] S_prev[c,j]
 *   G <- Diag(alpha) dX                 (dL/dS_prev)
 * and through x = y / sqrt(|y|^2 + eps) with r = 1/sqrt(|y|^2 + eps):
 *   dy = r (dx - x (x . dx)).
 * Every state S_t of the sequence is kept from a first forward sweep (the
 * plain way to have S_prev at each step of the reverse sweep).
 */
static void bwd_head(int64_t t0, int64_t t1, int32_t h, int32_t H, int32_t dk,
                     int32_t dv, const double* q, const double* k,
                     const double* v, const double* alpha, const double* beta,
                     const double* dout, double* G, double* states,
                     double* dq, double* dk_out, double* dv_out,
                     double* dalpha, double* dbeta, int32_t use_l2norm,
                     double scale, double eps, double* xq, double* xk,
                     double* w, double* dxq, double* dxk, double* e) {
  const size_t sz = (size_t)dk * (size_t)dv;
  /* forward sweep: states[i] = S after token t0 + i - 1 (states[0] = S_0) */
  for (int64_t t = t0; t < t1; ++t) {
    const int64_t i = t - t0;
    double* S = states + (size_t)(i + 1) * sz;
    memcpy(S, states + (size_t)i * sz, sizeof(double) * sz);
    const int64_t qk_off = (t * H + h) * (int64_t)dk;
    memcpy(xk, k + qk_off, sizeof(double) * (size_t)dk);
    if (use_l2norm) l2_normalise(xk, dk, eps);
    const double* a = alpha + qk_off;
    const double b = beta[t * H + h];
    const double* vt = v + (t * H + h) * (int64_t)dv;
    for (int32_t c = 0; c < dk; ++c)
      for (int32_t j = 0; j < dv; ++j) S[c * dv + j] *= a[c];
    for (int32_t j = 0; j < dv; ++j) w[j] = 0.0;
    for (int32_t c = 0; c < dk; ++c)
      for (int32_t j = 0; j < dv; ++j) w[j] += S[c * dv + j] * xk[c];
    for (int32_t c = 0; c < dk; ++c) {
      const double bk = b * xk[c];
      for (int32_t j = 0; j < dv; ++j) S[c * dv + j] += bk * (vt[j] - w[j]);
    }
  }
  /* reverse sweep */
  for (int64_t t = t1 - 1; t >= t0; --t) {
    const int64_t i = t - t0;
    const double* Sp = states + (size_t)i * sz;       /* S_prev */
    const double* St = states + (size_t)(i + 1) * sz; /* S after token t */
    const int64_t qk_off = (t * H + h) * (int64_t)dk;
    const int64_t v_off = (t * H + h) * (int64_t)dv;
    memcpy(xq, q + qk_off, sizeof(double) * (size_t)dk);
    memcpy(xk, k + qk_off, sizeof(double) * (size_t)dk);
    if (use_l2norm) {
      l2_normalise(xq, dk, eps);
      l2_normalise(xk, dk, eps);
    }
    const double* a = alpha + qk_off;
    const double b = beta[t * H + h];
    const double* vt = v + v_off;
    const double* go = dout + v_off;
    /* read-out: o = scale S^T x_q */
    for (int32_t c = 0; c < dk; ++c) {
      double acc = 0.0;
      for (int32_t j = 0; j < dv; ++j) {
        G[c * dv + j] += scale * xq[c] * go[j];
        acc += St[c * dv + j] * go[j];
      }
      dxq[c] = scale * acc;
    }
    /* X = Diag(alpha) S_prev, w = X^T x_k, u = v - w (recomputed) */
    for (int32_t j = 0; j < dv; ++j) w[j] = 0.0;
    for (int32_t c = 0; c < dk; ++c)
      for (int32_t j = 0; j < dv; ++j) w[j] += a[c] * Sp[c * dv + j] * xk[c];
    /* e = G^T x_k; u = v - w */
    for (int32_t j = 0; j < dv; ++j) e[j] = 0.0;
    for (int32_t c = 0; c < dk; ++c)
      for (int32_t j = 0; j < dv; ++j) e[j] += G[c * dv + j] * xk[c];
    double db = 0.0;
    for (int32_t j = 0; j < dv; ++j) db += e[j] * (vt[j] - w[j]);
    dbeta[t * H + h] = db;
    /* dx_k = beta G u - X du, du = beta e */
    for (int32_t c = 0; c < dk; ++c) {
      double acc1 = 0.0, acc2 = 0.0;
      for (int32_t j = 0; j < dv; ++j) {
        acc1 += G[c * dv + j] * (vt[j] - w[j]);
        acc2 += a[c] * Sp[c * dv + j] * (b * e[j]);
      }
      dxk[c] = b * acc1 - acc2;
    }
    for (int32_t j = 0; j < dv; ++j) dv_out[v_off + j] = b * e[j];
    /* dX = G - x_k du^T; dalpha; G <- Diag(alpha) dX */
    for (int32_t c = 0; c < dk; ++c) {
      double da = 0.0;
      for (int32_t j = 0; j < dv; ++j) {
        const double dX = G[c * dv + j] - xk[c] * (b * e[j]);
        da += dX * Sp[c * dv + j];
        G[c * dv + j] = a[c] * dX;
      }
      dalpha[qk_off + c] = da;
    }
    /* through the normalisation */
    if (use_l2norm) {
      const double* yq = q + qk_off;
      const double* yk = k + qk_off;
      double nq = 0.0, nk = 0.0, pq = 0.0, pk = 0.0;
      for (int32_t c = 0; c < dk; ++c) {
        nq += yq[c] * yq[c];
        nk += yk[c] * yk[c];
        pq += xq[c] * dxq[c];
        pk += xk[c] * dxk[c];
      }
      const double rq = 1.0 / sqrt(nq + eps), rk = 1.0 / sqrt(nk + eps);
      for (int32_t c = 0; c < dk; ++c) {
        dq[qk_off + c] = rq * (dxq[c] - xq[c] * pq);
        dk_out[qk_off + c] = rk * (dxk[c] - xk[c] * pk);
      }
    } else {
      for (int32_t c = 0; c < dk; ++c) {
        dq[qk_off + c] = dxq[c];
        dk_out[qk_off + c] = dxk[c];
      }
    }
  }
}

int32_t ckda_oracle_bwd(int32_t N, const int64_t* seq_start, int32_t H,
                        int32_t dk, int32_t dv, const double* q,
                        const double* k, const double* v, const double* alpha,
                        const double* beta, const double* h0,
                        const double* dout, const double* dht, double* dq,
                        double* dk_out, double* dv_out, double* dalpha,
                        double* dbeta, double* dh0, int32_t use_l2norm,
                        double scale, double eps) {
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0 || !seq_start) return ORACLE_BAD_ARG;
  if (seq_start[0] != 0) return ORACLE_BAD_ARG;
  int64_t longest = 0;
  for (int32_t n = 0; n < N; ++n) {
    if (seq_start[n + 1] < seq_start[n]) return ORACLE_BAD_ARG;
    if (seq_start[n + 1] - seq_start[n] > longest) longest = seq_start[n + 1] - seq_start[n];
  }
  if (seq_start[N] > 0 && (!q || !k || !v || !alpha || !beta || !dout || !dq ||
                           !dk_out || !dv_out || !dalpha || !dbeta))
    return ORACLE_BAD_ARG;

  int32_t failed = 0;
  const int64_t pairs = (int64_t)N * H;
#pragma omp parallel
  {
    const size_t sz = (size_t)dk * (size_t)dv;
    double* G = (double*)malloc(sizeof(double) * sz);
    double* states = (double*)malloc(sizeof(double) * sz * (size_t)(longest + 1));
    double* xq = (double*)malloc(sizeof(double) * (size_t)dk);
    double* xk = (double*)malloc(sizeof(double) * (size_t)dk);
    double* dxq = (double*)malloc(sizeof(double) * (size_t)dk);
    double* dxk = (double*)malloc(sizeof(double) * (size_t)dk);
    double* w = (double*)malloc(sizeof(double) * (size_t)dv);
    double* e = (double*)malloc(sizeof(double) * (size_t)dv);
    const int ok = G && states && xq && xk && dxq && dxk && w && e;
    if (!ok) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t p = 0; p < pairs; ++p) {
      if (!ok) continue;
      const int32_t n = (int32_t)(p / H);
      const int32_t h = (int32_t)(p % H);
      const int64_t st_off = ((int64_t)n * H + h) * (int64_t)sz;
      if (h0)
        memcpy(states, h0 + st_off, sizeof(double) * sz);
      else
        memset(states, 0, sizeof(double) * sz);
      if (dht)
        memcpy(G, dht + st_off, sizeof(double) * sz);
      else
        memset(G, 0, sizeof(double) * sz);
      bwd_head(seq_start[n], seq_start[n + 1], h, H, dk, dv, q, k, v, alpha, beta,
               dout, G, states, dq, dk_out, dv_out, dalpha, dbeta, use_l2norm,
               scale, eps, xq, xk, w, dxq, dxk, e);
      if (dh0) memcpy(dh0 + st_off, G, sizeof(double) * sz);
    }
    free(G);
    free(states);
    free(xq);
    free(xk);
    free(dxq);
    free(dxk);
    free(w);
    free(e);
  }
  return failed ? ORACLE_NO_MEMORY : ORACLE_OK;
}

/*
 * One decode step for N independent sequences (one token each): the same
 * per-token body as the forward, applied to the state cache.  state is
 * [N][H][dk][dv] and is updated in place; q,k,alpha are [N][H][dk],
 * v and o are [N][H][dv], beta is [N][H].
 */
int32_t ckda_oracle_step(int32_t N, int32_t H, int32_t dk, int32_t dv,
                         const double* q, const double* k, const double* v,
                         const double* alpha, const double* beta,
                         double* state, double* o, int32_t use_l2norm,
                         double scale, double eps) {
  if (N < 0 || H <= 0 || dk <= 0 || dv <= 0) return ORACLE_BAD_ARG;
  if (N == 0) return ORACLE_OK;
  if (!q || !k || !v || !alpha || !beta || !state || !o) return ORACLE_BAD_ARG;
  int64_t* starts = (int64_t*)malloc(sizeof(int64_t) * (size_t)(N + 1));
  if (!starts) return ORACLE_NO_MEMORY;
  for (int32_t n = 0; n <= N; ++n) starts[n] = n;
  /* The state is both the initial and the final state: each (n,h) block is
   * copied in before its tokens run and copied out afterwards by the same
   * thread, so aliasing h0 and ht is safe here. */
  const int32_t rc = ckda_oracle_fwd(N, starts, H, dk, dv, q, k, v, alpha,
                                     beta, state, o, state, use_l2norm, scale,
                                     eps);
  free(starts);
  return rc;
}
