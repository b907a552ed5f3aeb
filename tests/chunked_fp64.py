"""Test-only fp64 model of the chunked algebra the HIP forward implements.

It exists to pin that algebra against the sequential oracle: if this model
and the oracle agree to ~1e-12 on inputs with zero and negative gates, short
final chunks and every sub-block size, the factorisation the kernel uses is
exact (the kernel then differs from the oracle by rounding only).  It shares
no code with the HIP library and is used by the tests only.

Derivation (for one sequence and head; written out because the pages print
only the transition A_t = (I - beta_t k_t k_t^T) Diag(alpha_t), picx.dev
summary of the Complex KDA paper, section "Background"):

Within a chunk of C tokens with entry state S_0, write the update as
S_r = Diag(alpha_r) S_{r-1} + k_r u_r^T with u_r = beta_r (v_r - S~_r^T k_r)
and S~_r = Diag(alpha_r) S_{r-1}.  Unrolling, with the channel-wise decay
D(r<-j) = prod_{j<s<=r} alpha_s (rows are 0-based token positions; D(r<-r)=1,
and "from the chunk start" means j = -1):

    (I + A) U = Diag(beta) (V - Kt S_0),   A_rj = beta_r <k_r * D(r<-j), k_j>, j < r
    O   = Qt S_0 + P U,                    P_rj = <q_r * D(r<-j), k_j>,        j <= r
    S_C = Diag(g) S_0 + Kh^T U

with Kt_r = D(r<-(-1)) * k_r, Qt_r = D(r<-(-1)) * q_r, Kh_j = D(C-1<-j) * k_j
and g = D(C-1<-(-1)).  The per-channel decays are built without division
from products of alpha inside sub-blocks of `blk` rows:

    F_r = prod of alpha over the rows of r's sub-block up to and including r
    B_r = prod of alpha over the rows of r's sub-block after r
    G_I = prod of alpha over sub-block I

so that, for r in sub-block I and j in an earlier sub-block J,
D(r<-j) = F_r * (prod_{J<M<I} G_M) * B_j, a product of factors of modulus at
most one (exact for zero and negative gates).  Inside one sub-block,
D(r<-j) = F_r * (1 / F_j) whenever no |F| in the sub-block is below 2^-100
(then no factor overflows), else the product of alpha is taken directly.
Normalisation enters as row scales: k_hat = rk * k, q_hat = rq * q.
"""
import numpy as np

SAFE_LOG2 = -100.0


def _l2scale(x, use, eps=1e-6):
    if not use:
        return np.ones(x.shape[:-1])
    return 1.0 / np.sqrt((x * x).sum(-1) + eps)


def chunk_head(q, k, v, alpha, beta, S, use_l2norm, scale, C, blk, force_unsafe=False):
    """One sequence, one head.  q,k,alpha [T,dk], v [T,dv], beta [T], S [dk,dv].
    Returns (o [T,dv], S_final)."""
    T, dk = q.shape
    dv = v.shape[1]
    assert C % blk == 0
    nb = C // blk
    o = np.zeros((T, dv))
    rq_all = _l2scale(q, use_l2norm)
    rk_all = _l2scale(k, use_l2norm)
    for c0 in range(0, T, C):
        L = min(C, T - c0)
        # pad the last chunk with identity tokens (alpha=1, beta=0, q=k=v=0)
        qc = np.zeros((C, dk)); qc[:L] = q[c0:c0 + L]
        kc = np.zeros((C, dk)); kc[:L] = k[c0:c0 + L]
        vc = np.zeros((C, dv)); vc[:L] = v[c0:c0 + L]
        ac = np.ones((C, dk)); ac[:L] = alpha[c0:c0 + L]
        bc = np.zeros(C); bc[:L] = beta[c0:c0 + L]
        rq = np.ones(C); rq[:L] = rq_all[c0:c0 + L]
        rk = np.ones(C); rk[:L] = rk_all[c0:c0 + L]

        F = np.empty((C, dk))
        Bk = np.empty((C, dk))
        G = np.empty((nb, dk))
        safe = np.empty((nb, dk), dtype=bool)
        for I in range(nb):
            rows = slice(I * blk, (I + 1) * blk)
            F[rows] = np.cumprod(ac[rows], axis=0)
            # B_r: product of the rows after r inside the block
            rev = np.cumprod(ac[rows][::-1], axis=0)[::-1]
            Bk[rows][:-1] = rev[1:]
            Bk[(I + 1) * blk - 1] = 1.0
            G[I] = F[(I + 1) * blk - 1]
            with np.errstate(divide="ignore"):
                safe[I] = np.log2(np.abs(F[rows]).min(axis=0)) >= SAFE_LOG2
        if force_unsafe:
            safe[:] = False
        Gpre = np.ones((nb, dk))
        Gpost = np.ones((nb, dk))
        for I in range(1, nb):
            Gpre[I] = Gpre[I - 1] * G[I - 1]
        for I in range(nb - 2, -1, -1):
            Gpost[I] = Gpost[I + 1] * G[I + 1]
        g = Gpre[nb - 1] * G[nb - 1]

        def decay(r, j):   # D(r<-j) for j <= r, per channel
            I, J = r // blk, j // blk
            if I == J:
                direct = np.prod(ac[j + 1:r + 1], axis=0)
                with np.errstate(divide="ignore", invalid="ignore"):
                    fact = F[r] / F[j]
                return np.where(safe[I], fact, direct)
            mid = np.ones(dk)
            for M in range(J + 1, I):
                mid = mid * G[M]
            return F[r] * mid * Bk[j]

        A = np.zeros((C, C))
        P = np.zeros((C, C))
        for r in range(C):
            for j in range(r + 1):
                d = decay(r, j)
                P[r, j] = np.dot(qc[r] * d, kc[j])
                if j < r:
                    A[r, j] = bc[r] * rk[r] * rk[j] * np.dot(kc[r] * d, kc[j])
        X = np.linalg.inv(np.eye(C) + A)
        D0 = np.empty((C, dk))
        DC = np.empty((C, dk))
        for r in range(C):
            D0[r] = Gpre[r // blk] * F[r]
            DC[r] = Gpost[r // blk] * Bk[r]
        W = X @ ((bc * rk)[:, None] * (kc * D0))
        Ubar = X @ (bc[:, None] * vc)
        U = Ubar - W @ S
        Ok = (qc * D0) @ S + P @ (rk[:, None] * U)
        o[c0:c0 + L] = (scale * rq[:, None] * Ok)[:L]
        S = g[:, None] * S + (kc * DC).T @ (rk[:, None] * U)
    return o, S


def fwd(q, k, v, alpha, beta, h0=None, seq_start=None, use_l2norm=True, scale=1.0,
        C=64, blk=16, force_unsafe=False):
    """Same calling convention as oracle.fwd (dense [B,T,H,.] or packed)."""
    q, k, v, alpha, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, alpha, beta))
    out_shape = v.shape
    H, dk = q.shape[-2], q.shape[-1]
    if seq_start is None:
        B, T = q.shape[0], q.shape[1]
        starts = np.arange(B + 1) * T
    else:
        starts = np.asarray(seq_start)
    q, k, alpha = (a.reshape(-1, H, dk) for a in (q, k, alpha))
    v = v.reshape(-1, H, v.shape[-1])
    beta = beta.reshape(-1, H)
    dv = v.shape[-1]
    N = len(starts) - 1
    o = np.zeros(v.shape)
    ht = np.zeros((N, H, dk, dv))
    for n in range(N):
        s0, s1 = starts[n], starts[n + 1]
        for h in range(H):
            S = np.zeros((dk, dv)) if h0 is None else np.array(h0[n, h], dtype=np.float64)
            if s1 > s0:
                oo, S = chunk_head(q[s0:s1, h], k[s0:s1, h], v[s0:s1, h], alpha[s0:s1, h],
                                   beta[s0:s1, h], S, use_l2norm, scale, C, blk, force_unsafe)
                o[s0:s1, h] = oo
            ht[n, h] = S
    return o.reshape(out_shape), ht
