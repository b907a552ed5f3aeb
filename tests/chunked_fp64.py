"""Test-only fp64 model of the chunked algebra the HIP forward implements.

It exists to pin that algebra against the sequential oracle: if this model
and the oracle agree to ~1e-12 on inputs with zero and negative gates, short
final chunks and both code paths, the factorisation the kernel uses is exact
(the kernel then differs from the oracle by rounding only).  It shares no code
with the HIP library and is used by the tests only.

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
and g = D(C-1<-(-1)).

Regular chunks.  With the chunk's running gate product Ft_r = prod_{s<=r}
alpha_s (per channel), D(r<-j) = Ft_r * (1 / Ft_j), so

    A_rj = beta_r <k_r * Ft_r, k_j / Ft_j>,  P_rj = <q_r * Ft_r, k_j / Ft_j>,
    Kt = k * Ft,  Qt = q * Ft,  Kh_j = g * k_j / Ft_j,  g = Ft_{C-1}.

This is used when every |Ft_r| lies in [2^-100, 2^10]: then no factor
overflows and no quotient is formed by a zero (signs are exact).

Block-anchored chunks.  When the chunk-wide products leave that range (gates
that decay fast over C tokens) the products restart every 16 rows (the MFMA
tile height): Fb_r = prod of the gates of block(r) up to r, T_b the total of
block b and, for r in block I and j in block J <= I,
D(r<-j) = Fb_r * E_IJ / Fb_j with E_IJ = prod_{J<=b<I} T_b, so

    A_rj = beta_r <k_r * Fb_r * E_IJ, k_j / Fb_j>,  P_rj likewise with q_r,
    Kh_j = (k_j / Fb_j) * prod_{b>=J} T_b,

while Kt, Qt and g keep the plain products Ft.  This is used when the ratio
form is not and every |Fb_r| lies in the same range, a condition on 16
consecutive gates.

Irregular chunks (an exact zero gate, or gates so small that the running
product leaves that range) form the same A, P and Kh from direct products of
the gates instead of ratios: D(r<-j) built one gate at a time and Kh_j from
the suffix product prod_{s>j} alpha_s, with no division (the kernel's
direct path).  Both kinds of chunk then share X = (I + A)^{-1},
U = X Diag(beta) V - W S_0 with W = X Diag(beta) Kt, O and S_C.

Normalisation enters as row scales: k_hat = rk * k, q_hat = rq * q.
"""
import numpy as np

LO, HI = 2.0 ** -100, 2.0 ** 10
BLOCK = 16


def _in_range(F):
    mag = np.abs(F)
    return bool(np.all(np.isfinite(F)) and mag.min() >= LO and mag.max() <= HI)


def _l2scale(x, use, eps=1e-6):
    if not use:
        return np.ones(x.shape[:-1])
    return 1.0 / np.sqrt((x * x).sum(-1) + eps)


def _restarted(ac):
    """Per 16-row block and channel: the running product from the block start,
    restarted after a gate that is exactly zero (the zero's row takes 1, the
    empty product of the gates after it), and the block's zero mask."""
    C, dk = ac.shape
    Fr = np.ones((C, dk))
    Z = np.zeros((C, dk), dtype=bool)
    for b in range(C // BLOCK):
        f = np.ones(dk)
        for r in range(b * BLOCK, (b + 1) * BLOCK):
            z = ac[r] == 0
            f = np.where(z, 1.0, f * ac[r])
            Fr[r] = f
            Z[r] = z
    return Fr, Z


def _zero_form_ok(ac):
    """The masked block form applies: some gate is exactly zero, every
    (block, channel) holds one zero at most, and the restarted products are
    in range (nonzero gates that do not underflow over a block)."""
    if not np.any(ac == 0):
        return False
    Fr, Z = _restarted(ac)
    C = ac.shape[0]
    zc = Z.reshape(C // BLOCK, BLOCK, -1).sum(1)
    return bool(zc.max() <= 1) and _in_range(Fr)


def _zero_form(ac, kc, qc):
    """G = Kt Rk^T-like pair sums (without beta and the norms), P and Kh of a
    chunk with exact zero gates, in the masked block form the second
    transform kernel runs: with Fr the restarted block products, Lk = k Fr,
    Lq = q Fr, Rk = k / Fr;
      off-diagonal tile (I > J): rows r of I while no zero lies at or before r
        in I (the prefix D(r<-a_I)), rows j of J while no zero lies after j in
        J (the suffix D(e_J<-j)), the right side scaled by E_IJ = T'_J prod_{J<b<I} T_b
        (T'_J block J's product after its zero, T_b the plain block products);
      diagonal tile: the pairs before the block's zero plus the pairs at or
        after it (D across a zero is 0);
      Kh_j = Rk_j T'_J prod_{b>J} T_b while no zero follows j in its block, else 0."""
    C, dk = ac.shape
    nb = C // BLOCK
    Fr, Z = _restarted(ac)
    Lk, Lq, Rk = kc * Fr, qc * Fr, kc / Fr
    T = np.array([np.prod(ac[b * BLOCK:(b + 1) * BLOCK], axis=0) for b in range(nb)])
    Tr = Fr[BLOCK - 1::BLOCK]                       # T'_b: after the block's zero
    zb = Z.reshape(nb, BLOCK, dk)
    # per row: a zero at or before it in its block / after it in its block
    before = np.cumsum(zb, axis=1).reshape(C, dk) > 0
    after = (np.cumsum(zb[:, ::-1], axis=1)[:, ::-1] - zb).reshape(C, dk) > 0
    G = np.zeros((C, C))
    Pm = np.zeros((C, C))
    for I in range(nb):
        ri = slice(I * BLOCK, (I + 1) * BLOCK)
        for J in range(I + 1):
            rj = slice(J * BLOCK, (J + 1) * BLOCK)
            if I > J:
                E = Tr[J] * np.prod(T[J + 1:I], axis=0)
                left = ~before[ri]
                right = ~after[rj]
                G[ri, rj] = (Lk[ri] * left) @ (Rk[rj] * right * E).T
                Pm[ri, rj] = (Lq[ri] * left) @ (Rk[rj] * right * E).T
            else:
                for side in (False, True):            # before / at-or-after the zero
                    m_i = before[ri] == side
                    m_j = before[rj] == side
                    G[ri, rj] += (Lk[ri] * m_i) @ (Rk[rj] * m_j).T
                    Pm[ri, rj] += (Lq[ri] * m_i) @ (Rk[rj] * m_j).T
    later = np.array([np.prod(T[J + 1:], axis=0) for J in range(nb)])
    Kh = np.where(after, 0.0, Rk * np.repeat(Tr * later, BLOCK, axis=0))  # Kh / rk
    return G, Pm, Kh


def _direct_products(ac):
    """D[r, j] = prod_{j<s<=r} alpha_s (per channel) for j <= r, built one gate
    at a time (no division); zero above the diagonal."""
    C, dk = ac.shape
    D = np.zeros((C, C, dk))
    for j in range(C):
        d = np.ones(dk)
        D[j, j] = d
        for r in range(j + 1, C):
            d = d * ac[r]
            D[r, j] = d
    return D


def chunk_head(q, k, v, alpha, beta, S, use_l2norm, scale, C, force_irregular=False,
               paths=None):
    """One sequence, one head.  q,k,alpha [T,dk], v [T,dv], beta [T], S [dk,dv].
    Returns (o [T,dv], S_final).  `paths`, if a list, receives 'ratio',
    'block' or 'direct' per chunk."""
    T, dk = q.shape
    dv = v.shape[1]
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

        Ft = np.cumprod(ac, axis=0)
        g = Ft[C - 1]
        Kt = kc * Ft
        Qt = qc * Ft
        nb = C // BLOCK
        Fb = np.concatenate([np.cumprod(ac[b * BLOCK:(b + 1) * BLOCK], axis=0)
                             for b in range(nb)])
        if _in_range(Ft) and not force_irregular:
            if paths is not None:
                paths.append("ratio")
            Rk = kc / Ft
            A = np.tril((bc * rk)[:, None] * (Kt @ Rk.T) * rk[None, :], -1)
            P = np.tril(Qt @ Rk.T)
            Kh = g * Rk                                   # Kh / rk
        elif _zero_form_ok(ac) and not force_irregular:
            if paths is not None:
                paths.append("zero")
            G, Pm, Kh = _zero_form(ac, kc, qc)
            A = np.tril((bc * rk)[:, None] * G * rk[None, :], -1)
            P = np.tril(Pm)
        elif _in_range(Fb) and not force_irregular:
            if paths is not None:
                paths.append("block")
            Tb = Fb[BLOCK - 1::BLOCK]                     # [nb, dk] block totals
            Lk, Lq, Rk = kc * Fb, qc * Fb, kc / Fb
            G = np.zeros((C, C))
            Pm = np.zeros((C, C))
            for I in range(nb):
                ri = slice(I * BLOCK, (I + 1) * BLOCK)
                for J in range(I + 1):
                    rj = slice(J * BLOCK, (J + 1) * BLOCK)
                    E = np.prod(Tb[J:I], axis=0)          # 1 when J == I
                    G[ri, rj] = (Lk[ri] * E) @ Rk[rj].T
                    Pm[ri, rj] = (Lq[ri] * E) @ Rk[rj].T
            A = np.tril((bc * rk)[:, None] * G * rk[None, :], -1)
            P = np.tril(Pm)
            tail = np.array([np.prod(Tb[J:], axis=0) for J in range(nb)])
            Kh = Rk * np.repeat(tail, BLOCK, axis=0)      # Kh / rk
        else:
            if paths is not None:
                paths.append("direct")
            D = _direct_products(ac)
            G = np.einsum("rjc,rc,jc->rj", D, kc, kc)
            A = np.tril((bc * rk)[:, None] * G * rk[None, :], -1)
            P = np.tril(np.einsum("rjc,rc,jc->rj", D, qc, kc))
            suf = np.ones((C, dk))
            for j in range(C - 2, -1, -1):
                suf[j] = suf[j + 1] * ac[j + 1]
            Kh = suf * kc                                 # Kh / rk
        X = np.linalg.inv(np.eye(C) + A)
        W = X @ ((bc * rk)[:, None] * Kt)
        Ubar = X @ (bc[:, None] * vc)
        U = Ubar - W @ S
        Ok = Qt @ S + P @ (rk[:, None] * U)
        o[c0:c0 + L] = (scale * rq[:, None] * Ok)[:L]
        S = g[:, None] * S + Kh.T @ (rk[:, None] * U)
    return o, S


def fwd(q, k, v, alpha, beta, h0=None, seq_start=None, use_l2norm=True, scale=1.0,
        C=64, force_irregular=False, paths=None):
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
                                   beta[s0:s1, h], S, use_l2norm, scale, C, force_irregular,
                                   paths)
                o[s0:s1, h] = oo
            ht[n, h] = S
    return o.reshape(out_shape), ht


# ----------------------------------------------------------------- backward
def dalpha_straddle(ac, kh, qh, F, dKt0, dQt0, dG, dP, dKh, dg0, block=BLOCK):
    """dalpha of one chunk with no division by a gate and no cancellation
    between pair terms that do not depend on it.

    Every gate-dependent quantity of the chunk is a pair (r, j), r > j, of
    positions with the decay D(r<-j) = prod_{j<t<=r} alpha_t: the chunk rows,
    plus the chunk start (j = -1, for Kt, Qt and g) and the chunk end (r = C,
    for Kh and g; D(C<-j) = D(C-1<-j)).  With adj_rj the adjoint of that
    pair's decay (per channel), dL/dalpha_s is the sum over the pairs that
    straddle s (j < s <= r) of adj_rj D(r<-s) D(s-1<-j): the two partial
    products on either side of s, both bounded by 1.  The sum is split by the
    16-row tiles (tile b = rows [16b, 16b+16), a_b = 16b - 1, e_b = 16b + 15):
      rows of b and columns before b:  Pre_s * sum_{r>=s in b} D(r<-s) rho_r
      rows after b and columns of b:   Suf_s * sum_{j<s in b} D(s-1<-j) kappa_j
      rows after b, columns before b:  Pre_s * Suf_s * Gamma_b
      both in b:                       pairwise, with products inside the tile
    with Pre_s = D(s-1<-a_b), Suf_s = D(e_b<-s) (direct products inside the
    tile), rho_r = sum_{j<=a_b} adj_rj D(a_b<-j), kappa_j = sum_{r>e_b}
    adj_rj D(r<-e_b) and Gamma_b = sum adj_rj D(r<-e_b) D(a_b<-j) (anchored
    at the tile's own edges; formed from the chunk's running products F as
    ratios, which the ratio form's range on F keeps bounded and accurate).
    The suffix and prefix sums run as recurrences (sigma_s = rho_s +
    alpha_{s+1} sigma_{s+1}, pi_{s+1} = alpha_s pi_s + kappa_s), so no step
    divides by a gate and every term is formed once, with its own sign.

    Inputs (per chunk; C rows, last axis the channels): ac gates, kh, qh the
    normalised keys and queries, F the running products, dKt0 = -(Y^T dU) S0^T
    and dQt0 = scale dO S0^T (the start pairs' adjoints over Kt and Qt),
    dG, dP the adjoints of G = tril(Kt Rk^T, -1) and P = tril(Qt Rk^T),
    dKh = U dS1^T, dg0 = rowsum(dS1 * S0)."""
    C, dk = ac.shape
    nb = C // block
    dt = ac.dtype
    g = F[C - 1]
    Rk, Kt, Qt = kh / F, kh * F, qh * F
    one = np.ones(dk, dtype=dt)
    Fa = [one if b == 0 else F[block * b - 1] for b in range(nb)]   # F at a_b
    Fe = [F[block * b + block - 1] for b in range(nb)]               # F at e_b
    # row tile t: pair terms of its rows with the columns before tile b, for
    # b = 0..t (chunk-anchored, D = F_r / F_j), from products tile by tile
    X = {}
    rho = np.zeros((C, dk), dtype=dt)
    for t in range(nb):
        rt = slice(block * t, block * t + block)
        accK, accQ = dKt0[rt].copy(), dQt0[rt].copy()
        for b in range(t + 1):
            X[t, b] = Kt[rt] * accK + Qt[rt] * accQ
            if b == t:
                rho[rt] = Fa[t] * (kh[rt] * accK + qh[rt] * accQ)
            cb = slice(block * b, block * b + block)
            accK = accK + dG[rt, cb] @ Rk[cb]
            accQ = accQ + dP[rt, cb] @ Rk[cb]
    # column tile t: pair terms of its columns with the rows after tile t
    kap = np.zeros((C, dk), dtype=dt)
    for t in range(nb):
        ct = slice(block * t, block * t + block)
        accR = g * dKh[ct]
        for I in range(nb - 1, t, -1):
            ri = slice(block * I, block * I + block)
            accR = accR + dG[ri, ct].T @ Kt[ri] + dP[ri, ct].T @ Qt[ri]
        kap[ct] = (kh[ct] / Fe[t]) * accR
    # corners: rows after tile b (and the end) with columns before it (and the start)
    endterm = g * dKh * Rk                                           # (end, j) pairs
    Gam = []
    for b in range(nb):
        Z = g * dg0 + endterm[:block * b].sum(0)
        for I in range(b + 1, nb):
            Z = Z + X[I, b].sum(0)
        Gam.append(Z * (Fa[b] / Fe[b]))
    dal = np.zeros((C, dk), dtype=dt)
    for b in range(nb):
        lo = block * b
        a = ac[lo:lo + block]
        pre = np.ones((block, dk), dtype=dt)
        for i in range(1, block):
            pre[i] = pre[i - 1] * a[i - 1]
        suf = np.ones((block, dk), dtype=dt)
        for i in range(block - 2, -1, -1):
            suf[i] = suf[i + 1] * a[i + 1]
        sig = np.zeros((block, dk), dtype=dt)
        sig[block - 1] = rho[lo + block - 1]
        for i in range(block - 2, -1, -1):
            sig[i] = rho[lo + i] + a[i + 1] * sig[i + 1]
        pi = np.zeros((block, dk), dtype=dt)
        for i in range(1, block):
            pi[i] = a[i - 1] * pi[i - 1] + kap[lo + i - 1]
        # pairs inside the tile: for each row r, Phi_r(s) = sum_{j<s} adj_rj
        # D(s-1<-j) by a recurrence over s, then D(r<-s) Phi_r(s) summed over r
        psi = np.zeros((block, dk), dtype=dt)
        for ri in range(1, block):
            r = lo + ri
            phi = np.zeros(dk, dtype=dt)
            phis = []
            for si in range(1, ri + 1):        # phi = Phi_r(lo + si)
                j = lo + si - 1
                adj = (dG[r, j] * kh[r] + dP[r, j] * qh[r]) * kh[j]
                phi = a[si - 1] * phi + adj
                phis.append(phi)
            d = np.ones(dk, dtype=dt)          # D(r <- s), s from r down
            for si in range(ri, 0, -1):
                psi[si] += d * phis[si - 1]
                d = d * a[si]
        dal[lo:lo + block] = pre * sig + suf * pi + pre * suf * Gam[b] + psi
    return dal


def chunk_head_bwd(q, k, v, alpha, beta, S_init, dO, dS_end, use_l2norm, scale, C,
                   dalpha_form="straddle", dt=np.float64):
    """Gradients for one sequence and head through the chunked form, as the
    HIP backward computes them (chunk-anchored ratios; every running product
    must be nonzero).  Returns (dq, dk, dv, dalpha, dbeta, dS_init).  dt is the
    arithmetic type (float64, or float32 to see rounding behave as on the
    GPU's float32 path).

    Per chunk with entry state S0, exit-state gradient dS1 and output
    gradient dO, and Y = X Diag(beta), Z = V - Kt S0, U = Y Z:
      O = scale (Qt S0 + P U),  S1 = Diag(g) S0 + Kh^T U
      dU  = scale P^T dO + Kh dS1                     (state pass, reverse)
      dS0 = scale Qt^T dO + Diag(g) dS1 - Kt^T Y^T dU
      dV  = Y^T dU
      dQt = scale dO S0^T,  dP = scale dO U^T (lower),  dKh = U dS1^T,
      dg  = rowsum(dS1 * S0),  dY = dU Z^T,  dKt = -(Y^T dU) S0^T
      dX  = dY Diag(beta),  dbeta_j += sum_r X_rj dY_rj
      dA  = -X^T dX X^T (strictly lower),  A = Diag(beta) G
      dbeta_r += sum_j dA_rj G_rj,  dG = Diag(beta) dA
      dKt += dG Rk,  dQt += dP Rk,  dRk = dG^T Kt + dP^T Qt + g * dKh
      dk_hat = dKt * F + dRk / F,  dq_hat = dQt * F
    dalpha: dalpha_form="straddle" is dalpha_straddle (what the kernels
    compute); "ratio" is the earlier form
      Lam = dKt * Kt + dQt * Qt - dRk * Rk,  Lam_{C-1} += (dg + sum_j dKh_j Rk_j) g
      dalpha_s = (sum_{r>=s} Lam_r) / alpha_s
    whose reverse sums cancel pair terms that do not depend on alpha_s, so
    its rounding error grows like 1/|alpha_s|.
    Then dx = r (dx_hat - x_hat (x_hat . dx_hat)) through each norm."""
    q, k, v, alpha, beta, S_init, dO, dS_end = (np.asarray(x, dtype=dt) for x in
                                                (q, k, v, alpha, beta, S_init, dO, dS_end))
    T, dk = q.shape
    dv = v.shape[1]
    rq_all, rk_all = _l2scale(q, use_l2norm).astype(dt), _l2scale(k, use_l2norm).astype(dt)
    qh_all, kh_all = q * rq_all[:, None], k * rk_all[:, None]
    # forward sweep: entry state of every chunk
    starts = list(range(0, T, C))
    S = S_init.astype(np.float64)
    S0s = []
    for c0 in starts:
        S0s.append(S.astype(dt))
        L = min(C, T - c0)
        _, S = chunk_head(q[c0:c0 + L], k[c0:c0 + L], v[c0:c0 + L], alpha[c0:c0 + L],
                          beta[c0:c0 + L], S, use_l2norm, scale, C)
    dq, dk_, dvv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dal, dbe = np.zeros_like(alpha), np.zeros_like(beta)
    dS = dS_end.copy()
    for ci in range(len(starts) - 1, -1, -1):
        c0 = starts[ci]
        L = min(C, T - c0)
        S0 = S0s[ci]
        qh = np.zeros((C, dk), dtype=dt); qh[:L] = qh_all[c0:c0 + L]
        kh = np.zeros((C, dk), dtype=dt); kh[:L] = kh_all[c0:c0 + L]
        V = np.zeros((C, dv), dtype=dt); V[:L] = v[c0:c0 + L]
        G_O = np.zeros((C, dv), dtype=dt); G_O[:L] = dO[c0:c0 + L]
        ac = np.ones((C, dk), dtype=dt); ac[:L] = alpha[c0:c0 + L]
        bc = np.zeros(C, dtype=dt); bc[:L] = beta[c0:c0 + L]
        F = np.cumprod(ac, axis=0)
        g = F[C - 1]
        Kt, Qt, Rk = kh * F, qh * F, kh / F
        Kh = g * Rk
        G = np.tril(Kt @ Rk.T, -1)
        A = bc[:, None] * G
        X = np.linalg.inv(np.eye(C, dtype=dt) + A)
        Y = X * bc[None, :]
        P = np.tril(Qt @ Rk.T)
        Z = V - Kt @ S0
        U = Y @ Z
        dS1 = dS
        dU = scale * P.T @ G_O + Kh @ dS1
        dS = scale * Qt.T @ G_O + g[:, None] * dS1 - Kt.T @ (Y.T @ dU)
        dvv[c0:c0 + L] = (Y.T @ dU)[:L]
        dQt0 = scale * G_O @ S0.T
        dP = np.tril(scale * G_O @ U.T)
        dKh = U @ dS1.T
        dg0 = (dS1 * S0).sum(1)
        dY = dU @ Z.T
        dKt0 = -(Y.T @ dU) @ S0.T
        dX = dY * bc[None, :]
        db = (X * dY).sum(0)
        dA = np.tril(-X.T @ dX @ X.T, -1)
        db = db + (dA * G).sum(1)
        dG = bc[:, None] * dA
        dKt = dKt0 + dG @ Rk
        dQt = dQt0 + dP @ Rk
        dRk = dG.T @ Kt + dP.T @ Qt + g * dKh
        dkh = dKt * F + dRk / F
        dqh = dQt * F
        if dalpha_form == "straddle":
            da = dalpha_straddle(ac, kh, qh, F, dKt0, dQt0, dG, dP, dKh, dg0)
        else:
            Lam = dKt * Kt + dQt * Qt - dRk * Rk
            Lam[C - 1] += (dg0 + (dKh * Rk).sum(0)) * g
            da = np.cumsum(Lam[::-1], axis=0)[::-1] / ac
        dal[c0:c0 + L] = da[:L]
        dbe[c0:c0 + L] = db[:L]
        for name, xh, dxh, r, out in (("q", qh, dqh, rq_all, dq), ("k", kh, dkh, rk_all, dk_)):
            if use_l2norm:
                proj = (xh * dxh).sum(1, keepdims=True)
                out[c0:c0 + L] = (r[c0:c0 + L, None] * (dxh - xh * proj)[:L])
            else:
                out[c0:c0 + L] = dxh[:L]
    return dq, dk_, dvv, dal, dbe, dS


def bwd(q, k, v, alpha, beta, dO, h0=None, dht=None, seq_start=None, use_l2norm=True,
        scale=1.0, C=64, dalpha_form="straddle", dt=np.float64):
    """Same calling convention as oracle.bwd (plus the dalpha form and the
    arithmetic type of chunk_head_bwd)."""
    q, k, v, alpha, beta, dO = (np.asarray(a, dtype=np.float64) for a in (q, k, v, alpha, beta, dO))
    H, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    if seq_start is None:
        B, T = q.shape[0], q.shape[1]
        starts = np.arange(B + 1) * T
    else:
        starts = np.asarray(seq_start)
    shp = [x.shape for x in (q, k, v, alpha, beta)]
    q, k, alpha = (a.reshape(-1, H, dk) for a in (q, k, alpha))
    v, dO = v.reshape(-1, H, dv), dO.reshape(-1, H, dv)
    beta = beta.reshape(-1, H)
    N = len(starts) - 1
    outs = [np.zeros_like(x) for x in (q, k, v, alpha, beta)]
    dh0 = np.zeros((N, H, dk, dv))
    for n in range(N):
        s0, s1 = starts[n], starts[n + 1]
        for h in range(H):
            S = np.zeros((dk, dv)) if h0 is None else np.array(h0[n, h], dtype=np.float64)
            dS = np.zeros((dk, dv)) if dht is None else np.array(dht[n, h], dtype=np.float64)
            if s1 > s0:
                r = chunk_head_bwd(q[s0:s1, h], k[s0:s1, h], v[s0:s1, h], alpha[s0:s1, h],
                                   beta[s0:s1, h], S, dO[s0:s1, h], dS, use_l2norm, scale, C,
                                   dalpha_form, dt)
                for o_, g_ in zip(outs, r[:5]):
                    o_[s0:s1, h] = g_
                dS = r[5]
            dh0[n, h] = dS
    return tuple(o.reshape(s) for o, s in zip(outs, shp)) + (dh0,)
