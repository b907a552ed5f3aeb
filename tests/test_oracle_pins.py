"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test checks the oracle against something other than itself: closed forms
printed on the pages (stored under tests/golden with their citation), exact
invariants of the recurrence, textbook special cases, or brute-force dense
matrix products.  A plausible mistake in the oracle (a dropped decay, a wrong
sign, the write term applied before the gate, the read-out before the update,
a transposed state) fails at least one of them; ``test_pins_catch_mutants``
demonstrates that on mutated copies of the update rule.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "transition_2d.json")


def _transition(orc, alpha, beta, k):
    """Read the oracle's transition matrix off its own state update: with
    S_0 = I, v = 0 and one token, S_1 = A S_0 = A."""
    alpha = np.asarray(alpha, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = alpha.size
    q = np.zeros((1, 1, 1, d))
    v = np.zeros((1, 1, 1, d))
    h0 = np.eye(d)[None, None]
    _, ht = orc.fwd(q, k.reshape(1, 1, 1, d), v, alpha.reshape(1, 1, 1, d),
                       np.full((1, 1, 1), beta), h0=h0, use_l2norm=False)
    return ht[0, 0]


def _frac_pi(s):
    num, den = s.split("/")
    return math.pi * float(num) / float(den)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- P9: 2x2 forms
def pin_transition_matches_printed_2d_construction(orc):
    """picx.dev summary, 'Motivation: From Symmetry to Rotation': with beta=2,
    k=(cos t, sin t), D=Diag(alpha,1) the transition is
    [[-alpha cos2t, -sin2t], [-alpha sin2t, cos2t]] (golden cases)."""
    g = json.load(open(GOLDEN))
    for case in g["A_alpha_theta"]["cases"]:
        t = _frac_pi(case["theta_over_pi"])
        A = _transition(orc, [case["alpha"], 1.0], 2.0, [math.cos(t), math.sin(t)])
        np.testing.assert_allclose(A, np.array(case["A"]), atol=1e-14, rtol=0)
        ev = np.linalg.eigvals(A)
        tr, det = np.trace(A), np.linalg.det(A)
        disc = tr * tr - 4 * det
        assert abs(disc - case["disc"]) < 1e-12
        # complex-conjugate eigenvalues exactly when the discriminant is negative
        assert (abs(ev.imag).max() > 1e-9) == (case["disc"] < 0)


def pin_rotation_at_alpha_minus_one_is_by_two_theta(orc):
    """Same section: at alpha=-1 the transition is a rotation by 2 theta."""
    for t in np.linspace(-3.0, 3.0, 13):
        A = _transition(orc, [-1.0, 1.0], 2.0, [math.cos(t), math.sin(t)])
        R = np.array([[math.cos(2 * t), -math.sin(2 * t)],
                      [math.sin(2 * t), math.cos(2 * t)]])
        np.testing.assert_allclose(A, R, atol=1e-14)


def pin_discriminant_formula_random(orc):
    """Discriminant (1-alpha)^2 cos^2(2t) + 4 alpha decides real vs complex."""
    rng = _rng(11)
    mism = 0
    for _ in range(2000):
        a = rng.uniform(-1, 1)
        t = rng.uniform(-math.pi, math.pi)
        A = _transition(orc, [a, 1.0], 2.0, [math.cos(t), math.sin(t)])
        disc_page = (1 - a) ** 2 * math.cos(2 * t) ** 2 + 4 * a
        tr, det = np.trace(A), np.linalg.det(A)
        assert abs((tr * tr - 4 * det) - disc_page) < 1e-12
        if abs(disc_page) > 1e-9:
            cplx = abs(np.linalg.eigvals(A).imag).max() > 0
            mism += cplx != (disc_page < 0)
    assert mism == 0


def pin_prop2_block_and_eigen_condition(orc):
    """picx.dev summary, 'Theoretical Framework', Proposition 2: with sign
    matrix Diag(-1,+1) the 2D block is B(beta,t); non-real eigenvalues iff
    beta^2 cos^2(2t) < 4(beta-1), and then |lambda|^2 = det = beta - 1."""
    g = json.load(open(GOLDEN))
    for case in g["B_beta_theta"]["cases"]:
        t = _frac_pi(case["theta_over_pi"])
        B = _transition(orc, [-1.0, 1.0], case["beta"], [math.cos(t), math.sin(t)])
        np.testing.assert_allclose(B, np.array(case["B"]), atol=1e-14)
        ev = np.linalg.eigvals(B)
        assert (abs(ev.imag).max() > 1e-12) == case["complex"]
    rng = _rng(12)
    mism = 0
    for _ in range(2000):
        beta = rng.uniform(0, 2)
        t = rng.uniform(-math.pi, math.pi)
        B = _transition(orc, [-1.0, 1.0], beta, [math.cos(t), math.sin(t)])
        lhs = beta ** 2 * math.cos(2 * t) ** 2
        rhs = 4 * (beta - 1)
        if abs(lhs - rhs) < 1e-9:
            continue
        ev = np.linalg.eigvals(B)
        cplx = abs(ev.imag).max() > 1e-12
        mism += cplx != (lhs < rhs)
        if cplx:
            assert abs(abs(ev[0]) ** 2 - (beta - 1)) < 1e-12
    assert mism == 0


def pin_commutator_formula(orc):
    """'Motivation': (H_k D - D H_k)_ij = beta k_i k_j (alpha_i - alpha_j).
    H_k and D are symmetric, so A - A^T = H_k D - D H_k for A = H_k D."""
    rng = _rng(13)
    for d in (2, 3, 5, 8):
        a = rng.uniform(-1, 1, d)
        k = rng.normal(size=d)
        beta = rng.uniform(0, 2)
        A = _transition(orc, a, beta, k)
        comm = beta * np.outer(k, k) * (a[:, None] - a[None, :])
        np.testing.assert_allclose(A - A.T, comm, atol=1e-13)


def pin_scalar_gate_commutes(orc):
    """A scalar gate (the GDN case of 'Background') makes the commutator vanish:
    the transition is symmetric, hence has a real spectrum."""
    rng = _rng(14)
    for _ in range(20):
        d = 6
        a = rng.uniform(-1, 1)
        A = _transition(orc, np.full(d, a), rng.uniform(0, 2), rng.normal(size=d))
        np.testing.assert_allclose(A, A.T, atol=1e-14)
        assert abs(np.linalg.eigvals(A).imag).max() < 1e-12


def pin_positive_gates_give_real_spectrum(orc):
    """'Motivation': strictly positive channel gates still give a real
    spectrum (the matrix is similar to a symmetric one)."""
    rng = _rng(15)
    for _ in range(200):
        d = 5
        A = _transition(orc, rng.uniform(0.01, 1, d), rng.uniform(0, 2), rng.normal(size=d))
        assert abs(np.linalg.eigvals(A).imag).max() < 1e-7


def pin_theorem1_orthogonal_family(orc):
    """Theorem 1: (I - 2 k k^T) S with ||k|| = 1 and S = Diag(+-1) is
    orthogonal; the oracle's transition with alpha in {+-1}^n, beta = 2 and a
    unit key is exactly that matrix."""
    rng = _rng(16)
    for d in (2, 4, 7, 16):
        s = rng.choice([-1.0, 1.0], size=d)
        k = rng.normal(size=d)
        k /= np.linalg.norm(k)
        A = _transition(orc, s, 2.0, k)
        np.testing.assert_allclose(A.T @ A, np.eye(d), atol=1e-14)
        np.testing.assert_allclose(A, (np.eye(d) - 2 * np.outer(k, k)) @ np.diag(s), atol=1e-15)


# ---------------------------------------------------------------- P1 / P2 / P3
def pin_rotation_sequence_closed_form(orc):
    """P1: repeated rotations compose: S_T = R(2 T theta) S_0 (v = 0), and the
    read-out o_t = S_t^T q_t; embedded as a 2-channel block inside dk = 16
    whose other channels have alpha = 1 and k = 0 (they stay unchanged)."""
    rng = _rng(21)
    T, dk, dv, th = 37, 16, 8, 0.3137
    q = rng.normal(size=(1, T, 1, dk))
    k = np.zeros((1, T, 1, dk))
    k[..., 3] = math.cos(th)
    k[..., 9] = math.sin(th)
    alpha = np.ones((1, T, 1, dk))
    alpha[..., 3] = -1.0
    v = np.zeros((1, T, 1, dv))
    beta = np.full((1, T, 1), 2.0)
    h0 = rng.normal(size=(1, 1, dk, dv))
    o, ht = orc.fwd(q, k, v, alpha, beta, h0=h0, use_l2norm=False)
    S0 = h0[0, 0]
    for t in range(T):
        ang = 2 * (t + 1) * th
        R = np.array([[math.cos(ang), -math.sin(ang)], [math.sin(ang), math.cos(ang)]])
        St = S0.copy()
        St[[3, 9], :] = R @ S0[[3, 9], :]
        np.testing.assert_allclose(o[0, t, 0], St.T @ q[0, t, 0], atol=1e-12)
        if t == T - 1:
            np.testing.assert_allclose(ht[0, 0], St, atol=1e-12)


def pin_norm_preservation_orthogonal(orc):
    """P2: alpha in {+-1}, beta = 2, unit keys, v = 0: ||S_t||_F is constant."""
    rng = _rng(22)
    N, H, dk, dv, T = 2, 3, 16, 8, 50
    S = rng.normal(size=(N, H, dk, dv))
    n0 = np.linalg.norm(S, axis=(2, 3))
    for _ in range(T):
        k = rng.normal(size=(N, H, dk))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        a = rng.choice([-1.0, 1.0], size=(N, H, dk))
        _, S = orc.step(rng.normal(size=(N, H, dk)), k, np.zeros((N, H, dv)), a,
                           np.full((N, H), 2.0), S, use_l2norm=False)
        np.testing.assert_allclose(np.linalg.norm(S, axis=(2, 3)), n0, rtol=1e-13)


def pin_non_expansive_in_range_and_not_beyond(orc):
    """P3: alpha in [-1,1], beta in [0,2], unit keys, v = 0 never grow
    ||S||_F ('CKDA ... non-expansive' in the news article; the summary's
    Limitations note that beta > 2 gives this up).  The negative control with
    beta in (2, 3] must find growth, or the check would be vacuous."""
    rng = _rng(23)
    N, H, dk, dv = 4, 4, 8, 4

    def run(beta_lo, beta_hi, steps):
        S = rng.normal(size=(N, H, dk, dv))
        grew = False
        for _ in range(steps):
            k = rng.normal(size=(N, H, dk))
            k /= np.linalg.norm(k, axis=-1, keepdims=True)
            a = rng.uniform(-1, 1, size=(N, H, dk))
            b = rng.uniform(beta_lo, beta_hi, size=(N, H))
            prev = np.linalg.norm(S, axis=(2, 3))
            _, S = orc.step(np.zeros((N, H, dk)), k, np.zeros((N, H, dv)), a, b, S,
                               use_l2norm=False)
            now = np.linalg.norm(S, axis=(2, 3))
            grew |= bool((now > prev * (1 + 1e-12)).any())
            S = S / max(now.max(), 1e-300)  # keep the scale bounded
        return grew

    assert not run(0.0, 2.0, 60)
    assert run(2.5, 3.0, 60)


# ---------------------------------------------------------------- P4 / P5 / P6
def pin_beta_zero_is_diagonal_gating(orc):
    """P4: beta = 0 reduces the transition to Diag(alpha) and removes the
    write: o_t = scale S_0^T (prod_{s<=t} alpha_s * q_hat_t) and
    ht = Diag(prod alpha) h0.  Zeros and negative gates included."""
    rng = _rng(24)
    B, T, H, dk, dv = 2, 29, 2, 8, 5
    q = rng.normal(size=(B, T, H, dk))
    k = rng.normal(size=(B, T, H, dk))
    v = rng.normal(size=(B, T, H, dv))
    a = rng.uniform(-1, 1, size=(B, T, H, dk))
    a[0, 7, 1, 2] = 0.0
    a[1, 20, 0, :3] = 0.0
    h0 = rng.normal(size=(B, H, dk, dv))
    o, ht = orc.fwd(q, k, v, a, np.zeros((B, T, H)), h0=h0, scale=0.7, use_l2norm=True)
    qh = orc.l2norm(q)
    cum = np.cumprod(a, axis=1)
    for b in range(B):
        for h in range(H):
            for t in range(T):
                exp = 0.7 * h0[b, h].T @ (cum[b, t, h] * qh[b, t, h])
                np.testing.assert_allclose(o[b, t, h], exp, atol=1e-13)
            np.testing.assert_allclose(ht[b, h], cum[b, T - 1, h][:, None] * h0[b, h], atol=1e-14)
    assert np.all(ht[0, 1, 2] == 0.0)


def pin_scalar_gate_is_gated_deltanet(orc):
    """P5: alpha_t = a_t 1 ('Background', GDN) equals the scalar-gate loop
    S = a (I - beta k k^T) S + beta k v^T written with dense matrices."""
    rng = _rng(25)
    T, dk, dv = 40, 6, 4
    q = rng.normal(size=(1, T, 1, dk))
    k = rng.normal(size=(1, T, 1, dk))
    v = rng.normal(size=(1, T, 1, dv))
    a = rng.uniform(-1, 1, size=T)
    beta = rng.uniform(0, 2, size=(1, T, 1))
    o, ht = orc.fwd(q, k, v, np.broadcast_to(a[None, :, None, None], (1, T, 1, dk)),
                       beta, use_l2norm=False)
    S = np.zeros((dk, dv))
    for t in range(T):
        kk = k[0, t, 0]
        S = a[t] * (np.eye(dk) - beta[0, t, 0] * np.outer(kk, kk)) @ S \
            + beta[0, t, 0] * np.outer(kk, v[0, t, 0])
        np.testing.assert_allclose(o[0, t, 0], S.T @ q[0, t, 0], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ht[0, 0], S, rtol=1e-12, atol=1e-12)


def pin_sign_absorption_bit_exact(orc):
    """P6 ('Implementation', compiled-PyTorch variant): cumulative signs can be
    absorbed into keys and queries.  With sigma_t = prod_{s<=t} sgn(alpha_s)
    per channel, CKDA(q,k,v,alpha,beta) equals KDA(sigma q, sigma k, v,
    |alpha|, beta) and ht = Diag(sigma_T) ht_KDA -- bit for bit, since sign
    flips are exact in floating point."""
    rng = _rng(26)
    B, T, H, dk, dv = 2, 33, 3, 16, 8
    q = rng.normal(size=(B, T, H, dk))
    k = rng.normal(size=(B, T, H, dk))
    v = rng.normal(size=(B, T, H, dv))
    a = rng.uniform(-1, 1, size=(B, T, H, dk))
    a[a == 0] = 0.5
    beta = rng.uniform(0, 2, size=(B, T, H))
    h0 = rng.normal(size=(B, H, dk, dv))
    sig = np.cumprod(np.sign(a), axis=1)
    o1, ht1 = orc.fwd(q, k, v, a, beta, h0=h0, use_l2norm=True)
    o2, ht2 = orc.fwd(sig * q, sig * k, v, np.abs(a), beta, h0=h0, use_l2norm=True)
    assert np.array_equal(o1, o2)
    assert np.array_equal(ht1, sig[:, -1][..., None] * ht2)
    # vacuity: the signs do matter (dropping them changes the output)
    o3, _ = orc.fwd(q, k, v, np.abs(a), beta, h0=h0, use_l2norm=True)
    assert np.abs(o3 - o1).max() > 1e-2


# ---------------------------------------------------------------- P7 brute force
BRUTE_CASES = [(1, 1, 5), (2, 3, 17), (4, 4, 40), (8, 3, 31)]


def pin_dense_brute_force(orc, dk=4, dv=4, T=40):
    """P7: explicit dense transitions A_t = (I - beta k k^T) Diag(alpha) and
    S_t = A_t S_{t-1} + beta k v^T against the oracle's rank-one loop, with
    zeros and negative gates, l2norm on, a nonzero h0 and scale."""
    rng = _rng(27 + dk * 100 + T)
    B, H = 2, 2
    q = rng.normal(size=(B, T, H, dk))
    k = rng.normal(size=(B, T, H, dk))
    v = rng.normal(size=(B, T, H, dv))
    a = rng.uniform(-1, 1, size=(B, T, H, dk))
    a[rng.random(a.shape) < 0.1] = 0.0
    beta = rng.uniform(0, 2, size=(B, T, H))
    h0 = rng.normal(size=(B, H, dk, dv))
    scale = 0.37
    o, ht = orc.fwd(q, k, v, a, beta, h0=h0, scale=scale, use_l2norm=True)
    eps = 1e-6
    for b in range(B):
        for h in range(H):
            S = h0[b, h].copy()
            for t in range(T):
                kk = k[b, t, h] / math.sqrt(float(k[b, t, h] @ k[b, t, h]) + eps)
                qq = q[b, t, h] / math.sqrt(float(q[b, t, h] @ q[b, t, h]) + eps)
                A = (np.eye(dk) - beta[b, t, h] * np.outer(kk, kk)) @ np.diag(a[b, t, h])
                S = A @ S + beta[b, t, h] * np.outer(kk, v[b, t, h])
                np.testing.assert_allclose(o[b, t, h], scale * S.T @ qq, rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(ht[b, h], S, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- l2norm step
def pin_l2norm_pins(orc):
    """The in-op normalisation (dormouse review, section 2): unit norm up to
    eps, direction kept, zero rows map to zero, and power-of-two rows are
    exact: 4^m entries of +-2^e give +-2^-m exactly once sum x^2 >= 64."""
    rng = _rng(31)
    x = rng.normal(size=(50, 128))
    y = orc.l2norm(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), 1.0, atol=1e-8)
    np.testing.assert_allclose(y * np.linalg.norm(x, axis=1, keepdims=True), x, rtol=1e-6)
    assert np.all(orc.l2norm(np.zeros((2, 16))) == 0)
    z = np.zeros((1, 128))
    z[0, ::2] = 4.0           # 64 entries of 2^2: sum = 1024, norm 32
    z[0, 6] = -4.0
    y = orc.l2norm(z)
    np.testing.assert_allclose(y[0, ::2], np.where(np.arange(64) == 3, -0.125, 0.125), rtol=0, atol=1e-9)


# ---------------------------------------------------------------- P11 structure
def _rand_case(rng, B, T, H, dk, dv):
    return (rng.normal(size=(B, T, H, dk)), rng.normal(size=(B, T, H, dk)),
            rng.normal(size=(B, T, H, dv)), rng.uniform(-1, 1, size=(B, T, H, dk)),
            rng.uniform(0, 2, size=(B, T, H)))


def pin_split_resume_and_varlen_and_permutation(orc):
    """P11: (i) running T1 tokens then resuming from ht equals one run;
    (ii) packed sequences equal separate runs; (iii) permuting heads or batch
    rows permutes the outputs; (iv) a zero-length sequence returns h0."""
    rng = _rng(41)
    B, T, H, dk, dv = 3, 45, 2, 8, 6
    q, k, v, a, b = _rand_case(rng, B, T, H, dk, dv)
    h0 = rng.normal(size=(B, H, dk, dv))
    o, ht = orc.fwd(q, k, v, a, b, h0=h0)
    T1 = 19
    o1, ht1 = orc.fwd(q[:, :T1], k[:, :T1], v[:, :T1], a[:, :T1], b[:, :T1], h0=h0)
    o2, ht2 = orc.fwd(q[:, T1:], k[:, T1:], v[:, T1:], a[:, T1:], b[:, T1:], h0=ht1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(ht2, ht, rtol=1e-12, atol=1e-12)
    # (ii) packed: lengths 10, 0, 35 taken from the three rows
    lens = [10, 0, 35]
    starts = np.concatenate([[0], np.cumsum(lens)])
    pq = np.concatenate([q[i, :n] for i, n in enumerate(lens)])
    pk = np.concatenate([k[i, :n] for i, n in enumerate(lens)])
    pv = np.concatenate([v[i, :n] for i, n in enumerate(lens)])
    pa = np.concatenate([a[i, :n] for i, n in enumerate(lens)])
    pb = np.concatenate([b[i, :n] for i, n in enumerate(lens)])
    po, pht = orc.fwd(pq, pk, pv, pa, pb, h0=h0, seq_start=starts)
    for i, n in enumerate(lens):
        oi, hti = orc.fwd(q[i:i + 1, :n], k[i:i + 1, :n], v[i:i + 1, :n],
                             a[i:i + 1, :n], b[i:i + 1, :n], h0=h0[i:i + 1])
        np.testing.assert_array_equal(po[starts[i]:starts[i + 1]], oi[0])
        np.testing.assert_array_equal(pht[i], hti[0])
    np.testing.assert_array_equal(pht[1], h0[1])
    # (iii) permutations
    perm_b, perm_h = [2, 0, 1], [1, 0]
    op, htp = orc.fwd(q[perm_b][:, :, perm_h], k[perm_b][:, :, perm_h],
                         v[perm_b][:, :, perm_h], a[perm_b][:, :, perm_h],
                         b[perm_b][:, :, perm_h], h0=h0[perm_b][:, perm_h])
    np.testing.assert_array_equal(op, o[perm_b][:, :, perm_h])
    np.testing.assert_array_equal(htp, ht[perm_b][:, perm_h])


def pin_decode_steps_equal_prefill(orc):
    """P11: T single-token steps on a state cache equal one T-token forward."""
    rng = _rng(42)
    B, T, H, dk, dv = 2, 12, 3, 8, 8
    q, k, v, a, b = _rand_case(rng, B, T, H, dk, dv)
    h0 = rng.normal(size=(B, H, dk, dv))
    o, ht = orc.fwd(q, k, v, a, b, h0=h0, scale=0.5)
    S = h0
    for t in range(T):
        ot, S = orc.step(q[:, t], k[:, t], v[:, t], a[:, t], b[:, t], S, scale=0.5)
        np.testing.assert_allclose(ot, o[:, t], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(S, ht, rtol=1e-13, atol=1e-13)


def pin_thread_count_does_not_change_results(orc):
    rng = _rng(43)
    q, k, v, a, b = _rand_case(rng, 4, 20, 4, 8, 8)
    orc.set_num_threads(1)
    o1, h1 = orc.fwd(q, k, v, a, b)
    orc.set_num_threads(max(2, os.cpu_count() or 2))
    o2, h2 = orc.fwd(q, k, v, a, b)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)


# ---------------------------------------------------------------- gate activation
def pin_gate_activation_closed_forms(orc):
    """picx.dev summary, 'CKDA Definition': beta = 2 sigmoid(b) and the signed
    gate 2 sigmoid(a) - 1.  Checked against closed forms that do not share
    the oracle's expression: 2 sigmoid(a) - 1 = tanh(a/2) and
    2 sigmoid(b) = 1 + tanh(b/2) (numpy's tanh); the fixed points alpha(0) = 0
    and beta(0) = 1; odd symmetry of alpha; beta(b) + beta(-b) = 2; the ranges
    [-1,1] and [0,2] with their limits.  KDA range (the plain sigmoid, a
    reading): (1 + tanh(a/2)) / 2 and scipy's expit."""
    from scipy.special import expit
    a = np.concatenate([np.linspace(-30, 30, 601), [0.0, 1e-9, -1e-9, 50.0, -50.0]])
    b = np.concatenate([np.linspace(-20, 20, 401), [0.0, 60.0, -60.0]])
    al, be = orc.gates(a, b, True)
    np.testing.assert_allclose(al, np.tanh(a / 2), rtol=0, atol=4e-16)
    np.testing.assert_allclose(be, 1 + np.tanh(b / 2), rtol=0, atol=8e-16)
    assert al[a == 0.0].tolist() == [0.0] * int((a == 0.0).sum())
    assert be[b == 0.0].tolist() == [1.0] * int((b == 0.0).sum())
    al_neg, be_neg = orc.gates(-a, -b, True)
    np.testing.assert_allclose(al_neg, -al, rtol=0, atol=4e-16)
    np.testing.assert_allclose(be + be_neg, 2.0, rtol=0, atol=8e-16)
    assert al.min() >= -1 and al.max() <= 1 and be.min() >= 0 and be.max() <= 2
    assert abs(al[a == 50.0][0] - 1) < 1e-15 and abs(al[a == -50.0][0] + 1) < 1e-15
    assert abs(be[b == 60.0][0] - 2) < 1e-15 and be[b == -60.0][0] < 1e-25
    ak, bk = orc.gates(a, b, False)
    np.testing.assert_allclose(ak, (1 + np.tanh(a / 2)) / 2, rtol=1e-14, atol=2e-16)
    np.testing.assert_allclose(ak, expit(a), rtol=1e-14, atol=0)
    np.testing.assert_allclose(bk, expit(b), rtol=1e-14, atol=0)
    assert ak.min() > 0 and ak.max() <= 1


def pin_gate_activation_feeds_recurrence(orc):
    """The activated gates drive the recurrence as gates given directly: one
    token with S_0 = I and beta logit -> -inf (beta = 0) leaves
    S_1 = Diag(alpha) with alpha = tanh(a/2)."""
    a = np.array([-3.0, -0.5, 0.0, 0.25, 4.0])
    al, be = orc.gates(a, np.array([-800.0]), True)
    assert be[0] == 0.0
    A = _transition(orc, al, be[0], np.ones(5) / np.sqrt(5.0))
    np.testing.assert_allclose(A, np.diag(np.tanh(a / 2)), rtol=0, atol=1e-15)


# ---------------------------------------------------------------- test wrappers
PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__[4:] for p in PINS])
def test_pin(pin):
    pin(oracle.default())


@pytest.mark.parametrize("dk,dv,T", BRUTE_CASES)
def test_dense_brute_force_shapes(dk, dv, T):
    pin_dense_brute_force(oracle.default(), dk, dv, T)


# ---------------------------------------------------------------- mutants
# Each mutant plants one plausible mistake in a copy of the oracle's C source
# (on the CPU; the real source is untouched).  Every mutant must turn at least
# one pin red, or the pins would not be able to see that mistake.
MUTANTS = {
    "gate_dropped": ("S[c * dv + j] *= a[c];", "S[c * dv + j] *= 1.0;"),
    "gate_sign_dropped": ("S[c * dv + j] *= a[c];", "S[c * dv + j] *= fabs(a[c]);"),
    "gate_on_value_axis": ("S[c * dv + j] *= a[c];", "S[c * dv + j] *= a[j % dk];"),
    "delta_sign_flipped": ("+= bk * (vt[j] - w[j]);", "+= bk * (vt[j] + w[j]);"),
    "beta_dropped": ("const double bk = b * xk[c];", "const double bk = xk[c];"),
    "erase_uses_query": ("w[j] += S[c * dv + j] * xk[c];", "w[j] += S[c * dv + j] * xq[c];"),
    "readout_uses_key": ("ot[j] += S[c * dv + j] * xq[c];", "ot[j] += S[c * dv + j] * xk[c];"),
    "scale_dropped": ("ot[j] *= scale;", "ot[j] *= 1.0;"),
    "norm_without_sqrt": ("const double n = sqrt(ss + eps);", "const double n = ss + eps;"),
    "h0_ignored": ("if (h0)\n", "if (0)\n"),
    "ckda_alpha_unshifted": ("2.0 * sigmoid(a[i]) - 1.0", "sigmoid(a[i])"),
    "ckda_beta_undoubled": ("2.0 * sigmoid(b[i])", "sigmoid(b[i])"),
    "sigmoid_sign_flipped": ("exp(-x)", "exp(x)"),
    "gate_ranges_swapped": ("ckda_range ? 2.0 * sigmoid(a[i]) - 1.0 : sigmoid(a[i])",
                            "ckda_range ? sigmoid(a[i]) : 2.0 * sigmoid(a[i]) - 1.0"),
    "gate_after_erase": (
        "    /* 1. Diag(alpha) S: channel c of the key space scales row c. */\n"
        "    for (int32_t c = 0; c < dk; ++c)\n"
        "      for (int32_t j = 0; j < dv; ++j) S[c * dv + j] *= a[c];\n",
        ""),
}

# the mutant "gate_after_erase" re-inserts the gate after the erase step
_GATE_AFTER = ("    /* 3. S += beta k (v - w)^T. */\n",
               "    for (int32_t c = 0; c < dk; ++c)\n"
               "      for (int32_t j = 0; j < dv; ++j) S[c * dv + j] *= a[c];\n"
               "    /* 3. S += beta k (v - w)^T. */\n")


def _fast_pins():
    skip = {"pin_discriminant_formula_random", "pin_prop2_block_and_eigen_condition",
            "pin_positive_gates_give_real_spectrum", "pin_thread_count_does_not_change_results"}
    return [p for p in PINS if p.__name__ not in skip]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutants(name, tmp_path):
    src = open(oracle.SOURCE).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, "mutation target vanished from the oracle source"
    mutated = src.replace(old, new, 1)
    if name == "gate_after_erase":
        mutated = mutated.replace(*_GATE_AFTER, 1)
    path = tmp_path / "mut.c"
    path.write_text(mutated)
    lib = oracle.compile_source(str(path), str(tmp_path / ("libmut_%s.so" % name)))
    orc = oracle.Oracle(lib)
    red = []
    for pin in _fast_pins():
        try:
            pin(orc)
        except (AssertionError, ValueError, np.linalg.LinAlgError):
            red.append(pin.__name__)
    assert red, "mutant %s passed every pin" % name
