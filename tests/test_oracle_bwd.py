"""Pins of the oracle's gradients (oracle.bwd) against facts that do not come
from the oracle's own backward code.

* Directional finite differences of the oracle's forward: for a loss
  L = <o, R_o> + <ht, R_h> with random R, the central difference of L along a
  random direction of each input must equal the inner product of that
  input's gradient with the direction (fp64, relative agreement ~1e-8).  This
  checks every gradient term against the forward recurrence itself.
* A closed form: with alpha = 1 and beta = 0 the state never changes
  (S_t = h0), so o_t = scale h0^T q_t and every gradient has a short formula
  written out here in numpy.
* Mutants: each plants one plausible mistake in a copy of the backward code
  (a dropped term, a missing gate, a wrong state); each must fail a pin.
"""
import numpy as np
import pytest

import oracle


def _case(seed, B=2, T=7, H=2, dk=4, dv=3, zero=False, packed=False):
    rng = np.random.default_rng(seed)
    q, k = rng.normal(size=(B, T, H, dk)), rng.normal(size=(B, T, H, dk))
    v = rng.normal(size=(B, T, H, dv))
    a = rng.uniform(-1, 1, size=(B, T, H, dk))
    if zero:
        a[0, 2, 0, 1] = 0.0
        a[1, 4, 1, :] = 0.0
    b = rng.uniform(0, 2, size=(B, T, H))
    h0 = rng.normal(size=(B, H, dk, dv))
    starts = None
    if packed:
        q, k, v, a = (x.reshape(1, B * T, H, -1) for x in (q, k, v, a))
        b = b.reshape(1, B * T, H)
        starts = np.array([0, 3, 3, B * T - 2, B * T])
        h0 = rng.normal(size=(len(starts) - 1, H, dk, dv))
    return dict(q=q, k=k, v=v, alpha=a, beta=b, h0=h0, seq_start=starts)


def _loss(orc, c, Ro, Rh, l2, scale):
    o, ht = orc.fwd(c["q"], c["k"], c["v"], c["alpha"], c["beta"], h0=c["h0"],
                    seq_start=c["seq_start"], use_l2norm=l2, scale=scale)
    return float((o * Ro).sum() + (ht * Rh).sum())


def _fd_check(orc, c, l2, scale, seed, tol=1e-7):
    rng = np.random.default_rng(seed)
    o, ht = orc.fwd(c["q"], c["k"], c["v"], c["alpha"], c["beta"], h0=c["h0"],
                    seq_start=c["seq_start"], use_l2norm=l2, scale=scale)
    Ro, Rh = rng.normal(size=o.shape), rng.normal(size=ht.shape)
    grads = orc.bwd(c["q"], c["k"], c["v"], c["alpha"], c["beta"], Ro, h0=c["h0"], dht=Rh,
                    seq_start=c["seq_start"], use_l2norm=l2, scale=scale)
    names = ["q", "k", "v", "alpha", "beta", "h0"]
    eps = 1e-6
    for name, g in zip(names, grads):
        d = rng.normal(size=c[name].shape)
        cp, cm = dict(c), dict(c)
        cp[name] = c[name] + eps * d
        cm[name] = c[name] - eps * d
        fd = (_loss(orc, cp, Ro, Rh, l2, scale) - _loss(orc, cm, Ro, Rh, l2, scale)) / (2 * eps)
        an = float((g * d).sum())
        assert abs(fd - an) <= tol * max(1.0, abs(an)), (name, fd, an)


def pin_bwd_finite_differences(orc):
    _fd_check(orc, _case(1), True, 1.0, 11)
    _fd_check(orc, _case(2, dk=5, dv=2), False, 0.7, 12)


def pin_bwd_finite_differences_zero_gates_packed(orc):
    """Exact zero gates (the gradient at a zero gate is not zero) and a packed
    batch with an empty sequence."""
    _fd_check(orc, _case(3, zero=True), True, 1.3, 13)
    _fd_check(orc, _case(4, packed=True, zero=True), True, 1.0, 14)


def pin_bwd_frozen_state_closed_form(orc):
    """alpha = 1, beta = 0: S_t = h0 and o_t = scale h0^T q_t (no norm).  With
    G_t = dht + scale sum_{s>=t} q_s dO_s^T (the state adjoint just after
    token t):  dq_t = scale h0 dO_t, dk_t = 0, dv_t = 0,
    dbeta_t = (G_t^T k_t) . (v_t - h0^T k_t), dalpha_t = rowsum(G_t * h0),
    dh0 = G_1."""
    rng = np.random.default_rng(21)
    T, dk, dv, scale = 6, 4, 3, 0.9
    q, k, v = rng.normal(size=(1, T, 1, dk)), rng.normal(size=(1, T, 1, dk)), rng.normal(size=(1, T, 1, dv))
    a, b = np.ones((1, T, 1, dk)), np.zeros((1, T, 1))
    h0 = rng.normal(size=(1, 1, dk, dv))
    dO, dht = rng.normal(size=(1, T, 1, dv)), rng.normal(size=(1, 1, dk, dv))
    dq, dkk, dvv, da, db, dh0 = orc.bwd(q, k, v, a, b, dO, h0=h0, dht=dht, use_l2norm=False,
                                        scale=scale)
    H0 = h0[0, 0]
    G = dht[0, 0].copy()
    for t in range(T - 1, -1, -1):
        G = G + scale * np.outer(q[0, t, 0], dO[0, t, 0])
        np.testing.assert_allclose(dq[0, t, 0], scale * H0 @ dO[0, t, 0], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dkk[0, t, 0], 0.0, atol=1e-12)
        np.testing.assert_allclose(dvv[0, t, 0], 0.0, atol=1e-12)
        e = G.T @ k[0, t, 0]
        u = v[0, t, 0] - H0.T @ k[0, t, 0]
        np.testing.assert_allclose(db[0, t, 0], e @ u, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(da[0, t, 0], (G * H0).sum(1), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dh0[0, 0], G, rtol=1e-12, atol=1e-12)


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__[4:] for p in PINS])
def test_pin(pin):
    pin(oracle.default())


MUTANTS = {
    "dk_drops_erase_term": ("dxk[c] = b * acc1 - acc2;", "dxk[c] = b * acc1;"),
    "adjoint_gate_dropped": ("G[c * dv + j] = a[c] * dX;", "G[c * dv + j] = dX;"),
    "dv_beta_dropped": ("dv_out[v_off + j] = b * e[j];", "dv_out[v_off + j] = e[j];"),
    "dbeta_uses_v": ("db += e[j] * (vt[j] - w[j]);", "db += e[j] * vt[j];"),
    "dq_norm_projection_dropped": ("dq[qk_off + c] = rq * (dxq[c] - xq[c] * pq);",
                                   "dq[qk_off + c] = rq * dxq[c];"),
    "readout_scale_dropped": ("G[c * dv + j] += scale * xq[c] * go[j];",
                              "G[c * dv + j] += xq[c] * go[j];"),
    "dalpha_uses_new_state": ("da += dX * Sp[c * dv + j];", "da += dX * St[c * dv + j];"),
    "erase_adjoint_dropped": ("const double dX = G[c * dv + j] - xk[c] * (b * e[j]);",
                              "const double dX = G[c * dv + j];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_bwd_mutants(name, tmp_path):
    src = open(oracle.SOURCE).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutation target must appear once in the oracle source"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    orc = oracle.Oracle(oracle.compile_source(str(path), str(tmp_path / ("libbwd_%s.so" % name))))
    red = []
    for pin in PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            red.append(pin.__name__)
    assert red, "mutant %s passed every pin" % name


# ---------------------------------------------------------- gates from logits
def _gates_loss_grads(orc, seed, ckda_range):
    """A small case with logit gates; the loss L = <o, Ro> + <ht, Rh> through
    gates(a, b) and the forward; returns (a, b, loss function of (a, b),
    (dL/da, dL/db) from bwd and gates_bwd)."""
    rng = np.random.default_rng(seed)
    B, T, H, dk, dv = 2, 9, 2, 4, 3
    q, k, v = rng.normal(size=(B, T, H, dk)), rng.normal(size=(B, T, H, dk)), rng.normal(size=(B, T, H, dv))
    a = rng.normal(0, 2, size=(B, T, H, dk))
    b = rng.normal(0, 1.5, size=(B, T, H))
    h0 = rng.normal(size=(B, H, dk, dv))
    Ro, Rh = rng.normal(size=v.shape), rng.normal(size=(B, H, dk, dv))

    def loss(a_, b_):
        al, be = orc.gates(a_, b_, ckda_range=ckda_range)
        o, ht = orc.fwd(q, k, v, al, be, h0=h0)
        return float((o * Ro).sum() + (ht * Rh).sum())

    al, be = orc.gates(a, b, ckda_range=ckda_range)
    g = orc.bwd(q, k, v, al, be, Ro, h0=h0, dht=Rh)
    da, db = orc.gates_bwd(a, b, g[3], g[4], ckda_range=ckda_range)
    return a, b, loss, da, db


def pin_gates_bwd_finite_differences(orc):
    """dL/da and dL/db through the activation (both ranges) against central
    differences of the loss computed with the oracle's gates and forward."""
    for ckda_range in (True, False):
        a, b, loss, da, db = _gates_loss_grads(orc, 31 + int(ckda_range), ckda_range)
        rng = np.random.default_rng(33)
        eps = 1e-6
        for x, g, name in ((a, da, "a"), (b, db, "b")):
            d = rng.normal(size=x.shape)
            if name == "a":
                fd = (loss(a + eps * d, b) - loss(a - eps * d, b)) / (2 * eps)
            else:
                fd = (loss(a, b + eps * d) - loss(a, b - eps * d)) / (2 * eps)
            an = float((g * d).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (ckda_range, name, fd, an)


def pin_gates_bwd_closed_forms(orc):
    """At a logit of 0: dalpha/da = 1/2 (CKDA, alpha = 2 s(a) - 1) and 1/4
    (KDA, alpha = s(a)); the same for beta.  The derivative is even in the
    logit, and the CKDA derivative is twice the KDA one everywhere."""
    z = np.zeros(3)
    one = np.ones(3)
    da, db = orc.gates_bwd(z, z, one, one, ckda_range=True)
    assert np.all(da == 0.5) and np.all(db == 0.5)
    da, db = orc.gates_bwd(z, z, one, one, ckda_range=False)
    assert np.all(da == 0.25) and np.all(db == 0.25)
    x = np.linspace(-9, 9, 37)
    g = np.random.default_rng(34).normal(size=x.shape)
    c1, _ = orc.gates_bwd(x, x, g, g, ckda_range=True)
    c2, _ = orc.gates_bwd(-x, x, g, g, ckda_range=True)
    k1, _ = orc.gates_bwd(x, x, g, g, ckda_range=False)
    # (1 - s) is formed after s, so large |logit| lose a few digits to rounding
    np.testing.assert_allclose(c1, c2, rtol=1e-10, atol=0)
    np.testing.assert_allclose(c1, 2 * k1, rtol=1e-15, atol=0)


GATE_PINS = [pin_gates_bwd_finite_differences, pin_gates_bwd_closed_forms]


@pytest.mark.parametrize("pin", GATE_PINS, ids=[p.__name__[4:] for p in GATE_PINS])
def test_gate_pin(pin):
    pin(oracle.default())


GATE_MUTANTS = {
    "range_factor_dropped": ("const double f = ckda_range ? 2.0 : 1.0;",
                             "const double f = 1.0;"),
    "sigmoid_not_its_derivative": ("da[i] = dalpha[i] * f * s * (1.0 - s);",
                                   "da[i] = dalpha[i] * f * s;"),
    "beta_uses_alpha_logit": ("const double s = sigmoid(b[i]);", "const double s = sigmoid(a[i]);"),
}


@pytest.mark.parametrize("name", sorted(GATE_MUTANTS))
def test_gate_pins_catch_mutants(name, tmp_path):
    src = open(oracle.SOURCE).read()
    old, new = GATE_MUTANTS[name]
    assert src.count(old) == 1, "mutation target must appear once in the oracle source"
    path = tmp_path / "mut.c"
    path.write_text(src.replace(old, new))
    orc = oracle.Oracle(oracle.compile_source(str(path), str(tmp_path / ("libg_%s.so" % name))))
    red = []
    for pin in GATE_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError):
            red.append(pin.__name__)
    assert red, "mutant %s passed every gate pin" % name
