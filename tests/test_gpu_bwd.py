"""GPU parity of the chunked backward (ckda_chunk_bwd through the C ABI)
against the oracle's gradients (oracle.bwd, pinned by finite differences).

Tolerances (max-normalised error per tensor): float32 io 1e-4 and bf16 io
2e-2 for dq, dk, dv, dbeta, dh0 and for alpha * dalpha (the log-derivative of
the gates), everywhere.  dalpha itself is that log-derivative divided by
alpha in the ratio form, so its absolute error grows like 1/|alpha| as a gate
approaches zero (the derivative with respect to a near-zero gate is
ill-conditioned there); it is held to the same tolerances where
|alpha| >= 1/16, and the token-level path (exact zero gates) is exact."""
import numpy as np
import pytest
import torch

import gated_delta_rule_ckda_amd as ck
import oracle
from gated_delta_rule_ckda_amd import inputs
from tests.gpu_util import DEV, announce, dev, host, max_rel_err

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
ALPHA_MIN = 1.0 / 16
NAMES = ["dq", "dk", "dv", "dalpha", "dbeta", "dh0"]


def _grad_errs(g, r, alpha):
    """Errors per gradient; dalpha over |alpha| >= ALPHA_MIN (normalised by
    the max over all elements), a*dalpha everywhere."""
    errs = {n: max_rel_err(x, y) for n, x, y in zip(NAMES, g, r) if n != "dalpha"}
    m = np.abs(alpha) >= ALPHA_MIN
    den = np.abs(r[3]).max()
    errs["dalpha"] = float(np.abs(g[3] - r[3])[m].max() / den) if m.any() and den > 0 else 0.0
    errs["a*dalpha"] = max_rel_err(g[3] * alpha, r[3] * alpha)
    return errs


def _grad_case(seed, B, T, H, d, dtype, l2=True, zero_frac=0.0, gates="tanh", h0=True,
               dht=True, cu=None):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, T, H, d)).astype(np.float32) for _ in range(3))
    if not l2:  # unit keys: the method's range assumes them without the norm
        k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    if gates == "tanh":
        a = np.tanh(rng.normal(2, 1, (B, T, H, d))) * rng.choice([-1, 1], (B, T, H, d))
    elif gates == "uniform":
        a = rng.uniform(-1, 1, (B, T, H, d))
    else:  # kda: positive
        a = 1.0 / (1.0 + np.exp(-rng.normal(2, 1, (B, T, H, d))))
    a = a.astype(np.float32)
    if zero_frac:
        a[rng.random(a.shape) < zero_frac] = 0.0
    b = rng.uniform(0, 2, (B, T, H)).astype(np.float32)
    N = B if cu is None else len(cu) - 1
    s0 = (0.3 * rng.standard_normal((N, H, d, d))).astype(np.float32) if h0 else None
    dO = rng.standard_normal((B, T, H, d)).astype(np.float32)
    gS = rng.standard_normal((N, H, d, d)).astype(np.float32) if dht else None
    if dtype == "bf16":
        q, k, v, dO = (inputs.round_bf16(x) for x in (q, k, v, dO))
    return dict(q=q, k=k, v=v, alpha=a, beta=b, h0=s0, dO=dO, dht=gS, cu=cu)


def _check(c, dtype, chunk, l2=True, scale=1.0, gate="ckda"):
    cu = None if c["cu"] is None else torch.from_numpy(np.asarray(c["cu"], np.int32)).to(DEV)
    g = ck.chunk_bwd(dev(c["q"], dtype), dev(c["k"], dtype), dev(c["v"], dtype), dev(c["alpha"]),
                     dev(c["beta"]), dev(c["dO"], dtype),
                     h0=None if c["h0"] is None else dev(c["h0"]),
                     dht=None if c["dht"] is None else dev(c["dht"]), cu_seqlens=cu,
                     chunk_size=chunk, use_qk_l2norm=l2, scale=scale, gate=gate)
    torch.cuda.synchronize()
    g = [host(x) for x in g]
    r = oracle.bwd(c["q"], c["k"], c["v"], c["alpha"], c["beta"], c["dO"], h0=c["h0"],
                   dht=c["dht"], seq_start=c["cu"], use_l2norm=l2, scale=scale)
    errs = _grad_errs(g, r, c["alpha"])
    print("  " + " ".join("%s=%.2e" % kv for kv in errs.items()))
    for n, e in errs.items():
        assert e < TOL[dtype], (n, e)
    return g, r


@pytest.mark.parametrize("chunk,d", [(16, 16), (32, 32), (64, 32), (16, 64), (32, 64)])
@pytest.mark.parametrize("l2", [True, False])
def test_bwd_f32_parity(chunk, d, l2):
    announce("bwd f32 C=%d d=%d l2=%s" % (chunk, d, l2))
    _check(_grad_case(900 + chunk + d, 2, 2 * chunk + 13, 2, d, "f32", l2=l2), "f32", chunk,
           l2=l2, scale=0.8)


@pytest.mark.parametrize("chunk,d", [(64, 128), (32, 128), (64, 64), (16, 64)])
def test_bwd_bf16_parity(chunk, d):
    announce("bwd bf16 C=%d d=%d" % (chunk, d))
    _check(_grad_case(950 + chunk + d, 2, 3 * chunk + 7, 2, d, "bf16"), "bf16", chunk)


@pytest.mark.parametrize("dtype,chunk,d", [("f32", 32, 32), ("bf16", 64, 128)])
def test_bwd_zero_and_fast_gates_token_path(dtype, chunk, d):
    """Exact zero gates and uniform gates (whose chunk-wide products underflow)
    send chunks to the token-level kernel; both paths agree with the oracle,
    the gradient at a zero gate included."""
    announce("bwd irregular chunks %s C=%d d=%d" % (dtype, chunk, d))
    _check(_grad_case(970 + d, 2, 2 * chunk + 9, 2, d, dtype, zero_frac=0.03), dtype, chunk)
    _check(_grad_case(971 + d, 1, 2 * chunk, 2, d, dtype, gates="uniform"), dtype, chunk)


def test_bwd_kda_range_and_no_states():
    announce("bwd KDA gates, no h0 / dht")
    _check(_grad_case(980, 2, 77, 3, 32, "f32", gates="kda", h0=False, dht=False), "f32", 32,
           gate="kda")


def test_bwd_packed_with_empty_sequences():
    announce("bwd packed varlen")
    cu = [0, 0, 37, 37, 130, 200]
    c = _grad_case(990, 1, 200, 2, 32, "f32", cu=cu)
    _check(c, "f32", 32)


def test_bwd_gradient_of_zero_gate_is_not_zero():
    """The gradient at an exact zero gate is generally nonzero (the loss is
    affine in each gate); vacuity guard for the token path."""
    announce("bwd zero gate gradient")
    c = _grad_case(991, 1, 40, 1, 16, "f32")
    c["alpha"][0, 10, 0, :] = 0.0
    g, r = _check(c, "f32", 16)
    assert np.abs(r[3][0, 10, 0]).max() > 1e-3 and np.abs(g[3][0, 10, 0]).max() > 1e-3


def test_bwd_lm_layer_full_sampled():
    """The LM layer (B=8, T=4096, H=16, d=128, bf16, chunk 64) at full size,
    random output and final-state gradients; oracle gradients on sampled
    (batch, head) pairs."""
    announce("bwd LM layer full size")
    c = inputs.lm_layer(arm="ckda")
    rng = np.random.default_rng(77)
    dO = inputs.round_bf16(rng.standard_normal(c.v.shape).astype(np.float32))
    dht = rng.standard_normal((8, 16, 128, 128)).astype(np.float32)
    g = ck.chunk_bwd(dev(c.q, "bf16"), dev(c.k, "bf16"), dev(c.v, "bf16"), dev(c.alpha),
                     dev(c.beta), dev(dO, "bf16"), dht=dev(dht), chunk_size=64)
    torch.cuda.synchronize()
    g = [host(x) for x in g]
    oracle.set_num_threads(1)
    try:
        for (n, h) in [(0, 0), (5, 11)]:
            sl = lambda x: x[n:n + 1, :, h:h + 1]
            r = oracle.bwd(sl(c.q), sl(c.k), sl(c.v), sl(c.alpha), c.beta[n:n + 1, :, h:h + 1],
                           sl(dO), dht=dht[n:n + 1, h:h + 1])
            ours = [sl(g[0]), sl(g[1]), sl(g[2]), sl(g[3]), g[4][n:n + 1, :, h:h + 1],
                    g[5][n:n + 1, h:h + 1]]
            errs = _grad_errs(ours, r, sl(c.alpha))
            print("  pair", (n, h), " ".join("%s=%.2e" % kv for kv in errs.items()))
            assert max(errs.values()) < TOL["bf16"]
    finally:
        oracle.set_num_threads(oracle.max_threads())
