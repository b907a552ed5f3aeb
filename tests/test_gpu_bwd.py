"""GPU parity of the chunked backward (ckda_chunk_bwd through the C ABI)
against the oracle's gradients (oracle.bwd, pinned by finite differences).

Tolerances (max-normalised error per tensor, every element): float32 io 1e-4
and bf16 io 2e-2 for dq, dk, dv, dalpha, dbeta and dh0.  dalpha is formed
with no division by a gate (pairs of positions that straddle the gate, times
the partial gate products on either side of it), so gates near zero (1e-3,
1e-5) are held to the same bound as the others."""
import numpy as np
import pytest
import torch

import gated_delta_rule_ckda_amd as ck
import oracle
from gated_delta_rule_ckda_amd import inputs
from tests.gpu_util import DEV, announce, cover_pairs, dev, host, max_rel_err

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ["dq", "dk", "dv", "dalpha", "dbeta", "dh0"]


def _grad_errs(g, r):
    """Max-normalised error of each gradient over all of its elements."""
    return {n: max_rel_err(x, y) for n, x, y in zip(NAMES, g, r)}


def _grad_case(seed, B, T, H, d, dtype, l2=True, zero_frac=0.0, gates="tanh", h0=True,
               dht=True, cu=None):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((B, T, H, d)).astype(np.float32) for _ in range(3))
    if not l2:  # unit keys: the method's range assumes them without the norm
        k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    if gates in ("tanh", "tiny"):
        a = np.tanh(rng.normal(2, 1, (B, T, H, d))) * rng.choice([-1, 1], (B, T, H, d))
        if gates == "tiny":  # 4% of the gates at +-1e-3 or +-1e-5
            m = rng.random(a.shape) < 0.04
            a[m] = rng.choice([-1, 1], m.sum()) * rng.choice([1e-3, 1e-5], m.sum())
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
    errs = _grad_errs(g, r)
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


@pytest.mark.parametrize("chunk,d", [(64, 128), (32, 128), (16, 128), (64, 64), (32, 64), (16, 64)])
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


def _oracle_bwd_pairs(q, k, v, a, b, dO, dht, pairs):
    """oracle.bwd on (batch, head) pairs of a dense case, all in one packed
    call (one sequence per pair, one head), which the oracle runs in
    parallel; returns {(n, h): six gradients shaped [T, ...]}."""
    T = q.shape[1]
    cat = lambda x: np.concatenate([x[n, :, h:h + 1] for n, h in pairs], 0)[None]
    starts = np.arange(len(pairs) + 1, dtype=np.int64) * T
    dh = np.stack([dht[n, h:h + 1] for n, h in pairs], 0)
    r = oracle.bwd(cat(q), cat(k), cat(v), cat(a), cat(b), cat(dO), dht=dh, seq_start=starts)
    out = {}
    for i, p in enumerate(pairs):
        sl = slice(i * T, (i + 1) * T)
        out[p] = [r[0][0, sl, 0], r[1][0, sl, 0], r[2][0, sl, 0], r[3][0, sl, 0],
                  r[4][0, sl, 0], r[5][i, 0]]
    return out


def test_bwd_lm_layer_full_sampled():
    """The LM layer (B=8, T=4096, H=16, d=128, bf16, chunk 64) at full size,
    random output and final-state gradients; oracle gradients on 16 sampled
    (batch, head) pairs covering every batch and head index, every element
    of every gradient (dalpha included) held to the bf16 bound."""
    announce("bwd LM layer full size")
    c = inputs.lm_layer(arm="ckda")
    rng = np.random.default_rng(77)
    dO = inputs.round_bf16(rng.standard_normal(c.v.shape).astype(np.float32))
    dht = rng.standard_normal((8, 16, 128, 128)).astype(np.float32)
    g = ck.chunk_bwd(dev(c.q, "bf16"), dev(c.k, "bf16"), dev(c.v, "bf16"), dev(c.alpha),
                     dev(c.beta), dev(dO, "bf16"), dht=dev(dht), chunk_size=64)
    torch.cuda.synchronize()
    g = [host(x) for x in g]
    pairs = cover_pairs(8, 16)
    ref = _oracle_bwd_pairs(c.q, c.k, c.v, c.alpha, c.beta, dO, dht, pairs)
    worst = {}
    for (n, h) in pairs:
        ours = [g[0][n, :, h], g[1][n, :, h], g[2][n, :, h], g[3][n, :, h], g[4][n, :, h],
                g[5][n, h]]
        for name, e in _grad_errs(ours, ref[(n, h)]).items():
            worst[name] = max(worst.get(name, 0.0), e)
    print("  " + " ".join("%s=%.2e" % kv for kv in worst.items()))
    assert max(worst.values()) < TOL["bf16"]


@pytest.mark.parametrize("dtype,chunk,d", [("f32", 32, 32), ("f32", 64, 32), ("f32", 16, 64),
                                           ("bf16", 64, 128), ("bf16", 32, 64),
                                           ("bf16", 16, 128)])
def test_bwd_gates_near_zero(dtype, chunk, d):
    """Gates of +-1e-3 and +-1e-5 among tanh gates of both signs: dalpha is
    held to the bound on every element, with no mask (chunks whose running
    products stay in range take the MFMA form, the others the token path)."""
    announce("bwd gates near zero %s C=%d d=%d" % (dtype, chunk, d))
    _check(_grad_case(1100 + chunk + d, 2, 2 * chunk + 5, 2, d, dtype, gates="tiny"), dtype,
           chunk)


@pytest.mark.parametrize("dtype,chunk,d", [("f32", 16, 16), ("bf16", 16, 64), ("bf16", 64, 128)])
def test_bwd_uniform_gates(dtype, chunk, d):
    """alpha ~ U[-1, 1]: gates anywhere in the CKDA range, near zero included."""
    announce("bwd U[-1,1] gates %s C=%d d=%d" % (dtype, chunk, d))
    _check(_grad_case(1200 + chunk + d, 2, 3 * chunk + 1, 2, d, dtype, gates="uniform"), dtype,
           chunk)


def test_bwd_bf16_packed_chunk64():
    """bf16 packed batch at chunk 64, d=128 on the matrix-core passes: unequal
    lengths with empty sequences and a long chain, N * H = 16 (so the adjoint
    state pass's longest-first order and its workgroup mapping both act)."""
    announce("bwd bf16 packed C=64 d=128")
    lens = [0, 300, 17, 64, 0, 129, 451, 5]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    c = _grad_case(1300, 1, cu[-1], 2, 128, "bf16", cu=cu)
    _check(c, "bf16", 64)


@pytest.mark.parametrize("dtype,chunk,d", [("bf16", 64, 128), ("f32", 32, 32)])
def test_bwd_is_deterministic(dtype, chunk, d):
    """Two calls on the same inputs give bit-identical gradients (every
    reduction runs in a fixed order; no atomics)."""
    announce("bwd determinism %s C=%d d=%d" % (dtype, chunk, d))
    c = _grad_case(1400 + d, 2, 4 * chunk + 9, 4, d, dtype, gates="tiny")
    args = (dev(c["q"], dtype), dev(c["k"], dtype), dev(c["v"], dtype), dev(c["alpha"]),
            dev(c["beta"]), dev(c["dO"], dtype))
    kw = dict(h0=dev(c["h0"]), dht=dev(c["dht"]), chunk_size=chunk)
    g1 = [host(x) for x in ck.chunk_bwd(*args, **kw)]
    g2 = [host(x) for x in ck.chunk_bwd(*args, **kw)]
    torch.cuda.synchronize()
    for n, x, y in zip(NAMES, g1, g2):
        assert np.array_equal(x, y), n


def _check_general(c, dtype, chunk, gates="values", arm="ckda", gate_dtype="f32", Hk=None):
    """ckda_chunk_bwd with gate logits and/or grouped q/k heads against the
    oracle: logits through oracle.gates and oracle.gates_bwd, grouped heads
    as q, k repeated over the value heads (each q/k head serving H / Hk
    consecutive value heads) with their gradients summed back."""
    H = c["v"].shape[2]
    Hk = Hk or H
    G = H // Hk
    q, k = c["q"][:, :, ::G].copy(), c["k"][:, :, ::G].copy()  # the q/k heads
    a, b = c["alpha"], c["beta"]
    if gates == "logits" and gate_dtype == "bf16":
        a, b = inputs.round_bf16(a), inputs.round_bf16(b)
    cu = None if c["cu"] is None else torch.from_numpy(np.asarray(c["cu"], np.int32)).to(DEV)
    g = ck.chunk_bwd(dev(q, dtype), dev(k, dtype), dev(c["v"], dtype), dev(a, gate_dtype),
                     dev(b, gate_dtype), dev(c["dO"], dtype),
                     h0=None if c["h0"] is None else dev(c["h0"]),
                     dht=None if c["dht"] is None else dev(c["dht"]), cu_seqlens=cu,
                     chunk_size=chunk, gate=arm, gates=gates)
    torch.cuda.synchronize()
    g = [host(x) for x in g]
    qr, kr = np.repeat(q, G, axis=2), np.repeat(k, G, axis=2)
    if gates == "logits":
        al, be = oracle.gates(a, b, ckda_range=(arm == "ckda"))
    else:
        al, be = a, b
    r = list(oracle.bwd(qr, kr, c["v"], al, be, c["dO"], h0=c["h0"], dht=c["dht"],
                        seq_start=c["cu"]))
    if gates == "logits":
        r[3], r[4] = oracle.gates_bwd(a, b, r[3], r[4], ckda_range=(arm == "ckda"))
    if G > 1:
        sh = r[0].shape
        r[0] = r[0].reshape(sh[:2] + (Hk, G, sh[3])).sum(3)
        r[1] = r[1].reshape(sh[:2] + (Hk, G, sh[3])).sum(3)
    errs = _grad_errs(g, r)
    print("  " + " ".join("%s=%.2e" % kv for kv in errs.items()))
    for n, e in errs.items():
        assert e < TOL[dtype], (n, e)


@pytest.mark.parametrize("dtype,chunk,d,gate_dtype,arm", [
    ("f32", 32, 32, "f32", "ckda"), ("f32", 16, 16, "f32", "kda"),
    ("bf16", 64, 128, "bf16", "ckda"), ("bf16", 64, 128, "f32", "kda"),
    ("bf16", 32, 64, "bf16", "kda")])
def test_bwd_gate_logits(dtype, chunk, d, gate_dtype, arm):
    """Gates given as logits: the gradients of the logits a, b (and of q, k,
    v, h0) against the oracle's gradients taken through its activation."""
    announce("bwd logits %s C=%d d=%d %s logits, %s range" % (dtype, chunk, d, gate_dtype, arm))
    rng = np.random.default_rng(1500 + d + chunk)
    c = _grad_case(1500 + d, 2, 2 * chunk + 11, 2, d, dtype)
    if arm == "ckda":
        c["alpha"] = rng.normal(2, 2, c["alpha"].shape).astype(np.float32)
        c["alpha"][rng.random(c["alpha"].shape) < 0.02] = 0.0  # exact zero gates
    else:
        c["alpha"] = rng.normal(2, 1, c["alpha"].shape).astype(np.float32)
    c["beta"] = rng.normal(0, 1, c["beta"].shape).astype(np.float32)
    _check_general(c, dtype, chunk, gates="logits", arm=arm, gate_dtype=gate_dtype)


@pytest.mark.parametrize("dtype,chunk,d,Hk", [("f32", 32, 32, 2), ("f32", 16, 16, 1),
                                              ("bf16", 64, 128, 2), ("bf16", 32, 64, 1)])
def test_bwd_grouped_value_heads(dtype, chunk, d, Hk):
    """q, k on Hk heads serving H = 4 value heads: dq, dk of a q/k head are
    the sums over its value heads."""
    announce("bwd grouped heads %s C=%d d=%d Hk=%d" % (dtype, chunk, d, Hk))
    c = _grad_case(1600 + d + Hk, 2, 2 * chunk + 3, 4, d, dtype)
    _check_general(c, dtype, chunk, Hk=Hk)


def test_bwd_logits_grouped_packed():
    """bf16 logits, two q/k heads for four value heads, a packed batch with
    an empty sequence, chunk 64 at d = 128."""
    announce("bwd logits + grouped heads + packed")
    lens = [150, 0, 64, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    c = _grad_case(1700, 1, cu[-1], 4, 128, "bf16", cu=cu)
    rng = np.random.default_rng(1701)
    c["alpha"] = rng.normal(2, 2, c["alpha"].shape).astype(np.float32)
    c["beta"] = rng.normal(0, 1, c["beta"].shape).astype(np.float32)
    _check_general(c, "bf16", 64, gates="logits", gate_dtype="bf16", Hk=2)
