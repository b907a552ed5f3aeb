"""GPU parity of the fused gate activation: the chunked forward and the decode
step take pre-activation logits (float32 or bfloat16) and form the gates in
the kernels (CKDA range: alpha = 2 sigmoid(a) - 1, beta = 2 sigmoid(b); KDA
range: sigmoid for both), checked against the oracle's activation followed by
its recurrence."""
import numpy as np
import pytest
import torch

import gated_delta_rule_ckda_amd as ck
import oracle
from gated_delta_rule_ckda_amd import inputs
from tests.gpu_util import (DEV, TOL, announce, cover_pairs, dev, host, max_rel_err, oracle_gates,
                            oracle_pairs, run_chunk)

pytestmark = pytest.mark.gpu


def _check(case, tol=None):
    o, ht = run_chunk(case)
    ga, gb = oracle_gates(case, case.alpha, case.beta)
    ro, rh = oracle.fwd(case.q, case.k, case.v, ga, gb, h0=case.h0,
                        seq_start=case.cu_seqlens, use_l2norm=case.l2norm)
    tol = tol or TOL[case.dtype]
    eo, eh = max_rel_err(o, ro), max_rel_err(ht, rh)
    print("  err o=%.3e ht=%.3e (tol %.0e)" % (eo, eh, tol))
    assert eo < tol and eh < tol


@pytest.mark.parametrize("arm", ["ckda", "kda"])
@pytest.mark.parametrize("spread", ["lm", "wide"])
@pytest.mark.parametrize("chunk,d", [(16, 16), (32, 32), (16, 64)])
def test_chunk_f32_logits(arm, spread, chunk, d):
    announce("chunk f32 logits arm=%s spread=%s C=%d d=%d" % (arm, spread, chunk, d))
    c = inputs.logit_case(500 + chunk + d, 2, 3 * chunk + 5, 3, d, d, dtype="f32", chunk=chunk,
                          arm=arm, spread=spread, zero_frac=0.02 if arm == "ckda" else 0.0,
                          h0_std=0.5)
    _check(c)


@pytest.mark.parametrize("arm", ["ckda", "kda"])
@pytest.mark.parametrize("gate_dtype", ["bf16", "f32"])
@pytest.mark.parametrize("chunk,d", [(64, 128), (32, 64), (16, 128)])
def test_chunk_bf16_logits(arm, gate_dtype, chunk, d):
    announce("chunk bf16 io, %s logits arm=%s C=%d d=%d" % (gate_dtype, arm, chunk, d))
    c = inputs.logit_case(600 + chunk + d, 2, 4 * chunk + 7, 2, d, d, dtype="bf16", chunk=chunk,
                          arm=arm, gate_dtype=gate_dtype, spread="wide",
                          zero_frac=0.01 if arm == "ckda" else 0.0, h0_std=0.1)
    _check(c)


def test_chunk_packed_logits_with_empty_sequences():
    """Packed batch (with empty sequences) and bf16 logits: equal to the oracle
    per sequence."""
    announce("chunk packed bf16 logits")
    base = inputs.logit_case(701, 1, 300, 2, 64, 64, dtype="bf16", chunk=32, arm="ckda",
                             gate_dtype="bf16", spread="wide", zero_frac=0.01)
    base.cu_seqlens = np.array([0, 0, 77, 77, 200, 300], dtype=np.int32)
    base.h0 = (0.1 * np.random.default_rng(9).standard_normal((5, 2, 64, 64))).astype(np.float32)
    _check(base)


@pytest.mark.parametrize("arm", ["ckda", "kda"])
def test_lm_layer_bf16_logits_full_sampled(arm):
    """B=8 H=16 T=4096 d=128 bf16 chunk 64 with bf16 gate logits, at full size
    (the benchmark's logits configuration); oracle on sampled (batch, head)
    pairs."""
    announce("LM layer full size, bf16 logits, %s arm" % arm)
    c = inputs.lm_layer_logits(arm=arm)
    o, ht = run_chunk(c)
    o = o.reshape(c.v.shape)
    pairs = cover_pairs(8, 16)
    ref = oracle_pairs(c, pairs)
    worst_o = max(max_rel_err(o[n, :, h], ref[(n, h)][0]) for n, h in pairs)
    worst_h = max(max_rel_err(ht[n, h], ref[(n, h)][1]) for n, h in pairs)
    print("  err o=%.3e ht=%.3e" % (worst_o, worst_h))
    assert worst_o < TOL["bf16"] and worst_h < TOL["bf16"]


def test_logits_match_values_path():
    """The logits path and the values path, fed the oracle's gates rounded to
    float32, agree to float32 rounding of the gates (same kernels otherwise)."""
    announce("logits vs values path")
    c = inputs.logit_case(801, 2, 200, 2, 32, 32, dtype="f32", chunk=32, arm="ckda",
                          spread="wide", h0_std=0.3)
    o1, h1 = run_chunk(c)
    ga, gb = oracle_gates(c, c.alpha, c.beta)
    cv = inputs.Case(c.q, c.k, c.v, ga.astype(np.float32), gb.astype(np.float32), c.h0, None,
                     "f32", 32, True)
    o2, h2 = run_chunk(cv)
    assert max_rel_err(o1, o2) < 1e-5 and max_rel_err(h1, h2) < 1e-5


def _step_logits(rng, N, H, d, dtype, gate_dtype):
    c = inputs.logit_case(int(rng.integers(1 << 30)), N, 1, H, d, d, dtype=dtype,
                          arm="ckda", gate_dtype=gate_dtype, spread="wide")
    return (x.reshape((N, H) + x.shape[3:]) for x in (c.q, c.k, c.v, c.alpha)), \
        c.beta.reshape(N, H)


@pytest.mark.parametrize("arm", ["ckda", "kda"])
@pytest.mark.parametrize("dtype,gate_dtype", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("d", [32, 128])
def test_decode_logits(arm, dtype, gate_dtype, d):
    announce("decode logits arm=%s io=%s gates=%s d=%d" % (arm, dtype, gate_dtype, d))
    rng = np.random.default_rng(d + len(dtype) + len(gate_dtype))
    N, H = 9, 3
    (q, k, v, a), b = _step_logits(rng, N, H, d, dtype, gate_dtype)
    st0 = (0.1 * rng.standard_normal((N, H, d, d))).astype(np.float32)
    st = dev(st0)
    o = ck.recurrent_step(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(a, gate_dtype),
                          dev(b, gate_dtype), st, gate=arm, gates="logits")
    torch.cuda.synchronize()
    ga, gb = oracle.gates(a, b, ckda_range=(arm == "ckda"))
    ro, rs = oracle.step(q, k, v, ga, gb, st0)
    tol = TOL[dtype]
    assert max_rel_err(host(o), ro) < tol and max_rel_err(host(st), rs) < tol


@pytest.mark.parametrize("gate_dtype", ["f32", "bf16"])
def test_gate_limits_exact(gate_dtype):
    """Logits 0 and +-inf give the exact gates the definition fixes (CKDA
    range: alpha(0) = 0, alpha(+-inf) = +-1; beta(-inf) = 0), and huge logits
    give +-1 after rounding.  With beta = 0 the step is S' = Diag(alpha) S,
    so the new state is bit-exactly alpha * S, in both the decode step and
    the chunked forward."""
    announce("gate limits exact (%s logits)" % gate_dtype)
    N, H, d = 2, 2, 32
    rng = np.random.default_rng(5)
    av = np.array([0.0, np.inf, -np.inf, 200.0, -200.0, 0.0, 60.0, -60.0], np.float32)
    expect = np.array([0.0, 1.0, -1.0, 1.0, -1.0, 0.0, 1.0, -1.0])
    a = np.resize(av, (N, H, d)).astype(np.float32)
    ea = np.resize(expect, (N, H, d))
    b = np.full((N, H), -np.inf, np.float32)
    q = rng.standard_normal((N, H, d)).astype(np.float32)
    k = rng.standard_normal((N, H, d)).astype(np.float32)
    v = rng.standard_normal((N, H, d)).astype(np.float32)
    st0 = rng.standard_normal((N, H, d, d)).astype(np.float32)
    st = dev(st0)
    ck.recurrent_step(dev(q), dev(k), dev(v), dev(a, gate_dtype), dev(b, gate_dtype), st,
                      gate="ckda", gates="logits")
    torch.cuda.synchronize()
    assert np.array_equal(st.cpu().numpy(), (ea[..., None] * st0).astype(np.float32))
    # chunked forward: one token per sequence, the same gates
    o, ht = ck.chunk_fwd(dev(q[:, None]), dev(k[:, None]), dev(v[:, None]),
                         dev(a[:, None], gate_dtype), dev(b[:, None], gate_dtype), h0=dev(st0),
                         chunk_size=16, gate="ckda", gates="logits")
    torch.cuda.synchronize()
    assert np.array_equal(ht.cpu().numpy(), (ea[..., None] * st0).astype(np.float32))


@pytest.mark.parametrize("gate_dtype", ["f32", "bf16"])
def test_tiny_logits_give_tiny_gates(gate_dtype):
    """Logits near 0 give gates of about a/2 (tanh(a/2)), not an exact 0 (no
    cancellation in 2 sigmoid(a) - 1): with beta = 0 the new state is
    alpha * S, checked per element to 1e-6 relative in the decode step and
    the chunked forward."""
    announce("tiny logits (%s)" % gate_dtype)
    N, H, d = 2, 2, 32
    rng = np.random.default_rng(6)
    av = np.array([1e-9, -3e-8, 2e-6, -1e-3, 0.3, -0.45, 0.55, 1e-30], np.float32)
    a = inputs.round_bf16(av) if gate_dtype == "bf16" else av
    a = np.resize(a, (N, H, d)).astype(np.float32)
    expect = np.tanh(a.astype(np.float64) / 2)
    b = np.full((N, H), -np.inf, np.float32)
    q, k, v = (rng.standard_normal((N, H, d)).astype(np.float32) for _ in range(3))
    st0 = rng.standard_normal((N, H, d, d)).astype(np.float32)
    st = dev(st0)
    ck.recurrent_step(dev(q), dev(k), dev(v), dev(a, gate_dtype), dev(b, gate_dtype), st,
                      gate="ckda", gates="logits")
    _, ht = ck.chunk_fwd(dev(q[:, None]), dev(k[:, None]), dev(v[:, None]),
                         dev(a[:, None], gate_dtype), dev(b[:, None], gate_dtype),
                         h0=dev(st0), chunk_size=16, gate="ckda", gates="logits")
    torch.cuda.synchronize()
    ref = expect[..., None] * st0
    for got in (host(st), host(ht)):
        rel = np.abs(got - ref) / np.maximum(np.abs(ref), 1e-45)
        assert rel.max() < 1e-6, rel.max()
