"""Grouped value heads (q and k with Hk heads, v, gates and state with H, a
multiple of Hk): value head h reads query/key head h // (H // Hk), the
repeat of q and k over the value heads (dormouse review "RoPE into the KDA
q/k path", section 7).  Parity against the oracle run on the repeated q and
k, and bit-exact agreement with the same call made on repeated q and k."""
import numpy as np
import pytest
import torch

import gated_delta_rule_ckda_amd as ck
import oracle
from gated_delta_rule_ckda_amd import inputs
from tests.gpu_util import DEV, TOL, announce, dev, host, max_rel_err, run_chunk

pytestmark = pytest.mark.gpu


def repeat_qk(case):
    """The case with q and k repeated over the value heads (H heads each)."""
    G = case.v.shape[-2] // case.q.shape[-2]
    c = inputs.Case(np.repeat(case.q, G, axis=-2), np.repeat(case.k, G, axis=-2), case.v,
                    case.alpha, case.beta, case.h0, case.cu_seqlens, case.dtype, case.chunk,
                    case.l2norm, dict(case.meta), case.gates, case.gate_dtype, case.arm)
    return c


@pytest.mark.parametrize("dtype,chunk,d,Hk,H", [
    ("f32", 16, 32, 2, 4), ("f32", 32, 16, 1, 3), ("f32", 16, 64, 2, 6),
    ("bf16", 64, 128, 2, 8), ("bf16", 32, 64, 1, 4), ("bf16", 16, 128, 4, 8)])
def test_gva_chunk_parity_and_repeat_identity(dtype, chunk, d, Hk, H):
    announce("GVA chunk %s C=%d d=%d Hk=%d H=%d" % (dtype, chunk, d, Hk, H))
    c = inputs.gva_case(900 + chunk + d + H, 2, 3 * chunk + 9, Hk, H, d, d, dtype=dtype,
                        chunk=chunk, h0_std=0.3, zero_frac=0.01)
    o, ht = run_chunk(c)
    r = repeat_qk(c)
    o2, ht2 = run_chunk(r)
    assert np.array_equal(o, o2) and np.array_equal(ht, ht2)
    ro, rh = oracle.fwd(r.q, r.k, r.v, r.alpha, r.beta, h0=r.h0, use_l2norm=True)
    tol = TOL[dtype]
    eo, eh = max_rel_err(o, ro), max_rel_err(ht, rh)
    print("  err o=%.3e ht=%.3e (tol %.0e)" % (eo, eh, tol))
    assert eo < tol and eh < tol


def test_gva_packed_with_logits():
    announce("GVA packed, bf16 logits")
    c = inputs.gva_case(950, 1, 260, 2, 6, 64, 64, dtype="bf16", chunk=32, zero_frac=0.005)
    rng = np.random.default_rng(3)
    c.alpha = inputs.round_bf16(rng.uniform(-8, 8, c.alpha.shape).astype(np.float32))
    c.beta = inputs.round_bf16(rng.uniform(-6, 6, c.beta.shape).astype(np.float32))
    c.gates, c.gate_dtype = "logits", "bf16"
    c.cu_seqlens = np.array([0, 100, 100, 260], dtype=np.int32)
    c.h0 = (0.1 * rng.standard_normal((3, 6, 64, 64))).astype(np.float32)
    o, ht = run_chunk(c)
    r = repeat_qk(c)
    o2, ht2 = run_chunk(r)
    assert np.array_equal(o, o2) and np.array_equal(ht, ht2)
    ga, gb = oracle.gates(c.alpha, c.beta, ckda_range=True)
    ro, rh = oracle.fwd(r.q, r.k, r.v, ga, gb, h0=r.h0, seq_start=c.cu_seqlens, use_l2norm=True)
    assert max_rel_err(o, ro) < TOL["bf16"] and max_rel_err(ht, rh) < TOL["bf16"]


@pytest.mark.parametrize("dtype,d,Hk,H", [("bf16", 128, 4, 32), ("f32", 32, 1, 4),
                                          ("bf16", 64, 2, 6)])
def test_gva_decode(dtype, d, Hk, H):
    announce("GVA decode %s d=%d Hk=%d H=%d" % (dtype, d, Hk, H))
    N = 7
    c = inputs.gva_case(970 + d + H, N, 1, Hk, H, d, d, dtype=dtype)
    q, k = c.q[:, 0], c.k[:, 0]
    v, a, b = c.v[:, 0], c.alpha[:, 0], c.beta[:, 0]
    st0 = (0.1 * np.random.default_rng(4).standard_normal((N, H, d, d))).astype(np.float32)
    st = dev(st0)
    o = ck.recurrent_step(dev(q, dtype), dev(k, dtype), dev(v, dtype), dev(a), dev(b), st)
    G = H // Hk
    qr, kr = np.repeat(q, G, axis=1), np.repeat(k, G, axis=1)
    st2 = dev(st0)
    o2 = ck.recurrent_step(dev(qr, dtype), dev(kr, dtype), dev(v, dtype), dev(a), dev(b), st2)
    torch.cuda.synchronize()
    assert np.array_equal(host(o), host(o2)) and np.array_equal(host(st), host(st2))
    ro, rs = oracle.step(qr, kr, v, a, b, st0)
    assert max_rel_err(host(o), ro) < TOL[dtype] and max_rel_err(host(st), rs) < TOL[dtype]
