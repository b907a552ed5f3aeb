"""Sizes where 32-bit offsets would wrap: a long-context chunked forward
(4 sequences of 69,632 tokens) whose workspace is above 4 GiB and whose gate
tensor is above 2 GiB, a backward over 64 heads whose workspace is above
4 GiB, and a decode step whose state has more than 2^31 elements (9.7 GB).  Inputs are drawn on the device (seeded); the sampled
(sequence, head) pairs are copied to the host and held to the oracle: o at
the bf16 bound, the fp32 state of the decode step at the fp32 bound."""
import numpy as np
import pytest
import torch

import gated_delta_rule_ckda_amd as ck
import oracle
from gated_delta_rule_ckda_amd import inputs
from tests.gpu_util import TOL, announce, host, max_rel_err

pytestmark = pytest.mark.gpu


def test_chunk_fwd_long_context_beyond_4gib_workspace():
    B, T, H, d = 4, 69632, 16, 128
    announce("chunk fwd B=%d T=%d H=%d d=%d bf16 (workspace above 4 GiB)" % (B, T, H, d))
    x = inputs.device_lm_like(5000, B, T, H, d)
    desc = ck._make_desc(x["q"], x["v"], H, d, d, 64, "ckda", True, 1.0, None, ck.GATES_F32,
                         False)
    need = ck.chunk_fwd_workspace_size(desc, False)
    alpha_bytes = x["alpha"].numel() * 4
    assert need > 4 << 30 and alpha_bytes > 2 << 30, (need, alpha_bytes)
    o, ht = ck.chunk_fwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], h0=x["h0"],
                         chunk_size=64)
    torch.cuda.synchronize()
    pairs = [(0, 0), (1, 5), (2, 10), (3, 15), (3, 0), (0, 15)]

    def sel(t):
        return np.stack([host(t[n, :, h]) for n, h in pairs], 0)[:, :, None]

    q, k, v, a = (sel(x[n]) for n in ("q", "k", "v", "alpha"))
    b = np.stack([host(x["beta"][n, :, h]) for n, h in pairs], 0)[:, :, None]
    h0 = np.stack([host(x["h0"][n, h]) for n, h in pairs], 0)[:, None]
    ro, rh = oracle.fwd(q, k, v, a, b, h0=h0, use_l2norm=True)
    eo = max(max_rel_err(host(o[n, :, h]), ro[i, :, 0]) for i, (n, h) in enumerate(pairs))
    eh = max(max_rel_err(host(ht[n, h]), rh[i, 0]) for i, (n, h) in enumerate(pairs))
    print("  err o=%.3e ht=%.3e" % (eo, eh))
    assert eo < TOL["bf16"] and eh < TOL["bf16"]


def test_decode_step_state_beyond_2pow31_elements():
    N, H, d = 4608, 32, 128
    announce("decode step N=%d H=%d d=%d (state above 2^31 elements)" % (N, H, d))
    x = inputs.device_decode(5100, N, H, d)
    st = x["state"]
    assert st.numel() > 1 << 31, st.numel()  # element offsets beyond int32
    pairs = [(0, 0), (1000, 7), (4095, 31), (4096, 16), (4607, 31), (4607, 0)]
    s0 = np.stack([host(st[n, h]) for n, h in pairs], 0)[:, None]
    o = ck.recurrent_step(x["q"], x["k"], x["v"], x["alpha"], x["beta"], st)
    torch.cuda.synchronize()

    def sel(t):
        return np.stack([host(t[n, h]) for n, h in pairs], 0)[:, None]

    ro, rs = oracle.step(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["alpha"]),
                         np.array([[float(x["beta"][n, h])] for n, h in pairs]), s0)
    eo = max(max_rel_err(host(o[n, h]), ro[i, 0]) for i, (n, h) in enumerate(pairs))
    es = max(max_rel_err(host(st[n, h]), rs[i, 0]) for i, (n, h) in enumerate(pairs))
    print("  err o=%.3e state=%.3e" % (eo, es))
    assert eo < TOL["bf16"] and es < TOL["f32"]


def test_chunk_bwd_beyond_4gib_workspace():
    B, T, H, d = 2, 16384, 64, 128
    announce("chunk bwd B=%d T=%d H=%d d=%d bf16 (workspace above 4 GiB)" % (B, T, H, d))
    x = inputs.device_lm_like(5200, B, T, H, d, grads=True)
    desc = ck._make_desc(x["q"], x["v"], H, d, d, 64, "ckda", True, 1.0, None, ck.GATES_F32,
                         False)
    need = ck.chunk_bwd_workspace_size(desc, False)
    assert need > 4 << 30, need
    g = ck.chunk_bwd(x["q"], x["k"], x["v"], x["alpha"], x["beta"], x["dout"], h0=x["h0"],
                     dht=x["dht"], chunk_size=64)
    torch.cuda.synchronize()
    pairs = [(0, 0), (1, 21), (0, 42), (1, 63), (1, 0), (0, 63)]

    def sel(t):
        return np.stack([host(t[n, :, h]) for n, h in pairs], 0)[:, :, None]

    q, k, v, a, dO = (sel(x[n]) for n in ("q", "k", "v", "alpha", "dout"))
    b = np.stack([host(x["beta"][n, :, h]) for n, h in pairs], 0)[:, :, None]
    h0 = np.stack([host(x["h0"][n, h]) for n, h in pairs], 0)[:, None]
    dht = np.stack([host(x["dht"][n, h]) for n, h in pairs], 0)[:, None]
    r = oracle.bwd(q, k, v, a, b, dO, h0=h0, dht=dht, use_l2norm=True)
    names = ["dq", "dk", "dv", "dalpha", "dbeta", "dh0"]
    errs = {}
    for j, name in enumerate(names):
        gj = g[j]
        if name == "dh0":
            got = np.stack([host(gj[n, h]) for n, h in pairs], 0)[:, None]
        elif name == "dbeta":
            got = np.stack([host(gj[n, :, h]) for n, h in pairs], 0)[:, :, None]
        else:
            got = sel(gj)
        errs[name] = max_rel_err(got, r[j])
    print("  " + " ".join("%s=%.2e" % kv for kv in errs.items()))
    for name, e in errs.items():
        assert e < TOL["bf16"], (name, e)
