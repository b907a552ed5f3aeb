"""The training-step split: ckda_chunk_fwd_save writes the forward's o and ht
and keeps the backward's records; ckda_chunk_bwd_saved reads them instead of
recomputing the forward.  Both must match the unsplit calls bit for bit (the
records are the same kernels' output on the same inputs), and the saved
backward must be repeatable on one save (it only reads the records)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_ckda_amd as ck
import oracle
from gated_delta_rule_ckda_amd import inputs
from tests.gpu_util import DEV, announce, dev, host, max_rel_err

pytestmark = pytest.mark.gpu

NAMES = ["dq", "dk", "dv", "dalpha", "dbeta", "dh0"]


def _case(seed, B, T, H, Hk, d, dtype, gates, gate_dtype, lens=None):
    rng = np.random.default_rng(seed)
    if lens is not None:
        B, T = 1, int(sum(lens))
    q, k = (rng.standard_normal((B, T, Hk, d)).astype(np.float32) for _ in range(2))
    v, dO = (rng.standard_normal((B, T, H, d)).astype(np.float32) for _ in range(2))
    if gates == "logits":
        a = rng.normal(2, 2, (B, T, H, d)).astype(np.float32)
        b = rng.normal(0, 1, (B, T, H)).astype(np.float32)
        a[rng.random(a.shape) < 0.02] = 0.0  # logits of 0 (alpha exactly 0 in the CKDA range)
    else:
        a = (np.tanh(rng.normal(2, 1, (B, T, H, d))) * rng.choice([-1, 1], (B, T, H, d)))
        a[rng.random(a.shape) < 0.01] = 0.0  # exact zero gates: the redo launch and token path
        m = rng.random(a.shape) < 0.03
        a[m] = rng.choice([-1, 1], m.sum()) * 1e-4
        a = a.astype(np.float32)
        b = rng.uniform(0, 2, (B, T, H)).astype(np.float32)
    if gates == "logits" and gate_dtype == "bf16":
        a, b = inputs.round_bf16(a), inputs.round_bf16(b)
    N = B if lens is None else len(lens)
    h0 = (0.3 * rng.standard_normal((N, H, d, d))).astype(np.float32)
    dht = rng.standard_normal((N, H, d, d)).astype(np.float32)
    if dtype == "bf16":
        q, k, v, dO = (inputs.round_bf16(x) for x in (q, k, v, dO))
    cu = None if lens is None else np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return dict(q=q, k=k, v=v, a=a, b=b, dO=dO, h0=h0, dht=dht, cu=cu)


CASES = [
    # dtype, chunk, d, H, Hk, gates, gate dtype, packed lengths
    ("bf16", 64, 128, 4, 4, "values", "f32", None),
    ("bf16", 32, 64, 4, 2, "values", "f32", None),
    ("f32", 32, 32, 3, 3, "values", "f32", None),
    ("f32", 16, 64, 2, 1, "logits", "f32", None),
    ("bf16", 64, 128, 4, 2, "logits", "bf16", [150, 0, 64, 33]),
    ("bf16", 64, 64, 2, 2, "values", "f32", [0, 300, 17, 64, 129]),
]


@pytest.mark.parametrize("dtype,chunk,d,H,Hk,gates,gate_dtype,lens", CASES)
def test_fwd_save_and_bwd_saved_match_the_unsplit_calls(dtype, chunk, d, H, Hk, gates,
                                                          gate_dtype, lens):
    announce("fwd_save / bwd_saved %s C=%d d=%d H=%d Hk=%d %s %s packed=%s"
             % (dtype, chunk, d, H, Hk, gates, gate_dtype, lens is not None))
    c = _case(1800 + d + chunk + Hk, 2, 3 * chunk + 7, H, Hk, d, dtype, gates, gate_dtype, lens)
    cu = None if c["cu"] is None else torch.from_numpy(c["cu"]).to(DEV)
    gdt = gate_dtype if gates == "logits" else "f32"
    args = (dev(c["q"], dtype), dev(c["k"], dtype), dev(c["v"], dtype), dev(c["a"], gdt),
            dev(c["b"], gdt))
    kw = dict(h0=dev(c["h0"]), cu_seqlens=cu, chunk_size=chunk, gates=gates)
    o1, ht1 = ck.chunk_fwd(*args, **kw)
    o2, ht2, saved = ck.chunk_fwd_save(*args, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)
    dO = dev(c["dO"], dtype)
    bkw = dict(kw, dht=dev(c["dht"]))
    g_re = [host(x) for x in ck.chunk_bwd(*args, dO, **bkw)]
    g_s1 = [host(x) for x in ck.chunk_bwd(*args, dO, saved=saved, **bkw)]
    g_s2 = [host(x) for x in ck.chunk_bwd(*args, dO, saved=saved, **bkw)]
    torch.cuda.synchronize()
    for n, x, y, z in zip(NAMES, g_re, g_s1, g_s2):
        assert np.array_equal(x, y), n
        assert np.array_equal(y, z), n


def test_bwd_saved_against_the_oracle():
    """One saved backward checked against the oracle's gradients directly
    (bf16, chunk 64, d = 128, packed batch with an empty sequence)."""
    announce("bwd_saved vs oracle bf16 C=64 d=128 packed")
    lens = [0, 200, 77, 64]
    c = _case(1900, 1, 0, 2, 2, 128, "bf16", "values", "f32", lens)
    cu = torch.from_numpy(c["cu"]).to(DEV)
    args = (dev(c["q"], "bf16"), dev(c["k"], "bf16"), dev(c["v"], "bf16"), dev(c["a"]),
            dev(c["b"]))
    kw = dict(h0=dev(c["h0"]), cu_seqlens=cu, chunk_size=64)
    _, _, saved = ck.chunk_fwd_save(*args, **kw)
    g = ck.chunk_bwd(*args, dev(c["dO"], "bf16"), dht=dev(c["dht"]), saved=saved, **kw)
    torch.cuda.synchronize()
    g = [host(x) for x in g]
    r = oracle.bwd(c["q"], c["k"], c["v"], c["a"], c["b"], c["dO"], h0=c["h0"], dht=c["dht"],
                   seq_start=c["cu"].tolist())
    errs = {n: max_rel_err(x, y) for n, x, y in zip(NAMES, g, r)}
    print("  " + " ".join("%s=%.2e" % kv for kv in errs.items()))
    for n, e in errs.items():
        assert e < 2e-2, (n, e)


def test_training_step_split_at_full_size():
    """The LM layer at full size (B=8, T=4096, H=16, d=128, bf16, chunk 64),
    with 648 exact zero gates (so the transform pass's second launch and the
    backward's token path take part): ckda_chunk_fwd_save's o, ht and
    ckda_chunk_bwd_saved's six gradients equal ckda_chunk_fwd's and
    ckda_chunk_bwd's bit for bit."""
    announce("fwd_save / bwd_saved LM layer full size with zero gates")
    c = inputs.zero_gates(inputs.lm_layer(arm="ckda"))
    rng = np.random.default_rng(78)
    args = (dev(c.q, "bf16"), dev(c.k, "bf16"), dev(c.v, "bf16"), dev(c.alpha), dev(c.beta))
    dO = dev(inputs.round_bf16(rng.standard_normal(c.v.shape).astype(np.float32)), "bf16")
    dht = dev(rng.standard_normal((8, 16, 128, 128)).astype(np.float32))
    o1, ht1 = ck.chunk_fwd(*args, chunk_size=64)
    o2, ht2, saved = ck.chunk_fwd_save(*args, chunk_size=64)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)
    del o1, ht1, o2, ht2
    g1 = ck.chunk_bwd(*args, dO, dht=dht, chunk_size=64)
    g2 = ck.chunk_bwd(*args, dO, dht=dht, chunk_size=64, saved=saved)
    torch.cuda.synchronize()
    for n, x, y in zip(NAMES, g1, g2):
        assert torch.equal(x, y), n
