"""ckda_chunk_fwd_noalloc: the chunked forward on the library's static
per-GPU scratch instead of a caller workspace, for callers that cannot
allocate.  Checked through the C ABI against ckda_chunk_fwd on the same
inputs (same kernels, so bit for bit) and against the oracle, on two calls in
a row, the second with a smaller input than the first."""
import ctypes

import numpy as np
import pytest
import torch

import gated_delta_rule_ckda_amd as ck
from gated_delta_rule_ckda_amd import inputs
from tests.gpu_util import DEV, TOL, announce, dev, host, max_rel_err, oracle_pairs

pytestmark = pytest.mark.gpu


def _both(c):
    """(o, ht) from ckda_chunk_fwd and from ckda_chunk_fwd_noalloc."""
    cu = None if c.cu_seqlens is None else torch.from_numpy(c.cu_seqlens).to(DEV)
    args = (dev(c.q, c.dtype), dev(c.k, c.dtype), dev(c.v, c.dtype), dev(c.alpha), dev(c.beta))
    kw = dict(h0=None if c.h0 is None else dev(c.h0), cu_seqlens=cu, chunk_size=c.chunk,
              use_qk_l2norm=c.l2norm)
    o1, h1 = ck.chunk_fwd(*args, **kw)
    o2, h2 = ck.chunk_fwd_noalloc(*args, **kw)
    torch.cuda.synchronize()
    return (host(o1), host(h1)), (host(o2), host(h2))


def _check(c, pairs):
    (o1, h1), (o2, h2) = _both(c)
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)
    ref = oracle_pairs(c, pairs)
    if c.cu_seqlens is None:
        o = o2.reshape(c.v.shape)
        eo = max(max_rel_err(o[n, :, h], ref[(n, h)][0]) for n, h in pairs)
    else:
        cs = c.cu_seqlens
        eo = max(max_rel_err(o2[0, cs[n]:cs[n + 1], h], ref[(n, h)][0]) if cs[n + 1] > cs[n]
                 else 0.0 for n, h in pairs)
    eh = max(max_rel_err(h2[n, h], ref[(n, h)][1]) for n, h in pairs)
    print("  err o=%.3e ht=%.3e" % (eo, eh))
    tol = TOL[c.dtype]
    assert eo < tol and eh < tol


def test_noalloc_matches_chunk_fwd_twice_second_smaller():
    # first call: dense bf16 batch, several chunks and a ragged tail, h0 given
    announce("noalloc call 1: dense bf16 B=2 T=700 H=4 d=128 chunk 64")
    c1 = inputs.random_case(91, 2, 700, 4, 128, 128, dtype="bf16", chunk=64, alpha="tanh",
                            beta="2sig", h0_std=0.1)
    _check(c1, [(0, 0), (1, 3), (0, 2), (1, 1)])
    # second call, smaller: a packed batch with an empty sequence
    announce("noalloc call 2: packed bf16 lengths 130, 0, 61 H=2 d=128 chunk 64")
    lens = [130, 0, 61]
    big = inputs.random_case(92, 1, sum(lens), 2, 128, 128, dtype="bf16", chunk=64,
                             alpha="tanh", beta="2sig")
    h0 = (0.1 * np.random.default_rng(94).standard_normal((len(lens), 2, 128, 128))).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    c2 = inputs.Case(big.q, big.k, big.v, big.alpha, big.beta, h0, cu, "bf16", 64, True)
    _check(c2, [(0, 0), (0, 1), (1, 0), (2, 1)])


def test_noalloc_fp32_small_shape():
    announce("noalloc fp32 B=3 T=45 H=2 d=16 chunk 16")
    c = inputs.random_case(93, 3, 45, 2, 16, 16, dtype="f32", chunk=16, alpha="uniform",
                           beta="uniform", h0_std=0.5)
    _check(c, [(0, 0), (1, 1), (2, 0)])


def test_noalloc_refuses_a_call_beyond_the_scratch():
    """A descriptor whose workspace exceeds the static scratch is refused on
    the host (CKDA_ERR_WORKSPACE_TOO_SMALL), with nothing launched: o keeps
    its contents."""
    B, T, H, d = 4, 8192, 16, 128
    desc = ck.FwdDesc(B, T, H, d, d, B, 64, ck.BF16, ck.GATE_CKDA, 1, 1.0, ck.GATES_F32, H, 0)
    assert ck.chunk_fwd_workspace_size(desc, False) > ck.NOALLOC_SCRATCH_BYTES
    o = torch.full((16,), 7.0, device=DEV)
    p = ctypes.c_void_p(o.data_ptr())
    st = ck._load().ckda_chunk_fwd_noalloc(ctypes.byref(desc), p, p, p, p, p, None, None, p,
                                           None, None)
    assert st == 3
    assert "static scratch" in ck._load().ckda_last_error().decode()
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())
