"""The entry points under HIP graph capture: a chunked forward (with a
caller workspace, and on the library's static scratch) and a run of decode
steps, captured once and replayed several times with fresh inputs and eager
work between the replays.  The library enqueues only kernel launches (no
memsets, copies or allocations), so every replay must equal the eager call
on the same inputs bit for bit; the first replay of the forward is also held
to the oracle."""
import numpy as np
import pytest
import torch

import gated_delta_rule_ckda_amd as ck
from gated_delta_rule_ckda_amd import inputs
from tests.gpu_util import DEV, TOL, announce, dev, host, max_rel_err, oracle_pairs

pytestmark = pytest.mark.gpu


def _fwd_inputs(seed):
    c = inputs.random_case(seed, 2, 300, 4, 128, 128, dtype="bf16", chunk=64, alpha="tanh",
                           beta="2sig", h0_std=0.02)
    return c, [dev(c.q, "bf16"), dev(c.k, "bf16"), dev(c.v, "bf16"), dev(c.alpha), dev(c.beta),
               dev(c.h0)]


@pytest.mark.parametrize("noalloc", [False, True])
def test_chunk_fwd_graph_replays_equal_eager(noalloc):
    announce("chunk fwd under graph capture, noalloc=%s" % noalloc)
    c0, bufs = _fwd_inputs(4000)
    q, k, v, a, b, h0 = bufs
    o = torch.empty_like(v)
    ht = torch.empty((2, 4, 128, 128), device=DEV)
    desc = ck._make_desc(q, v, 4, 128, 128, 64, "ckda", True, 1.0, None, ck.GATES_F32, False)
    ws = torch.empty(ck.chunk_fwd_workspace_size(desc, False), device=DEV, dtype=torch.uint8)
    kw = dict(h0=h0, chunk_size=64, out=o, final_state=ht)

    def call():
        if noalloc:
            ck.chunk_fwd_noalloc(q, k, v, a, b, **kw)
        else:
            ck.chunk_fwd(q, k, v, a, b, workspace=ws, **kw)

    call()  # eager first call: one-time set-up happens outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(3):
        c, fresh = _fwd_inputs(4000 + r)
        for dst, src in zip(bufs, fresh):
            dst.copy_(src)
        g.replay()
        torch.cuda.synchronize()
        og, hg = host(o), host(ht)
        # eager on the same inputs, into other outputs and another workspace
        oe, he = ck.chunk_fwd(q, k, v, a, b, h0=h0, chunk_size=64)
        torch.cuda.synchronize()
        assert np.array_equal(og, host(oe)) and np.array_equal(hg, host(he)), r
        if r == 0:
            pairs = [(0, 0), (1, 3), (0, 2), (1, 1)]
            ref = oracle_pairs(c, pairs)
            o4 = og.reshape(c.v.shape)
            eo = max(max_rel_err(o4[n, :, h], ref[(n, h)][0]) for n, h in pairs)
            eh = max(max_rel_err(hg[n, h], ref[(n, h)][1]) for n, h in pairs)
            print("  replay 0: err o=%.3e ht=%.3e" % (eo, eh))
            assert eo < TOL["bf16"] and eh < TOL["bf16"]


def test_decode_steps_graph_replays_equal_eager():
    announce("decode steps under graph capture")
    N, H, d, steps = 8, 4, 128, 4
    s0 = dev(inputs.decode_state(seed=4100, N=N, H=H, d=d))
    st = s0.clone()
    toks = []
    for s in range(steps):
        q, k, v, a, b = inputs.decode_token(s, seed=4100, N=N, H=H, d=d)
        toks.append((dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), dev(a), dev(b)))
    outs = [torch.empty((N, H, d), device=DEV, dtype=torch.bfloat16) for _ in range(steps)]

    def run(state, dst):
        for (q, k, v, a, b), o in zip(toks, dst):
            ck.recurrent_step(q, k, v, a, b, state, out=o)

    run(st, outs)  # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(st, outs)
    for r in range(3):
        st.copy_(s0)
        g.replay()
        torch.cuda.synchronize()
        got = [host(o) for o in outs] + [host(st)]
        se = s0.clone()
        oe = [torch.empty_like(o) for o in outs]
        run(se, oe)
        torch.cuda.synchronize()
        want = [host(o) for o in oe] + [host(se)]
        assert all(np.array_equal(x, y) for x, y in zip(got, want)), r
