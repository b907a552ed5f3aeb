"""Helpers for the GPU parity tests (host-side marshalling and error metrics)."""
import sys

import numpy as np
import torch

DEV = "cuda:0"


def dev(x, dtype="f32"):
    """numpy float32 -> device tensor in the io dtype (bf16 values must already
    be bf16-representable, so the conversion is exact)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_rel_err(x, ref):
    """max |x - ref| / max |ref| over the whole tensor."""
    ref = np.asarray(ref, dtype=np.float64)
    den = np.abs(ref).max()
    return float(np.abs(np.asarray(x, dtype=np.float64) - ref).max() / (den if den > 0 else 1.0))


def announce(msg):
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


TOL = {"f32": 1e-4, "bf16": 2e-2}


def run_chunk(case, chunk=None, h0=None, ht=True, gate=None, scale=1.0, l2=None):
    """Run ckda_chunk_fwd on an inputs.Case; returns (o, ht) as fp64 numpy."""
    import gated_delta_rule_ckda_amd as ck
    dt = case.dtype
    cu = None if case.cu_seqlens is None else torch.from_numpy(case.cu_seqlens).to(DEV)
    h0a = case.h0 if h0 is None else h0
    o, st = ck.chunk_fwd(dev(case.q, dt), dev(case.k, dt), dev(case.v, dt),
                         dev(case.alpha, case.gate_dtype), dev(case.beta, case.gate_dtype),
                         h0=None if h0a is None else dev(h0a), cu_seqlens=cu,
                         chunk_size=chunk or case.chunk,
                         use_qk_l2norm=case.l2norm if l2 is None else l2,
                         gate=gate or case.arm, scale=scale, output_final_state=ht,
                         gates=case.gates)
    torch.cuda.synchronize()
    return host(o), (None if st is None else host(st))


def oracle_gates(case, a, b):
    """The gates the oracle runs on: the case's own, or the oracle's activation
    of its logits."""
    import oracle
    if case.gates == "logits":
        return oracle.gates(a, b, ckda_range=(case.arm == "ckda"))
    return a, b


def cover_pairs(N, H, extra=()):
    """(sequence, head) pairs in which every sequence index and every head
    index appears at least once: max(N, H) pairs, head (5 i + 3) mod H with
    sequence i mod N (5 is odd, so for a power-of-two H the heads are a
    permutation), plus `extra`."""
    n = max(N, H)
    step = 5 if np.gcd(5, H) == 1 else 1
    pairs = [(i % N, (step * i + 3) % H) for i in range(n)]
    for p in extra:
        if p not in pairs:
            pairs.append(p)
    return pairs


def oracle_pairs(case, pairs, scale=1.0):
    """Oracle on selected (sequence, head) pairs of a case; returns
    {(n,h): (o [T_n, dv], ht [dk, dv])}.  Pairs are independent, so this is the
    exact reference for those outputs.  All pairs go to the oracle in one
    packed call (one sequence per pair, one head), which it runs in parallel."""
    import oracle
    out = {}
    if case.cu_seqlens is None:
        starts = np.arange(case.q.shape[0] + 1) * case.q.shape[1]
        q, k, v, a, b = (x.reshape((-1,) + x.shape[2:]) for x in
                         (case.q, case.k, case.v, case.alpha, case.beta))
    else:
        starts = case.cu_seqlens.astype(np.int64)
        q, k, v, a, b = (x[0] for x in (case.q, case.k, case.v, case.alpha, case.beta))
    pairs = list(pairs)
    segs = [(int(starts[n]), int(starts[n + 1]), h) for n, h in pairs]

    def cat(x):
        return np.concatenate([x[s0:s1, h:h + 1] for s0, s1, h in segs], 0)[None]

    qs, ks, vs, as_, bs = (cat(x) for x in (q, k, v, a, b))
    ga, gb = oracle_gates(case, as_, bs)
    seq_start = np.concatenate([[0], np.cumsum([s1 - s0 for s0, s1, _ in segs])]).astype(np.int64)
    h0 = None
    if case.h0 is not None:
        h0 = np.stack([case.h0[n, h:h + 1] for n, h in pairs], 0)
    o, ht = oracle.fwd(qs, ks, vs, ga, gb, h0=h0, seq_start=seq_start,
                       use_l2norm=case.l2norm, scale=scale)
    for i, p in enumerate(pairs):
        out[p] = (o[0, seq_start[i]:seq_start[i + 1], 0], ht[i, 0])
    return out
