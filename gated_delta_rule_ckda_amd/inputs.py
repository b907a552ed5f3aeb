"""Seeded synthetic inputs for the tests and the benchmark.

Shared by the GPU path's callers and the oracle's callers; it holds random
number generation and storage rounding only, none of the method's arithmetic.
Every array is float32 numpy; arrays that travel as bfloat16 are already
rounded to bfloat16 (round to nearest even), so the GPU and the oracle see
bit-identical values.  Generators use numpy's PCG64 (`default_rng`) with a
fixed draw order q, k, v, alpha, beta, h0.

Workloads (shapes and value distributions of the method's workloads; no
dataset is involved -- the word-problem, language-model and long-context
evaluations the pages mention are stood in for by these synthetic tensors):
  tiny           B=1 H=2 T=64 d=16 fp32 chunk 16, alpha~U[-1,1], beta~U[0,2]
  state_tracking B=256 H=4 T=512 d=32 fp32 chunk 32, unit keys, alpha in
                 {-1,+1} plus U[-0.05,0.05] jitter, beta~U[1.8,2], no l2norm
  lm_layer       B=8 H=16 T=4096 d=128 bf16 chunk 64, l2norm; CKDA arm
                 alpha=tanh(N(2,1)), beta=2 sigmoid(N(0,1)); KDA arm
                 alpha=sigmoid(N(2,1)), beta=sigmoid(N(0,1))
  varlen         16 packed sequences, 65536 tokens, H=16 d=128 bf16 chunk 64,
                 CKDA-arm gates, h0~N(0, 0.02^2)
  decode         256 sequences x 1 token, H=32 d=128, bf16 q/k/v, state
                 ~N(0, 0.02^2), alpha~U[-1,1], beta~U[0,2], fresh draws per step
  fast_decay     a case with a fraction of its key channels redrawn as
                 fast-decaying gates: |alpha| ~ U[0.15, 0.4] with a random
                 sign (products over 64 tokens reach ~2^-120, over 16 tokens
                 stay above 2^-44)
  *_logits       the same workloads with the gates given as pre-activation
                 logits (alpha and beta of the Case hold a and b): CKDA arm
                 a = 2 N(2,1), b = N(0,1), so that 2 sigmoid(a) - 1 =
                 tanh(N(2,1)) and 2 sigmoid(b) follow the value workloads'
                 laws; KDA arm a = N(2,1), b = N(0,1)
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np


def round_bf16(x) -> np.ndarray:
    """float32 -> nearest bfloat16 value (ties to even), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


@dataclass
class Case:
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    h0: Optional[np.ndarray]
    cu_seqlens: Optional[np.ndarray]
    dtype: str            # "bf16" or "f32": storage of q, k, v, o
    chunk: int
    l2norm: bool
    meta: dict = field(default_factory=dict)
    gates: str = "values"     # "values": alpha, beta are the gates; "logits": a, b
    gate_dtype: str = "f32"   # storage of alpha, beta ("bf16" only for logits)
    arm: str = "ckda"         # gate range: "ckda" or "kda"

    @property
    def shape(self):
        return self.q.shape


def _io(x, dtype):
    x = np.asarray(x, dtype=np.float32)
    return round_bf16(x) if dtype == "bf16" else x


def random_case(seed, B, T, H, dk, dv, *, dtype="f32", chunk=16, l2norm=True,
                alpha="uniform", beta="uniform", h0_std=0.0, zero_frac=0.0) -> Case:
    """Generic dense case: q,k,v ~ N(0,1); alpha ~ U[-1,1] ('uniform'),
    tanh(N(2,1)) ('tanh'), sigmoid(N(2,1)) ('sigmoid'); beta ~ U[0,2]
    ('uniform'), 2 sigmoid(N(0,1)) ('2sig'), sigmoid(N(0,1)) ('sig').
    zero_frac sets that fraction of alpha entries to exactly 0.  Without the
    in-kernel normalisation the keys are drawn as unit-norm directions (the
    method's range assumes unit keys; raw N(0,1) keys would make the
    recurrence expand)."""
    rng = np.random.default_rng(seed)
    q = _io(rng.standard_normal((B, T, H, dk), dtype=np.float32), dtype)
    k = rng.standard_normal((B, T, H, dk), dtype=np.float32)
    if not l2norm:
        k64 = k.astype(np.float64)
        k = (k64 / np.sqrt((k64 * k64).sum(-1, keepdims=True))).astype(np.float32)
    k = _io(k, dtype)
    v = _io(rng.standard_normal((B, T, H, dv), dtype=np.float32), dtype)
    if alpha == "uniform":
        a = rng.uniform(-1, 1, (B, T, H, dk)).astype(np.float32)
    elif alpha == "tanh":
        a = np.tanh(rng.normal(2, 1, (B, T, H, dk))).astype(np.float32)
    elif alpha == "sigmoid":
        a = _sigmoid(rng.normal(2, 1, (B, T, H, dk))).astype(np.float32)
    else:
        raise ValueError(alpha)
    if zero_frac > 0:
        a[rng.random(a.shape) < zero_frac] = 0.0
    if beta == "uniform":
        b = rng.uniform(0, 2, (B, T, H)).astype(np.float32)
    elif beta == "2sig":
        b = (2 * _sigmoid(rng.normal(0, 1, (B, T, H)))).astype(np.float32)
    elif beta == "sig":
        b = _sigmoid(rng.normal(0, 1, (B, T, H))).astype(np.float32)
    else:
        raise ValueError(beta)
    h0 = None
    if h0_std > 0:
        h0 = (h0_std * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    return Case(q, k, v, a, b, h0, None, dtype, chunk, l2norm,
                dict(B=B, T=T, H=H, dk=dk, dv=dv, seed=seed))


def logit_case(seed, B, T, H, dk, dv, *, dtype="f32", chunk=16, l2norm=True, arm="ckda",
               gate_dtype="f32", spread="lm", zero_frac=0.0, h0_std=0.0) -> Case:
    """Dense case with logit gates.  q,k,v ~ N(0,1) (unit keys without the
    in-kernel norm).  spread='lm': the LM-layer logit laws of the module
    docstring; spread='wide': a ~ U[-8,8], b ~ U[-6,6] (gates over the whole
    range, with many negative ones in the CKDA arm).  zero_frac sets that
    fraction of the a logits to exactly 0 (alpha = 0 in the CKDA range)."""
    rng = np.random.default_rng(seed)
    q = _io(rng.standard_normal((B, T, H, dk), dtype=np.float32), dtype)
    k = rng.standard_normal((B, T, H, dk), dtype=np.float32)
    if not l2norm:
        k64 = k.astype(np.float64)
        k = (k64 / np.sqrt((k64 * k64).sum(-1, keepdims=True))).astype(np.float32)
    k = _io(k, dtype)
    v = _io(rng.standard_normal((B, T, H, dv), dtype=np.float32), dtype)
    if spread == "lm":
        a = rng.normal(2, 1, (B, T, H, dk)) * (2.0 if arm == "ckda" else 1.0)
        b = rng.normal(0, 1, (B, T, H))
    elif spread == "wide":
        a = rng.uniform(-8, 8, (B, T, H, dk))
        b = rng.uniform(-6, 6, (B, T, H))
    else:
        raise ValueError(spread)
    a = _io(a.astype(np.float32), gate_dtype)
    b = _io(b.astype(np.float32), gate_dtype)
    if zero_frac > 0:
        a[rng.random(a.shape) < zero_frac] = 0.0
    h0 = None
    if h0_std > 0:
        h0 = (h0_std * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    return Case(q, k, v, a, b, h0, None, dtype, chunk, l2norm,
                dict(B=B, T=T, H=H, dk=dk, dv=dv, seed=seed), gates="logits",
                gate_dtype=gate_dtype, arm=arm)


def gva_case(seed, B, T, Hk, H, dk, dv, *, dtype="f32", chunk=16, l2norm=True, h0_std=0.0,
             zero_frac=0.0) -> Case:
    """Grouped value heads: q, k with Hk heads; v, alpha, beta, state with H
    heads (H a multiple of Hk).  q,k,v ~ N(0,1); alpha = tanh(N(2,1)) with
    zero_frac exact zeros; beta = 2 sigmoid(N(0,1))."""
    rng = np.random.default_rng(seed)
    q = _io(rng.standard_normal((B, T, Hk, dk), dtype=np.float32), dtype)
    k = _io(rng.standard_normal((B, T, Hk, dk), dtype=np.float32), dtype)
    v = _io(rng.standard_normal((B, T, H, dv), dtype=np.float32), dtype)
    a = np.tanh(rng.normal(2, 1, (B, T, H, dk))).astype(np.float32)
    if zero_frac > 0:
        a[rng.random(a.shape) < zero_frac] = 0.0
    b = (2 * _sigmoid(rng.normal(0, 1, (B, T, H)))).astype(np.float32)
    h0 = None
    if h0_std > 0:
        h0 = (h0_std * rng.standard_normal((B, H, dk, dv))).astype(np.float32)
    return Case(q, k, v, a, b, h0, None, dtype, chunk, l2norm,
                dict(B=B, T=T, H=H, Hk=Hk, dk=dk, dv=dv, seed=seed))


def tiny(seed=1000) -> Case:
    c = random_case(seed, 1, 64, 2, 16, 16, dtype="f32", chunk=16, l2norm=True)
    c.meta["workload"] = "tiny CKDA forward B=1 H=2 T=64 d=16 fp32"
    return c


def state_tracking(seed=1001, B=256, T=512, H=4, d=32) -> Case:
    """Near-orthogonal rotation regime: unit-norm random key directions,
    alpha = +-1 (p=1/2) plus U[-0.05,0.05] jitter clamped to [-1,1],
    beta ~ U[1.8,2.0], q,v ~ N(0,1), h0 = 0, no in-kernel normalisation."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, d), dtype=np.float32)
    k = rng.standard_normal((B, T, H, d)).astype(np.float64)
    k = (k / np.sqrt((k * k).sum(-1, keepdims=True))).astype(np.float32)
    v = rng.standard_normal((B, T, H, d), dtype=np.float32)
    sgn = np.where(rng.random((B, T, H, d)) < 0.5, -1.0, 1.0)
    a = np.clip(sgn + rng.uniform(-0.05, 0.05, (B, T, H, d)), -1, 1).astype(np.float32)
    b = rng.uniform(1.8, 2.0, (B, T, H)).astype(np.float32)
    return Case(q, k, v, a, b, None, None, "f32", 32, False,
                dict(B=B, T=T, H=H, dk=d, dv=d, seed=seed,
                     workload="state-tracking layer B=%d H=%d T=%d d=%d fp32" % (B, H, T, d)))


def lm_layer(seed=1002, arm="ckda", B=8, T=4096, H=16, d=128) -> Case:
    """1.3B-LM-shaped layer.  The KDA arm reuses the q/k/v draws and redraws
    alpha and beta from seed + 1000."""
    rng = np.random.default_rng(seed)
    q = round_bf16(rng.standard_normal((B, T, H, d), dtype=np.float32))
    k = round_bf16(rng.standard_normal((B, T, H, d), dtype=np.float32))
    v = round_bf16(rng.standard_normal((B, T, H, d), dtype=np.float32))
    if arm == "ckda":
        a = np.tanh(rng.normal(2, 1, (B, T, H, d)).astype(np.float32))
        b = (2 * _sigmoid(rng.normal(0, 1, (B, T, H)))).astype(np.float32)
    elif arm == "kda":
        rng2 = np.random.default_rng(seed + 1000)
        a = _sigmoid(rng2.normal(2, 1, (B, T, H, d)).astype(np.float32)).astype(np.float32)
        b = _sigmoid(rng2.normal(0, 1, (B, T, H))).astype(np.float32)
    else:
        raise ValueError(arm)
    return Case(q, k, v, a.astype(np.float32), b, None, None, "bf16", 64, True,
                dict(B=B, T=T, H=H, dk=d, dv=d, seed=seed, arm=arm,
                     workload="LM layer forward B=%d H=%d T=%d d=%d bf16 %s range"
                              % (B, H, T, d, arm.upper())), arm=arm)


def lm_layer_logits(seed=1002, arm="ckda", B=8, T=4096, H=16, d=128, gate_dtype="bf16") -> Case:
    """The LM layer with its gates as logits in gate_dtype (laws in the module
    docstring).  q/k/v are the same draws as lm_layer(seed); the logits come
    from seed + 2000 (CKDA) or seed + 3000 (KDA)."""
    rng = np.random.default_rng(seed)
    q = round_bf16(rng.standard_normal((B, T, H, d), dtype=np.float32))
    k = round_bf16(rng.standard_normal((B, T, H, d), dtype=np.float32))
    v = round_bf16(rng.standard_normal((B, T, H, d), dtype=np.float32))
    if arm not in ("ckda", "kda"):
        raise ValueError(arm)
    rng2 = np.random.default_rng(seed + (2000 if arm == "ckda" else 3000))
    a = rng2.normal(2, 1, (B, T, H, d)) * (2.0 if arm == "ckda" else 1.0)
    b = rng2.normal(0, 1, (B, T, H))
    a = _io(a.astype(np.float32), gate_dtype)
    b = _io(b.astype(np.float32), gate_dtype)
    return Case(q, k, v, a, b, None, None, "bf16", 64, True,
                dict(B=B, T=T, H=H, dk=d, dv=d, seed=seed, arm=arm,
                     workload="LM layer forward B=%d H=%d T=%d d=%d bf16 %s range, %s gate logits"
                              % (B, H, T, d, arm.upper(), gate_dtype)),
                gates="logits", gate_dtype=gate_dtype, arm=arm)


def fast_decay(case: Case, seed=1005, frac=0.25, lo=0.15, hi=0.4) -> Case:
    """The case with about `frac` of its key channels (the same channels in
    every head and token) redrawn as gates of magnitude U[lo, hi] and random
    sign; the other arrays are shared, not copied.  Gate values only (not
    logits)."""
    if case.gates != "values":
        raise ValueError("fast_decay redraws gate values, not logits")
    rng = np.random.default_rng(seed)
    dk = case.alpha.shape[-1]
    fast = rng.random(dk) < frac
    a = case.alpha.copy()
    shape = a[..., fast].shape
    a[..., fast] = (rng.uniform(lo, hi, shape) * rng.choice([-1.0, 1.0], shape)).astype(np.float32)
    meta = dict(case.meta, fast_channels=int(fast.sum()),
                workload=case.meta.get("workload", "case") +
                ", %d of %d key channels |alpha|~U[%g,%g]" % (fast.sum(), dk, lo, hi))
    return Case(case.q, case.k, case.v, a, case.beta, case.h0, case.cu_seqlens, case.dtype,
                case.chunk, case.l2norm, meta, gates=case.gates, gate_dtype=case.gate_dtype,
                arm=case.arm)


def zero_gates(case: Case, n=648, seed=1006) -> Case:
    """The case with `n` gate entries (token, head, channel drawn uniformly)
    set to exactly zero: a gate value of 0, or a logit of 0 (which the CKDA
    activation 2 sigmoid(a) - 1 takes to exactly 0).  The other arrays are
    shared, not copied."""
    rng = np.random.default_rng(seed)
    a = case.alpha.copy()
    flat = a.reshape(-1)
    idx = rng.choice(flat.size, size=n, replace=False)
    flat[idx] = 0.0
    meta = dict(case.meta, zero_gates=n,
                workload=case.meta.get("workload", "case") + ", %d gates exactly 0" % n)
    return Case(case.q, case.k, case.v, a, case.beta, case.h0, case.cu_seqlens, case.dtype,
                case.chunk, case.l2norm, meta, gates=case.gates, gate_dtype=case.gate_dtype,
                arm=case.arm)


def varlen_lengths(seed=1003, n=16, total=65536, lo=1024, hi=8192):
    """n lengths ~ U{lo..hi} rescaled to sum to `total` (rounded; the
    remainder goes to the last length); redrawn with seed+1 while any length
    falls outside [lo, hi]."""
    s = seed
    while True:
        rng = np.random.default_rng(s)
        L = rng.integers(lo, hi + 1, n).astype(np.float64)
        L = np.round(L * total / L.sum()).astype(np.int64)
        L[-1] += total - L.sum()
        if L.min() >= lo and L.max() <= hi:
            return L, s
        s += 1


def varlen(seed=1003, n=16, total=65536, H=16, d=128) -> Case:
    lens, used = varlen_lengths(seed, n, total)
    rng = np.random.default_rng(seed)
    T = int(lens.sum())
    q = round_bf16(rng.standard_normal((1, T, H, d), dtype=np.float32))
    k = round_bf16(rng.standard_normal((1, T, H, d), dtype=np.float32))
    v = round_bf16(rng.standard_normal((1, T, H, d), dtype=np.float32))
    a = np.tanh(rng.normal(2, 1, (1, T, H, d)).astype(np.float32)).astype(np.float32)
    b = (2 * _sigmoid(rng.normal(0, 1, (1, T, H)))).astype(np.float32)
    h0 = (0.02 * rng.standard_normal((n, H, d, d))).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return Case(q, k, v, a, b, h0, cu, "bf16", 64, True,
                dict(B=1, T=T, H=H, dk=d, dv=d, seed=seed, lengths=lens.tolist(),
                     length_seed=used,
                     workload="packed varlen prefill %d seqs %d tokens H=%d d=%d bf16"
                              % (n, T, H, d)))


def decode_state(seed=1004, N=256, H=32, d=128) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (0.02 * rng.standard_normal((N, H, d, d), dtype=np.float32)).astype(np.float32)


def decode_token(step, seed=1004, N=256, H=32, d=128, dtype="bf16"):
    """Inputs of decode step `step` (seed + 1 + step): q,k,v [N,H,d] in the io
    dtype, alpha ~ U[-1,1] [N,H,d], beta ~ U[0,2] [N,H]."""
    rng = np.random.default_rng(seed + 1 + step)
    q = _io(rng.standard_normal((N, H, d), dtype=np.float32), dtype)
    k = _io(rng.standard_normal((N, H, d), dtype=np.float32), dtype)
    v = _io(rng.standard_normal((N, H, d), dtype=np.float32), dtype)
    a = rng.uniform(-1, 1, (N, H, d)).astype(np.float32)
    b = rng.uniform(0, 2, (N, H)).astype(np.float32)
    return q, k, v, a, b


def device_lm_like(seed, B, T, H, d, h0_std=0.02, device="cuda:0", grads=False):
    """A dense bf16 case too large to draw on the host in reasonable time,
    drawn on the device with torch's seeded generator in the order q, k, v,
    alpha, beta, h0: q, k, v ~ N(0,1) rounded to bfloat16 (nearest even),
    alpha = tanh(N(2,1)) and beta = 2 sigmoid(N(0,1)) in float32 (the LM
    layer's CKDA-range laws), h0 ~ N(0, h0_std^2).  Returns a dict of device
    tensors q, k, v [B,T,H,d], alpha [B,T,H,d], beta [B,T,H], h0 [B,H,d,d];
    the caller copies to the host the slices it checks.  With grads=True it
    also draws, after those, dout ~ N(0,1) in bfloat16 [B,T,H,d] and
    dht ~ N(0,1) float32 [B,H,d,d] for a backward call."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)

    def n(shape):
        return torch.randn(shape, device=device, generator=g, dtype=torch.float32)

    out = {}
    for name in ("q", "k", "v"):
        out[name] = n((B, T, H, d)).to(torch.bfloat16)
    out["alpha"] = torch.tanh(n((B, T, H, d)).add_(2.0))
    out["beta"] = torch.sigmoid(n((B, T, H))).mul_(2.0)
    out["h0"] = n((B, H, d, d)).mul_(h0_std)
    if grads:
        out["dout"] = n((B, T, H, d)).to(torch.bfloat16)
        out["dht"] = n((B, H, d, d))
    return out


def device_decode(seed, N, H, d, device="cuda:0"):
    """One decode step's inputs and state, drawn on the device with torch's
    seeded generator (order: state, q, k, v, alpha, beta): state ~ N(0, 0.02^2)
    float32 [N,H,d,d], q, k, v ~ N(0,1) rounded to bfloat16 [N,H,d],
    alpha ~ U[-1,1] [N,H,d], beta ~ U[0,2] [N,H]."""
    import torch
    g = torch.Generator(device=device).manual_seed(seed)
    out = {"state": torch.randn((N, H, d, d), device=device, generator=g).mul_(0.02)}
    for name in ("q", "k", "v"):
        out[name] = torch.randn((N, H, d), device=device, generator=g).to(torch.bfloat16)
    out["alpha"] = torch.rand((N, H, d), device=device, generator=g).mul_(2.0).sub_(1.0)
    out["beta"] = torch.rand((N, H), device=device, generator=g).mul_(2.0)
    return out
