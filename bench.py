#!/usr/bin/env python3
"""Benchmark of the chunked (Complex) Kimi Delta Attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one ckda_chunk_fwd call over the LM-layer workload (B=8, T=4096,
H=16, dk=dv=128, bf16 q/k/v, fp32 alpha/beta/state, chunk 64, in-kernel q/k
L2 norm, CKDA gate range), inputs resident in HBM: the transform pass over
all chunks, then the state pass.  Prints one JSON line with the headline
throughput (tokens/s), the roofline position of each pass's kernel timed on
its own (HBM-bound: algorithmic bytes / kernel time against 8 TB/s; the
dominant one is the headline roofline), the
oracle's CPU throughput on a bounded sample, and extra lines of context: the
KDA-range arm (throughput ratio), the same layer with bf16 gate logits
activated in-kernel, the same layer through the sign-absorption comparison
path, the packed varlen prefill and the decode step.  Inputs are synthetic (seeded), shaped like the method's workloads.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
CSRC = os.path.join(ROOT, "gated_delta_rule_ckda_amd", "csrc")
# sources each pass's kernel is built from (the traffic summary is keyed on them)
PASS_SOURCES = {
    "prep": ["chunk_prep.hip", "mfma_ops.h", "ckda_internal.h"],
    "state": ["chunk_state.hip", "mfma_ops.h", "ckda_internal.h"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "chunk_fwd_lm_layer_traffic.txt")


def chunk_flops(C, dk, dv):
    """Algorithmic flops of one chunk-head of the chunked form (triangles at
    half): A and P Gram blocks, the UT/WY transform and the inter-chunk
    products."""
    return (C * (C - 1) * dk + 2 * C * (C + 1) * dk + 2 * C * (C + 1) * dv + C ** 3 / 3
            + 6 * C * dk * dv)


def fwd_bytes(B, T, H, dk, dv, io_bytes, nseq, h0, gate_bytes=4):
    """Algorithmic HBM bytes of the whole forward: every input read once,
    every output written once."""
    tok = B * T
    b = tok * H * (2 * dk + dv) * io_bytes      # q, k, v
    b += tok * H * (dk + 1) * gate_bytes        # alpha, beta (or their logits)
    b += tok * H * dv * io_bytes                # o
    b += nseq * H * dk * dv * 4                 # ht
    if h0:
        b += nseq * H * dk * dv * 4
    return b


def block_bytes(C, dk, es):
    """Bytes of one (chunk, head) block of the workspace (layout of the
    transform pass's output, 256-byte aligned): X', -W, Qt', P', Kh'^T in the
    handoff type and g in float32; at chunk 64 in bf16 the first 32 rows of
    the lower-triangular X' and P' are stored half long (3/4 of C x C each)."""
    tri = (C // 2) * (C // 2) + (C // 2) * C if (C == 64 and es == 2) else C * C
    return -(-((2 * tri + 3 * C * dk) * es + 4 * dk) // 256) * 256


def pass_bytes(B, T, H, dk, dv, C, io_bytes, nseq, h0, gate_bytes=4):
    """Algorithmic bytes per launch of each pass: the method's inputs it
    reads, once each, and the method's outputs it writes, once each; the
    workspace blocks the transform pass hands to the state pass are the
    implementation's own traffic and are not counted (they are reported apart,
    see workspace_bytes).  The transform pass reads q, k, alpha, beta; the
    state pass reads v (and h0) and writes o and ht."""
    tok = B * T
    prep = tok * H * (2 * dk * io_bytes + (dk + 1) * gate_bytes)
    state = tok * H * dv * io_bytes * 2 + nseq * H * dk * dv * 4 * (2 if h0 else 1)
    return {"prep": prep, "state": state}


def workspace_bytes(B, T, H, dk, C, io_bytes):
    """Bytes of the blocks the transform pass writes and the state pass reads
    back (one per chunk-head): traffic beyond the algorithmic bytes."""
    return B * (-(-T // C)) * H * block_bytes(C, dk, io_bytes)


def src_hash(names):
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(CSRC, n), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(kernel):
    """HBM bytes per launch of `kernel` measured with rocprofv3 counters on
    the current sources, or None if they were taken on other sources."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get(kernel + ".src_sha256_16") != src_hash(PASS_SOURCES[kernel]):
        return None
    try:
        return float(kv[kernel + ".hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def to_dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda:0")
    return t.to(torch.bfloat16) if dtype == "bf16" else t


# Untimed back-to-back launches of the timed function before its warm-up
# steps.  After the GPU has idled (input generation, a host sleep, or the
# host gap between two workloads), the same forward runs up to 19% slower for
# its first 50 to 60 launches (about 25 ms) and then holds a steady time;
# other GPU work before it shortens that ramp but does not remove it.  The
# settle runs the function itself until this much wall time has passed, so
# that every timed loop measures the sustained rate.
SETTLE_MS = 150.0


def settle(fn, ms=SETTLE_MS):
    """Run `fn` back to back, untimed, for about `ms` of wall time (batches of
    up to 32 launches, one synchronisation per batch); returns the launches."""
    import torch
    if ms <= 0:
        return 0
    n, batch = 0, 1
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1000.0 < ms:
        for _ in range(batch):
            fn()
        torch.cuda.synchronize()
        n += batch
        batch = min(2 * batch, 32)
    return n


def time_launches(fn, steps, warmup, settle_ms=SETTLE_MS):
    """Average time of `fn` (one kernel launch on the current stream) over
    `steps` launches, with HIP events recorded on that stream, after the
    settle and `warmup` untimed launches."""
    import torch
    settle(fn, settle_ms)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall * 1000.0 / steps


def time_each(fn, steps, warmup, between=None, settle_ms=SETTLE_MS):
    """Per-launch times of `fn` (ms), each bracketed by its own pair of HIP
    events on the current stream; `between` (untimed) runs before each one."""
    import torch
    settle(fn, settle_ms)
    for _ in range(warmup):
        fn()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1 in ev:
        if between is not None:
            between()
        e0.record(stream)
        fn()
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in ev]


def ceilings():
    """Ceilings of this GPU measured in the same run: a plain device copy
    (1 GiB read, 1 GiB written), in-place read-modify-writes of a 512 MiB and
    a 2 GiB fp32 buffer (the decode step's access pattern, through torch's
    element-wise kernel) and a dense bf16 GEMM of 8192^3 through torch (the
    matrix cores as the vendor library reaches them)."""
    import torch
    n = 1 << 28
    a = torch.ones(n, device="cuda:0")
    b = torch.empty_like(a)
    ms_copy, _ = time_launches(lambda: b.copy_(a), 20, 3)
    half = a[: n // 2]
    ms_rmw, _ = time_launches(lambda: half.mul_(0.999), 20, 3)
    del a, b, half
    big = torch.ones(n * 2, device="cuda:0")
    ms_rmw2, _ = time_launches(lambda: big.mul_(0.999), 10, 2)
    del big
    m = 8192
    g = torch.Generator(device="cuda:0").manual_seed(9)
    x = torch.randn((m, m), device="cuda:0", generator=g).to(torch.bfloat16)
    y = torch.randn((m, m), device="cuda:0", generator=g).to(torch.bfloat16)
    z = torch.empty((m, m), device="cuda:0", dtype=torch.bfloat16)
    ms_mm, _ = time_launches(lambda: torch.matmul(x, y, out=z), 10, 3)
    del x, y, z
    torch.cuda.empty_cache()
    copy = 2 * n * 4 / (ms_copy / 1000.0) / 1e9
    rmw = 2 * (n // 2) * 4 / (ms_rmw / 1000.0) / 1e9
    rmw2 = 2 * (2 * n) * 4 / (ms_rmw2 / 1000.0) / 1e9
    mm = 2 * m ** 3 / (ms_mm / 1000.0) / 1e12
    return {"copy_GBs": round(copy, 1), "copy_frac": round(copy / HBM_PEAK_GBS, 4),
            "rmw_512MiB_GBs": round(rmw, 1), "rmw_512MiB_frac": round(rmw / HBM_PEAK_GBS, 4),
            "rmw_2GiB_GBs": round(rmw2, 1), "rmw_2GiB_frac": round(rmw2 / HBM_PEAK_GBS, 4),
            "bf16_gemm_8192_TFLOPs": round(mm, 1), "bf16_gemm_frac": round(mm / BF16_PEAK_TFLOPS, 4),
            "what": "torch copy_ of 1 GiB fp32; torch mul_ in place on 512 MiB and on 2 GiB "
                    "fp32 (back to back over 512 MiB, part of the buffer stays in the 256 MiB "
                    "last-level cache; over 2 GiB it cannot); torch.matmul bf16 "
                    "8192x8192x8192 (hipBLASLt)"}


def fwd_plan(case, gate, sign_absorb=False):
    import torch
    import gated_delta_rule_ckda_amd as ck
    dt = case.dtype
    q, k, v = to_dev(case.q, dt), to_dev(case.k, dt), to_dev(case.v, dt)
    a, b = to_dev(case.alpha, case.gate_dtype), to_dev(case.beta, case.gate_dtype)
    h0 = None if case.h0 is None else to_dev(case.h0, "f32")
    cu = None if case.cu_seqlens is None else torch.from_numpy(case.cu_seqlens).to("cuda:0")
    return ck.ChunkFwdPlan(q, k, v, a, b, h0=h0, cu_seqlens=cu, chunk_size=case.chunk,
                           use_qk_l2norm=case.l2norm, gate=gate, gates=case.gates,
                           sign_absorb=sign_absorb)


def time_passes_in_forward(plan, steps, warmup):
    """Each pass's launch times (ms, sorted) inside back-to-back forwards:
    every forward runs as ckda_chunk_fwd_prepare then ckda_chunk_fwd_finish
    (the same launches as one ckda_chunk_fwd call), with a HIP event on the
    launch stream before, between and after them, so each pass runs with
    the caches and clocks it meets in the workload (the transform pass after
    the previous forward's state pass)."""
    import torch

    def fwd():
        plan.prepare()
        plan.finish()

    settle(fwd)
    for _ in range(warmup):
        fwd()
    stream = torch.cuda.current_stream()
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(3)) for _ in range(steps)]
    torch.cuda.synchronize()
    for e0, e1, e2 in ev:
        e0.record(stream)
        plan.prepare()
        e1.record(stream)
        plan.finish()
        e2.record(stream)
    torch.cuda.synchronize()
    return (sorted(e0.elapsed_time(e1) for e0, e1, _ in ev),
            sorted(e1.elapsed_time(e2) for _, e1, e2 in ev))


def bench_fwd(case, steps, warmup, gate, passes=False, sign_absorb=False):
    """Whole forward per step (both passes, one ckda_chunk_fwd call on a
    preallocated workspace); with passes=True also each pass alone, and with
    passes="each" also the median and minimum of single pass launches and the
    sorted times of single forward steps, each after the last-level cache was
    evicted ("cold")."""
    import torch
    import gated_delta_rule_ckda_amd as ck
    plan = fwd_plan(case, gate, sign_absorb)
    q, k, v, a, b, h0, cu = plan.args

    def step():
        ck.chunk_fwd(q, k, v, a, b, h0=h0, cu_seqlens=cu, chunk_size=case.chunk,
                     use_qk_l2norm=case.l2norm, gate=gate, out=plan.o, final_state=plan.ht,
                     workspace=plan.ws, gates=case.gates, sign_absorb=sign_absorb)

    per = {}
    if passes == "each":
        # the contract's loop with no settle, started after the GPU idled
        torch.cuda.synchronize()
        time.sleep(1.0)
        per["from_idle"], _ = time_launches(step, steps, warmup, settle_ms=0)
    ms, wall_ms = time_launches(step, steps, warmup)
    if passes == "each":
        scratch = torch.zeros(1 << 28, device="cuda:0")
        per["cold"] = sorted(time_each(step, steps, 0, between=lambda: scratch.add_(1.0)))
        del scratch
    if passes:
        per["prep"], _ = time_launches(plan.prepare, steps, warmup)
        per["state"], _ = time_launches(plan.finish, steps, warmup)
        if passes == "each":
            for name, fn in (("prep", plan.prepare), ("state", plan.finish)):
                t = sorted(time_each(fn, steps, 0))
                per[name + "_alone_median"] = t[len(t) // 2]
                per[name + "_alone_min"] = t[0]
            per["prep_fwd"], per["state_fwd"] = time_passes_in_forward(plan, steps, warmup)
    del plan, q, k, v, a, b, h0, cu
    torch.cuda.empty_cache()
    return ms, wall_ms, per


def bench_bwd(case, steps, warmup):
    """ckda_chunk_bwd on the case (random dL/do and dL/dht), preallocated
    outputs and workspace; ms per call (the call recomputes the forward)."""
    import torch
    import gated_delta_rule_ckda_amd as ck
    dt = case.dtype
    q, k, v = to_dev(case.q, dt), to_dev(case.k, dt), to_dev(case.v, dt)
    a, b = to_dev(case.alpha, "f32"), to_dev(case.beta, "f32")
    g = torch.Generator(device="cuda:0").manual_seed(5)
    dout = torch.randn(v.shape, device="cuda:0", generator=g).to(v.dtype)
    B, T, H, dk = case.q.shape
    dht = torch.randn((B, H, dk, case.v.shape[-1]), device="cuda:0", generator=g)
    desc = ck._make_desc(q, v, H, dk, case.v.shape[-1], case.chunk, "ckda", case.l2norm, 1.0,
                         None, ck.GATES_F32, False)
    ws = torch.empty(ck.chunk_bwd_workspace_size(desc, False), device="cuda:0", dtype=torch.uint8)

    def step():
        ck.chunk_bwd(q, k, v, a, b, dout, dht=dht, chunk_size=case.chunk,
                     use_qk_l2norm=case.l2norm, workspace=ws)

    ms, _ = time_launches(step, steps, warmup)
    del q, k, v, a, b, dout, dht, ws
    torch.cuda.empty_cache()
    return ms


def bench_train(case, steps, warmup):
    """A training step's forward and backward on the case, two ways: the
    forward (ckda_chunk_fwd) then the backward that recomputes it
    (ckda_chunk_bwd), and the forward that keeps the backward's records
    (ckda_chunk_fwd_save) then the backward that reads them
    (ckda_chunk_bwd_saved); plus the saved backward alone.  ms per step."""
    import torch
    import gated_delta_rule_ckda_amd as ck
    dt = case.dtype
    q, k, v = to_dev(case.q, dt), to_dev(case.k, dt), to_dev(case.v, dt)
    a, b = to_dev(case.alpha, "f32"), to_dev(case.beta, "f32")
    g = torch.Generator(device="cuda:0").manual_seed(5)
    dout = torch.randn(v.shape, device="cuda:0", generator=g).to(v.dtype)
    B, T, H, dk = case.q.shape
    dv = case.v.shape[-1]
    dht = torch.randn((B, H, dk, dv), device="cuda:0", generator=g)
    desc = ck._make_desc(q, v, H, dk, dv, case.chunk, "ckda", case.l2norm, 1.0, None,
                         ck.GATES_F32, False)
    bws = torch.empty(ck.chunk_bwd_workspace_size(desc, False), device="cuda:0", dtype=torch.uint8)
    fws = torch.empty(ck.chunk_fwd_workspace_size(desc, False), device="cuda:0", dtype=torch.uint8)
    o = torch.empty_like(v)
    ht = torch.empty((B, H, dk, dv), device="cuda:0", dtype=torch.float32)
    kw = dict(chunk_size=case.chunk, use_qk_l2norm=case.l2norm)

    def step_recompute():
        ck.chunk_fwd(q, k, v, a, b, out=o, final_state=ht, workspace=fws, **kw)
        ck.chunk_bwd(q, k, v, a, b, dout, dht=dht, workspace=bws, **kw)

    def step_saved():
        ck.chunk_fwd_save(q, k, v, a, b, out=o, final_state=ht, saved=bws, **kw)
        ck.chunk_bwd(q, k, v, a, b, dout, dht=dht, saved=bws, **kw)

    def bwd_saved():
        ck.chunk_bwd(q, k, v, a, b, dout, dht=dht, saved=bws, **kw)

    out = {}
    out["step_recompute"], _ = time_launches(step_recompute, steps, warmup)
    out["step_saved"], _ = time_launches(step_saved, steps, warmup)
    out["bwd_saved"], _ = time_launches(bwd_saved, steps, warmup)  # on the last step's save
    out["saved_bytes"] = bws.numel()
    del q, k, v, a, b, dout, dht, bws, fws, o, ht
    torch.cuda.empty_cache()
    return out


def bwd_bytes(B, T, H, dk, dv, es):
    """Algorithmic bytes of the backward: q, k, v, dout read in the io type,
    alpha, beta read as fp32 (once); dq, dk, dv, dalpha, dbeta written as
    fp32 (once)."""
    tok = B * T * H
    return tok * (es * (2 * dk + 2 * dv) + 4 * dk + 4) + tok * 4 * (3 * dk + dv + 1)


def bench_decode(steps_inner=64, reps=3):
    """The decode workload: 64 consecutive in-place steps (fresh inputs per
    step, resident in HBM), timed as a whole and divided by 64."""
    import torch
    import gated_delta_rule_ckda_amd as ck
    from gated_delta_rule_ckda_amd import inputs
    N, H, d = 256, 32, 128
    st = to_dev(inputs.decode_state(N=N, H=H, d=d), "f32")
    toks = []
    for s in range(steps_inner):
        q, k, v, a, b = inputs.decode_token(s, N=N, H=H, d=d)
        toks.append((to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"), to_dev(a, "f32"),
                     to_dev(b, "f32")))
    o = torch.empty((N, H, d), device="cuda:0", dtype=torch.bfloat16)

    def run():
        for (q, k, v, a, b) in toks:
            ck.recurrent_step(q, k, v, a, b, st, out=o)

    ms, _ = time_launches(run, reps, 1)
    per = ms / steps_inner
    nbytes = N * H * (2 * d * d * 4 + 3 * d * 2 + d * 4 + 4 + d * 2)
    # the same steps with the 256 MiB last-level cache evicted before each
    # one: a read-modify-write of a 1 GiB scratch buffer, untimed
    scratch = torch.zeros(1 << 28, device="cuda:0")
    it = iter(range(1 << 30))

    def one():
        q, k, v, a, b = toks[next(it) % steps_inner]
        ck.recurrent_step(q, k, v, a, b, st, out=o)

    cold = sorted(time_each(one, steps_inner, 0, between=lambda: scratch.add_(1.0)))
    del st, toks, scratch
    torch.cuda.empty_cache()
    return per, nbytes, {"median": cold[len(cold) // 2], "min": cold[0]}


def cpu_baseline(case, pairs, scale=1.0, min_seconds=10.0):
    """Oracle throughput on the host cores on a bounded sample: the first
    `pairs` (batch, head) pairs of the workload over the full sequence length
    (pairs are independent, so this is the same per-token work), run
    repeatedly for about `min_seconds` (at least 3 runs); the median run is
    reported."""
    import oracle
    B, T, H = case.q.shape[:3]
    sel = [(i // H, i % H) for i in range(pairs)]
    q = np.stack([case.q[b, :, h] for b, h in sel], 0)[:, :, None]
    k = np.stack([case.k[b, :, h] for b, h in sel], 0)[:, :, None]
    v = np.stack([case.v[b, :, h] for b, h in sel], 0)[:, :, None]
    a = np.stack([case.alpha[b, :, h] for b, h in sel], 0)[:, :, None]
    be = np.stack([case.beta[b, :, h] for b, h in sel], 0)[:, :, None]
    threads = oracle.max_threads()
    runs = []
    start = time.perf_counter()
    while len(runs) < 3 or time.perf_counter() - start < min_seconds:
        t0 = time.perf_counter()
        oracle.fwd(q, k, v, a, be, use_l2norm=case.l2norm, scale=scale)
        runs.append(time.perf_counter() - t0)
    wall = sorted(runs)[len(runs) // 2]
    head_tokens = pairs * T
    # one core on a smaller sample of the same pairs
    p1 = max(1, pairs // 32)
    oracle.set_num_threads(1)
    runs1 = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.fwd(q[:p1], k[:p1], v[:p1], a[:p1], be[:p1], use_l2norm=case.l2norm, scale=scale)
        runs1.append(time.perf_counter() - t0)
    oracle.set_num_threads(threads)
    wall1 = sorted(runs1)[1]
    try:
        nproc = len(os.sched_getaffinity(0))
    except AttributeError:
        nproc = os.cpu_count()
    return {"value": (head_tokens / H) / wall, "unit": "tokens/s", "cores": threads,
            "one_core": {"value": (p1 * T / H) / wall1, "pairs": p1, "median_of": 3},
            "os_cpu_count": os.cpu_count(), "nproc": nproc,
            "kind": "oracle",
            "sample": "%d of %d (batch, head) pairs x T=%d tokens of the same workload, fp64 "
                      "sequential recurrence on %d OpenMP threads; median of %d runs (%.2f s each, "
                      "%.1f s in total); tokens counted as head-tokens / H"
                      % (pairs, B * H, T, threads, len(runs), wall, sum(runs))}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--only", choices=["all", "lm", "bwd", "decode"], default="all",
                    help="'lm': only the headline workload and its passes; 'bwd': only the "
                         "backward on the headline workload; 'decode': only the decode steps "
                         "(all three for profiling)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--cpu-pairs", type=int, default=128)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_ckda_amd import inputs
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)

    if args.only == "decode":
        per, dbytes, cold = bench_decode()
        print(json.dumps({"workload": "decode steps", "us_per_step": round(per * 1000.0, 2),
                          "achieved_GBs": round(dbytes / (per / 1000.0) / 1e9, 1),
                          "cold_us_median": round(cold["median"] * 1000.0, 2)}), flush=True)
        return

    case = inputs.lm_layer(arm="ckda")
    B, T, H, dk = case.q.shape
    dv = case.v.shape[3]
    C = case.chunk
    if args.only == "bwd":
        ms_bw = bench_bwd(case, args.steps, args.warmup)
        tr = bench_train(case, args.steps, args.warmup)
        print(json.dumps({"workload": "backward of the LM layer", "ms_per_call": round(ms_bw, 3),
                          "bwd_saved_ms": round(tr["bwd_saved"], 3),
                          "step_recompute_ms": round(tr["step_recompute"], 3),
                          "step_saved_ms": round(tr["step_saved"], 3),
                          "steps": args.steps, "warmup": args.warmup}), flush=True)
        return
    ms, wall_ms, per = bench_fwd(case, args.steps, args.warmup, "ckda", passes="each")
    tokens = B * T
    tok_s = tokens / (ms / 1000.0)
    nbytes = fwd_bytes(B, T, H, dk, dv, 2, B, False)
    flops = chunk_flops(C, dk, dv) * (B * T // C) * H
    tflops = flops / (ms / 1000.0) / 1e12
    pbytes = pass_bytes(B, T, H, dk, dv, C, 2, B, False)
    wbytes = workspace_bytes(B, T, H, dk, C, 2)
    names = {"prep": "prep_kernel<bf16, C=64, dk=128> (gate prefix, norms, UT/WY transform)",
             "state": "state_kernel<bf16, C=64, dk=dv=128, dv tile 64> (inter-chunk state + output)"}
    what = {"prep": "q, k (bf16), alpha, beta (fp32) read once",
            "state": "v read once (bf16), o written once (bf16), ht written once (fp32)"}
    timed = {"prep": "ckda_chunk_fwd_prepare (prep_kernel, then prep_redo_kernel, which with "
                     "no chunk flagged only scans the flags) inside back-to-back forwards, one "
                     "event pair per launch; ms_alone: the same call back to back with itself",
             "state": "ckda_chunk_fwd_finish (state_kernel) inside back-to-back forwards, one "
                      "event pair per launch; ms_alone: the same call back to back with itself"}
    passes = {}
    for kname in ("prep", "state"):
        t = per[kname + "_fwd"]
        kms = sum(t) / len(t)
        gbs = pbytes[kname] / (kms / 1000.0) / 1e9
        tr = load_traffic(kname)
        passes[kname] = {"kernel": names[kname], "ms": round(kms, 4),
                         "ms_median": round(t[len(t) // 2], 4),
                         "ms_min": round(t[0], 4),
                         "timed": timed[kname],
                         "ms_alone": round(per[kname], 4),
                         "ms_alone_median": round(per[kname + "_alone_median"], 4),
                         "ms_alone_min": round(per[kname + "_alone_min"], 4),
                         "algorithmic_bytes": pbytes[kname], "algorithmic": what[kname],
                         "achieved": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "workspace_bytes": wbytes,
                         "traffic": tr,
                         "traffic_over_algorithmic": (None if tr is None
                                                      else round(tr / pbytes[kname], 3))}
    dom = max(("prep", "state"), key=lambda n: passes[n]["ms"])
    e2e_gbs = nbytes / (ms / 1000.0) / 1e9
    cold = per["cold"]

    out = {
        "metric": "chunked CKDA fwd tokens/s + TFLOP/s (% MFMA peak), H=16 d=128 T=4096 bf16",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": case.meta["workload"], "B": B, "T": T, "H": H, "dk": dk, "dv": dv,
                   "chunk": C, "gate_range": "ckda", "use_qk_l2norm": True,
                   "alpha": "tanh(N(2,1))", "beta": "2 sigmoid(N(0,1))"},
        "tflops": round(tflops, 2),
        "mfma_frac": round(tflops / BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "hbm", "achieved": passes[dom]["achieved"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": passes[dom]["frac"], "traffic": passes[dom]["traffic"],
                     "kernel": passes[dom]["kernel"], "kernel_ms": passes[dom]["ms"],
                     "algorithmic_bytes": pbytes[dom], "passes": passes,
                     "end_to_end": {"algorithmic_bytes": nbytes, "achieved": round(e2e_gbs, 1),
                                    "frac": round(e2e_gbs / HBM_PEAK_GBS, 4)},
                     "wall_ms_per_step": round(wall_ms, 4)},
        "settle": {"ms": SETTLE_MS,
               "what": "before every timed loop (its warm-up steps included), the timed "
                       "function itself runs back to back untimed for this much wall time: "
                       "after the GPU idles, the forward runs up to 19% slower for its first "
                       "50-60 launches (about 25 ms)"},
    "from_idle": {"what": "the same warm-up and timed steps started after 1 s of GPU idle, "
                          "with no settle",
                  "ms_per_step": round(per["from_idle"], 4),
                  "tokens_per_s": round(tokens / (per["from_idle"] / 1000.0), 1)},
    "cold_cache": {"what": "each forward step alone, after a 1 GiB read-modify-write that "
                               "evicts the 256 MiB last-level cache (untimed)",
                       "steps": len(cold), "ms_median": round(cold[len(cold) // 2], 4),
                       "ms_min": round(cold[0], 4),
                       "tokens_per_s_median": round(tokens / (cold[len(cold) // 2] / 1000.0), 1)},
    }

    if args.only == "all":
        kda = inputs.lm_layer(arm="kda")
        ms_kda, _, _ = bench_fwd(kda, args.steps, args.warmup, "kda")
        del kda
        out["kda_range"] = {"tokens_per_s": round(tokens / (ms_kda / 1000.0), 1),
                            "ms_per_step": round(ms_kda, 4),
                            "ckda_over_kda": round(ms_kda / ms, 4),
                            "pages_context": "CKDA keeps ~96-97% of KDA kernel throughput on H100"}
        lg = inputs.lm_layer_logits(arm="ckda", gate_dtype="bf16")
        ms_lg, _, per_lg = bench_fwd(lg, args.steps, args.warmup, "ckda", passes=True)
        del lg
        lg_prep = pass_bytes(B, T, H, dk, dv, C, 2, B, False, gate_bytes=2)["prep"]
        out["gate_logits"] = {
            "workload": "LM layer as above, gates given as bf16 logits a, b and activated in "
                        "the transform pass (alpha = 2 sigmoid(a) - 1, beta = 2 sigmoid(b))",
            "tokens_per_s": round(tokens / (ms_lg / 1000.0), 1), "ms_per_step": round(ms_lg, 4),
            "prep_ms": round(per_lg["prep"], 4), "state_ms": round(per_lg["state"], 4),
            "prep_algorithmic_bytes": lg_prep,
            "prep_frac": round(lg_prep / (per_lg["prep"] / 1000.0) / 1e9 / HBM_PEAK_GBS, 4)}
        fd = inputs.fast_decay(case)
        ms_fd, _, per_fd = bench_fwd(fd, args.steps, args.warmup, "ckda", passes=True)
        out["fast_decay"] = {
            "workload": fd.meta["workload"] + " (chunk-wide gate products below 2^-100: "
                        "products restarted every 16 rows)",
            "tokens_per_s": round(tokens / (ms_fd / 1000.0), 1), "ms_per_step": round(ms_fd, 4),
            "prep_ms": round(per_fd["prep"], 4), "state_ms": round(per_fd["state"], 4),
            "over_headline": round(ms_fd / ms, 4)}
        del fd
        zg = inputs.zero_gates(case)
        ms_zg, _, per_zg = bench_fwd(zg, args.steps, args.warmup, "ckda", passes=True)
        del zg
        zl = inputs.zero_gates(inputs.lm_layer_logits(arm="ckda", gate_dtype="bf16"))
        ms_zl, _, per_zl = bench_fwd(zl, args.steps, args.warmup, "ckda", passes=True)
        del zl
        out["zero_gates"] = {
            "workload": "LM layer as the headline with 648 gates exactly 0 (token, head, channel "
                        "drawn uniformly); and the bf16-logit arm with 648 logits exactly 0",
            "ms_per_step": round(ms_zg, 4), "prep_ms": round(per_zg["prep"], 4),
            "over_headline": round(ms_zg / ms, 4),
            "logits_ms_per_step": round(ms_zl, 4), "logits_prep_ms": round(per_zl["prep"], 4),
            "logits_over_headline": round(ms_zl / ms, 4)}
        ms_sa, _, _ = bench_fwd(case, args.steps, args.warmup, "ckda", sign_absorb=True)
        out["sign_absorbed"] = {
            "workload": "LM layer as the headline, CKDA range run as a KDA forward on |alpha| "
                        "with the gates' cumulative signs folded into q and k (comparison path)",
            "tokens_per_s": round(tokens / (ms_sa / 1000.0), 1), "ms_per_step": round(ms_sa, 4),
            "native_over_absorbed": round(ms_sa / ms, 4)}
        ms_bw = bench_bwd(case, max(5, args.steps // 3), 2)
        bb = bwd_bytes(B, T, H, dk, dv, 2)
        out["backward"] = {
            "workload": "gradients of the headline forward (dq, dk, dv, dalpha, dbeta from "
                        "random dL/do and dL/dht; the call recomputes the forward)",
            "ms_per_call": round(ms_bw, 3), "tokens_per_s": round(tokens / (ms_bw / 1000.0), 1),
            "over_forward": round(ms_bw / ms, 2), "algorithmic_bytes": bb,
            "hbm_frac": round(bb / (ms_bw / 1000.0) / 1e9 / HBM_PEAK_GBS, 4)}
        tr = bench_train(case, max(5, args.steps // 3), 2)
        out["training_step"] = {
            "workload": "forward + backward of the headline layer per step: with the backward "
                        "recomputing the forward (ckda_chunk_fwd + ckda_chunk_bwd), and with the "
                        "forward keeping the backward's records (ckda_chunk_fwd_save + "
                        "ckda_chunk_bwd_saved)",
            "ms_recompute": round(tr["step_recompute"], 3), "ms_saved": round(tr["step_saved"], 3),
            "saved_over_recompute": round(tr["step_saved"] / tr["step_recompute"], 4),
            "bwd_saved_ms": round(tr["bwd_saved"], 3),
            "bwd_saved_hbm_frac": round(bb / (tr["bwd_saved"] / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
            "saved_bytes": tr["saved_bytes"]}
        vl = inputs.varlen()
        ms_vl, _, _ = bench_fwd(vl, max(5, args.steps // 3), 2, "ckda")
        vl_tok = int(vl.cu_seqlens[-1])
        vl_bytes = fwd_bytes(1, vl_tok, 16, 128, 128, 2, 16, True)
        out["varlen"] = {"workload": vl.meta["workload"], "lengths": vl.meta["lengths"],
                         "tokens_per_s": round(vl_tok / (ms_vl / 1000.0), 1),
                         "ms_per_step": round(ms_vl, 4),
                         "hbm_frac": round(vl_bytes / (ms_vl / 1000.0) / 1e9 / HBM_PEAK_GBS, 4)}
        del vl
        per, dbytes, cold = bench_decode()
        ceil = ceilings()
        out["decode"] = {"workload": "decode step 256 seqs x H=32 x d=128, bf16 q/k/v, fp32 state, "
                                     "64 in-place steps",
                         "us_per_step": round(per * 1000.0, 2),
                         "tokens_per_s": round(256 / (per / 1000.0), 1),
                         "achieved_GBs": round(dbytes / (per / 1000.0) / 1e9, 1),
                         "hbm_frac": round(dbytes / (per / 1000.0) / 1e9 / HBM_PEAK_GBS, 4),
                         "over_rmw_2GiB": round(dbytes / (per / 1000.0) / 1e9
                                                / ceil["rmw_2GiB_GBs"], 4),
                         "cold_cache": {
                             "what": "each step alone after a 1 GiB read-modify-write that "
                                     "evicts the last-level cache",
                             "us_median": round(cold["median"] * 1000.0, 2),
                             "us_min": round(cold["min"] * 1000.0, 2),
                             "hbm_frac_median": round(dbytes / (cold["median"] / 1000.0) / 1e9
                                                      / HBM_PEAK_GBS, 4)}}
        out["ceilings"] = ceil
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(case, args.cpu_pairs)
        out["cpu_baseline"]["gpu_over_cpu"] = round(tok_s / out["cpu_baseline"]["value"], 1)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
