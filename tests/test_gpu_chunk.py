"""GPU parity of the chunked forward (ckda_chunk_fwd through the C ABI)
against the fp64 oracle, the bit-exact normalisation layout through the
chunked path, and the structural invariants of the recurrence."""
import numpy as np
import pytest
import torch

import gated_delta_rule_ckda_amd as ck
import oracle
from gated_delta_rule_ckda_amd import inputs
from tests.gpu_util import (DEV, TOL, announce, cover_pairs, dev, host, max_rel_err, oracle_gates,
                            oracle_pairs, run_chunk)
from tests.test_gpu_decode import pow2_rows

pytestmark = pytest.mark.gpu


def _check(case, chunk=None, scale=1.0, tol=None):
    o, ht = run_chunk(case, chunk=chunk, scale=scale)
    ga, gb = oracle_gates(case, case.alpha, case.beta)
    ro, rh = oracle.fwd(case.q, case.k, case.v, ga, gb, h0=case.h0,
                        seq_start=case.cu_seqlens, use_l2norm=case.l2norm, scale=scale)
    tol = tol or TOL[case.dtype]
    eo, eh = max_rel_err(o, ro), max_rel_err(ht, rh)
    print("  err o=%.3e ht=%.3e (tol %.0e)" % (eo, eh, tol))
    assert eo < tol and eh < tol
    return o, ht


F32_SHAPES = [(16, 16), (32, 16), (64, 16), (16, 32), (32, 32), (64, 32), (16, 64), (32, 64)]


@pytest.mark.parametrize("chunk,d", F32_SHAPES)
@pytest.mark.parametrize("l2", [True, False])
def test_f32_parity(chunk, d, l2):
    announce("f32 parity C=%d d=%d l2=%s" % (chunk, d, l2))
    c = inputs.random_case(300 + chunk + d, 2, 3 * chunk + 5, 3, d, d, dtype="f32", chunk=chunk,
                           l2norm=l2, h0_std=0.5, zero_frac=0.02)
    _check(c, scale=0.8)


@pytest.mark.parametrize("chunk,d", [(64, 128), (32, 128), (16, 128), (64, 64), (32, 64), (16, 64)])
def test_bf16_parity(chunk, d):
    announce("bf16 parity C=%d d=%d" % (chunk, d))
    c = inputs.random_case(400 + chunk + d, 2, 4 * chunk + 7, 2, d, d, dtype="bf16", chunk=chunk,
                           alpha="tanh", beta="2sig", h0_std=0.1, zero_frac=0.01)
    _check(c)


def test_tiny_workload():
    announce("tiny workload B=1 H=2 T=64 d=16 fp32 chunk 16")
    _check(inputs.tiny())


def test_state_tracking_workload_full():
    """B=256 H=4 T=512 d=32 fp32 chunk 32, near-orthogonal transitions; also
    the per-(b,h) relative drift of ||ht||_F against the oracle."""
    announce("state-tracking workload full size")
    c = inputs.state_tracking()
    o, ht = run_chunk(c)
    ro, rh = oracle.fwd(c.q, c.k, c.v, c.alpha, c.beta, use_l2norm=False)
    eo, eh = max_rel_err(o, ro), max_rel_err(ht, rh)
    drift = np.abs(np.linalg.norm(ht, axis=(2, 3)) / np.linalg.norm(rh, axis=(2, 3)) - 1).max()
    print("  err o=%.3e ht=%.3e max ||S|| drift %.3e" % (eo, eh, drift))
    assert eo < TOL["f32"] and eh < TOL["f32"] and drift < TOL["f32"]


def test_orthogonal_norm_preserved():
    """Exactly orthogonal transitions (alpha in {+-1}, beta = 2, unit keys,
    v = 0): ||S_T||_F = ||h0||_F (Theorem 1 of the summary)."""
    announce("orthogonal norm preservation")
    rng = np.random.default_rng(8)
    B, T, H, d = 4, 300, 2, 32
    k = rng.standard_normal((B, T, H, d))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    c = inputs.Case(rng.standard_normal((B, T, H, d)).astype(np.float32), k,
                    np.zeros((B, T, H, d), np.float32),
                    rng.choice([-1.0, 1.0], (B, T, H, d)).astype(np.float32),
                    np.full((B, T, H), 2.0, np.float32),
                    rng.standard_normal((B, H, d, d)).astype(np.float32), None, "f32", 32, False)
    _, ht = run_chunk(c)
    n0 = np.linalg.norm(c.h0.astype(np.float64), axis=(2, 3))
    assert np.abs(np.linalg.norm(ht, axis=(2, 3)) / n0 - 1).max() < 1e-4


@pytest.mark.parametrize("arm", ["ckda", "kda"])
def test_lm_layer_workload_full_sampled(arm):
    """B=8 H=16 T=4096 d=128 bf16 chunk 64 at full size, in the benchmark's
    launch configuration; oracle on 16 sampled (batch, head) pairs that cover
    every batch index and every head index."""
    announce("LM layer workload full size, %s arm" % arm)
    c = inputs.lm_layer(arm=arm)
    o, ht = run_chunk(c, gate=arm)
    o = o.reshape(c.v.shape)
    pairs = cover_pairs(8, 16, extra=[(0, 0), (7, 15)])
    ref = oracle_pairs(c, pairs)
    worst_o = max(max_rel_err(o[n, :, h], ref[(n, h)][0]) for n, h in pairs)
    worst_h = max(max_rel_err(ht[n, h], ref[(n, h)][1]) for n, h in pairs)
    print("  err o=%.3e ht=%.3e" % (worst_o, worst_h))
    assert worst_o < TOL["bf16"] and worst_h < TOL["bf16"]


def test_varlen_workload_full_sampled():
    announce("varlen workload full size")
    c = inputs.varlen()
    o, ht = run_chunk(c)
    lens = np.diff(c.cu_seqlens)
    longest, shortest = int(lens.argmax()), int(lens.argmin())
    pairs = cover_pairs(len(lens), 16, extra=[(longest, 0), (shortest, 15)])
    ref = oracle_pairs(c, pairs)
    o = o[0]
    worst_o = max(max_rel_err(o[c.cu_seqlens[n]:c.cu_seqlens[n + 1], h], ref[(n, h)][0])
                  for n, h in pairs)
    worst_h = max(max_rel_err(ht[n, h], ref[(n, h)][1]) for n, h in pairs)
    print("  err o=%.3e ht=%.3e" % (worst_o, worst_h))
    assert worst_o < TOL["bf16"] and worst_h < TOL["bf16"]


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 64), ("bf16", 64, 32), ("f32", 32, 32),
                                           ("f32", 16, 16)])
def test_chunk_l2norm_layout_bit_exact(dtype, d, chunk):
    """Power-of-two q/k rows through the chunked path: (a) h0 = I, alpha = 1,
    beta = 0 gives o = q_hat exactly for every token and head; (b) one token
    per packed sequence with h0 = 0, alpha = 1, beta = 1, v = 1 gives
    ht[n, h, :, j] = k_hat exactly."""
    announce("chunk l2norm layout %s d=%d C=%d" % (dtype, d, chunk))
    B, T, H = 2, 2 * chunk + 3, 3
    xq, yq = pow2_rows(B * T * H, d, seed=11)
    xk, yk = pow2_rows(B * T * H, d, seed=12)
    q = xq.reshape(B, T, H, d)
    k = xk.reshape(B, T, H, d)
    ones = np.ones((B, T, H, d), np.float32)
    eye = np.broadcast_to(np.eye(d, dtype=np.float32), (B, H, d, d)).copy()
    c = inputs.Case(q, k, np.zeros((B, T, H, d), np.float32), ones,
                    np.zeros((B, T, H), np.float32), eye, None, dtype, chunk, True)
    o, _ = run_chunk(c)
    assert np.array_equal(o.reshape(-1, d).astype(np.float32), yq)
    # (b) packed: every token its own sequence
    N = B * T
    c2 = inputs.Case(q.reshape(1, N, H, d), k.reshape(1, N, H, d), np.ones((1, N, H, d), np.float32),
                     np.ones((1, N, H, d), np.float32), np.ones((1, N, H), np.float32),
                     np.zeros((N, H, d, d), np.float32), np.arange(N + 1, dtype=np.int32),
                     dtype, chunk, True)
    _, ht = run_chunk(c2)
    for j in (0, d - 1):
        assert np.array_equal(ht[:, :, :, j].reshape(-1, d).astype(np.float32), yk)


def test_chunk_size_invariance_and_determinism():
    announce("chunk-size invariance")
    c = inputs.random_case(21, 2, 200, 2, 128, 128, dtype="bf16", alpha="tanh", beta="2sig")
    outs = [run_chunk(c, chunk=C) for C in (16, 32, 64)]
    for o, ht in outs[1:]:
        assert max_rel_err(o, outs[0][0]) < TOL["bf16"]
        assert max_rel_err(ht, outs[0][1]) < TOL["bf16"]
    o2, ht2 = run_chunk(c, chunk=64)
    assert np.array_equal(o2, outs[2][0]) and np.array_equal(ht2, outs[2][1])


def test_split_resume_and_aliasing():
    """fwd(x[:T1]) -> ht, then fwd(x[T1:], h0=ht) equals fwd(x) on x[T1:];
    h0 and ht may be the same buffer."""
    announce("split resume")
    c = inputs.random_case(22, 2, 190, 2, 32, 32, dtype="f32", chunk=32, h0_std=0.3)
    o, ht = run_chunk(c)
    T1 = 77
    sl = lambda x, a, b: np.ascontiguousarray(x[:, a:b])
    c1 = inputs.Case(sl(c.q, 0, T1), sl(c.k, 0, T1), sl(c.v, 0, T1), sl(c.alpha, 0, T1),
                     sl(c.beta, 0, T1), c.h0, None, "f32", 32, True)
    c2 = inputs.Case(sl(c.q, T1, 190), sl(c.k, T1, 190), sl(c.v, T1, 190), sl(c.alpha, T1, 190),
                     sl(c.beta, T1, 190), None, None, "f32", 32, True)
    o1, ht1 = run_chunk(c1)
    # aliasing: pass one device buffer as both h0 and ht
    st = dev(ht1.astype(np.float32))
    o2, _ = ck.chunk_fwd(dev(c2.q), dev(c2.k), dev(c2.v), dev(c2.alpha), dev(c2.beta), h0=st,
                         chunk_size=32, final_state=st)
    torch.cuda.synchronize()
    assert max_rel_err(np.concatenate([o1, host(o2)], 1), o) < TOL["f32"]
    assert max_rel_err(host(st), ht) < TOL["f32"]


def test_varlen_equals_separate_runs_with_empty_sequences():
    announce("varlen vs separate")
    rng = np.random.default_rng(23)
    lens = [70, 0, 1, 128, 33]
    T, H, d = sum(lens), 2, 64
    big = inputs.random_case(24, 1, T, H, d, d, dtype="bf16", chunk=32, alpha="tanh", beta="2sig")
    h0 = (0.1 * rng.standard_normal((len(lens), H, d, d))).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    packed = inputs.Case(big.q, big.k, big.v, big.alpha, big.beta, h0, cu, "bf16", 32, True)
    po, pht = run_chunk(packed)
    for i, n in enumerate(lens):
        s = slice(cu[i], cu[i + 1])
        one = inputs.Case(big.q[:, s], big.k[:, s], big.v[:, s], big.alpha[:, s], big.beta[:, s],
                          h0[i:i + 1], None, "bf16", 32, True)
        if n == 0:
            assert np.array_equal(pht[i].astype(np.float32), h0[i])
            continue
        oo, hh = run_chunk(one)
        assert np.array_equal(po[:, s], oo) and np.array_equal(pht[i], hh[0])


def test_zero_and_tiny_gates_exact_path():
    """Blocks with exact zero gates and gates of 1e-35 take the direct-product
    fix-up path; both dtypes stay within tolerance, and a flipped or zeroed
    gate moves the output by more than the tolerance (vacuity)."""
    announce("zero and tiny gates")
    for dtype, d, chunk in (("f32", 32, 32), ("bf16", 128, 64)):
        c = inputs.random_case(25, 2, 150, 2, d, d, dtype=dtype, chunk=chunk, h0_std=0.2)
        rng = np.random.default_rng(26)
        m = rng.random(c.alpha.shape)
        c.alpha[m < 0.03] = 0.0
        c.alpha[(m >= 0.03) & (m < 0.06)] = 1e-35
        c.alpha[:, 40:56, 0, :] = 0.0     # a whole sub-block of zeros
        o, _ = _check(c)
        flipped = c.alpha.copy()
        flipped[0, 3, 0, :] *= -1
        c2 = inputs.Case(c.q, c.k, c.v, flipped, c.beta, c.h0, None, dtype, chunk, True)
        o2, _ = run_chunk(c2)
        assert max_rel_err(o2, o) > TOL[dtype]


@pytest.mark.parametrize("dtype,chunk,d", [("f32", 32, 32), ("f32", 64, 32), ("f32", 64, 16),
                                           ("bf16", 64, 128), ("bf16", 32, 64)])
def test_fast_decay_block_anchored(dtype, chunk, d):
    """A quarter of the key channels with |alpha| in [0.15, 0.4] (chunk-wide
    products near 2^-120 at chunk 64) and one channel at |alpha| = 0.02
    (0.02^16 ~ 2^-90, the edge of the 16-token range; 2^-180 over 32 tokens):
    these chunks keep the MFMA path with products restarted every 16 rows and
    match the oracle; a zeroed gate in one chunk still takes the direct path
    there alone."""
    announce("fast decay %s C=%d d=%d" % (dtype, chunk, d))
    c = inputs.random_case(40 + chunk + d, 2, 3 * chunk + 11, 2, d, d, dtype=dtype, chunk=chunk,
                           alpha="tanh", beta="2sig", h0_std=0.2)
    c = inputs.fast_decay(c, seed=41 + d)
    c.alpha = c.alpha.copy()
    c.alpha[..., 1] = 0.02 * np.sign(c.alpha[..., 1] + 0.5)
    _check(c)
    c.alpha[1, chunk + 3, 1, 5] = 0.0
    _check(c)


@pytest.mark.parametrize("arm", ["ckda", "kda"])
def test_lm_layer_fast_decay_full_sampled(arm):
    """The LM layer at full size with a quarter of its key channels decaying
    fast (|alpha| ~ U[0.15, 0.4], random sign); oracle on sampled pairs."""
    announce("LM layer full size, fast-decay channels, %s arm" % arm)
    c = inputs.fast_decay(inputs.lm_layer(arm=arm))
    if arm == "kda":
        c.alpha = np.abs(c.alpha)
    o, ht = run_chunk(c, gate=arm)
    o = o.reshape(c.v.shape)
    pairs = cover_pairs(8, 16)
    ref = oracle_pairs(c, pairs)
    worst_o = max(max_rel_err(o[n, :, h], ref[(n, h)][0]) for n, h in pairs)
    worst_h = max(max_rel_err(ht[n, h], ref[(n, h)][1]) for n, h in pairs)
    print("  err o=%.3e ht=%.3e" % (worst_o, worst_h))
    assert worst_o < TOL["bf16"] and worst_h < TOL["bf16"]


def test_decode_chain_equals_prefill():
    announce("decode chain vs prefill")
    c = inputs.random_case(27, 3, 40, 2, 128, 128, dtype="bf16", chunk=64, alpha="tanh",
                           beta="2sig", h0_std=0.1)
    o, ht = run_chunk(c)
    st = dev(c.h0)
    outs = []
    for t in range(40):
        outs.append(host(ck.recurrent_step(dev(c.q[:, t], "bf16"), dev(c.k[:, t], "bf16"),
                                           dev(c.v[:, t], "bf16"), dev(c.alpha[:, t]),
                                           dev(c.beta[:, t]), st)))
    assert max_rel_err(np.stack(outs, 1), o) < TOL["bf16"]
    assert max_rel_err(host(st), ht) < TOL["bf16"]


@pytest.mark.parametrize("dtype,d,chunk,packed", [("bf16", 128, 64, False), ("f32", 32, 32, True)])
def test_prepare_finish_equals_single_call(dtype, d, chunk, packed):
    """The transform and state passes launched separately (prepare once, finish
    twice on the same workspace) give bit-identical o and ht to ckda_chunk_fwd."""
    announce("prepare/finish split %s d=%d C=%d packed=%s" % (dtype, d, chunk, packed))
    if packed:
        lens = [37, 0, 100, 64]
        big = inputs.random_case(77, 1, sum(lens), 2, d, d, dtype=dtype, chunk=chunk)
        h0 = (0.3 * np.random.default_rng(79).standard_normal((len(lens), 2, d, d))).astype(np.float32)
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        c = inputs.Case(big.q, big.k, big.v, big.alpha, big.beta, h0, cu, dtype, chunk, True)
    else:
        c = inputs.random_case(78, 2, 3 * chunk + 11, 2, d, d, dtype=dtype, chunk=chunk,
                               alpha="tanh", beta="2sig", h0_std=0.2)
    o1, h1 = run_chunk(c)
    cu = None if c.cu_seqlens is None else torch.from_numpy(c.cu_seqlens).to(DEV)
    plan = ck.ChunkFwdPlan(dev(c.q, dtype), dev(c.k, dtype), dev(c.v, dtype), dev(c.alpha),
                           dev(c.beta), h0=None if c.h0 is None else dev(c.h0), cu_seqlens=cu,
                           chunk_size=chunk, use_qk_l2norm=c.l2norm)
    plan.prepare()
    o2, h2 = (host(t) for t in plan.finish())
    o3, h3 = (host(t) for t in plan.finish())
    torch.cuda.synchronize()
    assert np.array_equal(o1, o2) and np.array_equal(h1, h2)
    assert np.array_equal(o2, o3) and np.array_equal(h2, h3)


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 64), ("bf16", 64, 32), ("f32", 32, 32),
                                           ("f32", 16, 16)])
def test_single_zero_gates_masked_form(dtype, d, chunk):
    """Exact zero gates, at most one per (16-row block, channel) (the masked
    MFMA form of the second transform kernel), at block edges and in
    adjacent blocks, signed gates, a ragged tail; plus a block with two zeros
    of one channel (direct products)."""
    announce("single zero gates %s d=%d C=%d" % (dtype, d, chunk))
    c = inputs.random_case(311 + d, 2, 3 * chunk + 9, 2, d, d, dtype=dtype, chunk=chunk,
                           alpha="tanh", beta="2sig", h0_std=0.1)
    rng = np.random.default_rng(312)
    c.alpha = c.alpha * rng.choice([-1.0, 1.0], c.alpha.shape).astype(np.float32)
    T = c.alpha.shape[1]
    for (b, t, h, ch) in [(0, 0, 0, 1), (0, 15, 1, 2), (0, chunk - 1, 0, 3), (1, 15, 0, 4),
                          (1, 16, 0, 4), (0, T - 1, 1, 5), (1, chunk + 3, 1, 0),
                          (0, 2 * chunk + 5, 0, d - 1)]:
        c.alpha[b, t, h, ch] = 0.0
    o, ht = run_chunk(c)
    ro, rh = oracle.fwd(c.q, c.k, c.v, c.alpha, c.beta, h0=c.h0)
    eo, eh = max_rel_err(o, ro), max_rel_err(ht, rh)
    print("  err o=%.3e ht=%.3e" % (eo, eh))
    assert eo < TOL[dtype] and eh < TOL[dtype]
    c.alpha[0, 2, 1, 6] = 0.0
    c.alpha[0, 9, 1, 6] = 0.0
    o, ht = run_chunk(c)
    ro, rh = oracle.fwd(c.q, c.k, c.v, c.alpha, c.beta, h0=c.h0)
    assert max_rel_err(o, ro) < TOL[dtype] and max_rel_err(ht, rh) < TOL[dtype]


@pytest.mark.parametrize("logits", [False, True])
def test_lm_layer_zero_gates_full_sampled(logits):
    """The LM layer at full size with 648 gates exactly zero (gate values, or
    bf16 logits of 0, which the CKDA activation takes to 0); oracle on 16
    pairs covering every batch and head."""
    announce("LM layer full size, 648 zero gates, logits=%s" % logits)
    base = inputs.lm_layer_logits(arm="ckda", gate_dtype="bf16") if logits else inputs.lm_layer()
    c = inputs.zero_gates(base)
    o, ht = run_chunk(c, gate="ckda")
    o = o.reshape(c.v.shape)
    pairs = cover_pairs(8, 16)
    ref = oracle_pairs(c, pairs)
    worst_o = max(max_rel_err(o[n, :, h], ref[(n, h)][0]) for n, h in pairs)
    worst_h = max(max_rel_err(ht[n, h], ref[(n, h)][1]) for n, h in pairs)
    print("  err o=%.3e ht=%.3e" % (worst_o, worst_h))
    assert worst_o < TOL["bf16"] and worst_h < TOL["bf16"]
