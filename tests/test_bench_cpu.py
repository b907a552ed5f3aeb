"""Host logic of bench.py: the one-GPU contract, the algorithmic byte and
flop counts of the LM-layer workload, and the traffic keys of the committed
counter summary.  No GPU is used."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import gated_delta_rule_ckda_amd as ck  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_lm_layer_algorithmic_bytes_and_flops():
    # q, k, v read once (bf16), alpha (fp32, one per key channel) and beta
    # read once, o written once (bf16), ht written once (fp32), no h0
    B, T, H, d = 8, 4096, 16, 128
    tok = B * T * H
    expect = tok * 3 * d * 2 + tok * d * 4 + tok * 4 + tok * d * 2 + B * H * d * d * 4
    assert bench.fwd_bytes(B, T, H, d, d, 2, B, False) == expect == 815792128
    # chunked-form flops: 73.93 GFLOP over the 8192 chunk-heads of the layer
    total = bench.chunk_flops(64, d, d) * (B * T // 64) * H
    assert abs(total / 1e9 - 73.93) < 0.01


def test_pass_bytes_are_the_method_bytes_only():
    """Each pass's algorithmic bytes are the method's inputs it reads once and
    the method's outputs it writes once: the transform pass q, k, alpha,
    beta; the state pass v, o, ht.  The blocks one pass hands to the other
    are workspace, reported apart, and their size is the one the library
    lays out (the workspace is the blocks plus a 256-byte-aligned flag word
    per slot)."""
    B, T, H, d, C = 8, 4096, 16, 128, 64
    pb = bench.pass_bytes(B, T, H, d, d, C, 2, B, False)
    assert pb["prep"] == 538968064      # q, k bf16; alpha fp32 per channel; beta fp32
    assert pb["state"] == 276824064     # v, o bf16; ht fp32
    # the two passes together are the whole forward's algorithmic bytes
    assert pb["prep"] + pb["state"] == bench.fwd_bytes(B, T, H, d, d, 2, B, False)
    # with h0 the state pass also reads it; bf16 logits halve alpha's bytes
    assert bench.pass_bytes(B, T, H, d, d, C, 2, B, True)["state"] == 276824064 + B * H * d * d * 4
    tok = B * T * H
    assert bench.pass_bytes(B, T, H, d, d, C, 2, B, False, gate_bytes=2)["prep"] == \
        tok * (2 * d * 2 + (d + 1) * 2)
    blk = bench.block_bytes(C, d, 2)
    assert blk == 61952  # X' and P' packed: 6,144 bytes each instead of 8,192
    desc = ck.FwdDesc(B, T, H, d, d, B, C, ck.BF16, ck.GATE_CKDA, 1, 1.0, ck.GATES_F32, H, 0)
    maxc = B * (T // C)
    flags = -(-(4 * H * maxc) // 256) * 256
    ws = bench.workspace_bytes(B, T, H, d, C, 2)
    assert ws == H * maxc * blk == 507510784
    assert ck.chunk_fwd_workspace_size(desc, False) == flags + ws


def test_traffic_keys_follow_the_sources(tmp_path, monkeypatch):
    """A pass's counter bytes are used only while the summary's key matches
    the hash of that pass's current sources."""
    f = tmp_path / "traffic.txt"
    f.write_text("# counters\n"
                 "prep.src_sha256_16 = %s\nprep.hbm_bytes_per_launch = 1234\n"
                 "state.src_sha256_16 = 0000000000000000\nstate.hbm_bytes_per_launch = 5678\n"
                 % bench.src_hash(bench.PASS_SOURCES["prep"]))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.load_traffic("prep") == 1234.0
    assert bench.load_traffic("state") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.txt"))
    assert bench.load_traffic("prep") is None


@pytest.mark.parametrize("arg", ["--steps", "--warmup"])
def test_bench_flags_parse(arg):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), arg, "x"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "invalid int value" in r.stderr
