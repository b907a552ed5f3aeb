"""The C-ABI library loads on a machine without a GPU, exports every symbol
include/ckda.h declares, and rejects bad arguments on the host before any HIP
call (dummy, never-dereferenced pointers are used; no GPU is touched)."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_ckda_amd as ck

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ckda.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ckda_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ck.library_path())
    names = _declared()
    assert "ckda_chunk_fwd" in names and "ckda_recurrent_step" in names
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_matches_header():
    m = re.search(r"#define CKDA_ABI_VERSION (\d+)", open(HEADER).read())
    assert ck.abi_version() == int(m.group(1))


def test_status_strings():
    lib = ck._load()
    for s in range(5):
        assert lib.ckda_status_string(s) != b"unknown status"
    assert lib.ckda_status_string(99) == b"unknown status"


# Fake, 16-byte aligned, never-dereferenced device addresses.
BASE = 0x7F0000000000
P = {n: ctypes.c_void_p(BASE + i * (1 << 32)) for i, n in
     enumerate(["q", "k", "v", "alpha", "beta", "cu", "h0", "o", "ht", "ws"])}
WS_BYTES = 1 << 31


def _desc(**kw):
    d = dict(B=2, T=64, H=2, dk=128, dv=128, num_seqs=2, chunk_size=64, io_dtype=ck.BF16,
             gate_range=ck.GATE_CKDA, use_qk_l2norm=1, scale=1.0, gate_input=ck.GATES_F32,
             qk_heads=0, sign_absorb=0)
    d.update(kw)
    return ck.FwdDesc(**d)


def _fwd(desc, **over):
    p = dict(P)
    p.update(over)
    lib = ck._load()
    st = lib.ckda_chunk_fwd(ctypes.byref(desc) if desc is not None else None, p["q"], p["k"],
                            p["v"], p["alpha"], p["beta"], p.get("cu_seqlens"), p["h0"], p["o"],
                            p["ht"], p["ws"], p.get("ws_bytes", WS_BYTES), None)
    return st, lib.ckda_last_error().decode()


@pytest.mark.parametrize("over,needle", [
    (dict(B=0), "non-positive"), (dict(H=-1), "non-positive"), (dict(dk=0), "non-positive"),
    (dict(io_dtype=7), "io_dtype"), (dict(gate_range=3), "gate_range"),
    (dict(gate_input=3), "gate_input"), (dict(gate_input=-1), "gate_input"),
    (dict(qk_heads=3), "qk_heads"), (dict(qk_heads=-2), "qk_heads"),
    (dict(sign_absorb=2), "sign_absorb"),
    (dict(use_qk_l2norm=2), "use_qk_l2norm"), (dict(chunk_size=48), "chunk_size"),
    (dict(num_seqs=3), "num_seqs"),
])
def test_fwd_rejects_bad_descriptor(over, needle):
    st, msg = _fwd(_desc(**over))
    assert st == 1 and needle in msg


def test_fwd_null_and_alignment_and_aliasing():
    assert _fwd(None)[0] == 1
    st, msg = _fwd(_desc(), q=None)
    assert st == 1 and "NULL" in msg
    st, msg = _fwd(_desc(), k=ctypes.c_void_p(BASE + 8))
    assert st == 1 and "aligned" in msg
    st, msg = _fwd(_desc(), o=P["v"])
    assert st == 1 and "overlaps" in msg, msg
    st, msg = _fwd(_desc(), ht=ctypes.c_void_p(P["h0"].value + 64))
    assert st == 1 and "overlap" in msg


def test_fwd_cu_seqlens_needs_batch_one():
    st, msg = _fwd(_desc(B=2, num_seqs=3), cu_seqlens=ctypes.c_void_p(BASE + 5 * (1 << 32)))
    assert st == 1 and "cu_seqlens" in msg
    st, msg = _fwd(_desc(B=1, num_seqs=3), cu_seqlens=ctypes.c_void_p(BASE + 5 * (1 << 32) + 2))
    assert st == 1 and "aligned" in msg


def test_workspace_size_formula():
    """One block per (head, chunk): (2C^2 + 3C dk) elements + dk floats, rounded up to
    256 bytes (at chunk 64 in bf16 the lower-triangular X' and P' keep 3/4 of
    C^2 each: their first 32 rows half long), plus one int32 flag per (head,
    chunk) slot; dense batches have B*ceil(T/C) chunks, packed ones
    ceil(T/C) + N slots plus the chunk map (an int32 pair per slot, first[N+1],
    the owner per slot, the order[N])."""
    up = lambda x: -(-x // 256) * 256
    d = _desc(B=8, T=4096, H=16, dk=128, dv=128, num_seqs=8)
    blk = (2 * (32 * 32 + 32 * 64) + 3 * 64 * 128) * 2 + 128 * 4
    assert blk % 256 == 0 and blk == 61952
    assert ck.chunk_fwd_workspace_size(d, False) == up(4 * 16 * 8 * 64) + 16 * 8 * 64 * blk
    d = _desc(B=1, T=70, H=3, dk=32, dv=32, num_seqs=4, chunk_size=16, io_dtype=ck.F32)
    blk = up((2 * 16 * 16 + 3 * 16 * 32) * 4 + 32 * 4)
    maxc = -(-70 // 16) + 4
    assert ck.chunk_fwd_workspace_size(d, True) == (up(8 * maxc + 4 * (2 * 4 + 1 + maxc))
                                                   + up(4 * 3 * maxc) + 3 * maxc * blk)
    d = _desc(B=1, T=70000, H=3, dk=32, dv=32, num_seqs=100, chunk_size=16, io_dtype=ck.F32)
    maxc = -(-70000 // 16) + 100
    assert ck.chunk_fwd_workspace_size(d, True) == (up(8 * maxc + 4 * (2 * 100 + 1 + maxc))
                                                   + up(4 * 3 * maxc) + 3 * maxc * blk)
    # sign absorption adds two sign masks and the absorbed q, k, |alpha|, beta
    d0 = _desc(B=8, T=4096, H=16, dk=128, dv=128, num_seqs=8)
    d1 = _desc(B=8, T=4096, H=16, dk=128, dv=128, num_seqs=8, sign_absorb=1)
    tok, maxc = 8 * 4096, 8 * 64
    extra = (up(4 * 16 * maxc * 4) + up(4 * 8 * 16 * 4) + 2 * up(tok * 16 * 128 * 2)
             + up(tok * 16 * 128 * 4) + up(tok * 16 * 4))
    assert ck.chunk_fwd_workspace_size(d1, False) - ck.chunk_fwd_workspace_size(d0, False) == extra
    assert ck.chunk_fwd_workspace_size(_desc(T=0), False) == 0
    assert ck.chunk_fwd_workspace_size(_desc(chunk_size=48), False) == 0


def test_fwd_workspace_validation():
    st, msg = _fwd(_desc(), ws=None)
    assert st == 1 and "workspace is NULL" in msg
    st, msg = _fwd(_desc(), ws_bytes=1024)
    assert st == 3 and "needed" in msg
    st, msg = _fwd(_desc(), ws=ctypes.c_void_p(P["ws"].value + 128))
    assert st == 1 and "256-byte" in msg
    st, msg = _fwd(_desc(), ws=P["v"])
    assert st == 1 and "workspace overlaps v" in msg


def test_prepare_and_finish_validation():
    lib = ck._load()
    d = _desc()
    st = lib.ckda_chunk_fwd_prepare(ctypes.byref(d), P["q"], None, P["alpha"], P["beta"], None,
                                    P["ws"], WS_BYTES, None)
    assert st == 1 and "must not be NULL" in lib.ckda_last_error().decode()
    st = lib.ckda_chunk_fwd_finish(ctypes.byref(d), P["v"], None, P["h0"], None, P["ht"],
                                   P["ws"], WS_BYTES, None)
    assert st == 1 and "must not be NULL" in lib.ckda_last_error().decode()
    st = lib.ckda_chunk_fwd_finish(ctypes.byref(d), P["v"], None, P["h0"], P["o"], P["ht"],
                                   P["ws"], 64, None)
    assert st == 3 and "needed" in lib.ckda_last_error().decode()
    st = lib.ckda_chunk_fwd_prepare(ctypes.byref(d), P["q"], P["k"], P["alpha"], P["beta"], None,
                                    P["q"], WS_BYTES, None)
    assert st == 1 and "workspace overlaps q" in lib.ckda_last_error().decode()


def test_fwd_gate_byte_ranges_follow_gate_input():
    """bf16 logits take 2 bytes per gate, float32 gates 4: an o buffer placed
    right after a bf16 alpha overlaps a float32 alpha of the same shape.  dk=96
    has no kernel, so a call that passes every other check stops at
    CKDA_ERR_UNSUPPORTED and nothing is launched."""
    kw = dict(B=1, num_seqs=1, dk=96, dv=96)
    o = ctypes.c_void_p(P["alpha"].value + 64 * 2 * 96 * 2)
    st, msg = _fwd(_desc(gate_input=ck.GATES_LOGITS_BF16, **kw), o=o)
    assert st == 2, msg
    st, msg = _fwd(_desc(gate_input=ck.GATES_F32, **kw), o=o)
    assert st == 1 and "o overlaps alpha" in msg


def test_fwd_qk_byte_ranges_follow_qk_heads():
    """With grouped value heads q and k span T * Hk * dk elements: o right after
    q overlaps it at Hk = H but not at Hk = H / 2.  dk=96 has no kernel, so a
    call that passes every other check stops at CKDA_ERR_UNSUPPORTED."""
    kw = dict(B=1, num_seqs=1, H=4, dk=96, dv=96)
    o = ctypes.c_void_p(P["q"].value + 64 * 2 * 96 * 2)
    st, msg = _fwd(_desc(qk_heads=2, **kw), o=o)
    assert st == 2, msg
    st, msg = _fwd(_desc(qk_heads=4, **kw), o=o)
    assert st == 1 and "o overlaps q" in msg


def test_fwd_unsupported_shape():
    st, msg = _fwd(_desc(dk=96, dv=96))
    assert st == 2 and "no chunked kernel" in msg


def test_fwd_empty_is_ok_without_launch():
    # num_seqs == 0 with a packed batch: nothing to do, nothing enqueued
    if not ck.fwd_supported(64, 128, 128, ck.BF16):
        pytest.skip("no bf16 d=128 kernel in this build")
    st, _ = _fwd(_desc(B=1, T=0, num_seqs=0), cu_seqlens=ctypes.c_void_p(BASE + 5 * (1 << 32)))
    assert st == 0


def _step(N=4, H=2, dk=128, dv=128, dtype=ck.BF16, gate=ck.GATE_CKDA, l2=1, gi=ck.GATES_F32,
          hk=0, **over):
    p = dict(P)
    p.update(over)
    lib = ck._load()
    st = lib.ckda_recurrent_step(N, H, hk, dk, dv, dtype, gate, gi, l2, 1.0, p["q"], p["k"], p["v"],
                                 p["alpha"], p["beta"], p["h0"], p["ht"], p["o"], None)
    return st, lib.ckda_last_error().decode()


def test_step_validation():
    assert _step(N=-1)[0] == 1
    assert _step(H=0)[0] == 1
    assert _step(dtype=5)[0] == 1
    assert _step(gate=2)[0] == 1
    assert _step(gi=3)[0] == 1 and "gate_input" in _step(gi=3)[1]
    assert _step(N=0, gi=ck.GATES_LOGITS_BF16)[0] == 0
    assert _step(H=4, hk=3)[0] == 1 and "qk_heads" in _step(H=4, hk=3)[1]
    assert _step(N=0, H=4, hk=2)[0] == 0
    assert _step(l2=3)[0] == 1
    assert _step(q=None)[0] == 1
    assert _step(v=ctypes.c_void_p(BASE + 4))[0] == 1
    st, msg = _step(dk=48)
    assert st == 2
    st, msg = _step(o=P["q"])
    assert st == 1 and "overlaps" in msg
    st, msg = _step(ht=ctypes.c_void_p(P["h0"].value + 256))
    assert st == 1 and "partially" in msg
    # N == 0 with valid arguments: ok, nothing enqueued
    assert _step(N=0)[0] == 0
    # one launch covers at most 2^21 (sequence, head) states
    st, msg = _step(N=(1 << 20) + 1, H=2)
    assert st == 2 and "2^21" in msg


def test_l2norm_debug_validation():
    lib = ck._load()
    assert lib.ckda_l2norm_debug(P["q"], P["o"], 10, 0, ck.F32, None) == 1
    assert lib.ckda_l2norm_debug(P["q"], P["o"], 10, 2048, ck.F32, None) == 1
    assert lib.ckda_l2norm_debug(P["q"], P["q"], 10, 16, ck.F32, None) == 1
    assert lib.ckda_l2norm_debug(P["q"], P["o"], 0, 16, ck.F32, None) == 0


# ---------------------------------------------------------------- backward
PB = {n: ctypes.c_void_p(BASE + (20 + i) * (1 << 32)) for i, n in
      enumerate(["dout", "dht", "dq", "dk", "dv", "dalpha", "dbeta", "dh0"])}


def _bwd(desc, **over):
    p = dict(P)
    p.update(PB)
    p.update(over)
    lib = ck._load()
    st = lib.ckda_chunk_bwd(ctypes.byref(desc), p["q"], p["k"], p["v"], p["alpha"], p["beta"],
                            p.get("cu_seqlens"), p["h0"], p["dout"], p["dht"], p["dq"], p["dk"],
                            p["dv"], p["dalpha"], p["dbeta"], p["dh0"], p["ws"],
                            p.get("ws_bytes", WS_BYTES), None)
    return st, lib.ckda_last_error().decode()


@pytest.mark.parametrize("over,status,needle", [
    (dict(sign_absorb=1), 2, "sign-absorption"),
    (dict(qk_heads=3), 1, "qk_heads"),
    (dict(gate_input=7), 1, "gate_input"),
    (dict(chunk_size=48), 1, "chunk_size"),
    (dict(B=0), 1, "non-positive"),
])
def test_bwd_rejects_bad_descriptor(over, status, needle):
    st, msg = _bwd(_desc(**over))
    assert st == status and needle in msg, msg


@pytest.mark.parametrize("over,needle", [
    (dict(dq=None), "must not be NULL"),
    (dict(dbeta=None), "must not be NULL"),
    (dict(dalpha=ctypes.c_void_p(BASE + (23 << 32) + 8)), "not 16-byte aligned"),
    (dict(dv=P["q"]), "dv overlaps q"),
    (dict(dk=PB["dq"]), "dk overlaps dq"),
    (dict(ws=PB["dalpha"]), "overlaps"),
    (dict(ws_bytes=1024), "workspace has 1024 bytes"),
])
def test_bwd_rejects_bad_pointers(over, needle):
    st, msg = _bwd(_desc(), **over)
    # a workspace below the queried size has its own status
    want = 3 if "ws_bytes" in over else 1
    assert st == want and needle in msg, msg


def test_bwd_workspace_covers_forward_and_records():
    """The backward's workspace holds the forward's plus X (fp32 C x C), the
    entry state and the exit-state adjoint (dk x dv each), dU (C x dv) per
    (head, chunk) and one flag each, kept in the io type but X and the
    flags.  bf16 inputs need nothing more (their dP/dG and dq/dk parts run in
    one workgroup and hand over in LDS); fp32 inputs add the intra kernel's
    scratch."""
    lib = ck._load()
    hm = 3 * 2 * 5  # heads x (B * ceil(130 / 32)) chunk slots
    up = lambda x: (x + 255) // 256 * 256
    common = lambda es: up(4 * hm * 32 * 32) + 2 * up(es * hm * 64 * 64) + up(es * hm * 32 * 64) + up(4 * hm)
    for dt, extra in ((ck.BF16, common(2)),
                      (ck.F32, common(4) + up(4 * min(hm, 512) * 14 * 32 * 64))):
        d = _desc(B=2, T=130, H=3, dk=64, dv=64, chunk_size=32, io_dtype=dt)
        fwd = lib.ckda_chunk_fwd_workspace_size(ctypes.byref(d), 0)
        bwd = lib.ckda_chunk_bwd_workspace_size(ctypes.byref(d), 0)
        assert bwd == fwd + extra, dt


def test_noalloc_scratch_limit_is_checked_on_the_host():
    """ckda_chunk_fwd_noalloc refuses a call whose workspace would not fit its
    static scratch with CKDA_ERR_WORKSPACE_TOO_SMALL, and a NULL descriptor
    with CKDA_ERR_INVALID_ARGUMENT, before any HIP call (no GPU here); the
    scratch size the binding states is the header's."""
    lib = ck._load()
    m = re.search(r"#define CKDA_NOALLOC_SCRATCH_BYTES \((\d+)u \* 1024u \* 1024u\)",
                  open(HEADER).read())
    assert int(m.group(1)) << 20 == ck.NOALLOC_SCRATCH_BYTES
    big = _desc(B=4, T=8192, H=16, num_seqs=4)
    assert ck.chunk_fwd_workspace_size(big, False) > ck.NOALLOC_SCRATCH_BYTES
    st = lib.ckda_chunk_fwd_noalloc(ctypes.byref(big), P["q"], P["k"], P["v"], P["alpha"],
                                    P["beta"], None, P["h0"], P["o"], P["ht"], None)
    assert st == 3 and "static scratch" in lib.ckda_last_error().decode()
    assert lib.ckda_chunk_fwd_noalloc(None, P["q"], P["k"], P["v"], P["alpha"], P["beta"], None,
                                      P["h0"], P["o"], P["ht"], None) == 1
    # a call that fits but has a bad argument is refused by the shared checks
    small = _desc()
    assert ck.chunk_fwd_workspace_size(small, False) <= ck.NOALLOC_SCRATCH_BYTES
    st = lib.ckda_chunk_fwd_noalloc(ctypes.byref(small), P["q"], None, P["v"], P["alpha"],
                                    P["beta"], None, P["h0"], P["o"], P["ht"], None)
    assert st == 1 and "must not be NULL" in lib.ckda_last_error().decode()


def test_bwd_workspace_for_logits_and_grouped_heads():
    """Logit gates add float32 alpha and beta; grouped value heads add q and k
    on every value head (io type) and their float32 gradients; each part
    256-byte aligned after the plain backward's workspace."""
    lib = ck._load()
    up = lambda x: (x + 255) // 256 * 256
    B, T, H, d = 2, 130, 4, 64
    tok = B * T
    base = _desc(B=B, T=T, H=H, dk=d, dv=d, chunk_size=32, io_dtype=ck.BF16)
    core = lib.ckda_chunk_bwd_workspace_size(ctypes.byref(base), 0)
    lg = _desc(B=B, T=T, H=H, dk=d, dv=d, chunk_size=32, io_dtype=ck.BF16,
               gate_input=ck.GATES_LOGITS_BF16)
    assert lib.ckda_chunk_bwd_workspace_size(ctypes.byref(lg), 0) == \
        up(core) + up(4 * tok * H * d) + up(4 * tok * H)
    gv = _desc(B=B, T=T, H=H, dk=d, dv=d, chunk_size=32, io_dtype=ck.BF16, qk_heads=2)
    assert lib.ckda_chunk_bwd_workspace_size(ctypes.byref(gv), 0) == \
        up(core) + 2 * up(2 * tok * H * d) + 2 * up(4 * tok * H * d)
    # a workspace for the plain call is too small for the logits call
    st, msg = _bwd(lg, ws_bytes=core)
    assert st == 3 and "needed" in msg


def _fwd_save(desc, **over):
    p = dict(P)
    p.update(over)
    lib = ck._load()
    st = lib.ckda_chunk_fwd_save(ctypes.byref(desc) if desc is not None else None, p["q"], p["k"],
                                 p["v"], p["alpha"], p["beta"], p.get("cu_seqlens"), p["h0"],
                                 p["o"], p["ht"], p["ws"], p.get("ws_bytes", WS_BYTES), None)
    return st, lib.ckda_last_error().decode()


@pytest.mark.parametrize("desc_over,over,status,needle", [
    (dict(sign_absorb=1), {}, 2, "sign-absorption"),
    (dict(B=0), {}, 1, "non-positive"),
    ({}, dict(ws=None), 1, "saved is NULL"),
    ({}, dict(ws=ctypes.c_void_p(P["ws"].value + 16)), 1, "256-byte aligned"),
    ({}, dict(ws_bytes=4096), 3, "saved has 4096 bytes"),
    ({}, dict(ws=P["o"]), 1, "saved overlaps o"),
    ({}, dict(ws=P["alpha"]), 1, "saved overlaps alpha"),
    ({}, dict(o=P["q"]), 1, "overlaps"),
])
def test_fwd_save_validation(desc_over, over, status, needle):
    """The forward that keeps the backward's records takes the forward's
    checks plus the backward workspace's size, alignment and overlaps for
    `saved`, on the host before any HIP call."""
    st, msg = _fwd_save(_desc(**desc_over), **over)
    assert st == status and needle in msg, msg


def test_bwd_saved_takes_the_backward_checks():
    lib = ck._load()
    d = _desc()
    p = dict(P)
    p.update(PB)
    args = [p["q"], p["k"], p["v"], p["alpha"], p["beta"], None, p["h0"], p["dout"], p["dht"],
            p["dq"], p["dk"], p["dv"], p["dalpha"], p["dbeta"], p["dh0"], p["ws"]]
    assert lib.ckda_chunk_bwd_saved(ctypes.byref(d), *args, 1024, None) == 3
    assert "workspace has 1024 bytes" in lib.ckda_last_error().decode()
    assert lib.ckda_chunk_bwd_saved(ctypes.byref(_desc(sign_absorb=1)), *args, WS_BYTES, None) == 2
    bad = list(args)
    bad[9] = None  # dq
    assert lib.ckda_chunk_bwd_saved(ctypes.byref(d), *bad, WS_BYTES, None) == 1
