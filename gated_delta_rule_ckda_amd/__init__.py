"""Python binding of libckda.so: (Complex) Kimi Delta Attention on MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI of ``include/ckda.h``.  Tensors are torch CUDA
(HIP) tensors; calls are asynchronous on the current stream.  If the shared
library is missing the calls raise -- there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading

__all__ = ["chunk_fwd", "chunk_bwd", "chunk_bwd_workspace_size", "recurrent_step",
           "l2norm_debug", "fwd_supported",
           "library_path", "abi_version", "chunk_fwd_save", "CkdaError", "BF16", "F32", "GATE_KDA",
           "GATE_CKDA", "GATES_F32", "GATES_LOGITS_F32", "GATES_LOGITS_BF16", "ChunkFwdPlan"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "libckda.so")
_lock = threading.Lock()
_lib = None

BF16, F32 = 0, 1
GATE_KDA, GATE_CKDA = 0, 1
GATES_F32, GATES_LOGITS_F32, GATES_LOGITS_BF16 = 0, 1, 2
NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024  # CKDA_NOALLOC_SCRATCH_BYTES in include/ckda.h
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small",
           4: "HIP error"}


class CkdaError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__("%s: %s" % (_STATUS.get(status, status), detail))
        self.status = status


class FwdDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("num_seqs", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("io_dtype", ctypes.c_int32),
                ("gate_range", ctypes.c_int32), ("use_qk_l2norm", ctypes.c_int32),
                ("scale", ctypes.c_float), ("gate_input", ctypes.c_int32),
                ("qk_heads", ctypes.c_int32), ("sign_absorb", ctypes.c_int32)]


def library_path() -> str:
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB):
            raise ImportError(
                "libckda.so is not built (%s); run `python -m gated_delta_rule_ckda_amd.build` "
                "or __graft_entry__.build()" % _LIB)
        lib = ctypes.CDLL(_LIB)
        vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
        lib.ckda_chunk_fwd.restype = i32
        lib.ckda_chunk_fwd.argtypes = [ctypes.POINTER(FwdDesc), vp, vp, vp, vp, vp, vp, vp,
                                       vp, vp, vp, ctypes.c_size_t, vp]
        lib.ckda_chunk_fwd_noalloc.restype = i32
        lib.ckda_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(FwdDesc), vp, vp, vp, vp, vp, vp,
                                               vp, vp, vp, vp]
        lib.ckda_chunk_fwd_prepare.restype = i32
        lib.ckda_chunk_fwd_prepare.argtypes = [ctypes.POINTER(FwdDesc), vp, vp, vp, vp, vp, vp,
                                               ctypes.c_size_t, vp]
        lib.ckda_chunk_fwd_finish.restype = i32
        lib.ckda_chunk_fwd_finish.argtypes = [ctypes.POINTER(FwdDesc), vp, vp, vp, vp, vp, vp,
                                              ctypes.c_size_t, vp]
        lib.ckda_chunk_fwd_workspace_size.restype = ctypes.c_size_t
        lib.ckda_chunk_fwd_workspace_size.argtypes = [ctypes.POINTER(FwdDesc), i32]
        lib.ckda_chunk_bwd.restype = i32
        lib.ckda_chunk_bwd.argtypes = [ctypes.POINTER(FwdDesc)] + [vp] * 16 + [ctypes.c_size_t, vp]
        lib.ckda_chunk_fwd_save.restype = i32
        lib.ckda_chunk_fwd_save.argtypes = [ctypes.POINTER(FwdDesc)] + [vp] * 10 + [ctypes.c_size_t, vp]
        lib.ckda_chunk_bwd_saved.restype = i32
        lib.ckda_chunk_bwd_saved.argtypes = [ctypes.POINTER(FwdDesc)] + [vp] * 16 + [ctypes.c_size_t, vp]
        lib.ckda_chunk_bwd_workspace_size.restype = ctypes.c_size_t
        lib.ckda_chunk_bwd_workspace_size.argtypes = [ctypes.POINTER(FwdDesc), i32]
        lib.ckda_fwd_supported.restype = i32
        lib.ckda_fwd_supported.argtypes = [ctypes.POINTER(FwdDesc)]
        lib.ckda_recurrent_step.restype = i32
        lib.ckda_recurrent_step.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32, f32, vp,
                                            vp, vp, vp, vp, vp, vp, vp, vp]
        lib.ckda_l2norm_debug.restype = i32
        lib.ckda_l2norm_debug.argtypes = [vp, vp, ctypes.c_int64, i32, i32, vp]
        lib.ckda_status_string.restype = ctypes.c_char_p
        lib.ckda_status_string.argtypes = [i32]
        lib.ckda_last_error.restype = ctypes.c_char_p
        lib.ckda_last_error.argtypes = []
        lib.ckda_abi_version.restype = i32
        lib.ckda_abi_version.argtypes = []
        _lib = lib
        return lib


def abi_version() -> int:
    return int(_load().ckda_abi_version())


def _check(status):
    if status != 0:
        raise CkdaError(status, _load().ckda_last_error().decode())


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _gate_code(gate):
    if gate in ("ckda", GATE_CKDA):
        return GATE_CKDA
    if gate in ("kda", GATE_KDA):
        return GATE_KDA
    raise ValueError("gate must be 'ckda' or 'kda'")


def _gate_input(gates, alpha, beta):
    """ckda_gate_input_t for gates='values' (float32 gates) or gates='logits'
    (float32 or bfloat16 logits, activated in the kernels)."""
    import torch
    _require(alpha.dtype == beta.dtype, "alpha and beta must share a dtype")
    if gates == "values":
        _require(alpha.dtype == torch.float32, "gate values must be float32")
        return GATES_F32
    if gates == "logits":
        if alpha.dtype == torch.float32:
            return GATES_LOGITS_F32
        if alpha.dtype == torch.bfloat16:
            return GATES_LOGITS_BF16
        raise ValueError("gate logits must be float32 or bfloat16")
    raise ValueError("gates must be 'values' or 'logits'")


def _require(cond, msg):
    if not cond:
        raise ValueError(msg)


def _make_desc(q, v, H, dk, dv, chunk_size, gate, use_qk_l2norm, scale, cu_seqlens,
               gate_input=GATES_F32, sign_absorb=False):
    """H: value heads (v.shape[-2]); the q/k heads are q.shape[-2]."""
    if cu_seqlens is not None:
        B, T = 1, q.shape[-3] if q.dim() == 3 else q.shape[1]
        N = cu_seqlens.numel() - 1
    else:
        B, T = q.shape[0], q.shape[1]
        N = B
    return FwdDesc(B, T, H, dk, dv, N, chunk_size, _dtype_code(q), _gate_code(gate),
                   int(bool(use_qk_l2norm)), float(scale), gate_input, q.shape[-2],
                   int(bool(sign_absorb)))


def fwd_supported(chunk_size, dk, dv, dtype) -> bool:
    d = FwdDesc(1, 1, 1, dk, dv, 1, chunk_size, dtype, GATE_CKDA, 1, 1.0, GATES_F32, 0, 0)
    return bool(_load().ckda_fwd_supported(ctypes.byref(d)))


def chunk_fwd_workspace_size(desc: FwdDesc, packed: bool) -> int:
    """Bytes of workspace ckda_chunk_fwd needs for `desc`."""
    return int(_load().ckda_chunk_fwd_workspace_size(ctypes.byref(desc), int(bool(packed))))


def _fwd_call(q, k, v, alpha, beta, h0, cu_seqlens, chunk_size, use_qk_l2norm, gate, scale,
              output_final_state, out, final_state, gates, sign_absorb):
    """Checks shared by chunk_fwd and chunk_fwd_noalloc; returns (desc, o, ht)."""
    import torch
    H, dk, dv = v.shape[-2], q.shape[-1], v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta)):
        _require(t.is_cuda and t.is_contiguous(), "%s must be a contiguous device tensor" % name)
    _require(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share a dtype")
    gi = _gate_input(gates, alpha, beta)
    if cu_seqlens is not None:
        _require(cu_seqlens.dtype == torch.int32 and cu_seqlens.is_cuda,
                 "cu_seqlens must be an int32 device tensor")
    desc = _make_desc(q, v, H, dk, dv, chunk_size, gate, use_qk_l2norm, scale, cu_seqlens, gi,
                      sign_absorb)
    _require(q.numel() == desc.B * desc.T * desc.qk_heads * dk, "q has the wrong number of elements")
    _require(k.numel() == q.numel(), "k must match q")
    _require(alpha.numel() == desc.B * desc.T * H * dk, "alpha has the wrong number of elements")
    _require(v.numel() == desc.B * desc.T * H * dv, "v has the wrong number of elements")
    _require(beta.numel() == desc.B * desc.T * H, "beta has the wrong number of elements")
    if h0 is not None:
        _require(h0.dtype == torch.float32 and h0.is_contiguous()
                 and h0.numel() == desc.num_seqs * H * dk * dv, "h0 must be [N,H,dk,dv] float32")
    o = torch.empty_like(v) if out is None else out
    ht = None
    if output_final_state:
        ht = (torch.empty((desc.num_seqs, H, dk, dv), device=q.device, dtype=torch.float32)
              if final_state is None else final_state)
    return desc, o, ht


def chunk_fwd(q, k, v, alpha, beta, *, h0=None, cu_seqlens=None, chunk_size=64,
              use_qk_l2norm=True, gate="ckda", scale=1.0, output_final_state=True,
              out=None, final_state=None, workspace=None, stream=None, gates="values",
              sign_absorb=False):
    """Chunked prefill.  Dense: q,k [B,T,Hk,dk], alpha [B,T,H,dk], v [B,T,H,dv],
    beta [B,T,H]; Hk divides H (grouped value heads: value head h reads q/k
    head h // (H // Hk)).  Packed (cu_seqlens int32 [N+1]): leading [1,T,...]
    or [T,...].
    gates='values': alpha, beta are float32 gates; gates='logits': they are
    float32 or bfloat16 logits that the kernels activate.  sign_absorb=True
    runs the comparison strategy that folds the gates' cumulative signs into
    q and k (same result, more traffic).
    `workspace`: optional uint8 device tensor of at least
    chunk_fwd_workspace_size() bytes (allocated per call when omitted).
    Returns (o, ht) with ht [N,H,dk,dv] float32 (None if not requested)."""
    import torch
    lib = _load()
    desc, o, ht = _fwd_call(q, k, v, alpha, beta, h0, cu_seqlens, chunk_size, use_qk_l2norm, gate,
                            scale, output_final_state, out, final_state, gates, sign_absorb)
    need = chunk_fwd_workspace_size(desc, cu_seqlens is not None)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    _require(workspace.is_cuda and workspace.dtype == torch.uint8 and workspace.numel() >= need,
             "workspace must be a uint8 device tensor of at least %d bytes" % need)
    _check(lib.ckda_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                              _ptr(beta), _ptr(cu_seqlens), _ptr(h0), _ptr(o), _ptr(ht),
                              _ptr(workspace), workspace.numel(), _stream(stream)))
    return o, ht


def chunk_fwd_noalloc(q, k, v, alpha, beta, *, h0=None, cu_seqlens=None, chunk_size=64,
                      use_qk_l2norm=True, gate="ckda", scale=1.0, output_final_state=True,
                      out=None, final_state=None, stream=None, gates="values",
                      sign_absorb=False):
    """chunk_fwd through ckda_chunk_fwd_noalloc: no workspace, the library's
    static per-GPU scratch instead (NOALLOC_SCRATCH_BYTES).  The C call
    allocates nothing; pass `out` (and `final_state`) to keep this wrapper
    from allocating them.  Calls on one GPU must not overlap."""
    lib = _load()
    desc, o, ht = _fwd_call(q, k, v, alpha, beta, h0, cu_seqlens, chunk_size, use_qk_l2norm, gate,
                            scale, output_final_state, out, final_state, gates, sign_absorb)
    _check(lib.ckda_chunk_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                      _ptr(beta), _ptr(cu_seqlens), _ptr(h0), _ptr(o), _ptr(ht),
                                      _stream(stream)))
    return o, ht


def chunk_fwd_save(q, k, v, alpha, beta, *, h0=None, cu_seqlens=None, chunk_size=64,
                   use_qk_l2norm=True, gate="ckda", scale=1.0, output_final_state=True,
                   out=None, final_state=None, saved=None, stream=None, gates="values"):
    """chunk_fwd through ckda_chunk_fwd_save: the same (o, ht), plus the
    backward's records kept in `saved` (uint8 device tensor of at least
    chunk_bwd_workspace_size() bytes, allocated when omitted) for
    chunk_bwd(..., saved=saved).  Returns (o, ht, saved)."""
    import torch
    lib = _load()
    desc, o, ht = _fwd_call(q, k, v, alpha, beta, h0, cu_seqlens, chunk_size, use_qk_l2norm, gate,
                            scale, output_final_state, out, final_state, gates, False)
    need = chunk_bwd_workspace_size(desc, cu_seqlens is not None)
    if saved is None:
        saved = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    _require(saved.is_cuda and saved.dtype == torch.uint8 and saved.numel() >= need,
             "saved must be a uint8 device tensor of at least %d bytes" % need)
    _check(lib.ckda_chunk_fwd_save(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                   _ptr(beta), _ptr(cu_seqlens), _ptr(h0), _ptr(o), _ptr(ht),
                                   _ptr(saved), saved.numel(), _stream(stream)))
    return o, ht, saved


def chunk_bwd_workspace_size(desc: FwdDesc, packed: bool) -> int:
    """Bytes of workspace ckda_chunk_bwd needs for `desc`."""
    return int(_load().ckda_chunk_bwd_workspace_size(ctypes.byref(desc), int(bool(packed))))


def chunk_bwd(q, k, v, alpha, beta, dout, *, h0=None, dht=None, cu_seqlens=None, chunk_size=64,
              use_qk_l2norm=True, gate="ckda", scale=1.0, output_dh0=True, workspace=None,
              stream=None, gates="values", saved=None):
    """Gradients of chunk_fwd for dL/do = dout (dtype of v) and dL/dht = dht
    ([N,H,dk,dv] float32, None for zero).  Same layouts as chunk_fwd: q, k on
    Hk heads (grouped value heads when Hk < H), gates='values' (float32
    gates) or 'logits' (float32 or bfloat16 logits; the gradients are then
    those of the logits).  With `saved` (from chunk_fwd_save on the same
    inputs) the records are read from it (ckda_chunk_bwd_saved) instead of
    recomputed, and it serves as the workspace.  Returns float32 (dq, dk, dv,
    dalpha, dbeta, dh0) shaped like q, k, v, alpha, beta and [N,H,dk,dv] (dh0
    None unless output_dh0)."""
    import torch
    lib = _load()
    H, dk, dv = v.shape[-2], q.shape[-1], v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta),
                    ("dout", dout)):
        _require(t.is_cuda and t.is_contiguous(), "%s must be a contiguous device tensor" % name)
    _require(k.dtype == q.dtype and v.dtype == q.dtype and dout.dtype == q.dtype,
             "q, k, v, dout must share a dtype")
    gi = _gate_input(gates, alpha, beta)
    if cu_seqlens is not None:
        _require(cu_seqlens.dtype == torch.int32 and cu_seqlens.is_cuda,
                 "cu_seqlens must be an int32 device tensor")
    desc = _make_desc(q, v, H, dk, dv, chunk_size, gate, use_qk_l2norm, scale, cu_seqlens,
                      gi, False)
    Hk = desc.qk_heads
    _require(H % Hk == 0, "the q/k heads must divide the value heads")
    _require(q.numel() == desc.B * desc.T * Hk * dk, "q has the wrong number of elements")
    _require(k.numel() == q.numel(), "k must match q")
    _require(alpha.numel() == desc.B * desc.T * H * dk, "alpha has the wrong number of elements")
    _require(v.numel() == desc.B * desc.T * H * dv and dout.numel() == v.numel(),
             "v, dout have the wrong number of elements")
    _require(beta.numel() == desc.B * desc.T * H, "beta has the wrong number of elements")
    for name, t in (("h0", h0), ("dht", dht)):
        if t is not None:
            _require(t.dtype == torch.float32 and t.is_contiguous() and t.is_cuda
                     and t.numel() == desc.num_seqs * H * dk * dv,
                     "%s must be [N,H,dk,dv] float32" % name)
    f32 = dict(device=q.device, dtype=torch.float32)
    dq, dkk = (torch.empty(q.shape, **f32) for _ in range(2))
    dal = torch.empty(alpha.shape, **f32)
    dvv = torch.empty(v.shape, **f32)
    dbe = torch.empty(beta.shape, **f32)
    dh0 = torch.empty((desc.num_seqs, H, dk, dv), **f32) if output_dh0 else None
    need = chunk_bwd_workspace_size(desc, cu_seqlens is not None)
    fn = lib.ckda_chunk_bwd
    if saved is not None:
        _require(workspace is None, "pass either workspace or saved")
        workspace, fn = saved, lib.ckda_chunk_bwd_saved
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    _require(workspace.is_cuda and workspace.dtype == torch.uint8 and workspace.numel() >= need,
             "workspace must be a uint8 device tensor of at least %d bytes" % need)
    _check(fn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
              _ptr(cu_seqlens), _ptr(h0), _ptr(dout), _ptr(dht), _ptr(dq), _ptr(dkk), _ptr(dvv),
              _ptr(dal), _ptr(dbe), _ptr(dh0), _ptr(workspace), workspace.numel(),
              _stream(stream)))
    return dq, dkk, dvv, dal, dbe, dh0


class ChunkFwdPlan:
    """The two passes of chunk_fwd as separate launches on one workspace:
    prepare() runs the transform pass over all chunks, finish() the state
    pass (o and the final state).  Used to time the passes one by one."""

    def __init__(self, q, k, v, alpha, beta, *, h0=None, cu_seqlens=None, chunk_size=64,
                 use_qk_l2norm=True, gate="ckda", scale=1.0, out=None, final_state=None,
                 stream=None, gates="values", sign_absorb=False):
        import torch
        self.lib = _load()
        H, dk, dv = v.shape[-2], q.shape[-1], v.shape[-1]
        self.desc = _make_desc(q, v, H, dk, dv, chunk_size, gate, use_qk_l2norm, scale,
                               cu_seqlens, _gate_input(gates, alpha, beta), sign_absorb)
        self.args = (q, k, v, alpha, beta, h0, cu_seqlens)
        self.o = torch.empty_like(v) if out is None else out
        self.ht = (torch.empty((self.desc.num_seqs, H, dk, dv), device=q.device,
                               dtype=torch.float32) if final_state is None else final_state)
        need = chunk_fwd_workspace_size(self.desc, cu_seqlens is not None)
        self.ws = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
        self.stream = stream

    def prepare(self):
        q, k, v, alpha, beta, h0, cu = self.args
        _check(self.lib.ckda_chunk_fwd_prepare(ctypes.byref(self.desc), _ptr(q), _ptr(k),
                                               _ptr(alpha), _ptr(beta), _ptr(cu), _ptr(self.ws),
                                               self.ws.numel(), _stream(self.stream)))

    def finish(self):
        q, k, v, alpha, beta, h0, cu = self.args
        _check(self.lib.ckda_chunk_fwd_finish(ctypes.byref(self.desc), _ptr(v), _ptr(cu),
                                              _ptr(h0), _ptr(self.o), _ptr(self.ht),
                                              _ptr(self.ws), self.ws.numel(),
                                              _stream(self.stream)))
        return self.o, self.ht


def recurrent_step(q, k, v, alpha, beta, state, *, use_qk_l2norm=True, gate="ckda",
                   scale=1.0, out=None, new_state=None, stream=None, gates="values"):
    """One decode token per sequence: q,k [N,Hk,dk], alpha [N,H,dk], v [N,H,dv],
    beta [N,H], state [N,H,dk,dv] float32, updated in place unless new_state
    is given.  `gates` as for chunk_fwd.  Returns o [N,H,dv]."""
    import torch
    lib = _load()
    N, Hk, dk = q.shape
    H, dv = v.shape[-2], v.shape[-1]
    for name, t in (("q", q), ("k", k), ("v", v), ("alpha", alpha), ("beta", beta),
                    ("state", state)):
        _require(t.is_cuda and t.is_contiguous(), "%s must be a contiguous device tensor" % name)
    _require(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v must share a dtype")
    gi = _gate_input(gates, alpha, beta)
    _require(state.dtype == torch.float32, "state must be float32")
    _require(k.shape == q.shape and alpha.shape == (N, H, dk) and v.shape == (N, H, dv)
             and beta.shape == (N, H) and state.shape == (N, H, dk, dv), "shape mismatch")
    o = torch.empty_like(v) if out is None else out
    dst = state if new_state is None else new_state
    _check(lib.ckda_recurrent_step(N, H, Hk, dk, dv, _dtype_code(q), _gate_code(gate), gi,
                                   int(bool(use_qk_l2norm)), float(scale), _ptr(q), _ptr(k),
                                   _ptr(v), _ptr(alpha), _ptr(beta), _ptr(state), _ptr(dst),
                                   _ptr(o), _stream(stream)))
    return o


def l2norm_debug(x, stream=None):
    """Test export of the in-kernel normalisation over the last axis."""
    import torch
    lib = _load()
    _require(x.is_cuda and x.is_contiguous(), "x must be a contiguous device tensor")
    d = x.shape[-1]
    y = torch.empty(x.shape, device=x.device, dtype=torch.float32)
    _check(lib.ckda_l2norm_debug(_ptr(x), _ptr(y), x.numel() // d, d, _dtype_code(x),
                                 _stream(stream)))
    return y
