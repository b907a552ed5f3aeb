"""fp64 CPU oracle for the (Complex) Kimi Delta Attention recurrence.

TEST INFRASTRUCTURE ONLY.  The product library never imports, links or runs
anything in this package; only the tests, the package smoke check and the
benchmark's CPU-baseline leg do.  It shares no code with the HIP path: the C
source (``ckda_oracle.c``) includes only libc and OpenMP, and this binding
only marshals numpy arrays.

The recurrence (picx.dev summary of the Complex KDA paper, section
"Background", transition-matrix equation, read with a delta-rule write and a
read-out after the update):

    S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
    o_t = scale * S_t^T q_t

with q and k optionally L2-normalised per (token, head) over dk before the
recurrence (dormouse review "RoPE into the KDA q/k path", section 2).

Every function here has pins in ``tests/test_oracle_pins.py`` (closed forms
from the pages, invariants, brute force); none is left unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "ckda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libckda_oracle.so")
_lock = threading.Lock()
_default = None

EPS = 1e-6


def compile_source(src_path: str, out_path: str) -> str:
    """gcc -O2, plain C11 + OpenMP, no fast-math and no FMA contraction."""
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-ffp-contract=off", "-o", tmp, src_path, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def build(force: bool = True) -> str:
    """Compile the oracle library next to its source."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    return compile_source(SOURCE, _LIB_PATH)


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


class Oracle:
    """ctypes view of one build of ckda_oracle.c (the tests also load
    deliberately mutated builds through this class)."""

    def __init__(self, lib_path: str):
        lib = ctypes.CDLL(lib_path)
        dp = ctypes.POINTER(ctypes.c_double)
        i64p = ctypes.POINTER(ctypes.c_int64)
        lib.ckda_oracle_fwd.restype = ctypes.c_int32
        lib.ckda_oracle_fwd.argtypes = [
            ctypes.c_int32, i64p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            dp, dp, dp, dp, dp, dp, dp, dp, ctypes.c_int32, ctypes.c_double,
            ctypes.c_double]
        lib.ckda_oracle_step.restype = ctypes.c_int32
        lib.ckda_oracle_bwd.argtypes = [
            ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.c_int32, ctypes.c_int32,
            ctypes.c_int32] + [dp] * 14 + [ctypes.c_int32, ctypes.c_double, ctypes.c_double]
        lib.ckda_oracle_bwd.restype = ctypes.c_int32
        lib.ckda_oracle_step.argtypes = [
            ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            dp, dp, dp, dp, dp, dp, dp, ctypes.c_int32, ctypes.c_double,
            ctypes.c_double]
        lib.ckda_oracle_l2norm.restype = ctypes.c_int32
        lib.ckda_oracle_l2norm.argtypes = [ctypes.c_int64, ctypes.c_int32, dp, dp,
                                           ctypes.c_double]
        lib.ckda_oracle_gates.restype = ctypes.c_int32
        lib.ckda_oracle_gates.argtypes = [ctypes.c_int64, dp, ctypes.c_int64, dp,
                                          ctypes.c_int32, dp, dp]
        lib.ckda_oracle_gates_bwd.restype = ctypes.c_int32
        lib.ckda_oracle_gates_bwd.argtypes = [ctypes.c_int64, dp, dp, ctypes.c_int64, dp, dp,
                                              ctypes.c_int32, dp, dp]
        lib.ckda_oracle_set_num_threads.restype = None
        lib.ckda_oracle_set_num_threads.argtypes = [ctypes.c_int32]
        lib.ckda_oracle_max_threads.restype = ctypes.c_int32
        lib.ckda_oracle_max_threads.argtypes = []
        self.lib = lib
        self.path = lib_path

    def set_num_threads(self, n: int) -> None:
        self.lib.ckda_oracle_set_num_threads(int(n))

    def max_threads(self) -> int:
        return int(self.lib.ckda_oracle_max_threads())

    def l2norm(self, x, eps: float = EPS) -> np.ndarray:
        """Row-wise x / sqrt(sum x^2 + eps) over the last axis, in fp64."""
        x = _f64(x)
        d = x.shape[-1]
        y = np.empty_like(x)
        rc = self.lib.ckda_oracle_l2norm(x.size // d, d, _ptr(x), _ptr(y), eps)
        if rc != 0:
            raise ValueError("ckda_oracle_l2norm failed with code %d" % rc)
        return y

    def gates(self, a, b, ckda_range=True):
        """Gates from logits: alpha = 2 sigmoid(a) - 1, beta = 2 sigmoid(b) in
        the CKDA range, sigmoid for both in the KDA range.  fp64, shapes of a
        and b."""
        a, b = _f64(a), _f64(b)
        alpha = np.empty_like(a)
        beta = np.empty_like(b)
        rc = self.lib.ckda_oracle_gates(a.size, _ptr(a), b.size, _ptr(b),
                                        int(bool(ckda_range)), _ptr(alpha), _ptr(beta))
        if rc != 0:
            raise ValueError("ckda_oracle_gates failed with code %d" % rc)
        return alpha, beta

    def gates_bwd(self, a, b, dalpha, dbeta, ckda_range=True):
        """Gradients with respect to the logits a, b given those with respect
        to the gates they activate (chain rule through gates()).  fp64,
        shapes of a and b."""
        a, b, dalpha, dbeta = _f64(a), _f64(b), _f64(dalpha), _f64(dbeta)
        if dalpha.shape != a.shape or dbeta.shape != b.shape:
            raise ValueError("oracle.gates_bwd: gradients must match the logits' shapes")
        da = np.empty_like(a)
        db = np.empty_like(b)
        rc = self.lib.ckda_oracle_gates_bwd(a.size, _ptr(a), _ptr(dalpha), b.size, _ptr(b),
                                            _ptr(dbeta), int(bool(ckda_range)), _ptr(da),
                                            _ptr(db))
        if rc != 0:
            raise ValueError("ckda_oracle_gates_bwd failed with code %d" % rc)
        return da, db

    def fwd(self, q, k, v, alpha, beta, h0=None, seq_start=None, use_l2norm=True,
            scale=1.0, eps=EPS):
        """Sequential fp64 forward.

        Dense form: q,k,alpha [B,T,H,dk], v [B,T,H,dv], beta [B,T,H],
        h0 [B,H,dk,dv].  Packed form (seq_start given): q,k,alpha [T,H,dk]
        (or [1,T,H,dk]), ..., seq_start int [N+1], h0 [N,H,dk,dv].
        Returns (o, ht) in fp64 with o shaped like v.
        """
        q, k, v, alpha, beta = (_f64(a) for a in (q, k, v, alpha, beta))
        out_shape = v.shape
        if seq_start is None:
            B, T, H, dk = q.shape
            starts = np.arange(B + 1, dtype=np.int64) * T
        else:
            starts = np.ascontiguousarray(np.asarray(seq_start, dtype=np.int64))
            H, dk = q.shape[-2], q.shape[-1]
        N = len(starts) - 1
        dv = v.shape[-1]
        ttot = int(starts[-1])
        if q.size != ttot * H * dk or v.size != ttot * H * dv or beta.size != ttot * H:
            raise ValueError("oracle.fwd: shapes do not match seq_start")
        h0a = None if h0 is None else _f64(h0)
        if h0a is not None and h0a.size != N * H * dk * dv:
            raise ValueError("oracle.fwd: h0 has the wrong size")
        o = np.empty(out_shape, dtype=np.float64)
        ht = np.empty((N, H, dk, dv), dtype=np.float64)
        rc = self.lib.ckda_oracle_fwd(
            N, starts.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv,
            _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(h0a), _ptr(o),
            _ptr(ht), int(bool(use_l2norm)), float(scale), float(eps))
        if rc != 0:
            raise ValueError("ckda_oracle_fwd failed with code %d" % rc)
        return o, ht

    def bwd(self, q, k, v, alpha, beta, dout, h0=None, dht=None, seq_start=None,
            use_l2norm=True, scale=1.0, eps=EPS):
        """Gradients of fwd (same layouts) for dL/do = dout and dL/dht = dht
        (None: zero).  Returns (dq, dk, dv, dalpha, dbeta, dh0) in fp64,
        shaped like q, k, v, alpha, beta and [N,H,dk,dv]."""
        q, k, v, alpha, beta, dout = (_f64(a) for a in (q, k, v, alpha, beta, dout))
        if seq_start is None:
            B, T, H, dk = q.shape
            starts = np.arange(B + 1, dtype=np.int64) * T
        else:
            starts = np.ascontiguousarray(np.asarray(seq_start, dtype=np.int64))
            H, dk = q.shape[-2], q.shape[-1]
        N = len(starts) - 1
        dv = v.shape[-1]
        ttot = int(starts[-1])
        if (q.size != ttot * H * dk or v.size != ttot * H * dv or beta.size != ttot * H
                or dout.size != v.size):
            raise ValueError("oracle.bwd: shapes do not match seq_start")
        h0a = None if h0 is None else _f64(h0)
        dhta = None if dht is None else _f64(dht)
        for x in (h0a, dhta):
            if x is not None and x.size != N * H * dk * dv:
                raise ValueError("oracle.bwd: state has the wrong size")
        dq, dkk, dalpha = (np.empty(q.shape, np.float64) for _ in range(3))
        dvv = np.empty(v.shape, np.float64)
        dbeta = np.empty(beta.shape, np.float64)
        dh0 = np.empty((N, H, dk, dv), np.float64)
        rc = self.lib.ckda_oracle_bwd(
            N, starts.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), H, dk, dv,
            _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(h0a), _ptr(dout),
            _ptr(dhta), _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(dalpha), _ptr(dbeta), _ptr(dh0),
            int(bool(use_l2norm)), float(scale), float(eps))
        if rc != 0:
            raise ValueError("ckda_oracle_bwd failed with code %d" % rc)
        return dq, dkk, dvv, dalpha, dbeta, dh0

    def step(self, q, k, v, alpha, beta, state, use_l2norm=True, scale=1.0, eps=EPS):
        """One decode token per sequence: q,k,alpha [N,H,dk], v [N,H,dv],
        beta [N,H], state [N,H,dk,dv].  Returns (o, new_state) in fp64; the
        input array is not modified."""
        q, k, v, alpha, beta = (_f64(a) for a in (q, k, v, alpha, beta))
        N, H, dk = q.shape
        dv = v.shape[-1]
        st = np.array(state, dtype=np.float64, copy=True, order="C")
        o = np.empty((N, H, dv), dtype=np.float64)
        rc = self.lib.ckda_oracle_step(N, H, dk, dv, _ptr(q), _ptr(k), _ptr(v),
                                       _ptr(alpha), _ptr(beta), _ptr(st), _ptr(o),
                                       int(bool(use_l2norm)), float(scale), float(eps))
        if rc != 0:
            raise ValueError("ckda_oracle_step failed with code %d" % rc)
        return o, st


def default() -> Oracle:
    """The oracle built from ckda_oracle.c (compiled on first use)."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(_LIB_PATH):
                build()
            _default = Oracle(_LIB_PATH)
        return _default


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)


def max_threads() -> int:
    return default().max_threads()


def l2norm(x, eps: float = EPS) -> np.ndarray:
    return default().l2norm(x, eps)


def gates(*args, **kwargs):
    return default().gates(*args, **kwargs)


def gates_bwd(*args, **kwargs):
    return default().gates_bwd(*args, **kwargs)


def fwd(*args, **kwargs):
    return default().fwd(*args, **kwargs)


def step(*args, **kwargs):
    return default().step(*args, **kwargs)


def bwd(*args, **kwargs):
    return default().bwd(*args, **kwargs)
