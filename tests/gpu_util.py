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
