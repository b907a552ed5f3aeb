"""P8: the chunked factorisation used by the HIP forward, in fp64, equals the
sequential oracle to rounding (~1e-12), including exact zero and negative
gates, partial last chunks, every sub-block size and the fallback path for
sub-blocks whose running gate product gets too small to invert."""
import numpy as np
import pytest

import oracle
from tests import chunked_fp64


def _case(seed, B, T, H, dk, dv, zero_frac=0.05, tiny=False):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(B, T, H, dk))
    k = rng.normal(size=(B, T, H, dk))
    v = rng.normal(size=(B, T, H, dv))
    a = rng.uniform(-1, 1, size=(B, T, H, dk))
    a[rng.random(a.shape) < zero_frac] = 0.0
    if tiny:
        a[rng.random(a.shape) < 0.05] = 1e-35
    b = rng.uniform(0, 2, size=(B, T, H))
    h0 = rng.normal(size=(B, H, dk, dv))
    return q, k, v, a, b, h0


def _err(x, r):
    return np.abs(x - r).max() / max(np.abs(r).max(), 1e-300)


@pytest.mark.parametrize("C,blk,T", [(16, 16, 38), (32, 16, 70), (64, 16, 130), (64, 8, 64),
                                     (16, 4, 21), (32, 32, 33), (64, 16, 1)])
@pytest.mark.parametrize("l2", [True, False])
def test_chunked_equals_sequential(C, blk, T, l2):
    q, k, v, a, b, h0 = _case(100 + C + blk + T, 2, T, 2, 8, 5)
    ro, rh = oracle.fwd(q, k, v, a, b, h0=h0, use_l2norm=l2, scale=0.8)
    co, ch = chunked_fp64.fwd(q, k, v, a, b, h0=h0, use_l2norm=l2, scale=0.8, C=C, blk=blk)
    assert _err(co, ro) < 1e-11
    assert _err(ch, rh) < 1e-11


def test_fallback_path_and_tiny_gates():
    """Sub-blocks with |F| < 2^-100 take the direct-product path; forcing it
    everywhere must give the same answer."""
    q, k, v, a, b, h0 = _case(7, 2, 96, 2, 8, 4, tiny=True)
    ro, rh = oracle.fwd(q, k, v, a, b, h0=h0)
    for force in (False, True):
        co, ch = chunked_fp64.fwd(q, k, v, a, b, h0=h0, C=32, blk=16, force_unsafe=force)
        assert _err(co, ro) < 1e-11 and _err(ch, rh) < 1e-11


def test_packed_varlen():
    rng = np.random.default_rng(9)
    lens = [5, 0, 64, 33]
    starts = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv = starts[-1], 2, 8, 4
    q = rng.normal(size=(T, H, dk)); k = rng.normal(size=(T, H, dk))
    v = rng.normal(size=(T, H, dv)); a = rng.uniform(-1, 1, size=(T, H, dk))
    b = rng.uniform(0, 2, size=(T, H)); h0 = rng.normal(size=(len(lens), H, dk, dv))
    ro, rh = oracle.fwd(q, k, v, a, b, h0=h0, seq_start=starts)
    co, ch = chunked_fp64.fwd(q, k, v, a, b, h0=h0, seq_start=starts, C=16, blk=8)
    assert _err(co, ro) < 1e-11 and _err(ch, rh) < 1e-11
