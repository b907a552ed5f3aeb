"""P8: the chunked factorisation used by the HIP forward, in fp64, equals the
sequential oracle to rounding (~1e-12): the chunk-ratio form on regular
chunks, the block-anchored form on chunks whose gates decay fast, the
direct-product form on chunks with exact zero or vanishing gates,
partial last chunks and every chunk size."""
import numpy as np
import pytest

import oracle
from tests import chunked_fp64


def _case(seed, B, T, H, dk, dv, zero_frac=0.0, tiny=False, dist="tanh"):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(B, T, H, dk))
    k = rng.normal(size=(B, T, H, dk))
    v = rng.normal(size=(B, T, H, dv))
    if dist == "tanh":
        a = np.tanh(rng.normal(2, 1, size=(B, T, H, dk)))
    else:
        a = rng.uniform(-1, 1, size=(B, T, H, dk))
    a[rng.random(a.shape) < zero_frac] = 0.0
    if tiny:
        a[rng.random(a.shape) < 0.05] = 1e-35
    b = rng.uniform(0, 2, size=(B, T, H))
    h0 = rng.normal(size=(B, H, dk, dv))
    return q, k, v, a, b, h0


def _err(x, r):
    return np.abs(x - r).max() / max(np.abs(r).max(), 1e-300)


@pytest.mark.parametrize("C,T", [(16, 38), (32, 70), (64, 130), (64, 1), (16, 21), (32, 33)])
@pytest.mark.parametrize("l2", [True, False])
def test_ratio_form_equals_sequential(C, T, l2):
    q, k, v, a, b, h0 = _case(100 + C + T, 2, T, 2, 8, 5)
    if not l2:  # the method's range assumes unit keys when the in-op norm is off
        k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    paths = []
    ro, rh = oracle.fwd(q, k, v, a, b, h0=h0, use_l2norm=l2, scale=0.8)
    co, ch = chunked_fp64.fwd(q, k, v, a, b, h0=h0, use_l2norm=l2, scale=0.8, C=C, paths=paths)
    assert "ratio" in paths            # the ratio form is actually exercised
    assert _err(co, ro) < 1e-11
    assert _err(ch, rh) < 1e-11


def test_sign_changes_stay_on_ratio_form():
    """Negative gates alone keep a chunk regular (signs are exact in the
    running product); uniform gates over a short chunk stay regular too."""
    q, k, v, a, b, h0 = _case(5, 2, 64, 2, 8, 4, dist="uniform")
    paths = []
    ro, rh = oracle.fwd(q, k, v, a, b, h0=h0)
    co, ch = chunked_fp64.fwd(q, k, v, a, b, h0=h0, C=16, paths=paths)
    assert set(paths) == {"ratio"} and (a < 0).any()
    assert _err(co, ro) < 1e-11 and _err(ch, rh) < 1e-11


@pytest.mark.parametrize("C", [32, 64])
def test_fast_decay_takes_the_block_form(C):
    """Gates of 0.15..0.4 on a quarter of the channels underflow the chunk-wide
    product (0.27^64 ~ 2^-120) but not a 16-token block's: such chunks take the
    block-anchored form, which matches the oracle like the other two."""
    q, k, v, a, b, h0 = _case(11 + C, 2, 2 * C + 9, 2, 8, 4)
    rng = np.random.default_rng(C)
    a[..., :2] = rng.uniform(0.15, 0.4, size=a[..., :2].shape) * rng.choice([-1, 1], a[..., :2].shape)
    a[..., 2] = 0.02                      # 0.02^16 ~ 2^-90, still in range per block
    ro, rh = oracle.fwd(q, k, v, a, b, h0=h0)
    paths = []
    co, ch = chunked_fp64.fwd(q, k, v, a, b, h0=h0, C=C, paths=paths)
    assert "block" in paths and "direct" not in paths
    assert _err(co, ro) < 1e-11 and _err(ch, rh) < 1e-11


def test_irregular_chunks_take_the_direct_path():
    """Exact zeros and 1e-35 gates make chunks irregular; forcing every chunk
    through the direct-product form gives the same answer as the mix."""
    q, k, v, a, b, h0 = _case(7, 2, 96, 2, 8, 4, zero_frac=0.02, tiny=True)
    ro, rh = oracle.fwd(q, k, v, a, b, h0=h0)
    for force in (False, True):
        paths = []
        co, ch = chunked_fp64.fwd(q, k, v, a, b, h0=h0, C=32, force_irregular=force, paths=paths)
        assert "direct" in paths and (not force or set(paths) == {"direct"})
        assert _err(co, ro) < 1e-11 and _err(ch, rh) < 1e-11


def test_packed_varlen():
    rng = np.random.default_rng(9)
    lens = [5, 0, 64, 33]
    starts = np.concatenate([[0], np.cumsum(lens)])
    T, H, dk, dv = starts[-1], 2, 8, 4
    q = rng.normal(size=(T, H, dk)); k = rng.normal(size=(T, H, dk))
    v = rng.normal(size=(T, H, dv)); a = np.tanh(rng.normal(2, 1, size=(T, H, dk)))
    b = rng.uniform(0, 2, size=(T, H)); h0 = rng.normal(size=(len(lens), H, dk, dv))
    ro, rh = oracle.fwd(q, k, v, a, b, h0=h0, seq_start=starts)
    co, ch = chunked_fp64.fwd(q, k, v, a, b, h0=h0, seq_start=starts, C=16)
    assert _err(co, ro) < 1e-11 and _err(ch, rh) < 1e-11
