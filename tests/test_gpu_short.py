"""Dense batches shorter than or just around one chunk: T = 1, 2, C - 1, C
and C + 1 (one partial chunk, one exact chunk, a chunk and one token), for
the bf16 matrix-core path at chunk 64, d = 128 (packed X' and P' blocks) and
the fp32 path at chunk 16, d = 16: the forward against the oracle, and the
backward's six gradients against the oracle's."""
import pytest

from gated_delta_rule_ckda_amd import inputs
from tests.gpu_util import announce
from tests.test_gpu_bwd import _check as check_bwd
from tests.test_gpu_bwd import _grad_case
from tests.test_gpu_chunk import _check as check_fwd

pytestmark = pytest.mark.gpu

SHAPES = [("bf16", 64, 128), ("f32", 16, 16)]


@pytest.mark.parametrize("dtype,chunk,d", SHAPES)
@pytest.mark.parametrize("tpos", ["1", "2", "C-1", "C", "C+1"])
def test_short_sequences_forward(dtype, chunk, d, tpos):
    T = {"1": 1, "2": 2, "C-1": chunk - 1, "C": chunk, "C+1": chunk + 1}[tpos]
    announce("short forward %s C=%d d=%d T=%d" % (dtype, chunk, d, T))
    c = inputs.random_case(6000 + T + d, 3, T, 2, d, d, dtype=dtype, chunk=chunk, alpha="tanh",
                           beta="2sig", h0_std=0.1)
    check_fwd(c)


@pytest.mark.parametrize("dtype,chunk,d", SHAPES)
@pytest.mark.parametrize("tpos", ["1", "C-1", "C+1"])
def test_short_sequences_backward(dtype, chunk, d, tpos):
    T = {"1": 1, "C-1": chunk - 1, "C+1": chunk + 1}[tpos]
    announce("short backward %s C=%d d=%d T=%d" % (dtype, chunk, d, T))
    check_bwd(_grad_case(6100 + T + d, 2, T, 2, d, dtype), dtype, chunk)
