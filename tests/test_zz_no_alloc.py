"""The no-allocation filter gradient (dwconv_bwd_filter_noalloc) against the
workspace entry point it shares its kernels with, through the C ABI: the same
plan, the same inputs, bit-identical dW, and both within the bound of the
oracle.  Two calls in a row, the second on a smaller input, so the second
finds the first one's values in the library's scratch array."""
import numpy as np
import pytest
import torch

import depthwise_convolution_amd as dw
import oracle
from oracle import check
import synth

from gpu_helpers import to_dev, say, DEV

pytestmark = pytest.mark.gpu


def _inputs(shape, fmt, seed):
    N, H, W, C, FH, FW, S, D, P = shape
    OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
    rng = np.random.default_rng(seed)
    return (synth.to_storage(rng.standard_normal((N, H, W, C)), fmt),
            synth.to_storage(rng.standard_normal((N, OH, OW, C)), fmt))


def _both(shape, fmt, seed):
    """dW from the workspace entry point and from the no-allocation one."""
    N, H, W, C, FH, FW, S, D, P = shape
    x, dy = _inputs(shape, fmt, seed)
    xd, dyd = to_dev(x, fmt), to_dev(dy, fmt)
    h = dw.dwconv_create(*shape, fmt)
    try:
        desc = dw.dwconv_bwd_filter_describe(h)
        nbytes = dw.dwconv_bwd_filter_workspace(h)
        assert nbytes <= dw.DWCONV_SCRATCH_BYTES
        ws = torch.full((nbytes // 4 + 1,), float("nan"), dtype=torch.float32, device=DEV)
        ref = torch.full((FH * FW * C,), float("nan"), dtype=torch.float32, device=DEV)
        got = torch.full((FH * FW * C,), float("nan"), dtype=torch.float32, device=DEV)
        say(f"[gpu] bwd filter noalloc {fmt} {shape}: {desc[:60]}")
        dw.dwconv_bwd_filter(h, xd, dyd, ref, ws)
        dw.dwconv_bwd_filter_noalloc(h, xd, dyd, got)
        torch.cuda.synchronize()
    finally:
        dw.dwconv_destroy(h)
    return x, dy, ref.cpu().numpy(), got.cpu().numpy()


@pytest.mark.parametrize("fmt,big,small", [
    ("bf16", (32, 56, 56, 128, 31, 31, 1, 1, 15), (2, 20, 24, 16, 5, 5, 1, 1, 2)),
    ("f16", (64, 56, 56, 96, 7, 7, 1, 1, 3), (1, 9, 13, 8, 3, 3, 1, 1, 1)),
    ("f32", (64, 56, 56, 128, 3, 3, 1, 1, 1), (3, 11, 17, 4, 5, 3, 2, 1, 2)),
])
def test_noalloc_matches_workspace_entry(fmt, big, small):
    for i, shape in enumerate((big, small)):
        x, dy, ref, got = _both(shape, fmt, 300 + i)
        assert np.array_equal(ref.view(np.uint32), got.view(np.uint32)), (fmt, shape)
        FH, FW, C = shape[4], shape[5], shape[3]
        exact, scale = oracle.bwd_filter(x, dy, shape, fmt, threads=16)
        check.assert_float(got.reshape(FH, FW, C), "f32", exact, scale,
                           f"noalloc {fmt} {shape}")
