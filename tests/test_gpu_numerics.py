"""GPU numerics beyond the tolerance bound: what the matrix cores' rounding,
fp16 / bf16 subnormal inputs and non-finite inputs do, through the C ABI.

* The matrix-core error bound (one fp32 chain per output tile) rests on how
  one v_mfma_f32_16x16x32_{f16,bf16} adds its 32 products to the accumulator
  (the measured model in test_mfma_product_grouping).  The filter gradient is
  the one pass whose output stays fp32, so it shows the instruction's
  rounding directly.
* Subnormal fp16 inputs next to normal ones must not cost more than the bound
  (the paired-tap column stream and the matrix cores both take fp16 pairs).
* Non-finite inputs: the definition sends an Inf or NaN input to exactly the
  outputs whose taps read it.  The vector families do the same.  The matrix
  cores multiply every input column of a tile's K windows by the banded
  filter, zeros included, so an output may also turn NaN when one of its
  16-column block's windows holds a non-finite value in a row its filter
  rows read (rows past the filter in a packed group have zero inputs).
"""
import re

import numpy as np
import pytest
import torch

import depthwise_convolution_amd as dw
import oracle
from oracle import check
import synth

from gpu_helpers import run, to_dev, say, DEV

pytestmark = pytest.mark.gpu


def supported(shape, fmt, variant):
    try:
        h = dw.dwconv_create_variant(*shape, fmt, variant)
    except dw.DwconvError as e:
        if e.status == 2:
            return False
        raise
    dw.dwconv_destroy(h)
    return True


def describe(shape, fmt, variant):
    h = dw.dwconv_create_variant(*shape, fmt, variant)
    try:
        return dw.dwconv_plan_describe(h)
    finally:
        dw.dwconv_destroy(h)


# ------------------------------------------------ matrix-core rounding

def _bwf_exact(x, dy, shape, fmt):
    N, H, W, C, FH, FW, S, D, P = shape
    h = dw.dwconv_create(N, H, W, C, FH, FW, S, D, P, fmt)
    try:
        desc = dw.dwconv_bwd_filter_describe(h)
        ws = torch.empty(dw.dwconv_bwd_filter_workspace(h) // 4 + 1, dtype=torch.float32,
                         device=DEV)
        out = torch.full((FH * FW * C,), float("nan"), dtype=torch.float32, device=DEV)
        dw.dwconv_bwd_filter(h, to_dev(x, fmt), to_dev(dy, fmt), out, ws)
        torch.cuda.synchronize()
        return out.cpu().numpy(), desc
    finally:
        dw.dwconv_destroy(h)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_mfma_product_grouping(fmt):
    """dW[0,0,c] = sum_j x[j]*dy[j] over one output row of 32 columns: the 32
    products of one v_mfma_f32_16x16x32 instruction, K index = column.

    Measured model of the instruction (the error analysis of the matrix-core
    kernels rests on it): the 32 products form four groups of 8 consecutive
    k; inside a group every product is cut toward zero to a multiple of
    2^(e - 24), e the exponent of the group's largest product; the group sums
    and the accumulator are then added exactly and rounded once, to nearest
    even.  So one instruction errs by less than 7 * 2^-24 * sum|p| plus one
    rounding of its result.

    (a) 1 + 31 * 2^-25 (1 at column 0): the group of columns 0..7 loses its
        seven 2^-25 products, the other three groups are exact: 1 + 24 * 2^-25.
        (One rounding of the exact sum would give 1 + 2^-20, products added
        one at a time 1.)
    (b) 1 - 7 * 2^-25 (1 at column 0, -2^-25 at 1..7): cut toward zero, 1.
        (Rounding the exact sum gives 1 - 2^-23.)
    (c) 2^24 + 31 * 1: nothing falls below the groups' granularity, so the
        exact sum 2^24 + 31 is rounded once, the tie going to the even
        neighbour: 2^24 + 32 (one at a time: 2^24)."""
    shape = (1, 1, 32, 8, 1, 1, 1, 1, 0)
    cases = [  # x[0], dy[0], x[j], dy[j] (j = 1..nsmall), nsmall, expected
        (1.0, 1.0, 2.0 ** -12, 2.0 ** -13, 31, 1.0 + 24 * 2.0 ** -25),
        (1.0, 1.0, -2.0 ** -12, 2.0 ** -13, 7, 1.0),
        (2.0 ** 12, 2.0 ** 12, 1.0, 1.0, 31, 2.0 ** 24 + 32),
    ]
    for big_x, big_g, small_x, small_g, nsmall, expect in cases:
        x = np.zeros((1, 1, 32, 8))
        g = np.zeros((1, 1, 32, 8))
        x[0, 0, 1:1 + nsmall, :], g[0, 0, 1:1 + nsmall, :] = small_x, small_g
        x[0, 0, 0, :], g[0, 0, 0, :] = big_x, big_g
        xs, gs = synth.to_storage(x, fmt), synth.to_storage(g, fmt)
        # the stored values are the exact powers of two asked for
        assert np.array_equal(oracle.decode(xs, fmt), x)
        assert np.array_equal(oracle.decode(gs, fmt), g)
        got, desc = _bwf_exact(xs, gs, shape, fmt)
        say(f"[gpu] mfma grouping {fmt}: {desc[:40]} -> {got[0]!r}, expect {expect!r}")
        assert "mfma" in desc
        assert np.all(got == np.float32(expect)), (fmt, got, expect)


# ------------------------------------------------ subnormal inputs

def _subnormal_mix(shape, fmt, seed):
    """x: in every row, even columns hold normal values of magnitude about
    2^7 and odd columns subnormals (fp16: below 2^-14; bf16: below 2^-126),
    so every pair (x[j], x[j+1]) that a paired-tap or matrix-core product
    forms mixes the two; half the rows swap the roles.  w ~ N(0, 1/(FH*FW))."""
    N, H, W, C, FH, FW = shape[:6]
    rng = np.random.default_rng(seed)
    tiny = 2.0 ** -14 if fmt == "f16" else 2.0 ** -126
    normal = rng.choice([-1.0, 1.0], (N, H, W, C)) * rng.uniform(64, 256, (N, H, W, C))
    sub = rng.choice([-1.0, 1.0], (N, H, W, C)) * rng.uniform(0.05, 0.95, (N, H, W, C)) * tiny
    col = np.arange(W)[None, None, :, None]
    row = np.arange(H)[None, :, None, None]
    x = np.where((col + row // 2) % 2 == 0, normal, sub)
    w = rng.standard_normal((FH, FW, C)) / (FH * FW) ** 0.5
    xs, ws = synth.to_storage(x, fmt), synth.to_storage(w, fmt)
    dec = oracle.decode(xs, fmt)
    nz = dec[(col + row // 2 + 0 * dec) % 2 == 1]
    assert np.all(np.abs(nz) < tiny) and np.count_nonzero(nz) > nz.size // 2, \
        "the odd positions hold subnormals"
    return xs, ws


SUB_CASES = [
    # the paired-tap column stream (forced row-window family), the planner's
    # pick, and the matrix cores, on 5x5 and 7x7
    ((2, 20, 44, 32, 5, 5, 1, 1, 2), "rowwin"),
    ((2, 20, 44, 32, 5, 5, 1, 1, 2), "auto"),
    ((2, 20, 44, 32, 5, 5, 1, 1, 2), "mfma"),
    ((2, 20, 44, 32, 7, 7, 1, 1, 3), "mfma"),
    ((1, 20, 40, 16, 31, 31, 1, 1, 15), "mfma"),
    ((64, 28, 28, 96, 5, 5, 1, 1, 2), "auto"),
]


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_subnormal_inputs_forward(fmt):
    for i, (shape, fam) in enumerate(SUB_CASES):
        if not supported(shape, fmt, fam):
            continue
        xs, ws = _subnormal_mix(shape, fmt, 900 + i)
        b = np.random.default_rng(i).uniform(-0.1, 0.1, shape[3]).astype(np.float32)
        say(f"[gpu] subnormal fwd {fmt} {shape} {fam}: {describe(shape, fmt, fam)[:60]}")
        y, used = run(xs, ws, b, shape, fmt, fam, guard=256)
        ye, scale = oracle.fwd(xs, ws, b, shape[6], shape[7], shape[8], fmt, threads=8)
        rep = check.assert_float(y, fmt, ye, scale, f"subnormal {fmt} {shape} {fam}")
        say(f"      ok ({used}) {rep}")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_subnormal_inputs_sparse_filter(fmt):
    """Filters with only two adjacent taps set, (fh, fw) and (fh, fw + 1), so
    one pair of products makes up every output and the bound is stated
    against those two terms alone: a paired-tap instruction that mishandled
    the normal product next to a subnormal one would exceed it."""
    N, H, W, C = 2, 12, 40, 32
    for F, fam in [(5, "rowwin"), (5, "mfma"), (7, "mfma")]:
        for fw0 in range(F - 1):
            shape = (N, H, W, C, F, F, 1, 1, F // 2)
            if not supported(shape, fmt, fam):
                continue
            xs, _ = _subnormal_mix(shape, fmt, 990 + fw0)
            rng = np.random.default_rng(fw0)
            w = np.zeros((F, F, C))
            w[F // 2, fw0, :] = rng.uniform(0.5, 2.0, C) * rng.choice([-1, 1], C)
            w[F // 2, fw0 + 1, :] = rng.uniform(0.5, 2.0, C) * rng.choice([-1, 1], C)
            ws = synth.to_storage(w, fmt)
            say(f"[gpu] subnormal sparse {fmt} F={F} taps {fw0},{fw0 + 1} {fam}: "
                f"{describe(shape, fmt, fam)[:50]}")
            y, used = run(xs, ws, None, shape, fmt, fam, guard=64)
            ye, scale = oracle.fwd(xs, ws, None, 1, 1, F // 2, fmt, threads=4)
            check.assert_float(y, fmt, ye, scale, f"subnormal sparse {fmt} {F} {fw0} {fam}")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_subnormal_inputs_backward_data(fmt):
    """The gradient plays the input's part: subnormals next to normal values
    in dy, through the stride-1 backward-data pass (the forward kernels with
    the filter read rotated)."""
    for i, (shape, fam) in enumerate(SUB_CASES[:4]):
        N, H, W, C, FH, FW, S, D, P = shape
        OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
        gs, ws = _subnormal_mix((N, OH, OW, C, FH, FW), fmt, 950 + i)
        if not supported(shape, fmt, fam):
            continue
        h = dw.dwconv_create_variant(*shape, fmt, fam)
        try:
            desc = dw.dwconv_bwd_data_describe(h)
            dx = torch.empty((N, H, W, C), dtype={"f16": torch.float16,
                                                   "bf16": torch.bfloat16}[fmt], device=DEV)
            say(f"[gpu] subnormal bwd {fmt} {shape} {fam}: {desc[:60]}")
            dw.dwconv_bwd_data(h, to_dev(gs, fmt), to_dev(ws, fmt), dx)
            torch.cuda.synchronize()
        finally:
            dw.dwconv_destroy(h)
        host = (dx.view(torch.int16).cpu().numpy().view(np.uint16) if fmt == "bf16"
                else dx.cpu().numpy())
        ref, scale = oracle.bwd_data(gs, ws, shape, fmt, threads=8)
        rep = check.assert_float(host, fmt, ref, scale, f"subnormal bwd {fmt} {shape} {fam}")
        say(f"      ok {rep}")


# ------------------------------------------------ non-finite inputs

NONFINITE = [
    ((1, 24, 40, 16, 3, 3, 1, 1, 1), "f32"),
    ((1, 24, 40, 32, 5, 5, 1, 1, 2), "f16"),
    ((1, 24, 40, 32, 5, 5, 1, 1, 2), "bf16"),
    ((1, 24, 44, 16, 7, 7, 1, 1, 3), "f16"),
    ((1, 24, 44, 16, 7, 7, 1, 1, 3), "bf16"),
    ((1, 40, 40, 8, 31, 31, 1, 1, 15), "bf16"),
    ((1, 30, 30, 61, 5, 5, 2, 2, 4), "f32"),
]
FAMILIES = ["direct", "rowwin", "ldstile", "mfma"]


def _mfma_reach(shape, bad, P, desc):
    """Outputs the matrix-core family may turn NaN for the non-finite inputs
    `bad` (list of (ih, iw)): the rows whose filter rows read ih, and the
    16-column output blocks whose K windows hold iw.  One filter row per
    MFMA: windows of 32 columns at 16-column steps, 16 * (fragments + 1)
    columns from the block's first input column; PK rows per MFMA: J
    windows of 32 / PK columns (the plan description names both)."""
    N, H, W, C, FH, FW, S, D, _ = shape
    OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
    m = re.search(r"(\d+) windows of (\d+) cols", desc)
    span = int(m.group(1)) * int(m.group(2)) if m else 16 * ((FW + 15) // 16) + 16
    mask = np.zeros((OH, OW), bool)
    for ih, iw in bad:
        rows = [oh for oh in range(OH) if 0 <= ih - (oh - P) < FH]
        for oh in rows:
            for ow in range(OW):
                b0 = 16 * (ow // 16) - P
                if b0 <= iw < b0 + span:
                    mask[oh, ow] = True
    return mask


@pytest.mark.parametrize("case", range(len(NONFINITE)))
def test_nonfinite_inputs(case):
    """Inf, -Inf and NaN inputs: the outputs the oracle makes non-finite are
    non-finite of the same kind on every family; every other output matches
    the oracle within the bound, except (matrix cores only) those inside the
    reach described in the module docstring, which may be NaN instead."""
    shape, fmt = NONFINITE[case]
    N, H, W, C, FH, FW, S, D, P = shape
    rng = np.random.default_rng(1000 + case)
    x = rng.standard_normal((N, H, W, C))
    w = rng.standard_normal((FH, FW, C)) / (FH * FW) ** 0.5
    bad = [(H // 2, W // 3, 1, np.inf), (H // 3, W - 2, 3, -np.inf), (2, W // 2, 5, np.nan)]
    xs, ws = synth.to_storage(x, fmt), synth.to_storage(w, fmt)
    for ih, iw, c, v in bad:
        if fmt == "bf16":  # bit patterns: +Inf, -Inf, a quiet NaN
            xs[0, ih, iw, c] = {np.inf: 0x7f80, -np.inf: 0xff80}.get(v, 0x7fc0)
        else:
            xs[0, ih, iw, c] = v
    b = rng.uniform(-0.1, 0.1, C).astype(np.float32)
    ye, scale = oracle.fwd(xs, ws, b, S, D, P, fmt, threads=4)
    fin = np.isfinite(ye)
    assert not fin.all()
    for fam in FAMILIES:
        if not supported(shape, fmt, fam):
            continue
        say(f"[gpu] non-finite {fmt} {shape} {fam}: {describe(shape, fmt, fam)[:60]}")
        y, used = run(xs, ws, b, shape, fmt, fam, guard=64)
        yv = oracle.decode(y, fmt)
        # outputs whose taps read a non-finite input are non-finite; on the
        # vector families of the same kind as the oracle's (the matrix cores
        # may give NaN for an Inf: a second fragment's window can hold the
        # Inf against a zero of its band)
        assert not np.isfinite(yv[~fin]).any(), fam
        if fam != "mfma":
            assert np.array_equal(np.isnan(yv[~fin]), np.isnan(ye[~fin])), fam
            inf = ~fin & ~np.isnan(ye)
            assert np.array_equal(yv[inf], ye[inf]), fam
        keep = fin.copy()
        if fam == "mfma":
            reach = np.zeros_like(fin)
            desc = describe(shape, fmt, fam)
            for ih, iw, c, _ in bad:
                reach[0, :, :, c] |= _mfma_reach(shape, [(ih, iw)], P, desc)
            # inside the reach an output is NaN or else checked like the rest
            assert not np.isnan(yv[fin & ~reach]).any(), fam
            keep &= ~(reach & np.isnan(yv))
        rep = check.assert_float(np.where(keep, y, 0).astype(y.dtype), fmt,
                                 np.where(keep, ye, 0.0), np.where(keep, scale, 0.0),
                                 f"non-finite {fmt} {shape} {fam}")
        say(f"      ok ({used}) {rep}")
