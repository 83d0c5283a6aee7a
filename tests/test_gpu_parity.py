"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Floating point must satisfy the elementwise bound |y - y_exact| <=
1e-5 * sum|x*w| + 1e-6 on the value before the one final rounding to the
output format (oracle/check.py); int8 -> int32 must match bit for bit.
"""
import numpy as np
import pytest
import torch

import depthwise_convolution_amd as dw
import oracle
from oracle import check
import synth
from synth import WORKLOADS, make_inputs

from gpu_helpers import run, assert_matches_oracle, shape_of, say, DEV

pytestmark = pytest.mark.gpu

FAMILIES = ["auto", "direct", "rowwin", "ldstile", "mfma"]


def supported(shape, fmt, variant):
    try:
        h = dw.dwconv_create_variant(*shape, fmt, variant)
    except dw.DwconvError as e:
        if e.status == 2:
            return False
        raise
    dw.dwconv_destroy(h)
    return True


# ------------------------------------------------------- the five workloads

@pytest.mark.parametrize("name", ["tiny_f32_3x3", "mobilenet_f32_3x3", "convnext_f16_7x7",
                                  "strided_i8_5x5"])
def test_workload_full(name):
    wl = WORKLOADS[name]
    x, w, b = make_inputs(wl)
    shape = shape_of(wl)
    for fam in FAMILIES:
        if fam != "auto" and not supported(shape, wl.dtype, fam):
            continue
        say(f"[gpu] workload {name} family {fam} shape {shape}")
        y, used = run(x, w, b, shape, wl.dtype, fam, guard=4096)
        rep = assert_matches_oracle(y, x, w, b, shape, wl.dtype, f"{name}/{fam}({used})")
        say(f"      ok ({used}) {rep}")


def test_workload_largekernel_full():
    """32x56x56x128 bf16, 31x31: every one of the 12.85 M outputs of every
    family against one oracle pass (the oracle splits the batch over 16
    threads; each output is independent, so the result is the same)."""
    wl = WORKLOADS["largekernel_bf16_31x31"]
    x, w, b = make_inputs(wl)
    shape = shape_of(wl)
    say("[gpu] largekernel: oracle pass")
    ye, scale = oracle.fwd(x, w, b, wl.stride, wl.dilation, wl.pad, "bf16", threads=16)
    for fam in FAMILIES:
        if fam != "auto" and not supported(shape, "bf16", fam):
            continue
        say(f"[gpu] largekernel family {fam}")
        y, used = run(x, w, b, shape, "bf16", fam, guard=4096)
        rep = check.assert_float(y, "bf16", ye, scale, f"largekernel/{used}")
        say(f"      ok ({used}) {rep}")


# ------------------------------------------------------- random small shapes

@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16", "i8"])
def test_random_small(fmt):
    rng = np.random.default_rng({"f32": 1, "f16": 2, "bf16": 3, "i8": 4}[fmt])
    for i in range(40):
        wl = synth.random_small(rng, fmt)
        x, w, b = make_inputs(wl)
        shape = shape_of(wl)
        for fam in FAMILIES:
            if fam != "auto" and not supported(shape, fmt, fam):
                continue
            say(f"[gpu] random {fmt} #{i} {fam} shape {shape} bias={b is not None}")
            y, used = run(x, w, b, shape, fmt, fam, guard=64)
            assert_matches_oracle(y, x, w, b, shape, fmt, f"random {fmt} #{i} {used}")


# Shapes that reach each family's fast path with ragged tails: widths that
# are not multiples of any tile, channel counts one vector over a tile, one
# output row/column, filters larger than the image, heavy padding.
EDGE = [
    (1, 16, 16, 8, 3, 3, 1, 1, 1),
    (2, 9, 57, 132, 3, 3, 1, 1, 1),
    (1, 5, 5, 128, 3, 3, 1, 1, 0),        # 3x3 output
    (1, 1, 1, 64, 3, 3, 1, 1, 1),         # 1x1 image
    (1, 3, 3, 32, 7, 7, 1, 1, 3),         # filter larger than the image
    (2, 23, 17, 96, 7, 7, 1, 1, 3),
    (1, 40, 70, 104, 7, 7, 1, 1, 3),
    (1, 20, 20, 16, 31, 31, 1, 1, 15),
    (1, 64, 61, 24, 31, 31, 1, 1, 15),
    (2, 33, 35, 64, 5, 5, 2, 2, 4),
    (1, 30, 30, 32, 3, 3, 2, 1, 1),
    (1, 8, 8, 16, 3, 3, 1, 1, 6),         # padding wider than the filter
    (3, 14, 14, 48, 5, 5, 1, 1, 2),
    (1, 9, 11, 16, 1, 1, 1, 1, 0),        # 1x1 filter
    (2, 12, 13, 8, 1, 7, 1, 1, 3),        # 1x7: the first and last 3 output rows see padding only
    (1, 13, 10, 24, 7, 1, 1, 1, 0),       # 7x1
    (1, 10, 10, 1, 3, 3, 1, 1, 1),        # one channel
    (1, 2, 2, 8, 3, 3, 1, 1, 2),          # outputs whose taps are all padding
    (1, 5, 6, 8, 3, 3, 1, 3, 3),          # dilation wider than the image
    (1, 7, 7, 16, 3, 3, 3, 1, 0),         # stride equal to the filter
]


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16", "i8"])
def test_edge_shapes(fmt):
    rng = np.random.default_rng(5)
    for shape in EDGE:
        N, H, W, C, FH, FW, S, D, P = shape
        wl = synth.Workload("edge", fmt, N, H, W, C, FH, FW, S, D, P,
                            ("int", -128, 127) if fmt == "i8" else ("normal", 0.0, 1.0),
                            ("int", -128, 127) if fmt == "i8" else ("normal", 0.0, 1.0 / (FH * FW)),
                            ("int", -2**15, 2**15) if fmt == "i8" else ("uniform", -0.1, 0.1),
                            int(rng.integers(0, 2**31)))
        x, w, b = make_inputs(wl)
        for fam in FAMILIES:
            if fam != "auto" and not supported(shape, fmt, fam):
                continue
            say(f"[gpu] edge {fmt} {fam} shape {shape}")
            y, used = run(x, w, b, shape, fmt, fam, guard=256)
            assert_matches_oracle(y, x, w, b, shape, fmt, f"edge {fmt} {shape} {used}")


# ----------------------------------------------------- exact special cases

@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16", "i8"])
def test_delta_identity_bit_exact(fmt):
    """A centred one-hot filter with unit stride and same padding copies x to
    y exactly (no bias), in every family and dtype."""
    rng = np.random.default_rng(6)
    for F in (3, 5, 7, 31):
        shape = (2, 19, 23, 64, F, F, 1, 1, F // 2)
        wl = synth.Workload("delta", fmt, 2, 19, 23, 64, F, F, 1, 1, F // 2,
                            ("int", -128, 127) if fmt == "i8" else ("normal", 0.0, 1.0),
                            ("ones",), None, int(rng.integers(0, 2**31)))
        x, _, _ = make_inputs(wl)
        w = np.zeros((F, F, 64), x.dtype)
        w[F // 2, F // 2, :] = 1 if fmt == "i8" else synth.to_storage(np.ones(64), fmt)
        for fam in FAMILIES:
            if fam != "auto" and not supported(shape, fmt, fam):
                continue
            say(f"[gpu] delta {fmt} F={F} {fam}")
            y, used = run(x, w, None, shape, fmt, fam)
            want = x.astype(np.int32) if fmt == "i8" else x
            assert np.array_equal(y.view(np.uint8), np.ascontiguousarray(want).view(np.uint8)), \
                f"delta {fmt} F={F} {used}"


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16", "i8"])
def test_box_counts_exact(fmt):
    """x = 1, w = 1, no bias: each output is the number of taps inside the
    image, exactly (rounded once to the output format: 961 -> 960 in bf16)."""
    for shape in [(1, 16, 16, 8, 3, 3, 1, 1, 1), (2, 40, 37, 64, 31, 31, 1, 1, 15),
                  (1, 56, 56, 96, 7, 7, 1, 1, 3), (1, 33, 31, 16, 5, 5, 2, 2, 4)]:
        N, H, W, C, FH, FW, S, D, P = shape
        one = np.int8(1) if fmt == "i8" else synth.to_storage(np.ones(1), fmt)[0]
        x = np.full((N, H, W, C), one)
        w = np.full((FH, FW, C), one)
        OH = oracle.out_dim(H, FH, S, D, P)
        OW = oracle.out_dim(W, FW, S, D, P)
        cnt_h = np.array([sum(0 <= o * S - P + f * D < H for f in range(FH)) for o in range(OH)])
        cnt_w = np.array([sum(0 <= o * S - P + f * D < W for f in range(FW)) for o in range(OW)])
        cnt = (cnt_h[:, None] * cnt_w[None, :]).astype(np.float64)
        want = np.broadcast_to(cnt[None, :, :, None], (N, OH, OW, C))
        want = want.astype(np.int32) if fmt == "i8" else synth.to_storage(want, fmt)
        for fam in FAMILIES:
            if fam != "auto" and not supported(shape, fmt, fam):
                continue
            say(f"[gpu] box {fmt} {shape} {fam}")
            y, used = run(x, w, None, shape, fmt, fam)
            assert np.array_equal(y.view(np.uint8), np.ascontiguousarray(want).view(np.uint8)), \
                f"box {fmt} {shape} {used}"


# ------------------------------------------------ alignment, streams, repeats

@pytest.mark.parametrize("fmt", ["f32", "bf16", "i8"])
def test_misaligned_pointers_fall_back(fmt):
    """Tensors that start one element past a 16-byte boundary still give the
    right answer (the direct family runs them)."""
    shape = (2, 12, 13, 64, 3, 3, 1, 1, 1)
    wl = synth.Workload("mis", fmt, *shape,
                        ("int", -128, 127) if fmt == "i8" else ("normal", 0.0, 1.0),
                        ("int", -128, 127) if fmt == "i8" else ("normal", 0.0, 1 / 9),
                        ("int", -100, 100) if fmt == "i8" else ("uniform", -0.1, 0.1), 77)
    x, w, b = make_inputs(wl)
    from gpu_helpers import to_dev, y_torch_dtype, y_to_host
    xd = to_dev(np.concatenate([x.ravel()[:1], x.ravel()]), fmt)[1:]
    wd = to_dev(np.concatenate([w.ravel()[:1], w.ravel()]), fmt)[1:]
    bd = to_dev(np.concatenate([b[:1], b]), "f32")[1:]
    h = dw.dwconv_create(*shape, fmt)
    try:
        OH, OW = dw.dwconv_output_dims(h)
        yb = torch.empty(2 * OH * OW * 64 + 1, dtype=y_torch_dtype(fmt), device=DEV)
        y = yb[1:]
        say(f"[gpu] misaligned {fmt}")
        dw.dwconv_fwd(h, xd.data_ptr(), wd.data_ptr(), bd.data_ptr(), y.data_ptr(), None)
        torch.cuda.synchronize()
        yh = y_to_host(y, fmt).reshape(2, OH, OW, 64)
    finally:
        dw.dwconv_destroy(h)
    assert_matches_oracle(yh, x, w, b, shape, fmt, f"misaligned {fmt}")


def test_repeat_runs_bitwise_identical_and_stream():
    wl = WORKLOADS["convnext_f16_7x7"]
    x, w, b = make_inputs(wl, n=4)
    shape = (4,) + shape_of(wl)[1:]
    say("[gpu] repeat determinism on a side stream")
    y1, _ = run(x, w, b, shape, "f16")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y2, _ = run(x, w, b, shape, "f16")
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


# ------------------------------------------------ every compiled tiling

REG_TILES = {
    "f32": ["4x14p2ni", "4x14p2n", "2x28p2n", "4x8p2n"],
    "f16": ["4x14p2n", "2x14p2n"],
    "bf16": ["4x14p2n", "2x14p2n"],
}


@pytest.mark.parametrize("F", [5, 7, 9])
def test_column_stream_wide_filters(F):
    """The fp32 5x5 (two channels per lane), 7x7 and 9x9 (one) column
    streams: ragged
    row strips and column groups, an image shorter than a strip, odd
    channel-vector counts, padding from 0 to F - 1, against the oracle."""
    rng = np.random.default_rng(86 + F)
    for shape in [(2, 30, 19, 16, F, F, 1, 1, F // 2), (1, 5, 57, 8, F, F, 1, 1, F // 2),
                  (1, 33, 16, 6, F, F, 1, 1, 0), (1, 17, 17, 10, F, F, 1, 1, F - 1),
                  (3, 40, 41, 2, F, F, 1, 1, 1)]:
        wl = synth.Workload("csw", "f32", *shape, ("normal", 0.0, 1.0),
                            ("normal", 0.0, 1 / F**2), ("uniform", -0.1, 0.1),
                            int(rng.integers(0, 2**31)))
        x, w, b = make_inputs(wl)
        h = dw.dwconv_create(*shape, "f32")
        desc = dw.dwconv_plan_describe(h)
        dw.dwconv_destroy(h)
        assert desc.startswith("colstream") and f"{F}x{F}" in desc, desc
        say(f"[gpu] column stream {F}x{F} {shape}")
        y, used = run(x, w, b, shape, "f32", "auto", guard=512)
        assert_matches_oracle(y, x, w, b, shape, "f32", f"cs{F} {shape}")


@pytest.mark.parametrize("fmt", sorted(REG_TILES))
def test_each_column_stream_tiling(fmt, monkeypatch):
    """Each compiled column-stream tiling (picked through the tile tuning choice
    tuning hook) against the oracle, on shapes with ragged row and column
    strips, an image shorter than a strip, and a batch."""
    rng = np.random.default_rng(9)
    shapes = [(2, 30, 19, 64, 3, 3, 1, 1, 1), (1, 5, 57, 32, 3, 3, 1, 1, 1),
              (3, 17, 16, 128, 3, 3, 1, 1, 0), (1, 56, 56, 128, 3, 3, 1, 1, 2)]
    for tile in REG_TILES[fmt]:
        monkeypatch.setenv("DWCONV_TUNE", f"tile={tile}")
        for shape in shapes:
            N, H, W, C, FH, FW, S, D, P = shape
            wl = synth.Workload("tile", fmt, *shape, ("normal", 0.0, 1.0),
                                ("normal", 0.0, 1 / 9), ("uniform", -0.1, 0.1),
                                int(rng.integers(0, 2**31)))
            x, w, b = make_inputs(wl)
            say(f"[gpu] tile {tile} {fmt} shape {shape}")
            y, used = run(x, w, b, shape, fmt, "rowwin", guard=512)
            assert_matches_oracle(y, x, w, b, shape, fmt, f"tile {tile} {shape}")
            h = dw.dwconv_create_variant(*shape, fmt, "rowwin")
            desc = dw.dwconv_plan_describe(h)
            dw.dwconv_destroy(h)
            assert desc.startswith("colstream"), desc


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
@pytest.mark.parametrize("tile", ["4x14p1n"])
def test_paired_tap_column_stream(tile, fmt, monkeypatch):
    """fp16 / bf16 5x5 with the taps of each filter row paired for v_dot2
    (the fifth tap paired with a zero), each compiled tiling: ragged row and
    column strips, two channels (one channel pair per lane), padding 0 to 4,
    no bias, against the oracle; and the planner's pick of this family for a
    large map."""
    rng = np.random.default_rng(95)
    monkeypatch.setenv("DWCONV_TUNE", f"tile={tile}")
    for shape, bias in [((2, 23, 37, 16, 5, 5, 1, 1, 2), True), ((1, 30, 19, 2, 5, 5, 1, 1, 0), True),
                        ((3, 17, 29, 6, 5, 5, 1, 1, 1), False), ((1, 40, 33, 10, 5, 5, 1, 1, 4), True),
                        ((1, 9, 70, 64, 5, 5, 1, 1, 3), True)]:
        wl = synth.Workload("dot2", fmt, *shape, ("normal", 0.0, 1.0), ("normal", 0.0, 1 / 25),
                            ("uniform", -0.1, 0.1), int(rng.integers(0, 2**31)))
        x, w, b = make_inputs(wl)
        if not bias:
            b = None
        say(f"[gpu] paired-tap column stream {tile} {shape}")
        y, used = run(x, w, b, shape, fmt, "rowwin", guard=512)
        assert_matches_oracle(y, x, w, b, shape, fmt, f"dot2 {fmt} {tile} {shape}")
        h = dw.dwconv_create_variant(*shape, fmt, "rowwin")
        desc = dw.dwconv_plan_describe(h)
        dw.dwconv_destroy(h)
        assert desc.startswith("colstream: VEC=2") and "5x5" in desc, desc
    monkeypatch.delenv("DWCONV_TUNE")
    if fmt != "f16":
        return
    shape = (16, 112, 112, 64, 5, 5, 1, 1, 2)
    wl = synth.Workload("dot2", "f16", *shape, ("normal", 0.0, 1.0), ("normal", 0.0, 1 / 25),
                        ("uniform", -0.1, 0.1), 96)
    x, w, b = make_inputs(wl)
    say(f"[gpu] paired-tap column stream, planner's pick {shape}")
    h = dw.dwconv_create(*shape, "f16")
    desc = dw.dwconv_plan_describe(h)
    dw.dwconv_destroy(h)
    assert desc.startswith("colstream: VEC=2"), desc
    y, used = run(x, w, b, shape, "f16", "auto", guard=512)
    assert_matches_oracle(y, x, w, b, shape, "f16", f"dot2 auto {shape}")


# The compiled LDS-tile entries, (dtype, F, S, D): int8 with D dividing S
# runs the tap-packed kernel, the rest the flat-row kernel.
LDS_ENTRIES = [("i8", 5, 2, 2), ("i8", 3, 1, 1), ("i8", 5, 1, 1), ("i8", 7, 1, 1),
               ("i8", 3, 2, 1), ("i8", 3, 2, 2),
               ("f32", 5, 2, 2), ("f32", 3, 1, 1), ("f32", 7, 1, 1),
               ("f16", 5, 2, 2), ("f16", 3, 1, 1), ("f16", 7, 1, 1),
               ("bf16", 5, 2, 2), ("bf16", 3, 1, 1), ("bf16", 7, 1, 1)]


@pytest.mark.parametrize("entry", LDS_ENTRIES, ids=lambda e: "%s-%dx%d-s%d-d%d" % (e[0], e[1], e[1], e[2], e[3]))
def test_each_lds_tile_entry(entry, monkeypatch):
    """Each compiled LDS-tile kernel against the oracle: channel counts of
    one, a ragged odd count, exactly one 64-lane group, one more than that and
    several groups; images narrower and shorter than a tile; paddings of
    zero, half the span and a full span; tile heights 1, 3 and the planner's."""
    fmt, F, S, D = entry
    rng = np.random.default_rng(17)
    span = (F - 1) * D
    shapes = [(1, 9, 13, 1, F, F, S, D, span // 2),
              (2, 17, 23, 61, F, F, S, D, span // 2),
              (1, 20, 19, 64, F, F, S, D, 0),
              (1, 12, 40, 65, F, F, S, D, span),
              (1, 30, 7, 130, F, F, S, D, 1)]
    for tb in ("", "1", "3"):
        if tb:
            monkeypatch.setenv("DWCONV_TUNE", f"lds_tb={tb}")
        else:
            monkeypatch.delenv("DWCONV_TUNE", raising=False)
        for shape in shapes:
            N, H, W, C, FH, FW, S_, D_, P = shape
            if (H + 2 * P - D * (F - 1) - 1) < 0 or (W + 2 * P - D * (F - 1) - 1) < 0:
                continue
            if fmt == "i8":
                dist, wdist, bd = ("int", -128, 127), ("int", -128, 127), ("int", -2**15, 2**15)
            else:
                dist, wdist, bd = ("normal", 0.0, 1.0), ("normal", 0.0, 1.0 / F), ("uniform", -0.1, 0.1)
            wl = synth.Workload("lds", fmt, *shape, dist, wdist, bd, int(rng.integers(0, 2**31)))
            x, w, b = make_inputs(wl)
            if not supported(shape, fmt, "ldstile"):
                continue
            h = dw.dwconv_create_variant(*shape, fmt, "ldstile")
            desc = dw.dwconv_plan_describe(h)
            dw.dwconv_destroy(h)
            say(f"[gpu] lds entry {entry} TB={tb or 'auto'} shape {shape}: {desc[:60]}")
            y, used = run(x, w, b, shape, fmt, "ldstile", guard=512)
            assert used == "ldstile", used
            assert_matches_oracle(y, x, w, b, shape, fmt, f"lds {entry} tb={tb} {shape}")
            if fmt == "i8" and S % D == 0:
                assert "tap-packed" in desc, desc


MFMA_SLICES = {  # channel slice -> (dtype, F) combinations it is compiled for
    4: [("f16", 31), ("bf16", 31), ("f16", 5), ("bf16", 9), ("f16", 41), ("bf16", 51)],
    8: [("f16", 7), ("bf16", 7), ("f16", 5), ("bf16", 17)],
    16: [("f16", 7), ("bf16", 7)],
}


@pytest.mark.parametrize("al", [0, 1])
@pytest.mark.parametrize("cs", sorted(MFMA_SLICES))
def test_each_mfma_channel_slice(cs, al, monkeypatch):
    """Each MFMA channel slice (picked through the mfma_cs tuning
    choice) against the oracle: compiled and runtime filter heights, one and two
    16-tap fragments, ragged strips, a short image and several slices; A
    windows by DPP row shift (al=0) and by LDS reads (al=1, the compiled
    7x7 and 31x31 entries)."""
    monkeypatch.setenv("DWCONV_TUNE", f"mfma_cs={cs},mfma_al={al}")
    rng = np.random.default_rng(31 + cs)
    for fmt, F in MFMA_SLICES[cs]:
        for (N, H, W, C) in [(1, 23, 37, 2 * cs), (2, 9, 70, cs), (1, 40, 17, 3 * cs)]:
            shape = (N, H, W, C, F, F, 1, 1, F // 2)
            if not supported(shape, fmt, "mfma"):
                continue
            wl = synth.Workload("mfma", fmt, *shape, ("normal", 0.0, 1.0),
                                ("normal", 0.0, 1.0 / F), ("uniform", -0.1, 0.1),
                                int(rng.integers(0, 2**31)))
            x, w, b = make_inputs(wl)
            h = dw.dwconv_create_variant(*shape, fmt, "mfma")
            desc = dw.dwconv_plan_describe(h)
            dw.dwconv_destroy(h)
            assert f"x {cs} ch" in desc, desc
            say(f"[gpu] mfma cs {cs} {fmt} shape {shape}")
            y, used = run(x, w, b, shape, fmt, "mfma", guard=512)
            assert used == "mfma", used
            assert_matches_oracle(y, x, w, b, shape, fmt, f"mfma cs{cs} {shape}")


@pytest.mark.parametrize("nb", [2, 4])
def test_mfma_strip_widths(nb, monkeypatch):
    """Strips of 32 and 64 output columns (forced through the mfma_nb tuning choice)
    for the compiled 7x7 and 31x31 entries and runtime filter heights with
    one and two fragments, against the oracle; widths that leave a ragged
    last strip and an output narrower than one strip."""
    monkeypatch.setenv("DWCONV_TUNE", f"mfma_nb={nb}")
    rng = np.random.default_rng(60 + nb)
    for fmt, F in [("f16", 7), ("bf16", 31), ("bf16", 5), ("f16", 17)]:
        for (N, H, W, C) in [(1, 20, 45, 16), (2, 17, 13, 8)]:
            shape = (N, H, W, C, F, F, 1, 1, F // 2)
            wl = synth.Workload("mfma", fmt, *shape, ("normal", 0.0, 1.0),
                                ("normal", 0.0, 1.0 / F), ("uniform", -0.1, 0.1),
                                int(rng.integers(0, 2**31)))
            x, w, b = make_inputs(wl)
            h = dw.dwconv_create_variant(*shape, fmt, "mfma")
            desc = dw.dwconv_plan_describe(h)
            dw.dwconv_destroy(h)
            assert f"strips of {16 * nb} cols" in desc, desc
            say(f"[gpu] mfma strips of {16 * nb} columns, {fmt} shape {shape}")
            y, used = run(x, w, b, shape, fmt, "mfma", guard=512)
            assert used == "mfma", used
            assert_matches_oracle(y, x, w, b, shape, fmt, f"mfma nb{nb} {shape}")


@pytest.mark.parametrize("slots", [1, 2, 3])
def test_mfma_slot_renumbering(slots, monkeypatch):
    """The workgroups one CU holds at once take consecutive tiles of their
    XCD's range (mfma_slots=N forces N; unset, the planner takes the
    occupancy for filters of 16 rows or more and 1 below).  The renumbering
    must be a bijection on the grid: every output of grids with whole and
    partial dispatcher passes (8 XCDs x 32 CUs x N slots) matches the
    oracle, for a short and a tall filter."""
    monkeypatch.setenv("DWCONV_TUNE", f"mfma_slots={slots}")
    rng = np.random.default_rng(70 + slots)
    # 7x7 fp16: 12 slices x 2 strips x 32 images = 768 workgroups;
    # 31x31 bf16: 32 slices x 16 images = 512 workgroups
    for fmt, F, (N, H, W, C) in [("f16", 7, (32, 56, 56, 96)), ("bf16", 31, (16, 40, 60, 128))]:
        shape = (N, H, W, C, F, F, 1, 1, F // 2)
        wl = synth.Workload("mfma", fmt, *shape, ("normal", 0.0, 1.0),
                            ("normal", 0.0, 1.0 / F), ("uniform", -0.1, 0.1),
                            int(rng.integers(0, 2**31)))
        x, w, b = make_inputs(wl)
        say(f"[gpu] mfma slots {slots}, {fmt} shape {shape}")
        y, used = run(x, w, b, shape, fmt, "mfma", guard=512)
        assert used == "mfma", used
        assert_matches_oracle(y, x, w, b, shape, fmt, f"mfma slots{slots} {shape}")


ROW_PACKED = {  # tuning choice -> (dtype, FH, FW) the compiled entries cover
    "mfma_pk=2": [("bf16", 31, 31), ("f16", 31, 25), ("f16", 7, 7), ("bf16", 7, 9),
                  ("bf16", 13, 13), ("f16", 21, 25), ("bf16", 32, 17), ("f16", 1, 31)],
    "mfma_pk=4": [("f16", 31, 31), ("bf16", 31, 27), ("f16", 7, 7), ("bf16", 7, 5),
                  ("f16", 5, 5), ("bf16", 9, 9), ("f16", 3, 7), ("bf16", 2, 3)],
    "mfma_pk=2,mfma_cs=4,mfma_nb=2": [("f16", 9, 17), ("bf16", 15, 21)],
    "mfma_pk=4,mfma_cs=4": [("bf16", 6, 9), ("f16", 11, 8)],
    "mfma_pk=2,mfma_cs=8": [("bf16", 31, 31), ("f16", 31, 19)],
    "mfma_pk=2,mfma_nb=2": [("bf16", 31, 31), ("f16", 31, 33)],
    "mfma_pk=4,mfma_fhk=0": [("f16", 7, 7), ("bf16", 7, 9)],
    "mfma_pk=2,mfma_fhk=0": [("bf16", 31, 31), ("f16", 31, 21)],
    # filters of 34 to 65 taps and up to 64 rows: four and five windows with
    # the chain folded every 16 and 12 row pairs
    "mfma_pk=2,mfma_cs=4": [("f16", 41, 41), ("bf16", 51, 51), ("f16", 64, 65),
                            ("bf16", 33, 34), ("f16", 40, 50), ("bf16", 17, 49)],
    "mfma_pk=2,mfma_cs=4,mfma_nb=2,mfma_fhk=0": [("bf16", 41, 41), ("f16", 51, 51)],
    # each channel's row groups split over two wavefronts (the second half
    # empty for filters of one or two rows)
    "mfma_pk=2,mfma_ks=2": [("f16", 51, 51), ("bf16", 64, 65), ("f16", 17, 53),
                            ("bf16", 40, 41), ("bf16", 1, 50), ("f16", 3, 60)],
    "mfma_pk=2,mfma_ks=2,mfma_nb=2": [("f16", 57, 57), ("bf16", 33, 50)],
}


@pytest.mark.parametrize("tune", sorted(ROW_PACKED))
def test_mfma_row_packing(tune, monkeypatch):
    """Filter rows packed 2 or 4 to an MFMA (forced through the mfma_pk
    tuning choice, with the channel slice, strip width and kept-B choices
    of each compiled entry) against the oracle: 7- and 31-row filters (the
    last group has PK - FH mod PK rows of zero taps), filter widths that need
    the same number of windows, filters of 34 to 65 taps and up to 64 rows
    (folded chains), ragged strips and row blocks, images shorter than the
    filter, several channel slices; last row blocks of 7, 8 and 9
    rows and an output of 6 rows (blocks of at most 8 rows take the half
    form: 8 rows of two column blocks per MFMA row set)."""
    monkeypatch.setenv("DWCONV_TUNE", tune)
    pk = int(tune.split(",")[0].split("=")[1])
    rng = np.random.default_rng(70 + len(tune))
    for fmt, FH, FW in ROW_PACKED[tune]:
        for (N, H, W, C) in [(1, 23, 37, 16), (2, 9, 70, 8), (1, 40, 17, 24), (1, 56, 56, 8),
                             (1, 6, 45, 8)]:
            shape = (N, H, W, C, FH, FW, 1, 1, max(FH, FW) // 2)
            assert supported(shape, fmt, "mfma"), shape
            wl = synth.Workload("mfma", fmt, *shape, ("normal", 0.0, 1.0),
                                ("normal", 0.0, 1.0 / (FH * FW)), ("uniform", -0.1, 0.1),
                                int(rng.integers(0, 2**31)))
            x, w, b = make_inputs(wl)
            h = dw.dwconv_create_variant(*shape, fmt, "mfma")
            desc = dw.dwconv_plan_describe(h)
            dw.dwconv_destroy(h)
            assert f"{pk} filter rows per MFMA" in desc, desc
            for cs in (4, 8):
                if f"mfma_cs={cs}" in tune:
                    assert f"x {cs} ch" in desc, desc
            if "mfma_nb=2" in tune:
                assert "strips of 32 cols" in desc, desc
            if "mfma_ks=2" in tune:
                assert "row groups split over two wavefronts" in desc, desc
            say(f"[gpu] mfma {tune}, {fmt} shape {shape}")
            y, used = run(x, w, b, shape, fmt, "mfma", guard=512)
            assert used == "mfma", used
            assert_matches_oracle(y, x, w, b, shape, fmt, f"mfma {tune} {shape}")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_mfma_random_shapes(fmt):
    """Random stride-1 shapes on the matrix cores, every output against the
    oracle: filter heights 1 to 64 and widths 5 to 65 (one, two or four
    filter rows per MFMA as the planner picks them, folded chains for the
    tallest and widest), channel counts that are multiples of 4 or 8, ragged
    maps narrower or shorter than a strip or a row block, padding from none
    to more than half the filter, and a NaN guard band around y."""
    rng = np.random.default_rng({"f16": 91, "bf16": 92}[fmt])
    done = 0
    while done < 64:
        FH = int(rng.integers(1, 65))
        FW = int(rng.integers(5, 66))
        H = int(rng.integers(1, 49))
        W = int(rng.integers(1, 57))
        C = 4 * int(rng.integers(1, 7))
        P = int(rng.integers(0, max(FH, FW) // 2 + 3))
        shape = (1, H, W, C, FH, FW, 1, 1, P)
        if H + 2 * P - FH < 0 or W + 2 * P - FW < 0 or not supported(shape, fmt, "mfma"):
            continue
        h = dw.dwconv_create_variant(*shape, fmt, "mfma")
        desc = dw.dwconv_plan_describe(h)
        dw.dwconv_destroy(h)
        wl = synth.Workload("mfma_rand", fmt, *shape, ("normal", 0.0, 1.0),
                            ("normal", 0.0, 1.0 / (FH * FW)),
                            ("uniform", -0.1, 0.1) if rng.integers(0, 4) else None,
                            int(rng.integers(0, 2**31)))
        x, w, b = make_inputs(wl)
        say(f"[gpu] mfma random {fmt} #{done} shape {shape}: {desc[:70]}")
        y, used = run(x, w, b, shape, fmt, "mfma", guard=256)
        assert used == "mfma", used
        assert_matches_oracle(y, x, w, b, shape, fmt, f"mfma random {fmt} {shape} ({desc[:60]})")
        done += 1


# wide filters on the matrix cores: the compiled 31-row entry, ragged row
# blocks and strips, outputs narrower than one strip, non-square filters of
# 17 to 33 taps, one output row
WIDE = [((1, 56, 56, 8, 31, 31, 1, 1, 15), "bf16"),
          ((2, 33, 65, 12, 31, 31, 1, 1, 15), "f16"),
          ((1, 40, 20, 4, 17, 17, 1, 1, 8), "bf16"),
          ((1, 31, 97, 8, 5, 33, 1, 1, 16), "f16"),
          ((3, 70, 45, 4, 23, 19, 1, 1, 9), "bf16"),
          ((1, 1, 40, 4, 1, 25, 1, 1, 12), "f16"),
          ((1, 30, 30, 4, 31, 31, 1, 1, 1), "bf16"),
          ((2, 64, 64, 16, 31, 17, 1, 1, 3), "f16")]


@pytest.mark.parametrize("case", range(len(WIDE)))
def test_wide_filter_shapes(case):
    """Wide and non-square filters on the matrix cores, every output against
    the oracle, with a NaN guard band around y."""
    shape, fmt = WIDE[case]
    N, H, W, C, FH, FW, S, D, P = shape
    rng = np.random.default_rng(700 + case)
    wl = synth.Workload("wide", fmt, *shape, ("normal", 0.0, 1.0),
                        ("normal", 0.0, 1.0 / (FH * FW)), ("uniform", -0.1, 0.1),
                        int(rng.integers(0, 2**31)))
    x, w, b = make_inputs(wl)
    h = dw.dwconv_create_variant(*shape, fmt, "auto")
    desc = dw.dwconv_plan_describe(h)
    dw.dwconv_destroy(h)
    assert desc.startswith("mfma"), desc
    say(f"[gpu] wide filter {fmt} shape {shape}: {desc}")
    y, used = run(x, w, b, shape, fmt, "auto", guard=1024)
    assert used == "mfma", used
    rep = assert_matches_oracle(y, x, w, b, shape, fmt, f"wide {shape}")
    say(f"      ok {rep}")


# --------------------------------------------- tensors at the size limit

# just under 2^31 elements (the largest tensors a plan accepts): per-image
# element offsets reach the 32-bit range the kernels index within an image
BIG = [((1, 16383, 16384, 8, 3, 3, 1, 1, 1), "f32"),      # column stream
       ((1, 16383, 16384, 8, 7, 7, 1, 1, 3), "f16"),      # MFMA, 8-channel slices
       ((1, 16383, 16384, 8, 31, 31, 1, 1, 15), "bf16"),  # MFMA, two fragments
       ((2, 1100, 16000, 61, 5, 5, 2, 2, 4), "i8")]       # int8 tap-packed


@pytest.mark.parametrize("case", range(len(BIG)))
def test_size_limit_sampled(case):
    """The largest accepted tensors, input drawn on the GPU: 4000 random
    outputs plus the first and last pixels of every image, each against the
    oracle on the dilated FH x FW input patch that output reads (zeros
    outside the image), gathered from the device."""
    shape, fmt = BIG[case]
    N, H, W, C, FH, FW, S, D, P = shape
    OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
    rng = np.random.default_rng(900 + case)
    w = synth.to_storage(rng.normal(0, 1 / np.sqrt(FH * FW), (FH, FW, C)), fmt) if fmt != "i8" \
        else rng.integers(-128, 128, (FH, FW, C)).astype(np.int8)
    b = synth.to_storage(rng.uniform(-0.1, 0.1, C), "f32") if fmt != "i8" \
        else rng.integers(-2**15, 2**15 + 1, C).astype(np.int32)
    say(f"[gpu] size limit {fmt} {shape}: drawing the input on the device")
    x = synth.device_input((N, H, W, C), fmt, 910 + case, DEV)
    ydt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
           "i8": torch.int32}[fmt]
    y = torch.empty((N, OH, OW, C), dtype=ydt, device=DEV)
    wt = (torch.from_numpy(w.view(np.int16)).view(torch.bfloat16) if fmt == "bf16"
          else torch.from_numpy(w)).to(DEV)
    bt = torch.from_numpy(b).to(DEV)
    h = dw.dwconv_create(*shape, fmt)
    try:
        desc = dw.dwconv_plan_describe(h)
        say(f"      plan {desc[:60]}")
        dw.dwconv_fwd(h, x, wt, bt, y)
        torch.cuda.synchronize()
    finally:
        dw.dwconv_destroy(h)
    # sampled outputs: random, plus the corners of every image
    total = N * OH * OW * C
    idx = [rng.integers(0, total, 4000)]
    for n in range(N):
        for (oh, ow) in [(0, 0), (0, OW - 1), (OH - 1, 0), (OH - 1, OW - 1)]:
            idx.append(((n * OH + oh) * OW + ow) * C + np.arange(C))
    idx = np.unique(np.concatenate(idx))
    c_ = idx % C
    ow_ = (idx // C) % OW
    oh_ = (idx // (C * OW)) % OH
    n_ = idx // (C * OW * OH)
    # the dilated patch each sampled output reads, gathered on the device
    ih = oh_[:, None] * S - P + D * np.arange(FH)[None, :]          # npts x FH
    iw = ow_[:, None] * S - P + D * np.arange(FW)[None, :]          # npts x FW
    inside = ((ih >= 0) & (ih < H))[:, :, None] & ((iw >= 0) & (iw < W))[:, None, :]
    flat = ((n_[:, None, None] * H + np.clip(ih, 0, H - 1)[:, :, None]) * W
            + np.clip(iw, 0, W - 1)[:, None, :]) * C + c_[:, None, None]
    xf = x.view(-1)
    g = xf[torch.from_numpy(flat.reshape(-1)).to(DEV)]
    g = (g.view(torch.int16).cpu().numpy().view(np.uint16) if fmt == "bf16"
         else g.cpu().numpy()).reshape(flat.shape)
    zero = np.zeros((), g.dtype)
    patches = np.where(inside, g, zero)
    yv = y.view(-1)[torch.from_numpy(idx).to(DEV)]
    yv = (yv.view(torch.int16).cpu().numpy().view(np.uint16) if fmt == "bf16"
          else yv.cpu().numpy())
    del x, y
    torch.cuda.empty_cache()
    # the oracle, one channel at a time: every sampled output of channel c is
    # one 1 x 1 output of an FH x FW image (stride 1, dilation 1, no padding)
    for c in range(C):
        sel = np.nonzero(c_ == c)[0]
        if sel.size == 0:
            continue
        xs = np.ascontiguousarray(patches[sel][:, :, :, None])
        ws = np.ascontiguousarray(w[:, :, c:c + 1])
        bs = np.ascontiguousarray(b[c:c + 1])
        ye, scale = oracle.points(xs, ws, bs, 1, 1, 0, fmt, np.arange(sel.size))
        what = f"size limit {fmt} {shape} channel {c}"
        if fmt == "i8":
            check.assert_int(yv[sel], ye, what)
        else:
            check.assert_float(yv[sel], fmt, ye, scale, what)
    say(f"      ok: {idx.size} outputs")


# ------------------------------------------- filters of any size (row chunks)

@pytest.mark.parametrize("fmt", ["f32", "f32-tm8", "f16", "bf16"])
def test_row_chunks_any_filter(fmt, monkeypatch):
    """The row-chunk kernel (stride 1, dilation 1, any filter the compiled
    tilings do not cover): chunk-boundary widths (8, 9, 15, 16, 17), tall
    and flat filters, padding below, at and past half the filter, ragged
    widths, against the whole-tensor oracle."""
    rng = np.random.default_rng({"f32": 81, "f32-tm8": 84, "f16": 82, "bf16": 83}[fmt])
    if fmt == "f32-tm8":  # the 8-wide fp32 tiling (the chunk_tm tuning choice)
        monkeypatch.setenv("DWCONV_TUNE", "chunk_tm=8")
        fmt = "f32"
    vec = 4 if fmt == "f32" else 8
    cases = [(2, 23, 37, 2 * vec, 9, 9, 4), (1, 20, 41, vec, 8, 8, 3), (1, 17, 30, 3 * vec, 15, 16, 7),
             (1, 33, 35, vec, 17, 17, 8), (1, 12, 51, vec, 1, 33, 16), (1, 40, 20, 2 * vec, 33, 2, 1),
             (1, 52, 53, vec, 51, 51, 25), (2, 9, 14, vec, 6, 11, 0), (1, 16, 16, vec, 12, 12, 13)]
    for (N, H, W, C, FH, FW, P) in cases:
        shape = (N, H, W, C, FH, FW, 1, 1, P)
        if oracle.out_dim(H, FH, 1, 1, P) < 1 or oracle.out_dim(W, FW, 1, 1, P) < 1:
            continue
        h = dw.dwconv_create_variant(*shape, fmt, "rowwin")
        desc = dw.dwconv_plan_describe(h)
        dw.dwconv_destroy(h)
        if not desc.startswith("rowchunk"):
            continue  # a compiled tiling covers this filter
        wl = synth.Workload("chunk", fmt, *shape, ("normal", 0.0, 1.0),
                            ("normal", 0.0, 1.0 / (FH * FW)), ("uniform", -0.1, 0.1),
                            int(rng.integers(0, 2**31)))
        x, w, b = make_inputs(wl)
        say(f"[gpu] row chunks {fmt} {shape}")
        y, used = run(x, w, b, shape, fmt, "rowwin", guard=256)
        assert_matches_oracle(y, x, w, b, shape, fmt, f"rowchunk {fmt} {shape}")


@pytest.mark.parametrize("fmt", ["f32", "f16"])
def test_sweep_maps_sampled(fmt):
    """The filter-size sweep's three feature maps (two images instead of
    128) at the sweep's filter sizes, through the planner's choice:
    every output of the first and last rows and 3000 random ones, each
    against the oracle."""
    rng = np.random.default_rng(84 if fmt == "f32" else 85)
    for (H, W, C) in [(128, 128, 128), (64, 64, 256), (32, 32, 1024)]:
        for F in (3, 9, 17, 31, 51):
            shape = (2, H, W, C, F, F, 1, 1, F // 2)
            wl = synth.Workload("sweep", fmt, *shape, ("normal", 0.0, 1.0),
                                ("normal", 0.0, 1.0 / (F * F)), ("uniform", -0.1, 0.1),
                                int(rng.integers(0, 2**31)))
            x, w, b = make_inputs(wl)
            OH, OW = H, W
            idx = [rng.integers(0, 2 * OH * OW * C, 3000)]
            for n in (0, 1):
                for oh in (0, OH - 1):
                    idx.append(((n * OH + oh) * OW * C) + np.arange(OW * C))
            idx = np.unique(np.concatenate(idx))
            ye, scale = oracle.points(x, w, b, 1, 1, F // 2, fmt, idx)
            say(f"[gpu] sweep map {fmt} {shape}")
            y, used = run(x, w, b, shape, fmt, "auto", guard=256)
            check.assert_float(y.ravel()[idx], fmt, ye, scale, f"sweep {fmt} {shape} {used}")
