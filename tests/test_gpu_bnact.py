"""GPU parity of the forward pass with the fused prologue act(x*s + b)
("Flash-DWC: Making Depthwise Convolution Compute-Efficient on GPUs",
section 5.2) through the C ABI, against the oracle's fwd_bn_act: the same
elementwise bound as the forward pass, |y - y_exact| <= 1e-5 * scale + 1e-6
on the value before the final rounding, scale = sum |x*s + b| * |w|.  For
fp16 / bf16 data the convolution's input U = act(x*s + b) is in the data's
format (one fp32 fused multiply-add, then rounded to nearest even), as a
separate BN + Act pass would store it."""
import numpy as np
import pytest
import torch

import depthwise_convolution_amd as dw
import oracle
from oracle import check
import synth
from synth import WORKLOADS, make_inputs

from gpu_helpers import to_dev, y_torch_dtype, say, DEV, run, shape_of

pytestmark = pytest.mark.gpu


def bn_params(C, seed):
    rng = np.random.default_rng(seed)
    s = rng.uniform(0.5, 1.5, C).astype(np.float32)
    b = rng.normal(0.0, 0.5, C).astype(np.float32)
    return s, b


def run_bnact(x, w, bias, s, b, act, shape, fmt, guard=256, offset=0):
    """y on the host from dwconv_fwd_bn_act; y sits in a guarded buffer
    (offset elements into it, to make the pointers misaligned)."""
    N, H, W, C, FH, FW, S, D, P = shape
    h = dw.dwconv_create(N, H, W, C, FH, FW, S, D, P, fmt)
    try:
        OH, OW = dw.dwconv_output_dims(h)
        n_y = N * OH * OW * C
        tdt = y_torch_dtype(fmt)
        buf = torch.full((n_y + 2 * guard + offset,), float("nan"), dtype=tdt, device=DEV)
        y = buf[guard + offset:guard + offset + n_y]
        xd = to_dev(x, fmt)
        if offset:
            xs = torch.empty(xd.numel() + offset, dtype=xd.dtype, device=DEV)
            xs[offset:].copy_(xd.reshape(-1))
            xd = xs[offset:]
        dw.dwconv_fwd_bn_act(h, xd, to_dev(w, fmt), None if bias is None else to_dev(bias, "f32"),
                             torch.from_numpy(s).to(DEV), torch.from_numpy(b).to(DEV), act, y)
        torch.cuda.synchronize()
        host = buf.view(torch.int16).cpu().numpy().view(np.uint16) if fmt == "bf16" \
            else buf.cpu().numpy()
        band = np.concatenate([host[:guard + offset], host[guard + offset + n_y:]])
        if fmt == "bf16":
            assert np.all(band == band[0]) and band[0] & 0x7f80 == 0x7f80, "write outside y"
        else:
            assert np.all(np.isnan(band)), "write outside y"
        return host[guard + offset:guard + offset + n_y].reshape(N, OH, OW, C), \
            dw.dwconv_fwd_bn_act_describe(h)
    finally:
        dw.dwconv_destroy(h)


def check_bnact(y, x, w, bias, s, b, act, shape, fmt, what):
    N, H, W, C, FH, FW, S, D, P = shape
    ref, scale = oracle.fwd_bn_act(x, w, bias, s, b, act, S, D, P, fmt, threads=8)
    return check.assert_float(y, fmt, ref, scale, what)


@pytest.mark.parametrize("name", ["tiny_f32_3x3", "mobilenet_f32_3x3", "convnext_f16_7x7"])
def test_workload_bn_act(name):
    wl = WORKLOADS[name]
    x, w, bias = make_inputs(wl)
    shape = shape_of(wl)
    s, b = bn_params(wl.C, 300 + wl.seed)
    for act in ("relu", "relu6", "none"):
        say(f"[gpu] bn+act {name} {act}")
        y, desc = run_bnact(x, w, bias, s, b, act, shape, wl.dtype)
        rep = check_bnact(y, x, w, bias, s, b, act, shape, wl.dtype, f"bnact {name} {act}")
        say(f"      ok ({desc[:40]}) {rep}")
        if name == "mobilenet_f32_3x3":
            break  # one activation at full size is enough for the big one


# one shape per fused family: column stream (3x3, fp32 5x5 and 7x7), compiled row
# window (strided), row chunks (11x11), direct (a channel count with no 16-byte
# vectors)
FAMILY_SHAPES = [((2, 30, 19, 16, 3, 3, 1, 1, 1), "colstream"),
                 ((1, 33, 29, 8, 5, 5, 1, 1, 2), "colstream"),
                 ((1, 26, 23, 8, 7, 7, 1, 1, 3), "colstream"),
                 ((2, 33, 35, 16, 5, 5, 2, 2, 4), "rowwin"),
                 ((1, 24, 31, 16, 11, 11, 1, 1, 5), "rowchunk"),
                 ((2, 13, 17, 13, 3, 3, 1, 1, 1), "direct"),
                 ((1, 20, 20, 16, 31, 31, 1, 1, 15), "rowwin")]


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_each_fused_family(fmt):
    rng = np.random.default_rng({"f32": 301, "f16": 302, "bf16": 303}[fmt])
    for shape, _ in FAMILY_SHAPES:
        N, H, W, C, FH, FW, S, D, P = shape
        wl = synth.Workload("bn", fmt, *shape, ("normal", 0.0, 1.0),
                            ("normal", 0.0, 1.0 / (FH * FW)), ("uniform", -0.1, 0.1),
                            int(rng.integers(0, 2**31)))
        x, w, bias = make_inputs(wl)
        s, b = bn_params(C, int(rng.integers(0, 2**31)))
        act = ("none", "relu", "relu6")[int(rng.integers(0, 3))]
        say(f"[gpu] bn+act {fmt} {shape} {act}")
        y, desc = run_bnact(x, w, bias, s, b, act, shape, fmt)
        check_bnact(y, x, w, bias, s, b, act, shape, fmt, f"bnact {fmt} {shape} {desc[:20]}")


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_random_small_bn_act(fmt):
    rng = np.random.default_rng({"f32": 311, "f16": 312, "bf16": 313}[fmt])
    for i in range(25):
        wl = synth.random_small(rng, fmt)
        x, w, bias = make_inputs(wl)
        shape = shape_of(wl)
        s, b = bn_params(wl.C, int(rng.integers(0, 2**31)))
        act = ("none", "relu", "relu6")[i % 3]
        say(f"[gpu] bn+act random {fmt} #{i} {shape} {act}")
        y, desc = run_bnact(x, w, bias, s, b, act, shape, fmt, guard=64)
        check_bnact(y, x, w, bias, s, b, act, shape, fmt, f"bnact random {fmt} #{i} {desc[:20]}")


def test_misaligned_pointers_take_the_fallback():
    rng = np.random.default_rng(320)
    shape, fmt = (2, 17, 19, 32, 3, 3, 1, 1, 1), "f32"
    wl = synth.Workload("bn", fmt, *shape, ("normal", 0.0, 1.0), ("normal", 0.0, 1 / 9),
                        ("uniform", -0.1, 0.1), 321)
    x, w, bias = make_inputs(wl)
    s, b = bn_params(32, 322)
    y, _ = run_bnact(x, w, bias, s, b, "relu", shape, fmt, offset=1)
    check_bnact(y, x, w, bias, s, b, "relu", shape, fmt, "bnact misaligned")


ACT_F32 = {"none": lambda v: v,
           "relu": lambda v: np.maximum(v, np.float32(0)),
           "relu6": lambda v: np.minimum(np.maximum(v, np.float32(0)), np.float32(6))}


def stored_u(x, s, act, fmt):
    """U = act(x * s) (bn_shift 0, so the fused multiply-add is the float32
    product) in fmt, by numpy's float16 / torch's bfloat16 conversion."""
    if fmt == "f16":
        return ACT_F32[act](x.astype(np.float32) * s).astype(np.float16)
    xf = (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    u = torch.from_numpy(np.ascontiguousarray(ACT_F32[act](xf * s))).to(torch.bfloat16)
    return u.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_fused_prologue_is_forward_of_stored_u(fmt):
    """fp16 / bf16: the fused pass is the forward pass of U stored in the
    data's format.  With bn_shift = 0 the host forms the same U with library
    conversions, and where the fused kernel runs the forward tiling the
    outputs are bit-identical: the 7x7 and 31x31 layers' tilings on the
    matrix cores (two images), a one-row-per-MFMA filter, and the vector
    column stream and (fp16, strided) row window."""
    rng = np.random.default_rng({"f16": 341, "bf16": 342}[fmt])
    for shape in [(2, 56, 56, 96, 7, 7, 1, 1, 3), (2, 56, 56, 128, 31, 31, 1, 1, 15),
                  (1, 40, 21, 8, 35, 9, 1, 1, 4), (2, 30, 19, 16, 3, 3, 1, 1, 1)] + \
            ([(2, 33, 35, 16, 5, 5, 2, 2, 4)] if fmt == "f16" else []):
        N, H, W, C, FH, FW, S, D, P = shape
        wl = synth.Workload("bn", fmt, *shape, ("normal", 0.0, 1.0),
                            ("normal", 0.0, 1.0 / (FH * FW)), ("uniform", -0.1, 0.1),
                            int(rng.integers(0, 2**31)))
        x, w, bias = make_inputs(wl)
        s = rng.uniform(0.5, 1.5, C).astype(np.float32)
        h = dw.dwconv_create(*shape, fmt)
        fdesc, pdesc = dw.dwconv_fwd_bn_act_describe(h), dw.dwconv_plan_describe(h)
        dw.dwconv_destroy(h)
        if pdesc.startswith("mfma"):
            tiling = pdesc.split("banded GEMM, ", 1)[1].split(" walked", 1)[0].split(", A by")[0]
            assert fdesc.startswith("mfma with the prologue fused") and tiling in fdesc, \
                (pdesc, fdesc)
        else:
            assert fdesc == pdesc, (pdesc, fdesc)
        for act in ("relu", "relu6", "none"):
            say(f"[gpu] fused = forward of stored U {fmt} {shape} {act}")
            y0, _ = run(stored_u(x, s, act, fmt), w, bias, shape, fmt, "auto", guard=64)
            y1, _ = run_bnact(x, w, bias, s, np.zeros(C, np.float32), act, shape, fmt,
                              guard=64)
            assert np.array_equal(y0.view(np.uint8), y1.view(np.uint8)), (shape, act)


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_identity_prologue_matches_plain_forward(fmt):
    """bn_scale = 1, bn_shift = 0, no activation: x*1 + 0 is x exactly, so
    where the fused plan is the forward plan the outputs are bit-identical."""
    rng = np.random.default_rng(330)
    for shape in [(2, 30, 19, 16, 3, 3, 1, 1, 1), (1, 24, 31, 16, 9, 9, 1, 1, 4)]:
        if fmt != "f32" and shape[4] == 9:
            continue   # fp16/bf16 9x9 runs the matrix cores unfused
        C = shape[3]
        wl = synth.Workload("bn", fmt, *shape, ("normal", 0.0, 1.0), ("normal", 0.0, 0.1),
                            ("uniform", -0.1, 0.1), int(rng.integers(0, 2**31)))
        x, w, bias = make_inputs(wl)
        h = dw.dwconv_create(*shape, fmt)
        same = dw.dwconv_fwd_bn_act_describe(h) == dw.dwconv_plan_describe(h)
        dw.dwconv_destroy(h)
        assert same, shape
        y0, _ = run(x, w, bias, shape, fmt, "auto", guard=64)
        y1, _ = run_bnact(x, w, bias, np.ones(C, np.float32), np.zeros(C, np.float32), "none",
                          shape, fmt, guard=64)
        assert np.array_equal(y0.view(np.uint8), y1.view(np.uint8)), shape


@pytest.mark.parametrize("tune", ["", "mfma_pk=1"])
@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_mfma_fused_prologue(fmt, tune, monkeypatch):
    """The prologue fused into the matrix-core kernel (U rounded to the data's
    format as the ring is written): filters kept in registers (5x5, 7x7),
    runtime heights (31x31, a 25-row filter), ragged strips, several channel
    slices and every activation, against the oracle; with the planner's
    choice of filter rows per MFMA and with one row per MFMA."""
    monkeypatch.setenv("DWCONV_TUNE", tune)
    rng = np.random.default_rng({"f16": 311, "bf16": 312}[fmt] + len(tune))
    for shape in [(2, 23, 37, 16, 7, 7, 1, 1, 3), (1, 30, 45, 8, 5, 5, 1, 1, 2),
                  (1, 40, 33, 8, 13, 13, 1, 1, 6), (1, 26, 19, 8, 31, 31, 1, 1, 15),
                  (1, 35, 20, 8, 25, 9, 1, 1, 4), (1, 17, 70, 24, 7, 7, 1, 1, 3)]:
        N, H, W, C, FH, FW, S, D, P = shape
        wl = synth.Workload("bn", fmt, *shape, ("normal", 0.0, 1.0),
                            ("normal", 0.0, 1.0 / (FH * FW)), ("uniform", -0.1, 0.1),
                            int(rng.integers(0, 2**31)))
        x, w, bias = make_inputs(wl)
        s, b = bn_params(C, int(rng.integers(0, 2**31)))
        for act in ("none", "relu", "relu6"):
            say(f"[gpu] bn+act on the matrix cores {fmt} {shape} {act}")
            y, desc = run_bnact(x, w, bias, s, b, act, shape, fmt)
            assert desc.startswith("mfma with the prologue fused"), desc
            if tune:
                assert "filter rows per MFMA" not in desc, desc
            check_bnact(y, x, w, bias, s, b, act, shape, fmt, f"bnact mfma {fmt} {shape} {act}")


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_mfma_fused_prologue_random_shapes(fmt):
    """The fused prologue on the matrix cores over random stride-1 shapes
    (filters of 1 to 32 rows and 5 to 33 taps, channel counts that are
    multiples of 4 or 8, ragged maps, padding from none to past half the
    filter, a random activation), every output against the oracle."""
    rng = np.random.default_rng({"f16": 331, "bf16": 332}[fmt])
    done = 0
    while done < 40:
        FH = int(rng.integers(1, 33))
        FW = int(rng.integers(5, 34))
        H = int(rng.integers(1, 41))
        W = int(rng.integers(1, 49))
        C = 4 * int(rng.integers(1, 7))
        P = int(rng.integers(0, max(FH, FW) // 2 + 3))
        shape = (1, H, W, C, FH, FW, 1, 1, P)
        if H + 2 * P - FH < 0 or W + 2 * P - FW < 0:
            continue
        h = dw.dwconv_create(*shape, fmt)
        desc = dw.dwconv_fwd_bn_act_describe(h)
        dw.dwconv_destroy(h)
        if not desc.startswith("mfma with the prologue fused"):
            continue
        wl = synth.Workload("bn_rand", fmt, *shape, ("normal", 0.0, 1.0),
                            ("normal", 0.0, 1.0 / (FH * FW)), ("uniform", -0.1, 0.1),
                            int(rng.integers(0, 2**31)))
        x, w, bias = make_inputs(wl)
        s, b = bn_params(C, int(rng.integers(0, 2**31)))
        act = ("none", "relu", "relu6")[int(rng.integers(0, 3))]
        say(f"[gpu] bn+act random {fmt} #{done} {shape} {act}: {desc[:70]}")
        y, desc = run_bnact(x, w, bias, s, b, act, shape, fmt)
        check_bnact(y, x, w, bias, s, b, act, shape, fmt, f"bnact random {fmt} {shape} {act}")
        done += 1


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_mfma_fused_prologue_row_packed(fmt, monkeypatch):
    """The fused prologue with filter rows packed into the MFMA's K: four
    7-row filter rows (kept B operands, 8-channel slices, 32-column strips)
    and two 31-row filter rows (64-column strips), ragged strips, a map
    whose last 8 rows form a half row
    block (after the full blocks for 7 rows, first for 31), an output of 6
    rows and every activation, against the oracle."""
    rng = np.random.default_rng({"f16": 321, "bf16": 322}[fmt])
    cases = [("mfma_pk=4", 7, [(2, 23, 37, 16), (1, 56, 56, 8), (1, 6, 45, 8)]),
             ("mfma_pk=2", 31, [(1, 26, 19, 4), (1, 56, 56, 4), (2, 40, 70, 8)])]
    for tune, F, shapes in cases:
        monkeypatch.setenv("DWCONV_TUNE", tune)
        for (N, H, W, C) in shapes:
            shape = (N, H, W, C, F, F, 1, 1, F // 2)
            wl = synth.Workload("bn", fmt, *shape, ("normal", 0.0, 1.0),
                                ("normal", 0.0, 1.0 / (F * F)), ("uniform", -0.1, 0.1),
                                int(rng.integers(0, 2**31)))
            x, w, bias = make_inputs(wl)
            s, b = bn_params(C, int(rng.integers(0, 2**31)))
            for act in ("none", "relu", "relu6"):
                say(f"[gpu] bn+act packed rows {tune} {fmt} {shape} {act}")
                y, desc = run_bnact(x, w, bias, s, b, act, shape, fmt)
                assert desc.startswith("mfma with the prologue fused"), desc
                assert f"{tune[-1]} filter rows per MFMA" in desc, desc
                check_bnact(y, x, w, bias, s, b, act, shape, fmt,
                            f"bnact mfma {tune} {fmt} {shape} {act}")


def test_fp16_5x5_column_stream_prologue():
    """A large fp16 5x5 map plans the column stream, so the fused pass runs
    its prologue variant (widened inputs, one fma per tap) there, for every
    activation, against the oracle."""
    shape = (16, 112, 112, 64, 5, 5, 1, 1, 2)
    wl = synth.Workload("bn", "f16", *shape, ("normal", 0.0, 1.0), ("normal", 0.0, 1 / 25),
                        ("uniform", -0.1, 0.1), 331)
    x, w, bias = make_inputs(wl)
    s, b = bn_params(64, 332)
    for act in ("relu", "relu6", "none"):
        say(f"[gpu] bn+act fp16 5x5 column stream {act}")
        y, desc = run_bnact(x, w, bias, s, b, act, shape, "f16")
        assert desc.startswith("colstream: VEC=2"), desc
        check_bnact(y, x, w, bias, s, b, act, shape, "f16", f"bnact f16 5x5 {act}")
