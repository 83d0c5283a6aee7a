"""GPU parity of the backward-data pass through the C ABI against the CPU
oracle's scatter form (oracle.bwd_data): the same elementwise bound as the
forward pass, |dx - dx_exact| <= 1e-5 * sum|dy*w| + 1e-6 on the value before
the one final rounding."""
import numpy as np
import pytest
import torch

import depthwise_convolution_amd as dw
import oracle
from oracle import check
import synth
from synth import WORKLOADS, make_inputs

from gpu_helpers import to_dev, y_torch_dtype, say, DEV

pytestmark = pytest.mark.gpu

FAMILIES = ["auto", "direct", "rowwin", "ldstile", "mfma"]


def run_bwd(dy, w, shape, fmt, variant="auto", guard=512):
    """dx on the host; dx sits inside a NaN-filled buffer whose guard bands
    are checked for stray writes."""
    N, H, W, C, FH, FW, S, D, P = shape
    h = dw.dwconv_create_variant(N, H, W, C, FH, FW, S, D, P, fmt, variant)
    try:
        assert dw.dwconv_bwd_data_supported(h)
        desc = dw.dwconv_bwd_data_describe(h)
        n_x = N * H * W * C
        buf = torch.full((n_x + 2 * guard,), float("nan"), dtype=y_torch_dtype(fmt), device=DEV)
        dx = buf[guard:guard + n_x]
        dw.dwconv_bwd_data(h, to_dev(dy, fmt), to_dev(w, fmt), dx)
        torch.cuda.synchronize()
        host = (buf.view(torch.int16).cpu().numpy().view(np.uint16) if fmt == "bf16"
                else buf.cpu().numpy())
        band = np.concatenate([host[:guard], host[guard + n_x:]])
        if fmt == "bf16":
            assert np.all(band == band[0]) and band[0] & 0x7f80 == 0x7f80, "write outside dx"
        else:
            assert np.all(np.isnan(band)), "write outside dx"
        return host[guard:guard + n_x].reshape(N, H, W, C), desc
    finally:
        dw.dwconv_destroy(h)


def check_bwd(dx, dy, w, shape, fmt, what, threads=8):
    ref, scale = oracle.bwd_data(dy, w, shape, fmt, threads=threads)
    return check.assert_float(dx, fmt, ref, scale, what)


def supported(shape, fmt, variant):
    try:
        h = dw.dwconv_create_variant(*shape, fmt, variant)
    except dw.DwconvError as e:
        if e.status == 2:
            return False
        raise
    ok = dw.dwconv_bwd_data_supported(h)
    dw.dwconv_destroy(h)
    return ok


def grads(shape, fmt, seed):
    """A seeded output gradient and filter of the forward shape's sizes."""
    N, H, W, C, FH, FW, S, D, P = shape
    OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
    wl = synth.Workload("bwd", fmt, N, OH, OW, C, FH, FW, 1, 1, 0, ("normal", 0.0, 1.0),
                        ("normal", 0.0, 1.0 / (FH * FW) ** 0.5), None, seed)
    dy, w, _ = make_inputs(wl)
    return dy, w


@pytest.mark.parametrize("name", ["mobilenet_f32_3x3", "convnext_f16_7x7"])
def test_workload_bwd(name):
    wl = WORKLOADS[name]
    shape = (wl.N, wl.H, wl.W, wl.C, wl.FH, wl.FW, wl.stride, wl.dilation, wl.pad)
    dy, w = grads(shape, wl.dtype, 100 + wl.seed)
    for fam in FAMILIES:
        if fam != "auto" and not supported(shape, wl.dtype, fam):
            continue
        say(f"[gpu] bwd {name} family {fam}")
        dx, desc = run_bwd(dy, w, shape, wl.dtype, fam)
        rep = check_bwd(dx, dy, w, shape, wl.dtype, f"bwd {name}/{fam}")
        say(f"      ok ({desc[:50]}) {rep}")


def test_largekernel_bwd():
    """The 31x31 bf16 layer at its full size (32 images), every input
    gradient element against the oracle."""
    wl = WORKLOADS["largekernel_bf16_31x31"]
    shape = (wl.N, wl.H, wl.W, wl.C, wl.FH, wl.FW, wl.stride, wl.dilation, wl.pad)
    dy, w = grads(shape, wl.dtype, 104)
    say(f"[gpu] bwd largekernel N={wl.N}")
    dx, desc = run_bwd(dy, w, shape, wl.dtype)
    say(f"[gpu] bwd largekernel: oracle pass ({desc[:50]})")
    rep = check_bwd(dx, dy, w, shape, wl.dtype, "bwd largekernel", threads=16)
    say(f"      ok {rep}")


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_bwd_random_small(fmt):
    rng = np.random.default_rng({"f32": 61, "f16": 62, "bf16": 63}[fmt])
    done = 0
    while done < 30:
        F = int(rng.choice([1, 3, 5, 7, 9, 17, 31]))
        D = int(rng.integers(1, 3))
        P = int(rng.integers(0, D * (F - 1) + 1))
        H, W = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        C = int(rng.choice([1, 3, 8, 16, 24, 64, 96]))
        N = int(rng.integers(1, 3))
        shape = (N, H, W, C, F, F, 1, D, P)
        if oracle.out_dim(H, F, 1, D, P) < 1 or oracle.out_dim(W, F, 1, D, P) < 1:
            continue
        dy, w = grads(shape, fmt, int(rng.integers(0, 2**31)))
        for fam in FAMILIES:
            if fam != "auto" and not supported(shape, fmt, fam):
                continue
            say(f"[gpu] bwd {fmt} {shape} {fam}")
            dx, _ = run_bwd(dy, w, shape, fmt, fam)
            check_bwd(dx, dy, w, shape, fmt, f"bwd {shape}/{fam}")
        done += 1


def test_bwd_is_adjoint_of_fwd_on_gpu():
    """<fwd(x), dy> = <x, bwd(dy)> with both passes on the GPU (fp32, small
    integers: every product and sum is exact)."""
    rng = np.random.default_rng(64)
    for shape in [(2, 17, 13, 8, 3, 3, 1, 1, 1), (1, 30, 30, 16, 5, 5, 1, 2, 3),
                  (1, 12, 21, 4, 7, 7, 1, 1, 6)]:
        N, H, W, C, FH, FW, S, D, P = shape
        OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
        x = rng.integers(-4, 5, size=(N, H, W, C)).astype(np.float32)
        w = rng.integers(-4, 5, size=(FH, FW, C)).astype(np.float32)
        dy = rng.integers(-4, 5, size=(N, OH, OW, C)).astype(np.float32)
        conv = dw.DepthwiseConv2d(*shape, dtype="f32")
        y = conv(torch.from_numpy(x).to(DEV), torch.from_numpy(w).to(DEV))
        dx = conv.backward_data(torch.from_numpy(dy).to(DEV), torch.from_numpy(w).to(DEV))
        torch.cuda.synchronize()
        conv.close()
        lhs = float(np.sum(y.cpu().numpy().astype(np.float64) * dy))
        rhs = float(np.sum(x.astype(np.float64) * dx.cpu().numpy()))
        assert lhs == rhs, (shape, lhs, rhs)


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_bwd_any_shape(fmt):
    """The direct backward kernel: strides 1-3, dilations 1-3, non-square
    filters and padding past D(F-1), against the oracle; misaligned dx too."""
    rng = np.random.default_rng({"f32": 65, "f16": 66, "bf16": 67}[fmt])
    done = 0
    while done < 30:
        FH, FW = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        S, D = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        P = int(rng.integers(0, 2 * max(FH, FW) + 1))
        H, W = int(rng.integers(1, 30)), int(rng.integers(1, 30))
        C = int(rng.choice([1, 3, 8, 13, 32, 64]))
        N = int(rng.integers(1, 3))
        shape = (N, H, W, C, FH, FW, S, D, P)
        if oracle.out_dim(H, FH, S, D, P) < 1 or oracle.out_dim(W, FW, S, D, P) < 1:
            continue
        if S == 1 and FH == FW and P <= D * (FH - 1):
            continue  # the forward families' path, covered above
        dy, w = grads(shape, fmt, int(rng.integers(0, 2**31)))
        say(f"[gpu] bwd any {fmt} {shape}")
        dx, desc = run_bwd(dy, w, shape, fmt)
        assert desc.startswith("direct (backward data)"), desc
        check_bwd(dx, dy, w, shape, fmt, f"bwd any {shape}")
        done += 1


def test_bwd_any_shape_is_adjoint():
    """<fwd(x), dy> = <x, bwd(dy)> on the GPU for strided, dilated and
    non-square shapes (fp32 small integers: exact)."""
    rng = np.random.default_rng(68)
    for shape in [(2, 17, 13, 8, 3, 3, 2, 1, 1), (1, 30, 31, 16, 5, 3, 3, 2, 4),
                  (1, 12, 21, 4, 2, 7, 2, 3, 9), (2, 9, 9, 12, 3, 3, 1, 1, 4)]:
        N, H, W, C, FH, FW, S, D, P = shape
        OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
        x = rng.integers(-4, 5, size=(N, H, W, C)).astype(np.float32)
        w = rng.integers(-4, 5, size=(FH, FW, C)).astype(np.float32)
        dy = rng.integers(-4, 5, size=(N, OH, OW, C)).astype(np.float32)
        conv = dw.DepthwiseConv2d(*shape, dtype="f32")
        y = conv(torch.from_numpy(x).to(DEV), torch.from_numpy(w).to(DEV))
        dx = conv.backward_data(torch.from_numpy(dy).to(DEV), torch.from_numpy(w).to(DEV))
        torch.cuda.synchronize()
        conv.close()
        lhs = float(np.sum(y.cpu().numpy().astype(np.float64) * dy))
        rhs = float(np.sum(x.astype(np.float64) * dx.cpu().numpy()))
        assert lhs == rhs, (shape, lhs, rhs)


# ------------------------------------------------------------ backward filter

def run_bwf(x, dy, shape, fmt, ws_offset=0):
    """dw on the host (float32), from a NaN-filled buffer whose guard bands
    are checked; the workspace is filled with garbage first.  ws_offset
    floats of offset give a workspace that is not 16-byte aligned (the
    matrix-core pass 1 then gives way to the vector one)."""
    N, H, W, C, FH, FW, S, D, P = shape
    h = dw.dwconv_create(N, H, W, C, FH, FW, S, D, P, fmt)
    try:
        nbytes = dw.dwconv_bwd_filter_workspace(h)
        ws = torch.full((nbytes // 4 + 1 + ws_offset,), float("nan"), dtype=torch.float32,
                        device=DEV)[ws_offset:]
        guard, n_w = 256, FH * FW * C
        buf = torch.full((n_w + 2 * guard,), float("nan"), dtype=torch.float32, device=DEV)
        dwt = buf[guard:guard + n_w]
        dw.dwconv_bwd_filter(h, to_dev(x, fmt), to_dev(dy, fmt), dwt, ws)
        torch.cuda.synchronize()
        host = buf.cpu().numpy()
        assert np.all(np.isnan(np.concatenate([host[:guard], host[guard + n_w:]]))), \
            "write outside dw"
        return host[guard:guard + n_w].reshape(FH, FW, C), dw.dwconv_bwd_filter_describe(h)
    finally:
        dw.dwconv_destroy(h)


def check_bwf(dwv, x, dy, shape, fmt, what):
    ref, scale = oracle.bwd_filter(x, dy, shape, fmt, threads=16)
    return check.assert_float(dwv, "f32", ref, scale, what)


def bwf_inputs(shape, fmt, seed):
    N, H, W, C, FH, FW, S, D, P = shape
    OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
    rng = np.random.default_rng(seed)
    x = synth.to_storage(rng.standard_normal((N, H, W, C)), fmt)
    dy = synth.to_storage(rng.standard_normal((N, OH, OW, C)), fmt)
    return x, dy


@pytest.mark.parametrize("name", ["mobilenet_f32_3x3", "convnext_f16_7x7",
                                  "largekernel_bf16_31x31"])
def test_workload_bwd_filter(name):
    wl = WORKLOADS[name]
    N = wl.N
    shape = (N, wl.H, wl.W, wl.C, wl.FH, wl.FW, wl.stride, wl.dilation, wl.pad)
    x, dy = bwf_inputs(shape, wl.dtype, 200 + wl.seed)
    say(f"[gpu] bwd filter {name} N={N}")
    dwv, desc = run_bwf(x, dy, shape, wl.dtype)
    rep = check_bwf(dwv, x, dy, shape, wl.dtype, f"bwf {name}")
    say(f"      ok ({desc[:60]}) {rep}")


@pytest.mark.parametrize("fmt", ["f32", "f16", "bf16"])
def test_bwd_filter_random_small(fmt):
    rng = np.random.default_rng({"f32": 71, "f16": 72, "bf16": 73}[fmt])
    for _ in range(30):
        wl = synth.random_small(rng, fmt, max_hw=24, max_c=40, max_f=9)
        shape = (wl.N, wl.H, wl.W, wl.C, wl.FH, wl.FW, wl.stride, wl.dilation, wl.pad)
        x, dy = bwf_inputs(shape, fmt, wl.seed)
        say(f"[gpu] bwd filter {fmt} {shape}")
        dwv, _ = run_bwf(x, dy, shape, fmt)
        check_bwf(dwv, x, dy, shape, fmt, f"bwf {shape}")


def test_bwd_filter_long_rows_and_many_chunks():
    """Rows longer than one 64-pixel partial, a batch large enough for many
    chunks, and a channel count with no 16-byte vectors."""
    for shape, fmt in [((2, 9, 150, 16, 3, 5, 1, 1, 2), "f32"),
                       ((8, 40, 40, 24, 7, 7, 1, 1, 3), "f16"),
                       ((3, 33, 70, 7, 5, 3, 1, 2, 1), "bf16")]:
        x, dy = bwf_inputs(shape, fmt, 7)
        say(f"[gpu] bwd filter {fmt} {shape}")
        dwv, desc = run_bwf(x, dy, shape, fmt)
        check_bwf(dwv, x, dy, shape, fmt, f"bwf {shape} ({desc})")


def test_bwd_filter_bilinear_and_deterministic():
    """<fwd(x, w), dy> = <w, dW(x, dy)> with both passes on the GPU (fp32,
    small integers: exact), and two runs agree bit for bit."""
    rng = np.random.default_rng(74)
    for shape in [(2, 17, 13, 8, 3, 3, 1, 1, 1), (1, 30, 30, 16, 5, 5, 2, 2, 3),
                  (3, 12, 21, 4, 7, 3, 1, 1, 2)]:
        N, H, W, C, FH, FW, S, D, P = shape
        OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
        x = rng.integers(-4, 5, size=(N, H, W, C)).astype(np.float32)
        w = rng.integers(-4, 5, size=(FH, FW, C)).astype(np.float32)
        dy = rng.integers(-4, 5, size=(N, OH, OW, C)).astype(np.float32)
        conv = dw.DepthwiseConv2d(*shape, dtype="f32")
        xd, dyd = torch.from_numpy(x).to(DEV), torch.from_numpy(dy).to(DEV)
        y = conv(xd, torch.from_numpy(w).to(DEV))
        g1 = conv.backward_filter(xd, dyd)
        g2 = conv.backward_filter(xd, dyd)
        torch.cuda.synchronize()
        conv.close()
        lhs = float(np.sum(y.cpu().numpy().astype(np.float64) * dy))
        rhs = float(np.sum(w.astype(np.float64) * g1.cpu().numpy()))
        assert lhs == rhs, (shape, lhs, rhs)
        assert torch.equal(g1, g2)


def test_bwd_filter_mfma_tiles():
    """The matrix-core pass 1 (fp16 / bf16, stride 1): one and two 16-tap
    tiles per axis, window counts at their limits (OW + FW - 1 = 64 and 65),
    padding wider than the filter, 4- and 8-channel slices, images split into
    row chunks, and a workspace that is not 16-byte aligned (vector pass 1);
    each against the oracle."""
    cases = [((2, 20, 58, 8, 7, 7, 1, 1, 3), "f16"),      # OW + FW - 1 = 64: 2 windows
             ((2, 20, 59, 8, 7, 7, 1, 1, 3), "bf16"),     # 65: 4 windows
             ((1, 40, 23, 12, 17, 5, 1, 1, 8), "f16"),    # two row tiles
             ((1, 21, 40, 4, 3, 31, 1, 1, 15), "bf16"),   # two column tiles
             ((1, 52, 52, 4, 31, 31, 1, 1, 15), "f16"),   # 31 x 31, 3 windows
             ((1, 100, 20, 8, 3, 3, 1, 1, 1), "bf16"),    # rows split into chunks
             ((1, 30, 12, 16, 3, 5, 1, 1, 6), "f16"),     # padding past the filter
             ((3, 9, 9, 24, 9, 9, 1, 1, 0), "bf16")]      # no padding
    for shape, fmt in cases:
        x, dy = bwf_inputs(shape, fmt, 75)
        for off in (0, 1):
            dwv, desc = run_bwf(x, dy, shape, fmt, ws_offset=off)
            say(f"[gpu] bwd filter {fmt} {shape} ws+{4 * off}B ({desc[:40]})")
            if off == 0:
                assert desc.startswith("bwf mfma"), desc
            check_bwf(dwv, x, dy, shape, fmt, f"bwf {shape} ws+{off}")


def test_bwd_filter_mfma_tall_image_chunks():
    """A single tall image split into many row chunks (a batch of one gives
    too few workgroups otherwise): the chunk sums of one image are merged
    like those of separate images."""
    shape, fmt = (1, 1100, 6, 8, 3, 3, 1, 1, 1), "bf16"
    x, dy = bwf_inputs(shape, fmt, 76)
    dwv, desc = run_bwf(x, dy, shape, fmt)
    say(f"[gpu] bwd filter tall ({desc})")
    assert "Z=23" in desc, desc
    check_bwf(dwv, x, dy, shape, fmt, "bwf tall")


def test_bwd_filter_column_stream(monkeypatch):
    """The fp32 3x3 column stream: ragged strips in both directions, one
    channel vector (256 strips per workgroup), 12 vectors (21 strips, a tree
    over a count that is not a power of two), 65 vectors (two channel
    groups), padding past the filter; the same shapes through the vector
    pass 1 it replaces (the bwf_nocs tuning choice) also match the oracle."""
    cases = [(3, 17, 23, 4, 3, 3, 1, 1, 1), (2, 29, 30, 48, 3, 3, 1, 1, 1),
             (1, 15, 9, 260, 3, 3, 1, 1, 0), (2, 12, 13, 16, 3, 3, 1, 1, 2)]
    for shape in cases:
        x, dy = bwf_inputs(shape, "f32", 77)
        dwv, desc = run_bwf(x, dy, shape, "f32")
        say(f"[gpu] bwd filter colstream {shape} ({desc[:40]})")
        assert desc.startswith("bwf colstream"), desc
        check_bwf(dwv, x, dy, shape, "f32", f"bwf cs {shape}")
    monkeypatch.setenv("DWCONV_TUNE", "bwf_nocs=1")
    for shape in cases:
        x, dy = bwf_inputs(shape, "f32", 77)
        dwv, desc = run_bwf(x, dy, shape, "f32")
        assert desc.startswith("bwf:"), desc
        check_bwf(dwv, x, dy, shape, "f32", f"bwf vec {shape}")


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
def test_module_wrapper_all_passes(fmt):
    """DepthwiseConv2d (the Python wrapper over one plan) runs the forward
    pass, the fused prologue, the input gradient and the filter gradient,
    each against the oracle."""
    shape = (2, 14, 19, 16, 5, 5, 1, 1, 2)
    N, H, W, C, FH, FW, S, D, P = shape
    rng = np.random.default_rng({"f32": 71, "bf16": 72}[fmt])
    x = synth.to_storage(rng.standard_normal((N, H, W, C)), fmt)
    w = synth.to_storage(rng.normal(0.0, 0.2, (FH, FW, C)), fmt)
    b = synth.to_storage(rng.uniform(-0.1, 0.1, C), "f32")
    s = rng.uniform(0.5, 1.5, C).astype(np.float32)
    t = rng.normal(0.0, 0.5, C).astype(np.float32)
    conv = dw.DepthwiseConv2d(*shape, dtype=fmt)
    try:
        xd, wd, bd = to_dev(x, fmt), to_dev(w, fmt), to_dev(b, "f32")
        y = conv(xd, wd, bd)
        y2 = conv.forward_bn_act(xd, wd, torch.from_numpy(s).to(DEV),
                                 torch.from_numpy(t).to(DEV), act="relu6", bias=bd)
        dy, _ = grads(shape, fmt, 73)
        dyd = to_dev(dy, fmt)
        dx = conv.backward_data(dyd, wd)
        dW = conv.backward_filter(xd, dyd)
        torch.cuda.synchronize()
        host = {k: (v.view(torch.int16).cpu().numpy().view(np.uint16) if v.dtype == torch.bfloat16
                    else v.cpu().numpy()) for k, v in dict(y=y, y2=y2, dx=dx).items()}
    finally:
        conv.close()
    ref, scale = oracle.fwd(x, w, b, S, D, P, fmt, threads=8)
    check.assert_float(host["y"], fmt, ref, scale, f"module fwd {fmt}")
    ref, scale = oracle.fwd_bn_act(x, w, b, s, t, "relu6", S, D, P, fmt, threads=8)
    check.assert_float(host["y2"], fmt, ref, scale, f"module fwd_bn_act {fmt}")
    check_bwd(host["dx"], dy, w, shape, fmt, f"module bwd_data {fmt}")
    check_bwf(dW.cpu().numpy(), x, dy, shape, fmt, f"module bwd_filter {fmt}")


def test_one_plan_on_two_streams_at_once():
    """One handle used on two streams concurrently (the forward pass and the
    filter gradient, each stream with its own buffers and workspace): every
    result equals the same call made alone on the default stream."""
    shape = (4, 30, 29, 32, 7, 7, 1, 1, 3)
    N, H, W, C, FH, FW, S, D, P = shape
    rng = np.random.default_rng(91)
    xs = [synth.to_storage(rng.standard_normal((N, H, W, C)), "f16") for _ in range(2)]
    w = synth.to_storage(rng.normal(0.0, 1 / 7, (FH, FW, C)), "f16")
    conv = dw.DepthwiseConv2d(*shape, dtype="f16")
    try:
        xd = [to_dev(x, "f16") for x in xs]
        wd = to_dev(w, "f16")
        ref_y = [conv(x, wd) for x in xd]
        ref_dw = [conv.backward_filter(x, y) for x, y in zip(xd, ref_y)]
        torch.cuda.synchronize()
        streams = [torch.cuda.Stream(), torch.cuda.Stream()]
        out_y, out_dw = [None, None], [None, None]
        for rep in range(3):
            for k, st in enumerate(streams):
                with torch.cuda.stream(st):
                    out_y[k] = conv(xd[k], wd, stream=st)
                    out_dw[k] = conv.backward_filter(xd[k], out_y[k], stream=st)
            torch.cuda.synchronize()
            for k in range(2):
                assert torch.equal(out_y[k].view(torch.int16), ref_y[k].view(torch.int16)), (rep, k)
                assert torch.equal(out_dw[k], ref_dw[k]), (rep, k)
    finally:
        conv.close()


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_paired_tap_backward_data(fmt):
    """The fp16 / bf16 5x5 column stream with paired taps reading the filter rotated
    (backward data at stride 1), against the oracle's scatter form."""
    rng = np.random.default_rng(97)
    for shape in [(2, 23, 37, 16, 5, 5, 1, 1, 2), (1, 31, 20, 6, 5, 5, 1, 1, 4)]:
        N, H, W, C, FH, FW, S, D, P = shape
        OH = (H + 2 * P - (FH - 1) * D - 1) // S + 1
        OW = (W + 2 * P - (FW - 1) * D - 1) // S + 1
        dy = synth.to_storage(rng.normal(0.0, 1.0, (N, OH, OW, C)), fmt)
        w = synth.to_storage(rng.normal(0.0, 1 / 25, (FH, FW, C)), fmt)
        say(f"[gpu] bwd data paired taps {shape}")
        dx, desc = run_bwd(dy, w, shape, fmt, "rowwin")
        assert desc.startswith("colstream: VEC=2"), desc
        check_bwd(dx, dy, w, shape, fmt, f"bwd dot2 {fmt} {shape}")
