"""Pins of the oracle's backward passes (CPU): backward data, then backward filter.

The oracle writes the input gradient as the plain scatter over the forward's
taps ("Flash-DWC: Making Depthwise Convolution Compute-Efficient on GPUs",
section 5.1).  It is pinned here against things that do not share that code:

* the adjoint identity <fwd(x), dy> = <x, bwd(dy)>, exact on small integers,
  for any stride, dilation, padding and non-square filters;
* torch's CPU autograd of conv2d(groups=C) in float64 (a library routine);
* for stride 1, the page's own reading: a forward convolution of dy with the
  filter rotated by 180 degrees and padding D(F-1) - P;
* sum |dy*w| = bwd(|dy|, |w|);
* plausible mistakes planted in a copy of the backward function must each
  fail one of the above.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle


def _case(rng, max_hw=11, max_c=4, max_f=5):
    while True:
        FH, FW = int(rng.integers(1, max_f + 1)), int(rng.integers(1, max_f + 1))
        S, D = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        P = int(rng.integers(0, max(FH, FW) * D // 2 + 2))
        H, W = int(rng.integers(1, max_hw + 1)), int(rng.integers(1, max_hw + 1))
        N, C = int(rng.integers(1, 3)), int(rng.integers(1, max_c + 1))
        if oracle.out_dim(H, FH, S, D, P) > 0 and oracle.out_dim(W, FW, S, D, P) > 0:
            return (N, H, W, C, FH, FW, S, D, P)


def run_adjoint(lib, cases=80, seed=1):
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        shape = _case(rng)
        N, H, W, C, FH, FW, S, D, P = shape
        OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
        x = rng.integers(-8, 9, size=(N, H, W, C)).astype(np.float32)
        w = rng.integers(-8, 9, size=(FH, FW, C)).astype(np.float32)
        dy = rng.integers(-8, 9, size=(N, OH, OW, C)).astype(np.float32)
        y, _ = oracle.fwd(x, w, None, S, D, P, "f32", lib=lib)
        dx, _ = oracle.bwd_data(dy, w, shape, "f32", lib=lib)
        lhs = float(np.sum(y * dy.astype(np.float64)))
        rhs = float(np.sum(x.astype(np.float64) * dx))
        assert lhs == rhs, (shape, lhs, rhs)


def run_torch(lib, cases=40, seed=2):
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        shape = _case(rng)
        N, H, W, C, FH, FW, S, D, P = shape
        OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
        x = torch.zeros((N, C, H, W), dtype=torch.float64, requires_grad=True)
        w = rng.standard_normal((FH, FW, C)).astype(np.float32)
        dy = rng.standard_normal((N, OH, OW, C)).astype(np.float32)
        wt = torch.from_numpy(w.astype(np.float64)).permute(2, 0, 1).unsqueeze(1).contiguous()
        y = torch.nn.functional.conv2d(x, wt, stride=S, padding=P, dilation=D, groups=C)
        y.backward(torch.from_numpy(dy.astype(np.float64)).permute(0, 3, 1, 2))
        ref = x.grad.permute(0, 2, 3, 1).numpy()
        dx, _ = oracle.bwd_data(dy, w, shape, "f32", lib=lib)
        np.testing.assert_allclose(dx, ref, rtol=1e-12, atol=1e-12)


def run_rotated(lib, cases=40, seed=3):
    rng = np.random.default_rng(seed)
    done = 0
    while done < cases:
        shape = _case(rng)
        N, H, W, C, FH, FW, S, D, P = shape
        if S != 1 or FH != FW or D * (FH - 1) < P:
            continue
        OH, OW = oracle.out_dim(H, FH, 1, D, P), oracle.out_dim(W, FW, 1, D, P)
        w = rng.integers(-8, 9, size=(FH, FW, C)).astype(np.float32)
        dy = rng.integers(-8, 9, size=(N, OH, OW, C)).astype(np.float32)
        dx, _ = oracle.bwd_data(dy, w, shape, "f32", lib=lib)
        ref, _ = oracle.fwd(dy, w[::-1, ::-1].copy(), None, 1, D, D * (FH - 1) - P, "f32",
                            lib=lib)
        assert ref.shape == dx.shape and np.array_equal(ref, dx), shape
        done += 1


def run_scale(lib, cases=30, seed=4):
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        shape = _case(rng)
        N, H, W, C, FH, FW, S, D, P = shape
        OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
        w = rng.integers(-8, 9, size=(FH, FW, C)).astype(np.float32)
        dy = rng.integers(-8, 9, size=(N, OH, OW, C)).astype(np.float32)
        _, scale = oracle.bwd_data(dy, w, shape, "f32", lib=lib)
        ref, _ = oracle.bwd_data(np.abs(dy), np.abs(w), shape, "f32", lib=lib)
        assert np.array_equal(scale, ref), shape


def test_adjoint_identity():
    run_adjoint(None)


def test_matches_torch_autograd():
    run_torch(None)


def test_stride_one_is_rotated_forward():
    run_rotated(None)


def test_scale_is_abs_pass():
    run_scale(None)


def test_fp16_bf16_inputs_are_decoded_exactly():
    rng = np.random.default_rng(5)
    shape = (1, 7, 6, 3, 3, 3, 1, 1, 1)
    w = rng.standard_normal((3, 3, 3)).astype(np.float16)
    dy = rng.standard_normal((1, 7, 6, 3)).astype(np.float16)
    a, _ = oracle.bwd_data(dy, w, shape, "f16")
    b, _ = oracle.bwd_data(dy.astype(np.float32), w.astype(np.float32), shape, "f32")
    assert np.array_equal(a, b)


def test_rejects_int8_and_bad_shapes():
    with pytest.raises(ValueError):
        oracle.bwd_data(np.zeros((1, 3, 3, 2), np.int8), np.zeros((3, 3, 2), np.int8),
                        (1, 3, 3, 2, 3, 3, 1, 1, 1), "i8")
    with pytest.raises(ValueError):
        oracle.bwd_data(np.zeros((1, 4, 3, 2), np.float32), np.zeros((3, 3, 2), np.float32),
                        (1, 3, 3, 2, 3, 3, 1, 1, 1), "f32")


# Plausible mistakes in the backward function only (the forward is pinned on
# its own); each must fail at least one pin.  Every mutant stays in bounds.
BWD_MUTANTS = {
    "pad_sign": ("int ih = oh * S - P + fh * D;", "int ih = oh * S + P + fh * D;"),
    "no_width_dilation": ("int iw = ow * S - P + fw * D;", "int iw = ow * S - P + fw;"),
    "no_height_stride": ("int ih = oh * S - P + fh * D;", "int ih = oh - P + fh * D;"),
    "flipped_filter": ("double prod = g * w[((long long)fh * FW + fw) * C + c];",
                       "double prod = g * w[((long long)(FH - 1 - fh) * FW + (FW - 1 - fw)) * C + c];"),
    "dy_transposed": ("double g = dy[((n * OH + oh) * (long long)OW + ow) * C + c];",
                      "double g = dy[((n * OW + ow) * (long long)OH + oh) * C + c];"),
    "scale_signed": ("if (scale) scale[i] += fabs(prod);", "if (scale) scale[i] += prod;"),
}


def _bwd_pins(lib):
    failed = []
    for name, fn in [("adjoint", lambda: run_adjoint(lib, cases=40)),
                     ("torch", lambda: run_torch(lib, cases=20)),
                     ("rotated", lambda: run_rotated(lib, cases=20)),
                     ("scale", lambda: run_scale(lib, cases=15))]:
        try:
            fn()
        except (AssertionError, ValueError):
            failed.append(name)
    return failed


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_bwd_mutants_are_caught(tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "dwref.c")).read()
    head, tail = src.split("int dwref_bwd_data_f64(", 1)
    body, rest = tail.split("\n/* Backward filter", 1)   # this function only
    for name, (old, new) in BWD_MUTANTS.items():
        assert body.count(old) == 1, name
        path = tmp_path / f"bwd_{name}.c"
        path.write_text(head + "int dwref_bwd_data_f64(" + body.replace(old, new, 1) +
                        "\n/* Backward filter" + rest)
        so = tmp_path / f"libbwd_{name}.so"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", str(path),
                               "-o", str(so), "-lm"])
        failed = _bwd_pins(oracle.bind(str(so)))
        assert failed, f"mutant {name} passed every pin"
    assert _bwd_pins(oracle._load()) == []


# ---------------------------------------------------------------- backward filter

def run_bilinear(lib, cases=80, seed=11):
    """<conv(x, w), dy> = <w, dW(x, dy)>: the forward pass is linear in w."""
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        shape = _case(rng)
        N, H, W, C, FH, FW, S, D, P = shape
        OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
        x = rng.integers(-8, 9, size=(N, H, W, C)).astype(np.float32)
        w = rng.integers(-8, 9, size=(FH, FW, C)).astype(np.float32)
        dy = rng.integers(-8, 9, size=(N, OH, OW, C)).astype(np.float32)
        y, _ = oracle.fwd(x, w, None, S, D, P, "f32", lib=lib)
        dw, _ = oracle.bwd_filter(x, dy, shape, "f32", lib=lib)
        lhs = float(np.sum(y * dy.astype(np.float64)))
        rhs = float(np.sum(w.astype(np.float64) * dw))
        assert lhs == rhs, (shape, lhs, rhs)


def run_torch_filter(lib, cases=40, seed=12):
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        shape = _case(rng)
        N, H, W, C, FH, FW, S, D, P = shape
        OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
        x = rng.standard_normal((N, H, W, C)).astype(np.float32)
        dy = rng.standard_normal((N, OH, OW, C)).astype(np.float32)
        xt = torch.from_numpy(x.astype(np.float64)).permute(0, 3, 1, 2)
        wt = torch.zeros((C, 1, FH, FW), dtype=torch.float64, requires_grad=True)
        y = torch.nn.functional.conv2d(xt, wt, stride=S, padding=P, dilation=D, groups=C)
        y.backward(torch.from_numpy(dy.astype(np.float64)).permute(0, 3, 1, 2))
        ref = wt.grad[:, 0].permute(1, 2, 0).numpy()
        dw, _ = oracle.bwd_filter(x, dy, shape, "f32", lib=lib)
        np.testing.assert_allclose(dw, ref, rtol=1e-12, atol=1e-12)


def run_box_filter(lib, cases=40, seed=13):
    """x = dy = 1: each tap's gradient counts the outputs whose input for that
    tap lies inside the image, a product of two per-axis counts."""
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        shape = _case(rng)
        N, H, W, C, FH, FW, S, D, P = shape
        OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
        dw, _ = oracle.bwd_filter(np.ones((N, H, W, C), np.float32),
                                  np.ones((N, OH, OW, C), np.float32), shape, "f32", lib=lib)
        rows = [sum(1 for o in range(OH) if 0 <= o * S - P + f * D < H) for f in range(FH)]
        cols = [sum(1 for o in range(OW) if 0 <= o * S - P + f * D < W) for f in range(FW)]
        want = N * np.outer(rows, cols)[:, :, None] * np.ones((1, 1, C))
        assert np.array_equal(dw, want), shape


def run_scale_filter(lib, cases=30, seed=14):
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        shape = _case(rng)
        N, H, W, C, FH, FW, S, D, P = shape
        OH, OW = oracle.out_dim(H, FH, S, D, P), oracle.out_dim(W, FW, S, D, P)
        x = rng.integers(-8, 9, size=(N, H, W, C)).astype(np.float32)
        dy = rng.integers(-8, 9, size=(N, OH, OW, C)).astype(np.float32)
        _, scale = oracle.bwd_filter(x, dy, shape, "f32", lib=lib)
        ref, _ = oracle.bwd_filter(np.abs(x), np.abs(dy), shape, "f32", lib=lib)
        assert np.array_equal(scale, ref), shape


def test_filter_bilinear_identity():
    run_bilinear(None)


def test_filter_matches_torch_autograd():
    run_torch_filter(None)


def test_filter_box_counts():
    run_box_filter(None)


def test_filter_scale_is_abs_pass():
    run_scale_filter(None)


BWF_MUTANTS = {
    "pad_sign": ("int ih = oh * S - P + fh * D;", "int ih = oh * S + P + fh * D;"),
    "no_width_dilation": ("int iw = ow * S - P + fw * D;", "int iw = ow * S - P + fw;"),
    "no_height_stride": ("int ih = oh * S - P + fh * D;", "int ih = oh - P + fh * D;"),
    "tap_transposed": ("long long o = ((long long)fh * FW + fw) * C;",
                       "long long o = ((long long)(FH - 1 - fh) * FW + (FW - 1 - fw)) * C;"),
    "dy_transposed": ("dy + ((n * OH + oh) * (long long)OW + ow) * C;",
                      "dy + ((n * OW + ow) * (long long)OH + oh) * C;"),
    "scale_signed": ("scale[o + c] += fabs(prod);", "scale[o + c] += prod;"),
}


def _bwf_pins(lib):
    failed = []
    for name, fn in [("bilinear", lambda: run_bilinear(lib, cases=40)),
                     ("torch", lambda: run_torch_filter(lib, cases=20)),
                     ("box", lambda: run_box_filter(lib, cases=20)),
                     ("scale", lambda: run_scale_filter(lib, cases=15))]:
        try:
            fn()
        except (AssertionError, ValueError):
            failed.append(name)
    return failed


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_bwd_filter_mutants_are_caught(tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "dwref.c")).read()
    head, tail = src.split("int dwref_bwd_filter_f64(", 1)
    body, rest = tail.split("\n/* Forward pass with the per-channel affine", 1)  # this function
    for name, (old, new) in BWF_MUTANTS.items():
        assert body.count(old) == 1, name
        path = tmp_path / f"bwf_{name}.c"
        path.write_text(head + "int dwref_bwd_filter_f64(" + body.replace(old, new, 1) +
                        "\n/* Forward pass with the per-channel affine" + rest)
        so = tmp_path / f"libbwf_{name}.so"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", str(path),
                               "-o", str(so), "-lm"])
        failed = _bwf_pins(oracle.bind(str(so)))
        assert failed, f"mutant {name} passed every pin"
    assert _bwf_pins(oracle._load()) == []
