"""Pins for the CPU oracle: what the pages and the mathematics fix, checked
against the oracle without reference to the HIP path.

* worked numbers the pages print (tests/golden/*.json, each with its source);
* the output-extent formula against the halo-span formula;
* brute force on tiny inputs against two independent formulations -- a NumPy
  im2col-then-GEMV per channel (the formulation of "Flash-DWC", section 2.1)
  and torch's CPU conv2d with groups=C in float64 (a library special case) --
  and the textbook single-channel case against scipy's correlate2d;
* closed forms: all-ones box counts, shifted-delta filters, linearity,
  separability, channel permutation, bias added once, sum|x*w|;
* the int8 path against the float path on the same integers, and extremes.

``test_mutants_are_caught`` re-runs these pins against broken copies of the
oracle source to show that each plausible mistake fails at least one pin.
"""
import json
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch
from scipy.signal import correlate2d

import oracle
from oracle import forms
from synth import WORKLOADS

HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------------------
# worked numbers printed on the pages
# ----------------------------------------------------------------------------

def test_golden_halo_span(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "tiling_budget.json")))
    for case in g["halo_span"]:
        assert forms.halo_span(case["t"], case["s"], case["r"], case["d"]) == case["span"]


def test_golden_storage_budget(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "tiling_budget.json")))
    for case in g["storage"]:
        total = forms.tile_storage_bytes(case["th"], case["tw"], case["tc"], case["tm"],
                                         case["r"], in_bytes=1, w_bytes=1, acc_bytes=4,
                                         bias_bytes=4, double_buffer=case["double_buffer"])
        assert total == case["total"]
        if "exceeds_budget" in case:
            assert (total > g["budget"]) == case["exceeds_budget"]
    # the itemised single-buffer budget: 32 input, 36 weight, 32 partial, 8 bias
    c = g["storage"][0]
    span = forms.halo_span(c["th"], 1, c["r"], 1)
    assert span * span * c["tc"] == c["input"]
    assert c["tm"] * c["tc"] * c["r"] ** 2 == c["weights"]
    assert c["th"] * c["tw"] * c["tm"] * 4 == c["partials"]
    assert c["tm"] * 4 == c["bias"]
    # the same method on a depthwise tile of that shape: 32 + 18 + 32 + 8
    assert forms.tile_storage_bytes(2, 2, 2, 2, 3, depthwise=True) == 90


def test_golden_ragged_mask(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "tiling_budget.json")))["ragged"]
    assert forms.ragged_tiles(g["m"], g["tm"]) == (g["tiles"], g["last_valid"])


def test_golden_gemm_traffic(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "gemm_traffic.json")))
    m, k, n, b = g["m"], g["k"], g["n"], g["b"]
    assert forms.gemm_qmin(m, k, n, b) == g["qmin"]
    for t, q in g["qtile"].items():
        assert forms.gemm_qtile(m, k, n, b, int(t)) == q
    # the page's own snippet expands Q_tile at t = 1 by hand; both agree
    assert (m * k * n + k * n * m + m * n) * b == forms.gemm_qtile(m, k, n, b, 1)
    # larger blocks never add traffic, and one block covering C reaches Q_min
    for t in range(1, 9):
        assert forms.gemm_qtile(8, 5, 8, 4, t) >= forms.gemm_qtile(8, 5, 8, 4, t + 1)
    assert forms.gemm_qtile(8, 5, 8, 4, 8) == forms.gemm_qmin(8, 5, 8, 4)


def test_toeplitz_density():
    # "Flash-DWC", section 4.2: 16 GEMVs x 8 outputs x 9 taps in an m16n8k16
    # product fill 2304 of 4096 slots = 56.25 %
    assert forms.toeplitz_density(8, 9) == 9 / 16
    assert 16 * 8 * 9 / (16 * 8 * 16) == forms.toeplitz_density(8, 9)


# ----------------------------------------------------------------------------
# output extent
# ----------------------------------------------------------------------------

def test_dwc_flops_filter_growth():
    """Flash-DWC, section 6.1 (CUDA-core evaluation, small filters): going from
    a 3x3 to a 7x7 filter raises the FLOP count about 5.44-fold."""
    for n, oh, ow, c in [(1, 7, 9, 3), (128, 64, 64, 256)]:
        r = forms.dwc_flops(n, oh, ow, c, 7, 7) / forms.dwc_flops(n, oh, ow, c, 3, 3)
        assert round(r, 2) == 5.44


def _count_macs_and_elements(n, ih, iw, c, fh, fw, s, d, p):
    """Brute force: every (n, oh, ow, c, fh, fw) visit of the loop nest that
    defines the operation, and the set of distinct input and weight elements
    those visits name (padding positions name no element)."""
    oh_n, ow_n = oracle.out_dim(ih, fh, s, d, p), oracle.out_dim(iw, fw, s, d, p)
    macs = 0
    xs, ws = set(), set()
    for b in range(n):
        for oh in range(oh_n):
            for ow in range(ow_n):
                for ch in range(c):
                    for i in range(fh):
                        for j in range(fw):
                            macs += 1
                            ws.add((i, j, ch))
                            y, x = oh * s - p + i * d, ow * s - p + j * d
                            if 0 <= y < ih and 0 <= x < iw:
                                xs.add((b, y, x, ch))
    return macs, oh_n, ow_n, xs, ws


def test_dwc_flops_and_intensity_brute_force():
    """Flash-DWC, section 2.2: the FLOP count is two per multiply-add of the
    loop nest (the bias add is not counted), and the intensity bound divides
    it by the elements read once -- every input element and every weight.
    Brute force on shapes whose every input element is read (no stride gaps),
    so the distinct-element counts equal N*IH*IW*C and C*FH*FW."""
    for shape in [(1, 5, 6, 2, 3, 3, 1, 1, 1), (2, 4, 7, 3, 2, 3, 1, 1, 0),
                  (1, 6, 6, 1, 5, 5, 1, 1, 2), (2, 5, 5, 2, 3, 3, 1, 2, 2)]:
        n, ih, iw, c, fh, fw, s, d, p = shape
        macs, oh, ow, xs, ws = _count_macs_and_elements(*shape)
        assert len(xs) == n * ih * iw * c and len(ws) == c * fh * fw
        assert forms.dwc_flops(n, oh, ow, c, fh, fw) == 2 * macs
        assert forms.dwc_intensity_bound(n, ih, iw, c, oh, ow, fh, fw) == \
            pytest.approx(2 * macs / (len(xs) + len(ws)), rel=1e-15)


def test_dwc_intensity_vs_standard_convolution():
    """Flash-DWC, section 2.2: a standard convolution with IC input channels
    does IC times the work on the same input and IC times the weights, so its
    bound is etaS = IC * flops / (N*IH*IW*IC + OC*FH*FW*IC); for large batch
    and resolution etaD -> etaS / IC."""
    ih = iw = 56
    c, f = 128, 3
    prev = None
    for n in [1, 8, 64, 512, 4096]:
        eta_d = forms.dwc_intensity_bound(n, ih, iw, c, ih, iw, f, f)
        flops_std = c * forms.dwc_flops(n, ih, iw, c, f, f)   # every output sums IC channels
        eta_s = flops_std / (n * ih * iw * c + c * f * f * c)
        gap = abs(eta_d * c / eta_s - 1)
        assert prev is None or gap < prev
        prev = gap
    assert prev < 1e-3
    # and etaD stays near 2*FH*FW (= 18) for a 3x3 'same' layer, orders of
    # magnitude below etaS (section 2.2: low reuse per input element)
    assert 17 < forms.dwc_intensity_bound(64, 56, 56, 128, 56, 56, 3, 3) < 18
    assert eta_s > 100 * eta_d


def test_out_dim_is_span_inverse():
    for size in range(1, 30):
        for f in range(1, 8):
            for s in range(1, 4):
                for d in range(1, 4):
                    for p in range(0, 6):
                        o = oracle.out_dim(size, f, s, d, p)
                        assert o == forms.out_extent(size, f, s, d, p)
                        if o:
                            assert forms.halo_span(o, s, f, d) <= size + 2 * p
                            assert forms.halo_span(o + 1, s, f, d) > size + 2 * p


def test_workload_output_sizes():
    # the tiny workload's stated output is 1x16x16x8; the others are 56x56
    want = {"tiny_f32_3x3": 16, "mobilenet_f32_3x3": 56, "convnext_f16_7x7": 56,
            "largekernel_bf16_31x31": 56, "strided_i8_5x5": 56}
    for name, wl in WORKLOADS.items():
        assert oracle.out_dim(wl.H, wl.FH, wl.stride, wl.dilation, wl.pad) == want[name]
        assert oracle.out_dim(wl.W, wl.FW, wl.stride, wl.dilation, wl.pad) == want[name]
    assert oracle.out_dim(3, 5, 1, 1, 0) == 0       # filter wider than the input
    assert oracle.out_dim(3, 5, 1, 1, 1) == 1


# ----------------------------------------------------------------------------
# brute force against independent formulations
# ----------------------------------------------------------------------------

def im2col_gemv(x, w, bias, S, D, P):
    """Per channel: gather every output's FH*FW patch into a matrix (zero
    padded), then multiply by that channel's flattened filter."""
    N, H, W, C = x.shape
    FH, FW, _ = w.shape
    OH = (H + 2 * P - D * (FH - 1) - 1) // S + 1
    OW = (W + 2 * P - D * (FW - 1) - 1) // S + 1
    xp = np.zeros((N, H + 2 * P, W + 2 * P, C), np.float64)
    xp[:, P:P + H, P:P + W, :] = x
    cols = np.empty((N, OH, OW, FH * FW, C), np.float64)
    for fh in range(FH):
        for fw in range(FW):
            rows = fh * D + S * np.arange(OH)
            cc = fw * D + S * np.arange(OW)
            cols[:, :, :, fh * FW + fw, :] = xp[:, rows][:, :, cc]
    y = np.einsum("nhwkc,kc->nhwc", cols, w.reshape(FH * FW, C))
    if bias is not None:
        y = y + bias
    return y


def torch_ref(x, w, bias, S, D, P):
    C = x.shape[3]
    xt = torch.from_numpy(np.ascontiguousarray(x.transpose(0, 3, 1, 2))).double()
    wt = torch.from_numpy(np.ascontiguousarray(w.transpose(2, 0, 1))).double().unsqueeze(1)
    bt = None if bias is None else torch.from_numpy(np.asarray(bias, np.float64))
    y = torch.nn.functional.conv2d(xt, wt, bt, stride=S, padding=P, dilation=D, groups=C)
    return y.numpy().transpose(0, 2, 3, 1)


def _int_valued_case(rng):
    while True:
        FH, FW = rng.integers(1, 5, size=2)
        S, D = rng.integers(1, 4, size=2)
        P = int(rng.integers(0, 2 * max(FH, FW) + 1))
        H, W = rng.integers(1, 8, size=2)
        if (H + 2 * P - D * (FH - 1) - 1) >= 0 and (W + 2 * P - D * (FW - 1) - 1) >= 0:
            break
    N = int(rng.integers(1, 3))
    C = int(rng.integers(1, 6))
    x = rng.integers(-8, 9, size=(N, H, W, C)).astype(np.float32)
    w = rng.integers(-8, 9, size=(FH, FW, C)).astype(np.float32)
    b = rng.integers(-50, 51, size=C).astype(np.float32) if rng.integers(0, 2) else None
    return x, w, b, int(S), int(D), P


def run_brute_force(lib=None, cases=150, seed=123):
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        x, w, b, S, D, P = _int_valued_case(rng)
        y, scale = oracle.fwd(x, w, b, S, D, P, "f32", lib=lib)
        ref = im2col_gemv(x.astype(np.float64), w.astype(np.float64),
                          None if b is None else b.astype(np.float64), S, D, P)
        assert y.shape == ref.shape
        np.testing.assert_array_equal(y, ref)             # integer data: exact
        np.testing.assert_array_equal(y, torch_ref(x, w, b, S, D, P))
        # sum |x*w| is the same convolution on |x|, |w| without bias
        sref = im2col_gemv(np.abs(x.astype(np.float64)), np.abs(w.astype(np.float64)),
                           None, S, D, P)
        np.testing.assert_array_equal(scale, sref)


def test_brute_force_tiny():
    run_brute_force()


def test_brute_force_real_valued():
    # non-integer data: three formulations agree to fp64 rounding
    rng = np.random.default_rng(7)
    for _ in range(30):
        x, w, b, S, D, P = _int_valued_case(rng)
        x = rng.standard_normal(x.shape).astype(np.float32)
        w = rng.standard_normal(w.shape).astype(np.float32)
        y, _ = oracle.fwd(x, w, b, S, D, P, "f32")
        np.testing.assert_allclose(y, im2col_gemv(x.astype(np.float64), w.astype(np.float64),
                                                  None if b is None else b.astype(np.float64),
                                                  S, D, P), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(y, torch_ref(x, w, b, S, D, P), rtol=1e-12, atol=1e-12)


def run_textbook(lib=None):
    # "Outline of Programming Massively Parallel Processors ...", section
    # "2D Convolution": one channel, odd filter of radius r, unit stride, zero
    # ghost cells, output the size of the input -> scipy's correlate2d 'same'
    rng = np.random.default_rng(5)
    for r in range(0, 4):
        for (h, w_) in [(1, 1), (5, 9), (12, 7)]:
            x = rng.standard_normal((h, w_))
            f = rng.standard_normal((2 * r + 1, 2 * r + 1))
            y, _ = oracle.fwd(x.reshape(1, h, w_, 1).astype(np.float32),
                              f.reshape(2 * r + 1, 2 * r + 1, 1).astype(np.float32),
                              None, 1, 1, r, "f32", lib=lib)
            ref = correlate2d(x.astype(np.float32).astype(np.float64),
                              f.astype(np.float32).astype(np.float64),
                              mode="same", boundary="fill", fillvalue=0)
            np.testing.assert_allclose(y[0, :, :, 0], ref, rtol=1e-12, atol=1e-12)


def test_textbook_single_channel():
    run_textbook()


# ----------------------------------------------------------------------------
# closed forms and invariants
# ----------------------------------------------------------------------------

def _count(o, S, P, D, F, size):
    return sum(1 for f in range(F) if 0 <= o * S - P + f * D < size)


def run_box(lib=None):
    # X = 1, W = 1, no bias: each output counts the taps inside the image
    for (N, H, W, C, FH, FW, S, D, P) in [(1, 16, 16, 8, 3, 3, 1, 1, 1),
                                          (2, 9, 13, 3, 5, 4, 2, 2, 4),
                                          (1, 7, 7, 2, 7, 7, 1, 1, 3),
                                          (1, 31, 20, 1, 31, 31, 1, 1, 15),
                                          (1, 6, 5, 2, 3, 2, 3, 1, 5)]:
        x = np.ones((N, H, W, C), np.float32)
        w = np.ones((FH, FW, C), np.float32)
        y, _ = oracle.fwd(x, w, None, S, D, P, "f32", lib=lib)
        OH, OW = y.shape[1:3]
        for oh in range(OH):
            for ow in range(OW):
                want = _count(oh, S, P, D, FH, H) * _count(ow, S, P, D, FW, W)
                assert np.all(y[:, oh, ow, :] == want), (oh, ow)


def test_box_counts():
    run_box()


def run_delta(lib=None):
    # a filter with a single 1 at (a, b) copies the input shifted by the tap
    rng = np.random.default_rng(11)
    for (N, H, W, C, FH, FW, S, D, P) in [(2, 9, 8, 3, 3, 3, 1, 1, 1),
                                          (1, 14, 11, 2, 5, 3, 2, 2, 4),
                                          (1, 10, 10, 4, 4, 2, 3, 1, 0)]:
        x = rng.standard_normal((N, H, W, C)).astype(np.float32)
        for a in range(FH):
            for b in range(FW):
                w = np.zeros((FH, FW, C), np.float32)
                w[a, b, :] = 1
                y, _ = oracle.fwd(x, w, None, S, D, P, "f32", lib=lib)
                OH, OW = y.shape[1:3]
                for oh in range(OH):
                    ih = oh * S - P + a * D
                    for ow in range(OW):
                        iw = ow * S - P + b * D
                        want = x[:, ih, iw, :] if (0 <= ih < H and 0 <= iw < W) else 0
                        assert np.array_equal(y[:, oh, ow, :], np.broadcast_to(
                            np.asarray(want, np.float64), (N, C))), (a, b, oh, ow)
    # the centred delta with unit stride and same padding is the identity
    x = rng.standard_normal((2, 7, 9, 5)).astype(np.float32)
    w = np.zeros((5, 5, 5), np.float32)
    w[2, 2, :] = 1
    y, _ = oracle.fwd(x, w, None, 1, 1, 2, "f32", lib=lib)
    assert np.array_equal(y, x.astype(np.float64))


def test_delta_filters():
    run_delta()


def run_bias_once(lib=None):
    rng = np.random.default_rng(3)
    x = rng.integers(-5, 6, size=(2, 6, 7, 4)).astype(np.float32)
    w = rng.integers(-5, 6, size=(3, 3, 4)).astype(np.float32)
    b = np.array([1.5, -2.25, 1000.0, 0.0], np.float32)
    y0, _ = oracle.fwd(x, w, None, 1, 1, 1, "f32", lib=lib)
    y1, _ = oracle.fwd(x, w, b, 1, 1, 1, "f32", lib=lib)
    assert np.array_equal(y1 - y0, np.broadcast_to(b.astype(np.float64), y0.shape))
    # a zero filter leaves exactly the bias
    yb, _ = oracle.fwd(x, np.zeros_like(w), b, 1, 1, 1, "f32", lib=lib)
    assert np.array_equal(yb, np.broadcast_to(b.astype(np.float64), yb.shape))


def test_bias_added_once():
    run_bias_once()


def test_linearity():
    rng = np.random.default_rng(4)
    for S, D, P in [(1, 1, 1), (2, 2, 3), (3, 1, 0)]:
        x1 = rng.integers(-9, 10, size=(2, 8, 9, 3)).astype(np.float32)
        x2 = rng.integers(-9, 10, size=(2, 8, 9, 3)).astype(np.float32)
        w1 = rng.integers(-9, 10, size=(3, 4, 3)).astype(np.float32)
        w2 = rng.integers(-9, 10, size=(3, 4, 3)).astype(np.float32)
        f = lambda x, w: oracle.fwd(x, w, None, S, D, P, "f32")[0]
        assert np.array_equal(f(3 * x1 - 2 * x2, w1), 3 * f(x1, w1) - 2 * f(x2, w1))
        assert np.array_equal(f(x1, 2 * w1 + 5 * w2), 2 * f(x1, w1) + 5 * f(x1, w2))


def test_separable_filter():
    # "Flash-DWC", section 3.3: a 2-D filter is a stack of FH 1-D rows.  For
    # W = u (x) v the result is a 1-D correlation along width with v, then
    # along height with u.
    rng = np.random.default_rng(6)
    N, H, W, C, F = 2, 9, 10, 3, 3
    x = rng.integers(-9, 10, size=(N, H, W, C)).astype(np.float32)
    u = rng.integers(-4, 5, size=(F, C)).astype(np.float32)
    v = rng.integers(-4, 5, size=(F, C)).astype(np.float32)
    w = u[:, None, :] * v[None, :, :]
    y, _ = oracle.fwd(x, w, None, 1, 1, 1, "f32")
    xp = np.pad(x.astype(np.float64), ((0, 0), (1, 1), (1, 1), (0, 0)))
    t = sum(xp[:, :, j:j + W, :] * v[j] for j in range(F))      # along width
    ref = sum(t[:, i:i + H, :, :] * u[i] for i in range(F))     # then height
    assert np.array_equal(y, ref)


def test_channel_permutation():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((2, 6, 7, 6)).astype(np.float32)
    w = rng.standard_normal((3, 5, 6)).astype(np.float32)
    b = rng.standard_normal(6).astype(np.float32)
    perm = rng.permutation(6)
    y, _ = oracle.fwd(x, w, b, 2, 1, 2, "f32")
    yp, _ = oracle.fwd(x[..., perm], w[..., perm], b[perm], 2, 1, 2, "f32")
    assert np.array_equal(yp, y[..., perm])


def test_int8_matches_float_path():
    rng = np.random.default_rng(9)
    for _ in range(20):
        x, w, b, S, D, P = _int_valued_case(rng)
        xi = rng.integers(-128, 128, size=x.shape).astype(np.int8)
        wi = rng.integers(-128, 128, size=w.shape).astype(np.int8)
        bi = rng.integers(-2**15, 2**15 + 1, size=x.shape[3]).astype(np.int32)
        yi, _ = oracle.fwd(xi, wi, bi, S, D, P, "i8")
        yf, _ = oracle.fwd(xi.astype(np.float32), wi.astype(np.float32),
                           bi.astype(np.float32), S, D, P, "f32")
        assert np.array_equal(yi, yf.astype(np.int64))


def test_int8_extremes():
    # every tap -128 * -128, plus the largest bias: 25 * 16384 + 32768
    x = np.full((1, 5, 5, 3), -128, np.int8)
    w = np.full((5, 5, 3), -128, np.int8)
    b = np.full(3, 2**15, np.int32)
    y, _ = oracle.fwd(x, w, b, 1, 1, 0, "i8")
    assert y.shape == (1, 1, 1, 3) and np.all(y == 25 * 16384 + 32768)
    w[:] = 127
    y, _ = oracle.fwd(x, w, -b, 1, 1, 0, "i8")
    assert np.all(y == -25 * 128 * 127 - 32768)


def test_points_match_full_pass():
    rng = np.random.default_rng(10)
    for dtype in ("f32", "i8"):
        x, w, b, S, D, P = _int_valued_case(rng)
        if dtype == "i8":
            x, w, b = x.astype(np.int8), w.astype(np.int8), None
        y, s = oracle.fwd(x, w, b, S, D, P, dtype)
        idx = rng.integers(0, y.size, size=50)
        yp, sp = oracle.points(x, w, b, S, D, P, dtype, idx)
        assert np.array_equal(yp, y.ravel()[idx])
        if s is not None:
            assert np.array_equal(sp, s.ravel()[idx])


def test_threaded_split_is_identical():
    wl = WORKLOADS["tiny_f32_3x3"]
    rng = np.random.default_rng(12)
    x = rng.standard_normal((5, 9, 8, 3)).astype(np.float32)
    w = rng.standard_normal((3, 3, 3)).astype(np.float32)
    y1, s1 = oracle.fwd(x, w, None, 1, 1, 1, "f32", threads=1)
    y3, s3 = oracle.fwd(x, w, None, 1, 1, 1, "f32", threads=3)
    assert np.array_equal(y1, y3) and np.array_equal(s1, s3)
    assert wl.N == 1


def test_rejects_bad_shapes():
    x = np.zeros((1, 3, 3, 2), np.float32)
    with pytest.raises(ValueError):
        oracle.fwd(x, np.zeros((5, 5, 2), np.float32), None, 1, 1, 0, "f32")
    with pytest.raises(ValueError):
        oracle.fwd(x, np.zeros((3, 3, 3), np.float32), None, 1, 1, 0, "f32")
    with pytest.raises(ValueError):
        oracle.fwd(x, np.zeros((3, 3, 2), np.float32), None, 1, 1, 0, "f64")


# ----------------------------------------------------------------------------
# mutation check: plausible mistakes planted in a copy of the oracle (on the
# CPU) must each fail at least one pin
# ----------------------------------------------------------------------------

MUTANTS = {
    "pad_sign": ("int ih = oh * S - P + fh * D;", "int ih = oh * S + P + fh * D;"),
    "no_width_dilation": ("int iw = ow * S - P + fw * D;", "int iw = ow * S - P + fw;"),
    "no_height_stride": ("int ih = oh * S - P + fh * D;", "int ih = oh - P + fh * D;"),
    "flipped_filter": ("double wv = w[((long long)fh * FW + fw) * C + c];",
                       "double wv = w[((long long)(FH - 1 - fh) * FW + (FW - 1 - fw)) * C + c];"),
    "dropped_bias": ("double acc = bias ? bias[c] : 0.0;", "double acc = 0.0;"),
    "swapped_hw": ("double xv = x[((n * H + ih) * (long long)W + iw) * C + c];",
                   "double xv = x[((n * W + iw) * (long long)H + ih) * C + c];"),
    "out_dim_off_by_one": ("long long o = room / s + 1;", "long long o = room / s;"),
    "scale_signed": ("sabs += fabs(prod);", "sabs += prod;"),
}


def _pins(lib):
    failed = []
    for name, fn in [("brute", lambda: run_brute_force(lib, cases=60)),
                     ("textbook", lambda: run_textbook(lib)),
                     ("box", lambda: run_box(lib)),
                     ("delta", lambda: run_delta(lib)),
                     ("bias", lambda: run_bias_once(lib))]:
        try:
            fn()
        except (AssertionError, ValueError):
            failed.append(name)
    return failed


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_mutants_are_caught(tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "dwref.c")).read()
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) >= 1, name
        path = tmp_path / f"{name}.c"
        path.write_text(src.replace(old, new, 1))   # first hit: the float path
        so = tmp_path / f"lib{name}.so"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", str(path),
                               "-o", str(so), "-lm"])
        failed = _pins(oracle.bind(str(so)))
        assert failed, f"mutant {name} passed every pin"
    # and the unmutated source passes them all
    assert _pins(oracle._load()) == []
