"""Pins of the oracle's fused prologue (CPU): act(x * s + b) in front of the
convolution ("Flash-DWC: Making Depthwise Convolution Compute-Efficient on
GPUs", section 5.2, the BN + Act + DWC fusion).

The oracle writes it from the definition; it is pinned here against things
that do not share that code:

* identity affine and no activation: the plain forward pass, exactly;
* no activation: the closed form s*conv(x) + b*conv(ones) + bias (linearity),
  exact on small integers with dyadic s and b;
* ReLU where every pre-activation is >= 0 is the identity, where every one is
  <= 0 it leaves only the bias; ReLU6 below 6 is the identity;
* a saturated ReLU6 (s = 0, b = 10) gives 6 * conv(ones) + bias, which also
  fixes that padding positions are zeros of the activated input, not act(b);
* the error scale does not depend on the activation;
* torch's CPU conv2d(groups=C) on the activated, zero-padded input in float64;
* plausible mistakes planted in a copy of the function must each fail one of
  the above.

fp16 / bf16 data (U stored in the data's format after one fp32 fused
multiply-add, "Flash-DWC" section 4.1's mixed precision):

* through a 1x1 unit filter y is U itself and scale is |x*s + b|: U must be
  numpy's float32 -> float16 conversion / torch's float32 -> bfloat16
  conversion (both round to nearest even) of the activated fp32 value, over
  normal, subnormal, overflowing and exactly-halfway values;
* the fp32 value must be the float32 nearest to the exact x*s + b (ties to
  an even significand), decided with exact rational arithmetic;
* s = 1, b = 0 and no activation give the plain forward pass exactly, and
  with b = 0 any shape equals the plain forward pass of the library-rounded
  U;
* plausible mistakes in the rounding must each fail one of these.
"""
import fractions
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _case(rng, max_hw=10, max_c=4, max_f=5):
    while True:
        FH, FW = int(rng.integers(1, max_f + 1)), int(rng.integers(1, max_f + 1))
        S, D = int(rng.integers(1, 4)), int(rng.integers(1, 3))
        P = int(rng.integers(0, max(FH, FW) * D // 2 + 2))
        H, W = int(rng.integers(1, max_hw + 1)), int(rng.integers(1, max_hw + 1))
        N, C = int(rng.integers(1, 3)), int(rng.integers(1, max_c + 1))
        if oracle.out_dim(H, FH, S, D, P) > 0 and oracle.out_dim(W, FW, S, D, P) > 0:
            return (N, H, W, C, FH, FW, S, D, P)


def _ints(rng, shape, lo=-8, hi=8):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def run_identity(lib, cases=30, seed=21):
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        N, H, W, C, FH, FW, S, D, P = _case(rng)
        x = rng.normal(size=(N, H, W, C)).astype(np.float32)
        w = rng.normal(size=(FH, FW, C)).astype(np.float32)
        b = rng.normal(size=C).astype(np.float32)
        y0, s0 = oracle.fwd(x, w, b, S, D, P, "f32", lib=lib)
        y1, s1 = oracle.fwd_bn_act(x, w, b, np.ones(C), np.zeros(C), "none", S, D, P, "f32",
                                   lib=lib)
        assert np.array_equal(y0, y1) and np.array_equal(s0, s1)


def run_affine(lib, cases=40, seed=22):
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        N, H, W, C, FH, FW, S, D, P = _case(rng)
        x, w = _ints(rng, (N, H, W, C)), _ints(rng, (FH, FW, C))
        bias = _ints(rng, (C,))
        s = rng.choice([-2.0, -1.0, -0.5, 0.5, 1.0, 2.0], size=C).astype(np.float32)
        b = rng.choice([-3.0, -1.5, 0.0, 1.0, 2.5], size=C).astype(np.float32)
        yx, _ = oracle.fwd(x, w, None, S, D, P, "f32", lib=lib)
        y1, _ = oracle.fwd(np.ones_like(x), w, None, S, D, P, "f32", lib=lib)
        want = s.astype(np.float64) * yx + b.astype(np.float64) * y1 + bias
        got, _ = oracle.fwd_bn_act(x, w, bias, s, b, "none", S, D, P, "f32", lib=lib)
        assert np.array_equal(got, want)


def run_relu_regimes(lib, cases=30, seed=23):
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        N, H, W, C, FH, FW, S, D, P = _case(rng)
        w, bias = _ints(rng, (FH, FW, C)), _ints(rng, (C,))
        s = rng.choice([0.25, 0.5, 1.0], size=C).astype(np.float32)
        # every pre-activation in [0, 5]: ReLU and ReLU6 are the identity
        xp = _ints(rng, (N, H, W, C), 0, 4)
        bp = rng.choice([0.0, 0.5, 1.0], size=C).astype(np.float32)
        ref, _ = oracle.fwd_bn_act(xp, w, bias, s, bp, "none", S, D, P, "f32", lib=lib)
        for act in ("relu", "relu6"):
            got, _ = oracle.fwd_bn_act(xp, w, bias, s, bp, act, S, D, P, "f32", lib=lib)
            assert np.array_equal(got, ref), act
        # every pre-activation <= 0: only the bias is left
        xn = _ints(rng, (N, H, W, C), -8, 0)
        bn = rng.choice([-2.0, -0.5, 0.0], size=C).astype(np.float32)
        for act in ("relu", "relu6"):
            got, _ = oracle.fwd_bn_act(xn, w, bias, s, bn, act, S, D, P, "f32", lib=lib)
            assert np.array_equal(got, np.broadcast_to(bias.astype(np.float64), got.shape)), act


def run_saturated(lib, cases=30, seed=24):
    """s = 0, b = 10: the activated input is 10 (ReLU) or 6 (ReLU6) at every
    in-image position and 0 in the padding."""
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        N, H, W, C, FH, FW, S, D, P = _case(rng)
        x, w, bias = _ints(rng, (N, H, W, C)), _ints(rng, (FH, FW, C)), _ints(rng, (C,))
        y1, _ = oracle.fwd(np.ones_like(x), w, None, S, D, P, "f32", lib=lib)
        zero, ten = np.zeros(C, np.float32), np.full(C, 10.0, np.float32)
        for act, level in (("relu", 10.0), ("relu6", 6.0)):
            got, _ = oracle.fwd_bn_act(x, w, bias, zero, ten, act, S, D, P, "f32", lib=lib)
            assert np.array_equal(got, level * y1 + bias), act


def run_scale(lib, cases=20, seed=25):
    """scale = sum |x*s + b| * |w| over the in-image taps (the plain forward
    pass of |x*s + b| with |w|; exact on small integers and dyadic s, b),
    whatever the activation."""
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        N, H, W, C, FH, FW, S, D, P = _case(rng)
        x, w = _ints(rng, (N, H, W, C)), _ints(rng, (FH, FW, C))
        s = rng.choice([-2.0, -0.5, 0.5, 1.0], size=C).astype(np.float32)
        b = rng.choice([-3.0, -1.5, 0.0, 2.5], size=C).astype(np.float32)
        pre = np.abs(x * s + b).astype(np.float32)   # exact in fp32
        want, _ = oracle.fwd(pre, np.abs(w), None, S, D, P, "f32", lib=lib)
        for act in ("none", "relu", "relu6"):
            _, got = oracle.fwd_bn_act(x, w, None, s, b, act, S, D, P, "f32", lib=lib)
            assert np.array_equal(got, want), act


def run_torch(lib, cases=30, seed=26):
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        N, H, W, C, FH, FW, S, D, P = _case(rng)
        x = rng.normal(size=(N, H, W, C)).astype(np.float32)
        w = rng.normal(size=(FH, FW, C)).astype(np.float32)
        bias = rng.normal(size=C).astype(np.float32)
        s = rng.normal(size=C).astype(np.float32)
        b = (3 * rng.normal(size=C)).astype(np.float32)
        xt = torch.from_numpy(x.astype(np.float64)).permute(0, 3, 1, 2)
        pre = xt * torch.from_numpy(s.astype(np.float64)).view(1, C, 1, 1) + \
            torch.from_numpy(b.astype(np.float64)).view(1, C, 1, 1)
        wt = torch.from_numpy(w.astype(np.float64)).permute(2, 0, 1).unsqueeze(1)
        bt = torch.from_numpy(bias.astype(np.float64))
        for act, fn in (("none", lambda t: t), ("relu", torch.relu),
                        ("relu6", lambda t: torch.clamp(t, 0.0, 6.0))):
            ref = F.conv2d(fn(pre), wt, bt, stride=S, padding=P, dilation=D, groups=C)
            ref = ref.permute(0, 2, 3, 1).numpy()
            got, _ = oracle.fwd_bn_act(x, w, bias, s, b, act, S, D, P, "f32", lib=lib)
            assert got.shape == ref.shape
            assert np.allclose(got, ref, rtol=1e-12, atol=1e-12), act


def test_identity_is_plain_forward():
    run_identity(oracle._load())


def test_affine_closed_form():
    run_affine(oracle._load())


def test_relu_regimes():
    run_relu_regimes(oracle._load())


def test_saturated_activation_and_padding():
    run_saturated(oracle._load())


def test_scale_independent_of_activation():
    run_scale(oracle._load())


def test_matches_torch_conv2d():
    run_torch(oracle._load())


def test_rejects_int8_and_unknown_activation():
    x = np.zeros((1, 4, 4, 2), np.int8)
    w = np.zeros((3, 3, 2), np.int8)
    with pytest.raises(ValueError):
        oracle.fwd_bn_act(x, w, None, np.ones(2), np.zeros(2), "relu", 1, 1, 1, "i8")
    with pytest.raises(ValueError):
        oracle.fwd_bn_act(x.astype(np.float32), w.astype(np.float32), None, np.ones(2),
                          np.zeros(2), "gelu", 1, 1, 1, "f32")


BNACT_MUTANTS = {
    "scale_shift_swapped": ("bn_scale[c] + bn_shift[c];", "bn_shift[c] + bn_scale[c];"),
    "no_relu6_clip": ("if (act == 2 && u > 6.0) u = 6.0;", "if (act == 2 && u > 6.0) u = u;"),
    "relu_wrong_side": ("if (act >= 1 && u < 0.0) u = 0.0;", "if (act >= 1 && u > 0.0) u = 0.0;"),
    "relu_never": ("if (act >= 1 && u < 0.0) u = 0.0;", "if (act >= 3 && u < 0.0) u = 0.0;"),
    "padding_is_act_of_shift": (
        "if (iw < 0 || iw >= W) continue;",
        "if (iw < 0 || iw >= W) { double pu = bn_shift[c]; if (act >= 1 && pu < 0.0) pu = 0.0;"
        " if (act == 2 && pu > 6.0) pu = 6.0; acc += pu * w[((long long)fh * FW + fw) * C + c];"
        " continue; }"),
    "bias_through_affine": ("double acc = bias ? bias[c] : 0.0;",
                            "double acc = bias ? bias[c] * bn_scale[c] : 0.0;"),
    "scale_after_activation": ("sabs += fabs(pre) * fabs(wv);", "sabs += fabs(u * wv);"),
}


def _pins(lib):
    failed = []
    for name, fn in [("identity", lambda: run_identity(lib, cases=10)),
                     ("affine", lambda: run_affine(lib, cases=15)),
                     ("relu", lambda: run_relu_regimes(lib, cases=10)),
                     ("saturated", lambda: run_saturated(lib, cases=10)),
                     ("scale", lambda: run_scale(lib, cases=10)),
                     ("torch", lambda: run_torch(lib, cases=10))]:
        try:
            fn()
        except (AssertionError, ValueError):
            failed.append(name)
    return failed


# ---- fp16 / bf16: U in the storage format ----

ACT_F32 = {"none": lambda v: v,
           "relu": lambda v: np.maximum(v, np.float32(0)),
           "relu6": lambda v: np.minimum(np.maximum(v, np.float32(0)), np.float32(6))}


def _to_storage(v32, fmt):
    """float32 values -> the storage format's values as float64, by the
    libraries' own conversions (numpy float16; torch bfloat16)."""
    v32 = np.asarray(v32, np.float32)
    with np.errstate(over="ignore"):
        if fmt == "f16":
            return v32.astype(np.float16).astype(np.float64)
    return torch.from_numpy(v32.copy()).to(torch.bfloat16).to(torch.float64).numpy()


def _encode(v, fmt):
    """Values exactly representable in fmt -> the oracle's stored form."""
    if fmt == "f16":
        return np.asarray(v, np.float16)
    bits = np.asarray(v, np.float32).view(np.uint32) >> np.uint32(16)
    return bits.astype(np.uint16)


def _unit_filter(C, fmt):
    return _encode(np.ones((1, 1, C), np.float32), fmt)


def _storage_values(rng, fmt, n):
    """x values of fmt: normal ones over a wide exponent range, subnormals and
    values near the largest finite one."""
    mag = rng.normal(size=n) * np.exp2(rng.integers(-12, 12, size=n))
    if fmt == "f16":
        mag[: n // 8] = rng.normal(size=n // 8) * 2.0 ** -20       # subnormal
        mag[n // 8: n // 4] = rng.uniform(50000, 65504, size=n - n // 8 - (n - n // 4))
    else:
        mag[: n // 8] = rng.normal(size=n // 8) * 2.0 ** -130     # subnormal
        mag[n // 8: n // 4] = rng.uniform(2.0e38, 3.38e38, size=n - n // 8 - (n - n // 4))
    return _to_storage(mag.astype(np.float32), fmt)


def _u_through_unit_filter(lib, xv, s, b, act, fmt):
    N, H, W, C = xv.shape
    y, scale = oracle.fwd_bn_act(_encode(xv, fmt), _unit_filter(C, fmt), None, s, b, act,
                                 1, 1, 0, fmt, lib=lib)
    return y, scale


def run_storage_rounding(lib, fmt, seed=31):
    """b = 0: the fused multiply-add is the float32 product, so U is the
    library conversion of act(float32(x) * s)."""
    rng = np.random.default_rng(seed)
    C = 8
    xv = _storage_values(rng, fmt, 4 * 64 * C).reshape(4, 8, 8, C)
    s = np.concatenate([rng.uniform(0.5, 1.5, C // 2),
                        rng.normal(size=C - C // 2) * 1.37]).astype(np.float32)
    for act, fn in ACT_F32.items():
        with np.errstate(over="ignore"):
            want = _to_storage(fn(xv.astype(np.float32) * s), fmt)
        got, _ = _u_through_unit_filter(lib, xv, s, np.zeros(C, np.float32), act, fmt)
        assert np.array_equal(got, want), (fmt, act)


def run_storage_ties(lib, fmt, seed=32):
    """x in [1, 2) plus an odd multiple of half its last place: every value is
    exactly halfway between two neighbours of fmt, so only the tie rule
    decides."""
    rng = np.random.default_rng(seed)
    C, bits = 4, (10 if fmt == "f16" else 7)
    k = rng.integers(0, 2 ** bits, size=(2, 8, 8, C))
    xv = (1.0 + k * 2.0 ** -bits).astype(np.float32)
    b = (np.array([1, -1, 3, -3]) * 2.0 ** -(bits + 1)).astype(np.float32)
    want = _to_storage(xv + b, fmt)            # x + b is exact in float32
    got, _ = _u_through_unit_filter(lib, xv, np.ones(C, np.float32), b, "none", fmt)
    assert np.array_equal(got, want), fmt


def _nearest_f32(q):
    """The float32 nearest to the rational q, ties to an even significand."""
    f = np.float32(float(q))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(fractions.Fraction(float(c)) - q)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def run_fma(lib, fmt, seed=33):
    """scale through a unit filter is |x*s + b| in float32: it must be the
    float32 nearest to the exact value; U the library conversion of it."""
    rng = np.random.default_rng(seed)
    C = 8
    xv = _to_storage(rng.normal(size=(2, 6, 6, C)).astype(np.float32), fmt)
    s = rng.uniform(0.5, 1.5, C).astype(np.float32)
    b = (rng.normal(size=C) * 0.7).astype(np.float32)
    y, scale = _u_through_unit_filter(lib, xv, s, b, "none", fmt)
    for i in np.ndindex(xv.shape):
        c = i[3]
        q = (fractions.Fraction(float(xv[i])) * fractions.Fraction(float(s[c]))
             + fractions.Fraction(float(b[c])))
        pre = _nearest_f32(q)
        assert scale[i] == abs(float(pre)), (fmt, i)
        assert y[i] == _to_storage(np.array([pre]), fmt)[0], (fmt, i)


def run_storage_shapes(lib, fmt, cases=20, seed=34):
    """Any shape: s = 1, b = 0 and no activation is the plain forward pass;
    with b = 0 the fused pass is the plain pass of the library-rounded U."""
    rng = np.random.default_rng(seed)
    for _ in range(cases):
        N, H, W, C, FH, FW, S, D, P = _case(rng)
        xv = _to_storage(rng.normal(size=(N, H, W, C)).astype(np.float32), fmt)
        w = _encode(_to_storage(rng.normal(size=(FH, FW, C)).astype(np.float32), fmt), fmt)
        bias = rng.normal(size=C).astype(np.float32)
        y0, s0 = oracle.fwd(_encode(xv, fmt), w, bias, S, D, P, fmt, lib=lib)
        y1, s1 = oracle.fwd_bn_act(_encode(xv, fmt), w, bias, np.ones(C), np.zeros(C), "none",
                                   S, D, P, fmt, lib=lib)
        assert np.array_equal(y0, y1) and np.array_equal(s0, s1)
        s = rng.uniform(0.5, 1.5, C).astype(np.float32)
        for act, fn in ACT_F32.items():
            u = _to_storage(fn(xv.astype(np.float32) * s), fmt)
            want, _ = oracle.fwd(_encode(u, fmt), w, bias, S, D, P, fmt, lib=lib)
            got, _ = oracle.fwd_bn_act(_encode(xv, fmt), w, bias, s, np.zeros(C), act,
                                       S, D, P, fmt, lib=lib)
            assert np.array_equal(got, want), (fmt, act)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_storage_rounding_matches_library_conversion(fmt):
    run_storage_rounding(oracle._load(), fmt)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_storage_rounding_ties_to_even(fmt):
    run_storage_ties(oracle._load(), fmt)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_prologue_is_one_fp32_fused_multiply_add(fmt):
    run_fma(oracle._load(), fmt)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_storage_format_any_shape(fmt):
    run_storage_shapes(oracle._load(), fmt)


STORAGE_MUTANTS = {
    "u_not_rounded": ("if (fmt) u = round_storage(u, fmt);", ""),
    "truncated": ("double r = nearbyint(a / q) * q;", "double r = trunc(a / q) * q;"),
    "ties_away": ("double r = nearbyint(a / q) * q;", "double r = round(a / q) * q;"),
    "f16_as_bf16": ("if (fmt == 1) return round_binary(u, 10, -14, 65504.0);",
                    "if (fmt == 1) return round_binary(u, 7, -126, ldexp(255.0, 120));"),
    "no_subnormal_spacing": ("if (e < emin) e = emin;", ""),
    "no_overflow": ("if (r > maxf) r = INFINITY;", ""),
    "two_roundings": ("(double)fmaf((float)xv, (float)bn_scale[c],",
                      "(double)(float)((float)((float)xv * (float)bn_scale[c]) +"),
}


def _storage_pins(lib):
    failed = []
    for fmt in ("f16", "bf16"):
        for name, fn in [("rounding", lambda: run_storage_rounding(lib, fmt)),
                         ("ties", lambda: run_storage_ties(lib, fmt)),
                         ("fma", lambda: run_fma(lib, fmt)),
                         ("shapes", lambda: run_storage_shapes(lib, fmt, cases=6))]:
            try:
                fn()
            except (AssertionError, ValueError):
                failed.append(f"{fmt} {name}")
    return failed


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_storage_mutants_are_caught(tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "dwref.c")).read()
    for name, (old, new) in STORAGE_MUTANTS.items():
        assert src.count(old) == 1, name
        path = tmp_path / f"storage_{name}.c"
        path.write_text(src.replace(old, new, 1))
        so = tmp_path / f"libstorage_{name}.so"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", str(path),
                               "-o", str(so), "-lm"])
        failed = _storage_pins(oracle.bind(str(so)))
        assert failed, f"mutant {name} passed every pin"
    assert _storage_pins(oracle._load()) == []


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_bnact_mutants_are_caught(tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "dwref.c")).read()
    head, body = src.split("int dwref_fwd_bnact_f64(", 1)   # the last function
    for name, (old, new) in BNACT_MUTANTS.items():
        assert body.count(old) == 1, name
        path = tmp_path / f"bnact_{name}.c"
        path.write_text(head + "int dwref_fwd_bnact_f64(" + body.replace(old, new, 1))
        so = tmp_path / f"libbnact_{name}.so"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", str(path),
                               "-o", str(so), "-lm"])
        failed = _pins(oracle.bind(str(so)))
        assert failed, f"mutant {name} passed every pin"
    assert _pins(oracle._load()) == []
