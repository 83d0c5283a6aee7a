"""The tolerance checker and the seeded input generators (CPU only)."""
import numpy as np
import pytest
import torch

from oracle import check
import synth
from synth import WORKLOADS, make_inputs, round_to_format, to_storage


# ---------------------------------------------------------------- generators

def test_round_to_fp16_matches_numpy():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(200000), rng.standard_normal(2000) * 1e-5,
                        np.array([0.0, -0.0, 65504.0, 2.0**-24, 2.0**-25, 3 * 2.0**-25,
                                  1 + 2.0**-11, 1 + 3 * 2.0**-11])])
    r = round_to_format(v, "f16")
    np.testing.assert_array_equal(r, v.astype(np.float16).astype(np.float64))


def test_round_to_bf16_ties_and_exact_cases():
    # exact bf16 values stay; halfway cases go to the even neighbour
    one = 1.0
    ulp = 2.0**-7
    assert round_to_format(one + ulp / 2, "bf16") == one                 # tie -> even (1.0)
    assert round_to_format(one + 3 * ulp / 2, "bf16") == one + 2 * ulp   # tie -> even
    assert round_to_format(one + ulp / 2 + 2.0**-40, "bf16") == one + ulp
    # a double that rounds differently in one step than through fp32:
    # 1 + 2^-8 + 2^-30 is just above the tie; fp32 first would land on the tie
    v = one + 2.0**-8 + 2.0**-30
    assert round_to_format(v, "bf16") == one + ulp
    assert float(torch.tensor(np.float32(v)).to(torch.bfloat16).float()) == one
    # for values already in fp32, torch's fp32 -> bf16 rounding agrees
    rng = np.random.default_rng(1)
    f = rng.standard_normal(100000).astype(np.float32)
    tb = torch.from_numpy(f).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(round_to_format(f.astype(np.float64), "bf16"), tb)


def test_to_storage_f32_matches_generic_rounding():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(100000), rng.standard_normal(1000) * 1e-40])
    np.testing.assert_array_equal(to_storage(v, "f32").astype(np.float64),
                                  round_to_format(v, "f32"))
    np.testing.assert_array_equal(to_storage(v[:1000], "f16").astype(np.float64),
                                  round_to_format(v[:1000], "f16"))


def test_to_storage_roundtrip():
    rng = np.random.default_rng(2)
    v = rng.standard_normal(1000)
    bits = to_storage(v, "bf16")
    assert bits.dtype == np.uint16
    back = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    np.testing.assert_array_equal(back, round_to_format(v, "bf16"))
    with pytest.raises(ValueError):
        to_storage(np.array([1e6]), "f16")


def test_workload_inputs_are_seeded_and_shaped():
    wl = WORKLOADS["tiny_f32_3x3"]
    a = make_inputs(wl)
    b = make_inputs(wl)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    x, w, bias = a
    assert x.shape == (1, 16, 16, 8) and w.shape == (3, 3, 8) and bias.shape == (8,)
    assert x.dtype == np.float32 and np.abs(x).max() <= 1
    wl5 = WORKLOADS["strided_i8_5x5"]
    x, w, bias = make_inputs(wl5, n=2)
    assert x.dtype == np.int8 and bias.dtype == np.int32
    assert bias.min() >= -2**15 and bias.max() <= 2**15
    # variance, not standard deviation: W ~ N(0, 1/49) has std 1/7
    wl3 = WORKLOADS["convnext_f16_7x7"]
    _, w, _ = make_inputs(wl3, n=1)
    assert w.dtype == np.float16 and abs(float(w.astype(np.float64).std()) - 1 / 7) < 0.01


# ------------------------------------------------------------------- checker

def test_checker_accepts_correct_rounding():
    rng = np.random.default_rng(3)
    ye = rng.standard_normal(50000) * 3
    scale = np.abs(ye) + rng.uniform(0, 5, ye.shape)
    for fmt in ("f32", "f16", "bf16"):
        y = to_storage(ye, fmt)
        ok, rep = check.check_float(y, fmt, ye, scale)
        assert ok.all(), (fmt, rep)


def test_checker_rejects_wrong_values():
    ye = np.array([1.0, -2.5, 100.0, 0.0])
    scale = np.array([1.0, 1.0, 1.0, 1.0])
    for fmt in ("f32", "f16", "bf16"):
        good = to_storage(ye, fmt)
        # two ulps away (more than tau + half an ulp) must fail
        v, lo, hi = check.midpoints(good, fmt)
        ulp = 2 * (hi - v)
        bad = to_storage(v + 2 * ulp + 4 * check.tau(scale), fmt)
        ok, _ = check.check_float(bad, fmt, ye, scale)
        assert not ok.any(), fmt
    # NaN fails
    ok, _ = check.check_float(np.array([np.nan], np.float32), "f32", [0.0], [1.0])
    assert not ok.any()


def test_checker_tau_window():
    # an fp32 output off by exactly tau (plus rounding slack) passes, 2 tau fails
    ye = np.array([1.0])
    scale = np.array([10.0])
    t = check.tau(scale)[0]
    ok, _ = check.check_float(np.float32([1.0 + 0.9 * t]), "f32", ye, scale)
    assert ok.all()
    ok, _ = check.check_float(np.float32([1.0 + 2 * t]), "f32", ye, scale)
    assert not ok.any()


def test_checker_midpoints_zero_and_extremes():
    v, lo, hi = check.midpoints(np.array([0, 0x8000, 0x7f7f], np.uint16), "bf16")
    assert v[0] == 0 and v[1] == 0
    assert lo[0] == -2.0**-134 and hi[0] == 2.0**-134
    assert np.isfinite(hi[2]) and hi[2] > v[2]


def test_assert_int():
    check.assert_int(np.array([1, -2], np.int32), np.array([1, -2]))
    with pytest.raises(AssertionError):
        check.assert_int(np.array([1, -3], np.int32), np.array([1, -2]))
    with pytest.raises(AssertionError):
        check.assert_int(np.array([0], np.int32), np.array([2**31]))


def test_random_small_is_valid():
    rng = np.random.default_rng(4)
    for _ in range(200):
        wl = synth.random_small(rng, "f32")
        assert (wl.H + 2 * wl.pad - wl.dilation * (wl.FH - 1) - 1) >= 0
