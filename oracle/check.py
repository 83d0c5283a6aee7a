"""Tolerance rule for floating-point outputs.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The floating-point bound is stated elementwise against the output's own
sum |x*w|:  |y - y_ref| <= 1e-5 * sum|x*w| + 1e-6  (tau below).  For fp16 and
bf16 outputs the final rounding alone can exceed tau (half an ulp of |y| ~ 1 is
2^-11 or 2^-8), so the bound is read as a bound on the value *before* the one
final rounding: an output passes iff it is the round-to-nearest image, in its
own format, of some real v with |v - y_exact| <= tau.  With m- and m+ the
midpoints between y and its lower and upper neighbours in the output format,
that is  m- <= y_exact + tau  and  m+ >= y_exact - tau.  Neighbours are found
by stepping the bit pattern, so no value is ever rounded twice (fp64 -> fp32 ->
bf16 could misjudge a tie).  fp32 outputs use the same rule.
"""
import numpy as np

REL = 1e-5
ABS = 1e-6

_FMT = {
    # storage dtype, unsigned view, sign mask
    "f32": (np.float32, np.uint32, 0x80000000),
    "f16": (np.float16, np.uint16, 0x8000),
    "bf16": (None, np.uint16, 0x8000),
}


def _bits(y, fmt):
    store, uview, _ = _FMT[fmt]
    a = np.asarray(y)
    if fmt == "bf16":
        return a.astype(np.uint16).astype(np.int64)
    return a.astype(store).view(uview).astype(np.int64)


def _value(bits, fmt):
    """Bit patterns (int64) -> float64, exactly (NaN patterns stay NaN)."""
    with np.errstate(invalid="ignore"):
        return _value_raw(bits, fmt)


def _value_raw(bits, fmt):
    if fmt == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    if fmt == "f16":
        return bits.astype(np.uint16).view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def midpoints(y, fmt):
    """(value, lower midpoint, upper midpoint) in float64 for outputs ``y``
    stored in ``fmt`` ("f32", "f16" or "bf16"; bf16 as uint16 bits)."""
    sign = _FMT[fmt][2]
    b = _bits(y, fmt)
    mag = b & (sign - 1)
    key = np.where(b & sign, -mag, mag)          # monotone in the value; +0 and -0 -> 0

    def from_key(k):
        return np.where(k < 0, (-k) | sign, k)

    v = _value(b, fmt)
    lo = _value(from_key(key - 1), fmt)
    hi = _value(from_key(key + 1), fmt)
    with np.errstate(invalid="ignore", over="ignore"):
        # past the largest finite value the neighbour is +-inf: mirror the
        # spacing below it (both sides of the largest value share one binade)
        hi = np.where(np.isinf(hi), v + (v - lo), hi)
        lo = np.where(np.isinf(lo), v - (hi - v), lo)
        return v, (v + lo) / 2, (v + hi) / 2


def tau(scale):
    return REL * np.asarray(scale, np.float64) + ABS


def check_float(y, fmt, y_exact, scale):
    """Returns (ok: bool array, report: dict).  ``y`` are the outputs in their
    storage format, ``y_exact``/``scale`` the oracle's fp64 sum and sum|x*w|."""
    v, mlo, mhi = midpoints(y, fmt)
    t = tau(scale)
    ye = np.asarray(y_exact, np.float64)
    finite = np.isfinite(v)
    ok = finite & (mlo <= ye + t) & (mhi >= ye - t)
    err = np.where(finite, np.abs(v - ye), np.inf)
    denom = np.maximum(np.abs(ye), 1e-30)
    report = {
        "n": int(ok.size),
        "fail": int(ok.size - np.count_nonzero(ok)),
        "max_abs_err": float(err.max()) if err.size else 0.0,
        "max_err_over_tau": float((err / t).max()) if err.size else 0.0,
        # mean absolute relative error vs fp64, reported beside pass/fail
        "mare": float(np.mean(err / denom)) if err.size else 0.0,
    }
    return ok, report


def assert_float(y, fmt, y_exact, scale, what=""):
    ok, rep = check_float(y, fmt, y_exact, scale)
    if not ok.all():
        bad = np.flatnonzero(~ok.ravel())[:8]
        v = _value(_bits(y, fmt), fmt).ravel()
        detail = ", ".join(
            f"[{i}] got {v[i]!r} want {np.ravel(y_exact)[i]!r} tau {tau(np.ravel(scale)[i])!r}"
            for i in bad)
        raise AssertionError(f"{what}: {rep['fail']}/{rep['n']} outside tolerance: {detail}")
    return rep


def assert_int(y, y_exact, what=""):
    """int32 outputs must equal the exact int64 sums bit for bit."""
    ye = np.asarray(y_exact, np.int64)
    if ye.size and (ye.min() < -2**31 or ye.max() >= 2**31):
        raise AssertionError(f"{what}: exact result does not fit int32")
    got = np.asarray(y).astype(np.int64)
    bad = np.flatnonzero(got.ravel() != ye.ravel())
    if bad.size:
        i = bad[:8]
        raise AssertionError(f"{what}: {bad.size}/{ye.size} mismatches, e.g. at {i.tolist()}: "
                             f"got {got.ravel()[i].tolist()} want {ye.ravel()[i].tolist()}")
