"""Seeded synthetic inputs for the forward depthwise convolution.

Shared by the tests, the bench and the smoke check; used to feed both the HIP
library and the CPU oracle.  It holds no convolution arithmetic: only the
workload table (shapes, dtypes and value distributions), a seeded NumPy
generator and the host-side casts of the drawn float64 values to the storage
formats.

Storage formats: "f32" float32, "f16" float16, "bf16" uint16 bit patterns,
"i8" int8 (bias int32).  Float biases are float32.  Layouts are channel-last:
x N x H x W x C, w FH x FW x C, bias C.

Draws use ``numpy.random.Generator(PCG64(seed))`` in the order x, w, bias.
Float values are drawn in float64 and rounded once, to nearest-even, straight
into the storage format.  ``("normal", mean, var)`` takes a *variance*.
"""
from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: str
    N: int
    H: int
    W: int
    C: int
    FH: int
    FW: int
    stride: int
    dilation: int
    pad: int
    x_dist: tuple
    w_dist: tuple
    b_dist: tuple  # None: no bias
    seed: int
    note: str = field(default="", compare=False)


# The five workloads: a tiny correctness case and four real-size ones shaped
# like a MobileNet 3x3 layer, a ConvNeXt 7x7 layer, a large-kernel (31x31)
# layer and a strided, dilated int8 layer with a ragged channel count.
WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32_3x3", "f32", 1, 16, 16, 8, 3, 3, 1, 1, 1,
                 ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0), ("uniform", -1.0, 1.0), 1,
                 "1x16x16x8, 3x3, stride 1, pad 1, bias"),
        Workload("mobilenet_f32_3x3", "f32", 64, 56, 56, 128, 3, 3, 1, 1, 1,
                 ("normal", 0.0, 1.0), ("normal", 0.0, 1.0 / 9), ("uniform", -0.1, 0.1), 2,
                 "64x56x56x128 fp32, 3x3, stride 1, pad 1, bias"),
        Workload("convnext_f16_7x7", "f16", 64, 56, 56, 96, 7, 7, 1, 1, 3,
                 ("normal", 0.0, 1.0), ("normal", 0.0, 1.0 / 49), ("uniform", -0.1, 0.1), 3,
                 "64x56x56x96 fp16 in/out, fp32 accumulate, 7x7, pad 3, bias"),
        Workload("largekernel_bf16_31x31", "bf16", 32, 56, 56, 128, 31, 31, 1, 1, 15,
                 ("normal", 0.0, 1.0), ("normal", 0.0, 1.0 / 961), ("uniform", -0.1, 0.1), 4,
                 "32x56x56x128 bf16 in/out, fp32 accumulate, 31x31, pad 15, bias"),
        Workload("strided_i8_5x5", "i8", 16, 112, 112, 61, 5, 5, 2, 2, 4,
                 ("int", -128, 127), ("int", -128, 127), ("int", -2**15, 2**15), 5,
                 "16x112x112x61 int8 -> int32, 5x5, stride 2, dilation 2, pad 4, int32 bias"),
    ]
}

# significand bits (with the hidden bit) and exponent of the smallest
# subnormal, per float storage format
_FLOAT_FORMATS = {"f32": (24, -149), "f16": (11, -24), "bf16": (8, -133)}
_MAX_FINITE = {"f32": float(np.finfo(np.float32).max), "f16": 65504.0,
               "bf16": float.fromhex("0x1.fep127")}


def round_to_format(v, fmt):
    """float64 -> nearest value of ``fmt``, ties to even, as float64.

    One rounding step: v is scaled by the power of two of its own ulp in the
    target format (clamped at the subnormal ulp), rounded to an integer with
    numpy's half-to-even rounding, and scaled back."""
    sig, min_exp = _FLOAT_FORMATS[fmt]
    v = np.asarray(v, np.float64)
    _, e = np.frexp(v)
    ulp_e = np.maximum(e - sig, min_exp)
    r = np.ldexp(np.round(np.ldexp(v, -ulp_e)), ulp_e)
    if np.any(np.abs(r) > _MAX_FINITE[fmt]):
        raise ValueError(f"value out of {fmt} range")
    return r


def to_storage(v, fmt):
    """float64 -> storage array of ``fmt`` (one rounding, see round_to_format).

    fp32 and fp16 use numpy's own float64 casts, which round once to nearest
    even (the tests check that they agree with round_to_format); bf16 has no
    numpy type and goes through round_to_format."""
    v = np.asarray(v, np.float64)
    if fmt in ("f32", "f16"):
        with np.errstate(over="ignore"):
            r = v.astype(np.float32 if fmt == "f32" else np.float16)
        if not np.all(np.isfinite(r[np.isfinite(v)])):
            raise ValueError(f"value out of {fmt} range")
        return r
    r = round_to_format(v, fmt)
    if fmt == "bf16":
        # exact: r is a bf16 value, so fp32 holds it and its low 16 bits are 0
        return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    raise ValueError(fmt)


def _draw(rng, dist, shape):
    kind = dist[0]
    if kind == "uniform":
        return rng.uniform(dist[1], dist[2], size=shape)
    if kind == "normal":
        return rng.normal(dist[1], np.sqrt(dist[2]), size=shape)
    if kind == "int":  # closed range [lo, hi]
        return rng.integers(dist[1], dist[2] + 1, size=shape, dtype=np.int64)
    if kind == "ones":
        return np.ones(shape)
    raise ValueError(kind)


def make_inputs(wl: Workload, seed=None, n=None):
    """(x, w, bias) of workload ``wl`` in storage formats.  ``n`` overrides
    the batch size (the first n images of the same draw are NOT guaranteed;
    the whole draw changes with the shape)."""
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    N = wl.N if n is None else n
    xs = (N, wl.H, wl.W, wl.C)
    ws = (wl.FH, wl.FW, wl.C)
    x = _draw(rng, wl.x_dist, xs)
    w = _draw(rng, wl.w_dist, ws)
    b = None if wl.b_dist is None else _draw(rng, wl.b_dist, (wl.C,))
    if wl.dtype == "i8":
        return (x.astype(np.int8), w.astype(np.int8),
                None if b is None else b.astype(np.int32))
    return (to_storage(x, wl.dtype), to_storage(w, wl.dtype),
            None if b is None else to_storage(b, "f32"))


def random_small(rng, dtype, max_hw=20, max_c=70, max_f=7):
    """A random small workload for parity sweeps: ragged sizes, stride 1-3,
    dilation 1-3, padding 0..span, N(0,1) data (uniform integers for i8)."""
    while True:
        FH = int(rng.integers(1, max_f + 1))
        FW = int(rng.integers(1, max_f + 1))
        S = int(rng.integers(1, 4))
        D = int(rng.integers(1, 4))
        P = int(rng.integers(0, max(FH, FW) * D // 2 + 2))
        H = int(rng.integers(1, max_hw + 1))
        W = int(rng.integers(1, max_hw + 1))
        C = int(rng.integers(1, max_c + 1))
        N = int(rng.integers(1, 4))
        oh = (H + 2 * P - D * (FH - 1) - 1)
        ow = (W + 2 * P - D * (FW - 1) - 1)
        if oh >= 0 and ow >= 0:
            break
    if dtype == "i8":
        dist = ("int", -128, 127)
        bd = ("int", -2**15, 2**15)
    else:
        dist = ("normal", 0.0, 1.0)
        bd = ("uniform", -0.1, 0.1)
    return Workload(f"rand_{dtype}", dtype, N, H, W, C, FH, FW, S, D, P,
                    dist, dist, bd if rng.integers(0, 4) else None,
                    int(rng.integers(0, 2**31)))



def device_input(shape, fmt, seed, device):
    """A large seeded input drawn on the GPU by torch's generator (for
    tensors too big to draw and copy from the host in a test): N(0, 1) for
    the float formats (drawn in fp32, then rounded to the storage format by
    torch), uniform integers in [-128, 127] for int8.  Returns a torch
    tensor in the storage format (bf16 as torch.bfloat16)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    if fmt == "i8":
        return torch.randint(-128, 128, shape, generator=g, device=device, dtype=torch.int8)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return t.to({"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[fmt])
