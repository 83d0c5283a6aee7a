"""CPU oracle for the depthwise 2-D convolution (forward, backward data and
backward filter).

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
bench's ``cpu_baseline`` leg import this package.  The product path (the HIP
library and its Python binding) never imports, links or calls it, and it
shares no code with them.

The arithmetic lives in ``dwref.c`` (a plain loop nest, fp64 / int64); this
module only marshals numpy arrays into it:

* ``fwd``     -- the whole output, plus sum|x*w| per output for float dtypes;
* ``points``  -- selected outputs only (for shapes too large for a full pass);
* ``bwd_data`` -- the gradient with respect to the input (float dtypes), plus
  sum|dy*w| per input element;
* ``bwd_filter`` -- the gradient with respect to the filter (float dtypes),
  plus sum|x*dy| per tap;
* ``decode``  -- widens stored fp32 / fp16 / bf16 values to float64 exactly.

Storage formats (the same ones the library takes): ``"f32"`` float32,
``"f16"`` float16, ``"bf16"`` uint16 holding bfloat16 bit patterns, ``"i8"``
int8 with an int32 bias.  Float bias is float32.  Layouts are channel-last:
x is N x H x W x C, w is FH x FW x C, y is N x OH x OW x C ("Flash-DWC: Making
Depthwise Convolution Compute-Efficient on GPUs", section 2.3).
"""
import ctypes
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import build as _build

DTYPES = ("f32", "f16", "bf16", "i8")

_lib = None


def bind(path):
    """Loads an oracle library build from ``path`` and declares its entry
    points.  The tests use this to run the pins against deliberately broken
    copies of the oracle (mutation checks); everything else uses ``_load``."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.dwref_out_dim.argtypes = [I, I, I, I, I]
    lib.dwref_out_dim.restype = I
    lib.dwref_fwd_f64.argtypes = [P, P, P, P, P] + [I] * 11
    lib.dwref_fwd_f64.restype = I
    lib.dwref_fwd_i8.argtypes = [P, P, P, P] + [I] * 11
    lib.dwref_fwd_i8.restype = I
    lib.dwref_points_f64.argtypes = [P, P, P, P, ctypes.c_int64, P, P] + [I] * 9
    lib.dwref_points_f64.restype = I
    lib.dwref_points_i8.argtypes = [P, P, P, P, ctypes.c_int64, P] + [I] * 9
    lib.dwref_points_i8.restype = I
    lib.dwref_bwd_data_f64.argtypes = [P, P, P, P] + [I] * 11
    lib.dwref_bwd_data_f64.restype = I
    lib.dwref_bwd_filter_f64.argtypes = [P, P, P, P] + [I] * 11
    lib.dwref_bwd_filter_f64.restype = I
    lib.dwref_fwd_bnact_f64.argtypes = [P, P, P, P, P, I, I, P, P] + [I] * 11
    lib.dwref_fwd_bnact_f64.restype = I
    return lib


def _load():
    global _lib
    if _lib is None:
        _lib = bind(_build.ensure_built())
    return _lib


def out_dim(size: int, f: int, s: int, d: int, p: int, lib=None) -> int:
    """Largest output extent whose halo span fits the zero-padded input; 0 if none."""
    return (lib or _load()).dwref_out_dim(size, f, s, d, p)


def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored values -> float64, exactly."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"decode: no float format {dtype!r}")


def _ptr(a):
    return None if a is None else a.ctypes.data


def _prep(x, w, bias, dtype):
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    if x.ndim != 4 or w.ndim != 3 or x.shape[3] != w.shape[2]:
        raise ValueError("x must be N x H x W x C and w FH x FW x C")
    C = x.shape[3]
    if dtype == "i8":
        xx = np.ascontiguousarray(x, dtype=np.int8)
        ww = np.ascontiguousarray(w, dtype=np.int8)
        bb = None if bias is None else np.ascontiguousarray(bias, dtype=np.int32)
    else:
        xx = np.ascontiguousarray(decode(x, dtype))
        ww = np.ascontiguousarray(decode(w, dtype))
        bb = None if bias is None else np.ascontiguousarray(
            np.asarray(bias, dtype=np.float32).astype(np.float64))
    if bb is not None and bb.shape != (C,):
        raise ValueError("bias must have C elements")
    return xx, ww, bb


def fwd(x, w, bias, stride, dilation, pad, dtype, threads=1, lib=None):
    """Whole forward pass.

    Returns ``(y, scale)`` for float dtypes -- y the fp64 sum, scale the fp64
    sum of |x*w| over the same taps -- and ``(y, None)`` with int64 y for
    ``"i8"``.  ``threads`` > 1 splits the batch over threads (each output is
    independent, so the result is identical)."""
    xx, ww, bb = _prep(x, w, bias, dtype)
    N, H, W, C = xx.shape
    FH, FW = ww.shape[:2]
    lib = lib or _load()
    OH = out_dim(H, FH, stride, dilation, pad, lib)
    OW = out_dim(W, FW, stride, dilation, pad, lib)
    if OH < 1 or OW < 1:
        raise ValueError("no output: the filter span exceeds the padded input")
    if dtype == "i8":
        y = np.empty((N, OH, OW, C), np.int64)
        scale = None

        def run(n0, n1):
            return lib.dwref_fwd_i8(_ptr(xx), _ptr(ww), _ptr(bb), _ptr(y),
                                    N, H, W, C, FH, FW, stride, dilation, pad, n0, n1)
    else:
        y = np.empty((N, OH, OW, C), np.float64)
        scale = np.empty((N, OH, OW, C), np.float64)

        def run(n0, n1):
            return lib.dwref_fwd_f64(_ptr(xx), _ptr(ww), _ptr(bb), _ptr(y), _ptr(scale),
                                     N, H, W, C, FH, FW, stride, dilation, pad, n0, n1)
    threads = max(1, min(int(threads), N))
    if threads == 1:
        rcs = [run(0, N)]
    else:
        bounds = np.linspace(0, N, threads + 1).astype(int)
        with ThreadPoolExecutor(threads) as ex:
            rcs = list(ex.map(run, bounds[:-1], bounds[1:]))
    if any(rcs):
        raise ValueError("oracle rejected the shape")
    return y, scale


def points(x, w, bias, stride, dilation, pad, dtype, idx, lib=None):
    """Selected outputs: ``idx`` are flat indices into the N*OH*OW*C output."""
    xx, ww, bb = _prep(x, w, bias, dtype)
    N, H, W, C = xx.shape
    FH, FW = ww.shape[:2]
    ii = np.ascontiguousarray(idx, dtype=np.int64)
    lib = lib or _load()
    if dtype == "i8":
        y = np.empty(ii.shape, np.int64)
        rc = lib.dwref_points_i8(_ptr(xx), _ptr(ww), _ptr(bb), _ptr(ii), ii.size, _ptr(y),
                                 N, H, W, C, FH, FW, stride, dilation, pad)
        scale = None
    else:
        y = np.empty(ii.shape, np.float64)
        scale = np.empty(ii.shape, np.float64)
        rc = lib.dwref_points_f64(_ptr(xx), _ptr(ww), _ptr(bb), _ptr(ii), ii.size,
                                  _ptr(y), _ptr(scale),
                                  N, H, W, C, FH, FW, stride, dilation, pad)
    if rc:
        raise ValueError("oracle rejected the shape or an index")
    return y, scale


def bwd_data(dy, w, shape, dtype, threads=1, lib=None):
    """Gradient with respect to the input, from its definition (the adjoint
    of the forward pass; "Flash-DWC", section 5.1).  ``shape`` is the forward
    operation (N, H, W, C, FH, FW, stride, dilation, pad); dy is
    N x OH x OW x C in ``dtype`` (a float format).  Returns ``(dx, scale)`` in
    fp64, dx N x H x W x C and scale the sum of |dy*w| per dx element."""
    if dtype not in ("f32", "f16", "bf16"):
        raise ValueError("backward data is defined here for float dtypes")
    N, H, W, C, FH, FW, S, D, P = shape
    lib = lib or _load()
    OH = out_dim(H, FH, S, D, P, lib)
    OW = out_dim(W, FW, S, D, P, lib)
    if OH < 1 or OW < 1:
        raise ValueError("no output: the filter span exceeds the padded input")
    gg = np.ascontiguousarray(decode(dy, dtype))
    ww = np.ascontiguousarray(decode(w, dtype))
    if gg.shape != (N, OH, OW, C) or ww.shape != (FH, FW, C):
        raise ValueError("dy must be N x OH x OW x C and w FH x FW x C")
    dx = np.empty((N, H, W, C), np.float64)
    scale = np.empty((N, H, W, C), np.float64)

    def run(n0, n1):
        return lib.dwref_bwd_data_f64(_ptr(gg), _ptr(ww), _ptr(dx), _ptr(scale),
                                      N, H, W, C, FH, FW, S, D, P, n0, n1)
    threads = max(1, min(int(threads), N))
    if threads == 1:
        rcs = [run(0, N)]
    else:
        bounds = np.linspace(0, N, threads + 1).astype(int)
        with ThreadPoolExecutor(threads) as ex:
            rcs = list(ex.map(run, bounds[:-1], bounds[1:]))
    if any(rcs):
        raise ValueError("oracle rejected the shape")
    return dx, scale


def bwd_filter(x, dy, shape, dtype, threads=1, lib=None):
    """Gradient with respect to the filter, from its definition ("Flash-DWC",
    section 5.1).  ``shape`` is the forward operation (N, H, W, C, FH, FW,
    stride, dilation, pad); x is N x H x W x C and dy N x OH x OW x C in
    ``dtype`` (a float format).  Returns ``(dw, scale)`` in fp64, FH x FW x C,
    scale the sum of |x*dy| per tap.  ``threads`` > 1 splits the channels over
    threads (channels are independent, so the result is identical)."""
    if dtype not in ("f32", "f16", "bf16"):
        raise ValueError("backward filter is defined here for float dtypes")
    N, H, W, C, FH, FW, S, D, P = shape
    lib = lib or _load()
    OH = out_dim(H, FH, S, D, P, lib)
    OW = out_dim(W, FW, S, D, P, lib)
    if OH < 1 or OW < 1:
        raise ValueError("no output: the filter span exceeds the padded input")
    xx = np.ascontiguousarray(decode(x, dtype))
    gg = np.ascontiguousarray(decode(dy, dtype))
    if xx.shape != (N, H, W, C) or gg.shape != (N, OH, OW, C):
        raise ValueError("x must be N x H x W x C and dy N x OH x OW x C")
    dw = np.empty((FH, FW, C), np.float64)
    scale = np.empty((FH, FW, C), np.float64)

    def run(c0, c1):
        return lib.dwref_bwd_filter_f64(_ptr(xx), _ptr(gg), _ptr(dw), _ptr(scale),
                                        N, H, W, C, FH, FW, S, D, P, c0, c1)
    threads = max(1, min(int(threads), C))
    if threads == 1:
        rcs = [run(0, C)]
    else:
        bounds = np.linspace(0, C, threads + 1).astype(int)
        with ThreadPoolExecutor(threads) as ex:
            rcs = list(ex.map(run, bounds[:-1], bounds[1:]))
    if any(rcs):
        raise ValueError("oracle rejected the shape")
    return dw, scale


ACTS = {"none": 0, "relu": 1, "relu6": 2}
# the format U is stored in before the convolution: exact (fp32 data), or
# binary16 / bfloat16 after one fp32 fused multiply-add
FORMATS = {"f32": 0, "f16": 1, "bf16": 2}


def fwd_bn_act(x, w, bias, bn_scale, bn_shift, act, stride, dilation, pad, dtype, threads=1,
               lib=None):
    """Forward pass of U = act(x * bn_scale + bn_shift) -- a per-channel
    affine (folded batch normalization) and an activation fused in front of
    the convolution ("Flash-DWC", section 5.2) -- with zero padding of U.
    ``act`` is "none", "relu" or "relu6"; bn_scale and bn_shift hold C fp32
    values.  Float dtypes only.  fp32: U exact.  fp16 / bf16: U is what the
    separate BN + Act pass would store in that format (section 4.1: tensors
    kept in FP16, FP16 multiplications, FP32 accumulation): one fp32 fused
    multiply-add, the activation, then round to nearest even.  Returns
    ``(y, scale)`` in fp64, scale the sum of |x*s + b| * |w| over each
    output's taps."""
    if dtype not in ("f32", "f16", "bf16"):
        raise ValueError("the fused prologue is defined here for float dtypes")
    if act not in ACTS:
        raise ValueError(f"unknown activation {act!r}")
    xx, ww, bb = _prep(x, w, bias, dtype)
    N, H, W, C = xx.shape
    FH, FW = ww.shape[:2]
    ss = np.ascontiguousarray(np.asarray(bn_scale, dtype=np.float32).astype(np.float64))
    tt = np.ascontiguousarray(np.asarray(bn_shift, dtype=np.float32).astype(np.float64))
    if ss.shape != (C,) or tt.shape != (C,):
        raise ValueError("bn_scale and bn_shift must have C elements")
    lib = lib or _load()
    OH = out_dim(H, FH, stride, dilation, pad, lib)
    OW = out_dim(W, FW, stride, dilation, pad, lib)
    if OH < 1 or OW < 1:
        raise ValueError("no output: the filter span exceeds the padded input")
    y = np.empty((N, OH, OW, C), np.float64)
    scale = np.empty((N, OH, OW, C), np.float64)

    def run(n0, n1):
        return lib.dwref_fwd_bnact_f64(_ptr(xx), _ptr(ww), _ptr(bb), _ptr(ss), _ptr(tt),
                                       ACTS[act], FORMATS[dtype], _ptr(y), _ptr(scale),
                                       N, H, W, C, FH, FW, stride, dilation, pad, n0, n1)
    threads = max(1, min(int(threads), N))
    if threads == 1:
        rcs = [run(0, N)]
    else:
        bounds = np.linspace(0, N, threads + 1).astype(int)
        with ThreadPoolExecutor(threads) as ex:
            rcs = list(ex.map(run, bounds[:-1], bounds[1:]))
    if any(rcs):
        raise ValueError("oracle rejected the shape")
    return y, scale
