"""Helpers for the GPU tests: host <-> device copies of the storage formats,
running a plan through the C ABI, and checking against the oracle."""
import sys

import numpy as np
import torch

import depthwise_convolution_amd as dw
import oracle
from oracle import check

DEV = "cuda:0"
Y_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16, "i8": np.int32}


def say(msg):
    """Names the case before a GPU step, flushed, so a failing run shows it."""
    print(msg, file=sys.stderr, flush=True)


def to_dev(a, fmt):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if fmt == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def y_to_host(t, fmt):
    if fmt == "bf16":
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def y_torch_dtype(fmt):
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
            "i8": torch.int32}[fmt]


def run(x, w, b, shape, fmt, variant="auto", guard=0, y_prefill=None):
    """Runs one forward pass through the C ABI and returns y on the host.
    With ``guard`` > 0, y sits inside a larger buffer whose guard bands are
    filled with a sentinel and checked afterwards for stray writes."""
    N, H, W, C, FH, FW, S, D, P = shape
    h = dw.dwconv_create_variant(N, H, W, C, FH, FW, S, D, P, fmt, variant)
    try:
        OH, OW = dw.dwconv_output_dims(h)
        n_y = N * OH * OW * C
        tdt = y_torch_dtype(fmt)
        buf = torch.empty(n_y + 2 * guard, dtype=tdt, device=DEV)
        if tdt.is_floating_point:
            buf.fill_(float("nan") if y_prefill is None else y_prefill)
        else:
            buf.fill_(-0x55555556 if y_prefill is None else y_prefill)
        y = buf[guard:guard + n_y]
        xd, wd, bd = to_dev(x, fmt), to_dev(w, fmt), to_dev(b, "f32" if fmt != "i8" else "i8")
        dw.dwconv_fwd(h, xd, wd, bd, y)
        torch.cuda.synchronize()
        host = buf.view(torch.int16).cpu().numpy().view(np.uint16) if fmt == "bf16" \
            else buf.cpu().numpy()
        if guard:
            g = np.concatenate([host[:guard], host[guard + n_y:]])
            ref = to_sentinel(fmt, y_prefill)
            assert np.all(g.view(np.uint8) == np.full(g.shape, ref, g.dtype).view(np.uint8)), \
                "write outside y"
        return host[guard:guard + n_y].reshape(N, OH, OW, C), dw.dwconv_plan_variant(h)
    finally:
        dw.dwconv_destroy(h)


def to_sentinel(fmt, prefill):
    if fmt == "i8":
        return np.int32(-0x55555556 if prefill is None else prefill)
    t = torch.full((1,), float("nan") if prefill is None else prefill,
                   dtype=y_torch_dtype(fmt))
    return y_to_host(t, fmt)[0]


def assert_matches_oracle(y, x, w, b, shape, fmt, what=""):
    N, H, W, C, FH, FW, S, D, P = shape
    yo, scale = oracle.fwd(x, w, b, S, D, P, fmt, threads=8)
    if fmt == "i8":
        check.assert_int(y, yo, what)
        return None
    return check.assert_float(y, fmt, yo, scale, what)


def shape_of(wl):
    return (wl.N, wl.H, wl.W, wl.C, wl.FH, wl.FW, wl.stride, wl.dilation, wl.pad)
