"""Python binding of libdwconv.so, the gfx950 forward depthwise convolution.

The functions carry the C ABI's names (``include/dwconv.h``) and only marshal
arguments: every step of the computation runs in the HIP kernels.  Torch is
used for device memory and streams.  There is no CPU path: if the library is
missing, importing this package fails.

    h = dwconv_create(N, H, W, C, FH, FW, stride, dilation, pad, "f16")
    dwconv_fwd(h, x, w, bias, y)          # torch tensors on the GPU, or raw ints
    dwconv_destroy(h)

or, with allocation of the output:

    conv = DepthwiseConv2d(N, H, W, C, FH, FW, stride, dilation, pad, "f16")
    y = conv(x, w, bias)
"""
import ctypes
import os

# torch carries its own HIP and HSA runtimes (same sonames as /opt/rocm's).
# Loading it first makes libdwconv.so bind to those copies, so the process
# holds one HIP runtime and torch's device pointers and streams are valid in
# the library.  Loaded the other way round, two runtimes would share the GPU.
import torch  # noqa: E402,F401

__all__ = [
    "DWCONV_F32", "DWCONV_F16", "DWCONV_BF16", "DWCONV_I8",
    "DWCONV_SCRATCH_BYTES", "VARIANTS", "DwconvError", "DepthwiseConv2d", "library_path",
    "dwconv_create", "dwconv_create_variant", "dwconv_fwd", "dwconv_destroy",
    "dwconv_output_dims", "dwconv_plan_variant", "dwconv_plan_describe",
    "dwconv_plan_tile", "dwconv_status_string",
]

DWCONV_F32, DWCONV_F16, DWCONV_BF16, DWCONV_I8 = 0, 1, 2, 3
DWCONV_SCRATCH_BYTES = 64 << 20  # include/dwconv.h
VARIANTS = {"auto": 0, "direct": 1, "rowwin": 2, "ldstile": 3, "mfma": 4}
_VARIANT_NAMES = {v: k for k, v in VARIANTS.items()}
_DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2, "i8": 3}

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libdwconv.so")

if not os.path.exists(library_path):
    raise ImportError(
        f"{library_path} is missing: build it with "
        "`python -m depthwise_convolution_amd.build` (hipcc, gfx950)")

_lib = ctypes.CDLL(library_path)
_H = ctypes.c_void_p
_I = ctypes.c_int
_lib.dwconv_create.argtypes = [ctypes.POINTER(_H)] + [_I] * 10
_lib.dwconv_create.restype = _I
_lib.dwconv_create_variant.argtypes = [ctypes.POINTER(_H)] + [_I] * 11
_lib.dwconv_create_variant.restype = _I
_lib.dwconv_fwd.argtypes = [_H, _H, _H, _H, _H, _H]
_lib.dwconv_fwd.restype = _I
_lib.dwconv_destroy.argtypes = [_H]
_lib.dwconv_destroy.restype = _I
_lib.dwconv_output_dims.argtypes = [_H, ctypes.POINTER(_I), ctypes.POINTER(_I)]
_lib.dwconv_output_dims.restype = _I
_lib.dwconv_plan_variant.argtypes = [_H]
_lib.dwconv_plan_variant.restype = _I
_lib.dwconv_plan_describe.argtypes = [_H]
_lib.dwconv_plan_describe.restype = ctypes.c_char_p
_lib.dwconv_plan_tile.argtypes = [_H, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
_lib.dwconv_plan_tile.restype = _I
_lib.dwconv_status_string.argtypes = [_I]
_lib.dwconv_status_string.restype = ctypes.c_char_p
_lib.dwconv_fwd_bn_act.argtypes = [_H, _H, _H, _H, _H, _H, _I, _H, _H]
_lib.dwconv_fwd_bn_act.restype = _I
_lib.dwconv_fwd_bn_act_supported.argtypes = [_H]
_lib.dwconv_fwd_bn_act_supported.restype = _I
_lib.dwconv_fwd_bn_act_describe.argtypes = [_H]
_lib.dwconv_fwd_bn_act_describe.restype = ctypes.c_char_p
_lib.dwconv_bwd_data.argtypes = [_H, _H, _H, _H, _H]
_lib.dwconv_bwd_data.restype = _I
_lib.dwconv_bwd_data_supported.argtypes = [_H]
_lib.dwconv_bwd_data_supported.restype = _I
_lib.dwconv_bwd_data_describe.argtypes = [_H]
_lib.dwconv_bwd_data_describe.restype = ctypes.c_char_p
_lib.dwconv_bwd_filter_workspace.argtypes = [_H, ctypes.POINTER(ctypes.c_size_t)]
_lib.dwconv_bwd_filter_workspace.restype = _I
_lib.dwconv_bwd_filter.argtypes = [_H, _H, _H, _H, _H, _H]
_lib.dwconv_bwd_filter.restype = _I
_lib.dwconv_bwd_filter_noalloc.argtypes = [_H, _H, _H, _H, _H]
_lib.dwconv_bwd_filter_noalloc.restype = _I
_lib.dwconv_bwd_filter_describe.argtypes = [_H]
_lib.dwconv_bwd_filter_describe.restype = ctypes.c_char_p


class DwconvError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {dwconv_status_string(status)} (status {status})")


def dwconv_status_string(status: int) -> str:
    return _lib.dwconv_status_string(int(status)).decode()


def _dtype_code(dtype):
    if isinstance(dtype, int):
        return dtype
    if isinstance(dtype, str):
        if dtype not in _DTYPE_CODES:
            raise ValueError(f"unknown dtype {dtype!r}")
        return _DTYPE_CODES[dtype]
    import torch
    m = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2, torch.int8: 3}
    if dtype not in m:
        raise ValueError(f"unsupported dtype {dtype}")
    return m[dtype]


def dwconv_create_variant(N, H, W, C, FH, FW, stride, dilation, pad, dtype, variant):
    """Returns an opaque handle (int); raises DwconvError on a bad shape."""
    h = _H()
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    rc = _lib.dwconv_create_variant(ctypes.byref(h), N, H, W, C, FH, FW, stride,
                                    dilation, pad, _dtype_code(dtype), v)
    if rc != 0:
        raise DwconvError(rc, "dwconv_create")
    return h.value


def dwconv_create(N, H, W, C, FH, FW, stride, dilation, pad, dtype):
    return dwconv_create_variant(N, H, W, C, FH, FW, stride, dilation, pad, dtype, 0)


def dwconv_destroy(h) -> None:
    _lib.dwconv_destroy(h)


def dwconv_output_dims(h):
    oh, ow = _I(), _I()
    rc = _lib.dwconv_output_dims(h, ctypes.byref(oh), ctypes.byref(ow))
    if rc != 0:
        raise DwconvError(rc, "dwconv_output_dims")
    return oh.value, ow.value


def dwconv_plan_variant(h) -> str:
    return _VARIANT_NAMES.get(_lib.dwconv_plan_variant(h), "?")


def dwconv_plan_describe(h) -> str:
    return _lib.dwconv_plan_describe(h).decode()


def dwconv_plan_tile(h):
    """(rows, columns, channels) of the output tile whose input span the
    forward kernel fetches as one piece."""
    th, tw, tc = _I(), _I(), _I()
    rc = _lib.dwconv_plan_tile(h, ctypes.byref(th), ctypes.byref(tw), ctypes.byref(tc))
    if rc != 0:
        raise DwconvError(rc, "dwconv_plan_tile")
    return th.value, tw.value, tc.value


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous (channel-last as laid out)")
    return t.data_ptr()


def _stream(stream, like):
    if stream is None:
        import torch
        dev = like.device if hasattr(like, "device") else None
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def dwconv_fwd(h, x, w, bias, y, stream=None) -> None:
    """Enqueues the forward pass.  x, w, bias, y: GPU tensors (or raw device
    pointers as ints); bias may be None.  ``stream``: torch stream, raw
    hipStream_t int, or None for torch's current stream."""
    rc = _lib.dwconv_fwd(h, _ptr(x), _ptr(w), _ptr(bias), _ptr(y), _stream(stream, x))
    if rc != 0:
        raise DwconvError(rc, "dwconv_fwd")


ACTIVATIONS = {"none": 0, "relu": 1, "relu6": 2}


def dwconv_fwd_bn_act(h, x, w, bias, bn_scale, bn_shift, act, y, stream=None) -> None:
    """Enqueues the forward pass of act(x * bn_scale + bn_shift) (the fused
    batch-normalization + activation prologue): bn_scale and bn_shift are C
    float32 GPU tensors (or device pointers); ``act`` is "none", "relu",
    "relu6" or its number.  Other arguments as for ``dwconv_fwd``."""
    a = ACTIVATIONS[act] if isinstance(act, str) else int(act)
    rc = _lib.dwconv_fwd_bn_act(h, _ptr(x), _ptr(w), _ptr(bias), _ptr(bn_scale), _ptr(bn_shift),
                                a, _ptr(y), _stream(stream, x))
    if rc != 0:
        raise DwconvError(rc, "dwconv_fwd_bn_act")


def dwconv_fwd_bn_act_supported(h) -> bool:
    return bool(_lib.dwconv_fwd_bn_act_supported(h))


def dwconv_fwd_bn_act_describe(h) -> str:
    return _lib.dwconv_fwd_bn_act_describe(h).decode()


def dwconv_bwd_data(h, dy, w, dx, stream=None) -> None:
    """Enqueues the backward-data pass: dx (N x H x W x C) from dy
    (N x OH x OW x C) and the forward filter w.  Tensors or raw device
    pointers; ``stream`` as for ``dwconv_fwd``.  Raises DwconvError
    (unsupported) where the plan has no backward-data pass."""
    rc = _lib.dwconv_bwd_data(h, _ptr(dy), _ptr(w), _ptr(dx), _stream(stream, dy))
    if rc != 0:
        raise DwconvError(rc, "dwconv_bwd_data")


def dwconv_bwd_data_supported(h) -> bool:
    return bool(_lib.dwconv_bwd_data_supported(h))


def dwconv_bwd_data_describe(h) -> str:
    return _lib.dwconv_bwd_data_describe(h).decode()


def dwconv_bwd_filter_workspace(h) -> int:
    """Bytes of workspace dwconv_bwd_filter needs for this plan."""
    n = ctypes.c_size_t()
    rc = _lib.dwconv_bwd_filter_workspace(h, ctypes.byref(n))
    if rc != 0:
        raise DwconvError(rc, "dwconv_bwd_filter_workspace")
    return n.value


def dwconv_bwd_filter(h, x, dy, dw, workspace, stream=None) -> None:
    """Enqueues the backward-filter pass: dw (FH x FW x C, float32) from x and
    dy; ``workspace`` holds at least dwconv_bwd_filter_workspace(h) bytes."""
    rc = _lib.dwconv_bwd_filter(h, _ptr(x), _ptr(dy), _ptr(dw), _ptr(workspace),
                                _stream(stream, x))
    if rc != 0:
        raise DwconvError(rc, "dwconv_bwd_filter")


def dwconv_bwd_filter_noalloc(h, x, dy, dw, stream=None) -> None:
    """dwconv_bwd_filter with the library's own scratch array as the workspace
    (no allocation); DwconvError status 5 when the plan's workspace exceeds
    DWCONV_SCRATCH_BYTES.  Calls that overlap on one GPU share the array."""
    rc = _lib.dwconv_bwd_filter_noalloc(h, _ptr(x), _ptr(dy), _ptr(dw), _stream(stream, x))
    if rc != 0:
        raise DwconvError(rc, "dwconv_bwd_filter_noalloc")


def dwconv_bwd_filter_describe(h) -> str:
    return _lib.dwconv_bwd_filter_describe(h).decode()


class DepthwiseConv2d:
    """Owns a plan; ``conv(x, w, bias)`` allocates y with torch and runs the
    kernel.  x: N x H x W x C, w: FH x FW x C, bias: C (fp32, or int32 for
    int8) or None."""

    _TORCH_Y = {0: "float32", 1: "float16", 2: "bfloat16", 3: "int32"}

    def __init__(self, N, H, W, C, FH, FW, stride=1, dilation=1, pad=0, dtype="f32",
                 variant="auto"):
        self.shape = (N, H, W, C, FH, FW, stride, dilation, pad)
        self.dtype = _dtype_code(dtype)
        self.handle = dwconv_create_variant(N, H, W, C, FH, FW, stride, dilation, pad,
                                            self.dtype, variant)
        self.OH, self.OW = dwconv_output_dims(self.handle)

    @property
    def variant(self):
        return dwconv_plan_variant(self.handle)

    def describe(self):
        return dwconv_plan_describe(self.handle)

    def __call__(self, x, w, bias=None, y=None, stream=None):
        import torch
        N, _, _, C = self.shape[:4]
        if y is None:
            y = torch.empty((N, self.OH, self.OW, C), device=x.device,
                            dtype=getattr(torch, self._TORCH_Y[self.dtype]))
        dwconv_fwd(self.handle, x, w, bias, y, stream)
        return y

    def forward_bn_act(self, x, w, bn_scale, bn_shift, act="relu", bias=None, y=None,
                       stream=None):
        """y = conv(act(x * bn_scale + bn_shift)) with the prologue fused."""
        import torch
        N, _, _, C = self.shape[:4]
        if y is None:
            y = torch.empty((N, self.OH, self.OW, C), device=x.device,
                            dtype=getattr(torch, self._TORCH_Y[self.dtype]))
        dwconv_fwd_bn_act(self.handle, x, w, bias, bn_scale, bn_shift, act, y, stream)
        return y

    def backward_data(self, dy, w, dx=None, stream=None):
        """dx = the input gradient for output gradient dy (dtype of x)."""
        import torch
        N, H, W, C = self.shape[:4]
        if dx is None:
            dx = torch.empty((N, H, W, C), device=dy.device, dtype=dy.dtype)
        dwconv_bwd_data(self.handle, dy, w, dx, stream)
        return dx

    def backward_filter(self, x, dy, dw=None, workspace=None, stream=None):
        """dw (FH x FW x C, float32) = the filter gradient for input x and
        output gradient dy; allocates dw and the workspace with torch when
        they are not given."""
        import torch
        FH, FW = self.shape[4], self.shape[5]
        C = self.shape[3]
        if dw is None:
            dw = torch.empty((FH, FW, C), device=x.device, dtype=torch.float32)
        if workspace is None:
            workspace = torch.empty(dwconv_bwd_filter_workspace(self.handle), device=x.device,
                                    dtype=torch.uint8)
        dwconv_bwd_filter(self.handle, x, dy, dw, workspace, stream)
        return dw

    def close(self):
        if self.handle:
            dwconv_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
