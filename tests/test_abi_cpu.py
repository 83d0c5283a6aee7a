"""The C ABI on the CPU: the library loads without a GPU, exports every entry
point the header declares, and validates arguments before touching the GPU.
No test here launches a kernel."""
import ctypes
import os
import re

import numpy as np
import pytest

import depthwise_convolution_amd as dw
from synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            text = open(os.path.join(ROOT, "include", f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(dwconv_\w+)\s*\(", text))
    return names


def test_header_symbols_exported():
    names = declared_functions()
    assert {"dwconv_create", "dwconv_fwd", "dwconv_destroy"} <= names
    lib = ctypes.CDLL(dw.library_path)
    for n in sorted(names):
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
        assert hasattr(dw, n), f"{n} has no Python binding of the same name"


def test_status_strings():
    assert dw.dwconv_status_string(0) == "ok"
    assert dw.dwconv_status_string(1) == "invalid argument"
    assert dw.dwconv_status_string(99) == "unknown status"


@pytest.mark.parametrize("args", [
    (0, 8, 8, 4, 3, 3, 1, 1, 1),     # N < 1
    (1, 0, 8, 4, 3, 3, 1, 1, 1),     # H < 1
    (1, 8, 8, 0, 3, 3, 1, 1, 1),     # C < 1
    (1, 8, 8, 4, 0, 3, 1, 1, 1),     # FH < 1
    (1, 8, 8, 4, 3, 3, 0, 1, 1),     # stride < 1
    (1, 8, 8, 4, 3, 3, 1, 0, 1),     # dilation < 1
    (1, 8, 8, 4, 3, 3, 1, 1, -1),    # pad < 0
    (1, 2, 8, 4, 5, 3, 1, 1, 0),     # empty output (filter taller than input)
    (1, 8, 8, 4, 3, 3, 1, 4, 0),     # dilated span exceeds the input
    (65536, 256, 256, 64, 3, 3, 1, 1, 1),  # 2^38 elements
])
def test_create_rejects(args):
    with pytest.raises(dw.DwconvError) as e:
        dw.dwconv_create(*args, "f32")
    assert e.value.status == 1


def test_create_rejects_dtype_and_variant():
    for bad in (4, -1, 17):
        with pytest.raises(dw.DwconvError) as e:
            dw.dwconv_create(1, 8, 8, 4, 3, 3, 1, 1, 1, bad)
        assert e.value.status == 1
    with pytest.raises(dw.DwconvError) as e:
        dw.dwconv_create_variant(1, 8, 8, 4, 3, 3, 1, 1, 1, "f32", 9)
    assert e.value.status == 1
    # int8 filters whose products alone could overflow int32
    with pytest.raises(dw.DwconvError):
        dw.dwconv_create(1, 400, 400, 1, 363, 363, 1, 1, 181, "i8")


def test_create_null_out_pointer():
    lib = ctypes.CDLL(dw.library_path)
    lib.dwconv_create.argtypes = [ctypes.c_void_p] + [ctypes.c_int] * 10
    assert lib.dwconv_create(None, 1, 8, 8, 4, 3, 3, 1, 1, 1, 0) == 1


def test_output_dims_and_plan():
    h = dw.dwconv_create(16, 112, 112, 61, 5, 5, 2, 2, 4, "i8")
    try:
        assert dw.dwconv_output_dims(h) == (56, 56)
        assert dw.dwconv_plan_variant(h) in dw.VARIANTS
        assert dw.dwconv_plan_describe(h)
    finally:
        dw.dwconv_destroy(h)
    h = dw.dwconv_create(1, 16, 16, 8, 3, 3, 1, 1, 1, "f32")
    assert dw.dwconv_output_dims(h) == (16, 16)
    dw.dwconv_destroy(h)
    dw.dwconv_destroy(None)          # no-op


@pytest.mark.parametrize("shape,fmt,variant,tile", [
    ((64, 56, 56, 128, 3, 3, 1, 1, 1), "f32", "auto", (14, 4, 4)),     # column stream
    ((64, 56, 56, 96, 7, 7, 1, 1, 3), "f16", "auto", (56, 32, 8)),     # matrix-core strip
    ((16, 112, 112, 61, 5, 5, 2, 2, 4), "i8", "auto", (7, 16, 61)),    # int8 LDS tile
    ((2, 20, 20, 16, 5, 5, 1, 1, 2), "f32", "rowwin", (16, 4, 2)),     # column stream 5x5
    ((2, 20, 20, 16, 7, 7, 1, 1, 3), "f16", "rowwin", (1, 4, 8)),      # row window
    ((2, 20, 20, 16, 11, 11, 1, 1, 5), "f32", "rowwin", (1, 12, 4)),   # row chunks
    ((2, 9, 7, 5, 4, 2, 3, 2, 1), "bf16", "direct", (1, 1, 1)),
])
def test_plan_tile(shape, fmt, variant, tile):
    """The tile whose input span the forward kernel fetches as one piece,
    as the plan's description states it."""
    h = dw.dwconv_create_variant(*shape, fmt, variant)
    try:
        got = dw.dwconv_plan_tile(h)
        desc = dw.dwconv_plan_describe(h)
    finally:
        dw.dwconv_destroy(h)
    assert all(t is None or t == g for t, g in zip(tile, got)), (got, desc)
    assert min(got) >= 1
    if desc.startswith(("rowwin", "rowchunk", "colstream")):
        assert f"VEC={got[2]} " in desc and f"TM={got[1]} " in desc, desc
    with pytest.raises(dw.DwconvError):
        lib = ctypes.CDLL(dw.library_path)
        lib.dwconv_plan_tile.argtypes = [ctypes.c_void_p] * 4
        rc = lib.dwconv_plan_tile(None, None, None, None)
        raise dw.DwconvError(rc, "dwconv_plan_tile") if rc == 1 else AssertionError(rc)


@pytest.mark.parametrize("shape,fmt,block", [
    ((64, 56, 56, 128, 3, 3, 1, 1, 1), "f32", 64),
    ((4, 30, 30, 64, 9, 9, 1, 1, 4), "f32", 64),
    ((64, 56, 56, 128, 3, 3, 1, 1, 1), "f16", 256),
    ((4, 30, 30, 64, 3, 3, 1, 1, 1), "bf16", 256),
])
def test_column_stream_launch_shape(shape, fmt, block):
    """fp32 column streams launch one-wavefront workgroups, fp16/bf16 ones
    four-wavefront groups; either way the grid covers every lane's strip
    (channel vectors x column strips x row bands x images) exactly once."""
    h = dw.dwconv_create(*shape, fmt)
    try:
        desc = dw.dwconv_plan_describe(h)
        th, tm, vec = dw.dwconv_plan_tile(h)
    finally:
        dw.dwconv_destroy(h)
    assert desc.startswith("colstream"), desc
    N, H, W, C = shape[:4]
    lanes = (C // vec) * -(-W // tm) * -(-H // th) * N
    assert desc.endswith(f"{-(-lanes // block)} x {block}"), (desc, lanes)


@pytest.mark.parametrize("shape,family", [
    ((64, 56, 56, 96, 5, 5, 1, 1, 2), "colstream: VEC=2"),
    ((128, 64, 64, 256, 5, 5, 1, 1, 2), "colstream: VEC=2 ch/lane, TM=4 x TH=14"),
    ((16, 112, 112, 64, 5, 5, 1, 1, 2), "colstream: VEC=2 ch/lane, TM=4 x TH=14"),
    ((16, 112, 112, 64, 5, 5, 1, 1, 2), "colstream: VEC=2"),
    ((2, 30, 30, 32, 5, 5, 1, 1, 2), "mfma"),      # few lanes: the matrix cores
    ((64, 56, 56, 96, 5, 5, 1, 1, 2, "bf16"), "mfma"),  # bf16 stays on the matrix cores
    ((64, 56, 56, 96, 7, 7, 1, 1, 3), "mfma"),
])
def test_fp16_5x5_family(shape, family):
    """fp16 5x5 at stride 1 on a map of at least 64K lanes runs the column
    stream with paired taps; smaller maps, other filters and bf16 keep their
    families."""
    fmt = shape[9] if len(shape) > 9 else "f16"
    h = dw.dwconv_create(*shape[:9], fmt)
    try:
        desc = dw.dwconv_plan_describe(h)
    finally:
        dw.dwconv_destroy(h)
    assert desc.startswith(family), desc


def test_forced_variants():
    # the direct family takes every shape
    h = dw.dwconv_create_variant(2, 9, 7, 5, 4, 2, 3, 2, 1, "bf16", "direct")
    assert dw.dwconv_plan_variant(h) == "direct"
    dw.dwconv_destroy(h)
    # a family that cannot run the shape is reported, not substituted
    with pytest.raises(dw.DwconvError) as e:
        dw.dwconv_create_variant(2, 9, 7, 5, 4, 2, 3, 2, 1, "bf16", "rowwin")
    assert e.value.status == 2


def test_fwd_argument_errors_before_any_launch():
    lib = ctypes.CDLL(dw.library_path)
    V = ctypes.c_void_p
    lib.dwconv_fwd.argtypes = [V] * 6
    h = dw.dwconv_create(1, 8, 8, 4, 3, 3, 1, 1, 1, "f32")
    try:
        fake = 0x1000
        assert lib.dwconv_fwd(None, fake, fake, None, fake, None) == 1
        assert lib.dwconv_fwd(h, None, fake, None, fake, None) == 1
        assert lib.dwconv_fwd(h, fake, None, None, fake, None) == 1
        assert lib.dwconv_fwd(h, fake, fake, None, None, None) == 1
        lib.dwconv_output_dims.argtypes = [V, V, V]
        assert lib.dwconv_output_dims(None, None, None) == 1
    finally:
        dw.dwconv_destroy(h)


def test_one_hip_runtime_in_process():
    """The library binds to the HIP/HSA runtime torch loaded: one copy of
    each in the process, so torch's pointers and streams are valid in it."""
    maps = open("/proc/self/maps").read().splitlines()
    hip = {l.split()[-1] for l in maps if "libamdhip64" in l}
    hsa = {l.split()[-1] for l in maps if "libhsa-runtime64" in l}
    assert len(hip) == 1 and len(hsa) == 1, (hip, hsa)


def test_bwd_data_support_matrix():
    """Which forward plans carry a backward-data pass (host only, no GPU)."""
    cases = [((2, 9, 9, 8, 3, 3, 1, 1, 1, "f32"), True),
             ((2, 9, 9, 8, 7, 7, 1, 1, 3, "f16"), True),
             ((1, 20, 20, 16, 31, 31, 1, 1, 15, "bf16"), True),
             ((2, 9, 9, 8, 3, 3, 1, 2, 0, "f32"), True),     # dilated, no padding
             ((2, 9, 9, 8, 3, 3, 2, 1, 1, "f32"), "direct"),    # stride 2
             ((2, 9, 9, 8, 3, 5, 1, 1, 1, "f16"), "direct"),    # not square
             ((2, 9, 9, 8, 3, 3, 1, 1, 3, "bf16"), "direct"),   # pad > D(F-1)
             ((2, 9, 9, 8, 3, 3, 1, 1, 1, "i8"), False)]        # int8
    for (N, H, W, C, FH, FW, S, D, P, dt), want in cases:
        h = dw.dwconv_create(N, H, W, C, FH, FW, S, D, P, dt)
        try:
            shape = (N, H, W, C, FH, FW, S, D, P, dt)
            assert dw.dwconv_bwd_data_supported(h) == bool(want), shape
            desc = dw.dwconv_bwd_data_describe(h)
            assert bool(desc) == bool(want), shape
            # the forward families serve stride 1 with square filters; the
            # direct backward kernel everything else
            assert desc.startswith("direct (backward data)") == (want == "direct"), (shape, desc)
        finally:
            dw.dwconv_destroy(h)


def test_bwd_data_argument_errors():
    """NULL arguments and unsupported plans are refused before any launch."""
    lib = dw._lib
    h = dw.dwconv_create(1, 8, 8, 4, 3, 3, 1, 1, 1, "i8")    # int8: no bwd pass
    g = dw.dwconv_create(1, 8, 8, 4, 3, 3, 1, 1, 1, "f32")
    try:
        fake = 1 << 40   # never dereferenced: every path below returns first
        assert lib.dwconv_bwd_data(None, fake, fake, fake, None) == 1
        assert lib.dwconv_bwd_data(g, None, fake, fake, None) == 1
        assert lib.dwconv_bwd_data(g, fake, None, fake, None) == 1
        assert lib.dwconv_bwd_data(g, fake, fake, None, None) == 1
        assert lib.dwconv_bwd_data(h, fake, fake, fake, None) == 2
        assert dw.dwconv_bwd_data_supported(None) is False
        assert dw.dwconv_bwd_data_describe(None) == ""
    finally:
        dw.dwconv_destroy(h)
        dw.dwconv_destroy(g)


def test_bwd_filter_workspace_and_errors():
    """Workspace sizes and argument errors of the backward-filter pass (host
    only: every call below returns before any launch)."""
    lib = dw._lib
    h = dw.dwconv_create(2, 9, 9, 8, 3, 3, 1, 1, 1, "f32")
    q = dw.dwconv_create(2, 9, 9, 8, 3, 3, 1, 1, 1, "i8")
    try:
        n = dw.dwconv_bwd_filter_workspace(h)
        assert n > 0 and n % (3 * 3 * 8 * 4) == 0
        assert dw.dwconv_bwd_filter_describe(h).startswith("bwf")
        with pytest.raises(dw.DwconvError):
            dw.dwconv_bwd_filter_workspace(q)
        assert dw.dwconv_bwd_filter_describe(q) == ""
        fake = 1 << 40
        assert lib.dwconv_bwd_filter(h, None, fake, fake, fake, None) == 1
        assert lib.dwconv_bwd_filter(h, fake, fake, fake, None, None) == 1
        assert lib.dwconv_bwd_filter(h, fake, fake, fake + 2, fake, None) == 1   # dw misaligned
        assert lib.dwconv_bwd_filter(q, fake, fake, fake, fake, None) == 2
    finally:
        dw.dwconv_destroy(h)
        dw.dwconv_destroy(q)


def test_tuning_switch(monkeypatch):
    """DWCONV_TUNE (read at plan creation, host only): keys pick a compiled
    alternative, unknown keys and malformed entries are ignored, and a tiling
    no compiled kernel provides makes the forced family unsupported."""
    shape = (32, 56, 56, 128, 31, 31, 1, 1, 15)

    def desc(variant="auto"):
        h = dw.dwconv_create_variant(*shape, "bf16", variant)
        try:
            return dw.dwconv_plan_describe(h)
        finally:
            dw.dwconv_destroy(h)
    monkeypatch.delenv("DWCONV_TUNE", raising=False)
    assert "strips of 64 cols" in desc()
    monkeypatch.setenv("DWCONV_TUNE", "nothing=1,mfma_nb=2")
    assert "strips of 32 cols" in desc()
    monkeypatch.setenv("DWCONV_TUNE", "mfma_al=0")
    assert "DPP row shift" in desc()
    monkeypatch.setenv("DWCONV_TUNE", "bogus,mfma_nb")
    assert "strips of 64 cols" in desc()
    monkeypatch.setenv("DWCONV_TUNE", "tile=99x99")
    with pytest.raises(dw.DwconvError) as e:
        dw.dwconv_create_variant(64, 56, 56, 128, 3, 3, 1, 1, 1, "f32", "rowwin")
    assert e.value.status == 2


def test_bwd_filter_noalloc_errors():
    """The no-allocation filter gradient refuses, before touching the GPU, a
    plan whose workspace exceeds the library's scratch array, and NULL or
    misaligned arguments and int8 plans like dwconv_bwd_filter."""
    lib = dw._lib
    big = dw.dwconv_create(128, 128, 128, 128, 31, 31, 1, 1, 15, "f16")
    h = dw.dwconv_create(2, 9, 9, 8, 3, 3, 1, 1, 1, "f32")
    q = dw.dwconv_create(2, 9, 9, 8, 3, 3, 1, 1, 1, "i8")
    try:
        assert dw.dwconv_bwd_filter_workspace(big) > dw.DWCONV_SCRATCH_BYTES
        assert dw.dwconv_bwd_filter_workspace(h) <= dw.DWCONV_SCRATCH_BYTES
        fake = 1 << 40
        assert lib.dwconv_bwd_filter_noalloc(big, fake, fake, fake, None) == 5
        assert dw.dwconv_status_string(5) == "workspace larger than the library's scratch array"
        assert lib.dwconv_bwd_filter_noalloc(None, fake, fake, fake, None) == 1
        assert lib.dwconv_bwd_filter_noalloc(h, None, fake, fake, None) == 1
        assert lib.dwconv_bwd_filter_noalloc(h, fake, fake, None, None) == 1
        assert lib.dwconv_bwd_filter_noalloc(h, fake, fake, fake + 2, None) == 1  # dw misaligned
        assert lib.dwconv_bwd_filter_noalloc(q, fake, fake, fake, None) == 2
        # the five workloads' filter gradients fit the array
        for wl in WORKLOADS.values():
            if wl.dtype == "i8":
                continue
            g = dw.dwconv_create(wl.N, wl.H, wl.W, wl.C, wl.FH, wl.FW, wl.stride,
                                 wl.dilation, wl.pad, wl.dtype)
            try:
                assert dw.dwconv_bwd_filter_workspace(g) <= dw.DWCONV_SCRATCH_BYTES, wl.name
            finally:
                dw.dwconv_destroy(g)
    finally:
        for x in (big, h, q):
            dw.dwconv_destroy(x)


def test_fwd_bn_act_support_and_errors():
    """The fused-prologue forward pass: supported for float plans, not int8;
    NULL arguments and unknown activations are refused before any launch."""
    lib = dw._lib
    g = dw.dwconv_create(1, 8, 8, 4, 3, 3, 1, 1, 1, "f32")
    i = dw.dwconv_create(1, 8, 8, 4, 3, 3, 1, 1, 1, "i8")
    try:
        assert dw.dwconv_fwd_bn_act_supported(g) and not dw.dwconv_fwd_bn_act_supported(i)
        assert dw.dwconv_fwd_bn_act_describe(g) and dw.dwconv_fwd_bn_act_describe(i) == ""
        fake = 1 << 40   # never dereferenced: every call below returns first
        ok = (g, fake, fake, None, fake, fake, 1, fake, None)
        for k in (0, 1, 2, 4, 5, 7):   # handle, x, w, bn_scale, bn_shift, y
            args = list(ok)
            args[k] = None
            assert lib.dwconv_fwd_bn_act(*args) == 1, k
        for bad in (-1, 3, 7):
            args = list(ok)
            args[6] = bad
            assert lib.dwconv_fwd_bn_act(*args) == 1, bad
        args = list(ok)
        args[0] = i
        assert lib.dwconv_fwd_bn_act(*args) == 2
        assert dw.dwconv_fwd_bn_act_supported(None) is False
    finally:
        dw.dwconv_destroy(g)
        dw.dwconv_destroy(i)


def test_plans_from_many_host_threads():
    """Plans are host-side and immutable: creating, describing and
    destroying them from several threads at once gives each thread the same
    answers as a single thread."""
    import threading
    shapes = [((64, 56, 56, 128, 3, 3, 1, 1, 1), "f32"), ((64, 56, 56, 96, 7, 7, 1, 1, 3), "f16"),
              ((32, 56, 56, 128, 31, 31, 1, 1, 15), "bf16"), ((16, 112, 112, 61, 5, 5, 2, 2, 4), "i8"),
              ((2, 9, 7, 5, 4, 2, 3, 2, 1), "bf16")]

    def describe(shape, fmt):
        h = dw.dwconv_create(*shape, fmt)
        try:
            return (dw.dwconv_plan_describe(h), dw.dwconv_plan_tile(h), dw.dwconv_output_dims(h),
                    dw.dwconv_bwd_data_describe(h), dw.dwconv_bwd_filter_describe(h),
                    dw.dwconv_fwd_bn_act_describe(h))
        finally:
            dw.dwconv_destroy(h)

    want = [describe(*c) for c in shapes]
    errors = []

    def worker(k):
        try:
            for r in range(50):
                i = (k + r) % len(shapes)
                got = describe(*shapes[i])
                if got != want[i]:
                    errors.append((k, r, got, want[i]))
        except Exception as e:  # noqa: BLE001 -- reported below
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors[:3]


@pytest.mark.parametrize("shape,fmt,family", [
    ((64, 56, 56, 96, 7, 7, 1, 1, 3), "f16", "mfma with the prologue fused"),
    ((32, 56, 56, 128, 31, 31, 1, 1, 15), "bf16", "mfma with the prologue fused"),
    ((1, 20, 20, 16, 41, 41, 1, 1, 20), "f16", "rowchunk"),      # three fragments: VALU
    ((64, 56, 56, 128, 3, 3, 1, 1, 1), "f32", "colstream"),
    ((16, 112, 112, 61, 5, 5, 2, 2, 4), "f16", "direct"),        # no 16-byte vectors
])
def test_fused_prologue_family(shape, fmt, family):
    """Which kernel runs the fused-prologue pass: the forward family where
    it fuses the prologue -- on the matrix cores the forward plan's own
    tiling, with U rounded to the data's format as the ring is written --
    else a vector kernel."""
    h = dw.dwconv_create(*shape, fmt)
    try:
        desc = dw.dwconv_fwd_bn_act_describe(h)
        fwd = dw.dwconv_plan_describe(h)
    finally:
        dw.dwconv_destroy(h)
    assert desc.startswith(family), desc
    if family.startswith("mfma"):
        assert ("U rounded to fp16" if fmt == "f16" else "U rounded to bf16") in desc, desc
        tiling = fwd.split("banded GEMM, ", 1)[1].split(" walked", 1)[0]
        assert tiling in desc, (tiling, desc)


def test_counter_hash_ignores_comments_only():
    """The stored counter figures are keyed by a hash of the kernel sources'
    code: comments and layout do not change it, code and string literals do."""
    import bench
    src = 'int a = 1; // x\n/* y */ const char *s = "p // q /* r */";'
    assert bench.code_only(src) == 'int a = 1; const char *s = "p // q /* r */";'
    assert bench.code_only("int  a =\n 1; /* z */") == bench.code_only("int a = 1;")
    assert bench.code_only("int a = 1;") != bench.code_only("int a = 2;")
    assert bench.code_only('f("a");') != bench.code_only('f("b");')


def test_algorithmic_bytes_count_touched_inputs():
    """The bench's algorithmic bytes count the input elements some tap reads
    (unique bytes, "Tiles, halos and partial sums"): all of x for the
    stride-1 "same" layers, the even rows and columns -- 56 of 112 each --
    for the stride-2, dilation-2 5x5 int8 layer; brute force over a small
    strided shape agrees with the per-axis count."""
    import bench
    from synth import WORKLOADS
    for name in ("tiny_f32_3x3", "mobilenet_f32_3x3", "convnext_f16_7x7",
                 "largekernel_bf16_31x31"):
        wl = WORKLOADS[name]
        nbytes, _, OH, OW = bench.work(wl)
        x = wl.N * wl.H * wl.W * wl.C * bench.XB[wl.dtype]
        y = wl.N * OH * OW * wl.C * bench.YB[wl.dtype]
        assert nbytes == x + y + wl.FH * wl.FW * wl.C * bench.XB[wl.dtype] + wl.C * 4, name
    wl = WORKLOADS["strided_i8_5x5"]
    assert bench.touched(112, 56, 5, 2, 2, 4) == 56
    nbytes, _, OH, OW = bench.work(wl)
    assert nbytes == 16 * 56 * 56 * 61 + 16 * 56 * 56 * 61 * 4 + 25 * 61 + 61 * 4
    # brute force: mark every (ih, iw) some output's tap reads
    H, W, F, S, D, P = 11, 9, 3, 3, 2, 1
    OH = (H + 2 * P - D * (F - 1) - 1) // S + 1
    OW = (W + 2 * P - D * (F - 1) - 1) // S + 1
    hit = np.zeros((H, W), bool)
    for oh in range(OH):
        for ow in range(OW):
            for fh in range(F):
                for fw in range(F):
                    ih, iw = oh * S - P + fh * D, ow * S - P + fw * D
                    if 0 <= ih < H and 0 <= iw < W:
                        hit[ih, iw] = True
    assert hit.sum() == bench.touched(H, OH, F, S, D, P) * bench.touched(W, OW, F, S, D, P)
