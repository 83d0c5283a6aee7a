#!/usr/bin/env python3
"""Throughput of the forward depthwise convolution on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--variant auto|direct|rowwin|ldstile|mfma]
                    [--op fwd|bwd_data|bwd_filter|fwd_bn_act]
                    [--launch graph|eager] [--no-cpu] [--no-copy]

A step is one forward pass (one launch of the library's kernel) over one batch
of seeded synthetic input, launched back to back (--launch graph also captures
the K timed steps into one HIP graph and replays it).  Before each timed pass
the bench runs about 300 ms of untimed steps (--clock-ms): the GPU's clocks rise over the
first tens of milliseconds of sustained load (a compute-bound layer's launches
start about 20 % slower than they settle), and the timed steps are meant to
see the sustained state.  The inputs are copied to HBM before timing.  So
that no step finds its input in the 256 MB Infinity Cache (MALL) or in L2
from an earlier step, the bench keeps several copies of x and y, at least
1 GiB in all, and steps walk through them in turn.

Prints one JSON line.  The top-level fields are the named workload's (by
default the fp32 3x3 MobileNet-shaped layer); with no --workload, --op or
--variant the line also holds "workloads": the same record for each of the
five workloads (tiny fp32 3x3, MobileNet fp32 3x3, ConvNeXt fp16 7x7,
large-kernel bf16 31x31, strided int8 5x5), timed in the same run.
  value           algorithmic GB/s of K back-to-back steps (bytes / time per step)
  launch, graph   how the timed steps were launched; the graph replay's and
                  the eager launches' average per step
  roofline        the kernel's average duration (HIP events around the K
                  back-to-back steps, one launch each) against the roof that
                  binds it -- MI355X's 8 TB/s HBM, or for compute-bound
                  filters the matrix-core / VALU peak of the units it uses --
                  plus the HBM bytes per launch that the rocprofv3
                  FETCH_SIZE / WRITE_SIZE counters measured for this kernel,
                  scaled by what they read for a plain copy of known size
                  (profiles/counters.json; null once the sources changed)
  kernel          plan, average, and the spread of single launches (a second
                  pass with an event pair around each launch: mean, median,
                  min, p90; each pair adds the event packets' own time)
  copy_ceiling    a hand-written HBM copy (depthwise_convolution_amd/ceiling,
                  four 16-byte loads in flight per lane, non-temporal stores)
                  of the same byte count, back to back; torch_copy is torch's
                  device-to-device copy timed the same way
  cpu_baseline    the CPU oracle timed on this host's cores on a sample
Algorithmic bytes count the input elements some tap reads (all of x at
stride 1), w, bias and y once each; halo re-reads and padding are not
counted.  FLOPs are 2 per tap per output.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "depthwise-conv fwd GB/s + GFLOP/s and fraction of HBM roofline, 1 MI355X"
METRIC_BWD = ("depthwise-conv bwd-data GB/s + GFLOP/s and fraction of HBM roofline, "
              "1 MI355X")
METRIC_BWF = ("depthwise-conv bwd-filter GB/s + GFLOP/s and fraction of HBM roofline, "
              "1 MI355X")
METRIC_BNACT = ("depthwise-conv fwd with fused BN+ReLU prologue GB/s + GFLOP/s and fraction "
                "of HBM roofline, 1 MI355X")
DEFAULT_WORKLOAD = "mobilenet_f32_3x3"
HBM_PEAK_GBS = 8000.0
# Published dense peaks of MI355X used for compute-bound kernels.  The VALU
# figure is the fp32 FMA rate without packed-FP32 instructions (all HIP code
# here is built with them disabled): 256 CUs x 4 SIMDs x 16 lanes x 2 flop x
# 2.4 GHz = 78.6 TFLOP/s; int32 multiply-add runs at the same rate.
MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}
VALU_PEAK_TFLOPS = 78.6
# Vector dot-product instructions do more per lane and cycle, at the same
# issue rate: v_dot2_f32_{f16,bf16} two multiply-adds (4 flop), v_dot4_i32_i8
# four (8 ops): 157.3 TFLOP/s and 314.6 TOP/s over the chip.
VALU_PEAKS = {"fma": VALU_PEAK_TFLOPS, "dot2": 2 * VALU_PEAK_TFLOPS,
              "dot4": 4 * VALU_PEAK_TFLOPS}
MAX_BUFFER_SETS = 64
MALL_FLUSH_BYTES = 1 << 30
XB = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1}
YB = {"f32": 4, "f16": 2, "bf16": 2, "i8": 4}


def out_extent(size, f, s, d, p):
    return (size + 2 * p - d * (f - 1) - 1) // s + 1


def touched(size, out, f, s, d, p):
    """Input positions along one axis that at least one tap of one output
    reads: oh*S - P + fh*D inside [0, size)."""
    return len({o * s - p + k * d for o in range(out) for k in range(f)} & set(range(size)))


def work(wl):
    """(algorithmic bytes, flops, OH, OW) of one forward pass.  The bytes are
    the unique tensor bytes the operation must move ("Tiles, halos and partial
    sums": unique bytes are the lower bound): the input elements that some
    tap reads (all of x at stride 1; at stride 2 and dilation 2 only the even
    rows and columns), w, bias and y, each once."""
    OH = out_extent(wl.H, wl.FH, wl.stride, wl.dilation, wl.pad)
    OW = out_extent(wl.W, wl.FW, wl.stride, wl.dilation, wl.pad)
    rows = touched(wl.H, OH, wl.FH, wl.stride, wl.dilation, wl.pad)
    cols = touched(wl.W, OW, wl.FW, wl.stride, wl.dilation, wl.pad)
    xb = wl.N * rows * cols * wl.C * XB[wl.dtype]
    wb = wl.FH * wl.FW * wl.C * XB[wl.dtype]
    bb = wl.C * 4 if wl.b_dist is not None else 0
    yb = wl.N * OH * OW * wl.C * YB[wl.dtype]
    flops = 2 * wl.N * OH * OW * wl.C * wl.FH * wl.FW
    return xb + wb + bb + yb, flops, OH, OW


def tile_model(wl, tile, OH, OW):
    """HBM bytes if every tile fetched its own input span and filter slice
    from HBM, plus y once: the depthwise form of the tiled-GEMM traffic model
    (a Th x Tw x Tc tile reads ((Th-1)S+(FH-1)D+1) x ((Tw-1)S+(FW-1)D+1) x Tc
    inputs; "Tiles, halos and partial sums").  Compared with FETCH_SIZE it
    shows how much of the halo re-reading the caches absorb."""
    th, tw, tc = tile
    sh = (th - 1) * wl.stride + (wl.FH - 1) * wl.dilation + 1
    sw = (tw - 1) * wl.stride + (wl.FW - 1) * wl.dilation + 1
    ntiles = wl.N * -(-OH // th) * -(-OW // tw) * -(-wl.C // tc)
    reads = ntiles * (sh * sw + wl.FH * wl.FW) * tc * XB[wl.dtype]
    writes = wl.N * OH * OW * wl.C * YB[wl.dtype]
    return {"tile": [th, tw, tc], "span": [sh, sw], "tiles": ntiles, "read_bytes": reads,
            "write_bytes": writes, "bytes": reads + writes}


def valu_class(plan, dtype):
    """The vector instruction a non-matrix-core plan does its multiply-adds
    with: v_dot4_i32_i8 (int8 tap-packed tile), v_dot2_f32_{f16,bf16} (the
    fp16 / bf16 column stream with paired taps: two channels per lane, five or
    more taps), else one fma (or 24-bit integer multiply-add) per tap."""
    if "tap-packed" in plan or "v_dot4" in plan:
        return "dot4"
    if dtype in ("f16", "bf16") and plan.startswith("colstream: VEC=2"):
        return "dot2"
    return "fma"


def roofline(wl, variant, nbytes, flops, kernel_s, traffic, plan=""):
    """The roof that binds this kernel: HBM unless the arithmetic at the peak
    of the units the kernel uses (matrix cores for the mfma family, else the
    VALU rate of its instruction class) takes longer than moving the
    algorithmic bytes at 8 TB/s."""
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    if variant in ("mfma", "bwf_mfma"):
        bound, peak = "mfma", MFMA_PEAK_TFLOPS[wl.dtype]
    else:
        bound, peak = "alu", VALU_PEAKS[valu_class(plan, wl.dtype)]
    t_cmp = flops / (peak * 1e12)
    if t_hbm >= t_cmp:
        achieved = nbytes / kernel_s / 1e9
        return {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
    achieved = flops / kernel_s / 1e12
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic,
            "hbm_gbs": round(nbytes / kernel_s / 1e9, 2)}


# the source files each kernel family is compiled from
FAMILY_SOURCES = {"direct": ("k_direct.hip",), "rowwin": ("k_rowwin.hip",),
                  "ldstile": ("k_ldstile.hip",), "mfma": ("k_mfma.hip",),
                  "bwf": ("k_bwf.hip",), "bwf_mfma": ("k_bwf_mfma.hip", "k_bwf.hip")}


def code_only(text):
    """C/C++ source without its comments, whitespace runs collapsed: what a
    change to the compiled code changes (string and character literals are
    kept as they are)."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_sources_hash(variant):
    """Hash of the code (comments and layout left out) of one kernel family's
    source file and the headers every family includes; counter figures stored
    under profiles/ are reported only while it matches the hash they were
    taken with."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "depthwise_convolution_amd", "csrc")
    for f in ("dw_common.h", "plan.h") + FAMILY_SOURCES[variant]:
        h.update(f.encode())
        h.update(code_only(open(os.path.join(csrc, f), encoding="utf-8").read()).encode())
    return h.hexdigest()[:16]


def stored_traffic(workload, variant):
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{workload}/{variant}")
    except (ValueError, OSError):
        return None
    if not rec or rec.get("sources") != kernel_sources_hash(variant):
        return None
    return rec.get("hbm_bytes_per_launch")


def _copy_lib():
    import ctypes
    path = os.path.join(ROOT, "depthwise_convolution_amd", "libdwcopy.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.dwcopy_nt.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                              ctypes.c_void_p]
    lib.dwcopy_nt.restype = ctypes.c_int
    return lib


def copy_ceiling(torch, dev, stream, nbytes, sets, K, warmup, kind="nt"):
    """A plain copy that reads nbytes/2 and writes nbytes/2 (the same total as
    one pass), over the same number of rotating buffer sets, timed the same
    way: the practical HBM ceiling on this GPU, and the known-size kernel
    that calibrates the traffic counters.  kind "nt": the hand-written
    non-temporal copy (libdwcopy.so); "torch": torch's copy_."""
    half = nbytes // 2 // 16 * 16
    lib = _copy_lib() if kind == "nt" else None
    if kind == "nt" and lib is None:
        return None
    src = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(sets)]
    dst = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(sets)]
    for t in src:
        t.fill_(1)

    def one(i):
        if lib is not None:
            rc = lib.dwcopy_nt(src[i % sets].data_ptr(), dst[i % sets].data_ptr(), half,
                               stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"dwcopy_nt failed ({rc})")
        else:
            dst[i % sets].copy_(src[i % sets])
    for i in range(warmup):
        one(i)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    clock_warmup(torch, stream, one)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(K):
        one(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    return {"gbs": round(2 * half / (ms * 1e-3) / 1e9, 2), "avg_us": round(ms * 1e3, 3),
            "bytes": 2 * half,
            "kind": ("hand-written copy: 2048 workgroups, 16 KiB chunks, 4 x 16-byte loads in flight per lane, "
                     "non-temporal stores, back to back") if lib is not None
            else "torch copy_ (device to device), back to back"}


def cpu_baseline(wl, x, w, b, budget_s=20.0, op="fwd", bn=None):
    """The CPU oracle (test infrastructure, untuned) on this host's cores.
    Sample: whole images of the same workload, as many as fit the budget
    after a one-image probe.  For the backward-data pass x holds dy; for the
    fused-prologue pass bn is (scale, shift) as numpy fp32 arrays."""
    import oracle
    host_cores = len(os.sched_getaffinity(0))
    threads = max(1, min(16, host_cores))

    def run(n, t):
        if op == "bwd_filter":
            shape = (n, wl.H, wl.W, wl.C, wl.FH, wl.FW, wl.stride, wl.dilation, wl.pad)
            oracle.bwd_filter(x[:n], w[:n], shape, wl.dtype, threads=t)
        elif op == "bwd_data":
            shape = (n, wl.H, wl.W, wl.C, wl.FH, wl.FW, wl.stride, wl.dilation, wl.pad)
            oracle.bwd_data(x[:n], w, shape, wl.dtype, threads=t)
        elif op == "fwd_bn_act":
            oracle.fwd_bn_act(x[:n], w, b, bn[0], bn[1], "relu", wl.stride, wl.dilation,
                              wl.pad, wl.dtype, threads=t)
        else:
            oracle.fwd(x[:n], w, b, wl.stride, wl.dilation, wl.pad, wl.dtype, threads=t)

    def used(n):
        # the oracle splits the batch over threads (channels for the filter
        # gradient), so at most that many run
        return min(threads, wl.C if op == "bwd_filter" else n)

    def op_bytes(n):
        # algorithmic bytes of the pass over n images
        sub = type(wl)(**{**wl.__dict__, "N": n})
        nbytes, flops, OH, OW = work(sub)
        if op in ("bwd_data", "bwd_filter"):
            nbytes = (n * OH * OW + n * wl.H * wl.W) * wl.C * XB[wl.dtype] + \
                wl.FH * wl.FW * wl.C * (XB[wl.dtype] if op == "bwd_data" else 4)
        if op == "fwd_bn_act":
            nbytes += 2 * wl.C * 4
        return nbytes, flops

    run(1, 1)   # untimed: loads the oracle library and touches the inputs
    t0 = time.perf_counter()
    run(1, 1)
    per_image_1t = time.perf_counter() - t0
    n = int(max(1, min(wl.N, budget_s * threads / max(per_image_1t, 1e-6))))
    n = max(min(n, wl.N), min(threads, wl.N))
    # repeat a sample that finishes quickly until about 2 s have passed, so
    # that the rate is not one short, noisy measurement
    reps = 0
    t0 = time.perf_counter()
    while True:
        run(n, threads)
        reps += 1
        if time.perf_counter() - t0 >= min(2.0, budget_s):
            break
    dt = (time.perf_counter() - t0) / reps
    nbytes, flops = op_bytes(n)
    return {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": used(n),
            "host_cores": host_cores, "kind": "oracle",
            "gflops": round(flops / dt / 1e9, 3),
            "single_thread": {"value": round(op_bytes(1)[0] / per_image_1t / 1e9, 4),
                              "unit": "GB/s",
                              "sample": f"1 image, {per_image_1t:.4f} s (after one untimed run)"},
            "sample": f"{n} of {wl.N} images of {wl.name} ({op}; fp64/int64 loop nest, "
                      f"{used(n)} threads, {dt:.3f} s per run, mean of {reps})"}


# The pages' kernel sweep: square filters of growing size on three NHWC
# feature maps ("Flash-DWC: Making Depthwise Convolution Compute-Efficient on
# GPUs", Fig. 6 and the evaluation's filter-size sweep), stride 1 and same
# padding, fp32 and fp16 (fp32 accumulate).
SWEEP_SHAPES = [(128, 128, 128, 128), (128, 64, 64, 256), (128, 32, 32, 1024)]
SWEEP_FILTERS = "3,5,7,9,13,17,21,25,31,41,51"


def run_sweep(args):
    """TFLOP/s against the filter size; one JSON line per point on stdout,
    progress on stderr.  Inputs are drawn on the GPU (seeded)."""
    import torch
    import depthwise_convolution_amd as dw
    import synth
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    filters = [int(f) for f in args.sweep_filters.split(",")]
    dtypes = args.sweep_dtypes.split(",")
    shapes = SWEEP_SHAPES[:args.sweep_shapes]
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}
    summary = []
    for si, (N, H, W, C) in enumerate(shapes):
        for fmt in dtypes:
            x = synth.device_input((N, H, W, C), fmt, 7000 + 10 * si + len(fmt), dev)
            y = torch.empty((N, H, W, C), dtype=tdt[fmt], device=dev)
            rng = np.random.default_rng(7100 + si)
            for F in filters:
                P = F // 2
                w = synth.to_storage(rng.normal(0.0, 1.0 / F, (F, F, C)), fmt)
                b = synth.to_storage(rng.uniform(-0.1, 0.1, C), "f32")
                wt = (torch.from_numpy(w.view(np.int16)).view(torch.bfloat16) if fmt == "bf16"
                      else torch.from_numpy(w)).to(dev)
                bt = torch.from_numpy(b).to(dev)
                h = dw.dwconv_create(N, H, W, C, F, F, 1, 1, P, fmt)
                plan = dw.dwconv_plan_describe(h)
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                dw.dwconv_fwd(h, x, wt, bt, y, stream)   # warm-up
                e0.record(stream)
                dw.dwconv_fwd(h, x, wt, bt, y, stream)
                e1.record(stream)
                torch.cuda.synchronize()
                t1 = e0.elapsed_time(e1) * 1e-3
                K = int(max(1, min(20, args.sweep_seconds / max(t1, 1e-6))))
                e0.record(stream)
                for _ in range(K):
                    dw.dwconv_fwd(h, x, wt, bt, y, stream)
                e1.record(stream)
                torch.cuda.synchronize()
                dw.dwconv_destroy(h)
                t = e0.elapsed_time(e1) * 1e-3 / K
                flops = 2 * N * H * W * C * F * F
                nbytes = 2 * N * H * W * C * XB[fmt] + F * F * C * XB[fmt] + C * 4
                mfma = plan.startswith("mfma")
                peak = MFMA_PEAK_TFLOPS[fmt] if mfma else VALU_PEAKS[valu_class(plan, fmt)]
                bound = "hbm" if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (peak * 1e12) else (
                    "mfma" if mfma else "alu")
                rec = {"sweep": "filter size", "shape": [N, H, W, C], "dtype": fmt, "F": F,
                       "pad": P, "plan": plan, "us": round(t * 1e6, 2), "launches": K,
                       "tflops": round(flops / t / 1e12, 3), "gbs": round(nbytes / t / 1e9, 1),
                       "bound": bound,
                       "frac": round((nbytes / t / 1e9) / HBM_PEAK_GBS if bound == "hbm"
                                     else flops / t / 1e12 / peak, 4)}
                print(json.dumps(rec), flush=True)
                print(f"[sweep] {N}x{H}x{W}x{C} {fmt} F={F}: {t * 1e3:.3f} ms, "
                      f"{rec['tflops']:.2f} TFLOP/s ({plan.split(':')[0]})", file=sys.stderr,
                      flush=True)
                summary.append(rec)
            del x, y
            torch.cuda.empty_cache()
    return summary


CLOCK_WARMUP_MS = 300.0


def clock_warmup(torch, stream, step, ms=None):
    """Untimed steps, back to back, for about `ms` of GPU time (estimated from
    ten timed steps), so that the clocks have settled when the timed steps
    start.  Returns the number of steps run."""
    ms = CLOCK_WARMUP_MS if ms is None else ms
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(10):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    per = max(e0.elapsed_time(e1) / 10, 1e-3)
    n = int(min(50000, max(0.0, ms - 10 * per) / per))
    for i in range(n):
        step(i)
    return 10 + n


def measure(torch, dw, wl, op, variant_req, K, warmup, cpu_budget, with_copy=True,
            warm_cache=False, launch="eager"):
    """Times one workload's pass (op) and returns its record: value, kernel
    average and spread, roofline, copy ceilings and the CPU oracle baseline
    (cpu_budget seconds of host work; 0 skips it)."""
    from synth import make_inputs
    nbytes, flops, OH, OW = work(wl)
    bwd = op == "bwd_data"
    bwf = op == "bwd_filter"
    bna = op == "fwd_bn_act"
    print(f"[bench] {wl.name} ({op}): generating inputs", file=sys.stderr, flush=True)
    x, w, b = make_inputs(wl)
    if bna:
        # the forward pass plus the per-channel scale and shift it reads
        nbytes += 2 * wl.C * 4
    if bwf:
        # the pass reads x and dy (N x OH x OW x C, drawn like x) and writes
        # the fp32 filter gradient; w holds dy here
        w, _, _ = make_inputs(type(wl)(**{**wl.__dict__, "H": OH, "W": OW, "b_dist": None,
                                           "seed": wl.seed + 200}))
        b = None
        nbytes = (wl.N * OH * OW + wl.N * wl.H * wl.W) * wl.C * XB[wl.dtype] + \
            wl.FH * wl.FW * wl.C * 4
    if bwd:
        # the pass reads dy (N x OH x OW x C, drawn like x) and w, writes dx
        # (N x H x W x C); no bias
        x, _, _ = make_inputs(type(wl)(**{**wl.__dict__, "H": OH, "W": OW, "b_dist": None,
                                           "seed": wl.seed + 100}))
        b = None
        nbytes = (wl.N * OH * OW + wl.N * wl.H * wl.W) * wl.C * XB[wl.dtype] + \
            wl.FH * wl.FW * wl.C * XB[wl.dtype]

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def to_dev(a, fmt):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if fmt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    ydt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
           "i8": torch.int32}[wl.dtype]
    set_bytes = nbytes
    # enough rotating copies that no step finds its input in the MALL or L2
    # (a workload of a few KB stays cache-resident whatever is done: it is
    # reported as latency only)
    sets = min(MAX_BUFFER_SETS, max(2, -(-MALL_FLUSH_BYTES // set_bytes)))
    xd0 = to_dev(x, wl.dtype)
    xs = [xd0] + [xd0.clone() for _ in range(sets - 1)]
    yshape = (wl.N, wl.H, wl.W, wl.C) if bwd else (wl.N, OH, OW, wl.C)
    if bwf:
        # dy rotates with x; dw is tiny and written every step
        ydt, yshape = torch.float32, (wl.FH, wl.FW, wl.C)
        wd0 = to_dev(w, wl.dtype)
        dys = [wd0] + [wd0.clone() for _ in range(sets - 1)]
    ys = [torch.empty(yshape, dtype=ydt, device=dev) for _ in range(sets)]
    wd = to_dev(w, wl.dtype)
    bd = to_dev(b, "f32" if wl.dtype != "i8" else "i8")
    torch.cuda.synchronize()

    h = dw.dwconv_create_variant(wl.N, wl.H, wl.W, wl.C, wl.FH, wl.FW, wl.stride,
                                 wl.dilation, wl.pad, wl.dtype, variant_req)
    # the steps pass raw device pointers and the raw stream handle (the
    # tensors above stay alive), so a step costs the host one C call: the
    # small workloads are then bound by the launch itself, not by Python
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    xp, yp, wp, bp = [ptr(t) for t in xs], [ptr(t) for t in ys], ptr(wd), ptr(bd)
    sp = stream.cuda_stream
    bn_s = bn_b = None
    if bwf:
        desc = dw.dwconv_bwd_filter_describe(h)
        if not desc:
            raise SystemExit(f"bench.py: {wl.name} has no backward-filter pass in this build")
        variant = "bwf_mfma" if desc.startswith("bwf mfma") else "bwf"
        wsb = torch.empty(dw.dwconv_bwd_filter_workspace(h), dtype=torch.uint8, device=dev)

        dyp, wsp = [ptr(t) for t in dys], ptr(wsb)

        def step(i, st=sp):
            dw.dwconv_bwd_filter(h, xp[i % sets], dyp[i % sets], yp[i % sets], wsp, st)
    elif bwd:
        if not dw.dwconv_bwd_data_supported(h):
            raise SystemExit(f"bench.py: {wl.name} has no backward-data pass in this build")
        desc = dw.dwconv_bwd_data_describe(h)
        variant = next(v for v in ("mfma", "ldstile", "direct", "rowwin", "colstream")
                       if desc.startswith(v))
        variant = "rowwin" if variant == "colstream" else variant

        def step(i, st=sp):
            dw.dwconv_bwd_data(h, xp[i % sets], wp, yp[i % sets], st)
    elif bna:
        desc = dw.dwconv_fwd_bn_act_describe(h)
        if not desc:
            raise SystemExit(f"bench.py: {wl.name} has no fused-prologue pass")
        variant = next(v for v in ("mfma", "ldstile", "direct", "rowwin", "colstream",
                                   "rowchunk") if desc.startswith(v))
        variant = "rowwin" if variant in ("colstream", "rowchunk") else variant
        rs = np.random.default_rng(wl.seed + 300)
        bn_s = torch.from_numpy(rs.uniform(0.5, 1.5, wl.C).astype(np.float32)).to(dev)
        bn_b = torch.from_numpy(rs.normal(0.0, 0.5, wl.C).astype(np.float32)).to(dev)

        bsp, bbp = ptr(bn_s), ptr(bn_b)

        def step(i, st=sp):
            dw.dwconv_fwd_bn_act(h, xp[i % sets], wp, bp, bsp, bbp, "relu", yp[i % sets], st)
    else:
        variant = dw.dwconv_plan_variant(h)
        desc = dw.dwconv_plan_describe(h)

        def step(i, st=sp):
            dw.dwconv_fwd(h, xp[i % sets], wp, bp, yp[i % sets], st)
    print(f"[bench] plan: {desc}; {sets} buffer sets of {set_bytes / 1e6:.1f} MB",
          file=sys.stderr, flush=True)

    for i in range(warmup):
        step(i)
    # pass 1: K steps back to back, bracketed by synchronisation (one GPU:
    # no barrier needed) -> whole-job throughput, and (one launch per step)
    # the kernel's average duration, from HIP events on the launch stream;
    # the clocks are brought to their sustained state first
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    n_clock = clock_warmup(torch, stream, step)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    start.record(stream)
    for i in range(K):
        step(i)
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0
    total_ms = start.elapsed_time(end)
    # pass 2: the same K steps with a HIP event pair around every launch, on
    # the launch stream: the spread of single launches (each pair adds the
    # event packets' own time, so these run a little above pass 1's average)
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    clock_warmup(torch, stream, step)
    torch.cuda.synchronize()
    for i in range(K):
        ev0[i].record(stream)
        step(i)
        ev1[i].record(stream)
    torch.cuda.synchronize()
    kern_ms = np.array([a.elapsed_time(z) for a, z in zip(ev0, ev1)])
    # pass 1g (launch == "graph"): the same K steps captured once into a HIP
    # graph (on a side stream of default priority) and replayed, timed with
    # HIP events around the replay: the host submits one graph instead of K
    # launches
    graph = None
    if launch == "graph":
        try:
            g = torch.cuda.CUDAGraph()
            cs = torch.cuda.Stream(dev)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=cs):
                for i in range(K):
                    step(i, cs.cuda_stream)
            torch.cuda.synchronize()
            g.replay()
            clock_warmup(torch, stream, step)
            torch.cuda.synchronize()
            g0 = torch.cuda.Event(enable_timing=True)
            g1 = torch.cuda.Event(enable_timing=True)
            g0.record(stream)
            g.replay()
            g1.record(stream)
            torch.cuda.synchronize()
            graph = {"avg_us": round(g0.elapsed_time(g1) / K * 1e3, 3),
                     "eager_avg_us": round(total_ms / K * 1e3, 3),
                     "note": "the K steps captured into one HIP graph and replayed; "
                             "eager_avg_us: the same steps launched one by one"}
            del g
        except RuntimeError as e:
            graph = {"error": str(e)[:200]}
            print(f"[bench] graph capture failed ({e}); timing the eager launches",
                  file=sys.stderr, flush=True)
    # pass 3 (warm_cache), labelled: the same buffer set every step, so up
    # to 256 MB of it can stay in the MALL (not the headline figure)
    warm = None
    if warm_cache:
        w0 = torch.cuda.Event(enable_timing=True)
        w1 = torch.cuda.Event(enable_timing=True)
        clock_warmup(torch, stream, lambda i: step(0))
        torch.cuda.synchronize()
        w0.record(stream)
        for i in range(K):
            step(0)
        w1.record(stream)
        torch.cuda.synchronize()
        warm = {"avg_us": round(w0.elapsed_time(w1) / K * 1e3, 3),
                "note": "one buffer set reused every step; not the headline"}
    tmodel = tile_model(wl, dw.dwconv_plan_tile(h), OH, OW) if op == "fwd" else None
    dw.dwconv_destroy(h)

    # the timed region: the graph replay when it was captured, else the
    # eager launches
    launched = "graph" if graph and "avg_us" in graph else "eager"
    ms_per_step = graph["avg_us"] / 1e3 if launched == "graph" else total_ms / K
    kavg_ms = ms_per_step
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    traffic = stored_traffic(wl.name + (f":{op}" if op != "fwd" else ""), variant)
    print(f"[bench] {wl.name}: kernel avg {kavg_ms * 1e3:.2f} us over the timed region; "
          f"single launches with events: mean {kern_ms.mean() * 1e3:.2f}, median "
          f"{np.median(kern_ms) * 1e3:.2f}, min {kern_ms.min() * 1e3:.2f}, p90 "
          f"{np.percentile(kern_ms, 90) * 1e3:.2f} us; host wall {t_wall * 1e3 / K:.2f} ms/step",
          file=sys.stderr, flush=True)

    copy = tcopy = None
    if with_copy:
        copy = copy_ceiling(torch, dev, stream, nbytes, sets, K, warmup, "nt")
        tcopy = copy_ceiling(torch, dev, stream, nbytes, sets, K, warmup, "torch")
        for c in (copy, tcopy):
            if c:
                print(f"[bench] copy ceiling ({c['kind'][:22]}): {c['gbs']:.0f} GB/s "
                      f"({c['avg_us']:.2f} us per {nbytes / 2e6:.1f} MB read + write)",
                      file=sys.stderr, flush=True)
    del xs, ys

    cpu = None
    if cpu_budget > 0:
        print(f"[bench] {wl.name}: timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, x, w, b, budget_s=cpu_budget, op=op,
                           bn=(bn_s.cpu().numpy(), bn_b.cpu().numpy()) if bna else None)
    ceiling = copy or tcopy
    return {
        "workload": wl.name,
        "op": op,
        "dtype": wl.dtype,
        "value": round(value, 2),
        "unit": "GB/s",
        "ms_per_step": round(ms_per_step, 6),
        "gflops": round(flops / (ms_per_step * 1e-3) / 1e9, 2),
        "hbm_fraction": round(value / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": nbytes,
        "flops": flops,
        "config": {"workload": wl.name, "op": op, "N": wl.N, "H": wl.H, "W": wl.W,
                   "C": wl.C, "FH": wl.FH, "FW": wl.FW, "stride": wl.stride,
                   "dilation": wl.dilation, "pad": wl.pad, "bias": wl.b_dist is not None,
                   "layout": "NHWC", "parallelism": "single GPU"},
        "kernel": {"variant": variant, "plan": desc,
                   "avg_us": round(kavg_ms * 1e3, 3),
                   "single_launch_us": {
                       "mean": round(float(kern_ms.mean()) * 1e3, 3),
                       "median": round(float(np.median(kern_ms)) * 1e3, 3),
                       "min": round(float(kern_ms.min()) * 1e3, 3),
                       "p90": round(float(np.percentile(kern_ms, 90)) * 1e3, 3)},
                   "buffer_sets": sets},
        "warm_cache": warm,
        "launch": launched,
        "clock_warmup_steps": n_clock,
        "graph": graph,
        "tile_model": tmodel,
        "copy_ceiling": copy,
        "torch_copy": tcopy,
        "frac_of_copy": None if ceiling is None else round(value / ceiling["gbs"], 4),
        "roofline": roofline(wl, variant, nbytes, flops, kavg_ms * 1e-3, traffic, desc),
        "cpu_baseline": cpu,
    }


def main():
    global CLOCK_WARMUP_MS
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help=f"one workload (default {DEFAULT_WORKLOAD}, plus the other four in "
                         "the line's 'workloads')")
    ap.add_argument("--variant", default="auto")
    ap.add_argument("--op", default="fwd",
                    choices=["fwd", "bwd_data", "bwd_filter", "fwd_bn_act"],
                    help="the forward pass (default), backward data or backward filter")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="host seconds for the headline workload's CPU oracle sample "
                         "(a third of it for each other workload)")
    ap.add_argument("--warm-cache", action="store_true",
                    help="also time K steps on one buffer set (labelled warm cache)")
    ap.add_argument("--no-copy", action="store_true",
                    help="skip the copy ceiling measurements")
    ap.add_argument("--clock-ms", type=float, default=300.0,
                    help="untimed back-to-back steps before each timed pass, in ms of GPU "
                         "time, so that the clocks have settled (0: none)")
    ap.add_argument("--launch", default="eager", choices=["eager", "graph"],
                    help="eager (default): the K timed steps are launched one by one; "
                         "graph: also captured into one HIP graph and replayed (reported "
                         "beside, and the headline when the capture succeeds)")
    ap.add_argument("--sweep", action="store_true",
                    help="the filter-size sweep instead of the bench line: TFLOP/s against "
                         "F on three NHWC maps of 128 images (one JSON line per point)")
    ap.add_argument("--sweep-filters", default=SWEEP_FILTERS)
    ap.add_argument("--sweep-dtypes", default="f32,f16")
    ap.add_argument("--sweep-shapes", type=int, default=len(SWEEP_SHAPES),
                    help="how many of the three feature maps to sweep")
    ap.add_argument("--sweep-seconds", type=float, default=0.3,
                    help="timed launches per point: about this many seconds, 1 to 20")
    args = ap.parse_args()
    CLOCK_WARMUP_MS = args.clock_ms
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not "
              "supported (shard over the batch: one process per GPU, no exchange)",
              file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        run_sweep(args)
        return

    import torch
    import depthwise_convolution_amd as dw
    from synth import WORKLOADS

    all_five = args.workload is None and args.op == "fwd" and args.variant == "auto"
    name = args.workload or DEFAULT_WORKLOAD
    cpu_s = 0.0 if args.no_cpu else args.cpu_seconds
    head = measure(torch, dw, WORKLOADS[name], args.op, args.variant, args.steps,
                   args.warmup, cpu_s, not args.no_copy, args.warm_cache, args.launch)
    others = {}
    if all_five:
        for other in WORKLOADS.values():
            if other.name == name:
                continue
            others[other.name] = measure(torch, dw, other, "fwd", "auto", args.steps,
                                         args.warmup, cpu_s / 3, not args.no_copy,
                                         launch=args.launch)
    rec = {
        "metric": {"fwd": METRIC, "bwd_data": METRIC_BWD, "bwd_filter": METRIC_BWF,
                   "fwd_bn_act": METRIC_BNACT}[args.op],
        "value": head["value"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
    }
    rec.update({k: v for k, v in head.items()
                if k not in ("workload", "op", "dtype", "value", "unit", "ms_per_step",
                             "config")})
    if all_five:
        rec["workloads"] = {name: {k: v for k, v in head.items() if k != "config"}}
        rec["workloads"].update({k: {kk: vv for kk, vv in r.items() if kk != "config"}
                                 for k, r in others.items()})
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
