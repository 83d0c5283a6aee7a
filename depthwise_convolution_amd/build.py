"""Builds libdwconv.so (the gfx950 HIP kernels and the C ABI) in-tree.

    python -m depthwise_convolution_amd.build [-v] [-j N]

Every source is compiled by hipcc as HIP for gfx950 only.  Packed-FP32 VALU
instructions are disabled for all device code (hipcc -O3 would otherwise
form them from ordinary float code).
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libdwconv.so")
# the bench's copy-ceiling kernel: its own small library, outside the C ABI
COPY_SRC = os.path.join(HERE, "ceiling", "copy_ceiling.hip")
COPY_LIB = os.path.join(HERE, "libdwcopy.so")
OBJDIR = os.path.join(ROOT, "_build", "obj")

ARCH = "gfx950"
CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _hipcc():
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the HIP toolchain is required")
    return h


def _compile(src, verbose):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [_hipcc(), "-x", "hip", "-c", src, "-o", obj] + CFLAGS
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    # the host pass does not know the packed-fp32 feature and says so; keep
    # every other diagnostic visible
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l
                    and "(ignoring feature)" not in l)
    if verbose and msg.strip():
        print(msg, flush=True)
    return obj


def build(verbose=False, jobs=None):
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), os.cpu_count() or 4, 8)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    copy_obj = _compile(COPY_SRC, verbose)
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", COPY_LIB + ".tmp",
           copy_obj]
    subprocess.check_call(cmd)
    os.replace(COPY_LIB + ".tmp", COPY_LIB)
    return LIB


if __name__ == "__main__":
    j = None
    if "-j" in sys.argv:
        j = int(sys.argv[sys.argv.index("-j") + 1])
    print(build(verbose="-v" in sys.argv, jobs=j))
