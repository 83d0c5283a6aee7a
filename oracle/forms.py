"""Closed forms the pages state for tiling, storage and traffic.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  These are written from
the pages' formulas and pinned in the tests against the worked numbers the
pages print.  The HIP library has its own planner and never calls these.
"""
from math import ceil


def halo_span(t: int, s: int, r: int, d: int) -> int:
    """Input extent needed by an output extent ``t`` for stride ``s``, kernel
    size ``r`` and dilation ``d``: (t-1)s + (r-1)d + 1.

    "Tiles, halos and partial sums", section "Partition tensors to fit
    storage"; the same formula applies along height and width."""
    if min(t, s, r, d) < 1:
        raise ValueError("extents, stride, kernel and dilation must be >= 1")
    return (t - 1) * s + (r - 1) * d + 1


def out_extent(size: int, r: int, s: int, d: int, p: int) -> int:
    """Largest output extent whose halo span fits the zero-padded input
    ``size + 2p`` (0 if none).  Obtained by inverting ``halo_span``; written
    here as a search so that it is checked against the span itself."""
    t = 0
    while halo_span(t + 1, s, r, d) <= size + 2 * p:
        t += 1
    return t


def tile_storage_bytes(th, tw, tc, tm, r, s=1, d=1, in_bytes=1, w_bytes=1,
                       acc_bytes=4, bias_bytes=4, double_buffer=False,
                       depthwise=False):
    """On-chip bytes for one tile, counted the way the worked storage budget
    of "Tiles, halos and partial sums" counts them: the input halo
    (span_h x span_w x Tc), the weights, one partial sum per output of the
    tile (Th x Tw x Tm) and one bias per output channel.  Double buffering
    doubles the input and weight buffers only; partial sums and biases stay
    single.  Scales, addresses and control storage are excluded, as there.

    The page's example is a dense convolution, whose tile needs
    Tm x Tc x R x R weights.  ``depthwise=True`` applies the same method to a
    depthwise tile, where output channel = input channel (Tm must equal Tc)
    and the weights are Tc x R x R."""
    span_h = halo_span(th, s, r, d)
    span_w = halo_span(tw, s, r, d)
    inp = span_h * span_w * tc * in_bytes
    if depthwise:
        if tm != tc:
            raise ValueError("a depthwise tile has as many output as input channels")
        wts = tc * r * r * w_bytes
    else:
        wts = tm * tc * r * r * w_bytes
    partial = th * tw * tm * acc_bytes
    bias = tm * bias_bytes
    return (2 if double_buffer else 1) * (inp + wts) + partial + bias


def ragged_tiles(m: int, tm: int):
    """(number of tiles, valid elements in the last tile) when ``m`` elements
    are cut into tiles of ``tm``; "Tiles, halos and partial sums", last
    paragraph (the final tile is masked)."""
    n = ceil(m / tm)
    return n, m - (n - 1) * tm


def gemm_qmin(m: int, k: int, n: int, b: int) -> int:
    """Minimum device-memory traffic for C = AB (beta = 0): every operand read
    once and the product written once, b bytes per scalar.  "10.5 Почему важно
    повторно использовать данные" (why data reuse matters), the Q_min formula."""
    return (m * k + k * n + m * n) * b


def gemm_qtile(m: int, k: int, n: int, b: int, t: int) -> int:
    """Traffic of the same product cut into t x t output blocks with no reuse
    between blocks: A is re-read once per block column and B once per block
    row.  Same page, the Q_tile formula."""
    return b * (m * k * ceil(n / t) + k * n * ceil(m / t) + m * n)


def dwc_flops(n, oh, ow, c, fh, fw) -> int:
    """Two operations (multiply and add) per tap per output; the bias add is
    not counted.  "Flash-DWC: Making Depthwise Convolution Compute-Efficient
    on GPUs", section 2.2, numerator of the arithmetic-intensity bound."""
    return 2 * n * oh * ow * c * fh * fw


def dwc_intensity_bound(n, ih, iw, c, oh, ow, fh, fw) -> float:
    """Upper bound on operations per element moved for a depthwise convolution
    when every input and weight element is read once (same page, section 2.2).
    The output is not counted in that bound."""
    return dwc_flops(n, oh, ow, c, fh, fw) / (n * ih * iw * c + c * fh * fw)


def toeplitz_density(tm: int, ffrag: int) -> float:
    """Fraction of non-zeros in the banded K x TM filter matrix that turns one
    channel's GEMV into a GEMM, K = TM + Ffrag - 1 (same page, section 4.2):
    every one of the TM columns holds the Ffrag taps."""
    k = tm + ffrag - 1
    return (tm * ffrag) / (k * tm)
