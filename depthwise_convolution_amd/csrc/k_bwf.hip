// k_bwf.hip -- the backward-filter pass: the gradient with respect to the
// filter,
//
//   dW[fh,fw,c] = sum_{n, oh, ow} X[n, oh*S - P + fh*D, ow*S - P + fw*D, c]
//                                 * dY[n, oh, ow, c]
//
// ("Flash-DWC: Making Depthwise Convolution Compute-Efficient on GPUs",
// section 5.1).  The output is tiny (FH x FW x C) and every element is a long
// reduction over N*OH*OW positions, so, as the page does, the accumulation
// axis is split into Z chunks that run in parallel.  The page merges them
// with fp32 atomic adds; here they are merged deterministically in a second
// pass over a caller-provided workspace, with a pairwise sum.
//
// Pass 1 (k_bwf_partial): a lane owns one vector of VEC channels (one
// 16-byte load, or one element), one filter row fh, a chunk of 3, 5 or 8
// filter columns and a chunk of consecutive (n, oh) output rows.  It walks
// each output row once, in blocks of pixels whose loads are all issued before
// their arithmetic: per pixel one dY vector, and at stride 1 and dilation 1
// one window of input vectors shared by the block's taps; otherwise each
// tap's input is loaded directly.  Input
// positions outside the image count as zero.  Sums are fp32, with a fresh
// partial every 64 pixels and every row; the chunk's totals go to the
// workspace, ws[z][fh][fw][c].
//
// Pass 2 (k_bwf_reduce): one lane per filter element sums its Z chunk
// totals: blocks of 16 by a fixed tree, the block sums by a binary carry (a
// pairwise sum).  Worst-case rounding error of the whole reduction is about
// (64 + K + log2(Z) + 4) * 2^-24 * sum |x * dy| with K the 64-pixel partials
// one chunk adds up; the planner keeps K <= 64, so the bound stays under
// 1e-5 * sum |x * dy|.
#include "plan.h"

#include <stdio.h>
#include <string.h>

namespace dw {

namespace {
constexpr int BWF_SEG = 64;   // pixels per fresh partial
}  // namespace

// BWF_TAPS: filter columns per lane (3, 5 or 8, the smallest chunk that
// holds a filter row of up to 5 taps; wider rows take chunks of 8)
template <class DT, int VEC, bool SLIDE, int BWF_TAPS>
__global__ void __launch_bounds__(256)
k_bwf_partial(const typename DT::X *__restrict__ x, const typename DT::X *__restrict__ dy,
              float *__restrict__ ws, Shape s, int ncv, int nfc, int rpc, long long lanes) {
    using X = typename DT::X;
    // pixels per block of loads: enough loads in flight, registers <= 256
    // (without the sliding window each pixel already loads 1 + TAPS vectors)
    constexpr int U = !SLIDE ? (VEC == 1 ? 4 : 1)
                             : VEC == 1 ? 16 : VEC == 4 ? 8 : BWF_TAPS == 8 ? 2 : 4;
    const long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= lanes) return;
    const int cv = (int)(g % ncv);
    long long r = g / ncv;
    const int fc = (int)(r % nfc);
    r /= nfc;
    const int fh = (int)(r % s.FH);
    const int z = (int)(r / s.FH);
    const int c0 = cv * VEC;
    const int fw0 = fc * BWF_TAPS;
    const long long nrows = (long long)s.N * s.OH;
    const long long row0 = (long long)z * rpc;
    const long long row1 = row0 + rpc < nrows ? row0 + rpc : nrows;

    float acc[BWF_TAPS][VEC];
#pragma unroll
    for (int j = 0; j < BWF_TAPS; ++j)
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[j][v] = 0.0f;

    auto load = [&](float (&dst)[VEC], const X *src, bool ok) {
        if constexpr (VEC == 1) {
            dst[0] = ok ? DT::widen(*src) : 0.0f;
        } else {
            typedef uint32_t V4 __attribute__((ext_vector_type(4)));
            X e[VEC];
            static_assert(sizeof(X) * VEC == 16, "one 16-byte vector");
            if (ok) {
                V4 q = *reinterpret_cast<const V4 *>(src);
                __builtin_memcpy(e, &q, 16);
            }
#pragma unroll
            for (int v = 0; v < VEC; ++v) dst[v] = ok ? DT::widen(e[v]) : 0.0f;
        }
    };

    for (long long row = row0; row < row1; ++row) {
        const long long n = row / s.OH;
        const int oh = (int)(row % s.OH);
        const int ih = oh * s.S - s.P + fh * s.D;
        if ((unsigned)ih >= (unsigned)s.H) continue;  // the whole row taps padding
        const X *xr = x + ((n * s.H + ih) * (long long)s.W) * s.C + c0;
        const X *gr = dy + ((n * s.OH + oh) * (long long)s.OW) * s.C + c0;
        for (int seg = 0; seg < s.OW; seg += BWF_SEG) {
            const int seg1 = seg + BWF_SEG < s.OW ? seg + BWF_SEG : s.OW;
            float part[BWF_TAPS][VEC];
#pragma unroll
            for (int j = 0; j < BWF_TAPS; ++j)
#pragma unroll
                for (int v = 0; v < VEC; ++v) part[j][v] = 0.0f;
            // blocks of U pixels: every load of a block is issued before its
            // arithmetic (pixels past the segment read as zero gradients)
            for (int ow0 = seg; ow0 < seg1; ow0 += U) {
                float gv[U][VEC];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    load(gv[u], gr + (long long)(ow0 + u < seg1 ? ow0 + u : ow0) * s.C,
                         ow0 + u < seg1);
                if constexpr (SLIDE) {
                    // stride 1, dilation 1: tap j of pixel ow0 + u reads
                    // column ow0 + u - P + fw0 + j, window entry u + j
                    float xw[U + BWF_TAPS - 1][VEC];
#pragma unroll
                    for (int k = 0; k < U + BWF_TAPS - 1; ++k) {
                        const int iw = ow0 - s.P + fw0 + k;
                        const bool ok = (unsigned)iw < (unsigned)s.W;
                        load(xw[k], xr + (long long)(ok ? iw : 0) * s.C, ok);
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u)
#pragma unroll
                        for (int j = 0; j < BWF_TAPS; ++j)
#pragma unroll
                            for (int v = 0; v < VEC; ++v)
                                part[j][v] = __builtin_fmaf(xw[u + j][v], gv[u][v], part[j][v]);
                } else {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        float xw[BWF_TAPS][VEC];
#pragma unroll
                        for (int j = 0; j < BWF_TAPS; ++j) {
                            const int iw = (ow0 + u) * s.S - s.P + (fw0 + j) * s.D;
                            const bool ok = (unsigned)iw < (unsigned)s.W && fw0 + j < s.FW;
                            load(xw[j], xr + (long long)(ok ? iw : 0) * s.C, ok);
                        }
#pragma unroll
                        for (int j = 0; j < BWF_TAPS; ++j)
#pragma unroll
                            for (int v = 0; v < VEC; ++v)
                                part[j][v] = __builtin_fmaf(xw[j][v], gv[u][v], part[j][v]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < BWF_TAPS; ++j)
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[j][v] += part[j][v];
        }
    }
    float *out = ws + (((long long)z * s.FH + fh) * s.FW + fw0) * s.C + c0;
#pragma unroll
    for (int j = 0; j < BWF_TAPS; ++j)
        if (fw0 + j < s.FW) {
#pragma unroll
            for (int v = 0; v < VEC; ++v) out[(long long)j * s.C + v] = acc[j][v];
        }
}

// dW[e] = pairwise sum over z of ws[z][e]: blocks of 16 by a fixed tree, the
// block sums by a binary carry (level l holds the sum of 2^l blocks).
__global__ void __launch_bounds__(256)
k_bwf_reduce(const float *__restrict__ ws, float *__restrict__ dw, long long elems, int Z) {
    const long long e = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    if (e >= elems) return;
    constexpr int LV = 24;  // 2^24 blocks of 16 is far beyond any Z
    float lv[LV];
    bool has[LV];
#pragma unroll
    for (int l = 0; l < LV; ++l) {
        lv[l] = 0.0f;
        has[l] = false;
    }
    for (int z0 = 0; z0 < Z; z0 += 16) {
        float b[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) b[k] = z0 + k < Z ? ws[(long long)(z0 + k) * elems + e] : 0.0f;
#pragma unroll
        for (int w = 8; w >= 1; w /= 2)
#pragma unroll
            for (int k = 0; k < w; ++k) b[k] = b[k] + b[k + w];
        float sum = b[0];
        bool placed = false;
#pragma unroll
        for (int l = 0; l < LV; ++l) {
            if (!placed) {
                if (has[l]) {
                    sum = lv[l] + sum;
                    has[l] = false;
                } else {
                    lv[l] = sum;
                    has[l] = true;
                    placed = true;
                }
            }
        }
    }
    float total = 0.0f;
#pragma unroll
    for (int l = 0; l < LV; ++l)
        if (has[l]) total = total + lv[l];
    dw[e] = total;
}

hipError_t launch_bwf_reduce(const Shape &s, const float *ws, float *dw, int Z, hipStream_t st) {
    const long long elems = (long long)s.FH * s.FW * s.C;
    hipLaunchKernelGGL(k_bwf_reduce, dim3((uint32_t)((elems + 255) / 256)), dim3(256), 0, st, ws,
                       dw, elems, Z);
    return hipGetLastError();
}

template <class DT, int VEC, bool SLIDE, int TAPS>
static hipError_t launch_bwf(const BwfPlan &b, const void *x, const void *dy, float *dw,
                             void *ws, hipStream_t st) {
    const long long lanes = (long long)b.ncv * b.nfc * b.s.FH * b.Z;
    hipLaunchKernelGGL((k_bwf_partial<DT, VEC, SLIDE, TAPS>), dim3((uint32_t)((lanes + 255) / 256)),
                       dim3(256), 0, st, (const typename DT::X *)x,
                       (const typename DT::X *)dy, (float *)ws, b.s, b.ncv, b.nfc, b.rpc, lanes);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_bwf_reduce(b.s, (const float *)ws, dw, b.Z, st);
}

bool plan_bwd_filter(BwfPlan &b, const Plan &f) {
    memset(&b, 0, sizeof(b));
    if (f.dtype == DT_I8) return false;
    b.s = f.s;
    b.dtype = f.dtype;
    const int eb = f.elem_bytes;
    const bool vec_ok = (f.s.C * eb) % 16 == 0;
    const int VEC = vec_ok ? 16 / eb : 1;
    const bool slide = f.s.S == 1 && f.s.D == 1;
    const int taps = f.s.FW <= 3 ? 3 : f.s.FW <= 5 ? 5 : 8;
    b.vec = VEC;
    b.ncv = f.s.C / VEC;
    b.nfc = (f.s.FW + taps - 1) / taps;
    // about 128K lanes, each over a chunk of whole output rows, and no chunk
    // adding up more than 64 partials of 64 pixels (the error bound)
    const long long nrows = (long long)f.s.N * f.s.OH;
    const long long per_z = (long long)b.ncv * b.nfc * f.s.FH;
    const long long segs = (f.s.OW + BWF_SEG - 1) / BWF_SEG;
    long long Z = (131072 + per_z - 1) / per_z;
    if (Z > nrows) Z = nrows;
    if (Z < 1) Z = 1;
    long long rpc = (nrows + Z - 1) / Z;
    const long long rpc_max = 64 / segs > 0 ? 64 / segs : 1;
    if (rpc > rpc_max) rpc = rpc_max;
    Z = (nrows + rpc - 1) / rpc;
    if (rpc >= (1LL << 31) || Z >= (1LL << 24) || per_z * Z >= (1LL << 40)) return false;
    b.Z = (int)Z;
    b.rpc = (int)rpc;
    b.ws_bytes = (size_t)Z * f.s.FH * f.s.FW * f.s.C * sizeof(float);
#define BWF_PICK(DTT, V)                                                                   \
    (slide ? (taps == 3 ? launch_bwf<DTT, V, true, 3>                                      \
                        : taps == 5 ? launch_bwf<DTT, V, true, 5> : launch_bwf<DTT, V, true, 8>) \
           : (taps == 3 ? launch_bwf<DTT, V, false, 3>                                     \
                        : taps == 5 ? launch_bwf<DTT, V, false, 5> : launch_bwf<DTT, V, false, 8>))
    switch (f.dtype) {
        case DT_F32:
            b.vec_launch = BWF_PICK(F32, 4);
            b.one_launch = BWF_PICK(F32, 1);
            break;
        case DT_F16:
            b.vec_launch = BWF_PICK(F16, 8);
            b.one_launch = BWF_PICK(F16, 1);
            break;
        case DT_BF16:
            b.vec_launch = BWF_PICK(BF16, 8);
            b.one_launch = BWF_PICK(BF16, 1);
            break;
        default: return false;
    }
#undef BWF_PICK
    if (!vec_ok) b.vec_launch = b.one_launch;
    snprintf(b.desc, sizeof(b.desc),
             "bwf: %d ch/lane x filter row x %d taps, Z=%d chunks of %d rows (%s), "
             "pairwise merge, workspace %zu B",
             VEC, taps, b.Z, b.rpc, slide ? "sliding window" : "direct taps", b.ws_bytes);
    // fp16 / bf16 at stride 1: the matrix-core pass 1 for aligned tensors
    // (it sizes the workspace for both and describes itself)
    plan_bwf_mfma(b);
    return true;
}

}  // namespace dw
