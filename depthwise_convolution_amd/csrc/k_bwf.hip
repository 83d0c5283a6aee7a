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
// Pass 1, column stream (k_bwf_cs; stride 1, dilation 1, 3x3 and 5x5
// filters, 16-byte channel vectors): a lane owns VEC channels x TM output
// columns x TH output rows (a strip) and walks the strip's TH + FH - 1 input
// rows once, keeping the last FH gradient rows in registers, so each input
// and gradient vector is loaded once per strip.  Every tap's products go
// into one fp32 partial of TH * TM <= 64 pixels.  The workgroup's strips are
// summed in LDS by a fixed tree and one chunk sum per workgroup goes to the
// workspace.  (The matrix-core pass 1 for fp16 / bf16 is in k_bwf_mfma.hip.)
//
// Pass 2 (k_bwf_reduce): the Z chunk totals of each filter element are
// summed pairwise: blocks of 16 by a fixed tree, the block sums by a binary
// carry, the shares of up to 16 threads by a fixed tree.  Worst-case
// rounding error of the whole reduction is about (64 + K + log2(Z) + 5) *
// 2^-24 * sum |x * dy| with K the partials one chunk adds up (at most 64);
// the bound stays under 1e-5 * sum |x * dy|.
#include "plan.h"

#include <stdio.h>
#include <stdlib.h>
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

namespace {
template <class E, int VEC>
__device__ __forceinline__ void bwf_ld16(E (&dst)[VEC], const E *src) {
    static_assert(sizeof(E) * VEC == 16, "one 16-byte vector");
    typedef uint32_t V4 __attribute__((ext_vector_type(4)));
    const V4 q = *reinterpret_cast<const V4 *>(src);
    __builtin_memcpy(dst, &q, 16);
}
}  // namespace

template <class DT, int VEC, int FH, int FW, int TM, int TH, int PF>
__global__ void __launch_bounds__(256)
k_bwf_cs(const typename DT::X *__restrict__ x, const typename DT::X *__restrict__ dy,
         float *__restrict__ ws, Shape s, int ncv, int cg, int spw, int owg_n, int ohg_n,
         long long nstrips) {
    using X = typename DT::X;
    constexpr int NWIN = TM + FW - 1;  // input columns of a strip
    constexpr int NROW = TH + FH - 1;  // input rows of a strip
    constexpr int NK = FH * FW * VEC;  // partials per lane
    constexpr int RP = NK + 1;         // LDS row pitch (odd: rows on distinct banks)
    static_assert(TH * TM <= 64, "one fresh partial of at most 64 pixels per tap");
    __shared__ float red[256 * RP];

    // workgroup -> (strip block, channel group): the strips of a block are
    // consecutive, so neighbouring strips share halo rows in L2
    const int ngrp = (ncv + cg - 1) / cg;
    const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
    const int grp = bid % ngrp;
    const long long sb = bid / ngrp;
    const int tid = threadIdx.x;
    const int cvl = tid % cg, sl = tid / cg;
    const int cv = grp * cg + cvl;
    const long long strip = sb * spw + sl;
    const bool active = sl < spw && cv < ncv && strip < nstrips;

    float part[FH][FW][VEC];
#pragma unroll
    for (int fh = 0; fh < FH; ++fh)
#pragma unroll
        for (int fw = 0; fw < FW; ++fw)
#pragma unroll
            for (int v = 0; v < VEC; ++v) part[fh][fw][v] = 0.0f;

    if (active) {
        const int owg = (int)(strip % owg_n);
        const long long rr = strip / owg_n;
        const int ohg = (int)(rr % ohg_n);
        const long long n = rr / ohg_n;
        const int oh0 = ohg * TH, ow0 = owg * TM;
        const int ih0 = oh0 - s.P, iw0 = ow0 - s.P;
        const int c0 = cv * VEC;
        const X *xn = x + n * s.H * (long long)s.W * s.C + c0;
        const X *gn = dy + n * s.OH * (long long)s.OW * s.C + c0;
        // raw rows: input row k of the strip and gradient row k; positions
        // outside the image (or past OH / OW) are read from a clamped
        // in-bounds address and zeroed on use
        X xr[PF + 1][NWIN][VEC];
        X gr[TH][TM][VEC];
        auto fetch = [&](int k) {
            const int ih = ih0 + k;
            const X *xrow = xn + (long long)((unsigned)ih < (unsigned)s.H ? ih : 0) * s.W * s.C;
#pragma unroll
            for (int j = 0; j < NWIN; ++j) {
                const int iw = iw0 + j;
                bwf_ld16<X, VEC>(xr[k % (PF + 1)][j],
                                 xrow + (long long)((unsigned)iw < (unsigned)s.W ? iw : 0) * s.C);
            }
            if (k < TH) {
                const int oh = oh0 + k < s.OH ? oh0 + k : 0;
                const X *grow = gn + (long long)oh * s.OW * s.C;
#pragma unroll
                for (int t = 0; t < TM; ++t)
                    bwf_ld16<X, VEC>(gr[k][t],
                                     grow + (long long)(ow0 + t < s.OW ? ow0 + t : 0) * s.C);
            }
        };
#pragma unroll
        for (int k = 0; k < PF && k < NROW; ++k) fetch(k);
        float gw[TH][TM][VEC];
#pragma unroll
        for (int k = 0; k < NROW; ++k) {
            if (k + PF < NROW) fetch(k + PF);
            const bool rok = (unsigned)(ih0 + k) < (unsigned)s.H;
            float xw[NWIN][VEC];
#pragma unroll
            for (int j = 0; j < NWIN; ++j) {
                const bool ok = rok && (unsigned)(iw0 + j) < (unsigned)s.W;
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    xw[j][v] = ok ? DT::widen(xr[k % (PF + 1)][j][v]) : 0.0f;
            }
            if (k < TH) {
                const bool gok = oh0 + k < s.OH;
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    const bool ok = gok && ow0 + t < s.OW;
#pragma unroll
                    for (int v = 0; v < VEC; ++v) gw[k][t][v] = ok ? DT::widen(gr[k][t][v]) : 0.0f;
                }
            }
            // input row k meets gradient row o = k - fh through filter row fh
#pragma unroll
            for (int fh = 0; fh < FH; ++fh) {
                const int o = k - fh;
                if (o < 0 || o >= TH) continue;
#pragma unroll
                for (int fw = 0; fw < FW; ++fw)
#pragma unroll
                    for (int t = 0; t < TM; ++t)
#pragma unroll
                        for (int v = 0; v < VEC; ++v)
                            part[fh][fw][v] =
                                __builtin_fmaf(xw[t + fw][v], gw[o][t][v], part[fh][fw][v]);
            }
        }
    }

    // strips of the workgroup summed by a fixed tree over sl (lane rows of
    // the same channel vector are cg apart)
    float *mine = red + tid * RP;
#pragma unroll
    for (int fh = 0; fh < FH; ++fh)
#pragma unroll
        for (int fw = 0; fw < FW; ++fw)
#pragma unroll
            for (int v = 0; v < VEC; ++v) mine[(fh * FW + fw) * VEC + v] = part[fh][fw][v];
    __syncthreads();
    for (int w = 1; w < spw; w *= 2) {
        if (sl < spw && sl % (2 * w) == 0 && sl + w < spw) {
            const float *other = red + (tid + w * cg) * RP;
#pragma unroll
            for (int k = 0; k < NK; ++k) mine[k] = mine[k] + other[k];
        }
        __syncthreads();
    }
    // chunk sum of the workgroup: ws[sb][fh][fw][c], consecutive threads on
    // consecutive channels
    float *wz = ws + sb * (long long)FH * FW * s.C;
    const int per_tap = cg * VEC;
    for (int e = tid; e < FH * FW * per_tap; e += 256) {
        const int tap = e / per_tap, rem = e - tap * per_tap;
        const int cl = rem / VEC, v = rem - cl * VEC;
        const int cv2 = grp * cg + cl;
        if (cv2 < ncv) wz[(long long)tap * s.C + cv2 * VEC + v] = red[cl * RP + tap * VEC + v];
    }
}

// dW[e] = pairwise sum over z of ws[z][e].  ZL threads share an element:
// thread zl sums z in [zl*zc, (zl+1)*zc) -- blocks of 16 by a fixed tree, the
// block sums by a binary carry (level l holds the sum of 2^l blocks) -- and
// the ZL results are joined by a fixed tree in LDS.  Every z is added along a
// path of at most log2(Z) + 5 additions, whatever ZL is.
template <int ZL>
__global__ void __launch_bounds__(256)
k_bwf_reduce(const float *__restrict__ ws, float *__restrict__ dw, long long elems, int Z) {
    constexpr int EL = 256 / ZL;  // elements per workgroup
    __shared__ float red[256];
    const int el = threadIdx.x % EL, zl = threadIdx.x / EL;
    const long long e = (long long)blockIdx.x * EL + el;
    const int zc = (Z + ZL - 1) / ZL;
    const int z0 = zl * zc;
    const int z1 = z0 + zc < Z ? z0 + zc : Z;
    float total = 0.0f;
    if (e < elems) {
        constexpr int LV = 24;  // 2^24 blocks of 16 is far beyond any Z
        float lv[LV];
        bool has[LV];
#pragma unroll
        for (int l = 0; l < LV; ++l) {
            lv[l] = 0.0f;
            has[l] = false;
        }
        for (int zb = z0; zb < z1; zb += 16) {
            float b[16];
#pragma unroll
            for (int k = 0; k < 16; ++k)
                b[k] = zb + k < z1 ? ws[(long long)(zb + k) * elems + e] : 0.0f;
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
#pragma unroll
        for (int l = 0; l < LV; ++l)
            if (has[l]) total = total + lv[l];
    }
    if constexpr (ZL == 1) {
        if (e < elems) dw[e] = total;
    } else {
        red[threadIdx.x] = total;
        __syncthreads();
#pragma unroll
        for (int w = ZL / 2; w >= 1; w /= 2) {
            if (zl < w) red[threadIdx.x] = red[threadIdx.x] + red[threadIdx.x + w * EL];
            __syncthreads();
        }
        if (zl == 0 && e < elems) dw[e] = red[threadIdx.x];
    }
}

hipError_t launch_bwf_reduce(const Shape &s, const float *ws, float *dw, int Z, hipStream_t st) {
    const long long elems = (long long)s.FH * s.FW * s.C;
    // split each element's chunks over up to 16 threads, so that few
    // elements with many chunks still fill the chip
    int zl = 1;
    while (zl < 16 && (long long)zl * 32 < Z) zl *= 2;
    const uint32_t grid = (uint32_t)((elems + 256 / zl - 1) / (256 / zl));
#define RED(ZL_)                                                                          \
    case ZL_:                                                                             \
        hipLaunchKernelGGL(k_bwf_reduce<ZL_>, dim3(grid), dim3(256), 0, st, ws, dw, elems, Z); \
        break;
    switch (zl) {
        RED(1)
        RED(2)
        RED(4)
        RED(8)
        RED(16)
    }
#undef RED
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

template <class DT, int VEC, int F, int TM, int TH, int PF>
static hipError_t launch_bwf_cs(const BwfPlan &b, const void *x, const void *dy, float *dw,
                                void *ws, hipStream_t st) {
    hipLaunchKernelGGL((k_bwf_cs<DT, VEC, F, F, TM, TH, PF>), dim3(b.vgrid), dim3(256), 0, st,
                       (const typename DT::X *)x, (const typename DT::X *)dy, (float *)ws, b.s,
                       b.vaux[0], b.vaux[1], b.vaux[2], b.vaux[3], b.vaux[4], b.vstrips);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_bwf_reduce(b.s, (const float *)ws, dw, b.vZ, st);
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
    b.vZ = b.Z;
    snprintf(b.desc, sizeof(b.desc),
             "bwf: %d ch/lane x filter row x %d taps, Z=%d chunks of %d rows (%s), "
             "pairwise merge, workspace %zu B",
             VEC, taps, b.Z, b.rpc, slide ? "sliding window" : "direct taps", b.ws_bytes);
    // fp32 3x3 at stride 1 with 16-byte vectors: the column stream (each
    // input and gradient vector loaded once per strip) replaces the vector
    // pass 1 (fp16 / bf16 have the matrix-core pass)
    if (f.dtype == DT_F32 && vec_ok && slide && f.s.FH == 3 && f.s.FW == 3 &&
        tune_int("bwf_nocs", 0) == 0) {
        const int TM = 4, TH = 14;
        const int ncv = f.s.C / VEC;
        const int cg = ncv < 64 ? ncv : 64;
        const int spw = 256 / cg;
        const int owg_n = (f.s.OW + TM - 1) / TM, ohg_n = (f.s.OH + TH - 1) / TH;
        const long long nstrips = (long long)f.s.N * ohg_n * owg_n;
        const long long nsb = (nstrips + spw - 1) / spw;
        const long long grid = nsb * ((ncv + cg - 1) / cg);
        if (grid < (1LL << 31) && nsb < (1LL << 24)) {
            b.vZ = (int)nsb;
            b.vaux[0] = ncv;
            b.vaux[1] = cg;
            b.vaux[2] = spw;
            b.vaux[3] = owg_n;
            b.vaux[4] = ohg_n;
            b.vstrips = nstrips;
            b.vgrid = (uint32_t)grid;
            const size_t ws = (size_t)nsb * 9 * f.s.C * sizeof(float);
            if (ws > b.ws_bytes) b.ws_bytes = ws;
            b.vec_launch = launch_bwf_cs<F32, 4, 3, 4, 14, 2>;
            snprintf(b.desc, sizeof(b.desc),
                     "bwf colstream: %d ch x %d cols x %d rows per lane, %d strips per "
                     "workgroup summed in LDS, Z=%lld, %u x 256, pairwise merge, workspace %zu B",
                     VEC, TM, TH, spw, nsb, b.vgrid, b.ws_bytes);
        }
    }
    // fp16 / bf16 at stride 1: the matrix-core pass 1 for aligned tensors
    // (it sizes the workspace for both and describes itself)
    plan_bwf_mfma(b);
    return true;
}

}  // namespace dw
