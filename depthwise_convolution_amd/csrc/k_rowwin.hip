// k_rowwin.hip -- the "row window" kernel family: width-first register reuse.
//
// Each lane owns one vector of VEC channels (one 4/8/16-byte load) of TM
// consecutive outputs along one output row.  Lanes of a wavefront take
// consecutive channel vectors of the same pixels, so every load and store of
// the wavefront is contiguous along C (channel-last layout, "Flash-DWC:
// Making Depthwise Convolution Compute-Efficient on GPUs", section 2.3; the
// 128-byte coalescing of section 3.1 becomes 16 bytes per lane and up to
// 1 KiB per wavefront instruction here).
//
// The 2-D filter is walked as FH one-dimensional rows ("Flash-DWC", section
// 3.3).  For each filter row the lane loads the input run its TM outputs
// need once -- (TM-1)S + (FW-1)D + 1 pixels, the halo span of "Tiles, halos
// and partial sums" along width -- into registers, then sweeps the FW taps
// over it, so each loaded input is reused by every tap that touches it
// (width-first reuse).  Positions outside the image are generated as zeros,
// never fetched.  Each filter row accumulates into a fresh fp32 / int32
// partial that is then added to the running sum, which the bias seeds once.
//
// FW, TM, S and D are template parameters so that the window indices are
// compile-time constants and the window lives in registers; FH is a runtime
// loop.
#include "plan.h"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

namespace dw {

template <int BYTES>
struct VecT;
template <>
struct VecT<16> { using T = __attribute__((ext_vector_type(4))) unsigned int; };
template <>
struct VecT<8> { using T = __attribute__((ext_vector_type(2))) unsigned int; };
template <>
struct VecT<4> { using T = unsigned int; };

template <class E, int VEC>
__device__ __forceinline__ void load_vec(E (&dst)[VEC], const E *src) {
    using V = typename VecT<sizeof(E) * VEC>::T;
    V v = *reinterpret_cast<const V *>(src);
    __builtin_memcpy(dst, &v, sizeof(V));
}

template <class E, int VEC>
__device__ __forceinline__ void store_vec(E *dst, const E (&src)[VEC]) {
    constexpr int B = sizeof(E) * VEC;
    if constexpr (B <= 16) {
        using V = typename VecT<B>::T;
        V v;
        __builtin_memcpy(&v, src, B);
        *reinterpret_cast<V *>(dst) = v;
    } else {
        using V = typename VecT<16>::T;
        constexpr int PER = 16 / sizeof(E);
#pragma unroll
        for (int k = 0; k < B / 16; ++k) {
            V v;
            __builtin_memcpy(&v, src + k * PER, 16);
            *reinterpret_cast<V *>(dst + k * PER) = v;
        }
    }
}

// Loads the NWIN-pixel input run of one row starting at column iw0 and widens
// it to the accumulator type.  Columns outside the image read as zero: their
// address is clamped to column 0 (always inside the row, so the load is in
// bounds and branch-free) and the value is replaced by zero.
// BN: in-image values go through the fused prologue bn_act_stored (bs, bb: the
// lane's VEC scales and shifts); positions outside the image stay zero.
template <class DT, int VEC, int NWIN, bool BN = false>
__device__ __forceinline__ void load_window(typename DT::Acc (&xw)[NWIN][VEC],
                                            const typename DT::X *xr, int iw0, int W,
                                            int C, const float *bs = nullptr,
                                            const float *bb = nullptr, int act = 0) {
    using X = typename DT::X;
    X e[NWIN][VEC];
#pragma unroll
    for (int j = 0; j < NWIN; ++j) {
        const int iw = iw0 + j;
        const int iwc = (unsigned)iw < (unsigned)W ? iw : 0;
        load_vec<X, VEC>(e[j], xr + (long long)iwc * C);
    }
#pragma unroll
    for (int j = 0; j < NWIN; ++j) {
        const bool ok = (unsigned)(iw0 + j) < (unsigned)W;
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            typename DT::Acc val = DT::widen(e[j][v]);
            if constexpr (BN) val = bn_act_stored<DT>(val, bs[v], bb[v], act);
            xw[j][v] = ok ? val : typename DT::Acc(0);
        }
    }
}

// The lane's VEC fused-prologue scales and shifts (channels c0 ..).
template <int VEC>
__device__ __forceinline__ void load_bn(float (&bs)[VEC], float (&bb)[VEC], const float *bns,
                                        const float *bnb, int c0) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        bs[v] = bns[c0 + v];
        bb[v] = bnb[c0 + v];
    }
}

template <class Y, int VEC, bool NT>
__device__ __forceinline__ void store_out(Y *dst, const Y (&o)[VEC]) {
    if constexpr (NT) {
        // y is never read back by this kernel: stream it past the caches
        constexpr int B = sizeof(Y) * VEC;
        constexpr int VB = B < 16 ? B : 16;  // bytes per store
        static_assert(B % VB == 0, "whole vectors");
        using V = typename VecT<VB>::T;
#pragma unroll
        for (int k = 0; k < B / VB; ++k) {
            V v;
            __builtin_memcpy(&v, reinterpret_cast<const char *>(o) + VB * k, VB);
            __builtin_nontemporal_store(v, reinterpret_cast<V *>(dst) + k);
        }
    } else {
        store_vec<Y, VEC>(dst, o);
    }
}

// ---------------------------------------------------------------------------
// Row window: one output row per lane, any stride and dilation.
// ---------------------------------------------------------------------------
template <class DT, int VEC, int FW, int TM, int S, int D, bool BN>
__global__ void __launch_bounds__(256)
k_rowwin(const typename DT::X *__restrict__ x, const typename DT::X *__restrict__ w,
         const typename DT::Bias *__restrict__ bias, typename DT::Y *__restrict__ y,
         Shape s, int ncv, int owg_n, long long total, const float *__restrict__ bns,
         const float *__restrict__ bnb, int act) {
    using X = typename DT::X;
    using Acc = typename DT::Acc;
    constexpr int NWIN = (TM - 1) * S + (FW - 1) * D + 1;

    const uint32_t b = xcd_remap(blockIdx.x, gridDim.x);
    const long long g = (long long)b * blockDim.x + threadIdx.x;
    if (g >= total) return;
    const int cv = (int)(g % ncv);
    long long r = g / ncv;
    const int owg = (int)(r % owg_n);
    r /= owg_n;
    const int oh = (int)(r % s.OH);
    const long long n = r / s.OH;
    const int c0 = cv * VEC;
    const int ow0 = owg * TM;
    const int iw0 = ow0 * S - s.P;
    float bs[VEC], bb[VEC];
    if constexpr (BN) load_bn<VEC>(bs, bb, bns, bnb, c0);

    Acc acc[TM][VEC];
    {
        Acc b0[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) b0[v] = bias ? bias[c0 + v] : Acc(0);
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[t][v] = b0[v];
    }

    for (int fh = 0; fh < s.FH; ++fh) {
        const int ih = oh * S - s.P + fh * D;
        if ((unsigned)ih >= (unsigned)s.H) continue;  // generated zero rows
        const X *xr = x + ((n * s.H + ih) * (long long)s.W) * s.C + c0;

        Acc xw[NWIN][VEC];  // input run of this filter row, widened once
        load_window<DT, VEC, NWIN, BN>(xw, xr, iw0, s.W, s.C, bs, bb, act);
        Acc wt[FW][VEC];
#pragma unroll
        for (int fw = 0; fw < FW; ++fw) {
            X e[VEC];
            load_vec<X, VEC>(e, w + (long long)tap_index(s, fh, fw) * s.C + c0);
#pragma unroll
            for (int v = 0; v < VEC; ++v) wt[fw][v] = DT::widen(e[v]);
        }
        Acc row[TM][VEC];
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int v = 0; v < VEC; ++v) row[t][v] = Acc(0);
#pragma unroll
        for (int fw = 0; fw < FW; ++fw)
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    row[t][v] = mac<Acc>(row[t][v], xw[t * S + fw * D][v], wt[fw][v]);
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[t][v] += row[t][v];
    }

    typename DT::Y *yr = y + ((n * s.OH + oh) * (long long)s.OW + ow0) * s.C + c0;
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        if (ow0 + t < s.OW) {  // masked ragged tail along width
            typename DT::Y o[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) o[v] = DT::narrow(acc[t][v]);
            store_out<typename DT::Y, VEC, false>(yr + (long long)t * s.C, o);
        }
    }
}

// ---------------------------------------------------------------------------
// Row chunks: the row window for filters of any height and width at stride 1
// and dilation 1 (both runtime values).  A filter row is walked in chunks of
// CH taps; a chunk loads the TM + CH - 1 input vectors it needs and its CH
// filter vectors (zero past FW) and adds TM * CH products per channel into
// the filter row's fresh fp32 partial, which is added to the running sum at
// the end of the row ("Flash-DWC: Making Depthwise Convolution
// Compute-Efficient on GPUs", section 3.3: the 2-D filter as FH 1-D rows,
// each reusing one input run across its taps).
// ---------------------------------------------------------------------------
template <class DT, int VEC, int TM, int CH, bool BN>
__global__ void __launch_bounds__(256)
k_rowchunk(const typename DT::X *__restrict__ x, const typename DT::X *__restrict__ w,
           const typename DT::Bias *__restrict__ bias, typename DT::Y *__restrict__ y,
           Shape s, int ncv, int owg_n, long long total, const float *__restrict__ bns,
           const float *__restrict__ bnb, int act) {
    using X = typename DT::X;
    using Acc = typename DT::Acc;
    constexpr int NWIN = TM + CH - 1;

    const uint32_t b = xcd_remap(blockIdx.x, gridDim.x);
    const long long g = (long long)b * blockDim.x + threadIdx.x;
    if (g >= total) return;
    const int cv = (int)(g % ncv);
    long long r = g / ncv;
    const int owg = (int)(r % owg_n);
    r /= owg_n;
    const int oh = (int)(r % s.OH);
    const long long n = r / s.OH;
    const int c0 = cv * VEC;
    const int ow0 = owg * TM;
    const int iw0 = ow0 - s.P;
    const int nch = (s.FW + CH - 1) / CH;
    float bs[VEC], bb[VEC];
    if constexpr (BN) load_bn<VEC>(bs, bb, bns, bnb, c0);

    Acc acc[TM][VEC];
    {
        Acc b0[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) b0[v] = bias ? bias[c0 + v] : Acc(0);
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[t][v] = b0[v];
    }

    for (int fh = 0; fh < s.FH; ++fh) {
        const int ih = oh - s.P + fh;
        if ((unsigned)ih >= (unsigned)s.H) continue;  // generated zero rows
        const X *xr = x + ((n * s.H + ih) * (long long)s.W) * s.C + c0;
        Acc row[TM][VEC];
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int v = 0; v < VEC; ++v) row[t][v] = Acc(0);
        for (int k = 0; k < nch; ++k) {
            const int fw0 = k * CH;
            Acc xw[NWIN][VEC];
            load_window<DT, VEC, NWIN, BN>(xw, xr, iw0 + fw0, s.W, s.C, bs, bb, act);
            Acc wt[CH][VEC];
#pragma unroll
            for (int j = 0; j < CH; ++j) {
                X e[VEC];
                const bool ok = fw0 + j < s.FW;
                load_vec<X, VEC>(e, w + (long long)tap_index(s, fh, ok ? fw0 + j : 0) * s.C + c0);
#pragma unroll
                for (int v = 0; v < VEC; ++v) wt[j][v] = ok ? DT::widen(e[v]) : Acc(0);
            }
#pragma unroll
            for (int j = 0; j < CH; ++j)
#pragma unroll
                for (int t = 0; t < TM; ++t)
#pragma unroll
                    for (int v = 0; v < VEC; ++v)
                        row[t][v] = mac<Acc>(row[t][v], xw[t + j][v], wt[j][v]);
        }
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[t][v] += row[t][v];
    }

    typename DT::Y *yr = y + ((n * s.OH + oh) * (long long)s.OW + ow0) * s.C + c0;
#pragma unroll
    for (int t = 0; t < TM; ++t) {
        if (ow0 + t < s.OW) {  // masked ragged tail along width
            typename DT::Y o[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) o[v] = DT::narrow(acc[t][v]);
            store_out<typename DT::Y, VEC, false>(yr + (long long)t * s.C, o);
        }
    }
}

// ---------------------------------------------------------------------------
// Column stream (stride 1): each lane walks TH output rows of its TM x VEC
// strip.  Every input row of the strip's halo -- TH + (FH-1)D rows -- is
// loaded once; for each filter row fh it feeds output row o = i - fh*D, whose
// fresh row partial is added to that output's running sum.  Output row o
// starts at input row i = o (fh = 0, where the bias seeds it) and is complete
// and stored after input row o + (FH-1)D, so only FH rows of accumulators
// are live at any time (the loop is fully unrolled, indices are constants).
// The whole FH x FW x VEC filter slice stays in registers.  Every output is
// still one bias plus FH unrounded row partials; only the order in which the
// row partials are added depends on the walk direction.
//
// Loads run PF rows ahead of the arithmetic: the raw run of row i + PF is
// requested before row i is used, so each wavefront keeps PF + 1 rows of
// loads in flight instead of waiting on every row.  A row outside the image
// issues no loads (its run is zeros); columns outside it are fetched from a
// clamped in-bounds address and zeroed by a select, so the column loop has no
// divergent branches.
// ---------------------------------------------------------------------------
template <class E, int VEC>
__device__ __forceinline__ void load_vec_nt(E (&dst)[VEC], const E *src) {
    using V = typename VecT<sizeof(E) * VEC>::T;
    V v = __builtin_nontemporal_load(reinterpret_cast<const V *>(src));
    __builtin_memcpy(dst, &v, sizeof(V));
}

// NTL: 0 cached loads; 1 non-temporal loads; 2 non-temporal loads only for
// the window pixels [NT0, NT1) that no neighbouring strip reads (the shared
// edge pixels stay cached in L2 for the neighbour)
template <class X, int VEC, int NWIN, int NTL, int NT0, int NT1>
__device__ __forceinline__ void fetch_run(X (&e)[NWIN][VEC], const X *xn, int ih, int H,
                                          int iw0, int W, int C) {
    if ((unsigned)ih >= (unsigned)H) {  // generated zero row: nothing fetched
#pragma unroll
        for (int j = 0; j < NWIN; ++j)
#pragma unroll
            for (int v = 0; v < VEC; ++v) e[j][v] = X(0);
        return;
    }
    const X *xr = xn + (long long)ih * W * C;
#pragma unroll
    for (int j = 0; j < NWIN; ++j) {
        const int iw = iw0 + j;
        const int iwc = (unsigned)iw < (unsigned)W ? iw : 0;
        if (NTL == 1 || (NTL == 2 && j >= NT0 && j < NT1))  // j is unrolled
            load_vec_nt<X, VEC>(e[j], xr + (long long)iwc * C);
        else
            load_vec<X, VEC>(e[j], xr + (long long)iwc * C);
    }
}

// One strip's walk over its input rows, top-down (UP = false) or bottom-up.
// Bottom-up visits input row i = NROW-1 .. 0; output row o then receives its
// filter rows in the order fh = FH-1 .. 0, starts (bias) at fh = FH-1 and is
// stored after fh = 0.
template <class DT, int VEC, int FH, int FW, int TM, int TH, int D, int PF, bool NT, int NTL,
          bool UP, bool BN>
__device__ __forceinline__ void colstream_walk(const typename DT::X *xn,
                                               const typename DT::Acc (&wt)[FH][FW][VEC],
                                               const typename DT::Acc (&b0)[VEC],
                                               typename DT::Y *yn, const Shape &s, int ih0,
                                               int iw0, int oh0, int ow0, const float *bs,
                                               const float *bb, int act) {
    using X = typename DT::X;
    using Acc = typename DT::Acc;
    using Y = typename DT::Y;
    constexpr int NWIN = TM + (FW - 1) * D;
    constexpr int NROW = TH + (FH - 1) * D;
    constexpr int RING = PF + 1;
    // k-th visited row
    auto row_of = [](int k) { return UP ? NROW - 1 - k : k; };

    X raw[RING][NWIN][VEC];
#pragma unroll
    for (int k = 0; k < PF && k < NROW; ++k)
        fetch_run<X, VEC, NWIN, NTL, (FW - 1) * D, TM>(raw[k % RING], xn, ih0 + row_of(k), s.H, iw0, s.W, s.C);

    Acc acc[TH][TM][VEC];
#pragma unroll
    for (int k = 0; k < NROW; ++k) {
        const int i = row_of(k);
        if (k + PF < NROW)
            fetch_run<X, VEC, NWIN, NTL, (FW - 1) * D, TM>(raw[(k + PF) % RING], xn, ih0 + row_of(k + PF), s.H, iw0,
                                    s.W, s.C);
        const bool row_ok = (unsigned)(ih0 + i) < (unsigned)s.H;
        Acc xw[NWIN][VEC];
#pragma unroll
        for (int j = 0; j < NWIN; ++j) {
            const bool ok = row_ok && (unsigned)(iw0 + j) < (unsigned)s.W;
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                Acc val = DT::widen(raw[k % RING][j][v]);
                if constexpr (BN) val = bn_act_stored<DT>(val, bs[v], bb[v], act);
                xw[j][v] = ok ? val : Acc(0);
            }
        }
#pragma unroll
        for (int q = 0; q < FH; ++q) {
            const int fh = UP ? FH - 1 - q : q;
            const int o = i - fh * D;
            if (o < 0 || o >= TH) continue;
            Acc part[TM][VEC];
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int v = 0; v < VEC; ++v) part[t][v] = Acc(0);
#pragma unroll
            for (int fw = 0; fw < FW; ++fw)
#pragma unroll
                for (int t = 0; t < TM; ++t)
#pragma unroll
                    for (int v = 0; v < VEC; ++v)
                        part[t][v] = mac<Acc>(part[t][v], xw[t + fw * D][v], wt[fh][fw][v]);
            const bool first = UP ? fh == FH - 1 : fh == 0;
            const bool last = UP ? fh == 0 : fh == FH - 1;
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    acc[o][t][v] = (first ? b0[v] : acc[o][t][v]) + part[t][v];
            if (last && oh0 + o < s.OH) {
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    if (ow0 + t < s.OW) {
                        Y ov[VEC];
#pragma unroll
                        for (int v = 0; v < VEC; ++v) ov[v] = DT::narrow(acc[o][t][v]);
                        store_out<Y, VEC, NT>(yn + ((long long)o * s.OW + t) * s.C, ov);
                    }
                }
            }
        }
    }
}

// fp16 / bf16 filters of five or more taps: the taps of a filter row are
// taken two at a time along the width, (fw, fw+1), against the input pair
// (x[j], x[j+D]) of the same channel, with v_dot2(c)_f32_f16 /
// v_dot2_f32_bf16 (two products added into an fp32 sum): half the VALU
// operations of widening every input and using one fma per tap.  The
// instruction is not one rounding of the exact sum: on 2^20 random operand
// sets per format (subnormals included) it stayed within
// 4 * 2^-24 * (|c| + |a0*b0| + |a1*b1|), plus at most 7e-10 absolute for
// fp16 with a subnormal operand.  A 5-tap row partial is a chain of three,
// so an output of FH such partials errs by at most about
// (12 + FH) * 2^-24 * sum|x*w| + 3 FH * 7e-10, well inside the bound.  An odd
// filter width pairs its last tap with a zero tap and a zero input, so an
// Inf or NaN just past an output's window stays out of its sum.  Same walk,
// accumulator rotation and row partials as colstream_walk.
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
template <class DT>
struct Dot2;
template <>
struct Dot2<F16> {
    static __device__ __forceinline__ float dot(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                      c, false);
    }
};
template <>
struct Dot2<BF16> {
    static __device__ __forceinline__ float dot(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                               __builtin_bit_cast(bf16x2_t, b), c, false);
    }
};
template <class DT, int VEC, int FH, int FW, int TM, int TH, int D, int PF, bool NT, int NTL,
          bool UP>
__device__ __forceinline__ void colstream_walk_dot2(const typename DT::X *xn,
                                                    const uint32_t (&wp)[FH][(FW + 1) / 2][VEC],
                                                    const float (&b0)[VEC], typename DT::Y *yn,
                                                    const Shape &s, int ih0, int iw0, int oh0,
                                                    int ow0) {
    using X = typename DT::X;
    using Y = typename DT::Y;
    static_assert(VEC % 2 == 0, "channel pairs are whole dwords");
    constexpr int VD = VEC / 2;                 // dwords (channel pairs) per pixel
    constexpr int NWIN = TM + (FW - 1) * D;
    constexpr int NROW = TH + (FH - 1) * D;
    constexpr int RING = PF + 1;
    constexpr int NP = (FW + 1) / 2;
    auto row_of = [](int k) { return UP ? NROW - 1 - k : k; };
    // the raw run of one input row, kept as packed channel pairs; a row
    // outside the image is not fetched, columns outside it are read from a
    // clamped address and zeroed
    auto fetch = [&](uint32_t (&e)[NWIN][VD], int ih) {
        if ((unsigned)ih >= (unsigned)s.H) {  // generated zero row: nothing fetched
#pragma unroll
            for (int j = 0; j < NWIN; ++j)
#pragma unroll
                for (int u = 0; u < VD; ++u) e[j][u] = 0u;
            return;
        }
        const X *xr = xn + (long long)ih * s.W * s.C;
#pragma unroll
        for (int j = 0; j < NWIN; ++j) {
            const int iw = iw0 + j;
            const int iwc = (unsigned)iw < (unsigned)s.W ? iw : 0;
            load_vec<uint32_t, VD>(e[j], reinterpret_cast<const uint32_t *>(xr + (long long)iwc * s.C));
        }
    };

    uint32_t raw[RING][NWIN][VD];
#pragma unroll
    for (int k = 0; k < PF && k < NROW; ++k) fetch(raw[k % RING], ih0 + row_of(k));
    float acc[TH][TM][VEC];
#pragma unroll
    for (int k = 0; k < NROW; ++k) {
        const int i = row_of(k);
        if (k + PF < NROW) fetch(raw[(k + PF) % RING], ih0 + row_of(k + PF));
        const bool row_ok = (unsigned)(ih0 + i) < (unsigned)s.H;
        uint32_t xv[NWIN][VD];
#pragma unroll
        for (int j = 0; j < NWIN; ++j) {
            const bool ok = row_ok && (unsigned)(iw0 + j) < (unsigned)s.W;
#pragma unroll
            for (int u = 0; u < VD; ++u) xv[j][u] = ok ? raw[k % RING][j][u] : 0u;
        }
        // input pairs (x[j], x[j + D]) of each channel: the low halves of
        // the two dwords for the pair's first channel, the high halves for
        // its second
        uint32_t pr[NWIN][VEC];
#pragma unroll
        for (int j = 0; j < NWIN; ++j)
#pragma unroll
            for (int u = 0; u < VD; ++u) {
                const uint32_t a = xv[j][u], b = j + D < NWIN ? xv[j + D][u] : 0u;
                pr[j][2 * u] = __builtin_amdgcn_perm(b, a, 0x05040100u);
                pr[j][2 * u + 1] = __builtin_amdgcn_perm(b, a, 0x07060302u);
            }
#pragma unroll
        for (int q = 0; q < FH; ++q) {
            const int fh = UP ? FH - 1 - q : q;
            const int o = i - fh * D;
            if (o < 0 || o >= TH) continue;
            float part[TM][VEC];
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int v = 0; v < VEC; ++v) part[t][v] = 0.0f;
#pragma unroll
            for (int kp = 0; kp < NP; ++kp)
#pragma unroll
                for (int t = 0; t < TM; ++t)
#pragma unroll
                    for (int v = 0; v < VEC; ++v) {
                        // an odd width's last tap is paired with a zero tap:
                        // its input pair carries a zero too, so an Inf or NaN
                        // just past the output's window stays out of the sum
                        const int j = t + 2 * kp * D;
                        const uint32_t a =
                            (FW & 1) && kp == NP - 1
                                ? __builtin_amdgcn_perm(0u, xv[j][v / 2],
                                                        (v & 1) ? 0x0c0c0302u : 0x0c0c0100u)
                                : pr[j][v];
                        part[t][v] = Dot2<DT>::dot(a, wp[fh][kp][v], part[t][v]);
                    }
            const bool first = UP ? fh == FH - 1 : fh == 0;
            const bool last = UP ? fh == 0 : fh == FH - 1;
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    acc[o][t][v] = (first ? b0[v] : acc[o][t][v]) + part[t][v];
            if (last && oh0 + o < s.OH) {
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    if (ow0 + t < s.OW) {
                        Y ov[VEC];
#pragma unroll
                        for (int v = 0; v < VEC; ++v) ov[v] = DT::narrow(acc[o][t][v]);
                        store_out<Y, VEC, NT>(yn + ((long long)o * s.OW + t) * s.C, ov);
                    }
                }
            }
        }
    }
}

// Neighbouring strips share (FH-1)D input rows.  Strips walk in alternating
// directions, so that the two strips on either side of every boundary reach
// the shared rows at about the same time (both at the start of their walk, or
// both at the end) and the second request finds them in L2.
template <class DT, int VEC, int FH, int FW, int TM, int TH, int D, int PF, bool NT, int NTL,
          bool BN>
__global__ void __launch_bounds__(256)
k_colstream(const typename DT::X *__restrict__ x, const typename DT::X *__restrict__ w,
            const typename DT::Bias *__restrict__ bias, typename DT::Y *__restrict__ y,
            Shape s, int ncv, int owg_n, int ohg_n, long long total,
            const float *__restrict__ bns, const float *__restrict__ bnb, int act) {
    using X = typename DT::X;
    using Acc = typename DT::Acc;

    const uint32_t b = xcd_remap(blockIdx.x, gridDim.x);
    const long long g = (long long)b * blockDim.x + threadIdx.x;
    if (g >= total) return;
    const int cv = (int)(g % ncv);
    long long r = g / ncv;
    const int owg = (int)(r % owg_n);
    r /= owg_n;
    const int ohg = (int)(r % ohg_n);
    const long long n = r / ohg_n;
    const int c0 = cv * VEC;
    const int ow0 = owg * TM;
    const int oh0 = ohg * TH;
    const int iw0 = ow0 - s.P;
    const int ih0 = oh0 - s.P;
    const X *xn = x + (n * s.H) * (long long)s.W * s.C + c0;

    typename DT::Y *yn = y + ((n * s.OH + oh0) * (long long)s.OW + ow0) * s.C + c0;
    // fp16 / bf16, five or more taps, no prologue: taps paired for v_dot2
    constexpr bool DOT2 =
        (__is_same(DT, F16) || __is_same(DT, BF16)) && FW >= 5 && VEC % 2 == 0 && !BN;
    if constexpr (DOT2) {
        constexpr int NP = (FW + 1) / 2;
        uint32_t wp[FH][NP][VEC];
#pragma unroll
        for (int fh = 0; fh < FH; ++fh)
#pragma unroll
            for (int kp = 0; kp < NP; ++kp) {
                X e0[VEC], e1[VEC];
                load_vec<X, VEC>(e0, w + (long long)tap_index(s, fh, 2 * kp) * s.C + c0);
                if (2 * kp + 1 < FW)
                    load_vec<X, VEC>(e1, w + (long long)tap_index(s, fh, 2 * kp + 1) * s.C + c0);
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    wp[fh][kp][v] = (uint32_t)__builtin_bit_cast(uint16_t, e0[v]) |
                                    (2 * kp + 1 < FW
                                         ? (uint32_t)__builtin_bit_cast(uint16_t, e1[v]) << 16
                                         : 0u);
            }
        float bd[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) bd[v] = bias ? bias[c0 + v] : 0.0f;
        if (ohg & 1)
            colstream_walk_dot2<DT, VEC, FH, FW, TM, TH, D, PF, NT, NTL, true>(
                xn, wp, bd, yn, s, ih0, iw0, oh0, ow0);
        else
            colstream_walk_dot2<DT, VEC, FH, FW, TM, TH, D, PF, NT, NTL, false>(
                xn, wp, bd, yn, s, ih0, iw0, oh0, ow0);
        return;
    }
    Acc wt[FH][FW][VEC];
#pragma unroll
    for (int fh = 0; fh < FH; ++fh)
#pragma unroll
        for (int fw = 0; fw < FW; ++fw) {
            X e[VEC];
            load_vec<X, VEC>(e, w + (long long)tap_index(s, fh, fw) * s.C + c0);
#pragma unroll
            for (int v = 0; v < VEC; ++v) wt[fh][fw][v] = DT::widen(e[v]);
        }
    Acc b0[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) b0[v] = bias ? bias[c0 + v] : Acc(0);
    float bs[VEC], bb[VEC];
    if constexpr (BN) load_bn<VEC>(bs, bb, bns, bnb, c0);

    if (ohg & 1)
        colstream_walk<DT, VEC, FH, FW, TM, TH, D, PF, NT, NTL, true, BN>(
            xn, wt, b0, yn, s, ih0, iw0, oh0, ow0, bs, bb, act);
    else
        colstream_walk<DT, VEC, FH, FW, TM, TH, D, PF, NT, NTL, false, BN>(
            xn, wt, b0, yn, s, ih0, iw0, oh0, ow0, bs, bb, act);
}

template <class DT, int VEC, int FW, int TM, int S, int D, bool BN>
static hipError_t run_rowwin(const Plan &p, const void *x, const void *w, const void *bias,
                             const float *bns, const float *bnb, int act, void *y,
                             hipStream_t st) {
    long long total = (long long)p.aux0 * p.aux1 * p.s.N * p.s.OH;
    hipLaunchKernelGGL((k_rowwin<DT, VEC, FW, TM, S, D, BN>), dim3(p.grid), dim3(p.block), 0,
                       st, (const typename DT::X *)x, (const typename DT::X *)w,
                       (const typename DT::Bias *)bias, (typename DT::Y *)y, p.s, p.aux0,
                       p.aux1, total, bns, bnb, act);
    return hipGetLastError();
}
template <class DT, int VEC, int FW, int TM, int S, int D>
static hipError_t launch_rowwin(const Plan &p, const void *x, const void *w,
                                const void *bias, void *y, hipStream_t st) {
    return run_rowwin<DT, VEC, FW, TM, S, D, false>(p, x, w, bias, nullptr, nullptr, 0, y, st);
}
template <class DT, int VEC, int FW, int TM, int S, int D>
static hipError_t launch_rowwin_bn(const Plan &p, const void *x, const void *w,
                                   const void *bias, const float *bns, const float *bnb,
                                   int act, void *y, hipStream_t st) {
    return run_rowwin<DT, VEC, FW, TM, S, D, true>(p, x, w, bias, bns, bnb, act, y, st);
}

template <class DT, int VEC, int TM, int CH, bool BN>
static hipError_t run_rowchunk(const Plan &p, const void *x, const void *w, const void *bias,
                               const float *bns, const float *bnb, int act, void *y,
                               hipStream_t st) {
    long long total = (long long)p.aux0 * p.aux1 * p.s.N * p.s.OH;
    hipLaunchKernelGGL((k_rowchunk<DT, VEC, TM, CH, BN>), dim3(p.grid), dim3(p.block), 0, st,
                       (const typename DT::X *)x, (const typename DT::X *)w,
                       (const typename DT::Bias *)bias, (typename DT::Y *)y, p.s, p.aux0,
                       p.aux1, total, bns, bnb, act);
    return hipGetLastError();
}
template <class DT, int VEC, int TM, int CH>
static hipError_t launch_rowchunk(const Plan &p, const void *x, const void *w,
                                  const void *bias, void *y, hipStream_t st) {
    return run_rowchunk<DT, VEC, TM, CH, false>(p, x, w, bias, nullptr, nullptr, 0, y, st);
}
template <class DT, int VEC, int TM, int CH>
static hipError_t launch_rowchunk_bn(const Plan &p, const void *x, const void *w,
                                     const void *bias, const float *bns, const float *bnb,
                                     int act, void *y, hipStream_t st) {
    return run_rowchunk<DT, VEC, TM, CH, true>(p, x, w, bias, bns, bnb, act, y, st);
}

template <class DT, int VEC, int FH, int FW, int TM, int TH, int D, int PF, bool NT, int NTL,
          bool BN>
static hipError_t run_colstream(const Plan &p, const void *x, const void *w, const void *bias,
                                const float *bns, const float *bnb, int act, void *y,
                                hipStream_t st) {
    int ohg_n = (p.s.OH + TH - 1) / TH;
    long long total = (long long)p.aux0 * p.aux1 * ohg_n * p.s.N;
    hipLaunchKernelGGL((k_colstream<DT, VEC, FH, FW, TM, TH, D, PF, NT, NTL, BN>), dim3(p.grid),
                       dim3(p.block), 0, st, (const typename DT::X *)x,
                       (const typename DT::X *)w, (const typename DT::Bias *)bias,
                       (typename DT::Y *)y, p.s, p.aux0, p.aux1, ohg_n, total, bns, bnb, act);
    return hipGetLastError();
}
template <class DT, int VEC, int FH, int FW, int TM, int TH, int D, int PF, bool NT, int NTL>
static hipError_t launch_colstream(const Plan &p, const void *x, const void *w,
                                   const void *bias, void *y, hipStream_t st) {
    return run_colstream<DT, VEC, FH, FW, TM, TH, D, PF, NT, NTL, false>(p, x, w, bias, nullptr,
                                                                        nullptr, 0, y, st);
}
template <class DT, int VEC, int FH, int FW, int TM, int TH, int D, int PF, bool NT, int NTL>
static hipError_t launch_colstream_bn(const Plan &p, const void *x, const void *w,
                                      const void *bias, const float *bns, const float *bnb,
                                      int act, void *y, hipStream_t st) {
    return run_colstream<DT, VEC, FH, FW, TM, TH, D, PF, NT, NTL, true>(p, x, w, bias, bns, bnb,
                                                                       act, y, st);
}

// Compiled tilings.  th == 0: row window (any stride); th > 0: column stream
// of th rows (stride 1, FH fixed at compile time).  The first entry that
// matches a shape is the planner's choice; the tuning choice tile=TMxTH[...] picks
// another compiled entry for the same filter (tuning sweeps).
struct RegTile {
    int dtype, fh, fw, s, d, vec, tm, th, pf, nt, ntl;
    LaunchFn fn;
    LaunchBnFn bnfn;  // with the fused prologue (float formats)
};

#define RW(DTE, DTT, FW_, S_, D_, VEC_, TM_)                                          \
    {DTE, 0, FW_, S_, D_, VEC_, TM_, 0, 0, 0, 0, launch_rowwin<DTT, VEC_, FW_, TM_, S_, D_>, \
     launch_rowwin_bn<DTT, VEC_, FW_, TM_, S_, D_>}
#define RWI(DTE, DTT, FW_, S_, D_, VEC_, TM_)                                         \
    {DTE, 0, FW_, S_, D_, VEC_, TM_, 0, 0, 0, 0, launch_rowwin<DTT, VEC_, FW_, TM_, S_, D_>, \
     nullptr}
#define CS(DTE, DTT, FH_, FW_, D_, VEC_, TM_, TH_, PF_, NT_, NTL_)          \
    {DTE, FH_, FW_, 1, D_, VEC_, TM_, TH_, PF_, NT_, NTL_,                 \
     launch_colstream<DTT, VEC_, FH_, FW_, TM_, TH_, D_, PF_, NT_, NTL_>, \
     launch_colstream_bn<DTT, VEC_, FH_, FW_, TM_, TH_, D_, PF_, NT_, NTL_>}

static const RegTile kTiles[] = {
    // fp16 5x5: taps paired for v_dot2_f32_f16, two channels per lane.
    // 4 x 14 outputs per lane with one row prefetched measured within 15 %
    // of the best of six tilings on every map tried (8 x 16, up to 14 %
    // faster on the largest maps, needs more than 256 registers in the walk
    // shared with bf16)
    CS(DT_F16, F16, 5, 5, 1, 2, 4, 14, 1, 1, 0),
    // bf16 5x5 (v_dot2_f32_bf16): faster than the matrix cores only on some
    // maps (by 30 % on 128x32x32x1024, 25 % slower on 64x56x56x96), so the
    // planner keeps bf16 on the matrix cores; this tiling is the row-window
    // family's pick when that family is asked for
    CS(DT_BF16, BF16, 5, 5, 1, 2, 4, 14, 1, 1, 0),
    CS(DT_F32, F32, 3, 3, 1, 4, 4, 14, 2, 1, 2),
    CS(DT_F32, F32, 3, 3, 1, 4, 4, 14, 2, 1, 0),
    // 5x5: two channels per lane keep the 5 x 5 filter and 5 rows of
    // accumulators in registers (measured 18-32 % faster than the row window)
    CS(DT_F32, F32, 5, 5, 1, 2, 4, 16, 2, 1, 0),
    // 7x7 and 9x9 with one channel per lane, four columns and 16 rows (202
    // and 256 registers; measured 36-38 and 31 TFLOP/s on the 128-image maps
    // against 26 for two channels per lane at 7x7, 20 for the 7x7 row window
    // and 22 for 9x9 row chunks; 11x11 and 13x13 were no faster than row
    // chunks)
    CS(DT_F32, F32, 7, 7, 1, 1, 4, 16, 2, 1, 0),
    CS(DT_F32, F32, 9, 9, 1, 1, 4, 16, 2, 1, 0),
    CS(DT_F32, F32, 3, 3, 1, 4, 2, 28, 2, 1, 0),
    CS(DT_F32, F32, 3, 3, 1, 4, 4, 8, 2, 1, 0),
    // fp16 / bf16 3x3: four channels (8 bytes) per lane, four columns
    // (measured 18-28 % faster than eight channels and two columns, which
    // needed all 256 registers)
    CS(DT_F16, F16, 3, 3, 1, 4, 4, 14, 2, 1, 0),
    CS(DT_BF16, BF16, 3, 3, 1, 4, 4, 14, 2, 1, 0),
    CS(DT_F16, F16, 3, 3, 1, 8, 2, 14, 2, 1, 0),
    CS(DT_BF16, BF16, 3, 3, 1, 8, 2, 14, 2, 1, 0),
    RW(DT_F32, F32, 3, 1, 1, 4, 8),
    RW(DT_F32, F32, 5, 1, 1, 4, 8),
    RW(DT_F32, F32, 7, 1, 1, 4, 4),
    RW(DT_F32, F32, 3, 2, 1, 4, 4),
    RW(DT_F32, F32, 5, 2, 2, 4, 4),
    RW(DT_F16, F16, 3, 1, 1, 8, 4),
    RW(DT_F16, F16, 7, 1, 1, 8, 4),
    RW(DT_F16, F16, 5, 2, 2, 8, 2),
    RW(DT_BF16, BF16, 3, 1, 1, 8, 4),
    RW(DT_BF16, BF16, 7, 1, 1, 8, 4),
    RW(DT_BF16, BF16, 31, 1, 1, 2, 4),
    RWI(DT_I8, I8, 3, 1, 1, 4, 4),
    RWI(DT_I8, I8, 5, 2, 2, 4, 2),
};
#undef RW
#undef RWI
#undef CS

static bool tile_matches(const RegTile &k, const Plan &p) {
    if (k.dtype != p.dtype || k.fw != p.s.FW || k.s != p.s.S || k.d != p.s.D) return false;
    if (k.th > 0 && k.fh != p.s.FH) return false;
    return p.s.C % k.vec == 0;  // every pixel a whole number of vectors
}

// Filters no compiled tiling covers, at stride 1 and dilation 1, in float
// formats with whole 16-byte channel vectors: row chunks of 8 taps.
static bool plan_rowchunk(Plan &p) {
    if (p.s.S != 1 || p.s.D != 1 || p.dtype == DT_I8) return false;
    const int VEC = 16 / p.elem_bytes;
    // fp32: 12 outputs per lane (measured 3-8 % faster than 8 on the sweep
    // maps; 16 needed all 256 registers and was slower); the tuning choice
    // chunk_tm=8 picks 8
    int TM = p.dtype == DT_F32 ? 12 : 4;
    if (p.dtype == DT_F32 && tune_int("chunk_tm", 0) == 8) TM = 8;
    if (p.s.C % VEC != 0) return false;
    const int ncv = p.s.C / VEC;
    const int owg_n = (p.s.OW + TM - 1) / TM;
    const long long total = (long long)ncv * owg_n * p.s.OH * p.s.N;
    const long long blocks = (total + 255) / 256;
    if (blocks >= (1LL << 31)) return false;
    p.variant = V_ROWWIN;
    p.vec = VEC;
    p.tm = TM;
    p.th = 0;
    p.tile_h = 1;
    p.tile_w = TM;
    p.tile_c = VEC;
    p.block = 256;
    p.grid = (uint32_t)blocks;
    p.aux0 = ncv;
    p.aux1 = owg_n;
    switch (p.dtype) {
        case DT_F32:
            p.launch = TM == 12 ? launch_rowchunk<F32, 4, 12, 8> : launch_rowchunk<F32, 4, 8, 8>;
            p.bn_launch =
                TM == 12 ? launch_rowchunk_bn<F32, 4, 12, 8> : launch_rowchunk_bn<F32, 4, 8, 8>;
            break;
        case DT_F16:
            p.launch = launch_rowchunk<F16, 8, 4, 8>;
            p.bn_launch = launch_rowchunk_bn<F16, 8, 4, 8>;
            break;
        case DT_BF16:
            p.launch = launch_rowchunk<BF16, 8, 4, 8>;
            p.bn_launch = launch_rowchunk_bn<BF16, 8, 4, 8>;
            break;
        default: return false;
    }
    snprintf(p.desc, sizeof(p.desc),
             "rowchunk: VEC=%d ch/lane, TM=%d outputs/lane, 8-tap chunks of a %dx%d filter, "
             "%u x %d", VEC, TM, p.s.FH, p.s.FW, p.grid, p.block);
    return true;
}

bool plan_rowwin(Plan &p) {
    const RegTile *e = nullptr;
    // tuning choice tile=TMxTH[pPF[flags]], flags: n = non-temporal y
    // stores, l = non-temporal x loads, i = non-temporal loads of the pixels
    // no other strip reads (the table order is the default)
    int want_tm = 0, want_th = -1, want_pf = -1, want_nt = -1, want_ntl = -1;
    char tbuf[32];
    if (const char *env = tune("tile", tbuf, sizeof(tbuf))) {
        char rest[8] = {0};
        int got = sscanf(env, "%dx%dp%d%7s", &want_tm, &want_th, &want_pf, rest);
        if (got < 2) want_th = -1;
        if (got >= 3) {
            want_nt = strchr(rest, 'n') != nullptr;
            want_ntl = strchr(rest, 'l') != nullptr ? 1 : strchr(rest, 'i') != nullptr ? 2 : 0;
        }
    }
    for (const auto &k : kTiles) {
        if (!tile_matches(k, p)) continue;
        if (want_th >= 0 && (k.tm != want_tm || k.th != want_th)) continue;
        if (want_pf >= 0 && k.pf != want_pf) continue;
        if (want_nt >= 0 && k.nt != want_nt) continue;
        if (want_ntl >= 0 && k.ntl != want_ntl) continue;
        e = &k;
        break;
    }
    if (!e && want_th >= 0) return false;  // asked for a tiling that is not compiled
    if (!e) return plan_rowchunk(p);
    int ncv = p.s.C / e->vec;
    int owg_n = (p.s.OW + e->tm - 1) / e->tm;
    long long rows = e->th > 0 ? (long long)(p.s.OH + e->th - 1) / e->th : p.s.OH;
    long long total = (long long)ncv * owg_n * rows * p.s.N;
    // fp32 column streams launch one-wavefront workgroups: with four
    // wavefronts per group the 3x3 layer's 448 groups left some CUs two and
    // others one, and the single-wavefront launch measured 2-10 % faster on
    // fp32 3x3 to 9x9 (fp16/bf16 3x3 measured no gain and keeps 256)
    const int bs = e->th > 0 && p.elem_bytes == 4 ? 64 : 256;
    long long blocks = (total + bs - 1) / bs;
    if (blocks >= (1LL << 31)) return false;
    p.variant = V_ROWWIN;
    p.vec = e->vec;
    p.tm = e->tm;
    p.th = e->th;
    p.tile_h = e->th > 0 ? e->th : 1;
    p.tile_w = e->tm;
    p.tile_c = e->vec;
    p.block = bs;
    p.grid = (uint32_t)blocks;
    p.aux0 = ncv;
    p.aux1 = owg_n;
    p.launch = e->fn;
    p.bn_launch = e->bnfn;
    if (e->th > 0)
        snprintf(p.desc, sizeof(p.desc),
                 "colstream: VEC=%d ch/lane, TM=%d x TH=%d outputs/lane, %dx%d D=%d, "
                 "prefetch %d rows%s%s, %u x %d",
                 e->vec, e->tm, e->th, e->fh, e->fw, e->d, e->pf,
                 e->nt ? ", nt stores" : "",
                 e->ntl == 1 ? ", nt loads" : e->ntl == 2 ? ", nt loads of unshared pixels" : "",
                 p.grid, p.block);
    else
        snprintf(p.desc, sizeof(p.desc),
                 "rowwin: VEC=%d ch/lane, TM=%d outputs/lane, FW=%d S=%d D=%d, %u x %d",
                 e->vec, e->tm, e->fw, e->s, e->d, p.grid, p.block);
    return true;
}

}  // namespace dw
