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

template <class DT, int VEC, int FW, int TM, int S, int D>
__global__ void __launch_bounds__(256)
k_rowwin(const typename DT::X *__restrict__ x, const typename DT::X *__restrict__ w,
         const typename DT::Bias *__restrict__ bias, typename DT::Y *__restrict__ y,
         Shape s, int ncv, int owg_n, long long total) {
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

        // input run of this filter row, widened once
        Acc xw[NWIN][VEC];
#pragma unroll
        for (int j = 0; j < NWIN; ++j) {
            const int iw = iw0 + j;
            if ((unsigned)iw < (unsigned)s.W) {
                X e[VEC];
                load_vec<X, VEC>(e, xr + (long long)iw * s.C);
#pragma unroll
                for (int v = 0; v < VEC; ++v) xw[j][v] = DT::widen(e[v]);
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v) xw[j][v] = Acc(0);
            }
        }
        Acc wt[FW][VEC];
#pragma unroll
        for (int fw = 0; fw < FW; ++fw) {
            X e[VEC];
            load_vec<X, VEC>(e, w + ((long long)fh * FW + fw) * s.C + c0);
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
            store_vec<typename DT::Y, VEC>(yr + (long long)t * s.C, o);
        }
    }
}

template <class DT, int VEC, int FW, int TM, int S, int D>
static hipError_t launch_rowwin(const Plan &p, const void *x, const void *w,
                                const void *bias, void *y, hipStream_t st) {
    long long total = (long long)p.aux0 * p.aux1 * p.s.N * p.s.OH;
    hipLaunchKernelGGL((k_rowwin<DT, VEC, FW, TM, S, D>), dim3(p.grid), dim3(p.block), 0, st,
                       (const typename DT::X *)x, (const typename DT::X *)w,
                       (const typename DT::Bias *)bias, (typename DT::Y *)y, p.s, p.aux0,
                       p.aux1, total);
    return hipGetLastError();
}

struct RowwinEntry {
    int dtype, fw, s, d, vec, tm;
    LaunchFn fn;
};

#define RW(DTE, DTT, FW_, S_, D_, VEC_, TM_) \
    {DTE, FW_, S_, D_, VEC_, TM_, launch_rowwin<DTT, VEC_, FW_, TM_, S_, D_>}

static const RowwinEntry kRowwin[] = {
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
    RW(DT_I8, I8, 3, 1, 1, 4, 4),
    RW(DT_I8, I8, 5, 2, 2, 4, 2),
};
#undef RW

bool plan_rowwin(Plan &p) {
    const RowwinEntry *e = nullptr;
    for (const auto &k : kRowwin)
        if (k.dtype == p.dtype && k.fw == p.s.FW && k.s == p.s.S && k.d == p.s.D) {
            e = &k;
            break;
        }
    if (!e) return false;
    if (p.s.C % e->vec != 0) return false;  // every pixel a whole number of vectors
    int ncv = p.s.C / e->vec;
    int owg_n = (p.s.OW + e->tm - 1) / e->tm;
    long long total = (long long)ncv * owg_n * p.s.N * p.s.OH;
    long long blocks = (total + 255) / 256;
    if (blocks >= (1LL << 31)) return false;
    p.variant = V_ROWWIN;
    p.vec = e->vec;
    p.tm = e->tm;
    p.block = 256;
    p.grid = (uint32_t)blocks;
    p.aux0 = ncv;
    p.aux1 = owg_n;
    p.launch = e->fn;
    snprintf(p.desc, sizeof(p.desc),
             "rowwin: VEC=%d ch/lane, TM=%d outputs/lane, FW=%d S=%d D=%d, %u x %d",
             e->vec, e->tm, e->fw, e->s, e->d, p.grid, p.block);
    return true;
}

}  // namespace dw
