// k_direct.hip -- the "direct" kernel family: one lane per output element.
//
// Runs every shape, dtype and alignment, so it is the fallback for pointers
// that are not 16-byte aligned and for channel counts whose pixel is not a
// whole number of 16-byte vectors.  Consecutive lanes take consecutive
// channels of one output pixel, so each tap's loads are contiguous along C
// (channel-last layout, "Flash-DWC: Making Depthwise Convolution
// Compute-Efficient on GPUs", section 2.3).
//
// Each filter row is summed into its own fresh partial, which is then added
// to the running sum; the bias seeds that sum once, and nothing is rounded
// to the storage type before the final store ("Tiles, halos and partial
// sums", section "Partition tensors to fit storage"; "Flash-DWC", section
// 3.3 decomposes the 2-D filter into FH one-dimensional rows).
#include "plan.h"

#include <stdio.h>

namespace dw {

// BN: every in-image input value goes through the fused prologue
// act(x * bns[c] + bnb[c]) first (float formats only).
template <class DT, bool BN>
__global__ void __launch_bounds__(256)
k_direct(const typename DT::X *__restrict__ x, const typename DT::X *__restrict__ w,
         const typename DT::Bias *__restrict__ bias, typename DT::Y *__restrict__ y,
         Shape s, long long total, const float *__restrict__ bns,
         const float *__restrict__ bnb, int act) {
    using Acc = typename DT::Acc;
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
         o += stride) {
        int c = (int)(o % s.C);
        long long r = o / s.C;
        int ow = (int)(r % s.OW);
        r /= s.OW;
        int oh = (int)(r % s.OH);
        long long n = r / s.OH;
        Acc acc = bias ? bias[c] : Acc(0);
        Acc bs = Acc(0), bb = Acc(0);
        if constexpr (BN) {
            bs = bns[c];
            bb = bnb[c];
        }
        for (int fh = 0; fh < s.FH; ++fh) {
            int ih = oh * s.S - s.P + fh * s.D;
            if ((unsigned)ih >= (unsigned)s.H) continue;  // generated zero rows
            const typename DT::X *xr = x + ((n * s.H + ih) * (long long)s.W) * s.C + c;
            const typename DT::X *wc = w + c;
            Acc row = Acc(0);
            for (int fw = 0; fw < s.FW; ++fw) {
                int iw = ow * s.S - s.P + fw * s.D;
                if ((unsigned)iw >= (unsigned)s.W) continue;  // generated zeros
                Acc xv = DT::widen(xr[(long long)iw * s.C]);
                if constexpr (BN) xv = bn_act_stored<DT>(xv, bs, bb, act);
                row = mac<Acc>(row, xv, DT::widen(wc[(long long)tap_index(s, fh, fw) * s.C]));
            }
            acc += row;
        }
        y[o] = DT::narrow(acc);
    }
}

template <class DT>
static hipError_t launch_direct(const Plan &p, const void *x, const void *w,
                                const void *bias, void *y, hipStream_t st) {
    long long total = (long long)p.s.N * p.s.OH * p.s.OW * p.s.C;
    hipLaunchKernelGGL((k_direct<DT, false>), dim3(p.grid), dim3(p.block), 0, st,
                       (const typename DT::X *)x, (const typename DT::X *)w,
                       (const typename DT::Bias *)bias, (typename DT::Y *)y, p.s, total,
                       nullptr, nullptr, 0);
    return hipGetLastError();
}

template <class DT>
static hipError_t launch_direct_bn(const Plan &p, const void *x, const void *w,
                                   const void *bias, const float *bns, const float *bnb,
                                   int act, void *y, hipStream_t st) {
    long long total = (long long)p.s.N * p.s.OH * p.s.OW * p.s.C;
    hipLaunchKernelGGL((k_direct<DT, true>), dim3(p.grid), dim3(p.block), 0, st,
                       (const typename DT::X *)x, (const typename DT::X *)w,
                       (const typename DT::Bias *)bias, (typename DT::Y *)y, p.s, total, bns,
                       bnb, act);
    return hipGetLastError();
}

// Backward data for any shape (the gradient with respect to the input,
// "Flash-DWC: Making Depthwise Convolution Compute-Efficient on GPUs",
// section 5.1), one lane per input element:
//
//   dX[n,ih,iw,c] = sum over taps (fh, fw) with ih + P - fh*D = oh*S and
//                   iw + P - fw*D = ow*S, 0 <= oh < OH, 0 <= ow < OW,
//                   of dY[n,oh,ow,c] * W[fh,fw,c]
//
// i.e. the taps through which the forward pass read this input element.  As
// in the forward kernel, each filter row's products form a fresh fp32
// partial added to the running sum, rounded once at the store.  s is the
// forward shape; dy is N x OH x OW x C, dx is N x H x W x C.
template <class DT>
__global__ void __launch_bounds__(256)
k_bwd_direct(const typename DT::X *__restrict__ dy, const typename DT::X *__restrict__ w,
             typename DT::Y *__restrict__ dx, Shape s, long long total) {
    using Acc = typename DT::Acc;
    const long long stride = (long long)gridDim.x * blockDim.x;
    for (long long o = (long long)blockIdx.x * blockDim.x + threadIdx.x; o < total;
         o += stride) {
        const int c = (int)(o % s.C);
        long long r = o / s.C;
        const int iw = (int)(r % s.W);
        r /= s.W;
        const int ih = (int)(r % s.H);
        const long long n = r / s.H;
        Acc acc = Acc(0);
        for (int fh = 0; fh < s.FH; ++fh) {
            const int th = ih + s.P - fh * s.D;  // = oh * S for a contributing tap
            if (th < 0) break;                   // and for every later fh
            if (th % s.S) continue;
            const int oh = th / s.S;
            if (oh >= s.OH) continue;
            const typename DT::X *gr = dy + ((n * s.OH + oh) * (long long)s.OW) * s.C + c;
            Acc row = Acc(0);
            for (int fw = 0; fw < s.FW; ++fw) {
                const int tw = iw + s.P - fw * s.D;
                if (tw < 0) break;
                if (tw % s.S) continue;
                const int ow = tw / s.S;
                if (ow >= s.OW) continue;
                row = mac<Acc>(row, DT::widen(gr[(long long)ow * s.C]),
                               DT::widen(w[(long long)(fh * s.FW + fw) * s.C + c]));
            }
            acc += row;
        }
        dx[o] = DT::narrow(acc);
    }
}

template <class DT>
static hipError_t launch_bwd_direct(const Plan &p, const void *dy, const void *w,
                                    const void *, void *dx, hipStream_t st) {
    const long long total = (long long)p.s.N * p.s.H * p.s.W * p.s.C;
    hipLaunchKernelGGL(k_bwd_direct<DT>, dim3(p.grid), dim3(p.block), 0, st,
                       (const typename DT::X *)dy, (const typename DT::X *)w,
                       (typename DT::Y *)dx, p.s, total);
    return hipGetLastError();
}

bool plan_bwd_direct(Plan &b, const Plan &f) {
    b = f;
    b.s.flip = 0;
    b.bn_launch = b.bn_fallback = nullptr;
    const long long total = (long long)f.s.N * f.s.H * f.s.W * f.s.C;
    b.variant = V_DIRECT;
    b.block = 256;
    const long long blocks = (total + 255) / 256;
    b.grid = (uint32_t)(blocks < (1LL << 20) ? blocks : (1LL << 20));
    switch (f.dtype) {
        case DT_F32: b.launch = launch_bwd_direct<F32>; break;
        case DT_F16: b.launch = launch_bwd_direct<F16>; break;
        case DT_BF16: b.launch = launch_bwd_direct<BF16>; break;
        default: return false;
    }
    b.fallback = b.launch;
    snprintf(b.desc, sizeof(b.desc), "direct (backward data): 1 input element/lane, any "
             "stride, dilation and filter shape, %u x %d", b.grid, b.block);
    return true;
}

bool plan_direct(Plan &p) {
    long long total = (long long)p.s.N * p.s.OH * p.s.OW * p.s.C;
    p.variant = V_DIRECT;
    p.block = 256;
    long long blocks = (total + 255) / 256;
    // grid-stride beyond 2^20 workgroups: plenty to fill 256 CUs
    p.grid = (uint32_t)(blocks < (1LL << 20) ? blocks : (1LL << 20));
    p.vec = 1;
    p.tm = 1;
    p.tile_h = p.tile_w = p.tile_c = 1;
    switch (p.dtype) {
        case DT_F32: p.launch = launch_direct<F32>; p.bn_launch = launch_direct_bn<F32>; break;
        case DT_F16: p.launch = launch_direct<F16>; p.bn_launch = launch_direct_bn<F16>; break;
        case DT_BF16: p.launch = launch_direct<BF16>; p.bn_launch = launch_direct_bn<BF16>; break;
        case DT_I8: p.launch = launch_direct<I8>; p.bn_launch = nullptr; break;
        default: return false;
    }
    p.bn_fallback = p.bn_launch;
    snprintf(p.desc, sizeof(p.desc), "direct: 1 output/lane, %u x %d", p.grid, p.block);
    return true;
}

}  // namespace dw
