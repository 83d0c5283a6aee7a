// k_ldstile.hip -- the "ldstile" kernel family: an LDS-staged halo tile of
// flat NHWC rows, for any channel count.
//
// A workgroup computes a tile of TB output rows x 4*TM output columns x all C
// channels of one image.  Its input halo -- RB = (TB-1)S + (FH-1)D + 1 rows by
// CW = (4TM-1)S + (FW-1)D + 1 columns, the span formula of "Tiles, halos and
// partial sums" ("Partition tensors to fit storage") -- is copied into LDS
// first.  In channel-last layout the CW pixels of one tile row are one
// contiguous run of CW*C elements, whatever C is, so the copy is a plain
// 16-byte-granular copy of byte ranges: the run is widened to 16-byte
// boundaries (the extra bytes belong to neighbouring pixels and are never
// used) and needs neither C nor the pixel size to be a multiple of 16.
// Rows outside the image are not fetched; columns outside it are read as
// zeros by the arithmetic (generated padding).
//
// Each lane owns one channel (consecutive lanes, consecutive channels, so
// LDS reads and the int32 / fp stores are contiguous) and TM consecutive
// outputs of a row.  Per filter row it reads the input run those outputs need
// once into registers and sweeps the FW taps over it (width-first reuse,
// "Flash-DWC: Making Depthwise Convolution Compute-Efficient on GPUs", section
// 3.3); each filter row is summed into a fresh partial that is then added to
// the running sum, which the bias seeds once.  The lane's FH x FW filter taps
// stay in registers for the whole tile.
#include "plan.h"

#include <stdio.h>

namespace dw {

template <class DT, int FH, int FW, int S, int D, int TM>
__global__ void __launch_bounds__(256)
k_ldstile(const typename DT::X *__restrict__ x, const typename DT::X *__restrict__ w,
          const typename DT::Bias *__restrict__ bias, typename DT::Y *__restrict__ y,
          Shape s, int TB, int nrb, int nct, int rowb) {
    using X = typename DT::X;
    using Acc = typename DT::Acc;
    constexpr int EB = sizeof(X);
    constexpr int NWIN = (TM - 1) * S + (FW - 1) * D + 1;
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
    const int ct = bid % nct;
    const uint32_t r = bid / nct;
    const int rb = r % nrb;
    const int n = r / nrb;
    const int oh0 = rb * TB;
    const int ow0 = ct * 4 * TM;
    const int ih0 = oh0 * S - s.P;               // first tile row
    const int iw0 = ow0 * S - s.P;               // first tile column
    const int RB = (TB - 1) * S + (FH - 1) * D + 1;
    const int CW = (4 * TM - 1) * S + (FW - 1) * D + 1;
    const long long rowlen = (long long)s.W * s.C * EB;  // bytes of one image row
    const unsigned char *xb = reinterpret_cast<const unsigned char *>(x);

    // ---- stage: tile row rr holds the in-image columns of its CW-pixel run,
    // widened to 16-byte boundaries; lds row byte 16 + (g - a16) holds global
    // byte g, where a16 is the run's start rounded down to 16.  The (row,
    // chunk) pairs of the whole tile are one index space, SU loads per thread
    // in flight at a time. ----
    {
        typedef unsigned int u4 __attribute__((ext_vector_type(4)));
        constexpr int SU = 8;
        const int u_lo = iw0 < 0 ? -iw0 : 0;                // first in-image column
        const int u_hi = (iw0 + CW > s.W ? s.W - iw0 : CW);   // one past the last
        const long long runb = (long long)(u_hi - u_lo) * s.C * EB;
        const int maxch = (int)((runb + 30) >> 4) + 1;        // chunks per row, upper bound
        const int total = u_hi > u_lo ? RB * maxch : 0;
        for (int e0 = threadIdx.x; e0 < total; e0 += 256 * SU) {
            u4 v[SU];
            int dsto[SU];
#pragma unroll
            for (int q = 0; q < SU; ++q) {
                const int e = e0 + 256 * q;
                const int rr = e / maxch, k = e % maxch;
                const int ih = ih0 + rr;
                dsto[q] = -1;
                if (e < total && (unsigned)ih < (unsigned)s.H) {
                    const long long row0 = ((long long)n * s.H + ih) * rowlen;
                    const long long a = row0 + (long long)(iw0 + u_lo) * s.C * EB;
                    const long long a16 = a & ~15LL;
                    const int nchunk = (int)((((a + runb) + 15) & ~15LL) - a16) >> 4;
                    if (k < nchunk) {
                        v[q] = *reinterpret_cast<const u4 *>(xb + a16 + 16LL * k);
                        dsto[q] = rr * rowb + 16 + 16 * k;
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < SU; ++q)
                if (dsto[q] >= 0) *reinterpret_cast<u4 *>(lds + dsto[q]) = v[q];
        }
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ow_w = ow0 + wave * TM;             // this wavefront's first output column
    const int u_w = wave * TM * S;                // its first tile column
    for (int c = lane; c < s.C; c += 64) {
        const Acc bv = bias ? bias[c] : Acc(0);
        // the channel's whole filter, held in registers for the tile
        Acc wt[FH][FW];
#pragma unroll
        for (int fh = 0; fh < FH; ++fh)
#pragma unroll
            for (int fw = 0; fw < FW; ++fw)
                wt[fh][fw] = DT::widen(w[((long long)fh * FW + fw) * s.C + c]);
        for (int oh = oh0; oh < oh0 + TB && oh < s.OH; ++oh) {
            Acc acc[TM];
#pragma unroll
            for (int t = 0; t < TM; ++t) acc[t] = bv;
#pragma unroll
            for (int fh = 0; fh < FH; ++fh) {
                const int ih = oh * S - s.P + fh * D;
                if ((unsigned)ih >= (unsigned)s.H) continue;  // generated zero rows
                const int rr = ih - ih0;
                const long long row0 = ((long long)n * s.H + ih) * rowlen;
                const long long a = row0 + (long long)(iw0 + (iw0 < 0 ? -iw0 : 0)) * s.C * EB;
                // lds byte of (tile column u, channel c): 16 + (g - a16), with
                // g = row0 + (iw0 + u) * C * EB + c * EB
                const int base =
                    (int)(16 + row0 + (long long)iw0 * s.C * EB + c * EB - (a & ~15LL));
                const unsigned char *lr = lds + rr * rowb;
                Acc xw[NWIN];
#pragma unroll
                for (int j = 0; j < NWIN; ++j) {
                    const int u = u_w + j;
                    const int iw = iw0 + u;
                    const bool ok = (unsigned)iw < (unsigned)s.W && u < CW;
                    const int off = base + u * s.C * EB;
                    xw[j] = ok ? DT::widen(*reinterpret_cast<const X *>(lr + (ok ? off : 16)))
                               : Acc(0);
                }
                Acc part[TM];
#pragma unroll
                for (int t = 0; t < TM; ++t) part[t] = Acc(0);
#pragma unroll
                for (int fw = 0; fw < FW; ++fw)
#pragma unroll
                    for (int t = 0; t < TM; ++t)
                        part[t] = mac<Acc>(part[t], xw[t * S + fw * D], wt[fh][fw]);
#pragma unroll
                for (int t = 0; t < TM; ++t) acc[t] += part[t];
            }
            typename DT::Y *yr = y + (((long long)n * s.OH + oh) * s.OW + ow_w) * s.C + c;
#pragma unroll
            for (int t = 0; t < TM; ++t)
                if (ow_w + t < s.OW) yr[(long long)t * s.C] = DT::narrow(acc[t]);
        }
    }
}

template <class DT, int FH, int FW, int S, int D, int TM>
static hipError_t launch_ldstile(const Plan &p, const void *x, const void *w,
                                 const void *bias, void *y, hipStream_t st) {
    if (p.lds_bytes > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&k_ldstile<DT, FH, FW, S, D, TM>),
            hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_ldstile<DT, FH, FW, S, D, TM>), dim3(p.grid), dim3(256), p.lds_bytes, st,
                       (const typename DT::X *)x, (const typename DT::X *)w,
                       (const typename DT::Bias *)bias, (typename DT::Y *)y, p.s, p.th,
                       p.aux0, p.aux1, p.aux2);
    return hipGetLastError();
}

struct LdsEntry {
    int dtype, fh, fw, s, d, tm;
    LaunchFn fn;
};

#define LT(DTE, DTT, F_, S_, D_, TM_) \
    {DTE, F_, F_, S_, D_, TM_, launch_ldstile<DTT, F_, F_, S_, D_, TM_>}

static const LdsEntry kLds[] = {
    LT(DT_I8, I8, 5, 2, 2, 4),   LT(DT_I8, I8, 3, 1, 1, 4),   LT(DT_I8, I8, 5, 1, 1, 4),
    LT(DT_I8, I8, 7, 1, 1, 4),   LT(DT_I8, I8, 3, 2, 1, 4),
    LT(DT_F32, F32, 5, 2, 2, 4), LT(DT_F32, F32, 3, 1, 1, 4), LT(DT_F32, F32, 7, 1, 1, 4),
    LT(DT_F16, F16, 5, 2, 2, 4), LT(DT_F16, F16, 3, 1, 1, 4), LT(DT_F16, F16, 7, 1, 1, 4),
    LT(DT_BF16, BF16, 5, 2, 2, 4), LT(DT_BF16, BF16, 3, 1, 1, 4), LT(DT_BF16, BF16, 7, 1, 1, 4),
};
#undef LT

bool plan_ldstile(Plan &p) {
    const LdsEntry *e = nullptr;
    for (const auto &k : kLds)
        if (k.dtype == p.dtype && k.fh == p.s.FH && k.fw == p.s.FW && k.s == p.s.S &&
            k.d == p.s.D) {
            e = &k;
            break;
        }
    if (!e) return false;
    // the widened 16-byte copy may read up to 15 bytes past a run; it stays
    // inside x when the tensor is a whole number of 16-byte chunks
    const long long xbytes = (long long)p.s.N * p.s.H * p.s.W * p.s.C * p.elem_bytes;
    if (xbytes % 16 != 0) return false;
    const int CW = (4 * e->tm - 1) * p.s.S + (p.s.FW - 1) * p.s.D + 1;
    // a run of CW*C elements widened to 16-byte boundaries spans at most
    // CW*C*size + 30 bytes, written from row byte 16
    const int rowb = (int)(((long long)CW * p.s.C * p.elem_bytes + 48 + 15) & ~15LL);
    // rows per tile: as many as fit 40 KiB of LDS (several workgroups per CU)
    int TB = 1;
    auto rows = [&](int tb) { return (tb - 1) * p.s.S + (p.s.FH - 1) * p.s.D + 1; };
    while (TB < 16 && TB < p.s.OH && (long long)rows(TB + 1) * rowb <= 40 * 1024) ++TB;
    const long long lds = (long long)rows(TB) * rowb;
    if (lds > 160 * 1024) return false;
    const int nrb = (p.s.OH + TB - 1) / TB;
    const int nct = (p.s.OW + 4 * e->tm - 1) / (4 * e->tm);
    const long long blocks = (long long)nrb * nct * p.s.N;
    if (blocks >= (1LL << 31)) return false;
    p.variant = V_LDSTILE;
    p.tm = e->tm;
    p.th = TB;
    p.aux0 = nrb;
    p.aux1 = nct;
    p.aux2 = rowb;
    p.lds_bytes = (int)lds;
    p.block = 256;
    p.grid = (uint32_t)blocks;
    p.launch = e->fn;
    snprintf(p.desc, sizeof(p.desc),
             "ldstile: %d rows x %d cols x all %d ch per workgroup, halo %d x %d pixels in "
             "LDS (%lld B), lane = channel, TM=%d, %u x 256",
             TB, 4 * e->tm, p.s.C, rows(TB), CW, lds, e->tm, p.grid);
    return true;
}

}  // namespace dw
