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
// zeros by the arithmetic (generated padding).  When stride and dilation
// share a factor G, every tap row is oh*S - P + fh*D = -P (mod G): the other
// rows of the halo are never used, so only every G-th row is staged (and
// fetched from HBM).
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
#include <stdlib.h>

namespace dw {

// Flat staging shared by the LDS-tile kernels: tile row rr holds image row
// ih0 + G*rr -- the in-image columns of its CW-pixel run starting at image
// column iw0, widened to 16-byte boundaries; lds row byte 16 + (g - a16)
// holds global byte g, where a16 is the run's start rounded down to 16.  The
// (row, chunk) pairs of the whole tile are one index space, SU loads per
// thread in flight at a time.  Rows outside the image are not written.
template <int EB, int G>
__device__ __forceinline__ void stage_flat_rows(unsigned char *lds, const unsigned char *xb,
                                                const Shape &s, int n, int ih0, int iw0,
                                                int RB, int CW, int rowb) {
    typedef unsigned int u4 __attribute__((ext_vector_type(4)));
    constexpr int SU = 8;
    const long long rowlen = (long long)s.W * s.C * EB;   // bytes of one image row
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
            const int ih = ih0 + G * rr;
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

// Byte offset, within its staged lds row, of (tile column 0, channel 0) of
// image row ih: 16 + (g - a16) for the row's own 16-byte alignment.
template <int EB>
__device__ __forceinline__ int flat_row_base(const Shape &s, int n, int ih, int iw0) {
    const long long rowlen = (long long)s.W * s.C * EB;
    const long long a_off = (long long)(iw0 + (iw0 < 0 ? -iw0 : 0)) * s.C * EB;
    const int rmis = (int)((((long long)n * s.H + ih) * rowlen) & 15);
    return (int)(16 + rmis + (long long)iw0 * s.C * EB - ((rmis + a_off) & ~15LL));
}

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
    constexpr int G = gcd_c(S, D);                // tap rows are ih0 + G*k
    const int RB = ((TB - 1) * S + (FH - 1) * D) / G + 1;  // staged rows
    const int CW = (4 * TM - 1) * S + (FW - 1) * D + 1;
    const unsigned char *xb = reinterpret_cast<const unsigned char *>(x);
    const int lane = threadIdx.x & 63;

    // The lane's first channel's filter and bias are requested before the
    // staging copy, so their latency overlaps it.
    Acc wt[FH][FW];
    Acc bv = Acc(0);
    auto load_filter = [&](int c) {
        bv = bias ? bias[c] : Acc(0);
#pragma unroll
        for (int fh = 0; fh < FH; ++fh)
#pragma unroll
            for (int fw = 0; fw < FW; ++fw)
                wt[fh][fw] = DT::widen(w[(long long)tap_index(s, fh, fw) * s.C + c]);
    };
    if (lane < s.C) load_filter(lane);

    stage_flat_rows<EB, G>(lds, xb, s, n, ih0, iw0, RB, CW, rowb);
    __syncthreads();

    const int wave = threadIdx.x >> 6;
    const int ow_w = ow0 + wave * TM;             // this wavefront's first output column
    const int u_w = wave * TM * S;                // its first tile column
    for (int c = lane; c < s.C; c += 64) {
        if (c != lane) load_filter(c);
        for (int oh = oh0; oh < oh0 + TB && oh < s.OH; ++oh) {
            Acc acc[TM];
#pragma unroll
            for (int t = 0; t < TM; ++t) acc[t] = bv;
            // every filter row's window is read branch-free (positions
            // outside the image read row byte 16 of tile row 0 and are
            // replaced by zeros), so all FH x NWIN LDS reads can be in flight
            // together
            Acc xw[FH][NWIN];
#pragma unroll
            for (int fh = 0; fh < FH; ++fh) {
                const int ih = oh * S - s.P + fh * D;
                const bool rok = (unsigned)ih < (unsigned)s.H;
                const int ihc = rok ? ih : ih0;  // out of image: any row, zeroed below
                const int rr = (ihc - ih0) / G;
                // byte of (u = 0, c) in this row, relative to the row's lds start
                const int base = flat_row_base<EB>(s, n, ihc, iw0) + c * EB;
                const unsigned char *lr = lds + rr * rowb;
#pragma unroll
                for (int j = 0; j < NWIN; ++j) {
                    const int u = u_w + j;
                    const int iw = iw0 + u;
                    const bool ok = rok && (unsigned)iw < (unsigned)s.W && u < CW;
                    // outside the image: any staged byte (row byte 16), zeroed below
                    const int off = ok ? base + u * s.C * EB : 16;
                    const Acc v = DT::widen(*reinterpret_cast<const X *>(lr + off));
                    xw[fh][j] = ok ? v : Acc(0);
                }
            }
#pragma unroll
            for (int fh = 0; fh < FH; ++fh) {
                Acc part[TM];
#pragma unroll
                for (int t = 0; t < TM; ++t) part[t] = Acc(0);
#pragma unroll
                for (int fw = 0; fw < FW; ++fw)
#pragma unroll
                    for (int t = 0; t < TM; ++t)
                        part[t] = mac<Acc>(part[t], xw[fh][t * S + fw * D], wt[fh][fw]);
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

// ---------------------------------------------------------------------------
// Tap-packed int8 tile.  When the dilation D divides the stride S, every tap
// column of a tile is u = t*S + fw*D = 0 (mod D) and every tap row is
// ih0 + D*k: only one column in D and one row in D is ever read.  Those are
// staged channel-major -- tile row rr, channel c, tap column k = u / D -- so
// the taps fw..fw+3 that one output of one channel needs are four
// consecutive bytes, and one v_dot4_i32_i8 multiplies them by four packed
// filter taps (exact: int8 products summed into int32).  The filter row is
// padded to a whole number of 4-tap dwords with zero taps.  Positions outside
// the image are staged as zeros, so the arithmetic has no selects.
//
// Workgroup = TB output rows x 4*TM output columns x all C channels of one
// image; wavefront w owns the tile's output columns w*TM .. w*TM + TM - 1;
// lane = channel.  A lane's window of one staged row is ND aligned dwords; output t
// of tap dword q is a byte shift of two of them.
// ---------------------------------------------------------------------------
template <int FH, int FW, int S, int D, int TM>
__global__ void __launch_bounds__(256)
k_i8tap(const int8_t *__restrict__ x, const int8_t *__restrict__ w,
        const int32_t *__restrict__ bias, int32_t *__restrict__ y, Shape s, int TB, int nrb,
        int nct, int kqp, int rowb) {
    static_assert(S % D == 0, "tap columns share one residue mod D");
    constexpr int SD = S / D;                     // tap-column step between outputs
    constexpr int NQ = (FW + 3) / 4;              // 4-tap dwords per filter row
    static_assert((TM * SD) % 4 == 0, "each wavefront's window starts on a dword");
    constexpr int ND = ((TM - 1) * SD + 4 * NQ + 3) / 4;  // window dwords per staged row
    constexpr int KQ = (4 * TM - 1) * SD + FW;    // tap columns of the tile
    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

    const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
    const int ct = bid % nct;
    const uint32_t r = bid / nct;
    const int rb = r % nrb;
    const int n = r / nrb;
    const int oh0 = rb * TB;
    const int ow0 = ct * 4 * TM;
    const int ih0 = oh0 * S - s.P;                // image row of staged row 0
    const int iw0 = ow0 * S - s.P;                // image column of tap column 0
    const int RB = (TB - 1) * SD + FH;            // staged rows
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int ngrp = (s.C + 63) / 64;             // channel groups of 64 lanes

    // filter of the lane's first channel: the bytes are requested before the
    // staging copy (their latency overlaps it) and packed 4 taps per dword
    // after it
    int8_t t8[FH][4 * NQ];
    uint32_t wq[FH][NQ];
    int32_t bv = 0;
    auto fetch_filter = [&](int c) {
        const int8_t *wc = w + c;
#pragma unroll
        for (int fh = 0; fh < FH; ++fh)
#pragma unroll
            for (int fw = 0; fw < 4 * NQ; ++fw)
                t8[fh][fw] = fw < FW ? wc[tap_index(s, fh, fw) * s.C] : (int8_t)0;
        bv = bias ? bias[c] : 0;
    };
    auto pack_filter = [&]() {
#pragma unroll
        for (int fh = 0; fh < FH; ++fh)
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                wq[fh][q] = (uint32_t)(uint8_t)t8[fh][4 * q] |
                            ((uint32_t)(uint8_t)t8[fh][4 * q + 1] << 8) |
                            ((uint32_t)(uint8_t)t8[fh][4 * q + 2] << 16) |
                            ((uint32_t)(uint8_t)t8[fh][4 * q + 3] << 24);
    };
    if (lane < s.C) fetch_filter(lane);

    // ---- stage 1: the tap rows (image rows ih0 + D*rr) as flat NHWC byte
    // runs of CW pixels, copied in 16-byte chunks ----
    unsigned char *flat = lds;                                    // RB rows x rowb
    unsigned char *cm = lds + (long long)RB * rowb;               // RB x C x kqp
    const int CW = (4 * TM - 1) * S + (FW - 1) * D + 1;
    stage_flat_rows<1, D>(flat, reinterpret_cast<const unsigned char *>(x), s, n, ih0, iw0,
                          RB, CW, rowb);
    __syncthreads();

    // ---- stage 2: channel-major transpose of the tap columns: dword kd of
    // (row rr, channel c) packs tap columns 4kd .. 4kd+3 (tile columns
    // D*k); zeros outside the image.  Rows are shared out over the
    // wavefronts; lane = channel, so every byte read is one of 64 consecutive
    // bytes.  All KQ byte reads of a row are issued before any is used (reads
    // outside the image go to byte c of the first staged row and are masked)
    // so that their LDS latency is paid once per row. ----
    {
        constexpr int KQD = (KQ + 3) / 4;
        const int DC = D * s.C;
        for (int rr = wave; rr < RB; rr += 4) {
            const int ih = ih0 + D * rr;
            const bool rok = (unsigned)ih < (unsigned)s.H;
            const int base = rok ? rr * rowb + flat_row_base<1>(s, n, ih, iw0) : 0;
            for (int g = 0; g < ngrp; ++g) {
                const int c = 64 * g + lane;
                if (c >= s.C) break;
                uint32_t b8[4 * KQD];
#pragma unroll
                for (int k = 0; k < 4 * KQD; ++k) {
                    const int iw = iw0 + D * k;
                    const bool ok = rok && k < KQ && (unsigned)iw < (unsigned)s.W;
                    const uint32_t v = flat[ok ? base + k * DC + c : c];
                    b8[k] = ok ? v : 0u;
                }
#pragma unroll
                for (int kd = 0; kd < KQD; ++kd)
                    *reinterpret_cast<uint32_t *>(cm + ((long long)rr * s.C + c) * kqp + 4 * kd) =
                        b8[4 * kd] | (b8[4 * kd + 1] << 8) | (b8[4 * kd + 2] << 16) |
                        (b8[4 * kd + 3] << 24);
            }
        }
    }
    if (lane < s.C) pack_filter();
    __syncthreads();

    const int ow_w = ow0 + wave * TM;             // the wavefront's first output column
    const int kb = wave * TM * SD;                // its first tap column (dword aligned)
    for (int g = 0; g < ngrp; ++g) {
        const int c = 64 * g + lane;
        if (c >= s.C) break;
        if (g) {
            fetch_filter(c);
            pack_filter();
        }
        for (int oh = oh0; oh < oh0 + TB && oh < s.OH; ++oh) {
            int32_t acc[TM];
#pragma unroll
            for (int t = 0; t < TM; ++t) acc[t] = bv;
            uint32_t win[FH][ND];
#pragma unroll
            for (int fh = 0; fh < FH; ++fh) {
                const int rr = (oh - oh0) * SD + fh;
                const uint32_t *src = reinterpret_cast<const uint32_t *>(
                    cm + ((long long)rr * s.C + c) * kqp + kb);
#pragma unroll
                for (int i = 0; i < ND; ++i) win[fh][i] = src[i];
            }
#pragma unroll
            for (int fh = 0; fh < FH; ++fh)
#pragma unroll
                for (int t = 0; t < TM; ++t)
#pragma unroll
                    for (int q = 0; q < NQ; ++q) {
                        const int bo = t * SD + 4 * q;    // byte offset in the window
                        const int di = bo / 4, sh = bo % 4;
                        const uint32_t a =
                            sh ? __builtin_amdgcn_alignbyte(win[fh][di + 1], win[fh][di], sh)
                               : win[fh][di];
                        acc[t] = __builtin_amdgcn_sdot4((int)a, (int)wq[fh][q], acc[t], false);
                    }
            // y is never read back: stream it past the caches
            int32_t *yr = y + (((long long)n * s.OH + oh) * s.OW + ow_w) * s.C + c;
#pragma unroll
            for (int t = 0; t < TM; ++t)
                if (ow_w + t < s.OW) __builtin_nontemporal_store(acc[t], yr + (long long)t * s.C);
        }
    }
}

template <int FH, int FW, int S, int D, int TM>
static hipError_t launch_i8tap(const Plan &p, const void *x, const void *w, const void *bias,
                               void *y, hipStream_t st) {
    if (p.lds_bytes > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&k_i8tap<FH, FW, S, D, TM>),
            hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_i8tap<FH, FW, S, D, TM>), dim3(p.grid), dim3(256), p.lds_bytes, st,
                       (const int8_t *)x, (const int8_t *)w, (const int32_t *)bias,
                       (int32_t *)y, p.s, p.th, p.aux0, p.aux1, p.aux2, p.aux3);
    return hipGetLastError();
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

struct TapEntry {
    int fh, fw, s, d, tm;
    LaunchFn fn;
};

#define TT(F_, S_, D_, TM_) {F_, F_, S_, D_, TM_, launch_i8tap<F_, F_, S_, D_, TM_>}
static const TapEntry kTap[] = {
    TT(5, 2, 2, 4), TT(3, 1, 1, 4), TT(5, 1, 1, 4), TT(7, 1, 1, 4), TT(3, 2, 1, 4),
    TT(3, 2, 2, 4),
};
#undef TT

// Rows per tile: as many as fit lds_cap bytes of LDS while the grid keeps at
// least min_grid workgroups; the tuning choice lds_tb=n forces n rows.
template <class RowsFn>
static int pick_tb(const Plan &p, int nct, long long row_bytes, RowsFn rows, int min_grid,
                   long long lds_cap) {
    auto grid_of = [&](int tb) { return (long long)((p.s.OH + tb - 1) / tb) * nct * p.s.N; };
    int TB = 1;
    while (TB < 16 && TB < p.s.OH && (long long)rows(TB + 1) * row_bytes <= lds_cap &&
           grid_of(TB + 1) >= min_grid)
        ++TB;
    // tuning choice lds_tb=1..64: the tile height
    const int want = tune_int("lds_tb", 0);
    if (want >= 1 && want <= 64) TB = want < p.s.OH ? want : p.s.OH;
    return TB;
}

static bool plan_i8tap(Plan &p) {
    if (p.dtype != DT_I8 || p.s.S % p.s.D != 0) return false;
    const TapEntry *e = nullptr;
    for (const auto &k : kTap)
        if (k.fh == p.s.FH && k.fw == p.s.FW && k.s == p.s.S && k.d == p.s.D) {
            e = &k;
            break;
        }
    if (!e) return false;
    const int SD = p.s.S / p.s.D, TM = e->tm;
    const int KQ = (4 * TM - 1) * SD + p.s.FW;          // tap columns of a tile
    const int NQ = (p.s.FW + 3) / 4;
    const int ND = ((TM - 1) * SD + 4 * NQ + 3) / 4;
    // dwords per (row, channel): the staged columns and the last wavefront's
    // window must fit; an odd count puts the 64 lanes' reads on distinct banks
    int kqd = (KQ + 3) / 4;
    const int need = (3 * TM * SD) / 4 + ND;
    if (kqd < need) kqd = need;
    if (kqd % 2 == 0) ++kqd;
    const int kqp = 4 * kqd;
    // the flat copy may read up to 15 bytes past a run; it stays inside x
    // when the tensor is a whole number of 16-byte chunks
    const long long xbytes = (long long)p.s.N * p.s.H * p.s.W * p.s.C;
    if (xbytes % 16 != 0) return false;
    const int CW = (4 * TM - 1) * p.s.S + (p.s.FW - 1) * p.s.D + 1;
    const int rowb = (int)(((long long)CW * p.s.C + 48 + 15) & ~15LL);
    // per staged row: the flat run and its channel-major transpose
    const long long row_bytes = rowb + (long long)p.s.C * kqp;
    auto rows = [&](int tb) { return (tb - 1) * SD + p.s.FH; };
    const int nct = (p.s.OW + 4 * TM - 1) / (4 * TM);
    // two workgroups per CU: taller tiles cut the halo rows per output row,
    // which measured faster than more, smaller workgroups
    const int TB = pick_tb(p, nct, row_bytes, rows, 512, 80 * 1024);
    const long long lds = rows(TB) * row_bytes;
    if (lds > 160 * 1024) return false;
    const int nrb = (p.s.OH + TB - 1) / TB;
    const long long blocks = (long long)nrb * nct * p.s.N;
    if (blocks >= (1LL << 31)) return false;
    p.variant = V_LDSTILE;
    p.tm = TM;
    p.th = TB;
    p.tile_h = TB;
    p.tile_w = 4 * TM;
    p.tile_c = p.s.C;
    p.aux0 = nrb;
    p.aux1 = nct;
    p.aux2 = kqp;
    p.aux3 = rowb;
    p.lds_bytes = (int)lds;
    p.block = 256;
    p.grid = (uint32_t)blocks;
    p.launch = e->fn;
    snprintf(p.desc, sizeof(p.desc),
             "ldstile (int8 tap-packed): %d rows x %d cols x all %d ch per workgroup, %d tap "
             "rows x %d tap cols in LDS (%lld B), v_dot4 per 4 taps, %u x 256",
             TB, 4 * TM, p.s.C, rows(TB), KQ, lds, p.grid);
    return true;
}

bool plan_ldstile(Plan &p) {
    if (plan_i8tap(p)) return true;
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
    // staged rows of a tile: only every g-th halo row is ever a tap row
    const int g = gcd_c(p.s.S, p.s.D);
    auto rows = [&](int tb) { return ((tb - 1) * p.s.S + (p.s.FH - 1) * p.s.D) / g + 1; };
    const int nct = (p.s.OW + 4 * e->tm - 1) / (4 * e->tm);
    // at least three workgroups per CU, four fit LDS
    const int TB = pick_tb(p, nct, rowb, rows, 768, 40 * 1024);
    const long long lds = (long long)rows(TB) * rowb;
    if (lds > 160 * 1024) return false;
    const int nrb = (p.s.OH + TB - 1) / TB;
    const long long blocks = (long long)nrb * nct * p.s.N;
    if (blocks >= (1LL << 31)) return false;
    p.variant = V_LDSTILE;
    p.tm = e->tm;
    p.th = TB;
    p.tile_h = TB;
    p.tile_w = 4 * e->tm;
    p.tile_c = p.s.C;
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
