// k_bwf_mfma.hip -- the backward-filter pass on the gfx950 matrix cores
// (fp16 / bf16 in, fp32 accumulate; stride 1, dilation 1).
//
// "Flash-DWC: Making Depthwise Convolution Compute-Efficient on GPUs",
// section 5.1, defines the filter gradient as a sum over the batch and the
// output positions of input x output gradient for every tap:
//
//   dW[fh][fw][c] = sum_{n, oh, ow} X[n, oh - P + fh, ow - P + fw, c] * dY[n, oh, ow, c]
//
// For one channel and one output row oh, put j = ow + fw (a column of the
// input padded by P on the left).  Then the contribution of the row is a
// product of the padded input rows with a banded (Toeplitz) matrix built from
// the gradient row, which gfx950's v_mfma_f32_16x16x32_{f16,bf16} computes:
//
//   D[i][t] += sum_k A[i][k] * B[k][t]        A 16x32, B 32x16, D 16x16 fp32
//
//   i = fh - 16 I     (16 filter rows of row tile I)
//   t = fw - 16 T     (16 filter columns of column tile T)
//   k = j - 16 T - 32 m  (32 padded input columns of window m)
//   A[i][k] = Xpad[oh + fh][j]
//   B[k][t] = dY[oh][32 m + k - t]     (zero outside 0 <= ow < OW)
//
// B does not depend on T, so one B operand per window serves every tile; the
// windows m = 0 .. WN-1 cover every ow once for each filter column kept.
// This is the banded-GEMM shape the forward pass uses (section 4.2 of the
// same page) with the roles of the filter and the output gradient exchanged.
//
// Workgroup (4 wavefronts): one image, CS channels (CS / 4 per wavefront) and
// a chunk of output rows, walked 16 rows at a time.  The padded input rows a
// block needs sit in an LDS ring, channel-major, as in the forward kernel:
// a lane's row advances by one per output row, and every lane reads its A
// windows of each output row from the ring (measured 5-8 % faster than
// moving row oh's operands down one lane with a DPP row shift and reading
// only the new row); the row pitch of 16 (mod 32) elements puts the 16 rows
// of an A read on distinct LDS banks.  The block's 16 gradient rows
// sit in LDS too, with 16 zero columns in front, and a lane's 8 entries of
// B are 8 consecutive elements at a fixed per-lane offset, read as five
// dwords and a funnel shift.  The next block's input and gradient rows are
// loaded while the current block runs.
//
// Rounding: each MFMA cuts the products of each of its four groups of 8
// toward zero at 2^-24 of the group's largest, adds the groups and the
// accumulator exactly and rounds once (measured on gfx950).  The MFMA chain
// of a block holds at most 16 * WN <= 64 MFMAs; its result is added to a
// per-chunk fp32 total, at most 64 blocks per chunk; the chunk totals go to
// the workspace and are merged pairwise by pass 2.  The worst-case error is
// therefore about (64 + 64 + 7 + log2 Z + 4) * 2^-24 * sum |x * dy|, below
// 1e-5 * sum |x * dy| for every Z < 2^24.
#include "plan.h"

#include <stdio.h>
#include <stdlib.h>

namespace dw {

namespace {

typedef float bf_f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 bf_f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf_bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int bf_u32x4 __attribute__((ext_vector_type(4)));

template <class DT>
struct BwfMma;
template <>
struct BwfMma<F16> {
    static __device__ __forceinline__ bf_f32x4 run(bf_u32x4 a, bf_u32x4 b, bf_f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(bf_f16x8, a),
                                                      __builtin_bit_cast(bf_f16x8, b), c, 0, 0,
                                                      0);
    }
};
template <>
struct BwfMma<BF16> {
    static __device__ __forceinline__ bf_f32x4 run(bf_u32x4 a, bf_u32x4 b, bf_f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf_bf16x8, a),
                                                       __builtin_bit_cast(bf_bf16x8, b), c, 0,
                                                       0, 0);
    }
};

// LDS geometry of one workgroup.
template <int CS, int NI, int NT, int WN>
struct BwfTile {
    static constexpr int XR = 16 * NI + 15;             // ring rows
    static constexpr int XW = 16 * (NT - 1) + 32 * WN;  // ring columns (padded input)
    static constexpr int PITCH = XW % 32 == 16 ? XW : XW + 16;  // see the header
    static constexpr int GW = 32 * WN;                  // gradient columns per row
    static constexpr int GPITCH = GW + 24;              // 16 zero columns in front, slack behind
    static constexpr int ELEMS = CS * XR * PITCH + CS * 16 * GPITCH;
};

}  // namespace

template <class DT, int CS, int NI, int NT, int WN>
__global__ void __launch_bounds__(256, 2)  // at most 256 registers
k_bwf_mfma(const uint16_t *__restrict__ x, const uint16_t *__restrict__ dy,
           float *__restrict__ ws, Shape s, int ncs, int nrc, int rpc) {
    using T = BwfTile<CS, NI, NT, WN>;
    constexpr int XR = T::XR, XW = T::XW, PITCH = T::PITCH;
    constexpr int GW = T::GW, GPITCH = T::GPITCH;
    constexpr int NCH = CS / 4;     // channels per wavefront
    constexpr int NWIN = NT * WN;   // A windows per row tile
    static_assert(CS == 4 || CS == 8, "channel slice of 4 or 8");
    static_assert(16 * WN <= 64, "a block's MFMA chain stays within 64 MFMAs");
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];
    uint16_t *xt = lds;                    // [CS][XR][PITCH]
    uint16_t *gt = xt + CS * XR * PITCH;   // [CS][16][GPITCH]

    // workgroup -> (image, row chunk, channel slice); the slices of one
    // chunk run together and share the L2 lines of its pixels
    const uint32_t bid = xcd_remap(blockIdx.x, gridDim.x);
    const int cs = bid % ncs;
    const uint32_t r = bid / ncs;
    const int rc = r % nrc;
    const int n = r / nrc;
    const int c0 = cs * CS;
    const int oh0 = rc * rpc;
    const int oh1 = oh0 + rpc < s.OH ? oh0 + rpc : s.OH;
    const int nblk = (oh1 - oh0 + 15) / 16;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const uint16_t *xn = x + (long long)n * s.H * s.W * s.C + c0;
    const uint16_t *gn = dy + (long long)n * s.OH * s.OW * s.C + c0;
    const int WC = s.W * s.C;    // elements of one input row (< 2^31)
    const int GC = s.OW * s.C;   // elements of one gradient row

    typedef uint32_t PixV __attribute__((ext_vector_type(CS / 2)));
    auto ld1 = [](const uint16_t *src) { return *reinterpret_cast<const PixV *>(src); };

    // Column pair e = tid + 256 u of a 16-row chunk: row e / (XW/2), columns
    // 2 (e % (XW/2)) and the next one.
    constexpr int HX = XW / 2, NEWX = (16 * HX + 255) / 256;
    int xrow[NEWX], xcol[NEWX], xoff[NEWX];
    bool xin[NEWX], xok0[NEWX], xok1[NEWX];
#pragma unroll
    for (int u = 0; u < NEWX; ++u) {
        const int e = tid + 256 * u;
        xin[u] = e < 16 * HX;
        xrow[u] = e / HX;
        xcol[u] = 2 * (e % HX);
        const int iw = xcol[u] - s.P;
        xok0[u] = xin[u] && (unsigned)iw < (unsigned)s.W;
        xok1[u] = xin[u] && (unsigned)(iw + 1) < (unsigned)s.W;
        xoff[u] = iw * s.C;
    }
    constexpr int HG = GW / 2, NEWG = 16 * HG / 256;
    static_assert(16 * HG == 256 * NEWG, "gradient pairs fill the workgroup");
    int grow[NEWG], gcol[NEWG];
    bool gok0[NEWG], gok1[NEWG];
#pragma unroll
    for (int u = 0; u < NEWG; ++u) {
        const int e = tid + 256 * u;
        grow[u] = e / HG;
        gcol[u] = 2 * (e % HG);
        gok0[u] = gcol[u] < s.OW;
        gok1[u] = gcol[u] + 1 < s.OW;
    }

    // padded input rows oh0 + L for L in [L0, L0 + 16), below rlimit; zeros
    // outside the image
    auto fetch_x = [&](PixV(&v)[NEWX][2], int L0, int rlimit) {
#pragma unroll
        for (int u = 0; u < NEWX; ++u) {
            const int ih = oh0 + L0 + xrow[u] - s.P;
            const bool rok = (unsigned)ih < (unsigned)s.H && L0 + xrow[u] < rlimit;
            const uint16_t *src = xn + (long long)ih * WC + xoff[u];
            v[u][0] = rok && xok0[u] ? ld1(src) : (PixV)0u;
            v[u][1] = rok && xok1[u] ? ld1(src + s.C) : (PixV)0u;
        }
    };
    // channel-major scatter into the ring: local row L lives in slot L mod XR
    auto scatter_x = [&](const PixV(&v)[NEWX][2], int L0, int rlimit) {
        const int r0m = L0 % XR;
#pragma unroll
        for (int u = 0; u < NEWX; ++u) {
            if (!xin[u] || L0 + xrow[u] >= rlimit) continue;
            int slot = r0m + xrow[u];
            slot -= slot >= XR ? XR : 0;
            uint16_t *dst = xt + slot * PITCH + xcol[u];
#pragma unroll
            for (int k = 0; k < CS / 2; ++k) {
                const uint32_t a = v[u][0][k], b = v[u][1][k];
                *reinterpret_cast<uint32_t *>(dst + (2 * k) * XR * PITCH) =
                    (a & 0xffffu) | (b << 16);
                *reinterpret_cast<uint32_t *>(dst + (2 * k + 1) * XR * PITCH) =
                    (a >> 16) | (b & 0xffff0000u);
            }
        }
    };
    // gradient rows of block blk; rows past the chunk read as zeros
    auto fetch_g = [&](PixV(&v)[NEWG][2], int blk) {
#pragma unroll
        for (int u = 0; u < NEWG; ++u) {
            const int oh = oh0 + 16 * blk + grow[u];
            const bool rok = oh < oh1;
            const uint16_t *src = gn + (long long)oh * GC + (long long)gcol[u] * s.C;
            v[u][0] = rok && gok0[u] ? ld1(src) : (PixV)0u;
            v[u][1] = rok && gok1[u] ? ld1(src + s.C) : (PixV)0u;
        }
    };
    auto scatter_g = [&](const PixV(&v)[NEWG][2]) {
#pragma unroll
        for (int u = 0; u < NEWG; ++u) {
            uint16_t *dst = gt + grow[u] * GPITCH + 16 + gcol[u];
#pragma unroll
            for (int k = 0; k < CS / 2; ++k) {
                const uint32_t a = v[u][0][k], b = v[u][1][k];
                *reinterpret_cast<uint32_t *>(dst + (2 * k) * 16 * GPITCH) =
                    (a & 0xffffu) | (b << 16);
                *reinterpret_cast<uint32_t *>(dst + (2 * k + 1) * 16 * GPITCH) =
                    (a >> 16) | (b & 0xffff0000u);
            }
        }
    };

    // ---- prologue: the gradient buffer zeroed (its 16 leading columns stay
    // zero), ring rows [0, XR) and the first block's gradient rows ----
    {
        constexpr int GEL = CS * 16 * GPITCH;
        static_assert(GEL % 8 == 0, "16-byte zeroing");
        for (int e = 8 * tid; e < GEL; e += 8 * 256)
            *reinterpret_cast<bf_u32x4 *>(gt + e) = (bf_u32x4){0u, 0u, 0u, 0u};
        PixV g0[NEWG][2];
        fetch_g(g0, 0);
        for (int L0 = 0; L0 < XR; L0 += 64) {
            PixV v[4][NEWX][2];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (L0 + 16 * k < XR) fetch_x(v[k], L0 + 16 * k, XR);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (L0 + 16 * k < XR) scatter_x(v[k], L0 + 16 * k, XR);
        }
        __syncthreads();  // zeroing done before the gradient rows land
        scatter_g(g0);
        __syncthreads();
    }

    const int g = lane >> 4;    // k group of A/B, row group of D
    const int t16 = lane & 15;  // row of A, column of B and D
    // This lane's 8 entries of B in window m are gradient elements
    // 32m + 8g - t16 .. +7, stored 16 further on: read from the dword holding
    // element 32m + gb rounded down, shifted right by gsh bits.
    const int gb = 16 + 8 * g - t16;
    const int gbd = gb >> 1, gsh = 16 * (gb & 1);
    const uint16_t *xc[NCH];
    const uint32_t *gc[NCH];
#pragma unroll
    for (int ci = 0; ci < NCH; ++ci) {
        const int c = wave + 4 * ci;
        xc[ci] = xt + c * XR * PITCH + 8 * g;
        gc[ci] = reinterpret_cast<const uint32_t *>(gt + c * 16 * GPITCH) + gbd;
    }

    struct Ops {
        bf_u32x4 A[NCH][NI][NWIN];
        bf_u32x4 B[NCH][WN];
    };
    // A windows of output row oh0 + L: lane t16 of row tile I holds padded
    // row L + 16 I + t16, columns 16 T + 32 m + 8 g .. +7
    auto full_a = [&](Ops &o, int L) {
#pragma unroll
        for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
            for (int I = 0; I < NI; ++I) {
                const uint16_t *xr = xc[ci] + ((L + 16 * I + t16) % XR) * PITCH;
#pragma unroll
                for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                    for (int m = 0; m < WN; ++m)
                        o.A[ci][I][tt * WN + m] =
                            *reinterpret_cast<const bf_u32x4 *>(xr + 16 * tt + 32 * m);
            }
    };
    auto load_b = [&](Ops &o, int srow) {
#pragma unroll
        for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
            for (int m = 0; m < WN; ++m) {
                const uint32_t *gd = gc[ci] + srow * (GPITCH / 2) + 16 * m;
                uint32_t d[5];
#pragma unroll
                for (int q = 0; q < 5; ++q) d[q] = gd[q];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    o.B[ci][m][q] = __builtin_amdgcn_alignbit(d[q + 1], d[q], gsh);
            }
    };

    bf_f32x4 tot[NCH][NI][NT];
#pragma unroll
    for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
        for (int I = 0; I < NI; ++I)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) tot[ci][I][tt] = (bf_f32x4){0.f, 0.f, 0.f, 0.f};

    for (int blk = 0; blk < nblk; ++blk) {
        if (blk) __syncthreads();  // this block's ring and gradient rows are written
        // loads of the next block's 16 new input rows and its gradient rows
        const bool more = blk + 1 < nblk;
        PixV nx[NEWX][2], ng[NEWG][2];
        if (more) {
            fetch_x(nx, 16 * blk + XR, 1 << 30);
            fetch_g(ng, blk + 1);
        }
        const int nst = oh1 - oh0 - 16 * blk < 16 ? oh1 - oh0 - 16 * blk : 16;

        // one fresh MFMA chain per tile and block (at most 16 * WN MFMAs)
        bf_f32x4 acc[NCH][NI][NT];
#pragma unroll
        for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
            for (int I = 0; I < NI; ++I)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) acc[ci][I][tt] = (bf_f32x4){0.f, 0.f, 0.f, 0.f};
        auto mfmas = [&](const Ops &o) {
#pragma unroll
            for (int m = 0; m < WN; ++m)
#pragma unroll
                for (int I = 0; I < NI; ++I)
#pragma unroll
                    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                        for (int ci = 0; ci < NCH; ++ci)
                            acc[ci][I][tt] = BwfMma<DT>::run(o.A[ci][I][tt * WN + m],
                                                             o.B[ci][m], acc[ci][I][tt]);
        };
        Ops o[2];
        full_a(o[0], 16 * blk);
        load_b(o[0], 0);
#pragma unroll
        for (int st = 0; st < 16; ++st) {
            if (st < nst) {  // rows past the chunk's last are skipped (uniform)
                if (st + 1 < 16) {
                    full_a(o[(st + 1) & 1], 16 * blk + st + 1);
                    load_b(o[(st + 1) & 1], st + 1);
                }
                mfmas(o[st & 1]);
            }
            // keep later rows' operands (and their registers) below this
            // row's MFMAs
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
            for (int I = 0; I < NI; ++I)
#pragma unroll
                for (int tt = 0; tt < NT; ++tt) tot[ci][I][tt] += acc[ci][I][tt];

        __syncthreads();  // every wavefront is done with this block's rows
        if (more) {
            scatter_x(nx, 16 * blk + XR, 1 << 30);
            scatter_g(ng);
        }
    }

    // ---- chunk totals, regrouped through LDS into [fh][fw][CS] so that each
    // filter element's CS channels leave as one or two 16-byte stores ----
    __syncthreads();  // the ring is free
    float *ot = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int ci = 0; ci < NCH; ++ci) {
        const int c = wave + 4 * ci;
#pragma unroll
        for (int I = 0; I < NI; ++I)
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int fh = 16 * I + 4 * g + q, fw = 16 * tt + t16;
                    if (fh < s.FH && fw < s.FW) ot[(fh * s.FW + fw) * CS + c] = tot[ci][I][tt][q];
                }
    }
    __syncthreads();
    const int z = n * nrc + rc;
    float *wz = ws + (long long)z * s.FH * s.FW * s.C + c0;
    constexpr int V4 = CS / 4;
    const int nv = s.FH * s.FW * V4;
    for (int e = tid; e < nv; e += 256) {
        const int p = e / V4, q = e - p * V4;
        *reinterpret_cast<bf_f32x4 *>(wz + (long long)p * s.C + 4 * q) =
            *reinterpret_cast<const bf_f32x4 *>(ot + p * CS + 4 * q);
    }
}

template <class DT, int CS, int NI, int NT, int WN>
static hipError_t launch_bwf_mfma(const BwfPlan &b, const void *x, const void *dy, float *dw,
                                  void *ws, hipStream_t st) {
    if (b.mlds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&k_bwf_mfma<DT, CS, NI, NT, WN>),
            hipFuncAttributeMaxDynamicSharedMemorySize, b.mlds);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_bwf_mfma<DT, CS, NI, NT, WN>), dim3(b.mgrid), dim3(256), b.mlds, st,
                       (const uint16_t *)x, (const uint16_t *)dy, (float *)ws, b.s, b.mncs,
                       b.mnrc, b.mrpc);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_bwf_reduce(b.s, (const float *)ws, dw, b.mZ, st);
}

struct BwfMfmaEntry {
    int dtype, cs, ni, nt, wn;
    BwfLaunchFn fn;
    int elems;  // LDS elements of the ring and gradient rows
};

#define BM(DTE, DTT, CS_, NI_, NT_, WN_)                                   \
    {DTE, CS_, NI_, NT_, WN_, launch_bwf_mfma<DTT, CS_, NI_, NT_, WN_>, \
     BwfTile<CS_, NI_, NT_, WN_>::ELEMS}

// Cheapest first: one 16 x 16 tile before the 32 x 32 tiles, fewer windows
// before more, 8-channel slices (16-byte pixel loads) before 4.
static const BwfMfmaEntry kBwfMfma[] = {
    BM(DT_F16, F16, 8, 1, 1, 2),   BM(DT_BF16, BF16, 8, 1, 1, 2),
    BM(DT_F16, F16, 4, 1, 1, 2),   BM(DT_BF16, BF16, 4, 1, 1, 2),
    BM(DT_F16, F16, 4, 1, 1, 4),   BM(DT_BF16, BF16, 4, 1, 1, 4),
    BM(DT_F16, F16, 4, 2, 2, 2),   BM(DT_BF16, BF16, 4, 2, 2, 2),
    BM(DT_F16, F16, 4, 2, 2, 3),   BM(DT_BF16, BF16, 4, 2, 2, 3),
};
#undef BM

bool plan_bwf_mfma(BwfPlan &b) {
    const Shape &s = b.s;
    b.mfma_launch = nullptr;
    if (b.dtype != DT_F16 && b.dtype != DT_BF16) return false;
    if (s.S != 1 || s.D != 1 || s.FH > 32 || s.FW > 32) return false;
    if (tune_int("bwf_valu", 0)) return false;  // tuning choice: VALU pass 1 only
    const int ni = (s.FH + 15) / 16, nt = (s.FW + 15) / 16;
    const BwfMfmaEntry *e = nullptr;
    for (const auto &k : kBwfMfma) {
        if (k.dtype != b.dtype || s.C % k.cs != 0 || k.ni < ni || k.nt < nt) continue;
        // windows needed: every ow once for each kept filter column of the
        // widest column tile
        const int fwt = k.nt > 1 ? 16 : s.FW;
        if (32 * k.wn < s.OW + fwt - 1) continue;
        const int lds = 2 * k.elems;
        if (lds > 80 * 1024) continue;  // two workgroups per CU
        if (s.FH * s.FW * k.cs * 4 > lds) continue;  // the regrouped totals fit
        e = &k;
        break;
    }
    if (!e) return false;
    const long long ncs = s.C / e->cs;
    // rows per chunk: whole 16-row blocks, at most 64 of them (the error
    // bound); images are split only when the batch alone gives fewer than
    // 512 workgroups, and then into chunks of at least two blocks
    const int blk_img = (s.OH + 15) / 16;
    const long long base = (long long)s.N * ncs;
    long long nrc = 1;
    if (base < 512) {
        nrc = (512 + base - 1) / base;
        const long long cap = blk_img / 2 > 1 ? blk_img / 2 : 1;
        if (nrc > cap) nrc = cap;
    }
    long long bpc = (blk_img + nrc - 1) / nrc;
    if (bpc > 64) bpc = 64;
    const long long rpc = 16 * bpc;
    nrc = (s.OH + rpc - 1) / rpc;
    const long long grid = base * nrc;
    const long long Z = (long long)s.N * nrc;
    if (grid >= (1LL << 31) || Z >= (1LL << 24)) return false;
    b.mcs = e->cs;
    b.mncs = (int)ncs;
    b.mnrc = (int)nrc;
    b.mrpc = (int)rpc;
    b.mZ = (int)Z;
    b.mgrid = (uint32_t)grid;
    b.mlds = 2 * e->elems;
    b.mfma_launch = e->fn;
    const size_t ws = (size_t)Z * s.FH * s.FW * s.C * sizeof(float);
    if (ws > b.ws_bytes) b.ws_bytes = ws;
    snprintf(b.desc, sizeof(b.desc),
             "bwf mfma: 16x16x32 banded GEMM, %d x %d tiles, %d windows, %d ch x %d rows per "
             "workgroup, Z=%lld, LDS %d B, %u x 256, pairwise merge, workspace %zu B",
             e->ni, e->nt, e->wn, e->cs, (int)rpc, Z, b.mlds, b.mgrid, b.ws_bytes);
    return true;
}

}  // namespace dw
