// k_mfma.hip -- the "mfma" kernel family: depthwise convolution as banded GEMMs
// on the gfx950 matrix cores (fp16 / bf16 in, fp32 accumulate; stride 1,
// dilation 1).
//
// "Flash-DWC: Making Depthwise Convolution Compute-Efficient on GPUs",
// section 4.2, turns each channel's GEMV into a small dense GEMM: the taps of
// one filter fragment form a banded (Toeplitz) K x TM matrix whose column t
// holds the taps starting at row t, and TM consecutive outputs of one row
// become one length-K input vector; stacking several such vectors gives the
// left operand.  The pages pack this into NVIDIA's m16n8k16 shape.  Here the
// shape is gfx950's v_mfma_f32_16x16x32_{f16,bf16}:
//
//   D[i][t] += sum_k A[i][k] * B[k][t],   A 16x32, B 32x16, D 16x16 fp32
//
//   i  = one of 16 consecutive output rows (the 16 GEMVs)
//   t  = one of 16 consecutive output columns (TM = 16)
//   k  = one of 32 consecutive input columns (the input window, K = 32)
//   B[k][t] = w[fh][16f + k - t] for 0 <= k - t < 16, else 0
//
// A filter row of FW taps is cut into ceil(FW/16) fragments of 16 taps
// (31 taps -> 16 + 15).  Fragment f of output block b reads the input window
// starting at padded column 16(b+f), so windows are 16-element aligned and
// the window of (b, f=1) is the window of (b+1, f=0).  Only products inside
// one channel are formed: every MFMA works on a single channel, as the pages'
// one-GEMM-per-channel does.
//
// Workgroup (4 wavefronts; 8 for 16-channel slices, and for filters of 41 to
// 61 taps, whose 8 wavefronts split each channel's filter rows in two halves
// summed before the epilogue): one image, a strip of 16*NB output columns and
// CS channels, walked down 16 output rows at a time.  The input a row block needs -- the halo span (16 + FH - 1) rows x 16(NB + NFRAG) columns of
// "Tiles, halos and partial sums", with padding generated as zeros -- sits in
// an LDS ring, channel-major, so that one 16-byte LDS read gives a lane its 8
// consecutive columns of one channel (the A operand); each new block loads
// only its 16 new rows.  The row pitch is 16 (mod 32) elements, which puts the 16 rows
// an A read touches on distinct banks.  The filter slice is staged once as
// padded fragments -- 16 zeros, the fragment's 16 taps, 16 zeros -- so that
// a lane's 8 entries of B, B[k][t] = tap k - t, are 8 consecutive elements at
// a fixed per-lane offset, with the band's zeros built in; the lane reads
// them as five aligned dwords and a 16-bit funnel shift.
//
// Row packing (the default for filters of at most 32 rows and 33 taps, and
// of 34 to 65 taps and at most 64 rows): a
// banded fragment fills only FW of each column's 32 K entries, so the K of
// one MFMA instead holds 2 or 4 filter rows of 16 or 8 input columns each;
// the kernel comment below gives the operand layout.  Fewer MFMAs and one A
// read per group of rows instead of one per row.
//
// The partial sums stay fp32 in the MFMA accumulators for the whole filter,
// seeded once with the bias.  How one MFMA adds its products was measured on
// gfx950 (the same for fp16 and bf16): the 32 products form four groups of 8
// consecutive k; inside a group each product is cut toward zero to a
// multiple of 2^(e-24), e the exponent of the group's largest product; the
// group sums and the accumulator are added exactly and rounded once, to
// nearest even.  One MFMA therefore errs by less than 7 * 2^-24 * sum|p| of
// its own products plus one rounding of its result, and a chain of at most
// 64 MFMAs (FH <= 32, two fragments; with row packing at most 48, or 64
// where taller and wider filters fold the chain into an fp32 total) by less
// than (7 + 64) * 2^-24 * sum|x*w| < 1e-5 * sum|x*w|.  Each group of 8
// consecutive k lies in one filter row, packed or not.  The epilogue rounds once to
// fp16/bf16 and goes through LDS so that the stores are whole channel
// vectors of NHWC pixels, masked at the ragged right and bottom edges.
#include "plan.h"

#include <stdio.h>
#include <stdlib.h>

#include <type_traits>

namespace dw {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <class DT>
struct MfmaOp;
template <>
struct MfmaOp<F16> {
    static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
};
template <>
struct MfmaOp<BF16> {
    static __device__ __forceinline__ f32x4 run(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
};

// LDS geometry of one workgroup strip.  PK = 1: K windows of 32 input
// columns at steps of 16, NFRAG fragments of 16 taps per filter row.
// PK > 1 (row packing): the K of one MFMA holds PK filter rows of
// KW = 32 / PK input columns each, and NFRAG is the number J of KW-column
// windows one 16-column output block reads per group of PK rows.
template <int CS, int NB, int NFRAG, int PK = 1, int KS = 1>
struct MfmaTile {
    static constexpr int KW = 32 / PK;
    // distinct A windows per filter row (PK = 1) or row group (PK > 1)
    static constexpr int NWIN = PK == 1 ? NB + NFRAG - 1 : (PK / 2) * (NB - 1) + NFRAG;
    static constexpr int XW = PK == 1 ? 16 * (NB + NFRAG) : KW * NWIN;  // staged columns
    // elements per staged row: 16 (mod 32), i.e. 8 (mod 16) dwords, for
    // which the 16-byte A reads of 16 rows count no LDS bank conflicts
    // (measured on gfx950; 4 (mod 16) dwords counts one conflict cycle per
    // read, 0 (mod 16) several)
    static constexpr int PITCH = XW + (48 - XW % 32) % 32;
    static constexpr int ZLEN = 48;               // padded fragment length (PK = 1)
    // PK > 1: one padded filter row -- 16 zeros, the FW taps, zeros -- long
    // enough for the 5 dwords a lane reads from element
    // 16 + KW*j + (8g mod KW) - t16 of its row, a multiple of 8 elements
    // (of 4 with four or more windows: 1.2 KB less LDS, which keeps two
    // workgroups per CU up to 49-row filters)
    static constexpr int ZS = NFRAG >= 4 ? (18 + KW * NFRAG + 3) / 4 * 4
                                         : (18 + KW * NFRAG + 7) / 8 * 8;
    // wavefronts per workgroup; KS = 2: two wavefronts per channel, each
    // taking half of the filter's row groups
    static constexpr int NW = (CS >= 16 ? 8 : 4) * KS;
    static constexpr int NT = 64 * NW;                 // threads per workgroup
    static constexpr int NPAIR = 8 * XW;               // column pairs in 16 rows
    static constexpr int NEWP = (NPAIR + NT - 1) / NT; // column pairs per thread
    // output tile: pixel stride (an odd number of dwords) and row stride (4
    // mod 16 elements) chosen so that the regrouping writes of a wavefront
    // hit each LDS bank at most twice
    static constexpr int OPS = CS + 2;
    static constexpr int ORS = 16 * NB * OPS + 4;
};

// Workgroup (4 wavefronts, 8 for 16-channel slices or with KS = 2): one
// image, a strip of 16*NB output columns and CS channels, walking down the
// image 16 output rows at a time.  The
// XR = 16 + FH - 1 padded input rows a row block needs sit in an LDS ring;
// moving to the next block replaces the 16 oldest rows, whose loads are
// issued before the current block's MFMAs so that their latency is hidden.
// FHK > 0: filters of at most FHK rows and one fragment keep every B operand
// of the wavefront's channels in registers for the whole strip.
// AL: every lane reads its A windows of each filter row from LDS (no DPP)
// BN: the fused prologue.  Each in-image input value x becomes
// U = act(x * bn_scale[c] + bn_shift[c]) (one fp32 fused multiply-add, then
// the activation) rounded to the input format as the ring is written -- the
// value a separate BN + Act pass would store -- and the padding stays zero;
// everything after the ring is the plain pass.
// PK > 1 (row packing): the filter rows are taken PK at a time.  The K
// window of one MFMA is PK filter rows of KW = 32 / PK consecutive input
// columns each: lane (g, t16) holds row fh0 + 8g/KW + t16 of the ring,
// columns KW*h + (8g mod KW) .. +7, and
//   B_j[k][t] = w[fh0 + k/KW][KW*j + k mod KW - t]   (zero off the filter)
// so that the J = NFRAG windows h = (PK/2)*b + j, j < J, of output block b
// give its 16 outputs every tap of the PK rows.  A band of 31 taps fills
// 31 of each 48 K entries instead of 31 of 64 (one row per MFMA), and a
// 7-tap band 7 of 24 instead of 7 of 32: fewer MFMAs, and each lane reads
// one A window per group instead of one per row.  Rows past FH (the last
// group of a filter whose height is not a multiple of PK) have zero taps,
// and their A entries are set to zero, so an Inf or NaN in the ring does
// not reach outputs through them.
// KS = 2 (packed rows, runtime height): two wavefronts per channel, the
// first running the first half of the row groups into sums seeded with the
// bias, the second the rest into sums seeded with zero; before the epilogue
// the second half's sums go through LDS and are added to the first's (one
// more fp32 rounding).  For tiles so large that one 4-wavefront workgroup
// fills a CU, this gives each SIMD two wavefronts.
template <class DT, int CS, int NB, int NFRAG, int FHK, int FHT, bool AL = false, bool BN = false,
          int PK = 1, int KS = 1>
__global__ void __launch_bounds__((CS >= 16 ? 512 : 256) * KS, 2 / KS)  // at most 256 registers
k_mfma(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w,
       const float *__restrict__ bias, uint16_t *__restrict__ y, Shape s, int ncs, int nct,
       const float *__restrict__ bns, const float *__restrict__ bnb, int act, int slots) {
    using T = MfmaTile<CS, NB, NFRAG, PK, KS>;
    constexpr int XW = T::XW, PITCH = T::PITCH, ZLEN = T::ZLEN, ZS = T::ZS, KW = T::KW;
    constexpr int NW = T::NW, NT = T::NT;
    static_assert(NT == (CS >= 16 ? 512 : 256) * KS, "launch bounds match the tile");
    static_assert(KS == 1 || (KS == 2 && PK > 1 && FHT == 0 && FHK == 0),
                  "row groups split over two wavefronts: packed rows, runtime height");
    constexpr int NWC = NW / KS;            // wavefronts per row-group half
    constexpr int NCH = CS / NWC;           // channels per wavefront
    constexpr int NWIN = T::NWIN;           // distinct A windows per filter row / group
    static_assert(FHK == 0 || NFRAG == 1 || PK > 1, "kept B operands: one fragment");
    static_assert(FHT == 0 || FHK == 0 || FHT <= FHK || PK > 1, "kept B operands cover the filter");
    static_assert(PK == 1 || ((PK == 2 || PK == 4) && AL && (FHK == 0 || FHT > 0)),
                  "row packing: 2 or 4 rows, LDS-read A windows, kept B with a fixed height");
    // FHT > 0: the filter height is a compile-time constant and the
    // filter-row loop is fully unrolled, so the accumulators keep fixed
    // registers (a runtime loop made the compiler rotate them)
    extern __shared__ __attribute__((aligned(16))) uint16_t lds[];

    const int FH = FHT > 0 ? FHT : s.FH;            // filter height
    const int FHP = (FH + PK - 1) / PK * PK;        // filter rows staged (PK > 1)
    const int XR = 16 + FH - 1;                     // ring rows
    const int RING = CS * XR * PITCH;               // elements of one ring
    uint16_t *xt = lds;                             // [CS][XR][PITCH]
    uint16_t *zt = xt + RING;  // [CS][FH][NFRAG][ZLEN], PK > 1: [CS][FHP][ZS]
    const int ZT = PK == 1 ? CS * FH * NFRAG * ZLEN : CS * FHP * ZS;
    uint16_t *ot = zt + ZT;                         // [16][16*NB][CS]

    // workgroup -> (image, column strip, channel slice); channel slices vary
    // fastest so that the slices of one strip run together and share the L2
    // lines of its pixels
    const uint32_t bid = xcd_remap_slots(blockIdx.x, gridDim.x, slots);
    const int cs = bid % ncs;
    const uint32_t r = bid / ncs;
    const int ct = r % nct;
    const int n = r / nct;
    const int c0 = cs * CS;
    const int ow0 = ct * 16 * NB;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform, and visibly so: the bias loads indexed by it become
    // scalar loads, which no MFMA then waits on together with the ring refill
    // loads (a vector load of the bias made the first row block's MFMAs wait
    // for the refill of the next block)
    const int wave_id = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wave = wave_id % NWC;         // the wavefront's channels: wave + NWC * ci
    const int khalf = wave_id / NWC;        // its half of the row groups (KS = 2)
    const uint16_t *xn = x + (long long)n * s.H * s.W * s.C + c0;
    const int WC = s.W * s.C;  // elements of one image row (< 2^31)

    // Column pair e = tid + NT*u of a 16-row chunk is chunk row e / (XW/2),
    // tile columns 2 (e % (XW/2)) and the next one: the same for every chunk,
    // so computed once.
    constexpr int NEWP = T::NEWP, HALFW = XW / 2;
    int crow[NEWP], ccol[NEWP], cgoff[NEWP];
    bool cok0[NEWP], cok1[NEWP], cin[NEWP];
#pragma unroll
    for (int u = 0; u < NEWP; ++u) {
        const int e = tid + NT * u;
        cin[u] = e < 16 * HALFW;
        crow[u] = e / HALFW;
        ccol[u] = 2 * (e % HALFW);
        const int iw = ow0 - s.P + ccol[u];
        cok0[u] = cin[u] && (unsigned)iw < (unsigned)s.W;
        cok1[u] = cin[u] && (unsigned)(iw + 1) < (unsigned)s.W;
        cgoff[u] = iw * s.C;
    }
    // One pixel's CS channels as a packed vector (two channels per dword).
    typedef uint32_t PixV __attribute__((ext_vector_type(CS / 2)));
    static_assert(CS == 4 || CS == 8 || CS == 16, "channel slice of 4, 8 or 16");
    auto ld1 = [&](const uint16_t *src) { return *reinterpret_cast<const PixV *>(src); };
    // loads of padded input rows [R0, R0 + 16); zeros outside the image
    auto fetch = [&](PixV(&v)[NEWP][2], int R0, int rlimit) {
#pragma unroll
        for (int u = 0; u < NEWP; ++u) {
            const int ih = R0 + crow[u] - s.P;
            const bool rok = (unsigned)ih < (unsigned)s.H && R0 + crow[u] < rlimit;
            const uint16_t *src = xn + ih * WC + cgoff[u];
            v[u][0] = rok && cok0[u] ? ld1(src) : (PixV)0u;
            v[u][1] = rok && cok1[u] ? ld1(src + s.C) : (PixV)0u;
        }
    };
    // channel-major scatter into the ring, one dword (two columns) per
    // channel: padded row R lives in slot R mod XR
    // the fused prologue's per-channel scale and shift of the slice's channels
    float bnsc[BN ? CS : 1], bnsh[BN ? CS : 1];
    if constexpr (BN) {
#pragma unroll
        for (int c = 0; c < CS; ++c) {
            bnsc[c] = bns[c0 + c];
            bnsh[c] = bnb[c0 + c];
        }
    }
    auto scatter = [&](const PixV(&v)[NEWP][2], int R0, int rlimit) {
        const int r0m = R0 % XR;
#pragma unroll
        for (int u = 0; u < NEWP; ++u) {
            if (!cin[u] || R0 + crow[u] >= rlimit) continue;
            int slot = r0m + crow[u];
            slot -= slot >= XR ? XR : 0;
            uint16_t *dst = xt + slot * PITCH + ccol[u];
            if constexpr (!BN) {
#pragma unroll
                for (int k = 0; k < CS / 2; ++k) {
                    const uint32_t a = v[u][0][k], b = v[u][1][k];
                    *reinterpret_cast<uint32_t *>(dst + (2 * k) * XR * PITCH) =
                        (a & 0xffffu) | (b << 16);
                    *reinterpret_cast<uint32_t *>(dst + (2 * k + 1) * XR * PITCH) =
                        (a >> 16) | (b & 0xffff0000u);
                }
            } else {
                // in-image values become U in the input format; the
                // generated padding stays zero
                const int ih = R0 + crow[u] - s.P;
                const bool rok = (unsigned)ih < (unsigned)s.H;
                const bool in0 = rok && cok0[u], in1 = rok && cok1[u];
#pragma unroll
                for (int c = 0; c < CS; ++c) {
                    const int sh16 = 16 * (c & 1);
                    uint32_t h[2];
#pragma unroll
                    for (int col = 0; col < 2; ++col) {
                        const uint16_t xb = (uint16_t)(v[u][col][c / 2] >> sh16);
                        const float uv =
                            bn_act(DT::widen(__builtin_bit_cast(typename DT::X, xb)), bnsc[c],
                                   bnsh[c], act);
                        h[col] = (col ? in1 : in0)
                                     ? (uint32_t)__builtin_bit_cast(uint16_t, DT::narrow(uv))
                                     : 0u;
                    }
                    *reinterpret_cast<uint32_t *>(dst + c * XR * PITCH) = h[0] | (h[1] << 16);
                }
            }
        }
    };

    // ---- filter slice as padded fragments: fragment f of filter row fh of
    // channel c is 16 zeros, its 16 taps (zero past FW), 16 zeros; with row
    // packing, filter row fh is 16 zeros, its FW taps, zeros to ZS, and rows
    // FH .. FHP-1 are zero ----
    {
        const int zlen = ZT;
        static_assert(PK == 1 || CS * ZS % 8 == 0, "zero fill in 16-byte stores");
        for (int e = 8 * tid; e < zlen; e += 8 * NT)   // zlen is a multiple of 8
            *reinterpret_cast<u32x4 *>(zt + e) = (u32x4){0u, 0u, 0u, 0u};
        __syncthreads();
        // thread -> (fw = tid % 32 + 32j, fh = tid / 32 + RPP*k): no
        // divisions; the (at most 4) loads of a thread are issued before its
        // LDS writes
        constexpr int RPP = NT / 32;  // filter rows per pass of the workgroup
        for (int fw = tid & 31; fw < s.FW; fw += 32) {
            const int f = fw >> 4, q = fw & 15;
            for (int fh0 = tid >> 5; fh0 < FH; fh0 += 4 * RPP) {
                PixV v[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int fh = fh0 + RPP * k;
                    if (fh < FH) v[k] = ld1(w + (long long)tap_index(s, fh, fw) * s.C + c0);
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int fh = fh0 + RPP * k;
                    if (fh < FH) {
#pragma unroll
                        for (int c = 0; c < CS; ++c)
                            zt[PK == 1 ? ((c * FH + fh) * NFRAG + f) * ZLEN + 16 + q
                                       : (c * FHP + fh) * ZS + 16 + fw] =
                                (uint16_t)(v[k][c / 2] >> (16 * (c & 1)));
                    }
                }
            }
        }
    }
    // ---- prologue: padded rows [0, XR0) of the first row block; the loads
    // of up to four 16-row chunks are issued before any of them is written.
    // With row packing and 1 to 8 rows in the map's last 16 (a 56-row map),
    // those rows are a half block of 8 output rows (below).  For filters of
    // 16 rows or more it comes first, where it needs only 8 + FH - 1 input
    // rows before its MFMAs can start (31x31 on a 56-row map: 3.5 % faster
    // than last); for shorter filters it comes last (7x7: 1.3 % faster).
    const bool halfblk = PK > 1 && (s.OH - 1) % 16 < 8;
    const bool halffirst = halfblk && FH >= 16;
    const int XR0 = halffirst ? XR - 8 : XR;
    for (int R0 = 0; R0 < XR0; R0 += 64) {
        PixV v[4][NEWP][2];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (R0 + 16 * k < XR0) fetch(v[k], R0 + 16 * k, XR0);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (R0 + 16 * k < XR0) scatter(v[k], R0 + 16 * k, XR0);
    }
    __syncthreads();

    const int g = lane >> 4;    // k group of A/B, row group of D
    const int t16 = lane & 15;  // row of A, column of B and D
    // This lane's 8 entries of B are elements 16 + 8g - t16 .. +7 of the
    // padded fragment: B[k][t] = tap k - t.  They are read from the dword
    // holding element boff rounded down, shifted right by bsh bits.  With
    // row packing the lane's k range 8g .. 8g+7 is filter row pr of the
    // group, columns po .. po+7 of each KW-column window, and its B entries
    // of window j are elements 16 + KW*j + po - t16 .. +7 of padded row pr.
    const int pr = PK == 1 ? 0 : (8 * g) / KW;
    const int po = PK == 1 ? 8 * g : (8 * g) % KW;
    const int boff = PK == 1 ? 16 + 8 * g - t16 : 16 + po - t16;
    const int bsh = 16 * (boff & 1);
    const uint16_t *xc[NCH];
    const uint16_t *zc[NCH];
    float bv[NCH];
#pragma unroll
    for (int ci = 0; ci < NCH; ++ci) {
        const int c = wave + NWC * ci;
        xc[ci] = xt + c * XR * PITCH + po;
        zc[ci] = zt + (PK == 1 ? c * FH * NFRAG * ZLEN : (c * FHP + pr) * ZS) + (boff & ~1);
        bv[ci] = bias ? bias[c0 + c] : 0.0f;
    }
    auto load_b = [&](u32x4 &b, int ci, int fh, int f) {
        const uint32_t *zd =
            reinterpret_cast<const uint32_t *>(zc[ci] + (fh * NFRAG + f) * ZLEN);
        uint32_t d[5];
#pragma unroll
        for (int q = 0; q < 5; ++q) d[q] = zd[q];
#pragma unroll
        for (int q = 0; q < 4; ++q) b[q] = __builtin_amdgcn_alignbit(d[q + 1], d[q], bsh);
    };
    // row packing: window j of the group whose first filter row is fh0
    auto load_bp = [&](u32x4 &b, int ci, int fh0, int j) {
        const uint32_t *zd = reinterpret_cast<const uint32_t *>(zc[ci] + fh0 * ZS + KW * j);
        uint32_t d[5];
#pragma unroll
        for (int q = 0; q < 5; ++q) d[q] = zd[q];
#pragma unroll
        for (int q = 0; q < 4; ++q) b[q] = __builtin_amdgcn_alignbit(d[q + 1], d[q], bsh);
    };
    // row packing with kept B operands: the J windows of the groups that
    // start below filter row FHK (all of them when FHK >= FHT), the others
    // read from LDS for each row block
    constexpr int NGK = PK > 1 && FHK > 0 ? ((FHK < FHT ? FHK : FHT) + PK - 1) / PK : 1;
    u32x4 Bp[PK > 1 && FHK > 0 ? NCH : 1][NGK][PK > 1 && FHK > 0 ? NFRAG : 1];
    if constexpr (PK > 1 && FHK > 0) {
#pragma unroll
        for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
            for (int gi = 0; gi < NGK; ++gi)
#pragma unroll
                for (int j = 0; j < NFRAG; ++j) load_bp(Bp[ci][gi][j], ci, PK * gi, j);
    }
    constexpr int KB = PK > 1 ? 1 : FHT > 0 && FHK > 0 ? FHT : FHK > 0 ? FHK : 1;
    u32x4 Bk[NCH][KB];
    if constexpr (FHK > 0 && PK == 1) {
#pragma unroll
        for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
            for (int fh = 0; fh < KB; ++fh)
                if (fh < FH) load_b(Bk[ci][fh], ci, fh, 0);
    }

    // Output vectors of the previous row block.  A store reads its data
    // registers after issue, so a register it still holds cannot be
    // rewritten before the store has drained; keeping these registers out of
    // the allocator's hands until the next epilogue means no refill or MFMA
    // operand of the next block has to wait for the previous block's stores.
    // Thread tid stores NOUT consecutive pixels of output row tid / OTPR of
    // the block with buffer stores: one 32-bit lane offset, the pixel step
    // as a uniform offset, and the image's output range checked by the
    // buffer resource.
    constexpr int NOUT = 16 * 16 * NB / NT;
    constexpr int OTPR = NT / 16;  // threads per output row
    static_assert(16 * 16 * NB == NT * NOUT && NOUT * OTPR == 16 * NB, "output tile mapping");
    const int orow = tid / OTPR, ocol0 = NOUT * (tid % OTPR);
    PixV ov[NOUT];
#pragma unroll
    for (int k = 0; k < NOUT; ++k) ov[k] = (PixV)0u;
    uint32_t yoff = 0;
    const long long yimg = (long long)s.OH * s.OW * s.C;  // elements per image (< 2^31)
    const __amdgpu_buffer_rsrc_t yrs = __builtin_amdgcn_make_buffer_rsrc(
        y + n * yimg + c0, (short)0, (int)(uint32_t)(2 * (yimg - c0)), 0x00020000);

    // One row block: output rows a .. a+15 (a .. a+7 for a half block, NBC =
    // nbc = NB / 2 column blocks per MFMA row set instead of NB); `more`: a
    // full block follows.  The half block is a separate call, so that the
    // loop over the full ones carries none of its code or registers.
    auto block = [&](int a, bool more, auto nbc) {
        if (a) __syncthreads();  // ring rows of this block written; output tile free
        // prefetch the 16 rows the next block adds (the rows this block
        // needs are in the ring already)
        const int Rn = a + (decltype(nbc)::value < NB ? 8 : 16) + XR - 16;
        PixV nv[NEWP][2];
        if (more) fetch(nv, Rn, 1 << 30);

        int slot0 = a + t16;  // ring slot of this lane's row at fh = 0
        slot0 %= XR;
        // A half block (row packing, 8 output rows): its 16 MFMA rows are the
        // 8 rows of the first NB/2 column blocks and the same 8 rows of the
        // last NB/2 (one filter band serves both), so it takes half the
        // MFMAs.  Its row i is output row i mod 8, columns shifted by
        // (i / 8) * 8 * NB.
        constexpr bool half = decltype(nbc)::value < NB;

        // One fp32 MFMA chain per output tile, seeded with the bias: a chain
        // of at most 2 * 32 MFMAs stays within 1e-5 * sum|x*w| (one rounding
        // per MFMA plus the products cut inside its groups of 8, at most
        // 7 * 2^-24 of their magnitude over the whole chain).
        f32x4 acc[NCH][NB];
#pragma unroll
        for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                // with the row groups split over two wavefronts, the second
                // half's sums start at zero (the bias is added once)
                const float seed = KS > 1 && khalf ? 0.0f : bv[ci];
                acc[ci][b] = (f32x4){seed, seed, seed, seed};
            }
        // More than two fragments (filters wider than 32 taps): the chain of
        // 16 filter rows (at most 64 MFMAs) is added into a separate fp32
        // total, which the bias seeds, and restarts from zero.
        // Row packing where the chain could pass 64 MFMAs (four or more
        // windows for filters of 34 to 65 taps and up to 64 rows): the chain
        // of FG row groups (at most 64 MFMAs) is folded the same way.
        constexpr int FHMAX = FHT > 0 ? FHT : NFRAG >= 4 ? 64 : 32;
        constexpr bool FOLD = PK == 1 ? NFRAG > 2 : (FHMAX + PK - 1) / PK * NFRAG > 64;
        constexpr int FP = 16;             // filter rows per folded chain (PK = 1)
        constexpr int FG = 64 / NFRAG;     // row groups per folded chain (PK > 1)
        f32x4 tot[FOLD ? NCH : 1][FOLD ? NB : 1];
        auto fold = [&]() {
            if constexpr (FOLD) {
#pragma unroll
                for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        tot[ci][b] += acc[ci][b];
                        acc[ci][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
                    }
            }
        };
        if constexpr (FOLD) {
#pragma unroll
            for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    tot[ci][b] = acc[ci][b];
                    acc[ci][b] = (f32x4){0.f, 0.f, 0.f, 0.f};
                }
        }

        // A windows of filter row fh: lane t16 holds row fh + t16 of the row
        // block.  Row fh+1's windows are row fh's moved down one lane within
        // each 16-lane row (DPP row_shl:1); only lane 15 reads its new row
        // from LDS.  B operands (unless kept) and the next windows are
        // produced before the MFMAs of row fh issue.
        struct Ops {
            u32x4 A[NCH][NWIN];
            u32x4 B[NCH][FHK > 0 ? 1 : NFRAG];
        };
        auto full_a = [&](Ops &o) {
#pragma unroll
            for (int ci = 0; ci < NCH; ++ci) {
                const uint16_t *xr = xc[ci] + slot0 * PITCH;
#pragma unroll
                for (int win = 0; win < NWIN; ++win)
                    o.A[ci][win] = *reinterpret_cast<const u32x4 *>(xr + 16 * win);
            }
        };
        auto next_a = [&](Ops &o, const Ops &prev, int fh) {
            // this lane's row for filter row fh (only lane 15's is read)
            int slot = slot0 + fh;
            slot -= slot >= XR ? XR : 0;
#pragma unroll
            for (int ci = 0; ci < NCH; ++ci) {
                if constexpr (AL) {
                    const uint16_t *xr = xc[ci] + slot * PITCH;
#pragma unroll
                    for (int win = 0; win < NWIN; ++win)
                        o.A[ci][win] = *reinterpret_cast<const u32x4 *>(xr + 16 * win);
                    continue;
                }
#pragma unroll
                for (int win = 0; win < NWIN; ++win)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        o.A[ci][win][q] = __builtin_amdgcn_update_dpp(
                            0, (int)prev.A[ci][win][q], 0x101, 0xf, 0xf, true);
                if (t16 == 15) {
                    const uint16_t *xr = xc[ci] + slot * PITCH;
#pragma unroll
                    for (int win = 0; win < NWIN; ++win)
                        o.A[ci][win] = *reinterpret_cast<const u32x4 *>(xr + 16 * win);
                }
            }
        };
        auto load_bs = [&](Ops &o, int fh) {
            if constexpr (FHK == 0) {
#pragma unroll
                for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
                    for (int f = 0; f < NFRAG; ++f) load_b(o.B[ci][f], ci, fh, f);
            }
        };
        auto mfmas = [&](const Ops &o, int fh) {
#pragma unroll
            for (int f = 0; f < NFRAG; ++f)
#pragma unroll
                for (int b = 0; b < NB; ++b)
#pragma unroll
                    for (int ci = 0; ci < NCH; ++ci) {
                        u32x4 bb;
                        if constexpr (FHK > 0) {
                            bb = Bk[ci][0];
#pragma unroll
                            for (int k = 1; k < KB; ++k)
                                if (fh == k) bb = Bk[ci][k];
                        } else {
                            bb = o.B[ci][f];
                        }
                        acc[ci][b] = MfmaOp<DT>::run(o.A[ci][b + f], bb, acc[ci][b]);
                    }
        };

        if constexpr (PK > 1) {
            // Row packing: group gi covers filter rows PK*gi .. PK*gi+PK-1.
            // The unit of the pipeline is one channel's group: the LDS reads
            // of the next unit are issued before the MFMAs of the current
            // one (two units of operands in registers).  At most 8 groups of
            // 6 windows (FH <= 32, FW <= 33): a chain of at most 48 MFMAs
            // per tile, else folded every FG groups.  NBC column blocks per
            // MFMA row set: NB, or NB/2 in
            // a half block (each variant compiled on its own, so neither
            // carries the other's branches or registers).
            auto packed_rows = [&](auto nbc) {
                constexpr int NBC = decltype(nbc)::value;
                constexpr int NWC = (PK / 2) * (NBC - 1) + NFRAG;  // windows per group
                int slotp = a + (NBC < NB ? (t16 & 7) : t16) + pr;  // lane's ring row
                slotp %= XR;                                               // at fh0 = 0
                const int hoff = NBC < NB ? (t16 >> 3) * 8 * NB : 0;      // its column shift
                struct OpsU {
                    u32x4 A[NWC];
                    uint32_t R[FHK > 0 && FHK >= FHT ? 1 : NFRAG][5];
                };
                auto load_unit = [&](OpsU &o, int ci, int fh0) {
                    int sl = slotp + fh0;
                    sl -= sl >= XR ? XR : 0;
                    // rows past FH: zero A entries (the taps there are zero too)
                    const bool full = FHT > 0 && fh0 + PK <= FHT;
                    const bool ok = full || fh0 + pr < FH;
                    const uint16_t *xr = xc[ci] + sl * PITCH + hoff;
#pragma unroll
                    for (int h = 0; h < NWC; ++h) {
                        const u32x4 a = *reinterpret_cast<const u32x4 *>(xr + KW * h);
                        o.A[h] = ok ? a : (u32x4){0u, 0u, 0u, 0u};
                    }
                    if constexpr (!(FHK > 0 && FHK >= FHT)) {
                        if (FHK == 0 || fh0 >= PK * NGK) {
#pragma unroll
                            for (int j = 0; j < NFRAG; ++j) {
                                const uint32_t *zd = reinterpret_cast<const uint32_t *>(
                                    zc[ci] + fh0 * ZS + KW * j);
#pragma unroll
                                for (int q = 0; q < 5; ++q) o.R[j][q] = zd[q];
                            }
                        }
                    }
                };
                auto mfmas_unit = [&](const OpsU &o, int ci, int gi) {
                    u32x4 bb[NFRAG];
#pragma unroll
                    for (int j = 0; j < NFRAG; ++j) {
                        if (FHK > 0 && gi < NGK) {
                            bb[j] = Bp[ci][0][j];
#pragma unroll
                            for (int k = 1; k < NGK; ++k)
                                if (gi == k) bb[j] = Bp[ci][k][j];
                        } else if constexpr (!(FHK > 0 && FHK >= FHT)) {
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                bb[j][q] =
                                    __builtin_amdgcn_alignbit(o.R[j][q + 1], o.R[j][q], bsh);
                        }
                    }
#pragma unroll
                    for (int j = 0; j < NFRAG; ++j)
#pragma unroll
                        for (int b = 0; b < NBC; ++b)
                            acc[ci][b] =
                                MfmaOp<DT>::run(o.A[(PK / 2) * b + j], bb[j], acc[ci][b]);
                };
                // this wavefront's row groups [gb, ge): all of them, or one
                // half of them with KS = 2
                const int NG = FHP / PK;
                const int gb = KS > 1 && khalf ? (NG + 1) / 2 : 0;
                const int ge = KS > 1 && !khalf ? (NG + 1) / 2 : NG;
                OpsU o[2];
                if (gb < ge) load_unit(o[0], 0, PK * gb);
                if constexpr (FHT > 0) {
                    constexpr int NU = (FHT + PK - 1) / PK * NCH;
#pragma unroll
                    for (int u = 0; u < NU; ++u) {
                        if (u + 1 < NU)
                            load_unit(o[(u + 1) & 1], (u + 1) % NCH, PK * ((u + 1) / NCH));
                        mfmas_unit(o[u & 1], u % NCH, u / NCH);
                        if (FOLD && (u + 1) % NCH == 0 && (u + 1) / NCH % FG == 0) fold();
                        // keep the scheduler from hoisting later units' operands
                        // (and their registers) above this unit's MFMAs
                        __builtin_amdgcn_sched_barrier(0);
                    }
                } else {
                    // groups two at a time, so that a unit's operand buffer is
                    // fixed at compile time (2 * NCH units per step)
                    for (int gi0 = gb; gi0 < ge; gi0 += 2) {
#pragma unroll
                        for (int dg = 0; dg < 2; ++dg) {
                            const int gi = gi0 + dg;
                            if (gi >= ge) break;
#pragma unroll
                            for (int ci = 0; ci < NCH; ++ci) {
                                const int u = dg * NCH + ci;
                                const int nci = ci + 1 < NCH ? ci + 1 : 0;
                                const int ngi = ci + 1 < NCH ? gi : gi + 1;
                                if (ngi < ge) load_unit(o[(u + 1) & 1], nci, PK * ngi);
                                mfmas_unit(o[u & 1], ci, gi);
                            }
                            if (FOLD && (gi - gb + 1) % FG == 0) fold();
                        }
                    }
                }
            };
            packed_rows(nbc);
        } else if constexpr (FHT > 0 && FHK > 0) {
            // B operands kept in registers: one row of lookahead
            Ops o[2];
            full_a(o[0]);
#pragma unroll
            for (int fh = 0; fh < FHT; ++fh) {
                if (fh + 1 < FHT) next_a(o[(fh + 1) & 1], o[fh & 1], fh + 1);
                mfmas(o[fh & 1], fh);
                // keep the scheduler from hoisting later rows' operands
                // (and their registers) above this row's MFMAs
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if constexpr (FHT > 0) {
            // Software pipeline two filter rows deep: while the MFMAs of row
            // fh run, the operands of row fh+1 are formed from LDS data
            // loaded during row fh-1, and the LDS reads of row fh+2 are
            // issued, so no row waits for LDS.  The new row of lane 15 is
            // the DPP's old value: lanes 0..14 take lane t16+1 of row fh's
            // windows, lane 15 (no source in its row) keeps what it loaded.
            Ops o[2];   // formed operands of rows fh, fh+1
            u32x4 Lw[2][NCH][NWIN];          // loaded windows, rows fh+1, fh+2
            uint32_t Rb[2][NCH][NFRAG][5];   // loaded B dwords, rows fh+1, fh+2
            auto load_rows = [&](int fh) {
                int slot = slot0 + fh;
                slot -= slot >= XR ? XR : 0;
#pragma unroll
                for (int ci = 0; ci < NCH; ++ci)
                    if (AL || t16 == 15) {
                        const uint16_t *xr = xc[ci] + slot * PITCH;
#pragma unroll
                        for (int win = 0; win < NWIN; ++win)
                            Lw[fh & 1][ci][win] = *reinterpret_cast<const u32x4 *>(xr + 16 * win);
                    }
                {
#pragma unroll
                    for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
                        for (int f = 0; f < NFRAG; ++f) {
                            const uint32_t *zd = reinterpret_cast<const uint32_t *>(
                                zc[ci] + (fh * NFRAG + f) * ZLEN);
#pragma unroll
                            for (int q = 0; q < 5; ++q) Rb[fh & 1][ci][f][q] = zd[q];
                        }
                }
            };
            auto form = [&](int fh) {
                Ops &n = o[fh & 1];
                const Ops &p = o[(fh + 1) & 1];  // row fh - 1
#pragma unroll
                for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
                    for (int win = 0; win < NWIN; ++win)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            n.A[ci][win][q] =
                                AL ? Lw[fh & 1][ci][win][q]
                                   : __builtin_amdgcn_update_dpp((int)Lw[fh & 1][ci][win][q],
                                                                 (int)p.A[ci][win][q], 0x101, 0xf,
                                                                 0xf, false);
                {
#pragma unroll
                    for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
                        for (int f = 0; f < NFRAG; ++f)
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                n.B[ci][f][q] = __builtin_amdgcn_alignbit(
                                    Rb[fh & 1][ci][f][q + 1], Rb[fh & 1][ci][f][q], bsh);
                }
            };
            full_a(o[0]);
            load_bs(o[0], 0);
            if (FHT > 1) load_rows(1);
#pragma unroll
            for (int fh = 0; fh < FHT; ++fh) {
                if (fh + 2 < FHT) load_rows(fh + 2);
                if (fh + 1 < FHT) form(fh + 1);
                mfmas(o[fh & 1], fh);
                // keep the scheduler from hoisting later rows' operands
                // (and their registers) above this row's MFMAs
                __builtin_amdgcn_sched_barrier(0);
            }
        } else if constexpr (FHK > 0) {
            Ops o[2];
            full_a(o[0]);
#pragma unroll
            for (int fh = 0; fh < FHK; ++fh) {
                if (fh >= FH) break;
                if (fh + 1 < FH) next_a(o[(fh + 1) & 1], o[fh & 1], fh + 1);
                mfmas(o[fh & 1], fh);
            }
        } else {
            Ops o0, o1;
            full_a(o0);
            load_bs(o0, 0);
            int fh = 0;
            for (; fh + 1 < FH; fh += 2) {
                next_a(o1, o0, fh + 1);
                load_bs(o1, fh + 1);
                mfmas(o0, fh);
                if (fh + 2 < FH) {
                    next_a(o0, o1, fh + 2);
                    load_bs(o0, fh + 2);
                }
                mfmas(o1, fh + 1);
                if (FOLD && (fh + 2) % FP == 0) fold();
            }
            if (fh < FH) mfmas(o0, fh);
        }
        if constexpr (FOLD) {
            fold();
#pragma unroll
            for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
                for (int b = 0; b < NB; ++b) acc[ci][b] = tot[ci][b];
        }

        // two wavefronts per channel: the second half's sums are added to
        // the first half's through LDS (past the output tile), in a fixed
        // order
        constexpr int OPS = T::OPS, ORS = T::ORS;
        if constexpr (KS > 1) {
            f32x4 *red = reinterpret_cast<f32x4 *>(ot + 16 * ORS);
            if (khalf) {
#pragma unroll
                for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        red[((wave * NCH + ci) * NB + b) * 64 + lane] = acc[ci][b];
            }
            __syncthreads();
            if (!khalf) {
#pragma unroll
                for (int ci = 0; ci < NCH; ++ci)
#pragma unroll
                    for (int b = 0; b < NB; ++b)
                        acc[ci][b] += red[((wave * NCH + ci) * NB + b) * 64 + lane];
            }
        }
        // ---- epilogue: round once, regroup through LDS into NHWC vectors ----
#pragma unroll
        for (int ci = 0; ci < NCH; ++ci) {
            const int c = wave + NWC * ci;
            if (KS > 1 && khalf) break;  // the first half's wavefronts hold the sums
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    int row = 4 * g + q, col = 16 * b + t16;
                    if (half) {  // D row i: output row i mod 8, block b + (i / 8) NB/2
                        if (2 * b >= NB) continue;
                        col += (g >> 1) * 8 * NB;
                        row &= 7;
                    }
                    ot[row * ORS + col * OPS + c] =
                        __builtin_bit_cast(uint16_t, DT::narrow(acc[ci][b][q]));
                }
        }
        __syncthreads();  // block's ring rows consumed; output tile complete
        // The next block's rows go into the ring first: their loads were
        // issued before this block's MFMAs, and waiting for them here, with
        // no global stores outstanding yet, does not also wait for this
        // block's stores to be acknowledged.
        if (more) scatter(nv, Rn, 1 << 30);
        // The refill loads are consumed and the previous block's stores are
        // long done: say so on every path (vmcnt 0, other counters
        // untouched), so that later register reuse needs no wait.
        __builtin_amdgcn_s_waitcnt(0x0f70);
        // Every output pixel vector of the tile is read from LDS before the
        // first store is issued, so the LDS latency is paid once.
#pragma unroll
        for (int k = 0; k < NOUT; ++k) asm volatile("" : "+v"(ov[k]));
        asm volatile("" : "+v"(yoff));
#pragma unroll
        for (int k = 0; k < NOUT; ++k) {
            const uint32_t *src =
                reinterpret_cast<const uint32_t *>(ot + orow * ORS + (ocol0 + k) * OPS);
#pragma unroll
            for (int q = 0; q < CS / 2; ++q) ov[k][q] = src[q];
        }
        const int oh = a + orow, ow = ow0 + ocol0;
        yoff = 2u * (uint32_t)((oh * s.OW + ow) * s.C);
        // (the rows 8..15 of a half block's tile are not written)
        if (oh < s.OH && (!half || orow < 8)) {
#pragma unroll
            for (int k = 0; k < NOUT; ++k)
                if (ow + k < s.OW) {
                    if constexpr (CS == 16) {
                        __builtin_amdgcn_raw_buffer_store_b128(ov[k].lo, yrs, (int)yoff, 2 * k * s.C, 0);
                        __builtin_amdgcn_raw_buffer_store_b128(ov[k].hi, yrs, (int)yoff,
                                                               2 * k * s.C + 16, 0);
                    } else if constexpr (CS == 8) {
                        __builtin_amdgcn_raw_buffer_store_b128(ov[k], yrs, (int)yoff, 2 * k * s.C, 0);
                    } else {
                        __builtin_amdgcn_raw_buffer_store_b64(ov[k], yrs, (int)yoff, 2 * k * s.C, 0);
                    }
                }
        }
    };
    int a0 = 0;                                         // first full block
    const int a1 = halfblk && !halffirst ? (s.OH - 1) / 16 * 16 : s.OH;  // past the last
    if constexpr (PK > 1) {
        if (halffirst) {
            block(0, s.OH > 8, std::integral_constant<int, NB / 2>{});
            a0 = 8;
        }
    }
    for (int a = a0; a < a1; a += 16) block(a, a + 16 < s.OH, std::integral_constant<int, NB>{});
    if constexpr (PK > 1) {
        if (halfblk && !halffirst) block(a1, false, std::integral_constant<int, NB / 2>{});
    }
}

template <class DT, int CS, int NB, int NFRAG, int FHK, int FHT, bool AL, int PK, int KS = 1>
static hipError_t launch_mfma(const Plan &p, const void *x, const void *w, const void *bias,
                              void *y, hipStream_t st) {
    if (p.lds_bytes > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&k_mfma<DT, CS, NB, NFRAG, FHK, FHT, AL, false, PK, KS>),
            hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_mfma<DT, CS, NB, NFRAG, FHK, FHT, AL, false, PK, KS>), dim3(p.grid),
                       dim3(MfmaTile<CS, NB, NFRAG, PK, KS>::NT), p.lds_bytes, st,
                       (const uint16_t *)x, (const uint16_t *)w, (const float *)bias,
                       (uint16_t *)y, p.s, p.aux0, p.aux1, nullptr, nullptr, 0, p.aux2);
    return hipGetLastError();
}

template <int CS, int NB, int NFRAG, int PK, int KS = 1>
static int mfma_lds_bytes(const Shape &s) {
    using T = MfmaTile<CS, NB, NFRAG, PK, KS>;
    const int XR = 16 + s.FH - 1;
    const int xt = CS * XR * T::PITCH;
    const int fhp = (s.FH + PK - 1) / PK * PK;
    const int zt = PK == 1 ? CS * s.FH * NFRAG * T::ZLEN : CS * fhp * T::ZS;
    const int ot = 16 * T::ORS;
    // KS = 2: the second half's fp32 sums, 64 lanes x NB tiles per channel
    const int red = KS > 1 ? CS * NB * 64 * 16 : 0;
    return 2 * (xt + zt + ot) + red;
}

// The fused prologue: the forward tiling with U formed as the ring is
// written; the same LDS.
template <class DT, int CS, int NB, int NFRAG, int FHK, int FHT, int PK>
static hipError_t launch_mfma_bn(const Plan &p, const void *x, const void *w, const void *bias,
                                 const float *bn_scale, const float *bn_shift, int act, void *y,
                                 hipStream_t st) {
    if (p.lds_bytes > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(
            reinterpret_cast<const void *>(&k_mfma<DT, CS, NB, NFRAG, FHK, FHT, true, true, PK>),
            hipFuncAttributeMaxDynamicSharedMemorySize, p.lds_bytes);
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((k_mfma<DT, CS, NB, NFRAG, FHK, FHT, true, true, PK>), dim3(p.grid),
                       dim3(MfmaTile<CS, NB, NFRAG, PK>::NT), p.lds_bytes, st,
                       (const uint16_t *)x, (const uint16_t *)w, (const float *)bias,
                       (uint16_t *)y, p.s, p.aux0, p.aux1, bn_scale, bn_shift, act, p.aux2);
    return hipGetLastError();
}

struct MfmaEntry {
    int dtype, cs, nb, nfrag, fhk, fht, al, pk;
    LaunchFn fn;
    int (*lds)(const Shape &);
    const void *kfn;  // the kernel, for the occupancy query
    int ks = 1;
};
#define KFN(...) reinterpret_cast<const void *>(&k_mfma<__VA_ARGS__>)

#define MFA(DTE, DTT, CS_, NB_, NF_, FHK_, FHT_, AL_)                                 \
    {DTE,      CS_, NB_, NF_, FHK_, FHT_, AL_, 1, launch_mfma<DTT, CS_, NB_, NF_, FHK_, FHT_, AL_, 1>, \
     mfma_lds_bytes<CS_, NB_, NF_, 1>, KFN(DTT, CS_, NB_, NF_, FHK_, FHT_, AL_, false, 1, 1)}
// row packing: PK filter rows per MFMA, J windows of 32 / PK columns
#define MFP(DTE, DTT, CS_, NB_, J_, FHK_, FHT_, PK_)                                   \
    {DTE,      CS_, NB_, J_, FHK_, FHT_, true, PK_,                                     \
     launch_mfma<DTT, CS_, NB_, J_, FHK_, FHT_, true, PK_>, mfma_lds_bytes<CS_, NB_, J_, PK_>, \
     KFN(DTT, CS_, NB_, J_, FHK_, FHT_, true, false, PK_, 1)}
#define MFPD(CS_, NB_, J_, FHK_, FHT_, PK_) \
    MFP(DT_F16, F16, CS_, NB_, J_, FHK_, FHT_, PK_), MFP(DT_BF16, BF16, CS_, NB_, J_, FHK_, FHT_, PK_)
// two rows per MFMA, each channel's row groups split over two wavefronts
#define MFS(DTE, DTT, CS_, NB_, J_)                                                    \
    {DTE,      CS_, NB_, J_, 0, 0, true, 2, launch_mfma<DTT, CS_, NB_, J_, 0, 0, true, 2, 2>, \
     mfma_lds_bytes<CS_, NB_, J_, 2, 2>, KFN(DTT, CS_, NB_, J_, 0, 0, true, false, 2, 2), 2}
#define MFSD(CS_, NB_, J_) MFS(DT_F16, F16, CS_, NB_, J_), MFS(DT_BF16, BF16, CS_, NB_, J_)
#define MF(DTE, DTT, CS_, NB_, NF_, FHK_, FHT_) MFA(DTE, DTT, CS_, NB_, NF_, FHK_, FHT_, false)

// Each configuration twice: A windows read from LDS by every lane first
// (measured faster than the DPP row shift: 7x7, 31x31, and 41x41 / 51x51 by
// 15-20 %), then the DPP row shift (tuning choice mfma_al=0).
#define MF2(DTE, DTT, CS_, NB_, NF_, FHK_, FHT_) \
    MFA(DTE, DTT, CS_, NB_, NF_, FHK_, FHT_, true), MF(DTE, DTT, CS_, NB_, NF_, FHK_, FHT_)
#define MF2D(CS_, NB_, NF_, FHK_, FHT_) \
    MF2(DT_F16, F16, CS_, NB_, NF_, FHK_, FHT_), MF2(DT_BF16, BF16, CS_, NB_, NF_, FHK_, FHT_)

// Wider channel slices first (16-byte loads, more work per tile); the
// planner falls back to 4 channels when the 8-channel tile exceeds 64 KiB of
// LDS (tall filters), to keep several workgroups per CU.
static const MfmaEntry kMfma[] = {
    // Row packing first: 31x31 bf16 on 32x56x56x128 ran 72.5 us with two
    // rows per MFMA against 82 with four and 88 with one, and 68.7 us with
    // the B operands of the first 9 of its 16 row groups kept in registers
    // (252 registers; LDS, not registers, holds it at two workgroups per CU;
    // 6 groups: 71.4 us); 7x7 fp16 on 64x56x56x96 37.1 us with four rows (B
    // kept) against 39.7 with one and 41.4 with four rows and B read from
    // LDS.  Eight-channel slices (140 KB of LDS, one workgroup per CU: 79.9
    // us) and 32-column strips (95 us) were slower on the 31x31 layer; they
    // stay for the tuning choices and for outputs that a 64-column strip
    // would pad more.
    MFPD(4, 4, 3, 18, 31, 2), MFPD(8, 2, 3, 8, 7, 4),
    MFPD(4, 4, 3, 0, 31, 2),
    MFPD(4, 4, 6, 0, 31, 4), MFPD(8, 2, 2, 8, 7, 2),
    MFPD(8, 4, 3, 0, 31, 2), MFPD(4, 2, 3, 0, 31, 2), MFPD(8, 2, 3, 0, 7, 4),
    // row packing, any filter height up to 32: four rows for filters of at
    // most 9 taps, two rows for 10 to 17 and for 18 to 33 taps (on the f16
    // sweep maps 1.02-1.45x the speed of one row per MFMA at F = 7, 9, 17,
    // 21, 25, 31; 0.97-0.98 at F = 13 and 0.89 at F = 9 on 128x32x32x1024);
    // two rows for 34 to 65 taps and up to 64 rows, folded chains: two
    // 4-wavefront workgroups per CU where the tile fits 80 KB, else one
    // 8-wavefront workgroup with each channel's row groups split over two
    // wavefronts, else one 4-wavefront workgroup; 1.6-2.7x one row per MFMA
    // at F = 41 and 51
    MFPD(4, 4, 4, 0, 0, 2), MFSD(4, 4, 5), MFSD(4, 2, 5), MFSD(4, 4, 4), MFPD(4, 4, 5, 0, 0, 2),
    MFPD(4, 2, 4, 0, 0, 2), MFPD(4, 2, 5, 0, 0, 2),
    MFPD(8, 4, 3, 0, 0, 4), MFPD(8, 4, 2, 0, 0, 2), MFPD(8, 4, 3, 0, 0, 2),
    MFPD(4, 4, 3, 0, 0, 4), MFPD(4, 4, 2, 0, 0, 2), MFPD(4, 4, 3, 0, 0, 2),
    MFPD(8, 2, 3, 0, 0, 4), MFPD(8, 2, 2, 0, 0, 2), MFPD(8, 2, 3, 0, 0, 2),
    MFPD(4, 2, 3, 0, 0, 4), MFPD(4, 2, 2, 0, 0, 2), MFPD(4, 2, 3, 0, 0, 2),
    // compile-time filter heights of the common square filters
    MF2D(8, 4, 1, 8, 7),
    MF2D(4, 4, 2, 0, 31),
    // 32-byte pixel slices, 8 wavefronts (measured slower on 7x7: kept for
    // mfma_cs=16)
    MF(DT_F16, F16, 16, 4, 1, 8, 7),   MF(DT_BF16, BF16, 16, 4, 1, 8, 7),
    // any filter height
    MF2D(8, 4, 1, 8, 0), MF2D(8, 4, 1, 0, 0), MF2D(8, 4, 2, 0, 0),
    MF2D(4, 4, 1, 8, 0), MF2D(4, 4, 1, 0, 0), MF2D(4, 4, 2, 0, 0),
    // filters of 33 to 64 taps: one workgroup per CU (89-140 KB of LDS);
    // 64-column strips for three fragments measured 60-70 % faster than
    // 32-column ones on 64- and 128-wide outputs (four do not fit LDS)
    MF2D(4, 4, 3, 0, 0),
    MF2D(4, 2, 3, 0, 0), MF2D(4, 2, 4, 0, 0),
    // 32-column strips for outputs whose width 64-column strips would pad
    // more (OW = 32: half of a 64-column strip would be padding)
    MF2D(8, 2, 1, 8, 7),
    MF2D(4, 2, 2, 0, 31),
    MF2D(8, 2, 1, 8, 0), MF2D(8, 2, 1, 0, 0), MF2D(8, 2, 2, 0, 0),
    MF2D(4, 2, 1, 0, 0), MF2D(4, 2, 2, 0, 0),
};
#undef MF2D
#undef MF2
#undef MF
#undef MFA
#undef MFPD
#undef MFP

// The fused prologue: the forward tilings (A windows read from LDS) for
// filters of at most 33 taps, with U formed as the ring is written.  The
// planner takes the forward plan's own tiling when it is here, else the
// first that fits in this order (the forward order).
struct MfmaBnEntry {
    int dtype, cs, nb, nfrag, fhk, fht, pk;
    LaunchBnFn fn;
    int (*lds)(const Shape &);
    const void *kfn;
};
#define MBE(DTE, DTT, CS_, NB_, J_, FHK_, FHT_, PK_)                                  \
    {DTE, CS_, NB_, J_, FHK_, FHT_, PK_, launch_mfma_bn<DTT, CS_, NB_, J_, FHK_, FHT_, PK_>, \
     mfma_lds_bytes<CS_, NB_, J_, PK_>, KFN(DTT, CS_, NB_, J_, FHK_, FHT_, true, true, PK_, 1)}
#define MBD(CS_, NB_, J_, FHK_, FHT_, PK_) \
    MBE(DT_F16, F16, CS_, NB_, J_, FHK_, FHT_, PK_), MBE(DT_BF16, BF16, CS_, NB_, J_, FHK_, FHT_, PK_)
static const MfmaBnEntry kMfmaBn[] = {
    // fixed heights: 31x31 and 7x7
    MBD(4, 4, 3, 18, 31, 2), MBD(8, 2, 3, 8, 7, 4),
    // row packing, any height up to 32
    MBD(8, 4, 3, 0, 0, 4), MBD(8, 4, 2, 0, 0, 2), MBD(8, 4, 3, 0, 0, 2),
    MBD(4, 4, 3, 0, 0, 4), MBD(4, 4, 2, 0, 0, 2), MBD(4, 4, 3, 0, 0, 2),
    MBD(8, 2, 3, 0, 0, 4), MBD(8, 2, 2, 0, 0, 2), MBD(8, 2, 3, 0, 0, 2),
    MBD(4, 2, 3, 0, 0, 4), MBD(4, 2, 2, 0, 0, 2), MBD(4, 2, 3, 0, 0, 2),
    // one row per MFMA (filters taller than 32 rows, and mfma_pk=1)
    MBD(8, 4, 1, 8, 0, 1), MBD(8, 4, 1, 0, 0, 1), MBD(8, 4, 2, 0, 0, 1),
    MBD(4, 4, 1, 0, 0, 1), MBD(4, 4, 2, 0, 0, 1),
    MBD(8, 2, 1, 8, 0, 1), MBD(8, 2, 1, 0, 0, 1), MBD(8, 2, 2, 0, 0, 1),
    MBD(4, 2, 1, 0, 0, 1), MBD(4, 2, 2, 0, 0, 1),
};
#undef MBD
#undef MBE
#undef KFN

// Workgroups of kernel `kfn` that one CU holds at once, from the runtime's
// occupancy query; 1 when it cannot answer (no device).  The kernel hands
// the workgroups one CU holds consecutive tiles (xcd_remap_slots) only for
// filters of 16 rows or more: there the co-resident channel slices of one
// strip share their pixels' cache lines and the layer runs faster (31x31
// bf16: 58.5 against 59.6 us, with 4.5 % more bytes written).  For shorter
// filters the gain was within noise (7x7 fp16: 36.3 against 36.5 us) and
// the cost is not: workgroups dispatched as slots free up then take channel
// slices of many strips at once, the slices of one pixel reach L2 far apart
// in time, its partly written lines are evicted before they are whole, and
// HBM writes rose to 1.50 times y (1.025 with consecutive dispatch).
// The tuning choice mfma_slots=n sets the count.
static int cu_slots(const void *kfn, int block, int lds, int fh) {
    const int want = tune_int("mfma_slots", 0);
    if (want >= 1) return want;
    if (fh < 16) return 1;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kfn, block, lds) != hipSuccess) {
        (void)hipGetLastError();  // clear the error the query left
        return 1;
    }
    return n >= 1 ? n : 1;
}

// The strip width (in 16-column blocks) that pads fewer output columns; on a
// tie 32-column strips for one fragment and at least 7 filter rows
// (measured: 7x7 up to 5 % and 13x13 up to 40 % faster, 9x9 equal, 5x5 and
// two or more fragments slower), else 64.
static int strip_blocks(const Shape &s, int nfrag) {
    const int pad4 = (s.OW + 63) / 64 * 64, pad2 = (s.OW + 31) / 32 * 32;
    const bool tie2 = nfrag == 1 && s.FH >= 7;
    return pad2 < pad4 || (pad2 == pad4 && tie2) ? 2 : 4;
}

bool plan_mfma(Plan &p) {
    if (p.dtype != DT_F16 && p.dtype != DT_BF16) return false;
    if (p.s.S != 1 || p.s.D != 1) return false;
    // tuning choices: mfma_cs=4|8|16 the channel slice, mfma_al=0|1 A
    // windows by DPP row shift / from LDS for every lane, mfma_nb=2|4 strips
    // of 32 / 64 output columns, mfma_pk=1|2|4 filter rows per MFMA,
    // mfma_fhk=0|1|F B operands read from LDS / kept in registers / kept
    // for the filter rows below F, mfma_ks=1|2 one or two wavefronts per
    // channel
    const int want_cs = tune_int("mfma_cs", 0), want_al = tune_int("mfma_al", -1),
              want_nb = tune_int("mfma_nb", 0), want_pk = tune_int("mfma_pk", 0),
              want_fhk = tune_int("mfma_fhk", -1), want_ks = tune_int("mfma_ks", 0);
    const int nfrag = (p.s.FW + 15) / 16;
    const int nb_pref = want_nb ? want_nb : strip_blocks(p.s, nfrag);
    const MfmaEntry *e = nullptr;
    int lds = 0;
    // The first entry (in table order) that `want` accepts, covers the shape
    // and fits `cap` bytes of LDS (0: the channel slice's own cap).
    auto pick = [&](auto want, int cap) {
        for (const auto &k : kMfma) {
            if (!want(k)) continue;
            if (want_nb && k.nb != want_nb) continue;
            if (want_pk && k.pk != want_pk) continue;
            if (want_ks && k.ks != want_ks) continue;
            if (want_fhk >= 0 &&
                (want_fhk <= 1 ? (k.fhk > 0) != (want_fhk > 0) : k.fhk != want_fhk))
                continue;
            // windows per output block: fragments of 16 taps, or with row
            // packing the KW-column windows that span 16 + FW - 1 columns
            const int need = k.pk == 1 ? nfrag : (15 + p.s.FW + 32 / k.pk - 1) / (32 / k.pk);
            // taller filters only where the chain is folded (four or more
            // windows), and at most 64 rows
            if (k.pk > 1 && p.s.FH > (k.nfrag >= 4 ? 64 : 32)) continue;
            if (k.dtype != p.dtype || k.nfrag != need || p.s.C % k.cs != 0) continue;
            if (k.fhk && k.pk == 1 && p.s.FH > k.fhk) continue;
            if (k.fht && p.s.FH != k.fht) continue;
            if (want_cs && k.cs != want_cs) continue;
            if (want_al >= 0 && k.al != want_al) continue;
            const int bytes = k.lds(p.s);
            // 16-channel slices run one 8-wavefront workgroup per CU; narrower
            // ones aim for at least two per CU unless nothing else fits
            const bool last = k.cs == 4 || want_cs;
            const int lim = cap ? cap : k.cs == 16 || last ? 160 * 1024 : 64 * 1024;
            if (bytes <= lim) {
                e = &k;
                lds = bytes;
                return true;
            }
        }
        return false;
    };
    // Filters of 34 to 65 taps (four or five packed windows), at the
    // preferred strip width: two workgroups per CU where the tile fits half
    // the CU's LDS (35x35 on 64-column strips); else one 8-wavefront
    // workgroup whose wavefronts split each channel's row groups (41 to 57
    // taps: 1.25-1.3x one 4-wavefront workgroup per CU, and 1.25x two
    // workgroups on 32-column strips); else one 4-wavefront workgroup (61
    // taps on 64-column strips, where the split tile no longer fits).
    const bool tall = !want_nb && p.s.FW >= 34 && p.s.FW <= 65;
    if (tall) {
        auto packed = [&](const MfmaEntry &k, int ks) {
            return k.pk > 1 && k.nfrag >= 4 && k.ks == ks && k.nb == nb_pref;
        };
        pick([&](const MfmaEntry &k) { return packed(k, 1); }, 80 * 1024) ||
            pick([&](const MfmaEntry &k) { return packed(k, 2); }, 160 * 1024) ||
            pick([&](const MfmaEntry &k) { return packed(k, 1); }, 160 * 1024);
    }
    // otherwise the preferred strip width first
    if (!e) pick([&](const MfmaEntry &k) { return k.nb == nb_pref; }, 0);
    if (!e) pick([&](const MfmaEntry &k) { return k.nb != nb_pref; }, 0);
    if (!e) return false;  // tall filters: the tile does not fit LDS
    const int ncs = p.s.C / e->cs;
    const int nct = (p.s.OW + 16 * e->nb - 1) / (16 * e->nb);
    const long long blocks = (long long)ncs * nct * p.s.N;
    if (blocks >= (1LL << 31)) return false;
    p.variant = V_MFMA;
    p.cs = e->cs;
    p.tm = 16;
    p.th = 16;
    // a strip walks the whole image height; the ring loads each row once
    p.tile_h = p.s.OH;
    p.tile_w = 16 * e->nb;
    p.tile_c = e->cs;
    p.aux0 = ncs;
    p.aux1 = nct;
    p.block = (e->cs >= 16 ? 512 : 256) * e->ks;
    p.aux2 = cu_slots(e->kfn, p.block, lds, p.s.FH);
    p.aux3 = (int)(e - kMfma);  // the tiling, for the fused prologue's plan
    p.grid = (uint32_t)blocks;
    p.lds_bytes = lds;
    p.launch = e->fn;
    if (e->pk > 1)
        snprintf(p.desc, sizeof(p.desc),
                 "mfma: 16x16x32 banded GEMM, %d filter rows per MFMA (%d windows of %d "
                 "cols), strips of %d cols x %d ch walked 16 rows at a time%s, LDS %d B, %u x %d",
                 e->pk, e->nfrag, 32 / e->pk, 16 * e->nb, e->cs,
                 e->ks > 1 ? ", row groups split over two wavefronts per channel" : "", lds,
                 p.grid, p.block);
    else
        snprintf(p.desc, sizeof(p.desc),
                 "mfma: 16x16x32 banded GEMM, strips of %d cols x %d ch walked 16 rows at a "
                 "time, %d fragment(s) of 16 taps, A by %s, LDS %d B, %u x %d",
                 16 * e->nb, e->cs, nfrag, e->al ? "LDS reads" : "DPP row shift", lds, p.grid,
                 p.block);
    return true;
}

// The forward pass with the fused prologue on the matrix cores, for a plan
// whose forward pass runs there: the forward plan's own tiling when the
// fused table has it (the fused kernel is then the forward kernel with U
// formed as its ring is written), else the preferred strip width, 8-channel
// slices before 4, the first tiling whose ring fits LDS.
bool plan_mfma_bn(Plan &b, const Plan &f) {
    if (f.variant != V_MFMA) return false;
    const int nfrag = (f.s.FW + 15) / 16;
    // mfma_pk=1|2|4, mfma_cs=4|8 and mfma_fhk=0|1 (tuning) as forward
    const int want_pk = tune_int("mfma_pk", 0), want_cs = tune_int("mfma_cs", 0),
              want_fhk = tune_int("mfma_fhk", -1);
    const int nb_pref = strip_blocks(f.s, nfrag);
    const MfmaEntry &fe = kMfma[f.aux3];
    const MfmaBnEntry *e = nullptr;
    int lds = 0;
    auto fits = [&](const MfmaBnEntry &k) {
        if (want_pk && k.pk != want_pk) return false;
        if (want_cs && k.cs != want_cs) return false;
        if (want_fhk >= 0 && (k.fhk > 0) != (want_fhk > 0)) return false;
        const int need = k.pk == 1 ? nfrag : (15 + f.s.FW + 32 / k.pk - 1) / (32 / k.pk);
        if (k.dtype != f.dtype || k.nfrag != need || f.s.C % k.cs != 0) return false;
        if (k.pk > 1 && f.s.FH > 32) return false;
        if (k.fhk && k.pk == 1 && f.s.FH > k.fhk) return false;
        if (k.fht && f.s.FH != k.fht) return false;
        const int bytes = k.lds(f.s);
        if (bytes > 160 * 1024) return false;
        e = &k;
        lds = bytes;
        return true;
    };
    for (const auto &k : kMfmaBn)
        if (fe.ks == 1 && k.cs == fe.cs && k.nb == fe.nb && k.nfrag == fe.nfrag &&
            k.fhk == fe.fhk && k.fht == fe.fht && k.pk == fe.pk && fits(k))
            break;
    for (int pass = 0; pass < 2 && !e; ++pass)
        for (const auto &k : kMfmaBn)
            if ((pass == 0) == (k.nb == nb_pref) && fits(k)) break;
    if (!e) return false;
    const int ncs = f.s.C / e->cs;
    const int nct = (f.s.OW + 16 * e->nb - 1) / (16 * e->nb);
    const long long blocks = (long long)ncs * nct * f.s.N;
    if (blocks >= (1LL << 31)) return false;
    b = f;
    b.cs = e->cs;
    b.tile_w = 16 * e->nb;
    b.tile_c = e->cs;
    b.aux0 = ncs;
    b.aux1 = nct;
    b.block = 256;
    b.aux2 = cu_slots(e->kfn, b.block, lds, b.s.FH);
    b.grid = (uint32_t)blocks;
    b.lds_bytes = lds;
    b.launch = nullptr;
    b.bn_launch = e->fn;
    const char *fmt = f.dtype == DT_F16 ? "fp16" : "bf16";
    if (e->pk > 1)
        snprintf(b.desc, sizeof(b.desc),
                 "mfma with the prologue fused: %d filter rows per MFMA (%d windows of %d "
                 "cols), strips of %d cols x %d ch, U rounded to %s as the ring is written, "
                 "LDS %d B, %u x %d",
                 e->pk, e->nfrag, 32 / e->pk, 16 * e->nb, e->cs, fmt, lds, b.grid, b.block);
    else
        snprintf(b.desc, sizeof(b.desc),
                 "mfma with the prologue fused: strips of %d cols x %d ch, %d fragment(s), U "
                 "rounded to %s as the ring is written, LDS %d B, %u x %d",
                 16 * e->nb, e->cs, nfrag, fmt, lds, b.grid, b.block);
    return true;
}

}  // namespace dw
