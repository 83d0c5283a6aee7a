// plan.h -- host-side plan of one forward depthwise convolution: validated
// shape, output extent and the kernel family / tiling chosen for it.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "dw_common.h"

namespace dw {

enum DType { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_I8 = 3 };
enum Variant { V_AUTO = 0, V_DIRECT = 1, V_ROWWIN = 2, V_LDSTILE = 3, V_MFMA = 4 };

struct Plan;
using LaunchFn = hipError_t (*)(const Plan &, const void *x, const void *w,
                                const void *bias, void *y, hipStream_t);
// The forward pass with the fused prologue act(x * bn_scale + bn_shift).
using LaunchBnFn = hipError_t (*)(const Plan &, const void *x, const void *w,
                                  const void *bias, const float *bn_scale,
                                  const float *bn_shift, int act, void *y, hipStream_t);

struct Plan {
    Shape s;
    int dtype;
    int variant;          // family launched for aligned pointers
    int elem_bytes;       // bytes of one stored x / w element
    // kernel-specific tiling (meaning depends on the family)
    int vec;              // channels per lane (one 4/8/16-byte vector)
    int tm;               // consecutive outputs along width per lane
    int th;               // output rows per lane / tile
    int cs;               // channels per tile
    // the output tile whose input span the kernel fetches once (a lane's
    // register tile, or a workgroup's LDS tile or strip): rows x columns x
    // channels
    int tile_h, tile_w, tile_c;
    int lds_bytes;        // dynamic LDS per workgroup
    int block;            // threads per workgroup
    uint32_t grid;        // workgroups
    int aux0, aux1, aux2, aux3;  // family-specific extra launch parameters
    LaunchFn launch;      // launcher for `variant`
    LaunchFn fallback;    // launcher for misaligned pointers (direct family)
    LaunchBnFn bn_launch;   // the same tiling with the fused prologue (NULL: none)
    LaunchBnFn bn_fallback; // the direct family with the fused prologue
    char desc[256];
};

// Backward-filter plan: pass 1 writes Z chunk sums per filter element into a
// caller-provided fp32 workspace, pass 2 merges them.  vec_launch needs
// 16-byte aligned x and dy (and C * element size a multiple of 16);
// one_launch takes any alignment.
struct BwfPlan;
using BwfLaunchFn = hipError_t (*)(const BwfPlan &, const void *x, const void *dy,
                                   float *dw, void *ws, hipStream_t);
struct BwfPlan {
    Shape s;
    int dtype;
    int vec;              // channels per lane
    int ncv, nfc;         // channel vectors, 8-tap column chunks
    int Z, rpc;           // chunks of the (n, oh) rows, rows per chunk
    size_t ws_bytes;      // enough for every pass 1 (Z, vZ or mZ chunk sums)
    BwfLaunchFn vec_launch, one_launch;
    // vec_launch's own chunking when it is the column stream (else vZ = Z)
    int vZ, vaux[5];
    long long vstrips;
    uint32_t vgrid;
    // matrix-core pass 1 (fp16 / bf16, stride 1, dilation 1), used when x,
    // dy and the workspace are 16-byte aligned: workgroup = one image, cs
    // channels, a chunk of mrpc output rows; mZ = N * mnrc chunk sums
    BwfLaunchFn mfma_launch;
    int mcs, mncs, mnrc, mrpc, mZ, mlds;
    uint32_t mgrid;
    char desc[256];
};
bool plan_bwd_filter(BwfPlan &b, const Plan &forward);
// Fills the matrix-core fields of `b` (b.s and b.dtype set); false when the
// shape is not covered.
bool plan_bwf_mfma(BwfPlan &b);
// Pass 2: dw[e] = pairwise sum over z < Z of ws[z * FH*FW*C + e].
hipError_t launch_bwf_reduce(const Shape &s, const float *ws, float *dw, int Z, hipStream_t st);

// Tuning choices for testing and A/B timing, read at plan creation from the
// DWCONV_TUNE environment variable: comma-separated key=value pairs
// (include/dwconv.h lists the keys).  tune() returns the value of `key` in a
// caller buffer (NULL when absent), tune_int() its integer value or `dflt`.
const char *tune(const char *key, char *buf, int len);
int tune_int(const char *key, int dflt);

// Output extent along one axis; 0 when not even one output fits.
int out_extent(int in, int f, int s, int d, int p);

// Validates and fills `p`.  Returns a dwconv_status_t value.
int make_plan(Plan &p, int N, int H, int W, int C, int FH, int FW, int S, int D,
              int P, int dtype, int variant);

// Per-family planners, defined next to their kernels.  Each returns true and
// fills the tiling and launcher when it can run the shape.
bool plan_direct(Plan &p);
// Backward data for any float shape, one lane per input element; b gets the
// forward plan's shape (dy N x OH x OW x C in, dx N x H x W x C out).
bool plan_bwd_direct(Plan &b, const Plan &forward);
// The forward pass with the fused prologue: the forward plan itself when its
// family fuses it, else the row-window / row-chunk or the direct family for
// the same shape.  Float dtypes only.
bool plan_bn_act(Plan &b, const Plan &forward);
bool plan_rowwin(Plan &p);
bool plan_ldstile(Plan &p);
bool plan_mfma(Plan &p);
bool plan_mfma_bn(Plan &b, const Plan &forward);

}  // namespace dw
