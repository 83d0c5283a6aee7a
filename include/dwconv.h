/*
 * dwconv.h -- C ABI of the MI355X (gfx950) depthwise 2-D convolution: the
 * forward pass and its backward-data and backward-filter passes.
 *
 * Operation ("Flash-DWC: Making Depthwise Convolution Compute-Efficient on
 * GPUs", sections 2.1 and 2.3; "Tiles, halos and partial sums", section
 * "Partition tensors to fit storage"):
 *
 *   Y[n,oh,ow,c] = bias[c] + sum_{fh<FH, fw<FW}
 *                   X[n, oh*S - P + fh*D, ow*S - P + fw*D, c] * Wt[fh,fw,c]
 *
 * Every channel is filtered by its own FH x FW filter (input channels =
 * output channels = C).  The filter is applied as a correlation (not
 * flipped).  Input positions outside the image read as zero (padding is
 * generated, never fetched).  OH = floor((H + 2P - D(FH-1) - 1)/S) + 1, the
 * largest output extent whose input span (OH-1)S + (FH-1)D + 1 fits the
 * padded height; OW likewise.  Stride S, dilation D and padding P apply to
 * both axes; FH and FW may differ.
 *
 * Layouts (dense, row-major, channel last):
 *   x    N  x H  x W  x C
 *   w    FH x FW x C          (the filter re-laid channel-last)
 *   bias C                    (may be NULL: no bias)
 *   y    N  x OH x OW x C
 *
 * Element types per dtype:
 *   DWCONV_F32   x, w float     bias float   y float    accumulate fp32
 *   DWCONV_F16   x, w fp16      bias float   y fp16     accumulate fp32
 *   DWCONV_BF16  x, w bf16      bias float   y bf16     accumulate fp32
 *   DWCONV_I8    x, w int8      bias int32   y int32    accumulate int32 (exact)
 * The bias is in the accumulator type and is added once; partial sums are
 * never rounded to the storage type before the end; fp16/bf16 outputs are
 * rounded once, to nearest even, from the fp32 sum.
 *
 * Ownership: the caller allocates and owns every buffer (device memory),
 * including the backward-filter workspace.  The library allocates no device
 * memory; its code object holds one scratch array of DWCONV_SCRATCH_BYTES per
 * GPU, used only by dwconv_bwd_filter_noalloc.  A handle holds host-side plan
 * data only, is immutable after creation, and may be used from several host
 * threads and on several streams at once.
 *
 * Errors: every function returns a status and never throws.  Nothing here
 * synchronises the device.
 *
 * Tuning (for tests and A/B timing only): when a plan is created, the
 * environment variable DWCONV_TUNE may hold comma-separated key=value
 * choices that force a compiled alternative; unset, the planner chooses.
 * Keys: mfma_cs=4|8|16, mfma_al=0|1, mfma_nb=2|4, mfma_pk=1|2|4,
 * mfma_fhk=0|1|F, mfma_ks=1|2, mfma_slots=N (the matrix-core kernel's
 * channel slice, A-operand source, strip width, filter rows per MFMA, B
 * operands kept in registers, one or two wavefronts per channel, and the
 * workgroups per CU whose tiles are numbered consecutively), tile=TMxTH[pPF[n][l|i]] (a column-stream
 * tiling), chunk_tm=8, lds_tb=1..64 (the LDS tile's height), bwf_valu=1 and
 * bwf_nocs=1 (filter-gradient pass 1 on the vector kernel).  A choice that
 * no compiled kernel provides makes dwconv_create_variant fail with
 * DWCONV_ERR_UNSUPPORTED for that family.
 */
#ifndef DWCONV_H
#define DWCONV_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DWCONV_F32 = 0,
    DWCONV_F16 = 1,
    DWCONV_BF16 = 2,
    DWCONV_I8 = 3
} dwconv_dtype_t;

typedef enum {
    DWCONV_OK = 0,
    DWCONV_ERR_INVALID_ARG = 1,  /* bad shape, dtype, pointer or variant       */
    DWCONV_ERR_UNSUPPORTED = 2,  /* valid operation this build cannot run      */
    DWCONV_ERR_HIP = 3,          /* the HIP runtime reported an error          */
    DWCONV_ERR_ALLOC = 4,        /* host memory for the plan could not be had  */
    DWCONV_ERR_SCRATCH = 5       /* needs more than DWCONV_SCRATCH_BYTES        */
} dwconv_status_t;

/* Size of the library's own scratch array per GPU, used by
 * dwconv_bwd_filter_noalloc. */
#define DWCONV_SCRATCH_BYTES (64u << 20)

/* Kernel families.  AUTO lets the planner choose; the others force one (for
 * testing and A/B timing) and make dwconv_create fail with
 * DWCONV_ERR_UNSUPPORTED when that family cannot run the shape. */
typedef enum {
    DWCONV_VARIANT_AUTO = 0,
    DWCONV_VARIANT_DIRECT = 1,   /* one lane per output element; any shape      */
    DWCONV_VARIANT_ROWWIN = 2,   /* width-first register window, 16-B vectors   */
    DWCONV_VARIANT_LDSTILE = 3,  /* LDS halo tile + register window             */
    DWCONV_VARIANT_MFMA = 4      /* banded-filter GEMM on the matrix cores      */
} dwconv_variant_t;

/* Activation of the fused forward prologue (dwconv_fwd_bn_act). */
typedef enum {
    DWCONV_ACT_NONE = 0,         /* identity                                    */
    DWCONV_ACT_RELU = 1,         /* max(u, 0)                                   */
    DWCONV_ACT_RELU6 = 2         /* min(max(u, 0), 6)                           */
} dwconv_act_t;

typedef struct dwconv_plan *dwconv_handle_t;

/* Validates the operation and builds a plan.  Touches no GPU state.
 * Rejects (DWCONV_ERR_INVALID_ARG): out == NULL; N, H, W, C, FH, FW, stride
 * or dilation < 1; pad < 0; an empty output (OH < 1 or OW < 1); an unknown
 * dtype; tensors with 2^31 or more elements; for DWCONV_I8 a filter of more
 * than 131071 taps (FH*FW*128*128 would no longer fit int32).  With DWCONV_I8
 * the caller keeps bias + products inside int32; past it the sum wraps (two's
 * complement).  On failure *out is set to NULL. */
dwconv_status_t dwconv_create(dwconv_handle_t *out, int N, int H, int W, int C,
                              int FH, int FW, int stride, int dilation, int pad,
                              dwconv_dtype_t dtype);

/* As dwconv_create, with the kernel family forced (DWCONV_VARIANT_AUTO is the
 * same as dwconv_create). */
dwconv_status_t dwconv_create_variant(dwconv_handle_t *out, int N, int H, int W,
                                      int C, int FH, int FW, int stride,
                                      int dilation, int pad, dwconv_dtype_t dtype,
                                      dwconv_variant_t variant);

/* Enqueues the forward pass on `stream` (0 = the null stream) and returns
 * without waiting.  x, w, y: device pointers to the layouts above; bias:
 * device pointer or NULL.  y must not overlap x, w or bias.  Any alignment is
 * accepted (pointers that are not 16-byte aligned, or rows whose byte length
 * is not a multiple of 16, make the planner fall back to a slower kernel
 * family, never to an error).  Returns DWCONV_ERR_INVALID_ARG for a NULL
 * handle, x, w or y, and DWCONV_ERR_HIP if the launch fails. */
dwconv_status_t dwconv_fwd(dwconv_handle_t h, const void *x, const void *w,
                           const void *bias, void *y, hipStream_t stream);

/* Forward pass with a fused prologue ("Flash-DWC: Making Depthwise
 * Convolution Compute-Efficient on GPUs", section 5.2: batch normalization
 * and the activation that usually precede a depthwise convolution, applied to
 * its input inside the convolution kernel):
 *
 *   U[n,h,w,c]    = act(x[n,h,w,c] * bn_scale[c] + bn_shift[c])
 *   y[n,oh,ow,c]  = bias[c] + sum_{fh,fw} U[n, oh*S-P+fh*D, ow*S-P+fw*D, c]
 *                                         * w[fh,fw,c]
 *
 * U is computed in fp32 with one fused multiply-add and the activation per
 * input value; for fp16 and bf16 data it is then rounded to nearest even in
 * the data's format (the tensor a separate BN + Act pass would store, and
 * what section 4.1 of the same page multiplies: FP16 operands with FP32
 * accumulation); fp32 data keeps the fp32 value.  Padding positions are
 * zeros of U.  bn_scale and bn_shift are C fp32 device values each -- batch
 * normalization folded by the caller (scale = gamma / sqrt(var + eps),
 * shift = beta - mean * scale) -- owned by the caller, any 4-byte alignment.
 * x, w, bias and y as for dwconv_fwd; the forward pass's tolerance applies,
 * stated against sum |x*s + b| * |w|.  Every float family fuses the prologue: the
 * vector families form U as each input vector is loaded, the matrix cores as
 * their LDS ring is written, on the forward plan's own tiling.  LDS-tile
 * shapes run a row-window, row-chunk or direct kernel here.
 * Cost: measured on MI355X at 1.05x dwconv_fwd's time for the fp32 3x3
 * MobileNet layer, 1.07x for the fp16 7x7 ConvNeXt layer and 1.15x for the
 * bf16 31x31 large-kernel layer.
 * Enqueued on `stream` without waiting.  Returns DWCONV_ERR_INVALID_ARG for a
 * NULL handle, x, w, y, bn_scale or bn_shift or an unknown activation,
 * DWCONV_ERR_UNSUPPORTED for int8 and DWCONV_ERR_HIP if the launch fails. */
dwconv_status_t dwconv_fwd_bn_act(dwconv_handle_t h, const void *x, const void *w,
                                  const void *bias, const float *bn_scale,
                                  const float *bn_shift, dwconv_act_t act, void *y,
                                  hipStream_t stream);

/* 1 when dwconv_fwd_bn_act can run the handle's operation (float dtypes),
 * else 0 (also for NULL); and a one-line description of its kernel ("" if
 * none). */
int dwconv_fwd_bn_act_supported(dwconv_handle_t h);
const char *dwconv_fwd_bn_act_describe(dwconv_handle_t h);

/* Backward data: the gradient with respect to the input of the forward
 * operation the handle plans ("Flash-DWC: Making Depthwise Convolution
 * Compute-Efficient on GPUs", section 5.1):
 *
 *   dX[n,ih,iw,c] = sum over (oh, ow, fh, fw) with oh*S - P + fh*D = ih and
 *                   ow*S - P + fw*D = iw of dY[n,oh,ow,c] * Wt[fh,fw,c]
 *
 * At stride 1 with a square filter and P <= D(F-1) this is a forward pass
 * over dY with the filter rotated by 180 degrees and padding D(F-1) - P, run
 * by the forward kernels reading the filter rotated in place (no copy is
 * made); every other float shape runs a direct kernel that sums each input
 * element's taps.
 *   dy  N x OH x OW x C   (float / fp16 / bf16, as y)
 *   w   FH x FW x C       (the forward filter, not rotated)
 *   dx  N x H  x W  x C   (as x; overwritten)
 * Partial sums are fp32; fp16/bf16 dx is rounded once.  Enqueued on `stream`
 * without waiting; dx must not overlap dy or w; any alignment is accepted.
 * Returns DWCONV_ERR_INVALID_ARG for a NULL handle, dy, w or dx,
 * DWCONV_ERR_UNSUPPORTED when the plan has no backward-data pass (int8), and
 * DWCONV_ERR_HIP if the launch fails. */
dwconv_status_t dwconv_bwd_data(dwconv_handle_t h, const void *dy, const void *w,
                                void *dx, hipStream_t stream);

/* 1 when dwconv_bwd_data can run the handle's operation, else 0 (also for
 * NULL); and a one-line description of the kernel it launches ("" if none). */
int dwconv_bwd_data_supported(dwconv_handle_t h);
const char *dwconv_bwd_data_describe(dwconv_handle_t h);

/* Backward filter: the gradient with respect to the filter of the forward
 * operation the handle plans ("Flash-DWC: Making Depthwise Convolution
 * Compute-Efficient on GPUs", section 5.1):
 *
 *   dW[fh,fw,c] = sum_{n, oh, ow} X[n, oh*S - P + fh*D, ow*S - P + fw*D, c]
 *                                 * dY[n, oh, ow, c]
 *
 * (out-of-image X is zero).  Any stride, dilation, padding and filter shape.
 *   x          N x H x W x C      (as for the forward pass)
 *   dy         N x OH x OW x C    (as y)
 *   dw         FH x FW x C float  (fp32 for every float dtype; overwritten)
 *   workspace  at least dwconv_bwd_filter_workspace() bytes of device
 *              memory, 4-byte aligned, owned by the caller; its contents on
 *              entry do not matter and are undefined on return
 * The batch and output positions are split into chunks whose fp32 sums land
 * in the workspace; a second kernel adds them pairwise, so the result is the
 * same on every run (no atomics).  Enqueued on `stream` without waiting.
 * Returns DWCONV_ERR_INVALID_ARG for a NULL argument or a misaligned dw or
 * workspace, DWCONV_ERR_UNSUPPORTED for int8, DWCONV_ERR_HIP if a launch
 * fails. */
dwconv_status_t dwconv_bwd_filter_workspace(dwconv_handle_t h, size_t *bytes);
dwconv_status_t dwconv_bwd_filter(dwconv_handle_t h, const void *x, const void *dy,
                                  float *dw, void *workspace, hipStream_t stream);

/* Backward filter for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): dwconv_bwd_filter with the workspace taken from an array of
 * DWCONV_SCRATCH_BYTES (64 MiB) that the library's code object holds on every
 * GPU it runs on, until the process ends.  The same kernels and the same
 * result as dwconv_bwd_filter.  Allocates nothing and calls no allocating
 * routine; the first call on a device looks up that device's copy of the
 * array (hipGetSymbolAddress) with the device current.
 *   x, dy, dw   as for dwconv_bwd_filter (caller-owned device memory)
 * The array needs no clearing: pass 1 writes every value pass 2 reads.
 * Every call on one GPU shares that GPU's array, so calls that overlap on
 * one GPU (on different streams, or from several host threads without
 * ordering) race and give undefined results; calls in one stream order do
 * not.  Returns DWCONV_ERR_INVALID_ARG for a NULL argument or a misaligned
 * dw, DWCONV_ERR_UNSUPPORTED for int8, DWCONV_ERR_SCRATCH (before touching
 * the GPU) when dwconv_bwd_filter_workspace() exceeds DWCONV_SCRATCH_BYTES,
 * and DWCONV_ERR_HIP if the lookup or a launch fails. */
dwconv_status_t dwconv_bwd_filter_noalloc(dwconv_handle_t h, const void *x, const void *dy,
                                          float *dw, hipStream_t stream);

/* A one-line description of the backward-filter kernels ("" if none). */
const char *dwconv_bwd_filter_describe(dwconv_handle_t h);

/* Frees the plan.  NULL is a no-op. */
dwconv_status_t dwconv_destroy(dwconv_handle_t h);

/* Output extent of a plan. */
dwconv_status_t dwconv_output_dims(dwconv_handle_t h, int *OH, int *OW);

/* Kernel family the plan will launch for 16-byte aligned pointers, and a
 * one-line description of its tiling (static strings owned by the library or
 * the plan; valid until dwconv_destroy). */
dwconv_variant_t dwconv_plan_variant(dwconv_handle_t h);
const char *dwconv_plan_describe(dwconv_handle_t h);

/* The output tile of the plan's forward kernel whose input span is fetched
 * as one piece ("Tiles, halos and partial sums", "Partition tensors to fit
 * storage": a tile of Th x Tw outputs reads (Th-1)S + (FH-1)D + 1 by
 * (Tw-1)S + (FW-1)D + 1 input pixels): *tile_h rows x *tile_w columns x
 * *tile_c channels.  It is a lane's register tile (direct: 1 x 1 x 1; row
 * window: 1 x TM x VEC; column stream: TH x TM x VEC), a workgroup's LDS
 * tile (TB x 4TM x all C), or a matrix-core strip (all OH rows x 16NB
 * columns x CS channels).  Host only; DWCONV_ERR_INVALID_ARG for a NULL
 * argument. */
dwconv_status_t dwconv_plan_tile(dwconv_handle_t h, int *tile_h, int *tile_w, int *tile_c);

/* Static, human-readable name of a status. */
const char *dwconv_status_string(dwconv_status_t s);

#ifdef __cplusplus
}
#endif

#endif /* DWCONV_H */
