/*
 * dwref.c -- CPU oracle for the forward depthwise 2-D convolution.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file; only the test suite, the smoke check and the bench's CPU-baseline
 * leg do.  It shares no code, header or constant with the HIP library.
 *
 * What it computes (all references are to the pages this project follows):
 *
 *   * "Flash-DWC: Making Depthwise Convolution Compute-Efficient on GPUs",
 *     section 2.1 (standard vs. depthwise convolution): in a depthwise
 *     convolution every channel has its own FH x FW filter, IC = OC, and each
 *     output element is the inner product of one channel's input patch with
 *     that channel's filter.  Section 2.3 fixes the channel-last layout:
 *     X is N x IH x IW x C, Y is N x OH x OW x C and the filter is re-laid as
 *     FH x FW x C.
 *   * "Tiles, halos and partial sums", section "Partition tensors to fit
 *     storage": an output extent T with stride S, dilation D and kernel R needs
 *     an input extent (T-1)S + (R-1)D + 1, and border padding is generated
 *     (zeros), not fetched.  The output extent used here is the largest T
 *     whose span fits the zero-padded input H + 2P.  The same passage says the
 *     bias is added once and the partial sum is never rounded in between.
 *   * "Outline of Programming Massively Parallel Processors Parallel Concepts
 *     Part", section "2D Convolution": the filter is applied without flipping
 *     (input index = output index - radius + filter index) and positions that
 *     fall outside the image count as zero.
 *
 * So, for every n, oh, ow, c:
 *
 *   Y[n,oh,ow,c] = bias[c]
 *                + sum_{fh<FH, fw<FW} X[n, oh*S - P + fh*D, ow*S - P + fw*D, c]
 *                                     * W[fh, fw, c]
 *
 * with out-of-image X taken as zero.  Floating-point inputs arrive already
 * widened to double (every fp32/fp16/bf16 value is exact in double, and so is
 * every product of two of them); the sum is accumulated in double.  int8
 * inputs accumulate exactly in int64.  Alongside each float output the oracle
 * returns sum |x*w| over the same taps, the scale that the floating-point
 * tolerance is stated against.
 *
 * The loop nest is deliberately plain: no blocking, no reordering, one output
 * at a time.
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>

/* Output extent along one axis: the largest O >= 1 whose input span
 * (O-1)*S + (F-1)*D + 1 fits in IN + 2*P, or 0 when not even one output fits
 * or an argument is out of range. */
int dwref_out_dim(int in, int f, int s, int d, int p)
{
    if (in < 1 || f < 1 || s < 1 || d < 1 || p < 0) return 0;
    long long room = (long long)in + 2LL * p - (long long)(f - 1) * d - 1;
    if (room < 0) return 0;
    long long o = room / s + 1;
    if (o > 0x7fffffffLL) return 0;
    return (int)o;
}

static int shape_ok(int N, int H, int W, int C, int FH, int FW, int S, int D, int P,
                    int *OH, int *OW)
{
    if (N < 1 || C < 1) return 0;
    *OH = dwref_out_dim(H, FH, S, D, P);
    *OW = dwref_out_dim(W, FW, S, D, P);
    return *OH > 0 && *OW > 0;
}

/* One output element, floating point.  Returns the exact-ish (fp64) sum and
 * writes sum |x*w| to *scale. */
static double one_out_f64(const double *x, const double *w, const double *bias,
                          int H, int W, int C, int FH, int FW, int S, int D, int P,
                          long long n, int oh, int ow, int c, double *scale)
{
    double acc = bias ? bias[c] : 0.0;
    double sabs = 0.0;
    for (int fh = 0; fh < FH; ++fh) {
        int ih = oh * S - P + fh * D;
        if (ih < 0 || ih >= H) continue;          /* generated zero padding */
        for (int fw = 0; fw < FW; ++fw) {
            int iw = ow * S - P + fw * D;
            if (iw < 0 || iw >= W) continue;
            double xv = x[((n * H + ih) * (long long)W + iw) * C + c];
            double wv = w[((long long)fh * FW + fw) * C + c];
            double prod = xv * wv;
            acc += prod;
            sabs += fabs(prod);
        }
    }
    *scale = sabs;
    return acc;
}

static int64_t one_out_i8(const int8_t *x, const int8_t *w, const int32_t *bias,
                          int H, int W, int C, int FH, int FW, int S, int D, int P,
                          long long n, int oh, int ow, int c)
{
    int64_t acc = bias ? (int64_t)bias[c] : 0;
    for (int fh = 0; fh < FH; ++fh) {
        int ih = oh * S - P + fh * D;
        if (ih < 0 || ih >= H) continue;
        for (int fw = 0; fw < FW; ++fw) {
            int iw = ow * S - P + fw * D;
            if (iw < 0 || iw >= W) continue;
            int64_t xv = x[((n * H + ih) * (long long)W + iw) * C + c];
            int64_t wv = w[((long long)fh * FW + fw) * C + c];
            acc += xv * wv;
        }
    }
    return acc;
}

/* Full forward pass, floating point.  x: N*H*W*C doubles, w: FH*FW*C doubles,
 * bias: C doubles or NULL, y and scale: N*OH*OW*C doubles (scale may be NULL).
 * Only images [n0, n1) are computed, so a caller can split the batch.
 * Returns 0 on success, -1 on a bad shape. */
int dwref_fwd_f64(const double *x, const double *w, const double *bias,
                  double *y, double *scale,
                  int N, int H, int W, int C, int FH, int FW, int S, int D, int P,
                  int n0, int n1)
{
    int OH, OW;
    if (!shape_ok(N, H, W, C, FH, FW, S, D, P, &OH, &OW)) return -1;
    if (n0 < 0 || n1 > N || n0 > n1) return -1;
    for (long long n = n0; n < n1; ++n)
        for (int oh = 0; oh < OH; ++oh)
            for (int ow = 0; ow < OW; ++ow)
                for (int c = 0; c < C; ++c) {
                    long long o = ((n * OH + oh) * (long long)OW + ow) * C + c;
                    double s;
                    y[o] = one_out_f64(x, w, bias, H, W, C, FH, FW, S, D, P,
                                       n, oh, ow, c, &s);
                    if (scale) scale[o] = s;
                }
    return 0;
}

/* Full forward pass, int8 x int8 with an int32 bias, accumulated exactly in
 * int64.  Same layouts and batch split as dwref_fwd_f64. */
int dwref_fwd_i8(const int8_t *x, const int8_t *w, const int32_t *bias, int64_t *y,
                 int N, int H, int W, int C, int FH, int FW, int S, int D, int P,
                 int n0, int n1)
{
    int OH, OW;
    if (!shape_ok(N, H, W, C, FH, FW, S, D, P, &OH, &OW)) return -1;
    if (n0 < 0 || n1 > N || n0 > n1) return -1;
    for (long long n = n0; n < n1; ++n)
        for (int oh = 0; oh < OH; ++oh)
            for (int ow = 0; ow < OW; ++ow)
                for (int c = 0; c < C; ++c) {
                    long long o = ((n * OH + oh) * (long long)OW + ow) * C + c;
                    y[o] = one_out_i8(x, w, bias, H, W, C, FH, FW, S, D, P,
                                      n, oh, ow, c);
                }
    return 0;
}

/* Selected outputs only: idx[k] is a flat index into the N*OH*OW*C output.
 * Used where the full pass would take too long on the CPU. */
int dwref_points_f64(const double *x, const double *w, const double *bias,
                     const int64_t *idx, int64_t npts, double *y, double *scale,
                     int N, int H, int W, int C, int FH, int FW, int S, int D, int P)
{
    int OH, OW;
    if (!shape_ok(N, H, W, C, FH, FW, S, D, P, &OH, &OW)) return -1;
    long long total = (long long)N * OH * OW * C;
    for (int64_t k = 0; k < npts; ++k) {
        long long o = idx[k];
        if (o < 0 || o >= total) return -1;
        int c = (int)(o % C);
        long long r = o / C;
        int ow = (int)(r % OW); r /= OW;
        int oh = (int)(r % OH);
        long long n = r / OH;
        double s;
        y[k] = one_out_f64(x, w, bias, H, W, C, FH, FW, S, D, P, n, oh, ow, c, &s);
        if (scale) scale[k] = s;
    }
    return 0;
}

int dwref_points_i8(const int8_t *x, const int8_t *w, const int32_t *bias,
                    const int64_t *idx, int64_t npts, int64_t *y,
                    int N, int H, int W, int C, int FH, int FW, int S, int D, int P)
{
    int OH, OW;
    if (!shape_ok(N, H, W, C, FH, FW, S, D, P, &OH, &OW)) return -1;
    long long total = (long long)N * OH * OW * C;
    for (int64_t k = 0; k < npts; ++k) {
        long long o = idx[k];
        if (o < 0 || o >= total) return -1;
        int c = (int)(o % C);
        long long r = o / C;
        int ow = (int)(r % OW); r /= OW;
        int oh = (int)(r % OH);
        long long n = r / OH;
        y[k] = one_out_i8(x, w, bias, H, W, C, FH, FW, S, D, P, n, oh, ow, c);
    }
    return 0;
}

/* Backward data (the gradient with respect to the input), from its
 * definition: the forward pass is linear in X, and its adjoint sends every
 * output gradient dY[n,oh,ow,c] back along the taps that produced Y:
 *
 *   dX[n,ih,iw,c] = sum over (oh, ow, fh, fw) with oh*S - P + fh*D = ih and
 *                   ow*S - P + fw*D = iw of dY[n,oh,ow,c] * W[fh,fw,c]
 *
 * ("Flash-DWC: Making Depthwise Convolution Compute-Efficient on GPUs",
 * section 5.1: the input gradient of a depthwise convolution; for stride 1
 * the same sum is a depthwise convolution of dY with the filter rotated by
 * 180 degrees.)  Written here as the plain scatter over the forward's taps,
 * for any stride, dilation and padding.  dy: N*OH*OW*C, w: FH*FW*C,
 * dx and scale: N*H*W*C (scale = sum |dy*w| per dx element, may be NULL).
 * Images [n0, n1) only.  Returns 0, or -1 on a bad shape. */
int dwref_bwd_data_f64(const double *dy, const double *w, double *dx, double *scale,
                       int N, int H, int W, int C, int FH, int FW, int S, int D, int P,
                       int n0, int n1)
{
    int OH, OW;
    if (!shape_ok(N, H, W, C, FH, FW, S, D, P, &OH, &OW)) return -1;
    if (n0 < 0 || n1 > N || n0 > n1) return -1;
    for (long long n = n0; n < n1; ++n)
        for (long long i = (n * H) * (long long)W * C; i < ((n + 1) * H) * (long long)W * C; ++i) {
            dx[i] = 0.0;
            if (scale) scale[i] = 0.0;
        }
    for (long long n = n0; n < n1; ++n)
        for (int oh = 0; oh < OH; ++oh)
            for (int ow = 0; ow < OW; ++ow)
                for (int c = 0; c < C; ++c) {
                    double g = dy[((n * OH + oh) * (long long)OW + ow) * C + c];
                    for (int fh = 0; fh < FH; ++fh) {
                        int ih = oh * S - P + fh * D;
                        if (ih < 0 || ih >= H) continue;  /* a padding tap: no input */
                        for (int fw = 0; fw < FW; ++fw) {
                            int iw = ow * S - P + fw * D;
                            if (iw < 0 || iw >= W) continue;
                            double prod = g * w[((long long)fh * FW + fw) * C + c];
                            long long i = ((n * H + ih) * (long long)W + iw) * C + c;
                            dx[i] += prod;
                            if (scale) scale[i] += fabs(prod);
                        }
                    }
                }
    return 0;
}

/* Backward filter (the gradient with respect to the filter), from its
 * definition: the forward pass is linear in W, and the gradient of
 * sum Y*dY with respect to W[fh,fw,c] is the sum, over every output that
 * tap touched, of the input it multiplied times that output's gradient:
 *
 *   dW[fh,fw,c] = sum_{n, oh, ow} X[n, oh*S - P + fh*D, ow*S - P + fw*D, c]
 *                                 * dY[n, oh, ow, c]
 *
 * with out-of-image X taken as zero ("Flash-DWC: Making Depthwise
 * Convolution Compute-Efficient on GPUs", section 5.1: the filter gradient
 * is a convolution of the input with the output gradient, a reduction over
 * the batch and the output positions).  x: N*H*W*C, dy: N*OH*OW*C,
 * dw and scale: FH*FW*C (scale = sum |x*dy| per tap, may be NULL).
 *
 * Only channels [c0, c1) are computed (channels are independent, so callers
 * may split the channels over threads; every other element of dw and scale
 * is left untouched).  Every dW[fh,fw,c] starts at zero and receives its
 * products in the order of (n, oh, ow), the order of the sum above; the
 * outputs are visited in that order and each one adds its products to the
 * taps it touched, so the inputs are read along C.  fp64.  Returns 0, or -1
 * on a bad shape or channel range. */
int dwref_bwd_filter_f64(const double *x, const double *dy, double *dw, double *scale,
                         int N, int H, int W, int C, int FH, int FW, int S, int D, int P,
                         int c0, int c1)
{
    int OH, OW;
    if (!shape_ok(N, H, W, C, FH, FW, S, D, P, &OH, &OW)) return -1;
    if (c0 < 0 || c1 > C || c0 > c1) return -1;
    for (int fh = 0; fh < FH; ++fh)
        for (int fw = 0; fw < FW; ++fw)
            for (int c = c0; c < c1; ++c) {
                long long o = ((long long)fh * FW + fw) * C + c;
                dw[o] = 0.0;
                if (scale) scale[o] = 0.0;
            }
    for (long long n = 0; n < N; ++n)
        for (int oh = 0; oh < OH; ++oh)
            for (int ow = 0; ow < OW; ++ow) {
                const double *g = dy + ((n * OH + oh) * (long long)OW + ow) * C;
                for (int fh = 0; fh < FH; ++fh) {
                    int ih = oh * S - P + fh * D;
                    if (ih < 0 || ih >= H) continue;          /* padding: no input */
                    for (int fw = 0; fw < FW; ++fw) {
                        int iw = ow * S - P + fw * D;
                        if (iw < 0 || iw >= W) continue;
                        const double *xi = x + ((n * H + ih) * (long long)W + iw) * C;
                        long long o = ((long long)fh * FW + fw) * C;
                        for (int c = c0; c < c1; ++c) {
                            double prod = xi[c] * g[c];
                            dw[o + c] += prod;
                            if (scale) scale[o + c] += fabs(prod);
                        }
                    }
                }
            }
    return 0;
}

/* Round-to-nearest-even of a finite or infinite double v to a binary format
 * with `mant` stored significand bits and smallest normal exponent `emin`,
 * returned as a double (exact).  The quantum is the value of the last
 * significand bit at v's exponent, never finer than the subnormal spacing
 * 2^(emin - mant); results past `maxf` become infinities (IEEE 754
 * overflow under round-to-nearest); NaN stays NaN.  binary16: mant 10,
 * emin -14, maxf 65504.  bfloat16: mant 7, emin -126, maxf (2 - 2^-7) 2^127. */
static double round_binary(double v, int mant, int emin, double maxf)
{
    if (v != v || isinf(v)) return v;
    double a = fabs(v);
    int k;
    frexp(a, &k);                 /* a = m 2^k with 0.5 <= m < 1 (or a = 0) */
    int e = k - 1;                /* exponent of the leading bit */
    if (e < emin) e = emin;
    double q = ldexp(1.0, e - mant);
    double r = nearbyint(a / q) * q;  /* a / q is exact; ties go to even */
    if (r > maxf) r = INFINITY;
    return v < 0 ? -r : r;
}

/* The fused prologue's input value in the storage format: fmt 1 binary16,
 * 2 bfloat16. */
static double round_storage(double u, int fmt)
{
    if (fmt == 1) return round_binary(u, 10, -14, 65504.0);
    return round_binary(u, 7, -126, ldexp(255.0, 120));
}

/* Forward pass with the per-channel affine (batch normalization folded to a
 * scale and a shift) and an activation fused in front of the convolution
 * ("Flash-DWC: Making Depthwise Convolution Compute-Efficient on GPUs",
 * section 5.2: the common BN + Act + DWC pattern, with BN and Act applied to
 * the input inside the convolution kernel).  The convolution's input is
 *
 *   U[n,h,w,c] = act(X[n,h,w,c] * bn_scale[c] + bn_shift[c])
 *
 * with act 0 = identity, 1 = max(u, 0), 2 = min(max(u, 0), 6); positions
 * outside the image are zeros of U (the convolution pads its own input, so
 * they are not act(bn_shift)).  Then
 *
 *   Y[n,oh,ow,c] = bias[c] + sum over in-image taps of U * W[fh,fw,c]
 *
 * accumulated in fp64.  fmt 0 (fp32 data): U exact in fp64.  fmt 1 / 2
 * (fp16 / bf16 data): U is the tensor the separate BN + Act pass would store
 * in the data's format -- section 4.1 of the same page: mixed precision keeps
 * tensors in FP16 and multiplies FP16 operands, accumulating in FP32 -- so
 * X * s + b is one fp32 fused multiply-add (fmaf, rounded once), the
 * activation applies to that fp32 value, and U is it rounded to nearest even
 * in binary16 / bfloat16.  scale = sum over the same taps of |X*s + b| * |W|
 * (the magnitude before the activation; the fp32 value for fmt 1 / 2).  Same
 * layouts and batch split as dwref_fwd_f64.  Returns 0, or -1 on a bad shape,
 * activation or format. */
int dwref_fwd_bnact_f64(const double *x, const double *w, const double *bias,
                        const double *bn_scale, const double *bn_shift, int act, int fmt,
                        double *y, double *scale,
                        int N, int H, int W, int C, int FH, int FW, int S, int D, int P,
                        int n0, int n1)
{
    int OH, OW;
    if (!shape_ok(N, H, W, C, FH, FW, S, D, P, &OH, &OW)) return -1;
    if (n0 < 0 || n1 > N || n0 > n1 || act < 0 || act > 2 || fmt < 0 || fmt > 2)
        return -1;
    for (long long n = n0; n < n1; ++n)
        for (int oh = 0; oh < OH; ++oh)
            for (int ow = 0; ow < OW; ++ow)
                for (int c = 0; c < C; ++c) {
                    double acc = bias ? bias[c] : 0.0;
                    double sabs = 0.0;
                    for (int fh = 0; fh < FH; ++fh) {
                        int ih = oh * S - P + fh * D;
                        if (ih < 0 || ih >= H) continue;      /* zero of U */
                        for (int fw = 0; fw < FW; ++fw) {
                            int iw = ow * S - P + fw * D;
                            if (iw < 0 || iw >= W) continue;
                            double xv = x[((n * H + ih) * (long long)W + iw) * C + c];
                            double pre = fmt ? (double)fmaf((float)xv, (float)bn_scale[c],
                                                            (float)bn_shift[c])
                                             : xv * bn_scale[c] + bn_shift[c];
                            double u = pre;
                            if (act >= 1 && u < 0.0) u = 0.0;
                            if (act == 2 && u > 6.0) u = 6.0;
                            if (fmt) u = round_storage(u, fmt);
                            double wv = w[((long long)fh * FW + fw) * C + c];
                            acc += u * wv;
                            sabs += fabs(pre) * fabs(wv);
                        }
                    }
                    long long o = ((n * OH + oh) * (long long)OW + ow) * C + c;
                    y[o] = acc;
                    if (scale) scale[o] = sabs;
                }
    return 0;
}
