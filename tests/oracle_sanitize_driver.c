/* Host-only driver for the oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py builds it with
 * gcc together with oracle/dwref.c).  It calls every entry point of the
 * oracle on random small shapes -- strides, dilations, paddings up to the
 * filter span, non-square filters, one-pixel images, shapes with no output
 * -- with buffers of exactly the sizes the shapes need, so any access
 * outside them, and any signed overflow or invalid shift, stops the run. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int dwref_out_dim(int in, int f, int s, int d, int p);
int dwref_fwd_f64(const double *x, const double *w, const double *bias, double *y,
                  double *scale, int N, int H, int W, int C, int FH, int FW, int S, int D,
                  int P, int n0, int n1);
int dwref_fwd_i8(const int8_t *x, const int8_t *w, const int32_t *bias, int64_t *y, int N,
                 int H, int W, int C, int FH, int FW, int S, int D, int P, int n0, int n1);
int dwref_points_f64(const double *x, const double *w, const double *bias, const int64_t *idx,
                     int64_t npts, double *y, double *scale, int N, int H, int W, int C,
                     int FH, int FW, int S, int D, int P);
int dwref_points_i8(const int8_t *x, const int8_t *w, const int32_t *bias, const int64_t *idx,
                    int64_t npts, int64_t *y, int N, int H, int W, int C, int FH, int FW,
                    int S, int D, int P);
int dwref_bwd_data_f64(const double *dy, const double *w, double *dx, double *scale, int N,
                       int H, int W, int C, int FH, int FW, int S, int D, int P, int n0,
                       int n1);
int dwref_bwd_filter_f64(const double *x, const double *dy, double *dw, double *scale, int N,
                         int H, int W, int C, int FH, int FW, int S, int D, int P, int c0,
                         int c1);
int dwref_fwd_bnact_f64(const double *x, const double *w, const double *bias,
                        const double *bn_scale, const double *bn_shift, int act, int fmt,
                        double *y, double *scale, int N, int H, int W, int C, int FH, int FW,
                        int S, int D, int P, int n0, int n1);

static uint64_t rng = 88172645463325252ull;
static int rnd(int lo, int hi) { /* [lo, hi] */
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return lo + (int)(rng % (uint64_t)(hi - lo + 1));
}
static double *dbuf(size_t n) {
    double *p = malloc((n ? n : 1) * sizeof(double));
    for (size_t i = 0; i < n; ++i) p[i] = rnd(-100, 100) / 16.0;
    return p;
}
static int8_t *ibuf(size_t n) {
    int8_t *p = malloc(n ? n : 1);
    for (size_t i = 0; i < n; ++i) p[i] = (int8_t)rnd(-128, 127);
    return p;
}

int main(int argc, char **argv) {
    int cases = argc > 1 ? atoi(argv[1]) : 300, ran = 0;
    for (int t = 0; t < cases; ++t) {
        int N = rnd(1, 3), H = rnd(1, 9), W = rnd(1, 9), C = rnd(1, 5);
        int FH = rnd(1, 5), FW = rnd(1, 5), S = rnd(1, 3), D = rnd(1, 3);
        int P = rnd(0, (FH > FW ? FH : FW) * D);
        int OH = dwref_out_dim(H, FH, S, D, P), OW = dwref_out_dim(W, FW, S, D, P);
        size_t nx = (size_t)N * H * W * C, nw = (size_t)FH * FW * C;
        if (OH < 1 || OW < 1) {
            /* no output: every entry point refuses the shape */
            double *x = dbuf(nx), *w = dbuf(nw);
            if (dwref_fwd_f64(x, w, NULL, NULL, NULL, N, H, W, C, FH, FW, S, D, P, 0, N) != -1)
                return 2;
            free(x);
            free(w);
            continue;
        }
        size_t ny = (size_t)N * OH * OW * C;
        double *x = dbuf(nx), *w = dbuf(nw), *b = dbuf(C), *y = dbuf(ny), *sc = dbuf(ny);
        double *dx = dbuf(nx), *dxs = dbuf(nx), *dwv = dbuf(nw), *dws = dbuf(nw);
        double *bs = dbuf(C), *bb = dbuf(C);
        int8_t *xi = ibuf(nx), *wi = ibuf(nw);
        int32_t *bi = malloc(C * sizeof(int32_t));
        int64_t *yi = malloc(ny * sizeof(int64_t));
        for (int c = 0; c < C; ++c) bi[c] = rnd(-32768, 32768);
        int64_t idx[8];
        double yp[8], sp[8];
        int64_t yip[8];
        for (int k = 0; k < 8; ++k) idx[k] = rnd(0, (int)ny - 1);
        int bad = 0;
        bad |= dwref_fwd_f64(x, w, t & 1 ? b : NULL, y, sc, N, H, W, C, FH, FW, S, D, P, 0, N);
        bad |= dwref_fwd_i8(xi, wi, t & 1 ? bi : NULL, yi, N, H, W, C, FH, FW, S, D, P, 0, N);
        bad |= dwref_points_f64(x, w, b, idx, 8, yp, sp, N, H, W, C, FH, FW, S, D, P);
        bad |= dwref_points_i8(xi, wi, bi, idx, 8, yip, N, H, W, C, FH, FW, S, D, P);
        bad |= dwref_bwd_data_f64(y, w, dx, dxs, N, H, W, C, FH, FW, S, D, P, 0, N);
        bad |= dwref_bwd_filter_f64(x, y, dwv, dws, N, H, W, C, FH, FW, S, D, P, 0, C);
        bad |= dwref_fwd_bnact_f64(x, w, b, bs, bb, t % 3, (t / 3) % 3, y, sc, N, H, W, C, FH,
                                   FW, S, D, P, 0, N);
        if (bad) return 3;
        /* the points agree with the full passes */
        dwref_fwd_f64(x, w, b, y, sc, N, H, W, C, FH, FW, S, D, P, 0, N);
        dwref_fwd_i8(xi, wi, bi, yi, N, H, W, C, FH, FW, S, D, P, 0, N);
        for (int k = 0; k < 8; ++k)
            if (yp[k] != y[idx[k]] || sp[k] != sc[idx[k]] || yip[k] != yi[idx[k]]) return 4;
        free(x); free(w); free(b); free(y); free(sc); free(dx); free(dxs); free(dwv);
        free(dws); free(bs); free(bb); free(xi); free(wi); free(bi); free(yi);
        ++ran;
    }
    printf("oracle sanitizer driver: %d shapes with output, %d cases\n", ran, cases);
    return 0;
}
