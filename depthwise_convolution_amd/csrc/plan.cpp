// plan.cpp -- validation, output extent and kernel-family choice.  Host only;
// makes no HIP calls.
#include "plan.h"

#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/dwconv.h"

namespace dw {

// The input span of an output extent O is (O-1)S + (F-1)D + 1 ("Tiles, halos
// and partial sums", section "Partition tensors to fit storage"); the output
// extent is the largest O whose span fits the zero-padded input in + 2p.
int out_extent(int in, int f, int s, int d, int p) {
    if (in < 1 || f < 1 || s < 1 || d < 1 || p < 0) return 0;
    long long room = (long long)in + 2LL * p - (long long)(f - 1) * d - 1;
    if (room < 0) return 0;
    long long o = room / s + 1;
    return o > 0x7fffffffLL ? 0 : (int)o;
}

const char *tune(const char *key, char *buf, int len) {
    const char *env = getenv("DWCONV_TUNE");
    if (!env || !key || len < 1) return nullptr;
    const size_t kl = strlen(key);
    for (const char *p = env; *p;) {
        const char *end = strchr(p, ',');
        if (!end) end = p + strlen(p);
        if ((size_t)(end - p) > kl && strncmp(p, key, kl) == 0 && p[kl] == '=') {
            const int vl = (int)(end - p - kl - 1) < len - 1 ? (int)(end - p - kl - 1) : len - 1;
            memcpy(buf, p + kl + 1, vl);
            buf[vl] = 0;
            return buf;
        }
        p = *end ? end + 1 : end;
    }
    return nullptr;
}

int tune_int(const char *key, int dflt) {
    char buf[32];
    const char *v = tune(key, buf, sizeof(buf));
    return v ? atoi(v) : dflt;
}

static int elem_bytes_of(int dtype) {
    switch (dtype) {
        case DT_F32: return 4;
        case DT_F16: return 2;
        case DT_BF16: return 2;
        case DT_I8: return 1;
    }
    return 0;
}

// fp16 5x5 at stride 1: the column stream with paired taps (v_dot2_f32_f16)
// ran 8-95 % faster than the matrix cores on maps of 64K lanes and more, and
// slower on small ones, whose few wavefronts cannot hide its latency.
static bool dot2_column_stream(Plan &p) {
    if (p.dtype != DT_F16 || p.s.FH != 5 || p.s.FW != 5 || p.s.S != 1 || p.s.D != 1)
        return false;
    Plan q = p;
    if (!plan_rowwin(q) || q.th <= 0) return false;
    if ((long long)q.grid * q.block < 65536) return false;
    p = q;
    return true;
}

int make_plan(Plan &p, int N, int H, int W, int C, int FH, int FW, int S, int D,
              int P, int dtype, int variant) {
    memset(&p, 0, sizeof(p));
    if (N < 1 || H < 1 || W < 1 || C < 1 || FH < 1 || FW < 1 || S < 1 || D < 1 || P < 0)
        return DWCONV_ERR_INVALID_ARG;
    int eb = elem_bytes_of(dtype);
    if (eb == 0) return DWCONV_ERR_INVALID_ARG;
    if (variant < V_AUTO || variant > V_MFMA) return DWCONV_ERR_INVALID_ARG;
    int OH = out_extent(H, FH, S, D, P);
    int OW = out_extent(W, FW, S, D, P);
    if (OH < 1 || OW < 1) return DWCONV_ERR_INVALID_ARG;
    const long long lim = 1LL << 31;
    if ((long long)N * H * W * C >= lim || (long long)N * OH * OW * C >= lim ||
        (long long)FH * FW * C >= lim)
        return DWCONV_ERR_INVALID_ARG;
    if (dtype == DT_I8 && (long long)FH * FW > 131071) return DWCONV_ERR_INVALID_ARG;

    p.s = Shape{N, H, W, C, FH, FW, S, D, P, OH, OW};
    p.dtype = dtype;
    p.elem_bytes = eb;

    // The direct family runs every shape and alignment; it is also the
    // fallback for pointers that are not 16-byte aligned.
    Plan d = p;
    if (!plan_direct(d)) return DWCONV_ERR_UNSUPPORTED;

    bool ok = false;
    switch (variant) {
        case V_DIRECT: p = d; ok = true; break;
        case V_ROWWIN: ok = plan_rowwin(p); break;
        case V_LDSTILE: ok = plan_ldstile(p); break;
        case V_MFMA: ok = plan_mfma(p); break;
        case V_AUTO:
            // the banded GEMM wastes most of its K window on filters narrower
            // than 5 taps; there the vector families are preferred.  The
            // register families need whole 16-byte channel vectors; the LDS
            // tile takes any channel count.
            ok = dot2_column_stream(p) || (FW >= 5 && plan_mfma(p)) || plan_rowwin(p) ||
                 plan_ldstile(p);
            if (!ok) { p = d; ok = true; }
            break;
    }
    if (!ok) return DWCONV_ERR_UNSUPPORTED;
    p.fallback = d.launch;
    p.bn_fallback = d.bn_launch;
    return DWCONV_OK;
}

bool plan_bn_act(Plan &b, const Plan &f) {
    if (f.dtype == DT_I8) return false;
    if (f.bn_launch) {  // the forward plan's family fuses the prologue
        b = f;
        return true;
    }
    // the matrix-core family, where the forward pass runs there and the
    // prologue's extra rings fit LDS
    if (plan_mfma_bn(b, f)) return true;
    // else the row window / row chunks where they apply, else the direct
    // family (the LDS-tile family does not fuse the prologue)
    const Shape &s = f.s;
    for (int v : {V_ROWWIN, V_DIRECT}) {
        if (make_plan(b, s.N, s.H, s.W, s.C, s.FH, s.FW, s.S, s.D, s.P, f.dtype, v) ==
                DWCONV_OK &&
            b.bn_launch)
            return true;
    }
    return false;
}

}  // namespace dw
