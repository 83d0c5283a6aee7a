// api.cpp -- the extern "C" entry points declared in include/dwconv.h.
#include <mutex>
#include <new>
#include <stdint.h>

#include "../../include/dwconv.h"
#include "plan.h"

struct dwconv_plan {
    dw::Plan p;      // forward
    dw::Plan bnp;    // forward with the fused prologue, when has_bn
    bool has_bn;
    dw::Plan bwd;    // backward data, when has_bwd
    bool has_bwd;
    dw::BwfPlan bwf; // backward filter, when has_bwf
    bool has_bwf;
};

// Backward data at stride 1 is a forward pass over dY (N x OH x OW x C) with
// the filter rotated by 180 degrees and padding D(F-1) - P, whose output is
// exactly H x W ("Flash-DWC: Making Depthwise Convolution Compute-Efficient
// on GPUs", section 5.1): every forward kernel family serves it.  One padding
// serves both axes only for square filters; every other float shape (stride
// above 1, non-square filters, padding beyond D(F-1)) runs the direct
// backward kernel, which sums each input element's taps.
static bool plan_bwd_data(dw::Plan &b, const dw::Plan &f, int variant) {
    const dw::Shape &s = f.s;
    if (f.dtype == dw::DT_I8) return false;
    const int P2 = s.D * (s.FH - 1) - s.P;
    if (s.S == 1 && s.FH == s.FW && P2 >= 0) {
        int rc = dw::make_plan(b, s.N, s.OH, s.OW, s.C, s.FH, s.FW, 1, s.D, P2, f.dtype,
                               variant);
        if (rc != DWCONV_OK && variant != dw::V_AUTO)
            rc = dw::make_plan(b, s.N, s.OH, s.OW, s.C, s.FH, s.FW, 1, s.D, P2, f.dtype,
                               dw::V_AUTO);
        if (rc == DWCONV_OK && b.s.OH == s.H && b.s.OW == s.W) {
            b.s.flip = 1;
            return true;
        }
    }
    return dw::plan_bwd_direct(b, f);
}

// The filter gradient's workspace for callers that cannot allocate
// (dwconv_bwd_filter_noalloc): one array per GPU, in the library's code
// object, alive until the process ends.  Host code never passes the array's
// name to a kernel (on the host it is a stand-in, not a device address); it
// asks the runtime for this device's copy once, with the device current,
// and keeps the address per device.
static __device__ __align__(256) unsigned char scratch[DWCONV_SCRATCH_BYTES];

static hipError_t scratch_address(void **out) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return hipSuccess;
}

static bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

extern "C" {

dwconv_status_t dwconv_create_variant(dwconv_handle_t *out, int N, int H, int W, int C,
                                      int FH, int FW, int stride, int dilation, int pad,
                                      dwconv_dtype_t dtype, dwconv_variant_t variant) {
    if (!out) return DWCONV_ERR_INVALID_ARG;
    *out = nullptr;
    dwconv_plan *h = new (std::nothrow) dwconv_plan;
    if (!h) return DWCONV_ERR_ALLOC;
    int rc = dw::make_plan(h->p, N, H, W, C, FH, FW, stride, dilation, pad, (int)dtype,
                           (int)variant);
    if (rc != DWCONV_OK) {
        delete h;
        return (dwconv_status_t)rc;
    }
    h->has_bn = dw::plan_bn_act(h->bnp, h->p);
    h->has_bwd = plan_bwd_data(h->bwd, h->p, (int)variant);
    h->has_bwf = dw::plan_bwd_filter(h->bwf, h->p);
    *out = h;
    return DWCONV_OK;
}

dwconv_status_t dwconv_create(dwconv_handle_t *out, int N, int H, int W, int C, int FH,
                              int FW, int stride, int dilation, int pad,
                              dwconv_dtype_t dtype) {
    return dwconv_create_variant(out, N, H, W, C, FH, FW, stride, dilation, pad, dtype,
                                 DWCONV_VARIANT_AUTO);
}

dwconv_status_t dwconv_fwd(dwconv_handle_t h, const void *x, const void *w,
                           const void *bias, void *y, hipStream_t stream) {
    if (!h || !x || !w || !y) return DWCONV_ERR_INVALID_ARG;
    const dw::Plan &p = h->p;
    // The vectorised families need 16-byte aligned tensors; anything else
    // runs on the direct family, which takes any alignment.
    bool ok_align = aligned16(x) && aligned16(w) && aligned16(y) &&
                    (bias == nullptr || aligned16(bias));
    dw::LaunchFn fn = ok_align ? p.launch : p.fallback;
    hipError_t e = fn(p, x, w, bias, y, stream);
    return e == hipSuccess ? DWCONV_OK : DWCONV_ERR_HIP;
}

dwconv_status_t dwconv_fwd_bn_act(dwconv_handle_t h, const void *x, const void *w,
                                  const void *bias, const float *bn_scale,
                                  const float *bn_shift, dwconv_act_t act, void *y,
                                  hipStream_t stream) {
    if (!h || !x || !w || !y || !bn_scale || !bn_shift) return DWCONV_ERR_INVALID_ARG;
    if ((int)act < DWCONV_ACT_NONE || (int)act > DWCONV_ACT_RELU6) return DWCONV_ERR_INVALID_ARG;
    if (!h->has_bn) return DWCONV_ERR_UNSUPPORTED;
    const dw::Plan &p = h->bnp;
    bool ok_align = aligned16(x) && aligned16(w) && aligned16(y) &&
                    (bias == nullptr || aligned16(bias));
    dw::LaunchBnFn fn = ok_align ? p.bn_launch : p.bn_fallback;
    hipError_t e = fn(p, x, w, bias, bn_scale, bn_shift, (int)act, y, stream);
    return e == hipSuccess ? DWCONV_OK : DWCONV_ERR_HIP;
}

int dwconv_fwd_bn_act_supported(dwconv_handle_t h) { return h && h->has_bn ? 1 : 0; }

const char *dwconv_fwd_bn_act_describe(dwconv_handle_t h) {
    return h && h->has_bn ? h->bnp.desc : "";
}

dwconv_status_t dwconv_bwd_data(dwconv_handle_t h, const void *dy, const void *w, void *dx,
                                hipStream_t stream) {
    if (!h || !dy || !w || !dx) return DWCONV_ERR_INVALID_ARG;
    if (!h->has_bwd) return DWCONV_ERR_UNSUPPORTED;
    const dw::Plan &b = h->bwd;
    bool ok_align = aligned16(dy) && aligned16(w) && aligned16(dx);
    dw::LaunchFn fn = ok_align ? b.launch : b.fallback;
    hipError_t e = fn(b, dy, w, nullptr, dx, stream);
    return e == hipSuccess ? DWCONV_OK : DWCONV_ERR_HIP;
}

int dwconv_bwd_data_supported(dwconv_handle_t h) { return h && h->has_bwd ? 1 : 0; }

const char *dwconv_bwd_data_describe(dwconv_handle_t h) {
    return h && h->has_bwd ? h->bwd.desc : "";
}

dwconv_status_t dwconv_bwd_filter_workspace(dwconv_handle_t h, size_t *bytes) {
    if (!h || !bytes) return DWCONV_ERR_INVALID_ARG;
    if (!h->has_bwf) return DWCONV_ERR_UNSUPPORTED;
    *bytes = h->bwf.ws_bytes;
    return DWCONV_OK;
}

// Pass 1 (into the workspace) and pass 2 (the merge into dw) of the filter
// gradient.  The 16-byte channel vectors need aligned x and dy (the
// matrix-core pass also a 16-byte aligned workspace).
static dwconv_status_t run_bwd_filter(const dw::BwfPlan &b, const void *x, const void *dy,
                                      float *dw, void *workspace, hipStream_t stream) {
    dw::BwfLaunchFn fn = b.one_launch;
    if (aligned16(x) && aligned16(dy))
        fn = b.mfma_launch && aligned16(workspace) ? b.mfma_launch : b.vec_launch;
    hipError_t e = fn(b, x, dy, dw, workspace, stream);
    return e == hipSuccess ? DWCONV_OK : DWCONV_ERR_HIP;
}

dwconv_status_t dwconv_bwd_filter(dwconv_handle_t h, const void *x, const void *dy,
                                  float *dw, void *workspace, hipStream_t stream) {
    if (!h || !x || !dy || !dw || !workspace) return DWCONV_ERR_INVALID_ARG;
    if (!h->has_bwf) return DWCONV_ERR_UNSUPPORTED;
    // the workspace and dw are written as floats
    if (((uintptr_t)workspace & 3u) != 0 || ((uintptr_t)dw & 3u) != 0)
        return DWCONV_ERR_INVALID_ARG;
    return run_bwd_filter(h->bwf, x, dy, dw, workspace, stream);
}

dwconv_status_t dwconv_bwd_filter_noalloc(dwconv_handle_t h, const void *x, const void *dy,
                                          float *dw, hipStream_t stream) {
    if (!h || !x || !dy || !dw) return DWCONV_ERR_INVALID_ARG;
    if (!h->has_bwf) return DWCONV_ERR_UNSUPPORTED;
    if (((uintptr_t)dw & 3u) != 0) return DWCONV_ERR_INVALID_ARG;
    if (h->bwf.ws_bytes > (size_t)DWCONV_SCRATCH_BYTES) return DWCONV_ERR_SCRATCH;
    void *ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return DWCONV_ERR_HIP;
    return run_bwd_filter(h->bwf, x, dy, dw, ws, stream);
}

const char *dwconv_bwd_filter_describe(dwconv_handle_t h) {
    return h && h->has_bwf ? h->bwf.desc : "";
}

dwconv_status_t dwconv_destroy(dwconv_handle_t h) {
    delete h;
    return DWCONV_OK;
}

dwconv_status_t dwconv_output_dims(dwconv_handle_t h, int *OH, int *OW) {
    if (!h || !OH || !OW) return DWCONV_ERR_INVALID_ARG;
    *OH = h->p.s.OH;
    *OW = h->p.s.OW;
    return DWCONV_OK;
}

dwconv_variant_t dwconv_plan_variant(dwconv_handle_t h) {
    return h ? (dwconv_variant_t)h->p.variant : DWCONV_VARIANT_AUTO;
}

const char *dwconv_plan_describe(dwconv_handle_t h) { return h ? h->p.desc : ""; }

dwconv_status_t dwconv_plan_tile(dwconv_handle_t h, int *tile_h, int *tile_w, int *tile_c) {
    if (!h || !tile_h || !tile_w || !tile_c) return DWCONV_ERR_INVALID_ARG;
    *tile_h = h->p.tile_h;
    *tile_w = h->p.tile_w;
    *tile_c = h->p.tile_c;
    return DWCONV_OK;
}

const char *dwconv_status_string(dwconv_status_t s) {
    switch (s) {
        case DWCONV_OK: return "ok";
        case DWCONV_ERR_INVALID_ARG: return "invalid argument";
        case DWCONV_ERR_UNSUPPORTED: return "unsupported";
        case DWCONV_ERR_HIP: return "HIP runtime error";
        case DWCONV_ERR_ALLOC: return "out of host memory";
        case DWCONV_ERR_SCRATCH: return "workspace larger than the library's scratch array";
    }
    return "unknown status";
}

}  // extern "C"
