// dw_common.h -- shapes, element-type traits and small device helpers shared
// by the gfx950 depthwise-convolution kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dw {

// Operation shape.  Names follow "Flash-DWC: Making Depthwise Convolution
// Compute-Efficient on GPUs", section 2.1 (N, H = IH, W = IW, C = IC = OC,
// FH, FW, OH, OW) plus stride S, dilation D and padding P.
struct Shape {
    int N, H, W, C;
    int FH, FW;
    int S, D, P;
    int OH, OW;
    int flip;  // 1: the filter is read rotated by 180 degrees (backward data)
};

// Offset (in taps) of filter tap (fh, fw) in the FH x FW x C filter.  The
// backward-data pass is the forward pass with the filter rotated by 180
// degrees ("Flash-DWC: Making Depthwise Convolution Compute-Efficient on
// GPUs", section 5.1), read here in place instead of from a rotated copy.
__host__ __device__ __forceinline__ int tap_index(const Shape &s, int fh, int fw) {
    return s.flip ? (s.FH - 1 - fh) * s.FW + (s.FW - 1 - fw) : fh * s.FW + fw;
}

// ---------------------------------------------------------------------------
// Element-type traits.  X: stored input/filter element; Acc: accumulator;
// Bias: bias element (always the accumulator type); Y: stored output.
// ---------------------------------------------------------------------------
struct F32 {
    using X = float;
    using Acc = float;
    using Bias = float;
    using Y = float;
    static __device__ __forceinline__ float widen(float v) { return v; }
    static __device__ __forceinline__ float narrow(float a) { return a; }
};

struct F16 {
    using X = _Float16;
    using Acc = float;
    using Bias = float;
    using Y = _Float16;
    static __device__ __forceinline__ float widen(_Float16 v) { return (float)v; }
    // v_cvt_f16_f32 rounds to nearest even in the default rounding mode
    static __device__ __forceinline__ _Float16 narrow(float a) { return (_Float16)a; }
};

struct BF16 {
    using X = uint16_t;  // bfloat16 bit pattern
    using Acc = float;
    using Bias = float;
    using Y = uint16_t;
    static __device__ __forceinline__ float widen(uint16_t v) {
        return __uint_as_float((uint32_t)v << 16);
    }
    // fp32 -> bf16, round to nearest even on the dropped 16 bits; NaN stays NaN
    static __device__ __forceinline__ uint16_t narrow(float a) {
        uint32_t u = __float_as_uint(a);
        if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
        u += 0x7fffu + ((u >> 16) & 1u);
        return (uint16_t)(u >> 16);
    }
};

struct I8 {
    using X = int8_t;
    using Acc = int32_t;
    using Bias = int32_t;
    using Y = int32_t;
    static __device__ __forceinline__ int32_t widen(int8_t v) { return (int32_t)v; }
    static __device__ __forceinline__ int32_t narrow(int32_t a) { return a; }
};

template <class A>
__device__ __forceinline__ A mac(A acc, A a, A b);
template <>
__device__ __forceinline__ float mac<float>(float acc, float a, float b) {
    return __builtin_fmaf(a, b, acc);
}
// int8 operands widened to int32 fit 24 bits: a 24-bit multiply-add is
// exact and runs at full rate (a 32-bit multiply is quarter rate)
template <>
__device__ __forceinline__ int32_t mac<int32_t>(int32_t acc, int32_t a, int32_t b) {
    return acc + __mul24(a, b);
}

// The fused prologue of the forward pass ("Flash-DWC: Making Depthwise
// Convolution Compute-Efficient on GPUs", section 5.2: BN and the activation
// applied to the input inside the convolution kernel): the input value x,
// widened to fp32, becomes act(x * s + b) with one fused multiply-add; act
// 0 = identity, 1 = ReLU, 2 = ReLU6.  Padding positions are zeros of the
// result, so callers apply it to in-image values only.
__device__ __forceinline__ float bn_act(float x, float s, float b, int act) {
    float u = __builtin_fmaf(x, s, b);
    u = act >= 1 ? __builtin_fmaxf(u, 0.0f) : u;
    return act == 2 ? __builtin_fminf(u, 6.0f) : u;
}

// ... stored in the data's format before the convolution multiplies it:
// fp16 / bf16 round to nearest even (section 4.1 of the same page: mixed
// precision keeps tensors in FP16 and multiplies FP16 operands), as a
// separate BN + Act pass would store it; fp32 is unchanged.
template <class DT>
__device__ __forceinline__ float bn_act_stored(float x, float s, float b, int act) {
    return DT::widen(DT::narrow(bn_act(x, s, b, act)));
}

// Greatest common divisor (compile-time or host use).
__host__ __device__ constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// Workgroups are handed to the 8 XCDs of the chip round-robin, and each XCD
// has its own L2.  Renumber them so that a contiguous range of logical tiles
// (which share halo rows) lands on one XCD.  A bijection on [0, nb).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t b, uint32_t nb) {
    constexpr uint32_t NX = 8;
    uint32_t q = nb / NX, rem = nb % NX;
    uint32_t xcd = b % NX, k = b / NX;
    return xcd < rem ? xcd * (q + 1) + k : rem * (q + 1) + (xcd - rem) * q + k;
}

// xcd_remap, and then, inside each XCD's range, the workgroups that one pass
// of the XCD's dispatcher over its 32 CUs places on the same CU (positions
// k, k + 32, ..., k + 32 (slots - 1) of a pass of 32 slots when the CUs are
// filled breadth first) take consecutive logical tiles.  Positions past the
// last whole pass keep their order.  A bijection on [0, nb) for any slots.
__device__ __forceinline__ uint32_t xcd_remap_slots(uint32_t b, uint32_t nb, int slots) {
    constexpr uint32_t NX = 8, NCU = 32;
    const uint32_t q = nb / NX, rem = nb % NX;
    const uint32_t xcd = b % NX;
    uint32_t k = b / NX;
    const uint32_t cnt = q + (xcd < rem ? 1u : 0u);
    const uint32_t lo = xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q;
    if (slots > 1) {
        const uint32_t P = NCU * (uint32_t)slots;
        if (k < cnt / P * P) {
            const uint32_t i = k % P;
            k = k - i + (i % NCU) * (uint32_t)slots + i / NCU;
        }
    }
    return lo + k;
}

}  // namespace dw
