// copy_ceiling.hip -- a plain HBM copy for the bench's ceiling measurement
// (not part of the convolution library or its C ABI).
//
// k_copy_nt reads n16 16-byte vectors from src and writes them to dst: a grid-stride
// loop in which each workgroup copies a contiguous chunk of 4 x 256 vectors
// (16 KiB) per iteration, every lane keeping its four 16-byte loads in
// flight, and writes with non-temporal stores (the written data is never
// read back here).  Of the copy shapes measured on MI355X (one vector per
// lane and one workgroup per 256 vectors; four or eight loads per lane
// without a loop; loops of 1024 to 4096 workgroups) this one, with 2048
// workgroups, was the fastest, so it is the practical read + write ceiling
// the bench reports beside each kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) k_copy_nt(const u32x4 *__restrict__ src,
                                                 u32x4 *__restrict__ dst, size_t n16) {
    constexpr int U = 4, NT = 256;
    const size_t chunk = (size_t)NT * U;
    for (size_t base = (size_t)blockIdx.x * chunk + threadIdx.x; base < n16;
         base += (size_t)gridDim.x * chunk) {
        u32x4 v[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const size_t i = base + (size_t)k * NT;
            if (i < n16) v[k] = src[i];
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const size_t i = base + (size_t)k * NT;
            if (i < n16) __builtin_nontemporal_store(v[k], dst + i);
        }
    }
}

// Enqueues the copy of `bytes` (a multiple of 16; src and dst 16-byte
// aligned, not overlapping) on `stream`.  Returns 0, 1 for a bad argument, or
// 2 if the launch fails.
extern "C" int dwcopy_nt(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    if (!src || !dst || (bytes & 15u) || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u))
        return 1;
    const size_t n16 = bytes / 16;
    if (n16 == 0) return 0;
    hipLaunchKernelGGL(k_copy_nt, dim3(2048), dim3(256), 0, stream,
                       (const u32x4 *)src, (u32x4 *)dst, n16);
    return hipGetLastError() == hipSuccess ? 0 : 2;
}
