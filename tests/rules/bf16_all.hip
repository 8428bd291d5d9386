// Exhaustive device check of the library's fp32 -> bf16 conversion
// (pack_bf16x2, one v_cvt_pk_bf16_f32 per pair) -- TEST INFRASTRUCTURE.
//
// Every one of the 2^32 fp32 bit patterns is converted on the GPU and compared
// with the rule the library documents: round to nearest, ties to even, for
// every non-NaN input (denormals, infinities and the rounding into infinity
// included), and for a NaN the quiet NaN with the input's sign and top 7
// payload bits.  The rule is written out here in integer arithmetic; nothing
// in this file reads or writes memory other than its two result words.
//
// Built by the package's build step into tests/rules/libbf16_all.so; the GPU
// test calls bf16_check_all() through ctypes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "apexw_kernels.hpp"

namespace {

__device__ __forceinline__ uint32_t rule(uint32_t u) {
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;     // NaN: quiet
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;                     // nearest, ties to even
}

// Each thread takes the inputs i, i + stride, ... below 2^32 (a bounded
// loop), two per conversion; mismatches are counted per thread and added
// once, and the smallest mismatching input is kept.
__global__ __launch_bounds__(256) void bf16_all_kernel(unsigned long long *count,
                                                       unsigned long long *first,
                                                       unsigned long long *seen) {
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x * 2u;
    unsigned long long bad = 0, lowest = ~0ull, done = 0;
    for (uint64_t i = ((uint64_t)blockIdx.x * blockDim.x + threadIdx.x) * 2u; i < (1ull << 32);
         i += stride) {
        const uint32_t a = (uint32_t)i, b = (uint32_t)(i + 1u);
        const uint32_t w = apexw::pack_bf16x2(__uint_as_float(a), __uint_as_float(b));
        if ((w & 0xffffu) != rule(a)) { ++bad; lowest = lowest < a ? lowest : a; }
        if ((w >> 16) != rule(b)) { ++bad; lowest = lowest < b ? lowest : b; }
        done += 2;
    }
    atomicAdd(seen, done);
    if (bad) {
        atomicAdd(count, bad);
        atomicMin(first, lowest);
    }
}

}  // namespace

// Runs the check on the current device; returns 0 and the number of
// mismatching inputs (and the smallest one, or 2^64-1) in *out_count /
// *out_first and the number of inputs compared in *out_seen, or a nonzero HIP
// error code.
extern "C" int bf16_check_all(unsigned long long *out_count, unsigned long long *out_first,
                              unsigned long long *out_seen) {
    unsigned long long *d = nullptr;
    hipError_t e = hipMalloc((void **)&d, 3 * sizeof(unsigned long long));
    if (e != hipSuccess) return (int)e;
    const unsigned long long init[3] = {0ull, ~0ull, 0ull};
    e = hipMemcpy(d, init, sizeof init, hipMemcpyHostToDevice);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(bf16_all_kernel, dim3(65536), dim3(256), 0, 0, d, d + 1, d + 2);
        e = hipGetLastError();
    }
    unsigned long long res[3] = {0ull, 0ull, 0ull};
    if (e == hipSuccess) e = hipMemcpy(res, d, sizeof res, hipMemcpyDeviceToHost);
    (void)hipFree(d);
    if (e != hipSuccess) return (int)e;
    *out_count = res[0];
    *out_first = res[1];
    *out_seen = res[2];
    return 0;
}
