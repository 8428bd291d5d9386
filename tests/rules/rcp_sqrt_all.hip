// Device checks of the update's square root, reciprocal and short division
// (sqrt_rn, rcp_rn, div_short in the kernel header) -- TEST INFRASTRUCTURE.
//
//  1. sqrt_rn(x) for every fp32 x in [2^-96, 2^64), against the nearest
//     square root: s is the nearest iff (s - u-/2)^2 < x < (s + u+/2)^2, with
//     u- and u+ the gaps to s's neighbours (no x lies on a midpoint's square).
//  2. rcp_rn(b) for every fp32 b in [2^-126, 2^126], against the nearest
//     reciprocal: y is the nearest iff (y - u-/2)*b < 1 < (y + u+/2)*b.
//     Both tests are exact in fp64: the midpoints have 25 significant bits,
//     their squares and their products with b at most 50.
//     The same loop checks that v_rcp_f32 alone is within one ulp of 1/b
//     (y - u- < 1/b < y + u+), which the 8-bit encoding's tie guard assumes.
//  3. div_short(x, b, rcp_rn(b)) against IEEE division x / b on 2^32 pairs
//     drawn by a counter-based hash: |x| in [2^-96, 2^64) with either sign, b
//     in [2^-48, 2^29], uniform in exponent and significand -- the operand
//     ranges the update admits to the short form.
//
// Built by the package's build step into tests/rules/librcp_sqrt_all.so; the
// GPU test calls rcp_sqrt_check_all() through ctypes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "apexw_kernels.hpp"

namespace {

enum { kSqrtBad, kSqrtSeen, kRcpBad, kRcpSeen, kDivBad, kDivSeen, kRawBad, kSqrtFirst, kRcpFirst,
       kDivFirst, kRawFirst, kWords };

__device__ __forceinline__ double gap_above(float s) {
    return (double)__uint_as_float(__float_as_uint(s) + 1u) - (double)s;
}
__device__ __forceinline__ double gap_below(float s) {
    return (double)s - (double)__uint_as_float(__float_as_uint(s) - 1u);
}

__device__ __forceinline__ bool is_nearest_sqrt(float x, float s) {
    if (!(s > 0.0f) || !(s < 0x1p127f)) return false;
    const double lo = (double)s - 0.5 * gap_below(s), hi = (double)s + 0.5 * gap_above(s);
    return lo * lo < (double)x && (double)x < hi * hi;
}

__device__ __forceinline__ bool within_one_ulp_rcp(float b, float y) {
    if (!(y > 0.0f) || !(y < 0x1p127f)) return false;
    const double lo = (double)y - gap_below(y), hi = (double)y + gap_above(y);
    return lo * (double)b < 1.0 && 1.0 < hi * (double)b;
}

__device__ __forceinline__ bool is_nearest_rcp(float b, float y) {
    if (!(y > 0.0f) || !(y < 0x1p127f)) return false;
    const double lo = (double)y - 0.5 * gap_below(y), hi = (double)y + 0.5 * gap_above(y);
    return lo * (double)b < 1.0 && 1.0 < hi * (double)b;
}

// SplitMix64's output function: a bijective 64-bit mixer
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z += 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

// fp32 with a random significand and an exponent uniform in [e_lo, e_hi)
__device__ __forceinline__ float draw(uint64_t h, int e_lo, int e_hi) {
    const uint32_t e = (uint32_t)(e_lo + (int)((h >> 23) % (uint64_t)(e_hi - e_lo)));
    return __uint_as_float(((e + 127u) << 23) | (uint32_t)(h & 0x7fffffu));
}

__global__ __launch_bounds__(256) void rcp_sqrt_all_kernel(unsigned long long *out) {
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    unsigned long long c[7] = {0, 0, 0, 0, 0, 0, 0};
    unsigned long long f[4] = {~0ull, ~0ull, ~0ull, ~0ull};
    // 1. square root: bit patterns of [2^-96, 2^64)
    for (uint64_t u = 0x0f800000u + tid; u < 0x5f800000u; u += stride) {
        const float x = __uint_as_float((uint32_t)u);
        ++c[kSqrtSeen];
        if (!is_nearest_sqrt(x, apexw::sqrt_rn(x))) {
            ++c[kSqrtBad];
            f[0] = f[0] < u ? f[0] : u;
        }
    }
    // 2. reciprocal: bit patterns of [2^-126, 2^126]
    for (uint64_t u = 0x00800000u + tid; u <= 0x7e800000u; u += stride) {
        const float b = __uint_as_float((uint32_t)u);
        ++c[kRcpSeen];
        if (!is_nearest_rcp(b, apexw::rcp_rn(b))) {
            ++c[kRcpBad];
            f[1] = f[1] < u ? f[1] : u;
        }
        if (!within_one_ulp_rcp(b, __builtin_amdgcn_rcpf(b))) {
            ++c[kRawBad];
            f[3] = f[3] < u ? f[3] : u;
        }
    }
    // 3. short division on hashed pairs
    for (uint64_t i = tid; i < (1ull << 32); i += stride) {
        const uint64_t h1 = mix64(2 * i), h2 = mix64(2 * i + 1);
        float x = draw(h1, -96, 64);
        if (h1 >> 63) x = -x;
        const float b = draw(h2, -48, 29);
        ++c[kDivSeen];
        if (__float_as_uint(apexw::div_short(x, b, apexw::rcp_rn(b))) != __float_as_uint(x / b)) {
            ++c[kDivBad];
            f[2] = f[2] < i ? f[2] : i;
        }
    }
    for (int j = 0; j < 7; ++j)
        if (c[j]) atomicAdd(&out[j], c[j]);
    for (int j = 0; j < 4; ++j)
        if (f[j] != ~0ull) atomicMin(&out[kSqrtFirst + j], f[j]);
}

}  // namespace

// Runs the checks on the current device.  out[0..6]: square-root mismatches
// and inputs checked, reciprocal mismatches and inputs checked, division
// mismatches and pairs checked, raw reciprocals off by an ulp or more;
// out[7..10]: the first failing input (bit pattern, or pair index) of each
// check, 2^64-1 if none.  Returns 0 or a nonzero HIP error code.
extern "C" int rcp_sqrt_check_all(unsigned long long *out) {
    unsigned long long *d = nullptr;
    hipError_t e = hipMalloc((void **)&d, kWords * sizeof(unsigned long long));
    if (e != hipSuccess) return (int)e;
    unsigned long long init[kWords] = {0, 0, 0, 0, 0, 0, 0, ~0ull, ~0ull, ~0ull, ~0ull};
    e = hipMemcpy(d, init, sizeof init, hipMemcpyHostToDevice);
    if (e == hipSuccess) {
        hipLaunchKernelGGL(rcp_sqrt_all_kernel, dim3(65536), dim3(256), 0, 0, d);
        e = hipGetLastError();
    }
    unsigned long long res[kWords] = {};
    if (e == hipSuccess) e = hipMemcpy(res, d, sizeof res, hipMemcpyDeviceToHost);
    (void)hipFree(d);
    if (e != hipSuccess) return (int)e;
    for (int j = 0; j < kWords; ++j) out[j] = res[j];
    return 0;
}
