// apexw_kernels.hpp -- gfx950 device code of the fused multi-tensor AdamW step.
//
// One persistent, grid-stride kernel per moment format walks a table of
// 4096-element tiles (a tile never spans two tensors).  A workgroup of 256
// lanes (four wave64s) owns a tile: lane l of wave w takes, in each of four
// slots s, the 4 contiguous elements starting at s*1024 + w*256 + l*4, so
// each load instruction of a wave covers one contiguous 256-element run
// (fp32: 1 KiB as dwordx4, bf16: 512 B as dwordx2, 8-bit codes: 256 B), and
// in the 8-bit format that run is exactly one 256-element quantisation block.
// Every element is read once and written once: theta, g, m, v in; theta, m, v
// out (M041 section 04 ledger: 28 B per fp32 element).  The path is
// HBM-bandwidth bound, so there is no matrix-core work; the arithmetic is
// ordinary fp32 VALU code compiled without contraction.
//
// Sources: "Fused optimizers and state precision" (ai-infra-kb M041),
// sections 02 (update), 03 (groups, missing grads), 04 (scalar bias
// correction, one pass), 05 (block quantiser), 06 (skipped steps); "Apex
// fused optimizers" guide (qwbw.cn), section 4.3 (found_inf decided on the
// device, step advanced only without overflow).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "apexw.h"

namespace apexw {

constexpr int kThreads = 256;                 // lanes per workgroup
constexpr int kVec = 4;                       // contiguous elements per lane per slot
constexpr int kSlots = 4;                     // slots per tile
constexpr int kSlotElems = kThreads * kVec;   // 1024
constexpr int kTile = kSlotElems * kSlots;    // 4096 elements per tile
constexpr int kWaveElems = 64 * kVec;         // 256: one q8 block per wave-slot
static_assert(kWaveElems == APEXW_Q8_BLOCK, "a wave-slot is one 8-bit block");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Per-group scalars, formed on the host once per call.
struct GroupScalars {
    float beta1, one_minus_beta1, beta2, one_minus_beta2;
    float lr, decay, eps, pad_;
    double beta1_d, beta2_d;                  // for beta^t in fp64
};

// Per-tensor descriptor (device table, rewritten only when params change).
struct TensorDesc {
    void *param;
    void *m;
    void *v;
    float *m_scale;
    float *v_scale;
    int64_t numel;
    int32_t group;
    int32_t pad_[3];
};
static_assert(sizeof(TensorDesc) == 64, "descriptor is one 64-byte record");

struct TileRef {
    int32_t tensor;      // index into the descriptor table
    int32_t index;       // tile number within the tensor
};

struct KernelArgs {
    const TensorDesc *desc;
    const void *const *grads;        // grads[i] == nullptr: no grad this call
    const TileRef *tiles;            // this launch's tiles
    const int32_t *tensors;          // this launch's tensors (step epilogue)
    int32_t *steps;                  // int32 step counter per tensor
    uint32_t *ticket;                // workgroups finished (reset by the last)
    const float *found_inf;          // nullptr: never skip
    int32_t n_tiles;
    int32_t n_tensors;
    GroupScalars groups[APEXW_MAX_GROUPS];
};

// Scalars of one tensor at its advanced step count.
struct StepScalars {
    float beta1, one_minus_beta1, beta2, one_minus_beta2;
    float lr, decay, eps;
    float bc1, bc2;                  // 1 - beta1^t, 1 - beta2^t (fp32)
};

// beta^n in fp64: square-and-multiply from the least significant bit.
__device__ __forceinline__ double pow_uint(double b, uint32_t n) {
    double r = 1.0;
    while (n != 0u) {
        if (n & 1u) r = r * b;
        b = b * b;
        n >>= 1;
    }
    return r;
}

__device__ __forceinline__ StepScalars step_scalars(const GroupScalars &g,
                                                    int32_t t) {
    StepScalars s;
    s.beta1 = g.beta1;
    s.one_minus_beta1 = g.one_minus_beta1;
    s.beta2 = g.beta2;
    s.one_minus_beta2 = g.one_minus_beta2;
    s.lr = g.lr;
    s.decay = g.decay;
    s.eps = g.eps;
    s.bc1 = (float)(1.0 - pow_uint(g.beta1_d, (uint32_t)t));
    s.bc2 = (float)(1.0 - pow_uint(g.beta2_d, (uint32_t)t));
    return s;
}

// The AdamW update of one element (M041 section 02), fp32, each operation
// rounded, evaluated left to right as printed.
__device__ __forceinline__ void adamw_update(float &theta, float g, float &m,
                                             float &v, const StepScalars &s) {
    m = s.beta1 * m + s.one_minus_beta1 * g;
    v = s.beta2 * v + (s.one_minus_beta2 * g) * g;
    const float m_hat = m / s.bc1;
    const float v_hat = v / s.bc2;
    const float denom = sqrtf(v_hat) + s.eps;
    theta = theta * s.decay - (s.lr * m_hat) / denom;
}

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Nearest bf16, ties to even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------- loads

// Element types: 0 = fp32, 1 = bf16 (APEXW_F32 / APEXW_BF16).
template <int DT> struct Elem;
template <> struct Elem<APEXW_F32> { typedef float storage; };
template <> struct Elem<APEXW_BF16> { typedef uint16_t storage; };

template <int DT, bool NT>
__device__ __forceinline__ void load4(const void *base, int64_t e, float (&x)[kVec]) {
    if constexpr (DT == APEXW_F32) {
        const f32x4 *p = reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + e);
        f32x4 w = NT ? __builtin_nontemporal_load(p) : *p;
        x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
    } else {
        const u32x2 *p = reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(base) + e);
        u32x2 w = NT ? __builtin_nontemporal_load(p) : *p;
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
        x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    }
}

template <int DT, bool NT>
__device__ __forceinline__ void store4(void *base, int64_t e, const float (&x)[kVec]) {
    if constexpr (DT == APEXW_F32) {
        f32x4 *p = reinterpret_cast<f32x4 *>(static_cast<float *>(base) + e);
        f32x4 w = {x[0], x[1], x[2], x[3]};
        if (NT) __builtin_nontemporal_store(w, p); else *p = w;
    } else {
        u32x2 *p = reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(base) + e);
        u32x2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        if (NT) __builtin_nontemporal_store(w, p); else *p = w;
    }
}

template <int DT>
__device__ __forceinline__ float load1(const void *base, int64_t e) {
    if constexpr (DT == APEXW_F32) return static_cast<const float *>(base)[e];
    else return __uint_as_float((uint32_t)static_cast<const uint16_t *>(base)[e] << 16);
}

template <int DT>
__device__ __forceinline__ void store1(void *base, int64_t e, float x) {
    if constexpr (DT == APEXW_F32) static_cast<float *>(base)[e] = x;
    else static_cast<uint16_t *>(base)[e] = (uint16_t)f32_to_bf16_bits(x);
}

// ---------------------------------------------------------------- wave max

// Maximum over the 64 lanes of a wave, returned to every lane.
__device__ __forceinline__ float wave_max(float x) {
    // quad xor 1, quad xor 2, half-row mirror, row mirror: the max of each
    // 16-lane row reaches all of its lanes through DPP moves
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false)));
    x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false)));
    // across the four rows
    x = fmaxf(x, __shfl_xor(x, 16, 64));
    x = fmaxf(x, __shfl_xor(x, 32, 64));
    return x;
}

// ---------------------------------------------------------------- tiles

// One tile of a dense-state tensor (fp32 or bf16 moments).
template <int PT, int GT, int ST, bool NT>
__device__ __forceinline__ void tile_dense(const TensorDesc &d, const void *grad,
                                           int64_t base, int n,
                                           const StepScalars &s) {
    const int lane = threadIdx.x;
    const bool vec_ok =
        (((uintptr_t)d.param | (uintptr_t)grad) & 15u) == 0u;
    float th[kSlots][kVec], g[kSlots][kVec], m[kSlots][kVec], v[kSlots][kVec];
#pragma unroll
    for (int k = 0; k < kSlots; ++k) {
        const int off = k * kSlotElems + lane * kVec;
        const int64_t e = base + off;
        if (vec_ok && off + kVec <= n) {
            load4<PT, NT>(d.param, e, th[k]);
            load4<GT, NT>(grad, e, g[k]);
            load4<ST, NT>(d.m, e, m[k]);
            load4<ST, NT>(d.v, e, v[k]);
        } else {
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const bool ok = off + j < n;
                th[k][j] = ok ? load1<PT>(d.param, e + j) : 0.0f;
                g[k][j] = ok ? load1<GT>(grad, e + j) : 0.0f;
                m[k][j] = ok ? load1<ST>(d.m, e + j) : 0.0f;
                v[k][j] = ok ? load1<ST>(d.v, e + j) : 0.0f;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kSlots; ++k)
#pragma unroll
        for (int j = 0; j < kVec; ++j)
            adamw_update(th[k][j], g[k][j], m[k][j], v[k][j], s);
#pragma unroll
    for (int k = 0; k < kSlots; ++k) {
        const int off = k * kSlotElems + lane * kVec;
        const int64_t e = base + off;
        if (vec_ok && off + kVec <= n) {
            store4<PT, NT>(d.param, e, th[k]);
            store4<ST, NT>(d.m, e, m[k]);
            store4<ST, NT>(d.v, e, v[k]);
        } else {
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                if (off + j < n) {
                    store1<PT>(d.param, e + j, th[k][j]);
                    store1<ST>(d.m, e + j, m[k][j]);
                    store1<ST>(d.v, e + j, v[k][j]);
                }
            }
        }
    }
}

// 8-bit codes: m signed (scale absmax|m|/127), v unsigned (scale max v/255),
// one scale per 256-element block; all-zero block -> scale 0, codes 0.
__device__ __forceinline__ uint32_t encode_signed(float x, float s) {
    if (s == 0.0f) return 0u;
    float r = rintf(x / s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)(uint8_t)(int8_t)(int)r;
}

__device__ __forceinline__ uint32_t encode_unsigned(float x, float s) {
    if (s == 0.0f) return 0u;
    float r = rintf(x / s);
    r = fminf(fmaxf(r, 0.0f), 255.0f);
    return (uint32_t)(int)r;
}

// One tile of an 8-bit-state tensor.  Wave w, slot k handles block
// (base + k*1024 + w*256) / 256 of the tensor.
template <int PT, int GT, bool NT>
__device__ __forceinline__ void tile_q8(const TensorDesc &d, const void *grad,
                                        int64_t base, int n,
                                        const StepScalars &s) {
    const int lane = threadIdx.x;
    const int wave = lane >> 6;
    const bool vec_ok =
        (((uintptr_t)d.param | (uintptr_t)grad) & 15u) == 0u;
    const int8_t *mq = static_cast<const int8_t *>(d.m);
    const uint8_t *vq = static_cast<const uint8_t *>(d.v);
    float th[kSlots][kVec], g[kSlots][kVec], m[kSlots][kVec], v[kSlots][kVec];
#pragma unroll
    for (int k = 0; k < kSlots; ++k) {
        const int off = k * kSlotElems + lane * kVec;
        const int64_t e = base + off;
        const int64_t blk = (base + k * kSlotElems + wave * kWaveElems) / APEXW_Q8_BLOCK;
        const bool block_live = k * kSlotElems + wave * kWaveElems < n;
        const float sm = block_live ? d.m_scale[blk] : 0.0f;
        const float sv = block_live ? d.v_scale[blk] : 0.0f;
        if (off + kVec <= n) {
            const uint32_t cm = *reinterpret_cast<const uint32_t *>(mq + e);
            const uint32_t cv = *reinterpret_cast<const uint32_t *>(vq + e);
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                m[k][j] = (float)(int8_t)(cm >> (8 * j)) * sm;
                v[k][j] = (float)(uint8_t)(cv >> (8 * j)) * sv;
            }
            if (vec_ok) {
                load4<PT, NT>(d.param, e, th[k]);
                load4<GT, NT>(grad, e, g[k]);
            } else {
#pragma unroll
                for (int j = 0; j < kVec; ++j) {
                    th[k][j] = load1<PT>(d.param, e + j);
                    g[k][j] = load1<GT>(grad, e + j);
                }
            }
        } else {
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const bool ok = off + j < n;
                m[k][j] = ok ? (float)mq[e + j] * sm : 0.0f;
                v[k][j] = ok ? (float)vq[e + j] * sv : 0.0f;
                th[k][j] = ok ? load1<PT>(d.param, e + j) : 0.0f;
                g[k][j] = ok ? load1<GT>(grad, e + j) : 0.0f;
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kSlots; ++k)
#pragma unroll
        for (int j = 0; j < kVec; ++j)
            adamw_update(th[k][j], g[k][j], m[k][j], v[k][j], s);
#pragma unroll
    for (int k = 0; k < kSlots; ++k) {
        const int off = k * kSlotElems + lane * kVec;
        const int64_t e = base + off;
        const int64_t blk = (base + k * kSlotElems + wave * kWaveElems) / APEXW_Q8_BLOCK;
        const bool block_live = k * kSlotElems + wave * kWaveElems < n;
        // lanes past the end hold m = v = 0 after the update only if their
        // inputs were 0 and g = 0: mask them out of the block maxima
        float am = 0.0f, av = 0.0f;
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            if (off + j < n) {
                am = fmaxf(am, fabsf(m[k][j]));
                av = fmaxf(av, v[k][j]);
            }
        }
        am = wave_max(am);
        av = wave_max(av);
        if (!block_live) continue;             // uniform per wave
        const float sm = am / 127.0f;
        const float sv = av / 255.0f;
        if ((lane & 63) == 0) {
            d.m_scale[blk] = sm;
            d.v_scale[blk] = sv;
        }
        if (off + kVec <= n) {
            uint32_t cm = 0, cv = 0;
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                cm |= encode_signed(m[k][j], sm) << (8 * j);
                cv |= encode_unsigned(v[k][j], sv) << (8 * j);
            }
            *reinterpret_cast<uint32_t *>(const_cast<int8_t *>(mq) + e) = cm;
            *reinterpret_cast<uint32_t *>(const_cast<uint8_t *>(vq) + e) = cv;
            if (vec_ok) {
                store4<PT, NT>(d.param, e, th[k]);
            } else {
#pragma unroll
                for (int j = 0; j < kVec; ++j) store1<PT>(d.param, e + j, th[k][j]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                if (off + j < n) {
                    const_cast<int8_t *>(mq)[e + j] = (int8_t)encode_signed(m[k][j], sm);
                    const_cast<uint8_t *>(vq)[e + j] = (uint8_t)encode_unsigned(v[k][j], sv);
                    store1<PT>(d.param, e + j, th[k][j]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------- kernel

// ST: APEXW_STATE_F32 / _BF16 / _Q8.  PT, GT: parameter and grad types.
template <int ST, int PT, int GT, bool NT>
__global__ __launch_bounds__(kThreads) void adamw_step_kernel(KernelArgs a) {
    // found_inf (M041 section 06, Apex guide 4.3): the whole step is skipped
    // on the device; every workgroup reads the same flag, so all leave.
    if (a.found_inf != nullptr && *a.found_inf != 0.0f) return;

    for (int32_t tile = blockIdx.x; tile < a.n_tiles; tile += gridDim.x) {
        const TileRef tr = a.tiles[tile];
        const void *grad = a.grads[tr.tensor];
        if (grad == nullptr) continue;          // no grad: tensor untouched
        const TensorDesc d = a.desc[tr.tensor];
        const int32_t t = a.steps[tr.tensor] + 1;
        const StepScalars s = step_scalars(a.groups[d.group], t);
        const int64_t base = (int64_t)tr.index * kTile;
        const int64_t left = d.numel - base;
        const int n = left < kTile ? (int)left : kTile;
        if constexpr (ST == APEXW_STATE_F32)
            tile_dense<PT, GT, APEXW_F32, NT>(d, grad, base, n, s);
        else if constexpr (ST == APEXW_STATE_BF16)
            tile_dense<PT, GT, APEXW_BF16, NT>(d, grad, base, n, s);
        else
            tile_q8<PT, GT, NT>(d, grad, base, n, s);
    }

    // Step counters advance once every workgroup has read them: the last
    // workgroup to finish bumps t for this launch's tensors that had a grad
    // and re-arms the ticket for the next launch.
    __shared__ bool last;
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const uint32_t done = atomicAdd(a.ticket, 1u);
        last = (done == gridDim.x - 1);
    }
    __syncthreads();
    if (last) {
        __threadfence();
        for (int j = threadIdx.x; j < a.n_tensors; j += kThreads) {
            const int32_t i = a.tensors[j];
            if (a.grads[i] != nullptr) a.steps[i] += 1;
        }
        if (threadIdx.x == 0) atomicExch(a.ticket, 0u);
    }
}

// Zero fill of the state buffer (used once, at creation).
__global__ __launch_bounds__(kThreads) void fill_zero_kernel(uint32_t *p, int64_t n_words) {
    for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n_words;
         i += (int64_t)gridDim.x * kThreads)
        p[i] = 0u;
}

}  // namespace apexw
