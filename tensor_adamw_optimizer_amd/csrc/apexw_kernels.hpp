// apexw_kernels.hpp -- gfx950 device code of the fused multi-tensor AdamW step.
//
// The parameter list is cut into 256-element tiles (a tile never spans two
// tensors) and each tile is one workgroup of one wave64: lane l owns the 4
// contiguous elements 4l..4l+3, so every load instruction of the wave covers
// one contiguous 256-element run (fp32: 1 KiB as dwordx4, bf16: 512 B as
// dwordx2, 8-bit codes: 256 B as dword), and in the 8-bit format the tile is
// exactly one quantisation block.  Every element is read once and written
// once: theta, g, m, v in; theta, m, v out (28 B per fp32 element, the
// one-pass ledger of the M041 page, section 04).  Small one-tile workgroups
// keep many independent read and write streams in flight.  A step is one of:
//  * adamw_carry_step_kernel (8-bit: adamw_carry_pair_q8_kernel, two
//    consecutive blocks per workgroup, or adamw_carry_step_q8_kernel under a
//    workgroup cap) -- the default: one launch per (param, grad) dtype pair.  Every
//    workgroup takes its tensor's bias corrections 1-beta1^t, 1-beta2^t from
//    an array the previous step wrote; the first tile of each tensor
//    advances the tensor's step counter (only with a grad and without
//    found_inf) and writes the corrections for the step after into a second
//    array; carry_init_kernel starts the chain from the counters;
//  * adamw_prepare_kernel, then adamw_step_kernel -- one lane per tensor
//    writes each tensor's step record (grad pointer, fp32 group scalars,
//    bias corrections from fp64 square-and-multiply) and advances its
//    counter, then the update launches read the records (steps whose
//    hyperparameters live in device memory, and lists with an empty tensor);
//  * adamw_single_step_kernel -- small lists: every workgroup forms its
//    tensor's record itself and the last to finish, found through a tree of
//    arrival counters, advances the counters.
// With fp32 moments the path is HBM-bandwidth bound; with 8-bit moments the
// exact fp32 arithmetic (the correctly rounded division and square root per
// element, the block reductions, decode and encode) and each block's chain
// of memory round trips are the limit.  There is
// no contraction in the method, so no matrix-core work; the arithmetic is
// ordinary fp32 VALU code compiled without contraction, with exact shortcuts
// where the hardware offers them (bf16 pair conversion, square root from
// v_sqrt_f32 and v_rsq_f32 plus one residual correction, every division --
// by the per-tensor bias corrections and by the per-element denominator --
// from a correctly rounded reciprocal plus one residual correction, 8-bit
// codes from v_rcp_f32 plus a tie guard).
//
// Read-only passes for the mixed-precision recipe and clipping:
//  * unscale_check_kernel -- any non-finite unscaled grad sets found_inf;
//  * grad_norm_partials_kernel, grad_norm_reduce_kernel,
//    grad_norm_final_kernel -- the global grad norm in a fixed summation
//    order and the clip coefficient.
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
#include "apexw_plan.hpp"

namespace apexw {

constexpr int kPrepThreads = 256;             // lanes per prepare workgroup
constexpr int kFewTensors = 8;                // launches this small skip the tile table
static_assert(kTile == APEXW_Q8_BLOCK, "a tile is one 8-bit block");
static_assert(kF32 == APEXW_F32 && kBF16 == APEXW_BF16, "plan dtype codes are the ABI's");

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Address spaces.  Data pointers arrive through tables as generic pointers;
// casting them to the global space gives global_load/global_store (with the
// non-temporal bit) instead of flat accesses.  The per-tile metadata (tile
// table, descriptors, step records) is read-only for the whole
// update launch, so it is read through the constant space, which lets the
// compiler use scalar loads (scalar cache) for these wave-uniform values.
// (The single-launch kernel also reads the step counters that way; its last
// workgroup writes them only after every workgroup has read them, through a
// generic pointer.  In the carried step every workgroup loads its tensor's
// counter that way too, but only the tensor's first tile uses the value, and
// that tile writes the counter after its own read, which the written value
// depends on; the carried bias corrections are read from one array and
// written to the other, so no workgroup reads what this launch writes.  The
// 8-bit block scales are read that way too: each is read, then rewritten,
// by the one wave that owns its block, and read by no other.)
#define APEXW_GLOBAL __attribute__((address_space(1)))
#define APEXW_CONST __attribute__((address_space(4)))

template <typename T>
__device__ __forceinline__ APEXW_GLOBAL T *gptr(void *p) { return (APEXW_GLOBAL T *)p; }
template <typename T>
__device__ __forceinline__ const APEXW_GLOBAL T *gptr(const void *p) {
    return (const APEXW_GLOBAL T *)p;
}
template <typename T>
__device__ __forceinline__ const APEXW_CONST T *cptr(const void *p) {
    return (const APEXW_CONST T *)p;
}

// Per-group scalars, formed on the host once per call.
struct GroupScalars {
    float beta1, one_minus_beta1, beta2, one_minus_beta2;
    float lr, decay, eps;
    float x_lo;                               // step_x_lo(eps)
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
    int64_t first_tile;  // index of the tensor's first tile in the tile table
    int32_t group;
    int32_t pad_;
};
static_assert(sizeof(TensorDesc) == 64, "descriptor is one 64-byte record");

// Per-tensor record of one step, written by the prepare kernel: the grad to
// apply (nullptr: leave the tensor alone -- no grad, or the step is skipped)
// and every scalar the update needs, so the update kernel reads one record
// per tensor and nothing else besides the descriptor.
struct StepRecord {
    const void *grad;
    float beta1, one_minus_beta1, beta2, one_minus_beta2;
    float lr, decay, eps;
    float bc1, bc2;                  // 1 - beta1^t, 1 - beta2^t
    float inv_scale;                 // grads are unscaled by this first
    float clip_coef;                 // then multiplied by this (norm clipping)
    float rbc1, rbc2;                // 1/bc1, 1/bc2 correctly rounded
    float div_lo;                    // 2^-96 if bc1, bc2 >= 2^-60, else +inf (see div_uniform)
};
static_assert(sizeof(StepRecord) == 64, "step record is one 64-byte record");

// Bias corrections of a tensor's next step, carried from one step to the
// next (launch mode 3): 1 - beta^(t+1) for the counter t as it stands, their
// reciprocals and the short-division bound.  Two arrays in the workspace; a
// step reads one and the first tile of each tensor writes the other.
struct BiasRecord {
    float bc1, bc2;                  // 1 - beta1^(t+1), 1 - beta2^(t+1)
    float rbc1, rbc2;                // 1/bc1, 1/bc2 correctly rounded
    float div_lo;                    // as in StepRecord
    int32_t pad_[3];
};
static_assert(sizeof(BiasRecord) == 32, "bias record is one 32-byte record");

struct KernelArgs {
    const TensorDesc *desc;
    const void *const *grads;        // grads[i] == nullptr: no grad this call
    const int32_t *tile_tensor;      // tensor of each tile, XCD-major per launch
    StepRecord *records;             // per tensor, rewritten every step
    int32_t *steps;                  // int32 step counter per tensor
    const float *found_inf;          // nullptr: never skip
    const float *inv_scale;          // nullptr: 1 (grads are not scaled)
    float *found_inf_out;            // unscale check: set to 1 on a non-finite
    const apexw_group *groups_dev;   // non-null: hyperparameters read on the device
    const float *clip_coef;          // nullptr: 1 (no clipping)
    double *partials;                // grad-norm pass: fp64 sum of squares per read group
    double *partials2;               // grad-norm finalize: one per first-stage workgroup
    double *norm_out;                // grad-norm finalize: the norm (may be null)
    float *clip_out;                 // grad-norm finalize: the clip coefficient
    double max_norm;
    int64_t n_partials;              // grad norm: read groups over all launches
    int64_t group_begin;             // grad norm: this launch's first partial
    int64_t tile_begin;              // this launch's tiles: [begin, begin+count)
    int64_t tile_count;
    int64_t table_begin;             // this launch's part of tile_tensor
    int64_t table_stride;            // ceil(tile_count / kXcds)
    int32_t n_tensors;
    int32_t tensor_begin;            // single-launch step: this launch's tensors are
    int32_t tensor_count;            //   tensor_list[begin, begin+count)
    int32_t pad_;
    const int32_t *tensor_list;
    uint32_t *done;                  // single-launch step: arrival counters
    const BiasRecord *bias_cur;      // carried step: this step's bias corrections
    BiasRecord *bias_next;           //   and the next step's (written by first tiles)
    // carried step over a launch of at most kFewTensors tensors, none empty,
    // uncapped, with cached accesses (few = 0 otherwise): the few-tensor
    // kernels find a tile's tensor from these, not the tile table; entries
    // past `few` repeat the last tensor
    int32_t few;                     // tensors of the launch
    int32_t few_first[kFewTensors];  // launch-relative first tile of each
    int32_t few_tensor[kFewTensors]; // their tensor indices
    GroupScalars groups[APEXW_MAX_GROUPS];
};

// Scalars of one tensor at its advanced step count.
struct StepScalars {
    float beta1, one_minus_beta1, beta2, one_minus_beta2;
    float lr, decay, eps;
    float bc1, bc2;                  // 1 - beta1^t, 1 - beta2^t (fp32)
    float rbc1, rbc2;                // 1/bc1, 1/bc2 correctly rounded
    float div_lo;                    // 2^-96 if bc1, bc2 >= 2^-60, else +inf
    float x_lo;                      // 2^-96 if 0 <= eps <= 2^28, else +inf
    float inv_scale;                 // 1 unless grads arrive scaled
    float clip_coef;                 // 1 unless the grad norm is clipped
};

// The lower bound of |lr * m_hat| for the short form of the update's last
// division (adamw_update4): 2^-96 when eps lies in [0, 2^28], else +inf (every
// element then takes the division).  An integer test on the bit pattern
// (+0 .. 2^28 are the patterns 0 .. 0x4d800000; -0, negatives and NaNs lie
// above), so it needs no vector instruction.
__device__ __forceinline__ float step_x_lo(float eps) {
    return __float_as_uint(eps) <= 0x4d800000u ? 0x1p-96f : __builtin_inff();
}


// b1^n and b2^n in fp64: square-and-multiply from the least significant
// bit, the two powers in one loop (the same products for each as two
// separate loops would form, with their dependency chains interleaved).
__device__ __forceinline__ void pow2_uint(double b1, double b2, uint32_t n, double &r1, double &r2) {
    r1 = 1.0;
    r2 = 1.0;
    while (n != 0u) {
        if (n & 1u) {
            r1 = r1 * b1;
            r2 = r2 * b2;
        }
        b1 = b1 * b1;
        b2 = b2 * b2;
        n >>= 1;
    }
}

__device__ __forceinline__ StepScalars step_scalars(const StepRecord &r) {
    StepScalars s;
    s.beta1 = r.beta1;
    s.one_minus_beta1 = r.one_minus_beta1;
    s.beta2 = r.beta2;
    s.one_minus_beta2 = r.one_minus_beta2;
    s.lr = r.lr;
    s.decay = r.decay;
    s.eps = r.eps;
    s.bc1 = r.bc1;
    s.bc2 = r.bc2;
    s.rbc1 = r.rbc1;
    s.rbc2 = r.rbc2;
    s.div_lo = r.div_lo;
    s.x_lo = step_x_lo(r.eps);
    s.inv_scale = r.inv_scale;
    s.clip_coef = r.clip_coef;
    return s;
}

// True in every lane if p holds in any lane (the compare mask itself, read
// as a scalar: no per-lane materialisation of p).
__device__ __forceinline__ bool wave_any(bool p) { return __builtin_amdgcn_ballot_w64(p) != 0; }

// Square root rounded to nearest for x in [2^-96, 2^64): s = v_sqrt_f32(x)
// (within one ulp, not always the nearest), then one correction with the
// exact residual x - s*s (an fma) times half the reciprocal square root
// (v_rsq_f32), rounded once.  tests/rules/rcp_sqrt_all.hip checks the result
// on the device against the nearest square root for every fp32 x in that
// range (an exact fp64 test of the two midpoints; no mismatch).  The rule is
// exact for these instructions' own outputs, not for every pair of one-ulp
// approximations (tests/rules/rcp_sqrt_rule.c finds a few x per two binades
// that such pairs get wrong), so the device check is what establishes it.
__device__ __forceinline__ float sqrt_rn(float x) {
    const float s = __builtin_amdgcn_sqrtf(x);
    const float h = 0.5f * __builtin_amdgcn_rsqf(x);
    return fmaf(fmaf(-s, s, x), h, s);
}

// 1/b rounded to nearest for b in [2^-126, 2^126]: v_rcp_f32 (within one
// ulp) and one Newton step y + y*(1 - b*y), both products in fmas.
// tests/rules/rcp_sqrt_all.hip checks it on the device for every fp32 b in
// that range (no mismatch).  As with sqrt_rn, that holds for the hardware's
// own first approximation, not for every one-ulp one (a one-ulp-high start
// fails for 32 significands per binade in tests/rules/rcp_sqrt_rule.c).
__device__ __forceinline__ float rcp_rn(float b) {
    const float y = __builtin_amdgcn_rcpf(b);
    return fmaf(fmaf(-b, y, 1.0f), y, y);
}

// x / b correctly rounded, for a wave-uniform divisor b in [2^-60, 1] with
// y = 1/b correctly rounded (lo = 2^-96) -- and for the per-element divisor
// of the update's last division, whose range adamw_update4 states: q = x*y,
// then one correction with
// the exact residual r = fma(-q, b, x), q + r*y rounded once -- Markstein's
// correction step (P. Markstein, "Computation of elementary functions on the
// IBM RISC System/6000 processor", 1990: with y the correctly rounded
// reciprocal and q within an ulp of x/b, q + r*y rounds to the correctly
// rounded quotient).  tests/rules/div_exhaustive.c checks it bit for bit
// against IEEE division for every pair of fp32 significands of x and b in
// [1, 2) (2^46 pairs, no mismatch), and scaling x and b by powers of two
// scales every step exactly as long as nothing leaves the normal range: for
// 2^-96 <= |x| < 2^64 the residual's lowest bit stays >= 2^-143 and x*y <
// 2^124.  Other x (zero -- whose sign the short form loses --, subnormals,
// inf, NaN, huge) take the division, and so does every x when b is outside
// that range (lo = +inf then).
__device__ __forceinline__ float div_short(float x, float b, float y) {
    const float q = x * y;
    const float r = fmaf(-q, b, x);
    return fmaf(r, y, q);
}

__device__ __forceinline__ float div_uniform(float x, float b, float y, float lo) {
    float q = div_short(x, b, y);
    if (!(fabsf(x) >= lo && fabsf(x) < 0x1p64f)) {   // rare: skipped by the wave
        asm volatile("");                                                // not speculated
        q = x / b;
    }
    return q;
}

// The AdamW update (M041 section 02), fp32, each operation rounded,
// evaluated left to right as printed, on the unscaled and clipped grad (the
// mixed-precision recipe of M041 section 06: unscale, check, clip;
// multiplying by 1 is exact).
// SC: the step may scale the grads (inv_scale, clip_coef given); a plain
// step skips the two multiplies by 1, which change nothing.
//
// Exact shortcuts, none of which changes a bit of the result:
//  * m_hat = m when bc1 == 1 (1 - beta1^t rounds to 1 in fp32 once beta1^t <
//    2^-25, after about 160 steps for beta1 = 0.9): x / 1 == x; a
//    wave-uniform branch;
//  * v_hat, its root and the last division take short forms under one range
//    test.  For v >= div_lo = 2^-96 whose short quotient v_hat is below 2^56,
//    v < 2^64 (v_hat >= v: bc2 <= 1), so v_hat is the correctly rounded v /
//    bc2, in [2^-96, 2^56), where sqrt_rn is exact; with eps in [0, 2^28]
//    (x_lo finite) the divisor denom = root + eps lies in [2^-48, 2^29], where
//    rcp_rn is exact; and for 2^-96 <= |lr * m_hat| < 2^64 the quotient lies
//    in [2^-125, 2^112), so every step of the short division stays normal and
//    its residual exact (lowest bit >= 2^-143), and it returns the correctly
//    rounded quotient.  If any element of the wave fails the test (a zero --
//    whose sign the short form would lose --, a tiny, huge, infinite or NaN
//    value), the wave recomputes the last division of all its elements with
//    the IEEE division and the compiler's correctly rounded square root,
//    which agree with the short forms wherever those apply.
//
// The update of a lane's kVec elements, stage by stage over the elements (so
// that the bc1 test is one branch for all of them and writes x = lr * m_hat
// directly): short forms for all, and in the rare wave where any element
// needs it, the exact last division for all (a wave-uniform branch: no
// per-element exec-mask regions on the common path).  valid: the lane's
// elements inside the tensor (a tensor's last tile); the others are padding
// whose results are discarded, so they do not call for the exact path.
template <bool SC>
__device__ __forceinline__ void adamw_update4(float (&th)[kVec], const float (&g_in)[kVec],
                                              float (&m)[kVec], float (&v)[kVec],
                                              const StepScalars &s, int valid = kVec) {
    float x[kVec], td[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        const float g = SC ? (g_in[j] * s.inv_scale) * s.clip_coef : g_in[j];
        m[j] = s.beta1 * m[j] + s.one_minus_beta1 * g;
        v[j] = s.beta2 * v[j] + (s.one_minus_beta2 * g) * g;
    }
    if (__float_as_uint(s.bc1) == 0x3f800000u) {     // bc1 == 1: m_hat = m (scalar test)
#pragma unroll
        for (int j = 0; j < kVec; ++j) x[j] = s.lr * m[j];
    } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j) x[j] = s.lr * div_uniform(m[j], s.bc1, s.rbc1, s.div_lo);
    }
    bool ok = true;
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        td[j] = th[j] * s.decay;
        const float v_hat = div_short(v[j], s.bc2, s.rbc2);
        const float denom = sqrt_rn(v_hat) + s.eps;
        th[j] = td[j] - div_short(x[j], denom, rcp_rn(denom));
        // bitwise, not short-circuit: the comparisons are lane masks
        // combined by scalar instructions, with no branch between them
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wbitwise-instead-of-logical"
        ok &= ((v[j] >= s.div_lo) & (v_hat < 0x1p56f) & (fabsf(x[j]) >= s.x_lo) &
               (fabsf(x[j]) < 0x1p64f)) | (j >= valid);
#pragma clang diagnostic pop
    }
    if (wave_any(!ok)) {
        asm volatile("");                            // not speculated
#pragma unroll
        for (int j = 0; j < kVec; ++j) th[j] = td[j] - x[j] / (sqrtf(v[j] / s.bc2) + s.eps);
    }
}

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Nearest bf16 of two fp32 values, ties to even; a NaN stays a NaN with the
// quiet bit set and the top 7 payload bits kept.  gfx950 converts a pair in
// one instruction (v_cvt_pk_bf16_f32) whose result equals that rule for all
// 2^32 inputs, denormals included (an exhaustive device check).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return pack_bf16x2(f, 0.0f) & 0xffffu;
}

// ---------------------------------------------------------------- loads

// Element types: APEXW_F32 (fp32) or APEXW_BF16 (bf16 bit patterns).
template <int DT, bool NT>
__device__ __forceinline__ void load4(const void *base, int64_t e, float (&x)[kVec]) {
    if constexpr (DT == APEXW_F32) {
        const APEXW_GLOBAL f32x4 *p = gptr<f32x4>(static_cast<const float *>(base) + e);
        f32x4 w = NT ? __builtin_nontemporal_load(p) : *p;
        x[0] = w.x; x[1] = w.y; x[2] = w.z; x[3] = w.w;
    } else {
        const APEXW_GLOBAL u32x2 *p = gptr<u32x2>(static_cast<const uint16_t *>(base) + e);
        u32x2 w = NT ? __builtin_nontemporal_load(p) : *p;
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
        x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    }
}

template <int DT, bool NT>
__device__ __forceinline__ void store4(void *base, int64_t e, const float (&x)[kVec]) {
    if constexpr (DT == APEXW_F32) {
        APEXW_GLOBAL f32x4 *p = gptr<f32x4>(static_cast<float *>(base) + e);
        f32x4 w = {x[0], x[1], x[2], x[3]};
        if (NT) __builtin_nontemporal_store(w, p); else *p = w;
    } else {
        APEXW_GLOBAL u32x2 *p = gptr<u32x2>(static_cast<uint16_t *>(base) + e);
        u32x2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
        if (NT) __builtin_nontemporal_store(w, p); else *p = w;
    }
}

template <bool NT>
__device__ __forceinline__ uint32_t load_u32(const void *base, int64_t byte_off) {
    const APEXW_GLOBAL uint32_t *p = gptr<uint32_t>(static_cast<const char *>(base) + byte_off);
    return NT ? __builtin_nontemporal_load(p) : *p;
}

template <bool NT>
__device__ __forceinline__ void store_u32(void *base, int64_t byte_off, uint32_t w) {
    APEXW_GLOBAL uint32_t *p = gptr<uint32_t>(static_cast<char *>(base) + byte_off);
    if (NT) __builtin_nontemporal_store(w, p); else *p = w;
}

template <int DT>
__device__ __forceinline__ float load1(const void *base, int64_t e) {
    if constexpr (DT == APEXW_F32) return gptr<float>(base)[e];
    else return __uint_as_float((uint32_t)gptr<uint16_t>(base)[e] << 16);
}

template <int DT>
__device__ __forceinline__ void store1(void *base, int64_t e, float x) {
    if constexpr (DT == APEXW_F32) gptr<float>(base)[e] = x;
    else gptr<uint16_t>(base)[e] = (uint16_t)f32_to_bf16_bits(x);
}

// A tile's element offsets are multiples of 4, so an array's 4-element
// vector accesses are aligned exactly when its base pointer is (16 B for
// fp32, 8 B for bf16).  Arrays that are not -- views into flat buffers at odd
// offsets -- take 4 element accesses instead; the state arrays always align.
template <int DT>
__device__ __forceinline__ bool vec_aligned(const void *p) {
    return ((uintptr_t)p & (DT == APEXW_F32 ? 15u : 7u)) == 0u;
}

// bf16 data is fetched as raw words in either branch and widened after the
// branches join: widening inside a branch makes the compiler wait there for
// the load, and for every load issued before it, ahead of the next load.
template <int DT, bool NT>
__device__ __forceinline__ void load4_any(const void *base, int64_t e, float (&x)[kVec], bool vec) {
    if constexpr (DT == APEXW_F32) {
        if (vec) {
            load4<DT, NT>(base, e, x);
        } else {
#pragma unroll
            for (int j = 0; j < kVec; ++j) x[j] = load1<DT>(base, e + j);
        }
    } else {
        u32x2 w;
        if (vec) {
            const APEXW_GLOBAL u32x2 *p = gptr<u32x2>(static_cast<const uint16_t *>(base) + e);
            w = NT ? __builtin_nontemporal_load(p) : *p;
        } else {
            const APEXW_GLOBAL uint16_t *h = gptr<uint16_t>(base) + e;
            w.x = (uint32_t)h[0] | (uint32_t)h[1] << 16;
            w.y = (uint32_t)h[2] | (uint32_t)h[3] << 16;
        }
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
        x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    }
}

template <int DT, bool NT>
__device__ __forceinline__ void store4_any(void *base, int64_t e, const float (&x)[kVec], bool vec) {
    if (vec) {
        store4<DT, NT>(base, e, x);
    } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j) store1<DT>(base, e + j, x[j]);
    }
}

// ---------------------------------------------------------------- wave max

// Wave reductions of non-negative, NaN-free floats: for such values the
// order of the bit patterns as unsigned integers is the order of the
// numbers, so the reduction is integer (DPP moves).  max_dpp: one fused move
// and maximum; lanes of the rows a broadcast does not write receive 0 (the
// old operand), the identity of the maximum.
template <int CTRL, int ROWS>
__device__ __forceinline__ uint32_t max_dpp(uint32_t u) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, CTRL, ROWS, 0xF, false);
    return u > o ? u : o;
}

// Maxima over the 64 lanes of the wave of two sets of such values, returned
// wave-uniform: one
// v_permlane32_swap exchanges the upper half of a's lanes with the lower half
// of b's, so one maximum leaves a's pairwise maxima in lanes 0-31 and b's in
// lanes 32-63; the quad swaps and row mirrors give every 16-lane row its
// maximum, and row_bcast:15 carries row 0 into row 1 and row 2 into row 3,
// so lane 31 ends with a's maximum and lane 63 with b's -- nine instructions
// where two separate reductions take fourteen.
__device__ __forceinline__ void wave_max_nonneg2(float a, float b, float &max_a, float &max_b) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b),
                                                     false, false);
    uint32_t u = sw[0] > sw[1] ? sw[0] : sw[1];
    u = max_dpp<0xB1, 0xF>(u);       // quad_perm [1,0,3,2]
    u = max_dpp<0x4E, 0xF>(u);       // quad_perm [2,3,0,1]
    u = max_dpp<0x141, 0xF>(u);      // row_half_mirror
    u = max_dpp<0x140, 0xF>(u);      // row_mirror
    u = max_dpp<0x142, 0xA>(u);      // row_bcast:15, rows 1 and 3
    max_a = __uint_as_float(__builtin_amdgcn_readlane(u, 31));
    max_b = __uint_as_float(__builtin_amdgcn_readlane(u, 63));
}

// ---------------------------------------------------------------- tiles

// One 256-element tile of a tensor with fp32 or bf16 moments (ST = element
// type of m and v).  n = valid elements in this tile (1..256).  A full tile
// takes the vector path.  In a tensor's last, partial tile the update runs
// on all 4 values of every lane together (one converged pass), and only the
// valid elements of theta are stored.
// get() yields the step's scalars; it is called after the tile's loads are
// issued, so any memory reads or arithmetic it needs overlap with them.
template <int PT, int GT, int ST, bool NT, bool SC, typename Get>
__device__ __forceinline__ void tile_dense(const TensorDesc &d, const void *grad,
                                           int64_t base, int n, const Get &get) {
    const int off = threadIdx.x * kVec;
    const int64_t e = base + off;
    float th[kVec], g[kVec], m[kVec], v[kVec];
    if (n == kTile) {                                  // wave-uniform
        const bool pv = vec_aligned<PT>(d.param), gv = vec_aligned<GT>(grad);
        load4<ST, NT>(d.m, e, m);
        load4<ST, NT>(d.v, e, v);
        load4_any<GT, NT>(grad, e, g, gv);
        load4_any<PT, NT>(d.param, e, th, pv);
        const StepScalars s = get();
        adamw_update4<SC>(th, g, m, v, s);
        store4_any<PT, NT>(d.param, e, th, pv);
        store4<ST, NT>(d.m, e, m);
        store4<ST, NT>(d.v, e, v);
    } else {
        // m and v are read and written as whole vectors up to the end of
        // their last 128-byte line (the state arrays are padded for it, and
        // the padding is always written as +0); theta and g as vectors in
        // the lanes wholly inside the tensor, element by element in the one
        // lane that straddles its end
        constexpr int kChunk = ST == APEXW_F32 ? 32 : 64;
        const int n_pad = (n + kChunk - 1) / kChunk * kChunk;
        const bool pv = vec_aligned<PT>(d.param), gv = vec_aligned<GT>(grad);
        const bool inside = off + kVec <= n, padded = off < n_pad;
#pragma unroll
        for (int j = 0; j < kVec; ++j) m[j] = v[j] = 0.0f;
        if (padded) {
            load4<ST, NT>(d.m, e, m);
            load4<ST, NT>(d.v, e, v);
        }
        if (inside) {
            load4_any<GT, NT>(grad, e, g, gv);
            load4_any<PT, NT>(d.param, e, th, pv);
        } else {
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const bool ok = off + j < n;
                g[j] = ok ? load1<GT>(grad, e + j) : 0.0f;
                th[j] = ok ? load1<PT>(d.param, e + j) : 0.0f;
            }
        }
        const StepScalars s = get();
        adamw_update4<SC>(th, g, m, v, s, n - off);
#pragma unroll
        for (int j = 0; j < kVec; ++j)
            if (off + j >= n) m[j] = v[j] = 0.0f;      // padding: +0
        if (padded) {
            store4<ST, NT>(d.m, e, m);
            store4<ST, NT>(d.v, e, v);
        }
        if (inside) {
            store4_any<PT, NT>(d.param, e, th, pv);
        } else {
#pragma unroll
            for (int j = 0; j < kVec; ++j)
                if (off + j < n) store1<PT>(d.param, e + j, th[j]);
        }
    }
}

// 8-bit codes: m signed (scale absmax|m|/127), v unsigned (scale max v/255),
// one scale per 256-element block; an all-zero block has scale 0, codes 0.
//
// The code is round-half-even of the correctly rounded quotient x/s, clamped
// to the code range.  The quotient is not formed per element.  When s is a
// normal number (the usual case), inv = v_rcp_f32(s) is within one ulp of
// 1/s (tests/rules/rcp_sqrt_all.hip checks it for every normal s whose
// reciprocal is normal), so r = RN(x*inv) is within |x/s|*3*2^-24 of x/s,
// and RN(x/s) within |x/s|*2^-24; every |x| <= amax has |x/s| <=
// 127/(1 - 2^-24) (resp. 255/..), so both stay within 5e-5 of x/s and inside
// the code range.  When r is more
// than 2.5e-4 away from every half-integer, r and RN(x/s) therefore round to
// the same integer; otherwise (rare, or a NaN), or when s is zero, denormal
// or infinite, the quotient itself is rounded and clamped.  d = |r - rint(r)|
// is exact (Sterbenz) and at most 1/2, so "|d - 1/2| > 2.5e-4" is exactly
// "d < kTieBound", the float just above 1/2 - 2.5e-4: one comparison.
//
// The block scale amax/levels is the correctly rounded quotient, formed by
// div_short with 1/levels (a compile-time constant) for amax in
// [2^-100, FLT_MAX] -- the significand pairs of 127 and 255 are among those
// checked, and no step leaves the normal range there -- else by the
// division (zero, subnormal or infinite amax; wave-uniform, so no
// divergence).
constexpr float kTieBound = 0x1.ffbe78p-2f;   // RU(1/2 - 2.5e-4f) = 0.49975002

struct BlockScale {
    float s, inv;
    bool fast;      // s normal and finite: inv is usable
};

// amax: a block maximum, >= +0 and never a NaN (fmaxf passes NaNs over).
__device__ __forceinline__ BlockScale block_scale(float amax, float levels) {
    BlockScale b;
    b.s = div_short(amax, levels, 1.0f / levels);
    // amax in [2^-100, FLT_MAX] puts s = amax/levels (levels 127 or 255) in
    // [2^-108, 2^121]: normal, and its reciprocal normal too.  For amax >= +0
    // that range is the bit patterns 0x0d800000 .. 0x7f7fffff: one unsigned
    // compare of the pattern, on the scalar unit (amax is wave-uniform).
    b.fast = true;
    if (__float_as_uint(amax) - 0x0d800000u > 0x7f7fffffu - 0x0d800000u) {   // rare
        asm volatile("");
        b.s = amax / levels;
        b.fast = b.s >= 0x1p-126f && b.s <= 0x1p126f;
    }
    b.inv = __builtin_amdgcn_rcpf(b.s);
    return b;
}

// The code of x as an integer-valued float in [lo, hi].
__device__ __forceinline__ float code_value(float x, const BlockScale &b, float lo, float hi) {
    const float r = x * b.inv;
    float q = rintf(r);
    if (!b.fast || !(fabsf(r - q) < kTieBound)) {   // rare: skipped by the wave
        asm volatile("");                                          // not speculated
        q = b.s == 0.0f ? 0.0f : fminf(fmaxf(rintf(x / b.s), lo), hi);
    }
    return q;
}

// The signed code of x plus 128, an integer-valued float in [1, 255], with
// the offset inside the product: r = fma(x, inv, 128) rounds x*inv + 128
// once.  |x*inv - x/s| <= 127*2^-23 and the rounding at most 2^-17 (half an
// ulp below 256), so r is within 2.3e-5 of x/s + 128, and RN(x/s) + 128
// within 2.7e-5 of r (|x/s| <= 127/(1 - 2^-24)); when r is more than 2.5e-4
// from every half-integer the two round to the same integer, which is then
// in [1, 255].  r >= 0.99997, so r - rint(r) is exact (Sterbenz).  Otherwise
// (rare), or when s is not normal, the code_value rule gives the same code.
__device__ __forceinline__ float code_value_signed_128(float x, const BlockScale &b) {
    const float r = fmaf(x, b.inv, 128.0f);
    float q = rintf(r);
    if (!b.fast || !(fabsf(r - q) < kTieBound)) {   // rare: skipped by the wave
        asm volatile("");                                          // not speculated
        q = (b.s == 0.0f ? 0.0f : fminf(fmaxf(rintf(x / b.s), -127.0f), 127.0f)) + 128.0f;
    }
    return q;
}

// Four codes packed little-endian into one word (v_cvt_pk_u8_f32 writes an
// integer-valued float in [0, 255] into one byte); signed codes are packed
// offset by 128 and flipped back, which is two's complement per byte.
__device__ __forceinline__ uint32_t pack_codes_signed(const float (&x)[kVec], const BlockScale &b) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < kVec; ++j)
        w = __builtin_amdgcn_cvt_pk_u8_f32(code_value_signed_128(x[j], b), j, w);
    return w ^ 0x80808080u;
}

__device__ __forceinline__ uint32_t pack_codes_unsigned(const float (&x)[kVec], const BlockScale &b) {
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < kVec; ++j)
        w = __builtin_amdgcn_cvt_pk_u8_f32(code_value(x[j], b, 0.0f, 255.0f), j, w);
    return w;
}

// One tile = one 8-bit block (block index base/256 of the tensor): decode
// with the stored scales, update in fp32, reduce the block maxima over the
// wave, re-encode.  theta uses this step's fp32 moments.  A full tile is read
// in two phases: q8_load_full issues every load and only keeps the raw words,
// q8_finish_full decodes, updates, encodes and stores.

// Four values of an fp32 or bf16 array as loaded: one 16-byte or 8-byte
// vector, or element loads assembled into the same words.
template <int DT> struct Raw4;
template <> struct Raw4<APEXW_F32> { f32x4 w; };
template <> struct Raw4<APEXW_BF16> { u32x2 w; };

template <int DT, bool NT>
__device__ __forceinline__ Raw4<DT> load_raw4(const void *base, int64_t e, bool vec) {
    Raw4<DT> r;
    if constexpr (DT == APEXW_F32) {
        if (vec) {
            const APEXW_GLOBAL f32x4 *p = gptr<f32x4>(static_cast<const float *>(base) + e);
            r.w = NT ? __builtin_nontemporal_load(p) : *p;
        } else {
            const APEXW_GLOBAL float *h = gptr<float>(base) + e;
            r.w = f32x4{h[0], h[1], h[2], h[3]};
        }
    } else {
        if (vec) {
            const APEXW_GLOBAL u32x2 *p = gptr<u32x2>(static_cast<const uint16_t *>(base) + e);
            r.w = NT ? __builtin_nontemporal_load(p) : *p;
        } else {
            const APEXW_GLOBAL uint16_t *h = gptr<uint16_t>(base) + e;
            r.w.x = (uint32_t)h[0] | (uint32_t)h[1] << 16;
            r.w.y = (uint32_t)h[2] | (uint32_t)h[3] << 16;
        }
    }
    return r;
}

template <int DT>
__device__ __forceinline__ void widen4(const Raw4<DT> &r, float (&x)[kVec]) {
    if constexpr (DT == APEXW_F32) {
        x[0] = r.w.x; x[1] = r.w.y; x[2] = r.w.z; x[3] = r.w.w;
    } else {
        x[0] = bf16_lo(r.w.x); x[1] = bf16_hi(r.w.x);
        x[2] = bf16_lo(r.w.y); x[3] = bf16_hi(r.w.y);
    }
}

template <int PT, int GT>
struct Q8Raw {
    uint32_t cm, cv;                 // 4 codes of m and of v
    Raw4<GT> g;
    Raw4<PT> th;
    float sm, sv;                    // the block's stored scales
};

template <int PT, int GT, bool NT>
__device__ __forceinline__ Q8Raw<PT, GT> q8_load_full(const TensorDesc &d, const void *grad,
                                                      int64_t base) {
    const int64_t e = base + threadIdx.x * kVec;
    const int64_t blk = base / APEXW_Q8_BLOCK;
    Q8Raw<PT, GT> r;
    // the stored scales: wave-uniform, read through the constant space (scalar
    // loads; this wave alone writes them, after this read)
    r.sm = cptr<float>(d.m_scale)[blk];
    r.sv = cptr<float>(d.v_scale)[blk];
    r.cm = load_u32<NT>(d.m, e);
    r.cv = load_u32<NT>(d.v, e);
    r.g = load_raw4<GT, NT>(grad, e, vec_aligned<GT>(grad));
    r.th = load_raw4<PT, NT>(d.param, e, vec_aligned<PT>(d.param));
    return r;
}

// The block's new scales (lane 0 stores them) from its maxima.
__device__ __forceinline__ void q8_block_scales(const TensorDesc &d, int64_t blk, float am,
                                                float av, BlockScale &bm, BlockScale &bv) {
    wave_max_nonneg2(am, av, am, av);
    bm = block_scale(am, 127.0f);
    bv = block_scale(av, 255.0f);
    if (threadIdx.x == 0) {
        gptr<float>(static_cast<void *>(d.m_scale))[blk] = bm.s;
        gptr<float>(static_cast<void *>(d.v_scale))[blk] = bv.s;
    }
}

template <int PT, int GT, bool NT, bool SC>
__device__ __forceinline__ void q8_finish_full(const TensorDesc &d, int64_t base,
                                               const Q8Raw<PT, GT> &r, const StepScalars &s) {
    const int64_t e = base + threadIdx.x * kVec;
    float th[kVec], g[kVec], m[kVec], v[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        m[j] = (float)(int8_t)(r.cm >> (8 * j)) * r.sm;
        v[j] = (float)(uint8_t)(r.cv >> (8 * j)) * r.sv;
    }
    widen4<GT>(r.g, g);
    widen4<PT>(r.th, th);
    adamw_update4<SC>(th, g, m, v, s);
    // block maxima (a NaN moment is passed over; v >= 0, fabs makes a -0 +0)
    float am = 0.0f, av = 0.0f;
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        am = fmaxf(am, fabsf(m[j]));
        av = fmaxf(av, fabsf(v[j]));
    }
    BlockScale bm, bv;
    q8_block_scales(d, base / APEXW_Q8_BLOCK, am, av, bm, bv);
    store_u32<NT>(d.m, e, pack_codes_signed(m, bm));
    store_u32<NT>(d.v, e, pack_codes_unsigned(v, bv));
    store4_any<PT, NT>(d.param, e, th, vec_aligned<PT>(d.param));
}

// A tensor's last tile when it holds n < 256 elements: element accesses in
// the lane that straddles the end, elements past it left out of the maxima.
template <int PT, int GT, bool NT, bool SC>
__device__ __forceinline__ void q8_tile_partial(const TensorDesc &d, const void *grad,
                                                int64_t base, int n, const StepScalars &s) {
    const int off = threadIdx.x * kVec;
    const int64_t e = base + off;
    const int64_t blk = base / APEXW_Q8_BLOCK;
    const bool pv = vec_aligned<PT>(d.param), gv = vec_aligned<GT>(grad);
    const APEXW_GLOBAL int8_t *mq = gptr<int8_t>(static_cast<const void *>(d.m));
    const APEXW_GLOBAL uint8_t *vq = gptr<uint8_t>(static_cast<const void *>(d.v));
    const float sm_old = cptr<float>(d.m_scale)[blk];
    const float sv_old = cptr<float>(d.v_scale)[blk];
    float th[kVec], g[kVec], m[kVec], v[kVec];
    const bool full = off + kVec <= n;
    if (full) {
        const uint32_t cm = load_u32<NT>(d.m, e);
        const uint32_t cv = load_u32<NT>(d.v, e);
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            m[j] = (float)(int8_t)(cm >> (8 * j)) * sm_old;
            v[j] = (float)(uint8_t)(cv >> (8 * j)) * sv_old;
        }
        load4_any<GT, NT>(grad, e, g, gv);
        load4_any<PT, NT>(d.param, e, th, pv);
    } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const bool ok = off + j < n;
            m[j] = ok ? (float)mq[e + j] * sm_old : 0.0f;
            v[j] = ok ? (float)vq[e + j] * sv_old : 0.0f;
            g[j] = ok ? load1<GT>(grad, e + j) : 0.0f;
            th[j] = ok ? load1<PT>(d.param, e + j) : 0.0f;
        }
    }
    adamw_update4<SC>(th, g, m, v, s, n - off);
    float am = 0.0f, av = 0.0f;
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        if (off + j < n) {                    // elements past the end do not count
            am = fmaxf(am, fabsf(m[j]));
            av = fmaxf(av, fabsf(v[j]));
        }
    }
    BlockScale bm, bv;
    q8_block_scales(d, blk, am, av, bm, bv);
    if (full) {
        store_u32<NT>(d.m, e, pack_codes_signed(m, bm));
        store_u32<NT>(d.v, e, pack_codes_unsigned(v, bv));
        store4_any<PT, NT>(d.param, e, th, pv);
    } else {
        // codes up to the end of their last 128-byte line (zero codes past
        // the tensor: the state arrays are padded for it), theta to its end
        const int n_pad = (n + 127) / 128 * 128;
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            if (off + j < n) {
                gptr<int8_t>(d.m)[e + j] = (int8_t)(int)code_value(m[j], bm, -127.0f, 127.0f);
                gptr<uint8_t>(d.v)[e + j] = (uint8_t)(int)code_value(v[j], bv, 0.0f, 255.0f);
                store1<PT>(d.param, e + j, th[j]);
            } else if (off + j < n_pad) {
                gptr<int8_t>(d.m)[e + j] = 0;
                gptr<uint8_t>(d.v)[e + j] = 0;
            }
        }
    }
}

// One 8-bit tile in a single phase; get() yields the step's scalars after
// the tile's loads are issued.
template <int PT, int GT, bool NT, bool SC, typename Get>
__device__ __forceinline__ void tile_q8(const TensorDesc &d, const void *grad,
                                        int64_t base, int n, const Get &get) {
    if (n == kTile) {                          // wave-uniform
        const Q8Raw<PT, GT> r = q8_load_full<PT, GT, NT>(d, grad, base);
        q8_finish_full<PT, GT, NT, SC>(d, base, r, get());
    } else {
        q8_tile_partial<PT, GT, NT, SC>(d, grad, base, n, get());
    }
}

// Two consecutive full blocks of one tensor (base, base + 256) in one wave:
// one address computation for both (the second block's accesses differ by a
// constant offset), all loads issued before any arithmetic, both blocks'
// updates in one basic block, and their four maxima in two paired
// reductions.  Each block gets exactly what q8_finish_full gives it.
template <int PT, int GT, bool NT, bool SC>
__device__ __forceinline__ void q8_pair_full(const TensorDesc &d, const void *grad, int64_t base,
                                             const StepScalars &s) {
    const Q8Raw<PT, GT> r0 = q8_load_full<PT, GT, NT>(d, grad, base);
    const Q8Raw<PT, GT> r1 = q8_load_full<PT, GT, NT>(d, grad, base + kTile);
    const int64_t e = base + threadIdx.x * kVec;
    float th0[kVec], g0[kVec], m0[kVec], v0[kVec], th1[kVec], g1[kVec], m1[kVec], v1[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        m0[j] = (float)(int8_t)(r0.cm >> (8 * j)) * r0.sm;
        v0[j] = (float)(uint8_t)(r0.cv >> (8 * j)) * r0.sv;
        m1[j] = (float)(int8_t)(r1.cm >> (8 * j)) * r1.sm;
        v1[j] = (float)(uint8_t)(r1.cv >> (8 * j)) * r1.sv;
    }
    widen4<GT>(r0.g, g0);
    widen4<PT>(r0.th, th0);
    widen4<GT>(r1.g, g1);
    widen4<PT>(r1.th, th1);
    adamw_update4<SC>(th0, g0, m0, v0, s);
    adamw_update4<SC>(th1, g1, m1, v1, s);
    float am0 = 0.0f, av0 = 0.0f, am1 = 0.0f, av1 = 0.0f;
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        am0 = fmaxf(am0, fabsf(m0[j]));
        av0 = fmaxf(av0, fabsf(v0[j]));
        am1 = fmaxf(am1, fabsf(m1[j]));
        av1 = fmaxf(av1, fabsf(v1[j]));
    }
    wave_max_nonneg2(am0, am1, am0, am1);
    wave_max_nonneg2(av0, av1, av0, av1);
    const BlockScale bm0 = block_scale(am0, 127.0f), bv0 = block_scale(av0, 255.0f);
    const BlockScale bm1 = block_scale(am1, 127.0f), bv1 = block_scale(av1, 255.0f);
    const int64_t blk = base / APEXW_Q8_BLOCK;
    if (threadIdx.x == 0) {
        gptr<float>(static_cast<void *>(d.m_scale))[blk] = bm0.s;
        gptr<float>(static_cast<void *>(d.v_scale))[blk] = bv0.s;
        gptr<float>(static_cast<void *>(d.m_scale))[blk + 1] = bm1.s;
        gptr<float>(static_cast<void *>(d.v_scale))[blk + 1] = bv1.s;
    }
    const bool pv = vec_aligned<PT>(d.param);
    store_u32<NT>(d.m, e, pack_codes_signed(m0, bm0));
    store_u32<NT>(d.v, e, pack_codes_unsigned(v0, bv0));
    store4_any<PT, NT>(d.param, e, th0, pv);
    store_u32<NT>(d.m, e + kTile, pack_codes_signed(m1, bm1));
    store_u32<NT>(d.v, e + kTile, pack_codes_unsigned(v1, bv1));
    store4_any<PT, NT>(d.param, e + kTile, th1, pv);
}

// ---------------------------------------------------------------- kernels

// The fp32 scalars of a group, formed from its fp64 hyperparameters exactly
// as the host forms them (fp64 operations, then one rounding to fp32), for
// hyperparameters that live in device memory (graph-capturable steps).
__device__ __forceinline__ GroupScalars group_scalars(const apexw_group &G) {
    GroupScalars S;
    S.beta1 = (float)G.beta1;
    S.one_minus_beta1 = (float)(1.0 - G.beta1);
    S.beta2 = (float)G.beta2;
    S.one_minus_beta2 = (float)(1.0 - G.beta2);
    S.lr = (float)G.lr;
    S.decay = (float)(1.0 - G.lr * G.weight_decay);
    S.eps = (float)G.eps;
    S.x_lo = step_x_lo(S.eps);
    S.beta1_d = G.beta1;
    S.beta2_d = G.beta2;
    return S;
}

// Wave-uniform metadata reads through the constant space (scalar loads),
// copied out word by word.
template <typename T>
__device__ __forceinline__ T load_uniform(const T *tab, int32_t i) {
    static_assert(sizeof(T) % 8 == 0, "64-bit words");
    const APEXW_CONST uint64_t *p = cptr<uint64_t>(tab + i);
    uint64_t w[sizeof(T) / 8];
#pragma unroll
    for (int j = 0; j < (int)(sizeof(T) / 8); ++j) w[j] = p[j];
    T out;
    __builtin_memcpy(&out, w, sizeof out);
    return out;
}

// Bias corrections at step count t: 1 - beta^t from fp64 square-and-multiply
// rounded once to fp32, their correctly rounded reciprocals, and the range
// bound of the short division by them (div_uniform).
__device__ __forceinline__ BiasRecord bias_record(double beta1_d, double beta2_d, int32_t t) {
    BiasRecord b = {};
    double p1, p2;
    pow2_uint(beta1_d, beta2_d, (uint32_t)t, p1, p2);
    b.bc1 = (float)(1.0 - p1);
    b.bc2 = (float)(1.0 - p2);
    b.rbc1 = 1.0f / b.bc1;
    b.rbc2 = 1.0f / b.bc2;
    b.div_lo = b.bc1 >= 0x1p-60f && b.bc2 >= 0x1p-60f ? 0x1p-96f : __builtin_inff();   // both are <= 1
    return b;
}

// The step record of a tensor of group gi with a grad, at its advanced step
// count t: group scalars, bias corrections, the grad scale factors.
__device__ __forceinline__ StepRecord step_record(const KernelArgs &a, int32_t gi, const void *grad,
                                                  int32_t t, float inv_scale, float clip_coef) {
    GroupScalars g;
    if (a.groups_dev != nullptr)
        g = group_scalars(load_uniform(a.groups_dev, gi));
    else
        g = a.groups[gi];
    const BiasRecord b = bias_record(g.beta1_d, g.beta2_d, t);
    StepRecord r = {};
    r.grad = grad;
    r.beta1 = g.beta1;
    r.one_minus_beta1 = g.one_minus_beta1;
    r.beta2 = g.beta2;
    r.one_minus_beta2 = g.one_minus_beta2;
    r.lr = g.lr;
    r.decay = g.decay;
    r.eps = g.eps;
    r.bc1 = b.bc1;
    r.bc2 = b.bc2;
    r.rbc1 = b.rbc1;
    r.rbc2 = b.rbc2;
    r.div_lo = b.div_lo;
    r.inv_scale = inv_scale;
    r.clip_coef = clip_coef;
    return r;
}

// Before the update, one lane per tensor: unless found_inf is set (M041
// section 06, Apex guide 4.3), advance t of each tensor with a grad and write
// its step record (grad pointer, group scalars, bias corrections from fp64
// square-and-multiply); a tensor without a grad, or every tensor when
// found_inf is set, gets a record with no grad and no counter moves.  The
// flag is thus read once per tensor here instead of once per workgroup.
__global__ __launch_bounds__(kPrepThreads) void adamw_prepare_kernel(KernelArgs a) {
    const int32_t i = blockIdx.x * kPrepThreads + threadIdx.x;
    if (i >= a.n_tensors) return;
    StepRecord r = {};
    // every independent load first (flag, grad pointer, counter, group,
    // scale factors): one memory round trip instead of a chain of four.
    // found_inf, inv_scale and clip_coef are never NULL here: the host
    // passes device constants 0 / 1 / 1 in place of absent ones.
    const float fi = *a.found_inf;
    const void *g_ptr = a.grads[i];
    const int32_t t_old = a.steps[i];
    const int32_t gi = a.desc[i].group;
    const float inv_scale = *a.inv_scale;
    const float clip_coef = *a.clip_coef;
    asm volatile("" ::"v"(fi), "v"(g_ptr), "v"(t_old), "v"(gi), "v"(inv_scale), "v"(clip_coef));
    const void *grad = fi != 0.0f ? nullptr : g_ptr;
    if (grad != nullptr) {
        const int32_t t = t_old + 1;
        a.steps[i] = t;
        r = step_record(a, gi, grad, t, inv_scale, clip_coef);
    }
    a.records[i] = r;
}

// Position of tile k of a launch in its XCD-major tile table (the plan's
// table_position).
__device__ __forceinline__ int64_t table_pos(const KernelArgs &a, int64_t k) {
    return table_position(a.table_begin, a.table_stride, k);
}

// The update: one 256-element tile per workgroup (the grid-stride loop only
// runs more than once when the tile count exceeds the grid).
// ST: APEXW_STATE_F32 / _BF16 / _Q8.  PT, GT: parameter and grad types.
// SC: the grads are scaled (inv_scale and / or clip_coef given).
template <int ST, int PT, int GT, bool NT, bool SC>
__global__ __launch_bounds__(kThreads) void adamw_step_kernel(KernelArgs a) {
    const APEXW_CONST int32_t *tile_tensor = cptr<int32_t>(a.tile_tensor);
    int64_t k = blockIdx.x;                    // < tile_count: grid <= tiles
    int32_t i = tile_tensor[table_pos(a, k)];
    for (;;) {
        const StepRecord r = load_uniform(a.records, i);
        const TensorDesc d = load_uniform(a.desc, i);
        const int64_t base = (a.tile_begin + k - d.first_tile) * kTile;
        const int64_t left = d.numel - base;
        const int n = left < kTile ? (int)left : kTile;
        // Issue every metadata load before the branch (the compiler would
        // otherwise fetch the data pointers only after it, one more
        // round trip before the first data load); the empty asm only names
        // the values, it emits no instruction.
        asm volatile("" ::"s"(r.grad), "s"(d.param), "s"(d.m), "s"(d.v));
        if constexpr (ST == APEXW_STATE_Q8) asm volatile("" ::"s"(d.m_scale), "s"(d.v_scale));
        // no grad (absent, or the step is skipped): tensor untouched
        if (r.grad != nullptr && n > 0) {
            const auto s = [&] { return step_scalars(r); };
            if constexpr (ST == APEXW_STATE_F32)
                tile_dense<PT, GT, APEXW_F32, NT, SC>(d, r.grad, base, n, s);
            else if constexpr (ST == APEXW_STATE_BF16)
                tile_dense<PT, GT, APEXW_BF16, NT, SC>(d, r.grad, base, n, s);
            else
                tile_q8<PT, GT, NT, SC>(d, r.grad, base, n, s);
        }
        k += gridDim.x;
        if (k >= a.tile_count) break;
        i = tile_tensor[table_pos(a, k)];
    }
}

// The tensor of launch-relative tile k.  FEW (the loop-free kernels over a
// launch of at most kFewTensors tensors, none empty, with cached accesses --
// a small list, whose step is the latency of this chain): the last of the
// launch's tensors whose first tile is at or before k, by scalar compares
// on the kernel arguments.  Every bound and index sits at a constant offset,
// so they arrive with the other arguments in one round of loads and no
// memory round trip precedes the tile's metadata loads; the host repeats the
// last tensor in the unused entries, which then never change the result.  A
// separate kernel rather than a test of `few`: read unconditionally, the
// bounds cost launches of many tensors 1.8% (many-small list), and read
// after the test they take a second round.  Otherwise the tile table.
template <bool FEW>
__device__ __forceinline__ int32_t tile_owner(const KernelArgs &a, const APEXW_CONST int32_t *tile_tensor,
                                              int64_t k) {
    if constexpr (FEW) {
        // launch-relative tile indices fit 32 bits (lists have < 2^31 tiles)
        const int32_t k32 = (int32_t)k;
        int32_t t[kFewTensors];
#pragma unroll
        for (int u = 0; u < kFewTensors; ++u) {
            t[u] = a.few_tensor[u];
            // opaque to the optimizer: a choice between loaded values would
            // otherwise become one load at a chosen offset, a second round
            asm("" : "+s"(t[u]));
        }
        int32_t r = t[0];
#pragma unroll
        for (int u = 1; u < kFewTensors; ++u) r = k32 >= a.few_first[u] ? t[u] : r;
        return r;
    } else {
        return tile_tensor[table_pos(a, k)];
    }
}

// The carried step (launch mode 3): the whole step in one launch per dtype
// pair at any list size, with no prepare launch and no arrival counters.
// Every workgroup takes its tensor's bias corrections from bias_cur (formed
// for the counter as it stands, t + 1, by the previous step or by
// carry_init_kernel), its group's scalars from the kernel arguments and the
// flag and scale factors from device memory.  The first tile of each tensor
// alone advances the counter (only with a grad and without found_inf) and
// writes the corrections for the following step, at t + 2 or unchanged, into
// bias_next; no other workgroup uses the counter (every workgroup loads it
// with the metadata, only the first tile's value counts), so no ordering
// between workgroups is needed.  Results are bitwise those of the other
// modes: the same fp64 and fp32 operations form the same scalars.
//
// ONE: the grid has a workgroup per tile, so each takes exactly one tile and
// the body is straight-line code (no loop, so nothing is hoisted into a
// preheader that every wave would run for its one tile).
template <int ST, int PT, int GT, bool NT, bool SC, bool ONE = false, bool FEW = false>
__device__ __forceinline__ void carry_step(const KernelArgs &a) {
    static_assert(ONE || !FEW, "the few-tensor lookup is for the loop-free kernels");
    const APEXW_CONST int32_t *tile_tensor = cptr<int32_t>(a.tile_tensor);
    const float fi = *cptr<float>(a.found_inf);
    const float inv_scale = *cptr<float>(a.inv_scale);
    const float clip_coef = *cptr<float>(a.clip_coef);
    int64_t k = blockIdx.x;                    // < tile_count: grid <= tiles
    int32_t i = tile_owner<FEW>(a, tile_tensor, k);
    for (;;) {
        const TensorDesc d = load_uniform(a.desc, i);
        const void *g_ptr = reinterpret_cast<const void *>(cptr<uint64_t>(a.grads)[i]);
        const BiasRecord b = load_uniform(a.bias_cur, i);
        // the counter, read with the metadata (dense formats; only the first
        // tile of the tensor uses it, and writes it below, alone)
        const int32_t t_old = cptr<int32_t>(a.steps)[i];
        const int64_t base = (a.tile_begin + k - d.first_tile) * kTile;
        const int64_t left = d.numel - base;
        const int n = left < kTile ? (int)left : kTile;
        const bool first = base == 0;
        // the flag goes through the asm with the metadata: its test stays in
        // the loop, so its load completes with theirs instead of delaying the
        // first tile-table load
        float fl = fi;
        asm volatile("" : "+s"(fl) : "s"(g_ptr), "s"(d.param), "s"(d.m), "s"(d.v), "s"(d.group));
        if constexpr (ST == APEXW_STATE_Q8) asm volatile("" ::"s"(d.m_scale), "s"(d.v_scale));
        else asm volatile("" ::"s"(t_old));
        // no grad (absent, or the step is skipped): tensor untouched
        const void *grad = fl != 0.0f ? nullptr : g_ptr;
        BiasRecord nb = b;                     // a tensor that does not advance keeps them
        // (counter arithmetic wraps, as 32-bit unsigned: the corrections for
        // a step past the int32 maximum are formed ahead of time but only
        // used if such a step comes)
        const uint32_t t_new = (uint32_t)t_old + 1u;
        if (grad != nullptr && n > 0) {
            const auto s = [&] {
                const GroupScalars &G = a.groups[d.group];
                // dense formats: the first tile forms the next step's
                // corrections here, while the tile's loads are in flight (the
                // VALU-bound 8-bit update measured faster with them formed
                // after the tile, below)
                if constexpr (ST != APEXW_STATE_Q8)
                    if (first) nb = bias_record(G.beta1_d, G.beta2_d, (int32_t)(t_new + 1u));
                StepScalars r;
                r.beta1 = G.beta1;
                r.one_minus_beta1 = G.one_minus_beta1;
                r.beta2 = G.beta2;
                r.one_minus_beta2 = G.one_minus_beta2;
                r.lr = G.lr;
                r.decay = G.decay;
                r.eps = G.eps;
                r.bc1 = b.bc1;
                r.bc2 = b.bc2;
                r.rbc1 = b.rbc1;
                r.rbc2 = b.rbc2;
                r.div_lo = b.div_lo;
                r.x_lo = G.x_lo;
                r.inv_scale = inv_scale;
                r.clip_coef = clip_coef;
                return r;
            };
            if constexpr (ST == APEXW_STATE_F32)
                tile_dense<PT, GT, APEXW_F32, NT, SC>(d, grad, base, n, s);
            else if constexpr (ST == APEXW_STATE_BF16)
                tile_dense<PT, GT, APEXW_BF16, NT, SC>(d, grad, base, n, s);
            else
                tile_q8<PT, GT, NT, SC>(d, grad, base, n, s);
        }
        if (first && threadIdx.x == 0) {       // the tensor's first tile
            if constexpr (ST == APEXW_STATE_Q8) {
                if (grad != nullptr) {
                    const uint32_t t1 = (uint32_t)a.steps[i] + 1u;
                    a.steps[i] = (int32_t)t1;
                    const GroupScalars &G = a.groups[d.group];
                    nb = bias_record(G.beta1_d, G.beta2_d, (int32_t)(t1 + 1u));
                }
            } else if (grad != nullptr) {
                a.steps[i] = (int32_t)t_new;
            }
            a.bias_next[i] = nb;
        }
        if constexpr (ONE) break;
        k += gridDim.x;
        if (k >= a.tile_count) break;
        i = tile_owner<FEW>(a, tile_tensor, k);
    }
}

template <int ST, int PT, int GT, bool NT, bool SC, bool ONE, bool FEW>
__global__ __launch_bounds__(kThreads) void adamw_carry_step_kernel(KernelArgs a) {
    carry_step<ST, PT, GT, NT, SC, ONE, FEW>(a);
}

// The 8-bit carried step under a workgroup cap (a grid-stride loop over the
// tiles; uncapped launches take adamw_carry_pair_q8_kernel below).  Both
// 8-bit carried kernels run under a budget of 80 scalar registers (the
// compiler otherwise takes 93): the 8-bit update wants every wave the SIMDs
// can hold, and at 93 SGPRs the one-tile kernel measured 11% fewer waves in
// flight on MI355X, although the compiler counts 8 waves per SIMD either way,
// and ran 4-5% slower than at 78 (LoRA list, 53.7-54.5 against 51.3-51.8 us
// per step).  The dense formats keep their allocation (their residency is
// capped lower, and the budget's register moves cost bf16 moments 1%).
template <int PT, int GT, bool NT, bool SC>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_num_sgpr(80)))
void adamw_carry_step_q8_kernel(KernelArgs a) {
    carry_step<APEXW_STATE_Q8, PT, GT, NT, SC, false>(a);
}

// The step's scalars of a tile of tensor descriptor d in the carried step.
__device__ __forceinline__ StepScalars carry_scalars(const KernelArgs &a, const TensorDesc &d,
                                                     const BiasRecord &b, float inv_scale,
                                                     float clip_coef) {
    const GroupScalars &G = a.groups[d.group];
    StepScalars r;
    r.beta1 = G.beta1;
    r.one_minus_beta1 = G.one_minus_beta1;
    r.beta2 = G.beta2;
    r.one_minus_beta2 = G.one_minus_beta2;
    r.lr = G.lr;
    r.decay = G.decay;
    r.eps = G.eps;
    r.bc1 = b.bc1;
    r.bc2 = b.bc2;
    r.rbc1 = b.rbc1;
    r.rbc2 = b.rbc2;
    r.div_lo = b.div_lo;
    r.x_lo = G.x_lo;
    r.inv_scale = inv_scale;
    r.clip_coef = clip_coef;
    return r;
}

// After the tile at `base` of tensor i (8-bit carried step): if it is the
// tensor's first, advance the counter (with a grad) and write the next
// step's corrections, after the tile.
__device__ __forceinline__ void carry_first_tile_q8(const KernelArgs &a, int32_t i,
                                                    const TensorDesc &d, const BiasRecord &b,
                                                    int64_t base, const void *grad) {
    if (base != 0 || threadIdx.x != 0) return;
    BiasRecord nb = b;
    if (grad != nullptr) {
        const uint32_t t1 = (uint32_t)a.steps[i] + 1u;
        a.steps[i] = (int32_t)t1;
        const GroupScalars &G = a.groups[d.group];
        nb = bias_record(G.beta1_d, G.beta2_d, (int32_t)(t1 + 1u));
    }
    a.bias_next[i] = nb;
}

// The 8-bit carried step with two tiles per workgroup: workgroup w takes the
// logical tiles 2p and 2p+1 of its pair p (q8_pair_of_workgroup: runs of 16
// consecutive pairs per XCD, so that one L2 holds their scale lines).  When
// both lie in one tensor (every pair but at most one per tensor) they are
// consecutive blocks, and one metadata fetch, one address computation and
// one set of scalars serve both (q8_pair_full for two full blocks); a pair
// that spans two tensors takes its tiles one at a time, as carry_step does.
// Each block gets the same bits as with one tile per workgroup; the step
// measured 3.5% faster on MI355X (LoRA list, 43.8-44.0 against 45.4-45.8 us,
// same machine, alternating runs): the same VALU work per block, half the
// metadata chains and scalar work.
template <int PT, int GT, bool NT, bool SC, bool FEW>
__device__ __forceinline__ void carry_q8_one_tile(const KernelArgs &a,
                                                  const APEXW_CONST int32_t *tile_tensor,
                                                  int64_t k, float fi, float inv_scale,
                                                  float clip_coef) {
    const int32_t i = tile_owner<FEW>(a, tile_tensor, k);
    const TensorDesc d = load_uniform(a.desc, i);
    const void *g_ptr = reinterpret_cast<const void *>(cptr<uint64_t>(a.grads)[i]);
    const BiasRecord b = load_uniform(a.bias_cur, i);
    const int64_t base = (a.tile_begin + k - d.first_tile) * kTile;
    const int64_t left = d.numel - base;
    const int n = left < kTile ? (int)left : kTile;
    const void *grad = fi != 0.0f ? nullptr : g_ptr;
    if (grad != nullptr && n > 0)
        tile_q8<PT, GT, NT, SC>(d, grad, base, n,
                                [&] { return carry_scalars(a, d, b, inv_scale, clip_coef); });
    carry_first_tile_q8(a, i, d, b, base, grad);
}

template <int PT, int GT, bool NT, bool SC, bool FEW>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_num_sgpr(80)))
void adamw_carry_pair_q8_kernel(KernelArgs a) {
    const APEXW_CONST int32_t *tile_tensor = cptr<int32_t>(a.tile_tensor);
    const float fi = *cptr<float>(a.found_inf);
    const float inv_scale = *cptr<float>(a.inv_scale);
    const float clip_coef = *cptr<float>(a.clip_coef);
    // a permutation of the grid: k0 < tile_count, grid = ceil(tiles / 2)
    const int64_t k0 = 2 * (int64_t)q8_pair_of_workgroup(blockIdx.x, gridDim.x);
    const int32_t i = tile_owner<FEW>(a, tile_tensor, k0);
    const TensorDesc d = load_uniform(a.desc, i);
    const void *g_ptr = reinterpret_cast<const void *>(cptr<uint64_t>(a.grads)[i]);
    const BiasRecord b = load_uniform(a.bias_cur, i);
    const int64_t base = (a.tile_begin + k0 - d.first_tile) * kTile;
    const int64_t left = d.numel - base;
    if (left <= kTile) {                       // tile k0 ends its tensor: one tile at a time
        carry_q8_one_tile<PT, GT, NT, SC, FEW>(a, tile_tensor, k0, fi, inv_scale, clip_coef);
        if (k0 + 1 < a.tile_count)
            carry_q8_one_tile<PT, GT, NT, SC, FEW>(a, tile_tensor, k0 + 1, fi, inv_scale, clip_coef);
        return;
    }
    const void *grad = fi != 0.0f ? nullptr : g_ptr;
    if (grad != nullptr) {
        const StepScalars s = carry_scalars(a, d, b, inv_scale, clip_coef);
        if (left >= 2 * kTile) {
            q8_pair_full<PT, GT, NT, SC>(d, grad, base, s);
        } else {
            tile_q8<PT, GT, NT, SC>(d, grad, base, kTile, [&] { return s; });
            tile_q8<PT, GT, NT, SC>(d, grad, base + kTile, (int)(left - kTile), [&] { return s; });
        }
    }
    carry_first_tile_q8(a, i, d, b, base, grad);
}

// Starts (or restarts) the carried chain: one lane per tensor writes the
// bias corrections for its counter as it stands, t + 1, into bias_next.
__global__ __launch_bounds__(kPrepThreads) void carry_init_kernel(KernelArgs a) {
    const int32_t i = blockIdx.x * kPrepThreads + threadIdx.x;
    if (i >= a.n_tensors) return;
    const uint32_t t = (uint32_t)a.steps[i];
    const GroupScalars &G = a.groups[a.desc[i].group];
    a.bias_next[i] = bias_record(G.beta1_d, G.beta2_d, (int32_t)(t + 1u));
}

// Arrival counters of the single-launch step, per launch: kDoneFan
// first-level counters and one top counter, each alone in a 128-byte line
// (kDoneStride words apart).  Workgroup b arrives at counter b % kDoneFan;
// the last to arrive there clears it and arrives at the top counter; the last
// to arrive at the top has seen every workgroup arrive.  One counter for the
// whole grid would serialise one atomic per workgroup on one address.
constexpr int kDoneFan = 64;
constexpr int kDoneStride = 32;
constexpr int kDoneWords = (kDoneFan + 1) * kDoneStride;

// An arrival at a counter that expects `expected` arrivals per launch: a
// device-scope wrapping increment by lane 0 (the counter goes back to 0 on the
// last arrival, ready for the next launch), returning the count before it
// (0 in the other lanes).  Only a read-before-write order matters here (every
// counter read, then the advance); no data written before the increment is
// read after it in this launch, so no cache write-back is needed.
__device__ __forceinline__ uint32_t arrive(uint32_t *ctr, uint32_t expected) {
    uint32_t before = 0;
    if (threadIdx.x == 0) before = __builtin_amdgcn_atomic_inc32(ctr, expected - 1u, __ATOMIC_RELAXED, "agent");
    return before;
}

// True in every lane of the wave whose arrival was the last of `expected`.
__device__ __forceinline__ bool arrived_last(uint32_t before, uint32_t expected) {
    return (uint32_t)__builtin_amdgcn_readfirstlane((int)before) == expected - 1u;
}

// The whole step in one launch per dtype pair, for lists of few tiles (where
// the prepare launch costs about as much as the work): every workgroup forms
// its tensor's step record itself from the counter as it stands (t + 1), and
// the workgroup that arrives last -- after every workgroup has read the
// counters -- advances the counters of the launch's tensors that had a grad.
// A workgroup arrives at its first-level counter as soon as it has read its
// last counter, so that add's latency hides under the tile's loads; the
// first-level winners arrive at the top after their tiles.  Results are
// bitwise those of the two-kernel step.
template <int ST, int PT, int GT, bool SC>
__global__ __launch_bounds__(kThreads) void adamw_single_step_kernel(KernelArgs a) {
    const APEXW_CONST int32_t *tile_tensor = cptr<int32_t>(a.tile_tensor);
    const float fi = *cptr<float>(a.found_inf);
    const float inv_scale = *cptr<float>(a.inv_scale);
    const float clip_coef = *cptr<float>(a.clip_coef);
    const uint32_t grid = gridDim.x, c = blockIdx.x % kDoneFan;
    const uint32_t first_level = (grid - 1u - c) / kDoneFan + 1u;      // workgroups b % kDoneFan == c
    const uint32_t top_level = grid < (uint32_t)kDoneFan ? grid : (uint32_t)kDoneFan;
    uint32_t *const top = a.done + kDoneFan * kDoneStride;
    uint32_t before = 0, before_top = 0;
    bool checked = false, last1 = false;       // first-level result, once read
    int64_t k = blockIdx.x;                    // < tile_count: grid <= tiles
    for (;;) {
        const int32_t i = tile_tensor[table_pos(a, k)];
        const TensorDesc d = load_uniform(a.desc, i);
        const void *grad = reinterpret_cast<const void *>(cptr<uint64_t>(a.grads)[i]);
        const int32_t t_old = cptr<int32_t>(a.steps)[i];
        const bool last_tile = k + grid >= a.tile_count;
        if (last_tile) {
            // the counter read has returned before the add is issued: the
            // empty asm reads the loaded value
            asm volatile("" ::"s"(t_old) : "memory");
            before = arrive(a.done + c * kDoneStride, first_level);
        }
        const int64_t base = (a.tile_begin + k - d.first_tile) * kTile;
        const int64_t left = d.numel - base;
        const int n = left < kTile ? (int)left : kTile;
        if (fi == 0.0f && grad != nullptr && n > 0) {
            const auto s = [&] {
                // read the add's result here, once the tile's loads are in
                // flight (it was issued before them and returns first), not
                // after the stores, which would wait for them too; a
                // first-level winner arrives at the top right away, so that
                // add too overlaps the tile's work
                if (last_tile) {
                    last1 = arrived_last(before, first_level);
                    checked = true;
                    if (last1) before_top = arrive(top, top_level);
                }
                return step_scalars(step_record(a, d.group, grad, t_old + 1, inv_scale, clip_coef));
            };
            if constexpr (ST == APEXW_STATE_F32)
                tile_dense<PT, GT, APEXW_F32, false, SC>(d, grad, base, n, s);
            else if constexpr (ST == APEXW_STATE_BF16)
                tile_dense<PT, GT, APEXW_BF16, false, SC>(d, grad, base, n, s);
            else
                tile_q8<PT, GT, false, SC>(d, grad, base, n, s);
        }
        if (last_tile) break;
        k += grid;
    }
    if (!checked) {
        last1 = arrived_last(before, first_level);
        if (last1) before_top = arrive(top, top_level);
    }
    if (!last1 || !arrived_last(before_top, top_level)) return;
    if (fi != 0.0f) return;                    // a skipped step advances nothing
    for (int32_t j = threadIdx.x; j < a.tensor_count; j += kThreads) {
        const int32_t i = a.tensor_list[a.tensor_begin + j];
        const int32_t t = a.steps[i];
        const void *grad = a.grads[i];
        asm volatile("" ::"v"(t), "v"(grad));   // both loads in one round trip
        if (grad != nullptr) a.steps[i] = t + 1;
    }
}

// Mixed-precision recipe before the update (M041 section 06; Apex guide
// 4.3): unscale every present grad by inv_scale and set *found_inf_out to 1
// if any unscaled value is an infinity or a NaN.  The flag is only ever set
// (the caller clears it), by plain stores of the same value; grads are not
// rewritten -- the update applies inv_scale itself.  One wave per tile, the
// tiles of one (param, grad) dtype launch.
// The read passes below take their tiles in groups of kReadBatch (the plan's
// read_window): group j is XCD stripe x = j % 8 of the launch's tile table,
// entries 4c .. 4c+3 with c = j / 8, i.e. the logical tiles x + 8(4c + u),
// u = 0..3.  Its four table entries are one 16-byte load, then the four grad
// pointers and descriptor fields are fetched together, then every grad load
// of the group is issued before any is used, so one wave keeps four tiles in
// flight.  What each tile contributes does not depend on the grouping.

// A tile of a read group: grad (nullptr: absent), first element, valid
// length (0 for a tile past the launch end), logical tile index, position in
// the tile table.
struct ReadTile {
    const void *grad;
    int64_t base;
    int n;
    int64_t k;
    int64_t pos;
};

// The tiles of group j; false if the group starts past the launch end.  The
// 16-byte table load may reach 3 entries past a stripe's end (the table
// allocation is padded for it); such entries are never used.
__device__ __forceinline__ bool read_group(const KernelArgs &a, int64_t j,
                                           ReadTile (&t)[kReadBatch]) {
    const ReadWindow w = read_window(a.table_begin, a.table_stride, j);
    const int64_t k0 = w.k0;
    if (k0 >= a.tile_count) return false;
    const int64_t pos0 = w.pos0;
    const APEXW_CONST int32_t *row = cptr<int32_t>(a.tile_tensor) + pos0;
    int32_t ti[kReadBatch];
#pragma unroll
    for (int u = 0; u < kReadBatch; ++u) ti[u] = row[u];
#pragma unroll
    for (int u = 0; u < kReadBatch; ++u) {
        t[u].k = k0 + (int64_t)kXcds * u;
        t[u].pos = pos0 + u;
        const bool live = t[u].k < a.tile_count;
        const int32_t i = live ? ti[u] : ti[0];
        const APEXW_CONST int64_t *dd = cptr<int64_t>(&a.desc[i].numel);   // numel, first_tile
        t[u].grad = reinterpret_cast<const void *>(cptr<uint64_t>(a.grads)[i]);
        t[u].base = (a.tile_begin + (live ? t[u].k : k0) - dd[1]) * kTile;
        const int64_t left = dd[0] - t[u].base;
        t[u].n = !live ? 0 : left < kTile ? (int)left : kTile;
    }
    return true;
}

// The lane's 4 grad values of a tile (0 where absent or past the end).
template <int GT, bool NT>
__device__ __forceinline__ void load_tile_grads(const ReadTile &t, float (&g)[kVec]) {
    const int off = threadIdx.x * kVec;
    if (t.grad != nullptr && off + kVec <= t.n) {
        load4_any<GT, NT>(t.grad, t.base + off, g, vec_aligned<GT>(t.grad));
    } else {
#pragma unroll
        for (int j = 0; j < kVec; ++j)
            g[j] = t.grad != nullptr && off + j < t.n ? load1<GT>(t.grad, t.base + off + j) : 0.0f;
    }
}

// The grads of a read group.  When all four tiles are full, present and
// vector-aligned (the common case; a wave-uniform test) their four vector
// loads are issued back to back in straight-line code; the general path
// chooses per lane between vector and element loads, and there the compiler
// waits for every load in flight before each tile's loads, which would
// serialise the tiles of the group.
template <int GT, bool NT>
__device__ __forceinline__ void load_group_grads(const ReadTile (&t)[kReadBatch],
                                                 float (&g)[kReadBatch][kVec]) {
    bool full = true;
#pragma unroll
    for (int u = 0; u < kReadBatch; ++u)
        full = full && t[u].grad != nullptr && t[u].n == kTile && vec_aligned<GT>(t[u].grad);
    if (full) {
#pragma unroll
        for (int u = 0; u < kReadBatch; ++u)
            load4<GT, NT>(t[u].grad, t[u].base + threadIdx.x * kVec, g[u]);
    } else {
#pragma unroll
        for (int u = 0; u < kReadBatch; ++u) load_tile_grads<GT, NT>(t[u], g[u]);
    }
}

template <int GT, bool NT>
__global__ __launch_bounds__(kThreads) void unscale_check_kernel(KernelArgs a) {
    const float inv = a.inv_scale != nullptr ? *a.inv_scale : 1.0f;
    const int64_t groups = read_groups(a.table_stride);
    const int off = threadIdx.x * kVec;
    bool bad = false;
    for (int64_t jg = blockIdx.x; jg < groups; jg += gridDim.x) {
        ReadTile t[kReadBatch];
        float g[kReadBatch][kVec];
        if (!read_group(a, jg, t)) continue;
        load_group_grads<GT, NT>(t, g);
#pragma unroll
        for (int u = 0; u < kReadBatch; ++u)
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const float x = g[u][j] * inv;
                bad |= t[u].grad != nullptr && off + j < t[u].n && !(fabsf(x) <= 3.40282347e38f);
            }
    }
    if (wave_any(bad) && threadIdx.x == 0) *gptr<float>(static_cast<void *>(a.found_inf_out)) = 1.0f;
}

// ---------------------------------------------------------------- grad norm
//
// Global grad-norm clipping (the clip step of the M041 section 06 recipe):
// the norm of all present unscaled grads u = g * inv_scale (fp32, as the
// update uses them), squares and sums in fp64, reduced in a fixed order so
// the result does not depend on scheduling:
//  1. grad_norm_partials_kernel: the squares of each read group (four tiles
//     fixed by the tile table alone, not by the grid) are summed by one wave
//     -- per lane over the group's tiles in order, then wave_sum's fixed
//     order -- into partials[group_begin + j] for group j of the launch (the
//     launches' groups one after another, so consecutive groups fill whole
//     64-byte lines; a group that starts past its launch's end writes 0, so
//     every entry is written on every call); tiles without a grad contribute 0;
//     optionally sets found_inf_out like the unscale check;
//  2. grad_norm_reduce_kernel: workgroup b sums partials[b*C .. (b+1)*C) with
//     a strided loop and a tree in LDS into partials2[b];
//  3. grad_norm_final_kernel: one workgroup sums partials2 the same way and
//     writes the norm (fp64 sqrt) and the clip coefficient max_norm / norm
//     when norm > max_norm (fp64, rounded once to fp32), else 1.
//  For a list of at most kDirectPartials partials (one launch less for a
//  small list) step 2 is left out and step 3 sums the partials themselves.

// DPP move of a double (both halves) within 16-lane rows.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
    const int lo = __builtin_amdgcn_update_dpp(0, __double2loint(x), CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp(0, __double2hiint(x), CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double lane_f64(double x, int lane) {
    return __hiloint2double(__builtin_amdgcn_readlane(__double2hiint(x), lane),
                            __builtin_amdgcn_readlane(__double2loint(x), lane));
}

// Sum over the 64 lanes, the same value in every lane, in a fixed order:
// within each 16-lane row pairs at distance 1 and 2 (quad swaps), then the
// two quads of each half-row and the two half-rows (mirrors) -- each lane
// adds its partner's partial, and a + b == b + a, so the row's lanes agree
// bit for bit -- then (row0 + row1) + (row2 + row3).
__device__ __forceinline__ double wave_sum(double x) {
    x = x + dpp_f64<0xB1>(x);     // quad_perm [1,0,3,2]
    x = x + dpp_f64<0x4E>(x);     // quad_perm [2,3,0,1]
    x = x + dpp_f64<0x141>(x);    // row_half_mirror
    x = x + dpp_f64<0x140>(x);    // row_mirror
    return (lane_f64(x, 0) + lane_f64(x, 16)) + (lane_f64(x, 32) + lane_f64(x, 48));
}

template <int GT, bool NT>
__global__ __launch_bounds__(kThreads) void grad_norm_partials_kernel(KernelArgs a) {
    const float inv = a.inv_scale != nullptr ? *a.inv_scale : 1.0f;
    const int64_t groups = read_groups(a.table_stride);
    const int off = threadIdx.x * kVec;
    bool bad = false;
    for (int64_t jg = blockIdx.x; jg < groups; jg += gridDim.x) {
        ReadTile t[kReadBatch];
        float g[kReadBatch][kVec];
        if (!read_group(a, jg, t)) {      // starts past the launch end: contributes 0
            if (threadIdx.x == 0) gptr<double>(static_cast<void *>(a.partials))[a.group_begin + jg] = 0.0;
            continue;
        }
        load_group_grads<GT, NT>(t, g);
        double sq = 0.0;                  // the group's tiles in order, each lane's 4 values
#pragma unroll
        for (int u = 0; u < kReadBatch; ++u) {
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                const float x = g[u][j] * inv;
                if (t[u].grad != nullptr && off + j < t[u].n) {
                    bad |= !(fabsf(x) <= 3.40282347e38f);
                    sq = sq + (double)x * (double)x;
                }
            }
        }
        sq = wave_sum(sq);
        if (threadIdx.x == 0) gptr<double>(static_cast<void *>(a.partials))[a.group_begin + jg] = sq;
    }
    if (a.found_inf_out != nullptr && wave_any(bad) && threadIdx.x == 0)
        *gptr<float>(static_cast<void *>(a.found_inf_out)) = 1.0f;
}

constexpr int kReduceThreads = 256;
constexpr int kReduceBlocks = 256;
constexpr int64_t kDirectPartials = 8192;

// Fixed-order sum of src[lo, hi) by one workgroup: strided per thread, then a
// tree over the workgroup's threads in LDS.
__device__ __forceinline__ double block_sum(const double *src, int64_t lo, int64_t hi) {
    __shared__ double buf[kReduceThreads];
    double acc = 0.0;
    for (int64_t j = lo + threadIdx.x; j < hi; j += kReduceThreads)
        acc = acc + gptr<double>(static_cast<const void *>(src))[j];
    buf[threadIdx.x] = acc;
    __syncthreads();
    for (int w = kReduceThreads / 2; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) buf[threadIdx.x] = buf[threadIdx.x] + buf[threadIdx.x + w];
        __syncthreads();
    }
    return buf[0];
}

__global__ __launch_bounds__(kReduceThreads) void grad_norm_reduce_kernel(KernelArgs a) {
    const int64_t chunk = (a.n_partials + kReduceBlocks - 1) / kReduceBlocks;
    const int64_t lo = (int64_t)blockIdx.x * chunk;
    const int64_t hi = lo + chunk < a.n_partials ? lo + chunk : a.n_partials;
    const double sum = block_sum(a.partials, lo, hi > lo ? hi : lo);
    if (threadIdx.x == 0) gptr<double>(static_cast<void *>(a.partials2))[blockIdx.x] = sum;
}

__global__ __launch_bounds__(kReduceThreads) void grad_norm_final_kernel(KernelArgs a) {
    // after the reduce kernel: its kReduceBlocks sums; for few partials (no
    // reduce launch) the partials themselves; none at all (an empty tensor
    // list): the norm is 0
    const double sum = a.partials2 != nullptr ? block_sum(a.partials2, 0, kReduceBlocks)
                       : a.partials != nullptr ? block_sum(a.partials, 0, a.n_partials)
                                               : 0.0;
    if (threadIdx.x == 0) {
        const double norm = sqrt(sum);
        const float coef = norm > a.max_norm ? (float)(a.max_norm / norm) : 1.0f;
        if (a.norm_out != nullptr) *gptr<double>(static_cast<void *>(a.norm_out)) = norm;
        *gptr<float>(static_cast<void *>(a.clip_out)) = coef;
    }
}

// The inverse of a loss scale, formed the way the Apex fused-optimizer guide
// (section 4.3) forms the factor it hands to its kernel: the fp64 reciprocal
// of the scale, rounded once to fp32.
__global__ __launch_bounds__(kThreads) void inv_scale_kernel(const float *scale, float *inv) {
    if (threadIdx.x == 0) {
        const double s = (double)*gptr<float>(static_cast<const void *>(scale));
        *gptr<float>(static_cast<void *>(inv)) = (float)(1.0 / s);
    }
}

// Zero fill of the state buffer (used once, at creation).
__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t *p, int64_t n_words) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n_words;
         i += (int64_t)gridDim.x * 256)
        p[i] = 0u;
}

}  // namespace apexw
