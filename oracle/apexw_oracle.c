/*
 * apexw_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, scalar CPU definition of one fused multi-tensor AdamW step
 * with decoupled weight decay, scalar bias correction and fp32, bf16 or
 * blockwise-absmax 8-bit moment storage.  It exists to check the HIP library
 * against; only the tests, the package smoke check and the benchmark's CPU
 * baseline may load it.  It shares no code, header or constant with the HIP
 * path, and the product never calls it.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC (every fp32
 * operation below is a separately rounded IEEE operation; no FMA contraction).
 * That single-threaded build is the one the parity tests use.  The same
 * source built with -fopenmp in addition is a timing build for the host
 * baseline: the two "omp parallel for" loops below then split a tensor's
 * elements (or 8-bit blocks) over threads.  Every element and every block is
 * computed by the same operations either way, so the results are the same
 * bit for bit (a test checks it).
 *
 * Sources (cited by page title and section):
 *   [M041 §NN]  "Fused optimizers and state precision: optimize the reads and
 *               writes of the update separately from the state"
 *               (xuujii.github.io ai-infra-kb, item M041), section NN.
 *   [Apex §N]   "Apex fused optimizers" guide (qwbw.cn news 83927), section N.
 *   [Unsloth]   "ApexW optimizer measured in Unsloth: ties 8-bit AdamW with
 *               lower memory" (kongchang.com), results section.
 *
 * Readings of points the pages leave open (each is listed in the design
 * notes of the repository):
 *   R1  Arithmetic is fp32 with every operation separately rounded.  The
 *       update box of [M041 §02] is written in Python, and its own operator
 *       rules fix the order: equal-precedence operators group from the left
 *       and products and quotients bind tighter than sums.  So the new v adds
 *       beta2*v to ((1-beta2)*g)*g, and the step of theta is the product
 *       lr*m_hat divided by (sqrt(v_hat)+eps), subtracted from
 *       theta*(1-lr*wd).  No multiply-add is contracted.
 *   R2  Scalar coefficients (1-beta1), (1-beta2), (1-lr*wd), lr, eps, beta1,
 *       beta2 are formed in fp64 from the fp64 hyperparameters and rounded
 *       once to fp32.  beta^t is fp64 square-and-multiply over the bits of t
 *       from the least significant end; 1-beta^t is formed in fp64 and rounded
 *       once to fp32.
 *   R3  One int32 step counter per tensor; a tensor whose grad is absent does
 *       not advance it [M041 §03]; a found_inf step changes nothing at all
 *       [M041 §06], [Apex §4.3].
 *   R4  bf16 values are widened exactly and narrowed round-to-nearest-even.
 *   R5  8-bit state: blocks of 256 consecutive elements of one tensor from
 *       element 0 (a final partial block has its own scale); m is signed with
 *       scale absmax|m|/127, v unsigned with scale max(v)/255, codes are
 *       round-half-even of x/scale, an all-zero block has scale 0 and codes 0
 *       [M041 §05].  Decoding is code*scale.  The update of theta uses the
 *       fp32 moments of this step; re-encoding only affects what is stored.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

#define ORACLE_STATE_F32 0
#define ORACLE_STATE_BF16 1
#define ORACLE_STATE_Q8 2

#define ORACLE_BLOCK 256

typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
} oracle_group;

/* Threads the element loops use: 1 in the parity build, the OpenMP team
 * size in the timing build. */
#ifdef _OPENMP
#include <omp.h>
int32_t oracle_threads(void) { return (int32_t)omp_get_max_threads(); }
#else
int32_t oracle_threads(void) { return 1; }
#endif

/* ------------------------------------------------------------ conversions */

float oracle_bf16_to_f32(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* R4: nearest bf16, ties to the even significand. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u)          /* NaN stays a quiet NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7fffu + keep_lsb;
    return (uint16_t)(u >> 16);
}

void oracle_f32_to_bf16_array(int64_t n, const float *x, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_f32_to_bf16(x[i]);
}

/* R2: beta^e by square-and-multiply in fp64. */
double oracle_pow_int(double base, int32_t e)
{
    double result = 1.0;
    double b = base;
    uint32_t n = (uint32_t)e;
    while (n != 0u) {
        if (n & 1u)
            result = result * b;
        b = b * b;
        n >>= 1;
    }
    return result;
}

/* ------------------------------------------------------------ quantizer */

/* [M041 §05] block quantizer for a signed moment: the block's scale is its
 * largest magnitude over 127, each code is the value over the scale rounded
 * half to even (clamped to +-127), and decoding multiplies code by scale.  A
 * block whose values are all zero gets scale 0 and codes 0, the case the
 * section says is handled on its own. */
void oracle_quantize_signed(int64_t n, const float *x, int8_t *q, float *scale)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (a > amax)
            amax = a;
    }
    float s = amax / 127.0f;
    *scale = s;
    for (int64_t i = 0; i < n; ++i) {
        if (s == 0.0f) {
            q[i] = 0;
            continue;
        }
        float r = nearbyintf(x[i] / s);      /* default mode: half to even */
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[i] = (int8_t)r;
    }
}

/* R5: the same construction for the non-negative second moment, using the
 * full unsigned 8-bit range. */
void oracle_quantize_unsigned(int64_t n, const float *x, uint8_t *q, float *scale)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        if (x[i] > amax)
            amax = x[i];
    }
    float s = amax / 255.0f;
    *scale = s;
    for (int64_t i = 0; i < n; ++i) {
        if (s == 0.0f) {
            q[i] = 0;
            continue;
        }
        float r = nearbyintf(x[i] / s);
        if (r > 255.0f) r = 255.0f;
        if (r < 0.0f) r = 0.0f;
        q[i] = (uint8_t)r;
    }
}

void oracle_dequantize_signed(int64_t n, const int8_t *q, float scale, float *x)
{
    for (int64_t i = 0; i < n; ++i)
        x[i] = (float)q[i] * scale;
}

void oracle_dequantize_unsigned(int64_t n, const uint8_t *q, float scale, float *x)
{
    for (int64_t i = 0; i < n; ++i)
        x[i] = (float)q[i] * scale;
}

/* ------------------------------------------------------------ the update */

typedef struct {
    float beta1, one_minus_beta1, beta2, one_minus_beta2;
    float lr, decay, eps;
    float bc1, bc2;              /* 1 - beta1^t, 1 - beta2^t */
} step_scalars;

/* R2: the per-tensor scalars of one step at (already advanced) count t. */
static step_scalars make_scalars(const oracle_group *g, int32_t t)
{
    step_scalars s;
    s.beta1 = (float)g->beta1;
    s.one_minus_beta1 = (float)(1.0 - g->beta1);
    s.beta2 = (float)g->beta2;
    s.one_minus_beta2 = (float)(1.0 - g->beta2);
    s.lr = (float)g->lr;
    s.decay = (float)(1.0 - g->lr * g->weight_decay);
    s.eps = (float)g->eps;
    s.bc1 = (float)(1.0 - oracle_pow_int(g->beta1, t));
    s.bc2 = (float)(1.0 - oracle_pow_int(g->beta2, t));
    return s;
}

/* [M041 §02] one element, R1 order. */
static void adamw_element(float *theta, float g, float *m, float *v,
                          const step_scalars *s)
{
    float m_new = s->beta1 * (*m) + s->one_minus_beta1 * g;
    float v_new = s->beta2 * (*v) + (s->one_minus_beta2 * g) * g;
    float m_hat = m_new / s->bc1;
    float v_hat = v_new / s->bc2;
    float denom = sqrtf(v_hat) + s->eps;
    float th = (*theta) * s->decay - (s->lr * m_hat) / denom;
    *m = m_new;
    *v = v_new;
    *theta = th;
}

static float load_value(int32_t dtype, const void *base, int64_t i)
{
    if (dtype == ORACLE_BF16)
        return oracle_bf16_to_f32(((const uint16_t *)base)[i]);
    return ((const float *)base)[i];
}

static void store_value(int32_t dtype, void *base, int64_t i, float x)
{
    if (dtype == ORACLE_BF16)
        ((uint16_t *)base)[i] = oracle_f32_to_bf16(x);
    else
        ((float *)base)[i] = x;
}

static void update_tensor_dense(int64_t n, int32_t pdt, void *theta,
                                int32_t gdt, const void *grad, int32_t sdt,
                                void *m, void *v, const step_scalars *s,
                                float inv_scale, float clip_coef)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        float th = load_value(pdt, theta, i);
        float g = (load_value(gdt, grad, i) * inv_scale) * clip_coef;
        float mi = load_value(sdt, m, i);
        float vi = load_value(sdt, v, i);
        adamw_element(&th, g, &mi, &vi, s);
        store_value(pdt, theta, i, th);
        store_value(sdt, m, i, mi);
        store_value(sdt, v, i, vi);
    }
}

/* R5: decode a block, update it, re-encode it. */
static void update_tensor_q8(int64_t n, int32_t pdt, void *theta, int32_t gdt,
                             const void *grad, int8_t *mq, uint8_t *vq,
                             float *ms, float *vs, const step_scalars *s,
                             float inv_scale, float clip_coef)
{
    int64_t nblocks = (n + ORACLE_BLOCK - 1) / ORACLE_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t b = 0; b < nblocks; ++b) {
        float mf[ORACLE_BLOCK], vf[ORACLE_BLOCK];
        int64_t lo = b * ORACLE_BLOCK;
        int64_t len = n - lo < ORACLE_BLOCK ? n - lo : ORACLE_BLOCK;
        oracle_dequantize_signed(len, mq + lo, ms[b], mf);
        oracle_dequantize_unsigned(len, vq + lo, vs[b], vf);
        for (int64_t j = 0; j < len; ++j) {
            float th = load_value(pdt, theta, lo + j);
            float g = (load_value(gdt, grad, lo + j) * inv_scale) * clip_coef;
            adamw_element(&th, g, &mf[j], &vf[j], s);
            store_value(pdt, theta, lo + j, th);
        }
        oracle_quantize_signed(len, mf, mq + lo, &ms[b]);
        oracle_quantize_unsigned(len, vf, vq + lo, &vs[b]);
    }
}

/*
 * Mixed-precision recipe step before the update ([M041 §06]; [Apex §4.3]):
 * the grads are unscaled by inv_scale (one rounded fp32 multiply per element)
 * and checked for non-finite values.  Returns 1 if any unscaled value of any
 * present grad is an infinity or a NaN, else 0.
 */
int32_t oracle_unscale_check(int32_t n_tensors, const int64_t *numel,
                             const int32_t *grad_dtype, const void *const *grad,
                             float inv_scale)
{
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (grad[i] == NULL)
            continue;
        for (int64_t e = 0; e < numel[i]; ++e) {
            float g = load_value(grad_dtype[i], grad[i], e) * inv_scale;
            if (isnan(g) || isinf(g))
                return 1;
        }
    }
    return 0;
}

/*
 * One optimizer step over a tensor list, on unscaled grads g * inv_scale
 * (inv_scale = 1 is the plain step: multiplying by one is exact).
 *
 *   theta[i]      parameter values, fp32 or bf16 bits (param_dtype[i])
 *   grad[i]       gradient values, fp32 or bf16 bits, or NULL for "no grad"
 *   m[i], v[i]    state: fp32, bf16 bits, or int8 / uint8 codes (state_fmt)
 *   m_scale[i], v_scale[i]  per-256-block fp32 scales (8-bit state only)
 *   t[i]          int32 step counter per tensor
 *   inv_scale     fp32 factor applied to every grad value first
 *   found_inf     nonzero: the whole step is skipped, nothing is written
 *
 * Returns 0, or -1 on an argument it does not understand.
 */
int oracle_adamw_step_clipped(int32_t n_tensors, const int64_t *numel,
                              const int32_t *param_dtype, void *const *theta,
                              const int32_t *grad_dtype, const void *const *grad,
                              const int32_t *group_of, const oracle_group *groups,
                              int32_t n_groups, int32_t state_fmt, void *const *m,
                              void *const *v, float *const *m_scale,
                              float *const *v_scale, int32_t *t, float inv_scale,
                              float clip_coef, int32_t found_inf);

int oracle_adamw_step_scaled(int32_t n_tensors, const int64_t *numel,
                             const int32_t *param_dtype, void *const *theta,
                             const int32_t *grad_dtype, const void *const *grad,
                             const int32_t *group_of, const oracle_group *groups,
                             int32_t n_groups, int32_t state_fmt, void *const *m,
                             void *const *v, float *const *m_scale,
                             float *const *v_scale, int32_t *t, float inv_scale,
                             int32_t found_inf)
{
    return oracle_adamw_step_clipped(n_tensors, numel, param_dtype, theta,
                                     grad_dtype, grad, group_of, groups, n_groups,
                                     state_fmt, m, v, m_scale, v_scale, t,
                                     inv_scale, 1.0f, found_inf);
}

/*
 * Global grad-norm clipping, the step the recipe of [M041 §06] places after
 * the finite check (the pages name it but give no formula; reading: the
 * plain one).  The norm is the Euclidean norm of all present unscaled grads,
 * u = g * inv_scale rounded to fp32 as the update uses it, each square and
 * the running sum in fp64, the square root in fp64.
 */
double oracle_grad_norm(int32_t n_tensors, const int64_t *numel,
                        const int32_t *grad_dtype, const void *const *grad,
                        float inv_scale)
{
    double sum = 0.0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (grad[i] == NULL)
            continue;
        for (int64_t e = 0; e < numel[i]; ++e) {
            double u = (double)(load_value(grad_dtype[i], grad[i], e) * inv_scale);
            sum = sum + u * u;
        }
    }
    return sqrt(sum);
}

/* Clip coefficient: max_norm / norm when the norm exceeds max_norm (fp64,
 * rounded once to fp32), else 1 (also for a NaN norm). */
float oracle_clip_coef(double norm, double max_norm)
{
    if (norm > max_norm)
        return (float)(max_norm / norm);
    return 1.0f;
}

/*
 * One step on clipped, unscaled grads: every grad value becomes
 * (g * inv_scale) * clip_coef, two rounded fp32 multiplies, before the
 * update (inv_scale = clip_coef = 1 is the plain step).
 */
int oracle_adamw_step_clipped(int32_t n_tensors, const int64_t *numel,
                              const int32_t *param_dtype, void *const *theta,
                              const int32_t *grad_dtype, const void *const *grad,
                              const int32_t *group_of, const oracle_group *groups,
                              int32_t n_groups, int32_t state_fmt, void *const *m,
                              void *const *v, float *const *m_scale,
                              float *const *v_scale, int32_t *t, float inv_scale,
                              float clip_coef, int32_t found_inf)
{
    if (found_inf)
        return 0;                                   /* R3: skip everything */
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (grad[i] == NULL)
            continue;                               /* R3: no grad, no update */
        if (group_of[i] < 0 || group_of[i] >= n_groups)
            return -1;
        t[i] += 1;
        step_scalars s = make_scalars(&groups[group_of[i]], t[i]);
        if (state_fmt == ORACLE_STATE_F32 || state_fmt == ORACLE_STATE_BF16) {
            int32_t sdt = state_fmt == ORACLE_STATE_F32 ? ORACLE_F32 : ORACLE_BF16;
            update_tensor_dense(numel[i], param_dtype[i], theta[i],
                                grad_dtype[i], grad[i], sdt, m[i], v[i], &s,
                                inv_scale, clip_coef);
        } else if (state_fmt == ORACLE_STATE_Q8) {
            update_tensor_q8(numel[i], param_dtype[i], theta[i], grad_dtype[i],
                             grad[i], (int8_t *)m[i], (uint8_t *)v[i],
                             m_scale[i], v_scale[i], &s, inv_scale, clip_coef);
        } else {
            return -1;
        }
    }
    return 0;
}

/* The plain step: oracle_adamw_step_scaled with inv_scale = 1. */
int oracle_adamw_step(int32_t n_tensors, const int64_t *numel,
                      const int32_t *param_dtype, void *const *theta,
                      const int32_t *grad_dtype, const void *const *grad,
                      const int32_t *group_of, const oracle_group *groups,
                      int32_t n_groups, int32_t state_fmt, void *const *m,
                      void *const *v, float *const *m_scale,
                      float *const *v_scale, int32_t *t, int32_t found_inf)
{
    return oracle_adamw_step_scaled(n_tensors, numel, param_dtype, theta,
                                    grad_dtype, grad, group_of, groups,
                                    n_groups, state_fmt, m, v, m_scale, v_scale,
                                    t, 1.0f, found_inf);
}

/*
 * The same step for fp32 parameters, grads and state written as the three
 * separate loops of [M041 §04] (m pass, v pass, theta pass).  Used only to
 * show that the one-pass form computes the same numbers.
 */
int oracle_adamw_step_three_loops(int32_t n_tensors, const int64_t *numel,
                                  float *const *theta, const float *const *grad,
                                  const int32_t *group_of,
                                  const oracle_group *groups, int32_t n_groups,
                                  float *const *m, float *const *v, int32_t *t,
                                  int32_t found_inf)
{
    if (found_inf)
        return 0;
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (grad[i] == NULL)
            continue;
        if (group_of[i] < 0 || group_of[i] >= n_groups)
            return -1;
        t[i] += 1;
        step_scalars s = make_scalars(&groups[group_of[i]], t[i]);
        const float *g = grad[i];
        float *mi = m[i], *vi = v[i], *th = theta[i];
        int64_t n = numel[i];
        for (int64_t e = 0; e < n; ++e)
            mi[e] = s.beta1 * mi[e] + s.one_minus_beta1 * g[e];
        for (int64_t e = 0; e < n; ++e)
            vi[e] = s.beta2 * vi[e] + (s.one_minus_beta2 * g[e]) * g[e];
        for (int64_t e = 0; e < n; ++e) {
            float m_hat = mi[e] / s.bc1;
            float v_hat = vi[e] / s.bc2;
            th[e] = th[e] * s.decay - (s.lr * m_hat) / (sqrtf(v_hat) + s.eps);
        }
    }
    return 0;
}
