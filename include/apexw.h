/*
 * apexw.h -- C ABI of a fused multi-tensor AdamW step for AMD MI355X (gfx950).
 *
 * One call of apexw_step updates every parameter of an optimizer with the
 * decoupled-decay AdamW rule of "Fused optimizers and state precision"
 * (ai-infra-kb M041), section 02: with the tensor's step count t advanced by
 * one,
 *
 *     m     <- beta1*m + (1-beta1)*g
 *     v     <- beta2*v + (1-beta2)*g*g
 *     theta <- theta*(1-lr*weight_decay) - lr*m_hat/(sqrt(v_hat)+eps),
 *              m_hat = m/(1-beta1^t),  v_hat = v/(1-beta2^t)
 *
 * (no AMSGrad; section 04: the bias corrections are per-tensor scalars and
 * m_hat, v_hat are never stored).  By default a step is one launch per
 * (parameter dtype, grad dtype) pair present: every workgroup takes its
 * tensor's bias corrections from an array the previous step wrote, and the
 * first tile of each tensor advances the tensor's step counter and writes
 * the corrections for the step after (apexw_set_launch_mode lists the other
 * launch modes and when they are taken).  Moments are kept in one of three
 * formats (section 05): fp32, bf16, or 8-bit codes with one fp32 absmax scale
 * per 256-element block.  Per parameter group lr, betas, eps and weight decay
 * are honoured (section 03); a parameter whose grad is absent is left
 * completely alone (section 03), and a step for which the device flag
 * found_inf is set changes nothing (section 06; the Apex fused-optimizer
 * guide, section 4.3, capturable mode) -- decided on the device, without a
 * host synchronisation.
 *
 * Arithmetic: fp32, every operation separately rounded in the order the
 * section 02 box fixes when read with its own (Python) operator rules --
 * ((1-beta2)*g)*g, and (lr*m_hat)/(sqrt(v_hat)+eps) subtracted from
 * theta*(1-lr*weight_decay) -- correctly rounded division and square root; the
 * scalars (1-beta1), (1-beta2), (1-lr*wd), lr, eps are formed in fp64 and
 * rounded once to fp32; beta^t is fp64 square-and-multiply over the bits of t
 * from the least significant end and 1-beta^t is rounded once to fp32.  bf16
 * values are widened exactly and narrowed round-to-nearest-even.
 *
 * Ownership: the caller owns every device buffer -- parameters, grads, the
 * state buffer (apexw_state_bytes), the workspace (apexw_workspace_bytes) and
 * the found_inf flag -- and the stream.  The library allocates no device
 * memory; it keeps a small host handle and a pinned host staging area for
 * table uploads.  Buffers must stay valid while work that uses them is queued.
 *
 * Errors: every function returns APEXW_OK (0) or a negative APEXW_E* code; on
 * error nothing has been written to device memory, and apexw_last_error()
 * gives a message (per thread).  Functions are thread-safe on distinct
 * handles; one handle must not be used from two threads at once.
 */
#ifndef APEXW_H
#define APEXW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- return codes */
#define APEXW_OK 0
#define APEXW_EINVAL (-1)  /* bad size, count, pointer or hyperparameter */
#define APEXW_EDTYPE (-2)  /* unsupported element type or state format */
#define APEXW_ENOSPC (-3)  /* state or workspace buffer smaller than needed */
#define APEXW_EHIP (-4)    /* a HIP runtime call failed */
#define APEXW_ENOMEM (-5)  /* host allocation failed */
#define APEXW_ESPARSE (-6) /* a sparse gradient: not expressible through these
                              dense pointers; returned by language bindings */

/* ---- element types of parameters and grads (dense, contiguous) */
#define APEXW_F32 0
#define APEXW_BF16 1

/* ---- moment storage formats (section 05 of the M041 page) */
#define APEXW_STATE_F32 0   /* m, v fp32: 8 bytes per element */
#define APEXW_STATE_BF16 1  /* m, v bf16, rounded to nearest even: 4 bytes */
#define APEXW_STATE_Q8 2    /* m int8 codes (scale absmax|m|/127), v uint8
                               codes (scale max v/255), one fp32 scale each
                               per 256-element block: 2 bytes + 8/256 */

#define APEXW_Q8_BLOCK 256
#define APEXW_MAX_GROUPS 32

typedef struct apexw_opt *apexw_t;

/* Hyperparameters of one parameter group for one call (Apex guide, section
 * 4.2 parameter table; M041 section 03).  0 <= beta1, beta2 < 1; lr, eps and
 * weight_decay finite and >= 0. */
typedef struct {
    double lr;
    double beta1;
    double beta2;
    double eps;
    double weight_decay;
} apexw_group;

/* Byte offsets of one tensor's state inside the state buffer.  m and v hold
 * numel elements of the format's moment type (fp32, bf16 bits, int8, uint8);
 * m_scale / v_scale hold ceil(numel/256) fp32 scales for APEXW_STATE_Q8 and
 * are -1 otherwise. */
typedef struct {
    int64_t m;
    int64_t v;
    int64_t m_scale;
    int64_t v_scale;
} apexw_tensor_state;

/*
 * Bytes of optimizer state for n_tensors tensors of numel[i] elements in
 * format fmt: the moment payload (8, 4 or 2 bytes per element), for Q8 two
 * fp32 scales per 256-element block (blocks never span tensors), and one
 * int32 step counter per tensor, plus padding that puts each tensor's moment
 * arrays on 128-byte boundaries (none when numel times the moment size is a
 * multiple of 128 for every tensor).  The library writes the padding (zeros).
 * For the 392-tensor LoRA set of the "ApexW measured in Unsloth" page this is
 * 185.5015 / 92.7515 / 47.1011 MiB for F32 / BF16 / Q8, the page's
 * 185.501 / 92.751 / 47.101 MB optimizer-state figures.
 * Returns APEXW_EINVAL for n_tensors < 0, a NULL pointer with n_tensors > 0,
 * or a negative numel; APEXW_EDTYPE for an unknown fmt.
 */
int apexw_state_bytes(int32_t n_tensors, const int64_t *numel, int32_t fmt,
                      size_t *out_bytes);

/*
 * Where each tensor's state lives in the state buffer: out_tensors[i] for
 * i < n_tensors (caller-allocated array), and *out_steps the byte offset of
 * the int32[n_tensors] step counters.  Layout: all m arrays (tensor order),
 * then all v arrays, then (Q8) all m scales and all v scales, then the step
 * counters.  Same argument rules as apexw_state_bytes.
 */
int apexw_state_layout(int32_t n_tensors, const int64_t *numel, int32_t fmt,
                       apexw_tensor_state *out_tensors, int64_t *out_steps);

/*
 * Bytes of device workspace apexw_create needs for this tensor list (tensor
 * table, grad-pointer table, per-tensor step records, tile table, grad-norm
 * partial sums, two arrays of carried bias corrections).  Same argument rules
 * as apexw_state_bytes, minus fmt.
 */
int apexw_workspace_bytes(int32_t n_tensors, const int64_t *numel,
                          size_t *out_bytes);

/*
 * Create an optimizer over n_tensors tensors.
 *   numel[i]        element count of tensor i (>= 0)
 *   param_dtype[i]  APEXW_F32 or APEXW_BF16
 *   grad_dtype[i]   APEXW_F32 or APEXW_BF16
 *   group_of[i]     parameter group of tensor i, 0 <= group_of[i] < n_groups
 *   n_groups        1 .. APEXW_MAX_GROUPS
 *   fmt             APEXW_STATE_F32 / _BF16 / _Q8
 *   state_dev       device buffer of state_bytes >= apexw_state_bytes(...)
 *                   bytes, 256-byte aligned; zero-filled here on `stream`
 *                   (m = v = 0, scales 0, step counters 0)
 *   workspace_dev   device buffer of >= apexw_workspace_bytes(...) bytes,
 *                   256-byte aligned, used only by this handle
 *   stream          hipStream_t (NULL: the default stream); create queues its
 *                   table uploads and the zero fill there and waits for them
 * The arrays are copied; they need not outlive the call.  Returns
 * APEXW_EINVAL / APEXW_EDTYPE / APEXW_ENOSPC on bad arguments (nothing
 * written), APEXW_EHIP if a HIP call fails, APEXW_ENOMEM if host memory runs
 * out.
 */
int apexw_create(int32_t n_tensors, const int64_t *numel,
                 const int32_t *param_dtype, const int32_t *grad_dtype,
                 const int32_t *group_of, int32_t n_groups, int32_t fmt,
                 void *state_dev, size_t state_bytes, void *workspace_dev,
                 size_t workspace_bytes, void *stream, apexw_t *out);

/*
 * Queue one optimizer step on `stream` (hipStream_t; NULL: default stream).
 *   groups[g]     hyperparameters of group g for this call, n_groups entries
 *                 (must equal the count given to apexw_create)
 *   params[i]     device pointer to tensor i's values (param_dtype[i]); may
 *                 be NULL only when numel[i] == 0.  params itself NULL: the
 *                 array of the previous call (APEXW_EINVAL if there is none)
 *   grads[i]      device pointer to tensor i's grad (grad_dtype[i]), or NULL
 *                 when the tensor has no grad this call: then its values,
 *                 moments and step counter are not touched.  grads itself
 *                 NULL: the array of the previous call on this handle (step,
 *                 check or norm call; APEXW_EINVAL if there is none) -- for
 *                 callers whose grad buffers persist across steps
 *   found_inf_dev device pointer to one float, read by the GPU when the step
 *                 runs; nonzero (or NaN) skips the whole step -- nothing is
 *                 written; NULL means never skip
 * Never synchronises with the host.  The pointer tables are re-uploaded (one
 * asynchronous copy) only when params or grads differ from the previous call.
 * Launches: by default one update kernel per (param, grad) dtype pair
 * present, with the bias corrections carried from the previous step in the
 * workspace; other modes and the cases that take them: apexw_set_launch_mode.
 * All calls on one handle must be ordered on the GPU (one stream, or streams
 * the caller orders).  Non-finite grads with found_inf unset are not checked
 * and propagate into theta, m and v.  The step counters in the state buffer
 * are read by the step that follows; a caller that rewrites them there
 * directly (not through apexw_import_state) calls apexw_set_launch_mode
 * before the next step, which drops the carried corrections.
 */
int apexw_step(apexw_t h, const apexw_group *groups, int32_t n_groups,
               void *const *params, const void *const *grads,
               const float *found_inf_dev, void *stream);

/*
 * Options of apexw_step_ex; every pointer may be NULL.
 *   inv_scale   device float: grads arrive multiplied by a loss scale and are
 *               unscaled first, g * inv_scale (NULL: 1)
 *   clip_coef   device float: the unscaled grads are then multiplied by it,
 *               (g * inv_scale) * clip_coef, e.g. the coefficient written by
 *               apexw_clip_grad_norm (NULL: 1)
 *   found_inf   device float: nonzero or NaN skips the whole step (NULL:
 *               never skip)
 *   groups_dev  device array of n_groups apexw_group records read by the GPU
 *               when the step runs (NULL: the host `groups` argument)
 * Each factor is one rounded fp32 multiply; a factor of 1 changes nothing.
 */
typedef struct {
    const float *inv_scale;
    const float *clip_coef;
    const float *found_inf;
    const apexw_group *groups_dev;
} apexw_step_options;

/*
 * The general step: apexw_step with the options above.  groups may be NULL
 * when opts->groups_dev is set.  apexw_step, apexw_step_scaled and
 * apexw_step_device are this call with some options fixed.
 */
int apexw_step_ex(apexw_t h, const apexw_group *groups, int32_t n_groups,
                  void *const *params, const void *const *grads,
                  const apexw_step_options *opts, void *stream);

/*
 * Global grad-norm clipping, the clip step of the mixed-precision recipe
 * (M041 section 06; the pages give no formula -- the plain one is used).
 * One pass reads every present grad: u = g * (*inv_scale_dev) in fp32 (NULL:
 * 1); if found_inf_dev is not NULL, sets it to 1.0f when any u is an
 * infinity or a NaN, exactly as apexw_unscale_check; sums u*u in fp64 into
 * one partial per read group (four 256-element tiles fixed by the tile table,
 * not by the grid); then a fixed-order reduction (so the result does not
 * depend on scheduling) writes the norm sqrt(sum) (fp64) to
 * *norm_out_dev (may be NULL) and to *clip_coef_dev the factor
 * max_norm / norm if norm > max_norm (fp64, rounded once to fp32), else 1.
 * Pass clip_coef_dev (and the same inv_scale) in apexw_step_options.
 * max_norm must be finite and > 0.  Queued on `stream`, no host sync.
 * Errors: APEXW_EINVAL for a NULL handle, grads or clip_coef_dev or a bad
 * max_norm; APEXW_EHIP if a launch fails.
 */
int apexw_clip_grad_norm(apexw_t h, const void *const *grads,
                         const float *inv_scale_dev, double max_norm,
                         float *found_inf_dev, double *norm_out_dev,
                         float *clip_coef_dev, void *stream);

/*
 * apexw_clip_grad_norm for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same pass with the same results, bit for bit, but its fp64
 * partial sums live in a static device array of the library (8 MiB, one copy
 * per GPU, held until the process ends) instead of the handle's workspace.
 * The array holds one partial per read group of four tiles plus 256
 * second-stage sums, room for lists of up to about 1.07e9 elements; a larger
 * list gets APEXW_ENOSPC before anything is queued.  Every call on a GPU
 * shares that array and writes every entry it reads, so calls that overlap
 * on one GPU (other streams, other threads, other handles) race: order them.
 * The first call on a device looks up the array's address there.  Other
 * arguments and errors as apexw_clip_grad_norm.
 */
int apexw_clip_grad_norm_noalloc(apexw_t h, const void *const *grads,
                                 const float *inv_scale_dev, double max_norm,
                                 float *found_inf_dev, double *norm_out_dev,
                                 float *clip_coef_dev, void *stream);

/*
 * apexw_step on grads that arrive multiplied by a loss scale: every grad
 * value is first unscaled, g * (*inv_scale_dev) as one rounded fp32
 * multiply, then updated exactly as by apexw_step (the mixed-precision
 * recipe of the M041 page, section 06; the Apex guide, section 4.3, passes
 * inv_scale = 1/scale to its kernel the same way, with no host sync).
 *   inv_scale_dev  device pointer to one float, read by the GPU when the step
 *                  runs; NULL means 1 (then this is apexw_step).
 * Other arguments, errors and ordering as apexw_step.
 */
int apexw_step_scaled(apexw_t h, const apexw_group *groups, int32_t n_groups,
                      void *const *params, const void *const *grads,
                      const float *inv_scale_dev, const float *found_inf_dev,
                      void *stream);

/*
 * Unscale-and-check pass of the mixed-precision recipe (M041 section 06):
 * reads every present grad once and sets *found_inf_dev = 1.0f if any value
 * g * (*inv_scale_dev) (one rounded fp32 multiply; NULL inv_scale_dev means 1)
 * is an infinity or a NaN.  It never clears the flag (the caller zeroes it
 * before the first check of a step, so several checks can accumulate) and
 * never rewrites the grads: pass the same inv_scale to apexw_step_scaled,
 * which applies it inside the update.  grads: as for apexw_step (NULL entries
 * are skipped); found_inf_dev must not be NULL.  Queued on `stream`, no host
 * synchronisation.  Errors: APEXW_EINVAL for a NULL handle, grads or
 * found_inf_dev; APEXW_EHIP if a launch fails.
 */
int apexw_unscale_check(apexw_t h, const void *const *grads,
                        const float *inv_scale_dev, float *found_inf_dev,
                        void *stream);

/*
 * The unscaling factor for grads multiplied by a loss scale, formed as the
 * Apex fused-optimizer guide (section 4.3) forms the inv_scale it passes to
 * its kernel: the fp64 reciprocal of the scale rounded once to fp32,
 * *inv_scale_dev = (float)(1.0 / (double)*scale_dev).  For a power-of-two
 * scale this is the exact reciprocal; for other scales it can differ in the
 * last bit from a reciprocal taken in fp32.  One lane of one workgroup,
 * queued on `stream` (hipStream_t; NULL: the default stream), no host sync;
 * the two pointers are device pointers to one float each and may be equal.
 * Errors: APEXW_EINVAL for a NULL pointer; APEXW_EHIP if the launch fails.
 */
int apexw_inv_scale(const float *scale_dev, float *inv_scale_dev, void *stream);

/*
 * apexw_step_scaled with the group hyperparameters in device memory:
 * groups_dev points to n_groups apexw_group records that the GPU reads when
 * the step runs, and the fp32 scalars are formed there exactly as the host
 * forms them, so results are bit-identical to apexw_step_scaled with the same
 * values.  This makes the whole step capturable in a hipGraph with a learning
 * rate that changes between replays (capturable mode of the Apex guide,
 * section 4.2; the step counters already live on the device).  The values are
 * not validated (they are never read by the host): out-of-range
 * hyperparameters give unspecified numbers, never a fault.  Under stream
 * capture the parameter and grad pointers must equal those of the previous
 * call on the handle (the pointer tables are uploaded only outside capture);
 * otherwise APEXW_EINVAL.
 */
int apexw_step_device(apexw_t h, const apexw_group *groups_dev, int32_t n_groups,
                      void *const *params, const void *const *grads,
                      const float *inv_scale_dev, const float *found_inf_dev,
                      void *stream);

/*
 * Checkpoint of the optimizer state (the M041 page, section 08: a checkpoint
 * carries the state dtype and scales, the step counters and the recipe, not
 * only the parameters).  apexw_export_bytes gives the size of the blob;
 * apexw_export_state writes it to host memory dst_host: a header (format
 * version, state format, tensor count, group count), every tensor's numel,
 * parameter and grad dtype and group, the recipe `groups` (n_groups records,
 * usually those of the last step), and the raw state buffer (moments, 8-bit
 * scales, step counters).  It queues a device-to-host copy on `stream` and
 * waits for it.  apexw_import_state checks that a blob was written for a
 * handle of the same format, tensor sizes, dtypes and groups (APEXW_EINVAL
 * otherwise, nothing written), copies its state into the handle's state
 * buffer (waits for the copy), and returns the recipe in groups_out (may be
 * NULL; else n_groups must match).  A run resumed from a blob continues
 * bit for bit as the uninterrupted run.
 */
int apexw_export_bytes(apexw_t h, size_t *out_bytes);
int apexw_export_state(apexw_t h, const apexw_group *groups, int32_t n_groups,
                       void *dst_host, size_t dst_bytes, void *stream);
int apexw_import_state(apexw_t h, const void *src_host, size_t src_bytes,
                       apexw_group *groups_out, int32_t n_groups, void *stream);

/*
 * Copy the int32 step counter of every tensor (n_tensors values, in tensor
 * order) to host_out after the work queued on `stream`; synchronises that
 * stream.  A tensor's counter is the number of steps that updated it
 * (M041 sections 03 and 06: an absent grad or a skipped step does not count).
 * Errors: APEXW_EINVAL for a NULL handle or host_out; APEXW_EHIP.
 */
int apexw_read_steps(apexw_t h, int32_t *host_out, void *stream);

/*
 * Launch geometry of the handle: tile size in elements (256; one workgroup of
 * one wave64 per tile), number of tiles, and the largest workgroup count of
 * its update launches (the uncapped 8-bit carried step runs half as many,
 * two tiles each).  Any pointer may be NULL.
 */
int apexw_launch_info(apexw_t h, int32_t *tile_elems, int32_t *n_tiles,
                      int32_t *workgroups);

/*
 * Cap the workgroups of each update launch (0 restores the default: one per
 * tile, at most 2^24); under the cap a workgroup walks several tiles.  A cap
 * that is a multiple of 8 keeps each XCD on its own tile-table lines.
 * Results do not depend on it.
 */
int apexw_set_workgroups(apexw_t h, int32_t workgroups);

/*
 * Cap how many update workgroups may be resident on one compute unit at a
 * time, for every update launch (enforced through the dynamic LDS each
 * workgroup reserves; the kernel uses none).  0 restores the defaults, which
 * depend on the bytes each element moves (fp32 params and moments, 28 B: 14;
 * bf16 params, fp32 grads and moments, 24 B: 16; bf16 moments with fp32
 * grads, 16-18 B: 28; all-bf16 (14 B) or 8-bit moments: no cap).  Fewer
 * concurrent streams can keep the HBM read/write mix more efficient; results
 * do not depend on it.
 */
int apexw_set_occupancy(apexw_t h, int32_t workgroups_per_cu);

/*
 * Cache policy of the update kernel: 0 (default) chooses by size -- lists
 * whose parameters, grads and state together reach 64 MiB stream with
 * non-temporal loads and stores (in a training loop the forward and backward
 * passes evict the 256 MB Infinity Cache between steps, and streaming is then
 * the faster), smaller ones use ordinary (cached) accesses; 1 forces
 * streaming, 2 forces cached (fastest when steps run back to back with
 * nothing in between).  Results do not depend on it.
 */
int apexw_set_cache_policy(apexw_t h, int32_t policy);

/*
 * How a step is launched.  1: a prepare kernel (one lane per tensor: step
 * counter, bias corrections, per-tensor record) and then one update kernel
 * per (param, grad) dtype pair.  2: one kernel per dtype pair that does both:
 * every workgroup forms its tensor's record from the counter, and the last
 * workgroup to finish (found through a two-level tree of arrival counters in
 * the workspace) advances the counters.  It saves a launch, most of the cost
 * of a small list, but each workgroup's arrival costs a device-scope atomic:
 * on MI355X it is faster up to about 8,000 tiles.  Mode 2 needs a list of at
 * most 6144 tiles (1,572,864 elements) whose dtype pairs each hold a
 * non-empty tensor; APEXW_EINVAL otherwise.  3: one kernel per dtype pair at
 * any size, no atomics: every workgroup takes its tensor's bias corrections
 * from an array the previous step wrote, and the first tile of each tensor
 * advances its counter and writes the corrections for the following step
 * into a second array (the two alternate).  The chain of carried corrections
 * starts with a small kernel that forms them from the counters as they stand
 * -- on the first step, after any step in another mode, after a change of
 * beta1 or beta2, after apexw_import_state or apexw_set_launch_mode, and after
 * a step in which a dtype pair had no grad at all.  A step whose
 * hyperparameters live in device memory (apexw_step_device, groups_dev), or
 * one queued while its stream is being captured into a graph (a replay would
 * not move the chain on), takes mode 2 or 1 as mode 0 would without mode 3.
 * Mode 3 needs a non-empty list without empty tensors; APEXW_EINVAL
 * otherwise.  0 (default): mode 3 for such lists, else mode 2 for lists it
 * takes unless they stream (apexw_set_cache_policy), else mode 1.  Results do
 * not depend on the mode; steps of one handle queued on two streams at once
 * race in every mode.  Once a step of the handle has been queued under stream
 * capture, its eager steps no longer take mode 3 either: a replay of that
 * graph advances the counters with no host call, after which carried
 * corrections would be stale.  Every call of this function drops the carried
 * corrections (so a caller that wrote step counters into the state buffer
 * calls it before the next step) and re-admits mode 3 after a capture: call
 * it only once no graph holding a step of this handle will be replayed.
 */
int apexw_set_launch_mode(apexw_t h, int32_t mode);

/* The launch mode (1, 2 or 3) the handle's next step uses when its
 * hyperparameters come from the host and its stream is not being captured. */
int apexw_get_launch_mode(apexw_t h, int32_t *mode);

/* The largest cap in force over the handle's update launches (0: none). */
int apexw_get_occupancy(apexw_t h, int32_t *workgroups_per_cu);

/* Release the handle: waits until the handle's pending table uploads (host
 * to device copies out of its pinned staging area) have completed, then frees
 * its host memory.  Device buffers -- state, workspace -- stay the caller's;
 * work already queued that uses them must finish before they are freed. */
int apexw_destroy(apexw_t h);

/* Message of the last failed call on this thread ("" if none). */
const char *apexw_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* APEXW_H */
