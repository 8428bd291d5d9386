// apexw.hip -- host engine and C ABI of the fused multi-tensor AdamW step.
//
// The engine turns a parameter list into device tables once (tensor
// descriptors, the XCD-major table giving the tensor of every 256-element
// tile, built by apexw_plan.hpp), lays the optimizer state out in one
// caller-owned buffer, and on every step queues, by default, one carried-step
// launch per (parameter dtype, grad dtype) pair present, each with one
// workgroup per tile (per two tiles in the 8-bit format): the bias
// corrections come from the previous step, and each tensor's first tile
// advances its counter and writes the next ones.  It also allocates no
// device memory of its own except one fixed static array for the
// grad-norm entry point that allocates nothing.
// Steps whose hyperparameters live in device memory, steps queued under
// stream capture (and every step after one), and lists with an empty tensor
// take a prepare launch plus the update launches, or for small lists a single
// launch per pair (apexw_set_launch_mode).  Per call the engine only compares
// the param / grad pointer arrays with the previous call's (one asynchronous
// upload when they differ) and forms the per-group fp32 scalars, which travel
// in the kernel arguments.  It never synchronises with the host inside a
// step.
//
// Sources: "Fused optimizers and state precision" (ai-infra-kb M041),
// sections 02-06; "Apex fused optimizers" guide (qwbw.cn), sections 二/三
// (dtype rules, multi-tensor launches) and 4.2-4.3 (parameter groups, device
// overflow flag, step advanced only without overflow); "ApexW measured in
// Unsloth" (kongchang.com), results table (state bytes per format).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "apexw.h"
#include "apexw_kernels.hpp"

using namespace apexw;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

#define HIP_TRY(call)                                                        \
    do {                                                                     \
        hipError_t e_ = (call);                                              \
        if (e_ != hipSuccess)                                                \
            return fail(APEXW_EHIP, "%s failed: %s", #call,                  \
                        hipGetErrorString(e_));                              \
    } while (0)

// Every moment array starts and ends on a 128-byte boundary, the cache line:
// a tile's moments (1 KiB fp32, 512 B bf16, 256 B of 8-bit codes) then fill
// whole lines, so no line is shared by two tiles -- which run on different
// XCDs, whose separate L2s would each fetch it -- and the update writes a
// tensor's last partial line of m and v whole (zeros past the end), since a
// partly written line costs the memory a read-modify-write.
constexpr int64_t kMomentAlign = 128;
constexpr int64_t kTableAlign = 256;

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

int64_t ceil_div(int64_t x, int64_t a) { return (x + a - 1) / a; }

int moment_bytes(int32_t fmt) {
    switch (fmt) {
    case APEXW_STATE_F32: return 4;
    case APEXW_STATE_BF16: return 2;
    case APEXW_STATE_Q8: return 1;
    default: return 0;
    }
}

int check_list(int32_t n, const int64_t *numel) {
    if (n < 0) return fail(APEXW_EINVAL, "n_tensors must be >= 0 (got %d)", n);
    if (n > 0 && numel == nullptr) return fail(APEXW_EINVAL, "numel is NULL");
    for (int32_t i = 0; i < n; ++i)
        if (numel[i] < 0)
            return fail(APEXW_EINVAL, "numel[%d] is negative (%lld)", i,
                        (long long)numel[i]);
    return APEXW_OK;
}

// State layout: every m array, every v array, (Q8) every m scale array and
// every v scale array, then the int32 step counters.  Moment arrays start and
// end on 128-byte boundaries.
int compute_layout(int32_t n, const int64_t *numel, int32_t fmt,
                   apexw_tensor_state *per_tensor, int64_t *steps_off,
                   int64_t *total) {
    const int eb = moment_bytes(fmt);
    if (eb == 0) return fail(APEXW_EDTYPE, "unknown state format %d", fmt);
    int rc = check_list(n, numel);
    if (rc) return rc;
    int64_t off = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (per_tensor) per_tensor[i].m = off;
        off += round_up(numel[i] * eb, kMomentAlign);
    }
    for (int32_t i = 0; i < n; ++i) {
        if (per_tensor) per_tensor[i].v = off;
        off += round_up(numel[i] * eb, kMomentAlign);
    }
    if (fmt == APEXW_STATE_Q8) {
        for (int32_t i = 0; i < n; ++i) {
            if (per_tensor) per_tensor[i].m_scale = off;
            off += ceil_div(numel[i], APEXW_Q8_BLOCK) * 4;
        }
        for (int32_t i = 0; i < n; ++i) {
            if (per_tensor) per_tensor[i].v_scale = off;
            off += ceil_div(numel[i], APEXW_Q8_BLOCK) * 4;
        }
    } else if (per_tensor) {
        for (int32_t i = 0; i < n; ++i) per_tensor[i].m_scale = per_tensor[i].v_scale = -1;
    }
    if (steps_off) *steps_off = off;
    off += 4 * (int64_t)n;
    if (total) *total = off;
    return APEXW_OK;
}

// Workspace layout: descriptors | grad pointers | step records | tile table |
// grad-norm partial sums (one per tile, then one per reduce workgroup), each
// on a 256-byte boundary.
struct WsLayout {
    int64_t desc, grads, records, tiles, partials, partials2, consts, bias, done, tensors, total;
    int64_t n_tiles;
    bool single;                         // room for the single-launch step
};

// The constants region: 0.0f and 1.0f, passed to the step kernels in place
// of an absent found_inf flag, inv_scale or clip coefficient, so that they
// load all of them unconditionally.
constexpr float kConsts[2] = {0.0f, 1.0f};

constexpr int64_t kMaxGrid = 1 << 24;  // workgroups per launch (grid-stride above)

// Lists of at most this many tiles may take the single-launch step (one
// kernel per dtype pair, no prepare launch); the workspace then holds its
// arrival counters and the tensor list of every launch.
constexpr int64_t kSingleLaunchTiles = 6144;

WsLayout ws_layout(int32_t n, const int64_t *numel) {
    WsLayout w;
    w.n_tiles = 0;
    for (int32_t i = 0; i < n; ++i) w.n_tiles += ceil_div(numel[i], kTile);
    w.desc = 0;
    w.grads = w.desc + round_up((int64_t)n * (int64_t)sizeof(TensorDesc), kTableAlign);
    w.records = w.grads + round_up((int64_t)n * 8, kTableAlign);
    w.tiles = w.records + round_up((int64_t)n * (int64_t)sizeof(StepRecord), kTableAlign);
    // each launch's table is padded to a multiple of kXcds entries; the read
    // passes load table entries in fours and may read up to 3 past the end
    w.partials = w.tiles + round_up(table_entries_reserved(w.n_tiles) * 4, kTableAlign);
    // grad-norm partials: one per read group of every launch, the launches
    // one after another (a launch of t tiles has 8 * ceil(ceil(t/8)/4) <= t + 8
    // groups); entries of groups past a launch's end stay 0
    w.partials2 = w.partials + round_up((w.n_tiles + kMaxLaunches * kXcds) * 8, kTableAlign);
    w.consts = w.partials2 + round_up(kReduceBlocks * 8, kTableAlign);
    // the carried step's bias corrections: two arrays of one record per tensor
    w.bias = w.consts + round_up((int64_t)sizeof(kConsts), kTableAlign);
    w.done = w.bias + round_up(2 * (int64_t)n * (int64_t)sizeof(BiasRecord), kTableAlign);
    w.single = w.n_tiles <= kSingleLaunchTiles;
    w.tensors = w.done + (w.single ? round_up((int64_t)kMaxLaunches * kDoneWords * 4, kTableAlign) : 0);
    w.total = n == 0 ? 0 : w.tensors + (w.single ? round_up((int64_t)n * 4, kTableAlign) : 0);
    return w;
}

bool finite_nonneg(double x) { return std::isfinite(x) && x >= 0.0; }

using Launch = PlanLaunch;

// Default cap on update workgroups resident per compute unit for one launch
// (0: no cap), from the bytes each element moves.  Measured on MI355X: the
// heavier the per-tile traffic, the fewer one-wave streams per CU keep the
// HBM read/write mix most efficient (28 B/elem: 14, 24 B/elem: 16, 16 B/elem
// with bf16 moments: 28 -- 1% faster than uncapped, 26 to 30 alike); the
// leanest formats (14 B/elem and the 8-bit state) want every stream they
// can get.

int element_bytes(int32_t fmt, int pt, int gt) {
    const int p = pt == APEXW_F32 ? 4 : 2, g = gt == APEXW_F32 ? 4 : 2;
    return 2 * p + g + 4 * moment_bytes(fmt);
}

int default_occupancy(int32_t fmt, int pt, int gt) {
    const int b = element_bytes(fmt, pt, gt);
    if (b >= 25) return 14;
    if (b >= 23) return 16;
    if (b >= 21) return 20;
    if (b >= 15) return 28;
    return 0;
}

typedef void (*kernel_fn)(KernelArgs);

template <int ST, bool NT, bool SC>
kernel_fn pick_kernel(int pt, int gt) {
    if (pt == APEXW_F32 && gt == APEXW_F32) return adamw_step_kernel<ST, APEXW_F32, APEXW_F32, NT, SC>;
    if (pt == APEXW_F32 && gt == APEXW_BF16) return adamw_step_kernel<ST, APEXW_F32, APEXW_BF16, NT, SC>;
    if (pt == APEXW_BF16 && gt == APEXW_F32) return adamw_step_kernel<ST, APEXW_BF16, APEXW_F32, NT, SC>;
    return adamw_step_kernel<ST, APEXW_BF16, APEXW_BF16, NT, SC>;
}

template <bool NT, bool SC>
kernel_fn pick_format(int fmt, int pt, int gt) {
    if (fmt == APEXW_STATE_F32) return pick_kernel<APEXW_STATE_F32, NT, SC>(pt, gt);
    if (fmt == APEXW_STATE_BF16) return pick_kernel<APEXW_STATE_BF16, NT, SC>(pt, gt);
    return pick_kernel<APEXW_STATE_Q8, NT, SC>(pt, gt);
}

// streaming = non-temporal loads and stores (the single-use streams of a
// list far larger than the caches); a list whose parameters, grads and state
// fit the 256 MB Infinity Cache many times over keeps them cached instead.
// scaled = the step was given inv_scale or clip_coef.
kernel_fn kernel_for(int fmt, int pt, int gt, bool streaming, bool scaled) {
    if (streaming)
        return scaled ? pick_format<true, true>(fmt, pt, gt) : pick_format<true, false>(fmt, pt, gt);
    return scaled ? pick_format<false, true>(fmt, pt, gt) : pick_format<false, false>(fmt, pt, gt);
}

template <int ST, bool SC>
kernel_fn pick_single(int pt, int gt) {
    if (pt == APEXW_F32 && gt == APEXW_F32) return adamw_single_step_kernel<ST, APEXW_F32, APEXW_F32, SC>;
    if (pt == APEXW_F32 && gt == APEXW_BF16) return adamw_single_step_kernel<ST, APEXW_F32, APEXW_BF16, SC>;
    if (pt == APEXW_BF16 && gt == APEXW_F32) return adamw_single_step_kernel<ST, APEXW_BF16, APEXW_F32, SC>;
    return adamw_single_step_kernel<ST, APEXW_BF16, APEXW_BF16, SC>;
}

template <int ST, bool NT, bool SC, bool ONE, bool FEW>
kernel_fn pick_carry(int pt, int gt) {
    if (pt == APEXW_F32 && gt == APEXW_F32) return adamw_carry_step_kernel<ST, APEXW_F32, APEXW_F32, NT, SC, ONE, FEW>;
    if (pt == APEXW_F32 && gt == APEXW_BF16) return adamw_carry_step_kernel<ST, APEXW_F32, APEXW_BF16, NT, SC, ONE, FEW>;
    if (pt == APEXW_BF16 && gt == APEXW_F32) return adamw_carry_step_kernel<ST, APEXW_BF16, APEXW_F32, NT, SC, ONE, FEW>;
    return adamw_carry_step_kernel<ST, APEXW_BF16, APEXW_BF16, NT, SC, ONE, FEW>;
}

// The 8-bit carried step: under a workgroup cap the grid-stride kernel;
// otherwise (PAIR) the kernel that takes two tiles per workgroup, whose grid
// is half the tiles (carry_grid).
template <bool NT, bool SC, bool PAIR, bool FEW>
kernel_fn pick_carry_q8(int pt, int gt) {
    if constexpr (PAIR) {
        if (pt == APEXW_F32 && gt == APEXW_F32) return adamw_carry_pair_q8_kernel<APEXW_F32, APEXW_F32, NT, SC, FEW>;
        if (pt == APEXW_F32 && gt == APEXW_BF16) return adamw_carry_pair_q8_kernel<APEXW_F32, APEXW_BF16, NT, SC, FEW>;
        if (pt == APEXW_BF16 && gt == APEXW_F32) return adamw_carry_pair_q8_kernel<APEXW_BF16, APEXW_F32, NT, SC, FEW>;
        return adamw_carry_pair_q8_kernel<APEXW_BF16, APEXW_BF16, NT, SC, FEW>;
    } else {
        if (pt == APEXW_F32 && gt == APEXW_F32) return adamw_carry_step_q8_kernel<APEXW_F32, APEXW_F32, NT, SC>;
        if (pt == APEXW_F32 && gt == APEXW_BF16) return adamw_carry_step_q8_kernel<APEXW_F32, APEXW_BF16, NT, SC>;
        if (pt == APEXW_BF16 && gt == APEXW_F32) return adamw_carry_step_q8_kernel<APEXW_BF16, APEXW_F32, NT, SC>;
        return adamw_carry_step_q8_kernel<APEXW_BF16, APEXW_BF16, NT, SC>;
    }
}

// Workgroups of a carried launch of `tiles` tiles under the cap `wg`: one
// per tile when uncapped (wg == tiles), except in the 8-bit format, whose
// uncapped kernel takes two tiles per workgroup.
int64_t carry_grid(int fmt, int64_t tiles, int64_t wg) {
    if (wg == tiles && fmt == APEXW_STATE_Q8) return (tiles + 1) / 2;
    return wg;
}

// one_tile: the grid is not capped (a workgroup per tile, or per two tiles
// in the 8-bit format); the kernels then run their loop-free form.  few
// (only with one_tile, and only for cached accesses): the launch's tensors
// are found from the few-tensor bounds in the kernel arguments instead of
// the tile table.
template <int ST, bool NT, bool SC>
kernel_fn pick_carry_shape(int pt, int gt, bool one_tile, bool few) {
    if constexpr (ST == APEXW_STATE_Q8) {
        if (!one_tile) return pick_carry_q8<NT, SC, false, false>(pt, gt);
        if constexpr (!NT)                    // streamed launches read the table
            if (few) return pick_carry_q8<NT, SC, true, true>(pt, gt);
        return pick_carry_q8<NT, SC, true, false>(pt, gt);
    } else {
        if (!one_tile) return pick_carry<ST, NT, SC, false, false>(pt, gt);
        if constexpr (!NT)
            if (few) return pick_carry<ST, NT, SC, true, true>(pt, gt);
        return pick_carry<ST, NT, SC, true, false>(pt, gt);
    }
}

template <bool NT, bool SC>
kernel_fn pick_carry_format(int fmt, int pt, int gt, bool one_tile, bool few) {
    if (fmt == APEXW_STATE_F32) return pick_carry_shape<APEXW_STATE_F32, NT, SC>(pt, gt, one_tile, few);
    if (fmt == APEXW_STATE_BF16) return pick_carry_shape<APEXW_STATE_BF16, NT, SC>(pt, gt, one_tile, few);
    return pick_carry_shape<APEXW_STATE_Q8, NT, SC>(pt, gt, one_tile, few);
}

// The carried-step kernel (launch mode 3).
kernel_fn carry_kernel_for(int fmt, int pt, int gt, bool streaming, bool scaled, bool one_tile,
                           bool few) {
    if (streaming)
        return scaled ? pick_carry_format<true, true>(fmt, pt, gt, one_tile, few)
                      : pick_carry_format<true, false>(fmt, pt, gt, one_tile, few);
    return scaled ? pick_carry_format<false, true>(fmt, pt, gt, one_tile, few)
                  : pick_carry_format<false, false>(fmt, pt, gt, one_tile, few);
}

// The single-launch step kernel (cached accesses: such lists are small).
kernel_fn single_kernel_for(int fmt, int pt, int gt, bool scaled) {
    if (fmt == APEXW_STATE_F32)
        return scaled ? pick_single<APEXW_STATE_F32, true>(pt, gt) : pick_single<APEXW_STATE_F32, false>(pt, gt);
    if (fmt == APEXW_STATE_BF16)
        return scaled ? pick_single<APEXW_STATE_BF16, true>(pt, gt) : pick_single<APEXW_STATE_BF16, false>(pt, gt);
    return scaled ? pick_single<APEXW_STATE_Q8, true>(pt, gt) : pick_single<APEXW_STATE_Q8, false>(pt, gt);
}

// Bytes an optimizer touches per step (parameters, grads, state): above this
// the update streams past the caches.  Measured on MI355X with the 8-bit
// LoRA list (146 MB touched): streaming takes 65 us when the 256 MB Infinity
// Cache was flushed before the step, as a training loop's forward and
// backward passes do, against 71 us with cached accesses; only when steps
// run back to back with nothing in between is caching faster (55 against
// 57 us).  Small lists keep cached accesses (and the single launch).
constexpr int64_t kStreamingBytes = (int64_t)64 << 20;

}  // namespace

struct apexw_opt {
    int device = 0;
    int32_t n = 0, n_groups = 0, fmt = 0;
    std::vector<int64_t> numel;
    std::vector<int32_t> pdt, gdt, group_of;
    std::vector<apexw_tensor_state> layout;
    int64_t steps_off = 0;
    char *state = nullptr;
    char *ws = nullptr;
    WsLayout wl{};
    std::vector<Launch> launches;
    std::vector<int32_t> tensor_list;   // tensors of each launch, launch by launch
    std::vector<int64_t> first_tile;    // per tensor
    // host mirrors of the per-call tables
    std::vector<TensorDesc> desc;
    std::vector<void *> last_params;
    std::vector<const void *> last_grads;
    bool have_params = false, have_grads = false;
    // pinned staging ring for table uploads
    static constexpr int kRing = 4;
    char *pinned = nullptr;
    int64_t slot_bytes = 0;
    hipEvent_t ev[kRing] = {};
    bool ev_pending[kRing] = {};
    int next_slot = 0;
    int cu_count = 0;
    int64_t table_entries = 0;          // tile-table length (all launches, with padding)
    int lds_per_cu = 0, lds_per_block = 0;
    int32_t wg_override = 0;
    int32_t occupancy = 0;              // override for every launch (0: defaults)
    int cache_policy = 0;               // 0 auto, 1 streaming, 2 cached
    bool streaming_auto = true;
    bool single_ok = false;             // the single-launch step is available
    int launch_mode = 0;                // 0 auto, 1 prepare + update, 2 single launch, 3 carried
    // the carried step (mode 3): bias corrections for the next step live in
    // bias array carry_parity of the workspace when carry_valid, formed with
    // the betas below; any other kind of step, an import or a mode change
    // drops them
    bool carry_ok = false;              // no empty tensor: every tensor has a first tile
    bool carry_valid = false;
    // a step of this handle was queued under stream capture: a replay of
    // that graph moves the counters with no host call, so eager steps stop
    // carrying corrections (any carried record could be stale) until
    // apexw_set_launch_mode re-admits the carried step
    bool graph_steps = false;
    int carry_parity = 0;
    std::vector<double> carry_beta1, carry_beta2;
};

namespace {

struct DeviceGuard {
    int prev = -1;
    explicit DeviceGuard(int dev) {
        int cur = 0;
        if (hipGetDevice(&cur) == hipSuccess && cur != dev) {
            prev = cur;
            (void)hipSetDevice(dev);
        }
    }
    ~DeviceGuard() {
        if (prev >= 0) (void)hipSetDevice(prev);
    }
};

void release(apexw_opt *h) {
    if (!h) return;
    for (int s = 0; s < apexw_opt::kRing; ++s) {
        if (h->ev[s]) {
            if (h->ev_pending[s]) (void)hipEventSynchronize(h->ev[s]);
            (void)hipEventDestroy(h->ev[s]);
        }
    }
    if (h->pinned) (void)hipHostFree(h->pinned);
    delete h;
}

// Host copy of the descriptor table for the given parameter pointers
// (nullptr: none yet).
void fill_descriptors(apexw_opt *h, void *const *params) {
    for (int32_t i = 0; i < h->n; ++i) {
        TensorDesc &d = h->desc[i];
        std::memset(&d, 0, sizeof d);
        d.param = params ? params[i] : nullptr;
        d.m = h->state + h->layout[i].m;
        d.v = h->state + h->layout[i].v;
        d.m_scale = h->layout[i].m_scale >= 0
                        ? reinterpret_cast<float *>(h->state + h->layout[i].m_scale)
                        : nullptr;
        d.v_scale = h->layout[i].v_scale >= 0
                        ? reinterpret_cast<float *>(h->state + h->layout[i].v_scale)
                        : nullptr;
        d.numel = h->numel[i];
        d.first_tile = h->first_tile[i];
        d.group = h->group_of[i];
    }
}

// Upload the grad-pointer table, and the descriptors when params is given
// and differs from the last upload: one asynchronous copy from a pinned ring
// slot, only when something changed.
int upload_pointer_tables(apexw_opt *h, void *const *params, const void *const *grads,
                          hipStream_t st) {
    const size_t n = (size_t)h->n;
    if (n == 0) return APEXW_OK;
    const bool params_changed =
        params && (!h->have_params || std::memcmp(h->last_params.data(), params, n * sizeof(void *)));
    const bool grads_changed =
        !h->have_grads || std::memcmp(h->last_grads.data(), grads, n * sizeof(void *));
    if (!params_changed && !grads_changed) return APEXW_OK;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    HIP_TRY(hipStreamIsCapturing(st, &cap));
    if (cap != hipStreamCaptureStatusNone)
        return fail(APEXW_EINVAL, "parameter or grad pointers changed while the stream is being "
                                  "captured; call once with these pointers before capturing");
    const int s = h->next_slot;
    if (h->ev_pending[s]) HIP_TRY(hipEventSynchronize(h->ev[s]));
    char *slot = h->pinned + (int64_t)s * h->slot_bytes;
    int64_t begin = h->wl.grads;
    const int64_t end = h->wl.grads + (int64_t)n * 8;
    if (params_changed) {
        fill_descriptors(h, params);
        std::memcpy(slot + h->wl.desc, h->desc.data(), n * sizeof(TensorDesc));
        begin = h->wl.desc;
        std::memcpy(h->last_params.data(), params, n * sizeof(void *));
        h->have_params = true;
    }
    std::memcpy(slot + h->wl.grads, grads, n * sizeof(void *));
    HIP_TRY(hipMemcpyAsync(h->ws + begin, slot + begin, (size_t)(end - begin),
                           hipMemcpyHostToDevice, st));
    HIP_TRY(hipEventRecord(h->ev[s], st));
    h->ev_pending[s] = true;
    h->next_slot = (s + 1) % apexw_opt::kRing;
    std::memcpy(h->last_grads.data(), grads, n * sizeof(void *));
    h->have_grads = true;
    return APEXW_OK;
}

// A NULL params or grads array on a step call means "the arrays of the
// previous call" (persistent grad buffers need no new array each step).
int reuse_last(apexw_opt *h, void *const **params, const void *const **grads) {
    if (h->n == 0) return APEXW_OK;
    if (params && !*params) {
        if (!h->have_params) return fail(APEXW_EINVAL, "params is NULL and no earlier call gave them");
        *params = h->last_params.data();
    }
    if (!*grads) {
        if (!h->have_grads) return fail(APEXW_EINVAL, "grads is NULL and no earlier call gave them");
        *grads = h->last_grads.data();
    }
    return APEXW_OK;
}

bool streams(const apexw_opt *h) {
    return h->cache_policy == 0 ? h->streaming_auto : h->cache_policy == 1;
}

// The carried step: forced, or by default for every list without an empty
// tensor (steps with hyperparameters in device memory and steps being
// captured into a graph take another mode).
bool carry_launch(const apexw_opt *h) {
    return h->carry_ok && (h->launch_mode == 3 || h->launch_mode == 0) && !h->graph_steps;
}

// The single launch: forced, or by default for the lists it is made for
// (also when mode 3 is asked for but a step cannot take it).
bool single_launch(const apexw_opt *h) {
    return h->launch_mode == 2 ||
           ((h->launch_mode == 0 || h->launch_mode == 3) && h->single_ok && !streams(h));
}

int launch_cap(const apexw_opt *h) { return h->wg_override > 0 ? h->wg_override : (int)kMaxGrid; }

// Workgroups of a read pass over a launch of `tiles` tiles: a workgroup takes
// groups of kReadBatch tiles (read_groups() of them in all), about two groups
// each, at least 2048 workgroups, a multiple of the XCD count (one set per
// XCD).  Results do not depend on it.
int64_t read_pass_grid(const apexw_opt *h, int64_t tiles) {
    const int64_t groups = read_groups(ceil_div(tiles, kXcds));
    if (h->wg_override > 0) return std::min<int64_t>(groups, h->wg_override);
    const int64_t g = round_up(std::max<int64_t>(ceil_div(groups, 2), 2048), kXcds);
    return std::min(groups, g);
}

// One fp64 partial per read group, launch after launch, for the norm pass.
int64_t norm_partials(const apexw_opt *h) {
    int64_t n = 0;
    for (const Launch &L : h->launches) n += read_groups(L.table_stride);
    return n;
}

// Scratch of the norm pass that allocates nothing: a file-scope device array
// of kScratchBytes that every call on a GPU shares (each GPU has its own
// copy).  Layout: the per-group partials from offset 0, the kReduceBlocks
// second-stage sums at kScratchPartials2 -- 8 MiB is room for 1,048,320
// read groups, lists of up to about 1.07e9 elements.
constexpr int64_t kScratchBytes = (int64_t)8 << 20;
constexpr int64_t kScratchPartials2 = kScratchBytes - kReduceBlocks * 8;

int64_t norm_scratch_bytes(const apexw_opt *h) {
    return norm_partials(h) * 8 + kReduceBlocks * 8;
}

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// The device address of `scratch` on `device` (current), looked up once per
// device: in host code the array's name is only a stand-in for the symbol.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
char *g_scratch[kMaxDevices] = {};

int scratch_address(int device, char **out) {
    if (device < 0 || device >= kMaxDevices)
        return fail(APEXW_EINVAL, "device %d outside 0..%d", device, kMaxDevices - 1);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch[device]) {
        void *p = nullptr;
        HIP_TRY(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        g_scratch[device] = static_cast<char *>(p);
    }
    *out = g_scratch[device];
    return APEXW_OK;
}

// The grad-norm pass of a handle with its fp64 partial sums in `partials`
// (one per read group of every launch) and `partials2` (kReduceBlocks); every
// entry the reduction reads is written by this call first.
int clip_grad_norm_with(apexw_t h, const void *const *grads, const float *inv_scale_dev,
                        double max_norm, float *found_inf_dev, double *norm_out_dev,
                        float *clip_coef_dev, void *stream, double *partials, double *partials2) {
    if (!clip_coef_dev) return fail(APEXW_EINVAL, "clip_coef_dev is NULL");
    if (!(max_norm > 0.0) || !std::isfinite(max_norm))
        return fail(APEXW_EINVAL, "max_norm must be finite and > 0");
    if (int rc = reuse_last(h, nullptr, &grads)) return rc;
    DeviceGuard guard(h->device);
    hipStream_t st = static_cast<hipStream_t>(stream);
    int rc = upload_pointer_tables(h, nullptr, grads, st);
    if (rc) return rc;
    KernelArgs a;
    std::memset(&a, 0, sizeof a);
    a.desc = reinterpret_cast<const TensorDesc *>(h->ws + h->wl.desc);
    a.grads = reinterpret_cast<const void *const *>(h->ws + h->wl.grads);
    a.tile_tensor = reinterpret_cast<const int32_t *>(h->ws + h->wl.tiles);
    a.inv_scale = inv_scale_dev;
    a.found_inf_out = found_inf_dev;
    a.partials = partials;
    a.partials2 = partials2;
    a.norm_out = norm_out_dev;
    a.clip_out = clip_coef_dev;
    a.max_norm = max_norm;
    const int64_t n_partials = norm_partials(h);
    a.n_partials = n_partials;
    const bool streaming = streams(h);
    // every group writes its partial (0 without a grad), so no launch is skipped
    int64_t group_begin = 0;
    for (const Launch &L : h->launches) {
        a.group_begin = group_begin;
        group_begin += read_groups(L.table_stride);
        if (L.tile_count == 0) continue;
        a.tile_begin = L.tile_begin;
        a.tile_count = L.tile_count;
        a.table_begin = L.table_begin;
        a.table_stride = L.table_stride;
        const int64_t wg = read_pass_grid(h, L.tile_count);
        kernel_fn k = L.gt == APEXW_F32
                          ? (streaming ? grad_norm_partials_kernel<APEXW_F32, true>
                                       : grad_norm_partials_kernel<APEXW_F32, false>)
                          : (streaming ? grad_norm_partials_kernel<APEXW_BF16, true>
                                       : grad_norm_partials_kernel<APEXW_BF16, false>);
        hipLaunchKernelGGL(k, dim3((unsigned)wg), dim3(kThreads), 0, st, a);
        HIP_TRY(hipGetLastError());
    }
    if (h->n > 0 && n_partials > kDirectPartials) {
        hipLaunchKernelGGL(grad_norm_reduce_kernel, dim3(kReduceBlocks), dim3(kReduceThreads), 0,
                           st, a);
        HIP_TRY(hipGetLastError());
    } else {
        a.partials2 = nullptr;                // the final kernel sums the partials
        if (h->n == 0) a.partials = nullptr;  // no workspace: the norm is 0
    }
    hipLaunchKernelGGL(grad_norm_final_kernel, dim3(1), dim3(kReduceThreads), 0, st, a);
    HIP_TRY(hipGetLastError());
    return APEXW_OK;
}

}  // namespace

// ======================================================================= ABI

extern "C" {

const char *apexw_last_error(void) { return g_err; }

int apexw_state_bytes(int32_t n_tensors, const int64_t *numel, int32_t fmt,
                      size_t *out_bytes) {
    if (!out_bytes) return fail(APEXW_EINVAL, "out_bytes is NULL");
    int64_t total = 0;
    int rc = compute_layout(n_tensors, numel, fmt, nullptr, nullptr, &total);
    if (rc) return rc;
    *out_bytes = (size_t)total;
    return APEXW_OK;
}

int apexw_state_layout(int32_t n_tensors, const int64_t *numel, int32_t fmt,
                       apexw_tensor_state *out_tensors, int64_t *out_steps) {
    if (n_tensors > 0 && !out_tensors) return fail(APEXW_EINVAL, "out_tensors is NULL");
    if (!out_steps) return fail(APEXW_EINVAL, "out_steps is NULL");
    return compute_layout(n_tensors, numel, fmt, out_tensors, out_steps, nullptr);
}

int apexw_workspace_bytes(int32_t n_tensors, const int64_t *numel, size_t *out_bytes) {
    if (!out_bytes) return fail(APEXW_EINVAL, "out_bytes is NULL");
    int rc = check_list(n_tensors, numel);
    if (rc) return rc;
    *out_bytes = (size_t)ws_layout(n_tensors, numel).total;
    return APEXW_OK;
}

int apexw_create(int32_t n_tensors, const int64_t *numel, const int32_t *param_dtype,
                 const int32_t *grad_dtype, const int32_t *group_of, int32_t n_groups,
                 int32_t fmt, void *state_dev, size_t state_bytes, void *workspace_dev,
                 size_t workspace_bytes, void *stream, apexw_t *out) {
    if (!out) return fail(APEXW_EINVAL, "out is NULL");
    *out = nullptr;
    int rc = check_list(n_tensors, numel);
    if (rc) return rc;
    if (moment_bytes(fmt) == 0) return fail(APEXW_EDTYPE, "unknown state format %d", fmt);
    if (n_groups < 1 || n_groups > APEXW_MAX_GROUPS)
        return fail(APEXW_EINVAL, "n_groups must be in 1..%d (got %d)", APEXW_MAX_GROUPS, n_groups);
    if (n_tensors > 0 && (!param_dtype || !grad_dtype || !group_of))
        return fail(APEXW_EINVAL, "param_dtype, grad_dtype and group_of must not be NULL");
    for (int32_t i = 0; i < n_tensors; ++i) {
        if (param_dtype[i] != APEXW_F32 && param_dtype[i] != APEXW_BF16)
            return fail(APEXW_EDTYPE, "param_dtype[%d] = %d is not fp32 or bf16", i, param_dtype[i]);
        if (grad_dtype[i] != APEXW_F32 && grad_dtype[i] != APEXW_BF16)
            return fail(APEXW_EDTYPE, "grad_dtype[%d] = %d is not fp32 or bf16", i, grad_dtype[i]);
        if (group_of[i] < 0 || group_of[i] >= n_groups)
            return fail(APEXW_EINVAL, "group_of[%d] = %d outside 0..%d", i, group_of[i], n_groups - 1);
        if (numel[i] > ((int64_t)1 << 40))
            return fail(APEXW_EINVAL, "numel[%d] too large", i);
    }
    int64_t need_state = 0;
    compute_layout(n_tensors, numel, fmt, nullptr, nullptr, &need_state);
    const WsLayout wl = ws_layout(n_tensors, numel);
    if (wl.n_tiles > INT32_MAX) return fail(APEXW_EINVAL, "too many tiles");
    if ((!state_dev && need_state > 0) || (!workspace_dev && wl.total > 0))
        return fail(APEXW_EINVAL, "state_dev and workspace_dev must not be NULL");
    if (((uintptr_t)state_dev | (uintptr_t)workspace_dev) & (kTableAlign - 1))
        return fail(APEXW_EINVAL, "state_dev and workspace_dev must be 256-byte aligned");
    if ((int64_t)state_bytes < need_state)
        return fail(APEXW_ENOSPC, "state buffer has %zu bytes, needs %lld", state_bytes,
                    (long long)need_state);
    if ((int64_t)workspace_bytes < wl.total)
        return fail(APEXW_ENOSPC, "workspace has %zu bytes, needs %lld", workspace_bytes,
                    (long long)wl.total);

    apexw_opt *h = new (std::nothrow) apexw_opt;
    if (!h) return fail(APEXW_ENOMEM, "host allocation failed");
    try {
        h->n = n_tensors;
        h->n_groups = n_groups;
        h->fmt = fmt;
        h->numel.assign(numel, numel + n_tensors);
        h->pdt.assign(param_dtype, param_dtype + n_tensors);
        h->gdt.assign(grad_dtype, grad_dtype + n_tensors);
        h->group_of.assign(group_of, group_of + n_tensors);
        h->layout.resize(n_tensors);
        compute_layout(n_tensors, numel, fmt, h->layout.data(), &h->steps_off, nullptr);
        h->desc.resize(n_tensors);
        h->last_params.resize(n_tensors);
        h->last_grads.resize(n_tensors);
    } catch (const std::bad_alloc &) {
        delete h;
        return fail(APEXW_ENOMEM, "host allocation failed");
    }
    h->state = static_cast<char *>(state_dev);
    h->ws = static_cast<char *>(workspace_dev);
    h->wl = wl;

    auto bail = [&](int code) { release(h); return code; };
#define TRY(call)                                                             \
    do {                                                                      \
        hipError_t e_ = (call);                                               \
        if (e_ != hipSuccess)                                                 \
            return bail(fail(APEXW_EHIP, "%s failed: %s", #call,              \
                             hipGetErrorString(e_)));                         \
    } while (0)

    TRY(hipGetDevice(&h->device));
    TRY(hipDeviceGetAttribute(&h->cu_count, hipDeviceAttributeMultiprocessorCount, h->device));
    TRY(hipDeviceGetAttribute(&h->lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              h->device));
    TRY(hipDeviceGetAttribute(&h->lds_per_block, hipDeviceAttributeMaxSharedMemoryPerBlock,
                              h->device));

    // static tables: the tensor of every tile, tiles grouped by dtype pair;
    // (build_plan: logical tile k of a launch at table_position(begin, stride, k))
    {
        int64_t touched = need_state;
        for (int32_t i = 0; i < n_tensors; ++i)
            touched += numel[i] * ((param_dtype[i] == APEXW_F32 ? 4 : 2) +
                                   (grad_dtype[i] == APEXW_F32 ? 4 : 2));
        h->streaming_auto = touched >= kStreamingBytes;
    }
    Plan plan;
    if (!build_plan(n_tensors, numel, param_dtype, grad_dtype, &plan))
        return bail(fail(APEXW_ENOMEM, "host allocation failed"));
    const std::vector<int32_t> &tiles = plan.tiles;
    try {
        h->launches = plan.launches;
        h->tensor_list = plan.tensor_list;
        h->first_tile = plan.first_tile;
        h->table_entries = (int64_t)tiles.size();
        // the single launch needs a tile in every launch (a launch of empty
        // tensors only advances counters, which the prepare kernel does)
        h->single_ok = wl.single && n_tensors > 0;
        for (const Launch &L : h->launches) h->single_ok = h->single_ok && L.tile_count > 0;
        h->carry_ok = n_tensors > 0;
        for (int32_t i = 0; i < n_tensors; ++i) h->carry_ok = h->carry_ok && numel[i] > 0;
        h->carry_beta1.assign((size_t)n_groups, 0.0);
        h->carry_beta2.assign((size_t)n_groups, 0.0);
    } catch (const std::bad_alloc &) {
        return bail(fail(APEXW_ENOMEM, "host allocation failed"));
    }

    // pinned staging: the ring for per-call uploads (descriptors + grad
    // pointers), also used once here for the whole workspace: descriptors
    // (parameter pointers arrive with the first step), grad pointers and
    // step records zero, the tile table
    const int64_t per_call = wl.records;
    const int64_t static_bytes = wl.total;
    h->slot_bytes = std::max<int64_t>(per_call, kTableAlign);
    const int64_t pinned_bytes =
        std::max<int64_t>(h->slot_bytes * apexw_opt::kRing, static_bytes);
    TRY(hipHostMalloc((void **)&h->pinned, (size_t)std::max<int64_t>(pinned_bytes, kTableAlign),
                      hipHostMallocDefault));
    for (int s = 0; s < apexw_opt::kRing; ++s) TRY(hipEventCreateWithFlags(&h->ev[s], hipEventDisableTiming));

    hipStream_t st = static_cast<hipStream_t>(stream);
    char *stage = h->pinned;
    std::memset(stage, 0, (size_t)static_bytes);
    fill_descriptors(h, nullptr);
    if (n_tensors > 0)
        std::memcpy(stage + wl.desc, h->desc.data(), (size_t)n_tensors * sizeof(TensorDesc));
    if (!tiles.empty())
        std::memcpy(stage + wl.tiles, tiles.data(), tiles.size() * 4);
    if (wl.single && n_tensors > 0)           // arrival counters stay zero
        std::memcpy(stage + wl.tensors, h->tensor_list.data(), (size_t)n_tensors * 4);
    if (static_bytes > 0) std::memcpy(stage + wl.consts, kConsts, sizeof(kConsts));
    if (static_bytes > 0)
        TRY(hipMemcpyAsync(h->ws, stage, (size_t)static_bytes, hipMemcpyHostToDevice, st));
    const int64_t words = need_state / 4;
    if (words > 0) {
        const int64_t blocks = std::min<int64_t>(ceil_div(words, 256), 8 * (int64_t)h->cu_count);
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                           reinterpret_cast<uint32_t *>(h->state), words);
        TRY(hipGetLastError());
    }
    TRY(hipStreamSynchronize(st));
#undef TRY
    *out = h;
    return APEXW_OK;
}

int apexw_step(apexw_t h, const apexw_group *groups, int32_t n_groups, void *const *params,
               const void *const *grads, const float *found_inf_dev, void *stream) {
    apexw_step_options o = {nullptr, nullptr, found_inf_dev, nullptr};
    return apexw_step_ex(h, groups, n_groups, params, grads, &o, stream);
}

int apexw_step_scaled(apexw_t h, const apexw_group *groups, int32_t n_groups,
                      void *const *params, const void *const *grads,
                      const float *inv_scale_dev, const float *found_inf_dev, void *stream) {
    apexw_step_options o = {inv_scale_dev, nullptr, found_inf_dev, nullptr};
    return apexw_step_ex(h, groups, n_groups, params, grads, &o, stream);
}

int apexw_step_device(apexw_t h, const apexw_group *groups_dev, int32_t n_groups,
                      void *const *params, const void *const *grads,
                      const float *inv_scale_dev, const float *found_inf_dev, void *stream) {
    if (!groups_dev) return fail(APEXW_EINVAL, "groups_dev is NULL");
    apexw_step_options o = {inv_scale_dev, nullptr, found_inf_dev, groups_dev};
    return apexw_step_ex(h, nullptr, n_groups, params, grads, &o, stream);
}

int apexw_step_ex(apexw_t h, const apexw_group *groups, int32_t n_groups, void *const *params,
                  const void *const *grads, const apexw_step_options *opts, void *stream) {
    static const apexw_step_options none = {nullptr, nullptr, nullptr, nullptr};
    const apexw_step_options &o = opts ? *opts : none;
    if (!h) return fail(APEXW_EINVAL, "handle is NULL");
    if (n_groups != h->n_groups)
        return fail(APEXW_EINVAL, "n_groups is %d, the handle was created with %d", n_groups,
                    h->n_groups);
    if (!groups && !o.groups_dev) return fail(APEXW_EINVAL, "groups is NULL");
    if (int rc = reuse_last(h, &params, &grads)) return rc;
    const float *inv_scale_dev = o.inv_scale;
    const float *found_inf_dev = o.found_inf;
    if (o.groups_dev) groups = nullptr;

    KernelArgs a;
    std::memset(&a, 0, sizeof a);
    a.groups_dev = o.groups_dev;
    a.clip_coef = o.clip_coef;
    for (int32_t g = 0; groups && g < n_groups; ++g) {
        const apexw_group &G = groups[g];
        if (!finite_nonneg(G.lr) || !finite_nonneg(G.eps) || !finite_nonneg(G.weight_decay) ||
            !(G.beta1 >= 0.0 && G.beta1 < 1.0) || !(G.beta2 >= 0.0 && G.beta2 < 1.0))
            return fail(APEXW_EINVAL,
                        "group %d: need lr, eps, weight_decay finite and >= 0 and 0 <= beta < 1", g);
        // scalars formed in fp64 and rounded once to fp32
        GroupScalars &S = a.groups[g];
        S.beta1 = (float)G.beta1;
        S.one_minus_beta1 = (float)(1.0 - G.beta1);
        S.beta2 = (float)G.beta2;
        S.one_minus_beta2 = (float)(1.0 - G.beta2);
        S.lr = (float)G.lr;
        S.decay = (float)(1.0 - G.lr * G.weight_decay);
        S.eps = (float)G.eps;
        S.x_lo = S.eps <= 0x1p28f ? 0x1p-96f : INFINITY;    // as step_x_lo (eps >= 0 here)
        S.beta1_d = G.beta1;
        S.beta2_d = G.beta2;
    }
    for (int32_t i = 0; i < h->n; ++i)
        if (params[i] == nullptr && h->numel[i] > 0)
            return fail(APEXW_EINVAL, "params[%d] is NULL", i);

    DeviceGuard guard(h->device);
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipStreamCaptureStatus cap_status = hipStreamCaptureStatusNone;
    HIP_TRY(hipStreamIsCapturing(st, &cap_status));
    const bool capturing = cap_status != hipStreamCaptureStatusNone;
    if (capturing) h->graph_steps = true;
    int rc = upload_pointer_tables(h, params, grads, st);
    if (rc) return rc;

    bool any_grad = false;
    for (int32_t i = 0; i < h->n && !any_grad; ++i) any_grad = grads[i] != nullptr;
    if (!any_grad) return APEXW_OK;           // nothing to update, nothing advances

    a.desc = reinterpret_cast<const TensorDesc *>(h->ws + h->wl.desc);
    a.grads = reinterpret_cast<const void *const *>(h->ws + h->wl.grads);
    a.tile_tensor = reinterpret_cast<const int32_t *>(h->ws + h->wl.tiles);
    a.records = reinterpret_cast<StepRecord *>(h->ws + h->wl.records);
    a.steps = reinterpret_cast<int32_t *>(h->state + h->steps_off);
    const bool scaled = inv_scale_dev != nullptr || a.clip_coef != nullptr;
    const float *consts = reinterpret_cast<const float *>(h->ws + h->wl.consts);
    a.found_inf = found_inf_dev != nullptr ? found_inf_dev : consts;        // 0: no skip
    a.inv_scale = inv_scale_dev != nullptr ? inv_scale_dev : consts + 1;    // 1: unscaled
    a.clip_coef = a.clip_coef != nullptr ? a.clip_coef : consts + 1;        // 1: unclipped
    a.n_tensors = h->n;
    const bool streaming = streams(h);
    // the carried step needs the hyperparameters on the host (their betas
    // form the carried corrections) and a step that runs now: a captured
    // graph replays its launches without this host state moving on (and once
    // one has been captured, carry_launch refuses every later step)
    const bool carry = groups && carry_launch(h) && !capturing;
    if (!carry) h->carry_valid = false;
    const bool single = !carry && single_launch(h);
    bool carry_broken = false;                // a launch left out: restart the chain
    if (carry) {
        BiasRecord *bias = reinterpret_cast<BiasRecord *>(h->ws + h->wl.bias);
        bool same = h->carry_valid;
        for (int32_t g = 0; same && g < n_groups; ++g)
            same = groups[g].beta1 == h->carry_beta1[(size_t)g] &&
                   groups[g].beta2 == h->carry_beta2[(size_t)g];
        a.bias_cur = bias + (size_t)h->carry_parity * (size_t)h->n;
        a.bias_next = bias + (size_t)(1 - h->carry_parity) * (size_t)h->n;
        if (!same) {                          // (re)start from the counters as they stand
            KernelArgs ai = a;
            ai.bias_next = bias + (size_t)h->carry_parity * (size_t)h->n;
            hipLaunchKernelGGL(carry_init_kernel, dim3((unsigned)ceil_div(h->n, kPrepThreads)),
                               dim3(kPrepThreads), 0, st, ai);
            HIP_TRY(hipGetLastError());
            for (int32_t g = 0; g < n_groups; ++g) {
                h->carry_beta1[(size_t)g] = groups[g].beta1;
                h->carry_beta2[(size_t)g] = groups[g].beta2;
            }
        }
        h->carry_valid = false;               // until every launch of the step is queued
    } else if (single) {
        a.tensor_list = reinterpret_cast<const int32_t *>(h->ws + h->wl.tensors);
    } else {
        hipLaunchKernelGGL(adamw_prepare_kernel, dim3((unsigned)ceil_div(h->n, kPrepThreads)),
                           dim3(kPrepThreads), 0, st, a);
        HIP_TRY(hipGetLastError());
    }
    const int64_t cap = launch_cap(h);
    for (size_t li = 0; li < h->launches.size(); ++li) {
        const Launch &L = h->launches[li];
        // residency cap: the dynamic LDS a workgroup reserves (it uses none)
        const int occ = h->occupancy > 0 ? h->occupancy : default_occupancy(h->fmt, L.pt, L.gt);
        const unsigned lds = occ > 0 ? (unsigned)std::min(h->lds_per_cu / occ, h->lds_per_block) : 0u;
        // only empty tensors: their counters advanced in the prepare kernel
        // (the single launch is not used for lists with such a launch)
        if (L.tile_count == 0) continue;
        bool any = false;                     // no grads in this launch: skip it
        for (int32_t j = 0; j < L.tensor_count && !any; ++j)
            any = grads[h->tensor_list[L.tensor_begin + j]] != nullptr;
        if (!any) {
            carry_broken = true;              // its tensors carry nothing forward
            continue;
        }
        a.tile_begin = L.tile_begin;
        a.tile_count = L.tile_count;
        a.table_begin = L.table_begin;
        a.table_stride = L.table_stride;
        const int64_t wg = std::min(L.tile_count, cap);
        // few tensors, uncapped, cached accesses: the few-tensor kernel, for
        // which a small list's step is the latency of its metadata chain.  A
        // streamed launch (a list past 64 MB) reads the tile table instead:
        // bandwidth-bound, it measured 0.3-0.5% faster that way (few_large
        // 1.9418 against 1.9471 ms, bf16_state 1.3406 against 1.3441 ms,
        // four alternating runs each on MI355X).  No tensor is empty here:
        // the carried step takes no list with an empty tensor.
        a.few = 0;
        if (carry && !streaming && wg == L.tile_count &&
            L.tensor_count <= kFewTensors) {                      // carry_ok: none empty
            a.few = L.tensor_count;
            for (int32_t j = 0; j < kFewTensors; ++j) {
                const int32_t t = h->tensor_list[(size_t)(L.tensor_begin + std::min(j, L.tensor_count - 1))];
                a.few_tensor[j] = t;
                a.few_first[j] = (int32_t)(h->first_tile[(size_t)t] - L.tile_begin);
            }
        }
        if (carry) {
            hipLaunchKernelGGL(carry_kernel_for(h->fmt, L.pt, L.gt, streaming, scaled, wg == L.tile_count,
                                                a.few > 0),
                               dim3((unsigned)carry_grid(h->fmt, L.tile_count, wg)), dim3(kThreads),
                               lds, st, a);
        } else if (single) {
            a.tensor_begin = L.tensor_begin;
            a.tensor_count = L.tensor_count;
            a.done = reinterpret_cast<uint32_t *>(h->ws + h->wl.done) + li * kDoneWords;
            hipLaunchKernelGGL(single_kernel_for(h->fmt, L.pt, L.gt, scaled), dim3((unsigned)wg),
                               dim3(kThreads), lds, st, a);
        } else {
            hipLaunchKernelGGL(kernel_for(h->fmt, L.pt, L.gt, streaming, scaled), dim3((unsigned)wg),
                               dim3(kThreads), lds, st, a);
        }
        HIP_TRY(hipGetLastError());
    }
    if (carry) {
        h->carry_valid = !carry_broken;
        h->carry_parity ^= 1;
    }
    return APEXW_OK;
}

int apexw_inv_scale(const float *scale_dev, float *inv_scale_dev, void *stream) {
    if (!scale_dev || !inv_scale_dev) return fail(APEXW_EINVAL, "scale_dev and inv_scale_dev must not be NULL");
    hipLaunchKernelGGL(inv_scale_kernel, dim3(1), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       scale_dev, inv_scale_dev);
    HIP_TRY(hipGetLastError());
    return APEXW_OK;
}

int apexw_unscale_check(apexw_t h, const void *const *grads, const float *inv_scale_dev,
                        float *found_inf_dev, void *stream) {
    if (!h) return fail(APEXW_EINVAL, "handle is NULL");
    if (!found_inf_dev) return fail(APEXW_EINVAL, "found_inf_dev is NULL");
    if (int rc = reuse_last(h, nullptr, &grads)) return rc;
    DeviceGuard guard(h->device);
    hipStream_t st = static_cast<hipStream_t>(stream);
    int rc = upload_pointer_tables(h, nullptr, grads, st);
    if (rc) return rc;
    KernelArgs a;
    std::memset(&a, 0, sizeof a);
    a.desc = reinterpret_cast<const TensorDesc *>(h->ws + h->wl.desc);
    a.grads = reinterpret_cast<const void *const *>(h->ws + h->wl.grads);
    a.tile_tensor = reinterpret_cast<const int32_t *>(h->ws + h->wl.tiles);
    a.inv_scale = inv_scale_dev;
    a.found_inf_out = found_inf_dev;
    const bool streaming = streams(h);
    for (const Launch &L : h->launches) {
        if (L.tile_count == 0) continue;
        bool any = false;
        for (int32_t j = 0; j < L.tensor_count && !any; ++j)
            any = grads[h->tensor_list[L.tensor_begin + j]] != nullptr;
        if (!any) continue;
        a.tile_begin = L.tile_begin;
        a.tile_count = L.tile_count;
        a.table_begin = L.table_begin;
        a.table_stride = L.table_stride;
        const int64_t wg = read_pass_grid(h, L.tile_count);
        kernel_fn k = L.gt == APEXW_F32
                          ? (streaming ? unscale_check_kernel<APEXW_F32, true> : unscale_check_kernel<APEXW_F32, false>)
                          : (streaming ? unscale_check_kernel<APEXW_BF16, true> : unscale_check_kernel<APEXW_BF16, false>);
        hipLaunchKernelGGL(k, dim3((unsigned)wg), dim3(kThreads), 0, st, a);
        HIP_TRY(hipGetLastError());
    }
    return APEXW_OK;
}

int apexw_clip_grad_norm(apexw_t h, const void *const *grads, const float *inv_scale_dev,
                         double max_norm, float *found_inf_dev, double *norm_out_dev,
                         float *clip_coef_dev, void *stream) {
    if (!h) return fail(APEXW_EINVAL, "handle is NULL");
    return clip_grad_norm_with(h, grads, inv_scale_dev, max_norm, found_inf_dev, norm_out_dev,
                               clip_coef_dev, stream,
                               reinterpret_cast<double *>(h->ws + h->wl.partials),
                               reinterpret_cast<double *>(h->ws + h->wl.partials2));
}

int apexw_clip_grad_norm_noalloc(apexw_t h, const void *const *grads, const float *inv_scale_dev,
                                 double max_norm, float *found_inf_dev, double *norm_out_dev,
                                 float *clip_coef_dev, void *stream) {
    if (!h) return fail(APEXW_EINVAL, "handle is NULL");
    const int64_t need = norm_scratch_bytes(h);
    if (need > kScratchBytes)
        return fail(APEXW_ENOSPC, "the grad-norm partial sums of this list need %lld bytes; the "
                    "library's static scratch holds %lld (use apexw_clip_grad_norm)",
                    (long long)need, (long long)kScratchBytes);
    DeviceGuard guard(h->device);
    char *base = nullptr;
    if (int rc = scratch_address(h->device, &base)) return rc;
    // the per-group partials from the start, the second-stage sums at the end
    double *partials = reinterpret_cast<double *>(base);
    double *partials2 = reinterpret_cast<double *>(base + kScratchPartials2);
    if (reinterpret_cast<char *>(partials + norm_partials(h)) > reinterpret_cast<char *>(partials2) ||
        reinterpret_cast<char *>(partials2 + kReduceBlocks) > base + kScratchBytes)
        return fail(APEXW_ENOSPC, "grad-norm scratch layout exceeds the static array");
    return clip_grad_norm_with(h, grads, inv_scale_dev, max_norm, found_inf_dev, norm_out_dev,
                               clip_coef_dev, stream, partials, partials2);
}

// ---------------------------------------------------------------- checkpoint
//
// Blob: header | numel[n] int64 | param_dtype[n] int32 | grad_dtype[n] int32
// | group_of[n] int32 | groups[n_groups] apexw_group | pad to 256 | the raw
// state buffer (moments, block scales, step counters) in the layout of
// apexw_state_layout.

namespace {

struct BlobHeader {
    char magic[8];
    uint32_t version;
    int32_t fmt;
    int32_t n_tensors;
    int32_t n_groups;
    uint64_t state_bytes;
    uint64_t payload_offset;
};
const char kMagic[8] = {'A', 'P', 'E', 'X', 'W', 'S', 'T', '1'};

uint64_t blob_payload_offset(const apexw_opt *h) {
    const uint64_t n = (uint64_t)h->n;
    const uint64_t meta = sizeof(BlobHeader) + n * (8 + 4 + 4 + 4) +
                          (uint64_t)h->n_groups * sizeof(apexw_group);
    return (uint64_t)round_up((int64_t)meta, kTableAlign);
}

uint64_t state_total(const apexw_opt *h) { return (uint64_t)(h->steps_off + 4 * (int64_t)h->n); }

}  // namespace

int apexw_export_bytes(apexw_t h, size_t *out_bytes) {
    if (!h || !out_bytes) return fail(APEXW_EINVAL, "NULL argument");
    *out_bytes = (size_t)(blob_payload_offset(h) + state_total(h));
    return APEXW_OK;
}

int apexw_export_state(apexw_t h, const apexw_group *groups, int32_t n_groups, void *dst_host,
                       size_t dst_bytes, void *stream) {
    if (!h || !dst_host || !groups) return fail(APEXW_EINVAL, "NULL argument");
    if (n_groups != h->n_groups)
        return fail(APEXW_EINVAL, "n_groups is %d, the handle has %d", n_groups, h->n_groups);
    const uint64_t off = blob_payload_offset(h), sb = state_total(h);
    if (dst_bytes < off + sb)
        return fail(APEXW_ENOSPC, "destination has %zu bytes, needs %llu", dst_bytes,
                    (unsigned long long)(off + sb));
    char *p = static_cast<char *>(dst_host);
    std::memset(p, 0, (size_t)off);
    BlobHeader hd;
    std::memcpy(hd.magic, kMagic, 8);
    hd.version = 1;
    hd.fmt = h->fmt;
    hd.n_tensors = h->n;
    hd.n_groups = h->n_groups;
    hd.state_bytes = sb;
    hd.payload_offset = off;
    std::memcpy(p, &hd, sizeof hd);
    char *q = p + sizeof hd;
    const size_t n = (size_t)h->n;
    std::memcpy(q, h->numel.data(), n * 8); q += n * 8;
    std::memcpy(q, h->pdt.data(), n * 4); q += n * 4;
    std::memcpy(q, h->gdt.data(), n * 4); q += n * 4;
    std::memcpy(q, h->group_of.data(), n * 4); q += n * 4;
    std::memcpy(q, groups, (size_t)n_groups * sizeof(apexw_group));
    DeviceGuard guard(h->device);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (sb > 0) HIP_TRY(hipMemcpyAsync(p + off, h->state, (size_t)sb, hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
    return APEXW_OK;
}

int apexw_import_state(apexw_t h, const void *src_host, size_t src_bytes, apexw_group *groups_out,
                       int32_t n_groups, void *stream) {
    if (!h || !src_host) return fail(APEXW_EINVAL, "NULL argument");
    const char *p = static_cast<const char *>(src_host);
    BlobHeader hd;
    if (src_bytes < sizeof hd) return fail(APEXW_EINVAL, "blob too short for its header");
    std::memcpy(&hd, p, sizeof hd);
    if (std::memcmp(hd.magic, kMagic, 8) != 0 || hd.version != 1)
        return fail(APEXW_EINVAL, "not an optimizer-state blob of this format");
    if (hd.fmt != h->fmt || hd.n_tensors != h->n || hd.n_groups != h->n_groups)
        return fail(APEXW_EINVAL, "blob is for format %d, %d tensors, %d groups; the handle has "
                    "%d, %d, %d", hd.fmt, hd.n_tensors, hd.n_groups, h->fmt, h->n, h->n_groups);
    const uint64_t off = blob_payload_offset(h), sb = state_total(h);
    if (hd.payload_offset != off || hd.state_bytes != sb || src_bytes < off + sb)
        return fail(APEXW_EINVAL, "blob sizes do not match the handle's state layout");
    const char *q = p + sizeof hd;
    const size_t n = (size_t)h->n;
    if (std::memcmp(q, h->numel.data(), n * 8) != 0 ||
        std::memcmp(q + n * 8, h->pdt.data(), n * 4) != 0 ||
        std::memcmp(q + n * 12, h->gdt.data(), n * 4) != 0 ||
        std::memcmp(q + n * 16, h->group_of.data(), n * 4) != 0)
        return fail(APEXW_EINVAL, "blob's tensor sizes, dtypes or groups differ from the handle's");
    if (groups_out) {
        if (n_groups != h->n_groups)
            return fail(APEXW_EINVAL, "n_groups is %d, the handle has %d", n_groups, h->n_groups);
        std::memcpy(groups_out, q + n * 20, (size_t)n_groups * sizeof(apexw_group));
    }
    DeviceGuard guard(h->device);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (sb > 0) HIP_TRY(hipMemcpyAsync(h->state, p + off, (size_t)sb, hipMemcpyHostToDevice, st));
    HIP_TRY(hipStreamSynchronize(st));
    h->carry_valid = false;                  // new counters: the carried corrections are stale
    return APEXW_OK;
}

int apexw_read_steps(apexw_t h, int32_t *host_out, void *stream) {
    if (!h) return fail(APEXW_EINVAL, "handle is NULL");
    if (h->n > 0 && !host_out) return fail(APEXW_EINVAL, "host_out is NULL");
    if (h->n == 0) return APEXW_OK;
    DeviceGuard guard(h->device);
    hipStream_t st = static_cast<hipStream_t>(stream);
    HIP_TRY(hipMemcpyAsync(host_out, h->state + h->steps_off, (size_t)h->n * 4,
                           hipMemcpyDeviceToHost, st));
    HIP_TRY(hipStreamSynchronize(st));
    return APEXW_OK;
}

int apexw_launch_info(apexw_t h, int32_t *tile_elems, int32_t *n_tiles, int32_t *workgroups) {
    if (!h) return fail(APEXW_EINVAL, "handle is NULL");
    if (tile_elems) *tile_elems = kTile;
    if (n_tiles) *n_tiles = (int32_t)h->wl.n_tiles;
    if (workgroups) {
        const int64_t cap = h->wg_override > 0 ? h->wg_override : kMaxGrid;
        int64_t wg = 0;
        for (const Launch &L : h->launches) wg = std::max(wg, std::min(L.tile_count, cap));
        *workgroups = (int32_t)wg;
    }
    return APEXW_OK;
}

int apexw_set_workgroups(apexw_t h, int32_t workgroups) {
    if (!h) return fail(APEXW_EINVAL, "handle is NULL");
    if (workgroups < 0) return fail(APEXW_EINVAL, "workgroups must be >= 0");
    h->wg_override = workgroups;
    return APEXW_OK;
}

int apexw_set_occupancy(apexw_t h, int32_t workgroups_per_cu) {
    if (!h) return fail(APEXW_EINVAL, "handle is NULL");
    if (workgroups_per_cu < 0) return fail(APEXW_EINVAL, "workgroups_per_cu must be >= 0");
    h->occupancy = workgroups_per_cu;
    return APEXW_OK;
}

int apexw_set_cache_policy(apexw_t h, int32_t policy) {
    if (!h) return fail(APEXW_EINVAL, "handle is NULL");
    if (policy < 0 || policy > 2) return fail(APEXW_EINVAL, "policy must be 0, 1 or 2");
    h->cache_policy = policy;
    return APEXW_OK;
}

int apexw_set_launch_mode(apexw_t h, int32_t mode) {
    if (!h) return fail(APEXW_EINVAL, "handle is NULL");
    if (mode < 0 || mode > 3) return fail(APEXW_EINVAL, "mode must be 0, 1, 2 or 3");
    if (mode == 2 && !h->single_ok)
        return fail(APEXW_EINVAL, "the single-launch step needs a non-empty list of at most %lld "
                                  "tiles with a tile in every dtype pair it uses",
                    (long long)kSingleLaunchTiles);
    if (mode == 3 && !h->carry_ok)
        return fail(APEXW_EINVAL, "the carried step needs a non-empty list without empty tensors");
    h->launch_mode = mode;
    h->carry_valid = false;                  // also: counters written by the caller are re-read
    h->graph_steps = false;                  // the caller replays no captured step any more
    return APEXW_OK;
}

int apexw_get_launch_mode(apexw_t h, int32_t *mode) {
    if (!h || !mode) return fail(APEXW_EINVAL, "NULL argument");
    *mode = carry_launch(h) ? 3 : single_launch(h) ? 2 : 1;
    return APEXW_OK;
}

int apexw_get_occupancy(apexw_t h, int32_t *workgroups_per_cu) {
    if (!h || !workgroups_per_cu) return fail(APEXW_EINVAL, "NULL argument");
    int32_t occ = 0;
    for (const Launch &L : h->launches)
        occ = std::max<int32_t>(occ, h->occupancy > 0 ? h->occupancy
                                                      : default_occupancy(h->fmt, L.pt, L.gt));
    *workgroups_per_cu = occ;
    return APEXW_OK;
}

int apexw_destroy(apexw_t h) {
    if (!h) return fail(APEXW_EINVAL, "handle is NULL");
    DeviceGuard guard(h->device);
    release(h);
    return APEXW_OK;
}

}  // extern "C"
