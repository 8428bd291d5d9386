"""Benchmark of the fused multi-tensor AdamW step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one apexw_step call over the whole parameter list of the workload
(default: 8 bf16 [8192,8192] parameters with fp32 grads and fp32 moments,
536,870,912 params), with parameters, grads and state already resident in
HBM.  W untimed steps, then K timed steps between a barrier-free
torch.cuda.synchronize() on both sides.  Prints one JSON line: params/s
(value), achieved HBM GB/s on the algorithmic byte count and its fraction of
the 8 TB/s peak, the roofline object of the update kernel (its average
duration from HIP events recorded on the stream the kernel runs on), and the
oracle's throughput on a bounded sample, timed on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

# launch modes of the step (apexw_get_launch_mode) and the update kernel each runs
MODE_NAMES = {1: "prepare + update", 2: "single launch",
              3: "carried (one launch, bias corrections from the previous step)"}
MODE_KERNELS = {1: "adamw_step_kernel", 2: "adamw_single_step_kernel", 3: "adamw_carry_step_kernel"}

METRIC = "params updated/sec + achieved HBM GB/s (% of peak) per AdamW step, 1 MI355X"
HBM_PEAK_GBPS = 8000.0

# algorithmic bytes per element: read theta, g, m, v; write theta, m, v
ELEM = {"f32": 4, "bf16": 2}
MOMENT = {"f32": 4, "bf16": 2, "q8": 1}


def algorithmic_bytes(w) -> int:
    """Bytes the method must move per step: each of theta, g, m, v read once,
    theta, m, v written once, plus (8-bit) the two block scales read and
    written and the 4-byte step counter read and written per tensor."""
    total = 0
    for n, pd, gd in zip(w.numels, w.param_dtype, w.grad_dtype):
        mb = MOMENT[w.state_fmt]
        total += n * (2 * ELEM[pd] + ELEM[gd] + 4 * mb)
        if w.state_fmt == "q8":
            total += 2 * 2 * 4 * ((n + 255) // 256)
        total += 8
    return total


def kernel_source_hash() -> str:
    """Hash of the library's code with comments and blank space removed, so
    that a comment edit does not invalidate counters taken on the same code."""
    import re
    h = hashlib.sha256()
    for rel in ("tensor_adamw_optimizer_amd/csrc/apexw.hip",
                "tensor_adamw_optimizer_amd/csrc/apexw_kernels.hpp",
                "tensor_adamw_optimizer_amd/csrc/apexw_plan.hpp", "include/apexw.h"):
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s: float = 7.0):
    """The oracle on a bounded sample of the workload, timed on the host
    cores: a prefix of the first tensor (at most 2^24 elements), as many
    calls as fit in about budget_s, once with the single-threaded parity
    build and once with the OpenMP timing build of the same source (bitwise
    the same results).  value = the all-core figure."""
    import numpy as np
    import torch

    import oracle
    import workloads as W

    n_full = w.numels[0]
    n = min(n_full, 1 << 24)
    gen = torch.Generator().manual_seed(123)
    th0 = W.to_numpy_bits((torch.randn(n, generator=gen) * w.theta_std)
                          .to(W.TORCH_DTYPE[w.param_dtype[0]]))
    g = W.to_numpy_bits((torch.randn(n, generator=gen) * w.grad_std)
                        .to(W.TORCH_DTYPE[w.grad_dtype[0]]))
    grp = [w.groups[w.group_of[0]]]
    per_elem = (2 * ELEM[w.param_dtype[0]] + ELEM[w.grad_dtype[0]] + 4 * MOMENT[w.state_fmt]
                + (16.0 / 256 if w.state_fmt == "q8" else 0.0))

    def rate(threaded: bool):
        ref = oracle.OracleAdamW([n], w.param_dtype[:1], w.grad_dtype[:1], [0], w.state_fmt,
                                 threaded=threaded)
        th = th0.copy()
        ref.step([th], [g], grp)                              # warm-up call
        calls, t0 = 0, time.perf_counter()
        while True:
            ref.step([th], [g], grp)
            calls += 1
            el = time.perf_counter() - t0
            if el >= budget_s or calls >= 4000:
                break
        return n * calls / el, calls, el

    one, calls1, el1 = rate(False)
    threads = int(oracle.omp_lib().oracle_threads())
    many, calls_n, el_n = rate(True)
    return {
        "value": many,
        "unit": "params/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d of the %d params (prefix of tensor 0, %s params / %s grads / %s state); "
                  "all-core: OpenMP timing build of the scalar C oracle, %d threads, %d calls in "
                  "%.1f s; single-thread: the parity build, %d calls in %.1f s (gcc -O2, no "
                  "contraction; both builds give the same bits)"
                  % (n, w.n_params, w.param_dtype[0], w.grad_dtype[0], w.state_fmt, threads,
                     calls_n, el_n, calls1, el1),
        "single_thread_params_per_s": one,
        "all_core_params_per_s": many,
        "host_gbps_single_thread": one * per_elem / 1e9,
        "host_gbps_all_core": many * per_elem / 1e9,
        "algorithmic_bytes_per_param": per_elem,
        "nproc": os.cpu_count(),
        "cpus_available": len(os.sched_getaffinity(0)),
        "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS"),
        "cpu_model": _cpu_model(),
    }


def device_copy_gbps(torch, dev, stream) -> float:
    """A STREAM-style device copy for context: 1 GiB read + 1 GiB written."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    best = None
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        best = ms if best is None else min(best, ms)
    del src, dst
    return 2 * (1 << 30) / (best / 1e3) / 1e9


def torch_compare(torch, w, dev, steps, warmup):
    """torch.optim.AdamW (fused and foreach) against this library on the
    dtypes torch's fused kernel takes: grads and both moments in the
    parameter's dtype.  Context only; the grads are the workload's, cast."""
    import workloads as W
    from tensor_adamw_optimizer_amd import _lib as L

    res = {}
    params = W.init_params(w, dev)
    grads = [torch.randn(p.shape, device=dev).mul_(w.grad_std).to(p.dtype) for p in params]
    stream = torch.cuda.current_stream(dev)

    def timed(fn, host=None, key=None):
        """Average time per call between two events around `steps` calls; with
        `host`, also the host time per call (the calls only queue GPU work)."""
        for _ in range(warmup):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        t1 = time.perf_counter()
        b.record(stream)
        torch.cuda.synchronize()
        if host is not None:
            host[key] = (t1 - t0) / steps * 1e3
        return a.elapsed_time(b) / steps

    groups = []
    for gi, g in enumerate(w.groups):
        ps = [p for p, j in zip(params, w.group_of) if j == gi]
        groups.append({"params": ps, "lr": g.lr, "betas": (g.beta1, g.beta2), "eps": g.eps,
                       "weight_decay": g.weight_decay})
    for p, g in zip(params, grads):
        p.grad = g
    host = {}
    for mode in ("fused", "foreach"):
        opt = torch.optim.AdamW(groups, **{mode: True})
        ms = timed(opt.step, host, "torch_%s_adamw" % mode)
        res["torch_%s_adamw_ms" % mode] = ms
        del opt
        torch.cuda.empty_cache()
    # this library's torch wrapper, its own step(): reading .grad of every
    # parameter each step, and with flat_grads (one pointer table)
    from tensor_adamw_optimizer_amd import AdamW as ApexwAdamW
    state_name = {W.F32: "f32", W.BF16: "bf16"}[w.param_dtype[0]]
    if len(set(w.param_dtype)) == 1:
        opt = ApexwAdamW(groups, state=state_name)
        res["apexw_wrapper_step_ms"] = timed(opt.step, host, "apexw_wrapper")
        opt.close()
        del opt
        for p in params:
            p.grad = None
        opt = ApexwAdamW(groups, state=state_name, flat_grads=True)
        for p, g in zip(params, grads):
            p.grad.copy_(g)
        res["apexw_wrapper_flat_grads_step_ms"] = timed(opt.step, host, "apexw_wrapper_flat_grads")
        opt.close()
        del opt
        for p, g in zip(params, grads):
            p.grad = g
        torch.cuda.empty_cache()
    res["host_ms_per_call"] = host
    # this library on the same dtypes (moments in the parameter dtype)
    same_fmt = {W.F32: L.APEXW_STATE_F32, W.BF16: L.APEXW_STATE_BF16}[w.param_dtype[0]]
    dts = {W.F32: L.APEXW_F32, W.BF16: L.APEXW_BF16}
    if len(set(w.param_dtype)) == 1:
        sb = L.apexw_state_bytes(w.numels, same_fmt)
        wb = L.apexw_workspace_bytes(w.numels)
        state = torch.empty(sb, dtype=torch.uint8, device=dev)
        ws = torch.empty(wb, dtype=torch.uint8, device=dev)
        h = L.apexw_create(w.numels, [dts[d] for d in w.param_dtype], [dts[d] for d in w.param_dtype],
                           w.group_of, len(w.groups), same_fmt, state.data_ptr(), sb,
                           ws.data_ptr(), wb, stream.cuda_stream)
        pa = L.make_ptrs([p.data_ptr() for p in params])
        ga = L.make_ptrs([g.data_ptr() for g in grads])
        ga_groups = L.make_groups(w.groups)
        res["apexw_same_dtypes_ms"] = timed(
            lambda: L.apexw_step(h, ga_groups, len(w.groups), pa, ga, 0, stream.cuda_stream))
        L.apexw_destroy(h)
    res["compare_dtypes"] = "params, grads and moments all %s" % "+".join(sorted(set(w.param_dtype)))
    for p in params:
        p.grad = None
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="few_large",
                    choices=["few_large", "many_small", "bf16_state", "lora_q8", "tiny",
                             "few_large_shard8"])
    ap.add_argument("--workgroups", type=int, default=0, help="cap on workgroups per launch")
    ap.add_argument("--occupancy", type=int, default=0,
                    help="update workgroups per CU (0: the format's default)")
    ap.add_argument("--cache-policy", type=int, default=0,
                    help="0 auto, 1 streaming (non-temporal), 2 cached")
    ap.add_argument("--launch-mode", type=int, default=0,
                    help="0 auto, 1 prepare + update kernels, 2 single launch (small lists), "
                         "3 one launch with the bias corrections carried from the previous step")
    ap.add_argument("--amp", action="store_true",
                    help="time the mixed-precision recipe: zero found_inf, unscale-and-check "
                         "pass, update on grads scaled by 2^16")
    ap.add_argument("--clip", type=float, default=0.0,
                    help="with --amp: also clip the global grad norm to this value")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run a 1 GiB device copy 3x (counter calibration)")
    ap.add_argument("--flush-mall", action="store_true",
                    help="write 512 MiB between steps (evicts the 256 MB Infinity Cache) "
                         "and time each step on its own")
    ap.add_argument("--torch-compare", action="store_true",
                    help="also time torch.optim.AdamW (fused and foreach) and this library on "
                         "the dtypes torch supports for the workload (context only)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: it times the optimizer step on a single "
              "MI355X (--gpus 1); a step sharded over several GPUs is not implemented.",
              file=sys.stderr)
        return 2

    import torch

    import workloads as W
    from tensor_adamw_optimizer_amd import _lib as L

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    L.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = W.WORKLOADS[args.workload]()
    print("bench: workload %s, %d tensors, %d params" % (w.name, len(w.shapes), w.n_params),
          file=sys.stderr, flush=True)

    dt = {W.F32: L.APEXW_F32, W.BF16: L.APEXW_BF16}
    fmt = {W.STATE_F32: L.APEXW_STATE_F32, W.STATE_BF16: L.APEXW_STATE_BF16,
           W.STATE_Q8: L.APEXW_STATE_Q8}[w.state_fmt]
    params = W.init_params(w, dev)
    # every tensor gets a grad in the timed steps (a full update)
    grads = [g if g is not None else torch.randn(s, device=dev).mul_(w.grad_std)
             .to(W.TORCH_DTYPE[d])
             for g, s, d in zip(W.grads_for_call(w, 1, dev), w.shapes, w.grad_dtype)]
    state_bytes = L.apexw_state_bytes(w.numels, fmt)
    ws_bytes = L.apexw_workspace_bytes(w.numels)
    state = torch.empty(state_bytes, dtype=torch.uint8, device=dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    h = L.apexw_create(w.numels, [dt[d] for d in w.param_dtype], [dt[d] for d in w.grad_dtype],
                       w.group_of, len(w.groups), fmt, state.data_ptr(), state_bytes,
                       ws.data_ptr(), ws_bytes, stream.cuda_stream)
    if args.workgroups:
        L.apexw_set_workgroups(h, args.workgroups)
    if args.occupancy:
        L.apexw_set_occupancy(h, args.occupancy)
    if args.cache_policy:
        L.apexw_set_cache_policy(h, args.cache_policy)
    if args.launch_mode:
        L.apexw_set_launch_mode(h, args.launch_mode)
    launch_mode = L.apexw_get_launch_mode(h)
    occupancy = L.apexw_get_occupancy(h)
    tile, n_tiles, wgs = L.apexw_launch_info(h)
    params_arr = L.make_ptrs([p.data_ptr() for p in params])
    grads_arr = L.make_ptrs([g.data_ptr() for g in grads])
    groups_arr = L.make_groups(w.groups)
    found_inf = torch.zeros(1, dtype=torch.float32, device=dev)
    inv_scale = torch.tensor([1.0 / 65536.0], dtype=torch.float32, device=dev)
    if args.amp:
        for g in grads:
            g.mul_(65536.0)

    clip_coef = torch.ones(1, dtype=torch.float32, device=dev)

    def step():
        if args.amp and args.clip > 0:
            found_inf.zero_()
            L.apexw_clip_grad_norm(h, grads_arr, inv_scale.data_ptr(), args.clip,
                                   found_inf.data_ptr(), 0, clip_coef.data_ptr(), stream.cuda_stream)
            L.apexw_step_ex(h, groups_arr, len(w.groups), params_arr, grads_arr,
                            inv_scale_ptr=inv_scale.data_ptr(), clip_coef_ptr=clip_coef.data_ptr(),
                            found_inf_ptr=found_inf.data_ptr(), stream=stream.cuda_stream)
        elif args.amp:
            found_inf.zero_()
            L.apexw_unscale_check(h, grads_arr, inv_scale.data_ptr(), found_inf.data_ptr(),
                                  stream.cuda_stream)
            L.apexw_step_scaled(h, groups_arr, len(w.groups), params_arr, grads_arr,
                                inv_scale.data_ptr(), found_inf.data_ptr(), stream.cuda_stream)
        else:
            L.apexw_step(h, groups_arr, len(w.groups), params_arr, grads_arr,
                         found_inf.data_ptr(), stream.cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("bench: warm-up done", file=sys.stderr, flush=True)

    if args.flush_mall:
        # each step starts with a cold Infinity Cache; only the steps are timed
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
        torch.cuda.synchronize()
        for k in range(args.steps):
            flush.fill_(k & 0xFF)
            ev_a[k].record(stream)
            step()
            ev_b[k].record(stream)
        torch.cuda.synchronize()
        kernel_ms = [a.elapsed_time(b) for a, b in zip(ev_a, ev_b)]
        elapsed = sum(kernel_ms) / 1e3
        del flush
    else:
        # the timed region: K steps between two events, nothing else queued
        # (an event after every step would add several microseconds to each
        # step of a small list)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0.record(stream)
        for k in range(args.steps):
            step()
        ev1.record(stream)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        timed_avg_ms = ev0.elapsed_time(ev1) / args.steps
        # per-step spread from a second, untimed pass with an event per step
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        ev[0].record(stream)
        for k in range(args.steps):
            step()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        kernel_ms = [ev[k].elapsed_time(ev[k + 1]) for k in range(args.steps)]
    avg_kernel_s = (sum(kernel_ms) / len(kernel_ms) if args.flush_mall else timed_avg_ms) / 1e3
    print("bench: timed %d steps" % args.steps, file=sys.stderr, flush=True)
    max_mem = torch.cuda.max_memory_allocated(dev)

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    copy_gbps = device_copy_gbps(torch, dev, stream)

    ab = algorithmic_bytes(w)
    if args.amp:        # the check pass reads every grad once more
        ab += sum(n * ELEM[d] for n, d in zip(w.numels, w.grad_dtype))
    gbps = ab / avg_kernel_s / 1e9
    # the committed counters were taken in the default launch configuration
    default_launch = not (args.amp or args.workgroups or args.occupancy or args.cache_policy
                          or args.launch_mode)
    traffic = measured_traffic(w.name) if default_launch else None
    out = {
        "metric": METRIC,
        "value": w.n_params * args.steps / elapsed,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name + ("+amp" if args.amp else "") + ("+clip" if args.amp and args.clip > 0 else ""),
            "tensors": len(w.shapes),
            "params": w.n_params,
            "param_dtype": "+".join(sorted(set(w.param_dtype))),
            "grad_dtype": "+".join(sorted(set(w.grad_dtype))),
            "state": w.state_fmt,
            "groups": len(w.groups),
        },
        "hbm_gbps": (ab / (elapsed / args.steps)) / 1e9,
        "hbm_frac_of_peak": (ab / (elapsed / args.steps)) / 1e9 / HBM_PEAK_GBPS,
        "kernel_ms": {"avg": avg_kernel_s * 1e3,
                      "avg_from": "one event per flushed step" if args.flush_mall else
                      "two HIP events around the timed steps",
                      # per-step spread: an event after every step adds its
                      # own time, so these can exceed the average above
                      "per_step_min": min(kernel_ms),
                      "per_step_median": sorted(kernel_ms)[len(kernel_ms) // 2],
                      "per_step_max": max(kernel_ms),
                      "per_step_from": "flushed steps" if args.flush_mall else
                      "an untimed pass with an event after every step"},
        "residency": ("cache-resident (algorithmic bytes per step below the 256 MB "
                      "Infinity Cache)" if ab < (256 << 20) and not args.flush_mall
                      else "hbm" + (" (Infinity Cache flushed before each step)"
                                    if args.flush_mall else "")),
        "max_memory_allocated": max_mem,
        "launch": {"tile_elems": tile, "tiles": n_tiles, "workgroups": wgs,
                   "workgroups_per_cu_cap": occupancy,
                   "mode": MODE_NAMES[launch_mode]},
        "state_bytes": state_bytes,
        "roofline": {
            "bound": "hbm",
            "achieved": gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": ab,
            "kernel": MODE_KERNELS[launch_mode].replace(
                "carry_step_kernel",
                ("carry_step_q8_kernel" if args.workgroups else "carry_pair_q8_kernel")
                if w.state_fmt == W.STATE_Q8 else "carry_step_kernel")
            + ((" + grad_norm kernels" if args.clip > 0 else " + unscale_check_kernel") if args.amp else ""),
        },
    }
    out["context"] = {"device_copy_gbps": copy_gbps,
                      "device_copy": "torch copy_ of 1 GiB, read + write bytes / time, best of 5"}
    L.apexw_destroy(h)
    del params, grads, state, ws
    torch.cuda.empty_cache()
    if args.torch_compare:
        out["context"].update(torch_compare(torch, w, dev, args.steps, args.warmup))
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
