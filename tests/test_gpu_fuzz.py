"""Randomised GPU parity: 48 seeded configurations (and 8 wider ones, see
test_wide_random_configuration_against_oracle), each a random tensor
list (sizes 0 .. 50,000, every (param, grad) dtype pair, 1-4 groups with
random hyperparameters including edge values), a random state format,
launch mode, cache policy and workgroup cap, and 4 calls with random absent
grads, a random skipped call and, on some calls, an inv_scale and a clip
coefficient (from the device norm pass on some calls, through either
entry point); parameters and
grads sometimes views at odd element offsets
into larger buffers (no vector alignment), and the hyperparameters
sometimes read from device memory, and on some calls the unscale-and-check
pass deciding the skip (an inf or a NaN planted now and then) -- theta,
moments, 8-bit scales and
counters bit for bit against the oracle after the last call (two NaNs count
as equal: a degenerate group -- lr = 0 with eps = 0 -- can make 0/0, and the
sign of the NaN that makes is not fixed by IEEE 754)."""
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import (GpuOpt, bits, n_bit_mismatch, n_bit_mismatch_nan_equal, norm_rel_bound,
                         say, stable_max_norm)
from tensor_adamw_optimizer_amd import _lib as L

pytestmark = pytest.mark.gpu
DEV = "cuda"
FORMATS = [W.STATE_F32, W.STATE_BF16, W.STATE_Q8]


def _view(src: torch.Tensor, rng) -> torch.Tensor:
    """A device copy of src, at an odd element offset into a larger buffer
    with probability 0.3 (misaligned for vector accesses), else plain."""
    if src.numel() == 0 or rng.random() >= 0.3:
        return src.to(DEV)
    off = int(rng.integers(1, 4))
    buf = torch.zeros(src.numel() + off, dtype=src.dtype, device=DEV)
    buf[off:].copy_(src)
    return buf[off:]


def _device_groups(groups):
    arr = L.make_groups(groups)
    raw = bytes(ctypes.string_at(ctypes.addressof(arr), ctypes.sizeof(L.apexw_group) * len(groups)))
    return torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(DEV)


def _random_group(rng):
    pick = rng.integers(0, 6)
    lr = float(10 ** rng.uniform(-5, -1))
    beta1 = float(rng.choice([0.0, 0.5, 0.9, 0.99, 0.9999]))
    beta2 = float(rng.choice([0.0, 0.9, 0.999, 0.99999]))
    eps = float(rng.choice([0.0, 1e-12, 1e-8, 1e-3]))
    wd = float(rng.choice([0.0, 0.01, 0.1, 2.0]))
    if pick == 0:
        lr = 0.0
    return W.Group(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=wd)


# seeds per run: 48 and 8 by default; APEXW_FUZZ_SEEDS / APEXW_FUZZ_WIDE_SEEDS
# ask for more (12,600 and 1,500 have been run)
N_SEEDS = int(os.environ.get("APEXW_FUZZ_SEEDS", "48"))
N_WIDE_SEEDS = int(os.environ.get("APEXW_FUZZ_WIDE_SEEDS", "8"))


@pytest.mark.parametrize("seed", range(N_SEEDS))
def test_random_configuration_against_oracle(seed):
    _random_configuration(seed, wide=False)


@pytest.mark.parametrize("seed", range(N_WIDE_SEEDS))
def test_wide_random_configuration_against_oracle(seed):
    """As above with up to 159 tensors (the tile table, not the few-tensor
    lookup) of up to 300,000 elements, six calls, and the step counters of
    some lists started far along (157, 1000, 2^20, 2^31 - 7), written into
    the state buffer and followed by the documented resync call."""
    _random_configuration(seed, wide=True)


def _random_configuration(seed, wide):
    rng = np.random.default_rng((50_000 if wide else 1000) + seed)
    n = int(rng.integers(1, 160 if wide else 25))
    top = 300_000 if wide else 50_000
    sizes = [0 if rng.random() < 0.05 else int(np.exp(rng.uniform(0, np.log(top)))) for _ in range(n)]
    pdt = [str(rng.choice([W.F32, W.BF16])) for _ in range(n)]
    gdt = [str(rng.choice([W.F32, W.BF16])) for _ in range(n)]
    n_groups = int(rng.integers(1, 5))
    group_of = [int(rng.integers(0, n_groups)) for _ in range(n)]
    groups = [_random_group(rng) for _ in range(n_groups)]
    fmt = FORMATS[seed % 3]
    say("case: fuzz", "wide" if wide else "", seed, "n", n, "fmt", fmt, "groups", n_groups)
    gen = torch.Generator().manual_seed(2000 + seed)
    p_cpu = [(torch.randn(s, generator=gen) * 0.02).to(W.TORCH_DTYPE[d]) for s, d in zip(sizes, pdt)]
    params = [_view(p, rng) for p in p_cpu]
    dev_groups = rng.random() < 0.3
    th_ref = [bits(p) for p in p_cpu]
    opt = GpuOpt(sizes, pdt, gdt, group_of, n_groups, fmt)
    try:
        L.apexw_set_launch_mode(opt.h, int(rng.choice([0, 1, 2, 3])))
    except L.ApexwError:
        L.apexw_set_launch_mode(opt.h, 1)             # the single launch or carried step is not available
    L.apexw_set_cache_policy(opt.h, int(rng.choice([0, 1, 2])))
    L.apexw_set_workgroups(opt.h, int(rng.choice([0, 0, 1, 7, 64, 100])))
    ref = oracle.OracleAdamW(sizes, pdt, gdt, group_of, fmt)
    fi = torch.zeros(1, device=DEV)
    inv_t = torch.zeros(1, device=DEV)
    clip_t = torch.zeros(1, device=DEV)
    calls = 6 if wide else 4
    skip_call = int(rng.integers(0, calls + 2))         # past the last call: no skipped call
    t0 = int(rng.choice([0, 0, 157, 1000, 1 << 20, (1 << 31) - 7])) if wide else 0
    if t0:
        opt.steps().copy_(torch.full((n,), t0, dtype=torch.int32))
        ref.t[:n] = t0
        L.apexw_set_launch_mode(opt.h, L.apexw_get_launch_mode(opt.h))   # resync the chain
    chk_rng = np.random.default_rng((770_000 if wide else 760_000) + seed)
    for k in range(calls):
        scaled = rng.random() < 0.5
        inv = float(np.float32(2.0 ** -int(rng.integers(0, 12)) if rng.random() < 0.7
                               else rng.uniform(0.1, 1.0))) if scaled else 1.0
        clip = float(np.float32(rng.uniform(0.2, 1.0))) if scaled and rng.random() < 0.5 else None
        g_cpu = [(torch.randn(s, generator=gen) * 1e-3 / inv).to(W.TORCH_DTYPE[d]) for s, d in zip(sizes, gdt)]
        present = [rng.random() < 0.85 for _ in range(n)]
        skip = k == skip_call
        fi.fill_(1.0 if skip else 0.0)
        pa = L.make_ptrs([p.data_ptr() for p in params])
        g_dev = [_view(g, rng) if ok else None for g, ok in zip(g_cpu, present)]
        ga = L.make_ptrs([0 if g is None else (g.data_ptr() or 16) for g in g_dev])
        if scaled:
            inv_t.fill_(inv)
            if clip is not None:
                clip_t.fill_(clip)
        g_np = [bits(g) if ok else None for g, ok in zip(g_cpu, present)]
        if clip is None and chk_rng.random() < 0.25:
            # the mixed-precision check decides the skip: sometimes an inf or
            # a NaN in one present grad (its own generator, so the other
            # draws are those of the runs without it)
            live = [i for i in range(n) if present[i] and sizes[i] > 0]
            if live and chk_rng.random() < 0.5:
                i = live[int(chk_rng.integers(0, len(live)))]
                e = int(chk_rng.integers(0, sizes[i]))
                bad = float("inf") if chk_rng.random() < 0.5 else float("nan")
                g_dev[i].view(-1)[e] = bad
                g_np[i][e] = (np.float32(bad) if gdt[i] == W.F32
                              else np.uint16(0x7F80 if bad == float("inf") else 0x7FC0))
            fi.zero_()
            L.apexw_unscale_check(opt.h, ga, inv_t.data_ptr() if scaled else 0, fi.data_ptr(),
                                  opt.stream)
            skip = ref.unscale_check(g_np, inv)
            torch.cuda.synchronize()
            assert fi.item() == (1.0 if skip else 0.0), (seed, k)
        if clip is not None and rng.random() < 0.5:
            # the coefficient from the device norm pass instead (and its check)
            want = ref.grad_norm(g_np, inv)
            rel = norm_rel_bound(g_np)
            max_norm = stable_max_norm(ref, want, rel, float(rng.uniform(1e-4, 1e-1)))
            norm_t = torch.zeros(1, dtype=torch.float64, device=DEV)
            chk = torch.zeros(1, device=DEV)
            # (the entry point that allocates nothing on some calls: the same bits)
            norm_fn = (L.apexw_clip_grad_norm_noalloc if chk_rng.random() < 0.5
                       else L.apexw_clip_grad_norm)
            norm_fn(opt.h, ga, inv_t.data_ptr(), max_norm, chk.data_ptr(), norm_t.data_ptr(),
                    clip_t.data_ptr(), opt.stream)
            torch.cuda.synchronize()
            assert abs(norm_t.item() - want) <= rel * want, (seed, k)
            clip = ref.clip_coef(want, max_norm)
            assert clip_t.item() == clip and chk.item() == 0.0, (seed, k)
        table = _device_groups(groups) if dev_groups else None
        L.apexw_step_ex(opt.h, None if dev_groups else L.make_groups(groups), n_groups, pa, ga,
                        inv_scale_ptr=inv_t.data_ptr() if scaled else 0,
                        clip_coef_ptr=clip_t.data_ptr() if clip is not None else 0,
                        found_inf_ptr=fi.data_ptr(),
                        groups_dev_ptr=table.data_ptr() if dev_groups else 0, stream=opt.stream)
        ref.step(th_ref, g_np, groups,
                 found_inf=skip, inv_scale=inv if scaled else None, clip_coef=clip)
        torch.cuda.synchronize()
    assert np.array_equal(bits(opt.steps()), ref.t[:n])
    for i in range(n):
        assert n_bit_mismatch_nan_equal(bits(params[i]), th_ref[i]) == 0, (seed, i)
        m, v = opt.moments(i)
        assert n_bit_mismatch_nan_equal(bits(m), ref.m[i]) == 0, (seed, i)
        assert n_bit_mismatch_nan_equal(bits(v), ref.v[i]) == 0, (seed, i)
        if fmt == W.STATE_Q8:
            ms, vs = opt.scales(i)
            assert n_bit_mismatch(bits(ms), ref.m_scale[i]) == 0, (seed, i)
            assert n_bit_mismatch(bits(vs), ref.v_scale[i]) == 0, (seed, i)
    opt.close()


N_SESSION_SEEDS = int(os.environ.get("APEXW_FUZZ_SESSION_SEEDS", "8"))


@pytest.mark.parametrize("seed", range(N_SESSION_SEEDS))
def test_random_session_against_oracle(seed):
    """One tensor list stepped ten times while the knobs change between
    calls: the launch mode (whichever the list admits), the workgroup cap,
    the residency cap, the cache policy, a checkpoint exported and imported
    into the same handle or into a fresh one that takes over, a step with
    the hyperparameters in device memory, and betas changed for a call --
    every change the carried chain has to survive or restart after.  Theta,
    moments, scales and counters bit for bit against the oracle after every
    call (NaNs compared as NaNs)."""
    rng = np.random.default_rng(90_000 + seed)
    n = int(rng.integers(1, 40))
    sizes = [0 if rng.random() < 0.05 else int(np.exp(rng.uniform(0, np.log(60_000)))) for _ in range(n)]
    pdt = [str(rng.choice([W.F32, W.BF16])) for _ in range(n)]
    gdt = [str(rng.choice([W.F32, W.BF16])) for _ in range(n)]
    n_groups = int(rng.integers(1, 4))
    group_of = [int(rng.integers(0, n_groups)) for _ in range(n)]
    groups = [_random_group(rng) for _ in range(n_groups)]
    fmt = FORMATS[seed % 3]
    say("case: fuzz session", seed, "n", n, "fmt", fmt, "groups", n_groups)
    gen = torch.Generator().manual_seed(91_000 + seed)
    p_cpu = [(torch.randn(s, generator=gen) * 0.02).to(W.TORCH_DTYPE[d]) for s, d in zip(sizes, pdt)]
    params = [p.to(DEV) for p in p_cpu]
    th_ref = [bits(p) for p in p_cpu]
    opt = GpuOpt(sizes, pdt, gdt, group_of, n_groups, fmt)
    ref = oracle.OracleAdamW(sizes, pdt, gdt, group_of, fmt)
    fi = torch.zeros(1, device=DEV)
    pa = L.make_ptrs([p.data_ptr() for p in params])
    for k in range(10):
        action = str(rng.choice(["mode", "cap", "occupancy", "policy", "export_same",
                                 "export_fresh", "device", "betas", "none"]))
        step_groups = groups
        if action == "mode":
            try:
                L.apexw_set_launch_mode(opt.h, int(rng.choice([0, 1, 2, 3])))
            except L.ApexwError:
                pass                                  # a mode the list does not admit
        elif action == "cap":
            L.apexw_set_workgroups(opt.h, int(rng.choice([0, 1, 5, 64, 1000])))
        elif action == "occupancy":
            L.apexw_set_occupancy(opt.h, int(rng.choice([0, 1, 4, 14, 40])))
        elif action == "policy":
            L.apexw_set_cache_policy(opt.h, int(rng.choice([0, 1, 2])))
        elif action in ("export_same", "export_fresh"):
            blob = L.apexw_export_state(opt.h, L.make_groups(groups), n_groups, opt.stream)
            if action == "export_fresh":              # a new handle takes over from the blob
                new = GpuOpt(sizes, pdt, gdt, group_of, n_groups, fmt)
                opt.close()
                opt = new
            L.apexw_import_state(opt.h, blob, n_groups, opt.stream)
        elif action == "betas":                       # this call only
            step_groups = [W.Group(lr=g.lr, beta1=float(rng.choice([0.0, 0.8, 0.9])),
                                   beta2=float(rng.choice([0.9, 0.999])), eps=g.eps,
                                   weight_decay=g.weight_decay) for g in groups]
        g_cpu = [(torch.randn(s, generator=gen) * 1e-3).to(W.TORCH_DTYPE[d]) for s, d in zip(sizes, gdt)]
        present = [rng.random() < 0.85 for _ in range(n)]
        skip = rng.random() < 0.1
        fi.fill_(1.0 if skip else 0.0)
        g_dev = [g.to(DEV) if ok else None for g, ok in zip(g_cpu, present)]
        ga = L.make_ptrs([0 if g is None else (g.data_ptr() or 16) for g in g_dev])
        g_np = [bits(g) if ok else None for g, ok in zip(g_cpu, present)]
        if action == "device":
            table = _device_groups(step_groups)
            L.apexw_step_ex(opt.h, None, n_groups, pa, ga, found_inf_ptr=fi.data_ptr(),
                            groups_dev_ptr=table.data_ptr(), stream=opt.stream)
        else:
            L.apexw_step(opt.h, L.make_groups(step_groups), n_groups, pa, ga, fi.data_ptr(),
                         opt.stream)
        ref.step(th_ref, g_np, step_groups, found_inf=skip)
        torch.cuda.synchronize()
        assert np.array_equal(bits(opt.steps()), ref.t[:n]), (seed, k, action)
        for i in range(n):
            assert n_bit_mismatch_nan_equal(bits(params[i]), th_ref[i]) == 0, (seed, k, action, i)
            m, v = opt.moments(i)
            assert n_bit_mismatch_nan_equal(bits(m), ref.m[i]) == 0, (seed, k, action, i)
            assert n_bit_mismatch_nan_equal(bits(v), ref.v[i]) == 0, (seed, k, action, i)
            if fmt == W.STATE_Q8:
                ms, vs = opt.scales(i)
                assert n_bit_mismatch(bits(ms), ref.m_scale[i]) == 0, (seed, k, action, i)
                assert n_bit_mismatch(bits(vs), ref.v_scale[i]) == 0, (seed, k, action, i)
    opt.close()


N_GRAPH_SEEDS = int(os.environ.get("APEXW_FUZZ_GRAPH_SEEDS", "6"))


@pytest.mark.parametrize("seed", range(N_GRAPH_SEEDS))
def test_random_graph_session_against_oracle(seed):
    """Twelve calls on persistent buffers in which one step is captured into
    a graph at a random point (with the hyperparameters of that moment, or
    read from a device table that later calls rewrite), and the calls after
    it are eager steps or replays in random order, with learning-rate
    changes, skipped calls, and at most one resync (apexw_set_launch_mode,
    after which no replay follows).  Every call against the oracle."""
    rng = np.random.default_rng(95_000 + seed)
    n = int(rng.integers(1, 12))
    sizes = [int(np.exp(rng.uniform(0, np.log(20_000)))) for _ in range(n)]
    pdt = [str(rng.choice([W.F32, W.BF16])) for _ in range(n)]
    gdt = [str(rng.choice([W.F32, W.BF16])) for _ in range(n)]
    n_groups = int(rng.integers(1, 3))
    group_of = [int(rng.integers(0, n_groups)) for _ in range(n)]
    groups = [_random_group(rng) for _ in range(n_groups)]
    fmt = FORMATS[seed % 3]
    on_device = bool(rng.random() < 0.5)
    capture_at = int(rng.integers(1, 6))
    say("case: fuzz graph session", seed, "n", n, "fmt", fmt, "device groups", on_device,
        "capture after call", capture_at)
    gen = torch.Generator().manual_seed(96_000 + seed)
    p_cpu = [(torch.randn(s, generator=gen) * 0.02).to(W.TORCH_DTYPE[d]) for s, d in zip(sizes, pdt)]
    params = [p.to(DEV) for p in p_cpu]
    grads = [torch.zeros(s, dtype=W.TORCH_DTYPE[d], device=DEV) for s, d in zip(sizes, gdt)]
    th_ref = [bits(p) for p in p_cpu]
    opt = GpuOpt(sizes, pdt, gdt, group_of, n_groups, fmt)
    ref = oracle.OracleAdamW(sizes, pdt, gdt, group_of, fmt)
    fi = torch.zeros(1, device=DEV)
    pa = L.make_ptrs([p.data_ptr() for p in params])
    ga = L.make_ptrs([g.data_ptr() for g in grads])
    table = _device_groups(groups)
    graph, captured_groups, replays_allowed = None, None, True
    for k in range(12):
        if rng.random() < 0.3:                        # a schedule's change
            groups = [W.Group(lr=g.lr * 0.5, beta1=g.beta1, beta2=g.beta2, eps=g.eps,
                              weight_decay=g.weight_decay) for g in groups]
            table.copy_(_device_groups(groups))
        g_cpu = [(torch.randn(s, generator=gen) * 1e-3).to(W.TORCH_DTYPE[d]) for s, d in zip(sizes, gdt)]
        for g, x in zip(grads, g_cpu):
            g.copy_(x.to(DEV))
        skip = bool(rng.random() < 0.1)
        fi.fill_(1.0 if skip else 0.0)
        torch.cuda.synchronize()
        replay = graph is not None and replays_allowed and rng.random() < 0.5
        if replay:
            graph.replay()
            used = groups if on_device else captured_groups
        else:
            L.apexw_step(opt.h, L.make_groups(groups), n_groups, pa, ga, fi.data_ptr(), opt.stream)
            used = groups
        ref.step(th_ref, [bits(x) for x in g_cpu], used, found_inf=skip)
        torch.cuda.synchronize()
        assert np.array_equal(bits(opt.steps()), ref.t[:n]), (seed, k, replay)
        for i in range(n):
            assert n_bit_mismatch_nan_equal(bits(params[i]), th_ref[i]) == 0, (seed, k, replay, i)
            m, v = opt.moments(i)
            assert n_bit_mismatch_nan_equal(bits(m), ref.m[i]) == 0, (seed, k, replay, i)
            assert n_bit_mismatch_nan_equal(bits(v), ref.v[i]) == 0, (seed, k, replay, i)
        if k + 1 == capture_at:                       # capture one step (not run by capturing)
            graph = torch.cuda.CUDAGraph()
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                with torch.cuda.graph(graph, stream=s):
                    st = torch.cuda.current_stream().cuda_stream
                    if on_device:
                        L.apexw_step_device(opt.h, table.data_ptr(), n_groups, pa, ga, 0,
                                            fi.data_ptr(), st)
                    else:
                        L.apexw_step(opt.h, L.make_groups(groups), n_groups, pa, ga,
                                     fi.data_ptr(), st)
            torch.cuda.synchronize()
            captured_groups = groups
        elif graph is not None and replays_allowed and rng.random() < 0.15:
            L.apexw_set_launch_mode(opt.h, 0)         # no replay follows from here on
            replays_allowed = False
    opt.close()
