"""GPU tests of the checkpoint blob and of graph capture, through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import GpuOpt, bits, n_bit_mismatch, say
from tensor_adamw_optimizer_amd import _lib as L

pytestmark = pytest.mark.gpu
DEV = "cuda"

SIZES = [3, 300, 4097, 12000, 256]
PDT = [W.F32, W.BF16, W.F32, W.BF16, W.F32]
GDT = [W.F32, W.F32, W.BF16, W.BF16, W.F32]
GROUP_OF = [0, 1, 0, 1, 0]
GROUPS = [W.Group(lr=1e-3, weight_decay=0.1), W.Group(lr=4e-4, beta1=0.8, eps=1e-6)]


def _inputs(seed, calls):
    gen = torch.Generator().manual_seed(seed)
    p = [(torch.randn(s, generator=gen) * 0.02).to(W.TORCH_DTYPE[d]) for s, d in zip(SIZES, PDT)]
    gs = [[(torch.randn(s, generator=gen) * 1e-3).to(W.TORCH_DTYPE[d]) for s, d in zip(SIZES, GDT)]
          for _ in range(calls)]
    return p, gs


def _run(opt, params, gs_cpu, groups=GROUPS):
    ga = L.make_groups(groups)
    pa = L.make_ptrs([p.data_ptr() for p in params])
    for gs in gs_cpu:
        g_dev = [g.to(DEV) for g in gs]
        L.apexw_step(opt.h, ga, len(groups), pa, L.make_ptrs([g.data_ptr() for g in g_dev]), 0,
                     opt.stream)
        torch.cuda.synchronize()


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
def test_resume_from_blob_is_bitwise_the_uninterrupted_run(fmt):
    say("case: checkpoint resume", fmt)
    p_cpu, gs = _inputs(31, 10)
    # uninterrupted
    pa = [p.to(DEV) for p in p_cpu]
    a = GpuOpt(SIZES, PDT, GDT, GROUP_OF, 2, fmt)
    _run(a, pa, gs)
    # 5 calls, export, a fresh handle and fresh parameter copies, import, 5 more
    pb = [p.to(DEV) for p in p_cpu]
    b = GpuOpt(SIZES, PDT, GDT, GROUP_OF, 2, fmt)
    _run(b, pb, gs[:5])
    blob = L.apexw_export_state(b.h, L.make_groups(GROUPS), 2, b.stream)
    assert len(blob) == L.apexw_export_bytes(b.h)
    saved_params = [p.clone() for p in pb]
    b.close()
    c = GpuOpt(SIZES, PDT, GDT, GROUP_OF, 2, fmt)
    recipe = L.apexw_import_state(c.h, blob, 2, c.stream)
    assert [(r.lr, r.beta1, r.beta2, r.eps, r.weight_decay) for r in recipe] == \
        [(g.lr, g.beta1, g.beta2, g.eps, g.weight_decay) for g in GROUPS]
    pc = [p.clone() for p in saved_params]
    _run(c, pc, gs[5:])
    assert torch.equal(a.state[:a.state_bytes], c.state[:c.state_bytes])
    for x, y in zip(pa, pc):
        assert torch.equal(x.view(torch.uint8) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.uint8) if y.dtype == torch.bfloat16 else y)
    assert list(bits(c.steps())) == [10] * len(SIZES)
    a.close()
    c.close()


def test_import_rejects_foreign_or_damaged_blobs():
    say("case: checkpoint rejection")
    p_cpu, gs = _inputs(32, 2)
    params = [p.to(DEV) for p in p_cpu]
    a = GpuOpt(SIZES, PDT, GDT, GROUP_OF, 2, W.STATE_F32)
    _run(a, params, gs)
    blob = L.apexw_export_state(a.h, L.make_groups(GROUPS), 2, a.stream)
    other = GpuOpt(SIZES[:-1] + [255], PDT, GDT, GROUP_OF, 2, W.STATE_F32)
    q8 = GpuOpt(SIZES, PDT, GDT, GROUP_OF, 2, W.STATE_Q8)
    before = (other.state.clone(), q8.state.clone(), a.state.clone())
    bad_magic = b"X" + blob[1:]
    for h, data in ((other.h, blob), (q8.h, blob), (a.h, blob[:-4]), (a.h, bad_magic),
                    (a.h, blob[:10])):
        with pytest.raises(L.ApexwError) as e:
            L.apexw_import_state(h, data, 2, a.stream)
        assert e.value.code == L.APEXW_EINVAL
    torch.cuda.synchronize()
    assert torch.equal(before[0], other.state) and torch.equal(before[1], q8.state)
    assert torch.equal(before[2], a.state)
    for o in (a, other, q8):
        o.close()


def _group_table(groups):
    arr = L.make_groups(groups)
    raw = bytes(ctypes.string_at(ctypes.addressof(arr), ctypes.sizeof(L.apexw_group) * len(groups)))
    return torch.frombuffer(bytearray(raw), dtype=torch.uint8).to(DEV)


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_Q8])
def test_device_groups_equal_host_groups(fmt):
    say("case: device hyperparameters", fmt)
    p_cpu, gs = _inputs(33, 4)
    pa = [p.to(DEV) for p in p_cpu]
    pb = [p.to(DEV) for p in p_cpu]
    a = GpuOpt(SIZES, PDT, GDT, GROUP_OF, 2, fmt)
    b = GpuOpt(SIZES, PDT, GDT, GROUP_OF, 2, fmt)
    table = _group_table(GROUPS)
    _run(a, pa, gs)
    pab = L.make_ptrs([p.data_ptr() for p in pb])
    for g in gs:
        g_dev = [x.to(DEV) for x in g]
        L.apexw_step_device(b.h, table.data_ptr(), 2, pab, L.make_ptrs([x.data_ptr() for x in g_dev]),
                            0, 0, b.stream)
        torch.cuda.synchronize()
    assert torch.equal(a.state[:a.state_bytes], b.state[:b.state_bytes])
    for x, y in zip(pa, pb):
        assert n_bit_mismatch(bits(x), bits(y)) == 0
    a.close()
    b.close()


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
def test_graph_capture_replays_match_oracle(fmt, mode):
    """Capture [zero found_inf, unscale check, step with device hyperparameters]
    once; replay it 6 times with new grads, a new learning rate and (once) an
    overflow written in place between replays, with eager work and
    synchronisations in between; every replay is checked against the oracle.
    Both launch modes (the single launch's arrival counters must come back
    to zero in every replay)."""
    say("case: graph capture", fmt, "mode", mode)
    p_cpu, gs = _inputs(34, 7)
    params = [p.to(DEV) for p in p_cpu]
    grads = [g.to(DEV) for g in gs[0]]
    opt = GpuOpt(SIZES, PDT, GDT, GROUP_OF, 2, fmt)
    L.apexw_set_launch_mode(opt.h, mode)
    # the default is the carried step, which a captured step does not take
    # (it falls back to the single launch for a list this small)
    assert L.apexw_get_launch_mode(opt.h) == (3 if mode == 0 else 1)
    ref = oracle.OracleAdamW(SIZES, PDT, GDT, GROUP_OF, fmt)
    th_ref = [bits(p) for p in p_cpu]
    fi = torch.zeros(1, device=DEV)
    inv = torch.ones(1, device=DEV)
    table = _group_table(GROUPS)
    pa = L.make_ptrs([p.data_ptr() for p in params])
    ga = L.make_ptrs([g.data_ptr() for g in grads])

    def recipe(stream):
        fi.zero_()
        L.apexw_unscale_check(opt.h, ga, inv.data_ptr(), fi.data_ptr(), stream)
        L.apexw_step_device(opt.h, table.data_ptr(), 2, pa, ga, inv.data_ptr(), fi.data_ptr(), stream)

    # one eager call with these pointers (uploads the tables), checked too
    recipe(torch.cuda.current_stream().cuda_stream)
    ref.step(th_ref, [bits(g) for g in gs[0]], GROUPS)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            recipe(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    # capture must not have run anything
    assert list(bits(opt.steps())) == [1] * len(SIZES)
    lrs = [2e-3, 1e-3, 5e-4, 5e-4, 2.5e-4, 1e-4]
    for r, k in enumerate(range(1, 7)):
        groups = [W.Group(lr=lrs[r], weight_decay=0.1), W.Group(lr=lrs[r] * 0.4, beta1=0.8, eps=1e-6)]
        table.copy_(_group_table(groups))
        new = [g.clone() for g in gs[k]]
        if k == 3:
            new[2][17] = float("nan")
        for g, x in zip(grads, new):
            g.copy_(x.to(DEV))
        junk = torch.randn(1 << 16, device=DEV).sum()          # eager work in between
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        found = ref.unscale_check([bits(x) for x in new], 1.0)
        assert found == (k == 3) and fi.item() == (1.0 if found else 0.0)
        ref.step(th_ref, [bits(x) for x in new], groups, found_inf=found)
        assert np.array_equal(bits(opt.steps()), ref.t), r
        for i in range(len(SIZES)):
            assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, (r, i)
            m, v = opt.moments(i)
            assert n_bit_mismatch(bits(m), ref.m[i]) == 0 and n_bit_mismatch(bits(v), ref.v[i]) == 0
        del junk
    assert list(ref.t) == [6] * len(SIZES)
    # (the replays above moved every counter, so `graph` is not empty)
    # a pointer change under capture is refused: nothing is captured, and
    # torch says so when the capture ends
    other = [g.clone() for g in grads]
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with pytest.warns(UserWarning, match="empty"):
            with pytest.raises(L.ApexwError):
                with torch.cuda.graph(g2, stream=s):
                    L.apexw_step_device(opt.h, table.data_ptr(), 2, pa,
                                        L.make_ptrs([g.data_ptr() for g in other]), 0, 0,
                                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    opt.close()


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_Q8])
def test_capture_between_carried_steps(fmt):
    """Eager steps in the default (carried) mode, then a plain apexw_step
    (hyperparameters from the host) captured into a graph -- the capture takes
    the single launch, not the carried step -- replayed 3 times, which
    advances the counters with no host call, then eager carried steps again:
    they must restart their chain from the counters as the replays left
    them.  Every call is checked against the oracle."""
    say("case: capture between carried steps", fmt)
    p_cpu, gs = _inputs(41, 10)
    params = [p.to(DEV) for p in p_cpu]
    grads = [g.to(DEV) for g in gs[0]]
    opt = GpuOpt(SIZES, PDT, GDT, GROUP_OF, 2, fmt)
    assert L.apexw_get_launch_mode(opt.h) == 3
    ref = oracle.OracleAdamW(SIZES, PDT, GDT, GROUP_OF, fmt)
    th_ref = [bits(p) for p in p_cpu]
    pa = L.make_ptrs([p.data_ptr() for p in params])
    ga = L.make_ptrs([g.data_ptr() for g in grads])
    groups = L.make_groups(GROUPS)

    def check(k):
        assert np.array_equal(bits(opt.steps()), ref.t), k
        for i in range(len(SIZES)):
            assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, (k, i)
            m, v = opt.moments(i)
            assert n_bit_mismatch(bits(m), ref.m[i]) == 0 and n_bit_mismatch(bits(v), ref.v[i]) == 0, (k, i)

    def eager(k):
        for g, x in zip(grads, gs[k]):
            g.copy_(x.to(DEV))
        L.apexw_step(opt.h, groups, 2, pa, ga, 0, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        ref.step(th_ref, [bits(x) for x in gs[k]], GROUPS)
        check(k)

    for k in range(3):
        eager(k)
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            L.apexw_step(opt.h, groups, 2, pa, ga, 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    check("after capture")                            # capture ran nothing
    for k in range(3, 6):
        for g, x in zip(grads, gs[k]):
            g.copy_(x.to(DEV))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref.step(th_ref, [bits(x) for x in gs[k]], GROUPS)
        check(k)
    for k in range(6, 10):
        eager(k)
    assert list(ref.t) == [10] * len(SIZES)
    opt.close()


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_Q8])
def test_replays_between_eager_steps(fmt):
    """A step captured into a graph, then eager steps and replays taking
    turns: capture, eager, replay, eager, replay, eager.  Each replay moves
    the counters with no host call, so after the capture the eager steps must
    not take the carried step (its corrections would be those of the counter
    before the replay); apexw_set_launch_mode re-admits it once no replay is
    coming.  Every call is checked against the oracle."""
    say("case: replays between eager steps", fmt)
    p_cpu, gs = _inputs(47, 12)
    params = [p.to(DEV) for p in p_cpu]
    grads = [g.to(DEV) for g in gs[0]]
    opt = GpuOpt(SIZES, PDT, GDT, GROUP_OF, 2, fmt)
    ref = oracle.OracleAdamW(SIZES, PDT, GDT, GROUP_OF, fmt)
    th_ref = [bits(p) for p in p_cpu]
    pa = L.make_ptrs([p.data_ptr() for p in params])
    ga = L.make_ptrs([g.data_ptr() for g in grads])
    groups = L.make_groups(GROUPS)
    st = torch.cuda.current_stream().cuda_stream

    def check(k):
        assert np.array_equal(bits(opt.steps()), ref.t), k
        for i in range(len(SIZES)):
            assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, (k, i)
            m, v = opt.moments(i)
            assert n_bit_mismatch(bits(m), ref.m[i]) == 0 and n_bit_mismatch(bits(v), ref.v[i]) == 0, (k, i)

    def load(k):
        for g, x in zip(grads, gs[k]):
            g.copy_(x.to(DEV))
        torch.cuda.synchronize()
        ref.step(th_ref, [bits(x) for x in gs[k]], GROUPS)

    def eager(k):
        load(k)
        L.apexw_step(opt.h, groups, 2, pa, ga, 0, st)
        torch.cuda.synchronize()
        check(k)

    eager(0)
    eager(1)
    assert L.apexw_get_launch_mode(opt.h) == 3
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            L.apexw_step(opt.h, groups, 2, pa, ga, 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    check("after capture")
    assert L.apexw_get_launch_mode(opt.h) != 3
    for k in range(2, 8):
        if k % 2 == 0:
            eager(k)
        else:
            load(k)
            graph.replay()
            torch.cuda.synchronize()
            check(k)
    L.apexw_set_launch_mode(opt.h, 0)                # no replay follows
    assert L.apexw_get_launch_mode(opt.h) == 3
    for k in range(8, 12):
        eager(k)
    assert list(ref.t) == [12] * len(SIZES)
    opt.close()


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
def test_carried_step_with_device_hyperparameters_in_between(fmt):
    """The carried step forced (mode 3), with steps whose hyperparameters live
    in device memory mixed in (they take another mode and drop the carried
    corrections; the next host step starts them again), betas changing on
    the device-side calls: 10 calls, each checked against the oracle."""
    say("case: carried step and device hyperparameters", fmt)
    p_cpu, gs = _inputs(43, 10)
    params = [p.to(DEV) for p in p_cpu]
    opt = GpuOpt(SIZES, PDT, GDT, GROUP_OF, 2, fmt)
    L.apexw_set_launch_mode(opt.h, 3)
    ref = oracle.OracleAdamW(SIZES, PDT, GDT, GROUP_OF, fmt)
    th_ref = [bits(p) for p in p_cpu]
    pa = L.make_ptrs([p.data_ptr() for p in params])
    st = torch.cuda.current_stream().cuda_stream
    for k in range(10):
        device_call = k in (2, 3, 6)
        groups = GROUPS if not device_call else \
            [W.Group(lr=2e-3, weight_decay=0.1, beta2=0.99), W.Group(lr=4e-4, beta1=0.85, eps=1e-6)]
        g_dev = [g.to(DEV) for g in gs[k]]
        ga = L.make_ptrs([g.data_ptr() for g in g_dev])
        if device_call:
            table = _group_table(groups)
            L.apexw_step_device(opt.h, table.data_ptr(), 2, pa, ga, 0, 0, st)
        else:
            L.apexw_step(opt.h, L.make_groups(groups), 2, pa, ga, 0, st)
        torch.cuda.synchronize()
        ref.step(th_ref, [bits(g) for g in gs[k]], groups)
        assert np.array_equal(bits(opt.steps()), ref.t), k
        for i in range(len(SIZES)):
            assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, (k, i)
            m, v = opt.moments(i)
            assert n_bit_mismatch(bits(m), ref.m[i]) == 0 and n_bit_mismatch(bits(v), ref.v[i]) == 0, (k, i)
    assert L.apexw_get_launch_mode(opt.h) == 3
    opt.close()
