"""GPU parity of the mixed-precision recipe rows: the unscale-and-check pass
(found_inf produced on the device) and the update on scaled grads, through
the C ABI, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import GpuOpt, bits, n_bit_mismatch, say
from tensor_adamw_optimizer_amd import _lib as L

pytestmark = pytest.mark.gpu
DEV = "cuda"

SIZES = [1, 3, 255, 256, 257, 4095, 4097, 70000, 0]


def _grads_arr(gs):
    return L.make_ptrs([0 if g is None else (g.data_ptr() or 16) for g in gs])


@pytest.mark.parametrize("inv", [1.0 / 65536.0, 1.0, 8.0])
def test_unscale_check_flags_exactly_the_nonfinite(inv):
    say("case: unscale check, inv", inv)
    n = len(SIZES) * 2
    sizes = SIZES * 2
    gdt = [(W.F32, W.BF16)[i % 2] for i in range(n)]
    pdt = [(W.F32, W.BF16)[(i // 2) % 2] for i in range(n)]
    opt = GpuOpt(sizes, pdt, gdt, [0] * n, 1, W.STATE_F32)
    ref = oracle.OracleAdamW(sizes, pdt, gdt, [0] * n, "f32")
    inv_t = torch.tensor([inv], dtype=torch.float32, device=DEV)
    fi = torch.zeros(1, device=DEV)
    gen = torch.Generator().manual_seed(5)
    rng = np.random.default_rng(5)
    for trial in range(24):
        g_cpu = [(torch.randn(s, generator=gen) * 1e-2).to(W.TORCH_DTYPE[d]) for s, d in zip(sizes, gdt)]
        kind = trial % 6
        t = int(rng.integers(0, n))
        while sizes[t] == 0:
            t = int(rng.integers(0, n))
        pos = int(rng.integers(0, sizes[t])) if trial % 2 else sizes[t] - 1
        if kind == 1:
            g_cpu[t][pos] = float("inf")
        elif kind == 2:
            g_cpu[t][pos] = float("nan")
        elif kind == 3:
            g_cpu[t][pos] = -float("inf")
        elif kind == 4:
            g_cpu[t][pos] = 3.0e38 if gdt[t] == W.F32 else 3.0e38   # overflows only when inv > 1
        absent = [(i + trial) % 7 == 0 for i in range(n)]
        g_dev = []
        for i, g in enumerate(g_cpu):
            if absent[i]:
                g_dev.append(None)
            elif i == 5:                              # not 16-byte aligned
                buf = torch.zeros(g.numel() + 1, dtype=g.dtype, device=DEV)
                buf[1:].copy_(g)
                g_dev.append(buf[1:])
            else:
                g_dev.append(g.to(DEV))
        fi.zero_()
        L.apexw_unscale_check(opt.h, _grads_arr(g_dev), inv_t.data_ptr(), fi.data_ptr(), opt.stream)
        torch.cuda.synchronize()
        want = ref.unscale_check([None if a else bits(g) for g, a in zip(g_cpu, absent)], inv)
        assert bool(fi.item() == 1.0) == want, (trial, kind, t, pos)
        assert fi.item() in (0.0, 1.0)
    # the flag is never cleared by a clean check
    fi.fill_(1.0)
    clean = [torch.zeros(s, dtype=W.TORCH_DTYPE[d], device=DEV) for s, d in zip(sizes, gdt)]
    L.apexw_unscale_check(opt.h, _grads_arr(clean), inv_t.data_ptr(), fi.data_ptr(), opt.stream)
    torch.cuda.synchronize()
    assert fi.item() == 1.0
    opt.close()


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
def test_amp_loop_on_device_matches_oracle(fmt):
    """zero found_inf -> unscale_check -> step_scaled, every call on the
    device; grads arrive scaled by 2^16 (one call also by a non-power-of-two
    scale); call 4 overflows and must leave everything untouched."""
    say("case: amp loop", fmt)
    n = len(SIZES)
    sizes = SIZES
    pdt = [(W.BF16, W.F32)[i % 2] for i in range(n)]
    gdt = [(W.F32, W.BF16)[(i // 2) % 2] for i in range(n)]
    groups = [W.Group(lr=1e-3, weight_decay=0.1), W.Group(lr=3e-4)]
    group_of = [i % 2 for i in range(n)]
    gen = torch.Generator().manual_seed(9)
    p_cpu = [(torch.randn(s, generator=gen) * 0.02).to(W.TORCH_DTYPE[d]) for s, d in zip(sizes, pdt)]
    params = [p.to(DEV) for p in p_cpu]
    opt = GpuOpt(sizes, pdt, gdt, group_of, 2, fmt)
    ref = oracle.OracleAdamW(sizes, pdt, gdt, group_of, fmt)
    th_ref = [bits(p) for p in p_cpu]
    fi = torch.zeros(1, device=DEV)
    inv_t = torch.zeros(1, device=DEV)
    pa = L.make_ptrs([p.data_ptr() for p in params])
    ga = L.make_groups(groups)
    for k in range(1, 9):
        scale = 65536.0 if k != 6 else 3000.0
        inv = float(np.float32(1.0 / scale))
        g_cpu = [(torch.randn(s, generator=gen) * 1e-3 * scale).to(W.TORCH_DTYPE[d])
                 for s, d in zip(sizes, gdt)]
        if k == 4:
            g_cpu[7][123] = float("inf")
        g_dev = [g.to(DEV) for g in g_cpu]
        inv_t.fill_(inv)
        fi.zero_()
        L.apexw_unscale_check(opt.h, _grads_arr(g_dev), inv_t.data_ptr(), fi.data_ptr(), opt.stream)
        L.apexw_step_scaled(opt.h, ga, 2, pa, _grads_arr(g_dev), inv_t.data_ptr(), fi.data_ptr(),
                            opt.stream)
        g_np = [bits(g) for g in g_cpu]
        found = ref.unscale_check(g_np, inv)
        assert found == (k == 4)
        ref.step(th_ref, g_np, groups, found_inf=found, inv_scale=inv)
    torch.cuda.synchronize()
    assert np.array_equal(bits(opt.steps()), ref.t)
    assert list(ref.t) == [7] * n
    for i in range(n):
        assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, i
        m, v = opt.moments(i)
        assert n_bit_mismatch(bits(m), ref.m[i]) == 0, i
        assert n_bit_mismatch(bits(v), ref.v[i]) == 0, i
        if fmt == W.STATE_Q8:
            ms, vs = opt.scales(i)
            assert n_bit_mismatch(bits(ms), ref.m_scale[i]) == 0, i
            assert n_bit_mismatch(bits(vs), ref.v_scale[i]) == 0, i
    opt.close()


def test_few_large_amp_full_size_sampled():
    """The 537M-parameter list with grads scaled by 2^16: three calls of the
    device-only recipe; sampled elements against the oracle."""
    w = W.few_large()
    say("case: few_large amp")
    params = W.init_params(w, DEV)
    opt = GpuOpt(w.numels, w.param_dtype, w.grad_dtype, w.group_of, 1, w.state_fmt)
    rng = np.random.default_rng(3)
    idx = [torch.as_tensor(np.unique(np.concatenate([np.arange(256), rng.choice(n, 20000, replace=False),
                                                       np.arange(n - 256, n)]))).to(DEV) for n in w.numels]
    ref = oracle.OracleAdamW([int(i.numel()) for i in idx], w.param_dtype, w.grad_dtype, w.group_of, "f32")
    th_ref = [bits(p.reshape(-1)[i]) for p, i in zip(params, idx)]
    fi = torch.zeros(1, device=DEV)
    inv_t = torch.tensor([1.0 / 65536.0], device=DEV)
    pa = L.make_ptrs([p.data_ptr() for p in params])
    ga = L.make_groups(w.groups)
    for k in range(1, 4):
        g = [x.mul_(65536.0) for x in W.grads_for_call(w, k, DEV)]
        fi.zero_()
        L.apexw_unscale_check(opt.h, _grads_arr(g), inv_t.data_ptr(), fi.data_ptr(), opt.stream)
        L.apexw_step_scaled(opt.h, ga, 1, pa, _grads_arr(g), inv_t.data_ptr(), fi.data_ptr(), opt.stream)
        ref.step(th_ref, [bits(x.reshape(-1)[i]) for x, i in zip(g, idx)], w.groups,
                 inv_scale=1.0 / 65536.0)
        del g
    torch.cuda.synchronize()
    assert fi.item() == 0.0
    for j in range(len(params)):
        m, v = opt.moments(j)
        assert n_bit_mismatch(bits(params[j].reshape(-1)[idx[j]]), th_ref[j]) == 0
        assert n_bit_mismatch(bits(m[idx[j]]), ref.m[j]) == 0
        assert n_bit_mismatch(bits(v[idx[j]]), ref.v[j]) == 0
    opt.close()
