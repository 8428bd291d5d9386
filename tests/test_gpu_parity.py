"""GPU parity: the HIP library, called through its C ABI, against the oracle
on the same seeded inputs.

Bars: fp32 state -- elementwise relative error <= 1e-5 on theta, m, v after
every call (the design target, and what is observed, is a bitwise match);
bf16 state -- bitwise against the oracle's bf16-state mode and <= 1e-2
(normwise) against the fp32-state oracle on the moments; 8-bit state --
codes equal or within 1, scales within 1e-6 relative; step counters and the
skip / grad=None behaviour bit-exact.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tensor_adamw_optimizer_amd import _lib as L
from gpu_helpers import (GpuOpt, as_f32, assert_fp32_state_parity, bits, n_bit_mismatch,
                         normwise_err, rel_err_elementwise, say)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")


def _oracle_for(w: W.Workload, idx=None, state_fmt=None):
    idx = range(len(w.shapes)) if idx is None else idx
    return oracle.OracleAdamW([w.numels[i] for i in idx], [w.param_dtype[i] for i in idx],
                              [w.grad_dtype[i] for i in idx], [w.group_of[i] for i in idx],
                              state_fmt or w.state_fmt)


# =================================================================== tiny

@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_tiny_every_call_against_oracle(mode):
    """525,315 fp32 params, 20 calls, call 7 skipped, [3] has no grad on odd
    calls: theta, m, v and t compared after every call; every launch mode
    (the default is the carried step)."""
    _need_gpu()
    w = W.tiny()
    say("case: tiny", w.describe(), "mode", mode)
    p_cpu = W.init_params(w, "cpu")
    params = [p.to(DEV) for p in p_cpu]
    grads = [torch.empty(s, dtype=torch.float32, device=DEV) for s in w.shapes]
    opt = GpuOpt(w.numels, w.param_dtype, w.grad_dtype, w.group_of, len(w.groups), w.state_fmt)
    L.apexw_set_launch_mode(opt.h, mode)
    assert L.apexw_get_launch_mode(opt.h) == (3 if mode == 0 else mode)
    ref = _oracle_for(w)
    th_ref = [bits(p) for p in p_cpu]
    fi = torch.zeros(1, dtype=torch.float32, device=DEV)
    total_mismatch = 0
    for k in range(1, w.steps + 1):
        g_cpu = W.grads_for_call(w, k, "cpu")
        for gb, g in zip(grads, g_cpu):
            if g is not None:
                gb.copy_(g)
        skip = w.skip_call(k)
        fi.fill_(1.0 if skip else 0.0)
        opt.step(w.groups, params, [gb if g is not None else None for gb, g in zip(grads, g_cpu)],
                 found_inf=fi)
        ref.step(th_ref, [None if g is None else bits(g) for g in g_cpu], w.groups, found_inf=skip)
        torch.cuda.synchronize()
        for i in range(len(w.shapes)):
            m, v = opt.moments(i)
            total_mismatch += assert_fp32_state_parity("theta%d@%d" % (i, k), bits(params[i]), th_ref[i])
            total_mismatch += assert_fp32_state_parity("m%d@%d" % (i, k), bits(m), ref.m[i])
            total_mismatch += assert_fp32_state_parity("v%d@%d" % (i, k), bits(v), ref.v[i])
        assert np.array_equal(bits(opt.steps()), ref.t), (bits(opt.steps()), ref.t)
    # 20 calls minus the skipped call 7; the [3] tensor has grads on the 10 even calls
    assert list(ref.t) == [19, 19, 19, 10]
    assert total_mismatch == 0
    opt.close()


# =================================================================== edge cases

EDGE_SIZES = [1, 3, 5, 255, 256, 257, 1023, 4095, 4096, 4097, 8191, 12289, 0, 100003]


# (cache policy, launch mode): the small list's default (cached, single
# launch: the list has empty tensors, so not the carried step), streaming
# (prepare + update), cached prepare + update, the single launch forced
# under a streaming policy, and the carried step cached and streaming (on the
# list without its empty tensors)
MODES = [(0, 0), (1, 0), (0, 1), (1, 2), (0, 3), (1, 3)]


@pytest.mark.parametrize("policy,mode", MODES)
@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
def test_ragged_mixed_dtypes_groups_and_misalignment(fmt, policy, mode):
    """Every (param, grad) dtype pair in one optimizer (one launch each), ragged
    sizes, empty tensors, three groups, a parameter and a grad that are not
    16-byte aligned, grads absent on some calls, one skipped call; cached
    and streaming accesses, both launch modes."""
    _need_gpu()
    say("case: ragged", fmt, "policy", policy, "mode", mode)
    sizes = EDGE_SIZES * 2
    if mode == 3:                            # the carried step needs no empty tensor
        sizes = [s if s else 2 for s in sizes]
    n = len(sizes)
    pdt = [(W.F32, W.BF16)[(i // 2) % 2] for i in range(n)]
    gdt = [(W.F32, W.BF16)[i % 2] for i in range(n)]
    group_of = [i % 3 for i in range(n)]
    groups = [W.Group(lr=1e-2, weight_decay=0.1), W.Group(lr=3e-3, beta1=0.8, beta2=0.99, eps=1e-6),
              W.Group(lr=5e-4, weight_decay=0.01)]
    gen = torch.Generator().manual_seed(7)
    p_cpu = [(torch.randn(s, generator=gen) * 0.02).to(W.TORCH_DTYPE[d]) for s, d in zip(sizes, pdt)]
    # tensor 3 and 10 live one element into a larger buffer: not 16-byte aligned
    bases = {}
    params = []
    for i, p in enumerate(p_cpu):
        if i in (3, 10):
            buf = torch.zeros(p.numel() + 1, dtype=p.dtype, device=DEV)
            buf[1:].copy_(p)
            bases[i] = buf
            params.append(buf[1:])
        else:
            params.append(p.to(DEV))
    opt = GpuOpt(sizes, pdt, gdt, group_of, 3, fmt)
    L.apexw_set_cache_policy(opt.h, policy)
    L.apexw_set_launch_mode(opt.h, mode)
    ref = oracle.OracleAdamW(sizes, pdt, gdt, group_of, fmt)
    th_ref = [bits(p) for p in p_cpu]
    fi = torch.zeros(1, device=DEV)
    for k in range(1, 9):
        g_cpu = [(torch.randn(s, generator=gen) * 1e-3).to(W.TORCH_DTYPE[d]) for s, d in zip(sizes, gdt)]
        present = [not ((i + k) % 5 == 0) for i in range(n)]
        gdev = []
        for i, (g, ok) in enumerate(zip(g_cpu, present)):
            if not ok:
                gdev.append(None)
            elif i == 5:
                gb = torch.zeros(g.numel() + 3, dtype=g.dtype, device=DEV)
                gb[3:].copy_(g)
                gdev.append(gb[3:])
            else:
                gdev.append(g.to(DEV))
        skip = k == 4
        fi.fill_(1.0 if skip else 0.0)
        opt.step(groups, params, gdev, found_inf=fi)
        ref.step(th_ref, [bits(g) if ok else None for g, ok in zip(g_cpu, present)], groups,
                 found_inf=skip)
    torch.cuda.synchronize()
    assert np.array_equal(bits(opt.steps()), ref.t)
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


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
def test_found_inf_leaves_everything_bitwise(fmt, mode):
    _need_gpu()
    say("case: found_inf", fmt, "mode", mode)
    sizes = [5000, 4096, 77]
    opt = GpuOpt(sizes, [W.BF16, W.F32, W.F32], [W.F32, W.BF16, W.F32], [0, 0, 0], 1, fmt)
    L.apexw_set_launch_mode(opt.h, mode)
    params = [torch.randn(sizes[0], device=DEV).to(torch.bfloat16), torch.randn(sizes[1], device=DEV),
              torch.randn(sizes[2], device=DEV)]
    grads = [torch.randn(sizes[0], device=DEV) * 1e-3,
             (torch.randn(sizes[1], device=DEV) * 1e-3).to(torch.bfloat16),
             torch.randn(sizes[2], device=DEV) * 1e-3]
    g = [W.Group(lr=1e-3, weight_decay=0.1)]
    for _ in range(3):
        opt.step(g, params, grads)
    torch.cuda.synchronize()
    before = [bits(p) for p in params] + [bits(opt.state)]
    fi = torch.ones(1, device=DEV)
    for val in (1.0, float("inf"), float("nan"), -2.0):
        fi.fill_(val)
        opt.step(g, params, grads, found_inf=fi)
    torch.cuda.synchronize()
    after = [bits(p) for p in params] + [bits(opt.state)]
    for a, b in zip(before, after):
        assert np.array_equal(a, b)
    assert list(bits(opt.steps())) == [3, 3, 3]
    fi.fill_(0.0)
    opt.step(g, params, grads, found_inf=fi)
    torch.cuda.synchronize()
    assert list(bits(opt.steps())) == [4, 4, 4]
    opt.close()


def _bf16_rounding_patterns() -> np.ndarray:
    """fp32 bit patterns covering every case of nearest-even rounding to
    bf16: all 65536 low halves under each sign and exponent with an even and
    an odd last kept bit (zeros, denormals, infinities and NaNs included),
    and every high half under 16 low halves around the ties."""
    sign_exp = np.arange(512, dtype=np.uint32) << 7
    highs = np.concatenate([sign_exp | 0x00, sign_exp | 0x7F])
    lows = np.arange(65536, dtype=np.uint32)
    a = ((highs[:, None] << 16) | lows[None, :]).reshape(-1)
    few_lows = np.array([0, 1, 0x3FFF, 0x7FFE, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xC000, 0xFFFE,
                         0xFFFF, 0x1234, 0x4321, 0x7000, 0x9000, 0xF00D], np.uint32)
    b = ((np.arange(65536, dtype=np.uint32)[:, None] << 16) | few_lows[None, :]).reshape(-1)
    return np.concatenate([a, b])


def test_bf16_rounding_every_case_against_oracle():
    """With beta1 = 0 the new m is the grad itself, so the bf16 m the library
    stores is the grad rounded to bf16; m, v and the bf16 parameter after one
    step match the oracle bit for bit on every rounding case (a NaN only has
    to stay a NaN: payloads through the arithmetic are not compared)."""
    _need_gpu()
    say("case: bf16 rounding, all cases")
    g_bits = _bf16_rounding_patterns()
    n = int(g_bits.size)
    grp = [W.Group(lr=1e-3, beta1=0.0, beta2=0.999, eps=1e-8, weight_decay=0.0)]
    opt = GpuOpt([n], [W.BF16], [W.F32], [0], 1, W.STATE_BF16)
    g_dev = torch.from_numpy(g_bits.view(np.int32)).to(DEV).view(torch.float32)
    theta = torch.zeros(n, dtype=torch.bfloat16, device=DEV)
    opt.step(grp, [theta], [g_dev])
    torch.cuda.synchronize()
    ref = oracle.OracleAdamW([n], [W.BF16], [W.F32], [0], W.STATE_BF16)
    th_ref = [np.zeros(n, np.uint16)]
    ref.step(th_ref, [g_bits.view(np.float32)], grp)
    m_gpu, v_gpu = (bits(t) for t in opt.moments(0))
    for name, got, want in (("m", m_gpu, ref.m[0]), ("v", v_gpu, ref.v[0]),
                            ("theta", bits(theta), th_ref[0])):
        got_nan = np.isnan(oracle.bf16_to_f32(got))
        want_nan = np.isnan(oracle.bf16_to_f32(want))
        assert np.array_equal(got_nan, want_nan), name
        bad = int(np.count_nonzero(got[~got_nan] != want[~want_nan]))
        assert bad == 0, "%s: %d of %d values differ" % (name, bad, n)
    # the m path really is the plain conversion of the grad (0 + (-0) is +0)
    g32 = g_bits.view(np.float32)
    keep = ~np.isnan(g32) & (g_bits != 0x80000000)
    assert np.array_equal(ref.m[0][keep], oracle.f32_to_bf16(g32)[keep])
    opt.close()


def _extreme_values(n: int, rng: np.random.Generator, finite: bool, max_abs: float) -> np.ndarray:
    """fp32 values mixing the cases floating point treats specially: normal
    N(0, 1e-3) values, signed zeros, denormals, tiny normals, large values up
    to max_abs and, unless ``finite``, infinities and NaNs."""
    x = (rng.standard_normal(n) * 1e-3).astype(np.float32)
    kind = rng.integers(0, 20, n)
    sign = np.where(rng.integers(0, 2, n) == 1, -1.0, 1.0).astype(np.float32)
    den = (rng.integers(1, 1 << 23, n, dtype=np.uint32)).view(np.float32) * sign
    tiny = (10.0 ** rng.uniform(-38, -25, n)).astype(np.float32) * sign
    big = (10.0 ** rng.uniform(3, np.log10(max_abs), n)).astype(np.float32) * sign
    x = np.where(kind == 0, np.float32(0.0) * sign, x)
    x = np.where(kind == 1, den, x)
    x = np.where(kind == 2, tiny, x)
    x = np.where(kind == 3, big, x)
    if not finite:
        x = np.where(kind == 4, np.float32(np.inf) * sign, x)
        x = np.where(kind == 5, np.float32(np.nan), x)
    return x.astype(np.float32)


def _same_bits_or_both_nan(name, got, want, as_float):
    got_nan, want_nan = np.isnan(as_float(got)), np.isnan(as_float(want))
    assert np.array_equal(got_nan, want_nan), "%s: NaN positions differ" % name
    u = lambda a: a.view(np.uint32) if a.dtype == np.float32 else a     # compare bits
    bad = int(np.count_nonzero(u(got)[~got_nan] != u(want)[~want_nan]))
    assert bad == 0, "%s: %d of %d values differ" % (name, bad, got.size)


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
def test_extreme_values_against_oracle(fmt):
    """Grads and parameters with signed zeros, denormals, tiny and huge values
    (and, for the fp32 and bf16 moments, infinities and NaNs, which the
    update simply propagates); groups with eps = 0 (0/0 appears) and with
    beta1 = 0; six calls.  Every finite value bit-exact against the oracle,
    NaNs in the same places.  The 8-bit codes are defined for finite moments
    only, so that format gets finite inputs whose squares stay finite."""
    _need_gpu()
    say("case: extreme values", fmt)
    rng = np.random.default_rng(11)
    sizes = [4096, 4096, 1000, 777]
    pdt = [W.F32, W.BF16, W.F32, W.BF16]
    gdt = [W.F32, W.BF16, W.BF16, W.F32]
    group_of = [0, 1, 2, 0]
    groups = [W.Group(lr=1e-3, weight_decay=0.1), W.Group(lr=1e-2, eps=0.0),
              W.Group(lr=1e-3, beta1=0.0, weight_decay=0.01)]
    finite = fmt == W.STATE_Q8
    max_abs = 1e18 if finite else 3e38

    def host(x, dt):
        return x.copy() if dt == W.F32 else oracle.f32_to_bf16(x)

    def dev(h, dt):
        t = torch.from_numpy(h.view(np.int32) if dt == W.F32 else h.view(np.int16)).to(DEV)
        return t.view(torch.float32 if dt == W.F32 else torch.bfloat16)

    th_ref = [host(_extreme_values(n, rng, finite, max_abs), d) for n, d in zip(sizes, pdt)]
    params = [dev(h, d) for h, d in zip(th_ref, pdt)]
    opt = GpuOpt(sizes, pdt, gdt, group_of, len(groups), fmt)
    ref = oracle.OracleAdamW(sizes, pdt, gdt, group_of, fmt)
    for k in range(6):
        g_host = [host(_extreme_values(n, rng, finite, max_abs), d) for n, d in zip(sizes, gdt)]
        opt.step(groups, params, [dev(h, d) for h, d in zip(g_host, gdt)])
        ref.step(th_ref, g_host, groups)
    torch.cuda.synchronize()
    f32 = lambda a: a.view(np.float32)
    for i in range(len(sizes)):
        as_p = f32 if pdt[i] == W.F32 else oracle.bf16_to_f32
        _same_bits_or_both_nan("theta%d" % i, bits(params[i]), th_ref[i], as_p)
        m, v = (bits(t) for t in opt.moments(i))
        if fmt == W.STATE_Q8:
            assert np.array_equal(m, ref.m[i]) and np.array_equal(v, ref.v[i]), i
            ms, vs = (bits(t) for t in opt.scales(i))
            assert np.array_equal(ms.view(np.uint32), ref.m_scale[i].view(np.uint32)), i
            assert np.array_equal(vs.view(np.uint32), ref.v_scale[i].view(np.uint32)), i
        else:
            as_s = f32 if fmt == W.STATE_F32 else oracle.bf16_to_f32
            _same_bits_or_both_nan("m%d" % i, m, ref.m[i], as_s)
            _same_bits_or_both_nan("v%d" % i, v, ref.v[i], as_s)
    assert np.array_equal(bits(opt.steps()), ref.t)
    opt.close()


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
def test_views_into_flat_buffers_against_oracle(fmt):
    """Parameters and grads that are views into flat buffers at arbitrary
    element offsets (so most are not 16- or 8-byte aligned, and a parameter
    and its grad are misaligned differently): bit-exact against the oracle
    after three calls."""
    _need_gpu()
    say("case: flat-buffer views", fmt)
    rng = np.random.default_rng(5)
    sizes = [int(x) for x in rng.integers(1, 9000, 40)]
    pdt = [(W.F32, W.BF16)[i % 2] for i in range(len(sizes))]
    gdt = [(W.F32, W.BF16)[(i // 2) % 2] for i in range(len(sizes))]
    groups = [W.Group(lr=1e-3, weight_decay=0.1), W.Group(lr=3e-3, beta1=0.8, eps=1e-6)]
    group_of = [i % 2 for i in range(len(sizes))]
    flat = {W.F32: torch.zeros(sum(sizes) + 7, device=DEV),
            W.BF16: torch.zeros(sum(sizes) + 7, dtype=torch.bfloat16, device=DEV)}
    gflat = {W.F32: torch.zeros(sum(sizes) + 7, device=DEV),
             W.BF16: torch.zeros(sum(sizes) + 7, dtype=torch.bfloat16, device=DEV)}
    params, poff, goff = [], {W.F32: 1, W.BF16: 3}, {W.F32: 2, W.BF16: 1}
    views_g = []
    for n, pd, gd in zip(sizes, pdt, gdt):
        params.append(flat[pd][poff[pd]:poff[pd] + n])
        poff[pd] += n
        views_g.append(gflat[gd][goff[gd]:goff[gd] + n])
        goff[gd] += n
    gen = torch.Generator().manual_seed(9)
    p_cpu = [(torch.randn(n, generator=gen) * 0.02).to(W.TORCH_DTYPE[d]) for n, d in zip(sizes, pdt)]
    for p, c in zip(params, p_cpu):
        p.copy_(c)
    th_ref = [bits(c) for c in p_cpu]
    opt = GpuOpt(sizes, pdt, gdt, group_of, len(groups), fmt)
    ref = oracle.OracleAdamW(sizes, pdt, gdt, group_of, fmt)
    for k in range(3):
        g_cpu = [(torch.randn(n, generator=gen) * 1e-3).to(W.TORCH_DTYPE[d]) for n, d in zip(sizes, gdt)]
        for v, c in zip(views_g, g_cpu):
            v.copy_(c)
        opt.step(groups, params, views_g)
        ref.step(th_ref, [bits(c) for c in g_cpu], groups)
    torch.cuda.synchronize()
    for i in range(len(sizes)):
        assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, i
        m, v = (bits(t) for t in opt.moments(i))
        assert n_bit_mismatch(m, ref.m[i]) == 0 and n_bit_mismatch(v, ref.v[i]) == 0, i
    opt.close()


def test_null_arrays_reuse_the_previous_call_and_read_steps():
    """params / grads passed as NULL arrays mean the previous call's arrays:
    three calls with NULL arrays after one explicit call give the same bits
    as four explicit calls; apexw_read_steps copies the counters."""
    _need_gpu()
    say("case: NULL arrays reuse the previous call")
    w = W.tiny()
    outs = []
    for reuse in (False, True):
        p_cpu = W.init_params(w, "cpu")
        params = [p.to(DEV) for p in p_cpu]
        grads = [torch.randn(s, generator=torch.Generator().manual_seed(3)).mul_(1e-3).to(DEV)
                 for s in w.shapes]
        opt = GpuOpt(w.numels, w.param_dtype, w.grad_dtype, w.group_of, 1, w.state_fmt)
        pa = L.make_ptrs([p.data_ptr() for p in params])
        ga = L.make_ptrs([g.data_ptr() for g in grads])
        for k in range(4):
            if reuse and k > 0:
                L.apexw_step(opt.h, L.make_groups(w.groups), 1, None, None, 0, opt.stream)
            else:
                L.apexw_step(opt.h, L.make_groups(w.groups), 1, pa, ga, 0, opt.stream)
        torch.cuda.synchronize()
        outs.append((torch.cat([p.reshape(-1) for p in params]).cpu(), opt.state.cpu()))
        assert L.apexw_read_steps(opt.h, len(w.numels), opt.stream) == [4] * len(w.numels)
        opt.close()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    # a fresh handle has no previous arrays
    opt = GpuOpt(w.numels, w.param_dtype, w.grad_dtype, w.group_of, 1, w.state_fmt)
    with pytest.raises(L.ApexwError) as e:
        L.apexw_step(opt.h, L.make_groups(w.groups), 1, None, None, 0, opt.stream)
    assert e.value.code == L.APEXW_EINVAL
    opt.close()


def test_thirty_two_groups_with_edge_hyperparameters_against_oracle():
    """The maximum of 32 parameter groups, each with its own hyperparameters
    -- among them lr = 0 (theta unchanged), beta2 = 0, a decay factor
    1 - lr*wd below zero, a large eps, eps = 0, beta1 = 0, betas within
    1e-7 of 1 (tiny bias corrections) -- over 64 tensors of mixed dtypes,
    three calls, bit-exact against the oracle in every state format."""
    _need_gpu()
    say("case: 32 groups")
    rng = np.random.default_rng(21)
    groups = []
    for gi in range(32):
        groups.append(W.Group(lr=float(10 ** rng.uniform(-5, -1)), beta1=float(rng.uniform(0, 0.99)),
                              beta2=float(rng.uniform(0.5, 0.9999)), eps=float(10 ** rng.uniform(-10, -4)),
                              weight_decay=float(rng.uniform(0, 0.2))))
    groups[0] = W.Group(lr=0.0, weight_decay=0.5)
    groups[1] = W.Group(lr=1e-3, beta2=0.0)
    groups[2] = W.Group(lr=0.5, weight_decay=3.0)          # 1 - lr*wd = -0.5
    groups[3] = W.Group(lr=1e-2, eps=1.0)
    groups[4] = W.Group(lr=1e-3, eps=0.0)
    groups[5] = W.Group(lr=1e-3, beta1=0.0, beta2=0.999999)
    groups[6] = W.Group(lr=1e-3, beta1=0.9999999, beta2=0.99999999)   # bias corrections ~1e-7, 1e-8
    sizes = [int(x) for x in rng.integers(1, 3000, 64)]
    pdt = [(W.F32, W.BF16)[i % 2] for i in range(64)]
    gdt = [(W.F32, W.BF16)[(i // 2) % 2] for i in range(64)]
    group_of = [i % 32 for i in range(64)]
    for fmt in (W.STATE_F32, W.STATE_BF16, W.STATE_Q8):
        gen = torch.Generator().manual_seed(22)
        p_cpu = [(torch.randn(n, generator=gen) * 0.02).to(W.TORCH_DTYPE[d]) for n, d in zip(sizes, pdt)]
        params = [p.to(DEV) for p in p_cpu]
        th_ref = [bits(p) for p in p_cpu]
        opt = GpuOpt(sizes, pdt, gdt, group_of, 32, fmt)
        ref = oracle.OracleAdamW(sizes, pdt, gdt, group_of, fmt)
        for k in range(3):
            g_cpu = [(torch.randn(n, generator=gen) * 1e-3).to(W.TORCH_DTYPE[d]) for n, d in zip(sizes, gdt)]
            opt.step(groups, params, [g.to(DEV) for g in g_cpu])
            ref.step(th_ref, [bits(g) for g in g_cpu], groups)
        torch.cuda.synchronize()
        for i in range(64):
            assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, (fmt, i)
            m, v = (bits(t) for t in opt.moments(i))
            assert n_bit_mismatch(m, ref.m[i]) == 0 and n_bit_mismatch(v, ref.v[i]) == 0, (fmt, i)
        # lr = 0: theta of group 0's tensors is unchanged
        for i in (0, 32):
            assert n_bit_mismatch(bits(params[i]), bits(p_cpu[i])) == 0
        opt.close()


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_Q8])
def test_large_step_counters_against_oracle(fmt):
    """Step counters set far along (as a resumed run would have them, written
    straight into the caller-owned state buffer, up to t = 2^31 - 2 so the
    step reaches the largest int32): beta^t by square-and-multiply over all
    31 bits, bias corrections that round to 1, bit-exact against the oracle
    in both launch modes."""
    _need_gpu()
    say("case: large step counters", fmt)
    sizes = [1000, 4096, 77]
    t0 = [2 ** 31 - 2, 1_000_003, 12_345]
    groups = [W.Group(lr=1e-3, weight_decay=0.1, beta1=0.9, beta2=0.999999)]
    for mode in (1, 2, 3):
        gen = torch.Generator().manual_seed(91)
        p_cpu = [torch.randn(n, generator=gen) * 0.02 for n in sizes]
        params = [p.to(DEV) for p in p_cpu]
        th_ref = [bits(p) for p in p_cpu]
        opt = GpuOpt(sizes, [W.F32] * 3, [W.F32] * 3, [0, 0, 0], 1, fmt)
        L.apexw_set_launch_mode(opt.h, mode)
        ref = oracle.OracleAdamW(sizes, [W.F32] * 3, [W.F32] * 3, [0, 0, 0], fmt)
        opt.steps().copy_(torch.tensor(t0, dtype=torch.int32))
        ref.t[:3] = t0
        for k in range(1 if mode == 2 else 2):
            g_cpu = [torch.randn(n, generator=gen) * 1e-3 for n in sizes]
            if k == 1:                              # t[0] is at the int32 maximum now
                g_cpu[0] = None
            opt.step(groups, params, [None if g is None else g.to(DEV) for g in g_cpu])
            ref.step(th_ref, [None if g is None else bits(g) for g in g_cpu], groups)
        torch.cuda.synchronize()
        assert np.array_equal(bits(opt.steps()), ref.t[:3])
        assert ref.t[0] == 2 ** 31 - 1
        for i in range(3):
            assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, (mode, i)
            m, v = (bits(t) for t in opt.moments(i))
            assert n_bit_mismatch(m, ref.m[i]) == 0 and n_bit_mismatch(v, ref.v[i]) == 0, (mode, i)
        opt.close()


def test_single_launch_counters_over_many_steps():
    """The single-launch step's arrival counters must be back at zero after
    every launch: 300 steps of a two-launch list (two dtype pairs) in the
    single-launch mode, with the workgroup cap changed at random between
    steps (below, at and above the 64 first-level counters; the expected
    arrival counts change with it), random skipped steps and random absent
    grads; step counters against their definition after every step, and
    theta, m, v bit-exact against the oracle at the end."""
    _need_gpu()
    say("case: single launch, 300 steps")
    sizes = [70_000, 513, 129_000, 1]
    pdt = [W.F32, W.BF16, W.F32, W.BF16]
    gdt = [W.F32, W.F32, W.F32, W.F32]
    groups = [W.Group(lr=1e-3, weight_decay=0.05)]
    rng = np.random.default_rng(123)
    gen = torch.Generator().manual_seed(124)
    p_cpu = [(torch.randn(n, generator=gen) * 0.02).to(W.TORCH_DTYPE[d]) for n, d in zip(sizes, pdt)]
    params = [p.to(DEV) for p in p_cpu]
    th_ref = [bits(p) for p in p_cpu]
    opt = GpuOpt(sizes, pdt, gdt, [0] * 4, 1, W.STATE_F32)
    L.apexw_set_launch_mode(opt.h, 2)
    ref = oracle.OracleAdamW(sizes, pdt, gdt, [0] * 4, W.STATE_F32)
    fi = torch.zeros(1, device=DEV)
    want = np.zeros(4, np.int32)
    caps = [0, 1, 5, 63, 64, 65, 200, 513]
    for k in range(300):
        L.apexw_set_workgroups(opt.h, int(rng.choice(caps)))
        present = rng.random(4) < 0.8
        skip = rng.random() < 0.1
        g_cpu = [torch.randn(n, generator=gen) * 1e-3 for n in sizes]
        fi.fill_(1.0 if skip else 0.0)
        opt.step(groups, params, [g.to(DEV) if ok else None for g, ok in zip(g_cpu, present)],
                 found_inf=fi)
        ref.step(th_ref, [bits(g) if ok else None for g, ok in zip(g_cpu, present)], groups,
                 found_inf=skip)
        if not skip:
            want += present.astype(np.int32)
        torch.cuda.synchronize()
        assert np.array_equal(bits(opt.steps()), want), (k, bits(opt.steps()), want)
    assert np.array_equal(ref.t[:4], want)
    for i in range(4):
        assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, i
        m, v = opt.moments(i)
        assert n_bit_mismatch(bits(m), ref.m[i]) == 0 and n_bit_mismatch(bits(v), ref.v[i]) == 0, i
    opt.close()


def test_all_grads_absent_and_pointer_changes():
    """No grads at all: nothing changes.  Grads moved to new buffers between
    calls: the library follows the new pointers."""
    _need_gpu()
    say("case: absent grads / moved grads")
    w = W.tiny()
    p_cpu = W.init_params(w, "cpu")
    params = [p.to(DEV) for p in p_cpu]
    opt = GpuOpt(w.numels, w.param_dtype, w.grad_dtype, w.group_of, 1, w.state_fmt)
    ref = _oracle_for(w)
    th_ref = [bits(p) for p in p_cpu]
    opt.step(w.groups, params, [None] * 4)
    ref.step(th_ref, [None] * 4, w.groups)
    for k in range(1, 6):
        g_cpu = W.grads_for_call(w, k, "cpu")
        g_cpu = [g if g is not None else torch.zeros(s) for g, s in zip(g_cpu, w.shapes)]
        g_dev = [g.to(DEV) for g in g_cpu]      # fresh allocations every call
        keep = [torch.empty(1 << 20, device=DEV) for _ in range(k)]  # shift the allocator
        opt.step(w.groups, params, g_dev)
        ref.step(th_ref, [bits(g) for g in g_cpu], w.groups)
        del keep
    torch.cuda.synchronize()
    for i in range(4):
        assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0
    assert list(bits(opt.steps())) == [5, 5, 5, 5]
    opt.close()


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
@pytest.mark.parametrize("wg,mode", [(1, 2), (7, 2), (63, 2), (64, 2), (65, 2), (300, 2), (0, 2),
                                     (1, 1), (300, 1), (1, 3), (7, 3), (300, 3), (0, 3)])
def test_results_do_not_depend_on_grid(wg, mode, fmt):
    """Workgroup caps (a workgroup then walks several tiles) in both launch
    modes -- for the single launch, caps below, at and above the 64 counters
    of the arrival tree's first level -- against prepare + update at the
    default grid, over three calls (the arrival counters must reset)."""
    _need_gpu()
    say("case: grid", wg, "mode", mode, "fmt", fmt)
    w = dataclasses.replace(W.many_small(n_tensors=120), state_fmt=fmt)   # 5,847 tiles
    outs = []
    for setting, md in ((wg, mode), (0, 1)):
        params = W.init_params(w, DEV)
        opt = GpuOpt(w.numels, w.param_dtype, w.grad_dtype, w.group_of, 3, w.state_fmt)
        L.apexw_set_workgroups(opt.h, setting)
        L.apexw_set_launch_mode(opt.h, md)
        for k in range(1, 4):
            opt.step(w.groups, params, W.grads_for_call(w, k, DEV))
        torch.cuda.synchronize()
        outs.append((torch.cat([p.reshape(-1) for p in params]).cpu(), opt.state.cpu()))
        opt.close()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_Q8])
def test_results_do_not_depend_on_tensor_order(fmt):
    """The same tensors listed in a shuffled order (so their tiles, launch
    positions and table stripes all change): every tensor's theta, moments,
    scales and counter are bitwise the same."""
    _need_gpu()
    say("case: tensor order", fmt)
    w = dataclasses.replace(W.many_small(n_tensors=120), state_fmt=fmt)
    n = len(w.shapes)
    perm = np.random.default_rng(31).permutation(n)
    runs = []
    for order in (np.arange(n), perm):
        p_all = W.init_params(w, DEV)
        params = [p_all[i] for i in order]
        opt = GpuOpt([w.numels[i] for i in order], [w.param_dtype[i] for i in order],
                     [w.grad_dtype[i] for i in order], [w.group_of[i] for i in order], 3, fmt)
        for k in range(1, 4):
            g_all = W.grads_for_call(w, k, DEV)
            opt.step(w.groups, params, [g_all[i] for i in order])
        torch.cuda.synchronize()
        res = {}
        for j, i in enumerate(order):
            m, v = opt.moments(j)
            res[int(i)] = [bits(params[j]), bits(m), bits(v)]
            if fmt == W.STATE_Q8:
                res[int(i)] += [bits(t) for t in opt.scales(j)]
        runs.append(res)
        opt.close()
    for i in range(n):
        for a, b in zip(runs[0][i], runs[1][i]):
            assert n_bit_mismatch(a, b) == 0, i


# =================================================================== configs

def _sampled_run(w: W.Workload, sample_tensors, elems=None, seed=0, every=None,
                 ref_fmt=None, calls=None):
    """Run the whole workload on the GPU; run the oracle on a sample: whole
    tensors ``sample_tensors`` or, with ``elems`` (dict i -> index array), the
    given elements (for fp32 / bf16 state, where elements are independent).
    Returns (opt, params, ref, th_ref, idx)."""
    calls = calls or w.steps
    params = W.init_params(w, DEV)
    grads = [torch.empty(s, dtype=W.TORCH_DTYPE[d], device=DEV) for s, d in zip(w.shapes, w.grad_dtype)]
    opt = GpuOpt(w.numels, w.param_dtype, w.grad_dtype, w.group_of, len(w.groups), w.state_fmt)
    idx = {}
    for i in sample_tensors:
        idx[i] = (torch.arange(w.numels[i]) if elems is None or i not in elems
                  else torch.as_tensor(elems[i]))
    sel = list(sample_tensors)
    sub_n = [int(idx[i].numel()) for i in sel]
    ref = oracle.OracleAdamW(sub_n, [w.param_dtype[i] for i in sel], [w.grad_dtype[i] for i in sel],
                             [w.group_of[i] for i in sel], ref_fmt or w.state_fmt)
    idx_dev = {i: idx[i].to(DEV) for i in sel}
    th_ref = [bits(params[i].reshape(-1)[idx_dev[i]]) for i in sel]
    fi = torch.zeros(1, device=DEV)
    for k in range(1, calls + 1):
        g_list = W.grads_for_call(w, k, DEV, out=grads)
        skip = w.skip_call(k)
        fi.fill_(1.0 if skip else 0.0)
        opt.step(w.groups, params, g_list, found_inf=fi)
        ref.step(th_ref, [None if g_list[i] is None else bits(g_list[i].reshape(-1)[idx_dev[i]])
                          for i in sel], w.groups, found_inf=skip)
        if every and k % every == 0:
            say("  call", k)
    torch.cuda.synchronize()
    return opt, params, ref, th_ref, idx_dev


def _spread_indices(n, count, rng):
    """Sorted sample of element indices: the first and last tile plus random
    elements in between."""
    head = np.arange(min(n, 4096))
    tail = np.arange(max(0, n - 4096), n)
    mid = rng.choice(n, size=min(n, count), replace=False)
    return np.unique(np.concatenate([head, tail, mid]))


def test_many_small_reduced_full_oracle():
    """2,000 log-uniform tensors (3 groups round-robin), 10 calls, every
    element against the oracle."""
    _need_gpu()
    w = W.many_small(n_tensors=2000)
    say("case: many_small reduced", w.describe())
    opt, params, ref, th_ref, idx = _sampled_run(w, range(len(w.shapes)))
    mism = 0
    for j, i in enumerate(range(len(w.shapes))):
        m, v = opt.moments(i)
        for name, a, b in (("theta", bits(params[i]), th_ref[j]), ("m", bits(m), ref.m[j]),
                           ("v", bits(v), ref.v[j])):
            assert rel_err_elementwise(a, b) <= 1e-5, (name, i)
            mism += n_bit_mismatch(a, b)
    assert np.array_equal(bits(opt.steps()), ref.t)
    say("  bit mismatches:", mism)
    assert mism == 0
    opt.close()


def test_many_small_full_size_sampled():
    """The 20,000-tensor list (about 189M params), 10 calls; 400 whole tensors
    (the smallest, the largest, random) against the oracle."""
    _need_gpu()
    w = W.many_small()
    say("case: many_small full", w.describe())
    rng = np.random.default_rng(0)
    order = np.argsort(w.numels)
    pick = sorted(set(order[:50].tolist() + order[-50:].tolist() +
                      rng.choice(len(w.shapes), 300, replace=False).tolist()))
    opt, params, ref, th_ref, idx = _sampled_run(w, pick)
    for j, i in enumerate(pick):
        m, v = opt.moments(i)
        assert rel_err_elementwise(bits(params[i]), th_ref[j]) <= 1e-5
        assert rel_err_elementwise(bits(m), ref.m[j]) <= 1e-5
        assert rel_err_elementwise(bits(v), ref.v[j]) <= 1e-5
        assert n_bit_mismatch(bits(params[i]), th_ref[j]) == 0
    st = bits(opt.steps())
    assert np.all(st == 10)
    opt.close()


def _few_large_check(w):
    rng = np.random.default_rng(1)
    elems = {i: _spread_indices(w.numels[i], 60000, rng) for i in range(len(w.shapes))}
    opt, params, ref, th_ref, idx = _sampled_run(w, range(len(w.shapes)), elems=elems)
    for i in range(len(w.shapes)):
        m, v = opt.moments(i)
        gm, gv = bits(m[idx[i]]), bits(v[idx[i]])
        gth = bits(params[i].reshape(-1)[idx[i]])
        nb = n_bit_mismatch(gth, th_ref[i]) + n_bit_mismatch(gm, ref.m[i]) + n_bit_mismatch(gv, ref.v[i])
        say("  tensor %d: theta rel %.3g, m rel %.3g, v rel %.3g, bit mismatches %d / %d" % (
            i, rel_err_elementwise(gth, th_ref[i]), rel_err_elementwise(gm, ref.m[i]),
            rel_err_elementwise(gv, ref.v[i]), nb, 3 * gth.size))
        if w.state_fmt == W.STATE_F32:
            assert rel_err_elementwise(gm, ref.m[i]) <= 1e-5
            assert rel_err_elementwise(gv, ref.v[i]) <= 1e-5
            assert rel_err_elementwise(gth, th_ref[i]) <= 1e-5
        assert nb == 0
    assert np.all(bits(opt.steps()) == w.steps)
    return opt, params, idx


def test_few_large_full_size_sampled():
    """8 bf16 [8192,8192] params, fp32 grads and state, 10 calls (the
    benchmark's launch configuration); 60k+ elements per tensor, including the
    first and last tiles, against the oracle."""
    _need_gpu()
    w = W.few_large()
    say("case: few_large", w.describe())
    opt, _, _ = _few_large_check(w)
    opt.close()


def test_few_large_zero1_share_full_size_sampled():
    """One of 8 ranks' ZeRO-1 share of that list (a 1024-row slice of every
    tensor, 67.1M params), the launch configuration the benchmark times for
    it; 60k+ elements per tensor, including the first and last tiles, against
    the oracle."""
    _need_gpu()
    w = W.few_large_shard(ranks=8)
    say("case: few_large_shard8", w.describe())
    opt, _, _ = _few_large_check(w)
    opt.close()


def test_bf16_state_full_size_sampled_and_against_fp32_state():
    """The same list with bf16 moments: bitwise against the oracle's bf16
    mode, and within 1e-2 (normwise) of the fp32-state oracle on m and v."""
    _need_gpu()
    w = W.bf16_state()
    say("case: bf16_state", w.describe())
    rng = np.random.default_rng(2)
    pick = [0, 7]
    elems = {i: _spread_indices(w.numels[i], 30000, rng) for i in pick}
    opt, params, ref, th_ref, idx = _sampled_run(w, pick, elems=elems)
    # fp32-state oracle on the same inputs
    ref32 = oracle.OracleAdamW([len(elems[i]) for i in pick], [W.BF16] * 2, [W.F32] * 2, [0, 0], "f32")
    p0 = W.init_params(w, DEV)
    th32 = [bits(p0[i].reshape(-1)[idx[i]]) for i in pick]
    del p0
    for k in range(1, w.steps + 1):
        g = W.grads_for_call(w, k, DEV)
        ref32.step(th32, [bits(g[i].reshape(-1)[idx[i]]) for i in pick], w.groups)
        del g
    for j, i in enumerate(pick):
        m, v = opt.moments(i)
        gm, gv = bits(m[idx[i]]), bits(v[idx[i]])
        assert n_bit_mismatch(gm, ref.m[j]) == 0 and n_bit_mismatch(gv, ref.v[j]) == 0
        assert n_bit_mismatch(bits(params[i].reshape(-1)[idx[i]]), th_ref[j]) == 0
        em, ev = normwise_err(gm, ref32.m[j]), normwise_err(gv, ref32.v[j])
        eth = normwise_err(bits(params[i].reshape(-1)[idx[i]]), th32[j])
        say("  tensor %d vs fp32-state oracle: m %.3g v %.3g theta %.3g (normwise)" % (i, em, ev, eth))
        assert em <= 1e-2 and ev <= 1e-2
    opt.close()


def _q8_check(opt, params, ref, th_ref, pick, label):
    worst_code, worst_scale = 0, 0.0
    for j, i in enumerate(pick):
        m, v = opt.moments(i)
        ms, vs = opt.scales(i)
        dm = np.abs(bits(m).astype(np.int32) - ref.m[j].astype(np.int32))
        dv = np.abs(bits(v).astype(np.int32) - ref.v[j].astype(np.int32))
        worst_code = max(worst_code, int(dm.max(initial=0)), int(dv.max(initial=0)))
        for a, b in ((bits(ms), ref.m_scale[j]), (bits(vs), ref.v_scale[j])):
            worst_scale = max(worst_scale, rel_err_elementwise(a, b))
        assert n_bit_mismatch(bits(params[i]), th_ref[j]) == 0, i
        assert n_bit_mismatch(bits(m), ref.m[j]) == 0 and n_bit_mismatch(bits(v), ref.v[j]) == 0, i
    say("  %s: worst code diff %d, worst scale rel %.3g" % (label, worst_code, worst_scale))
    assert worst_code <= 1 and worst_scale <= 1e-6


def test_lora_q8_reduced_full_oracle():
    """Two LoRA layers (28 tensors), 40 calls, every code and scale."""
    _need_gpu()
    w = W.lora_q8(layers=2)
    say("case: lora_q8 reduced", w.describe())
    pick = list(range(len(w.shapes)))
    opt, params, ref, th_ref, _ = _sampled_run(w, pick, calls=40)
    _q8_check(opt, params, ref, th_ref, pick, "2 layers, 40 calls")
    assert np.all(bits(opt.steps()) == 40)
    opt.close()


def test_lora_q8_full_size_sampled():
    """392 LoRA tensors (24.3M params), 250 calls; 30 whole tensors (each
    shape class) against the oracle."""
    _need_gpu()
    w = W.lora_q8()
    say("case: lora_q8 full", w.describe())
    pick = list(range(0, 14)) + list(range(14 * 27, 14 * 28)) + [150, 151]
    opt, params, ref, th_ref, _ = _sampled_run(w, pick, every=50)
    _q8_check(opt, params, ref, th_ref, pick, "28 layers, 250 calls")
    assert np.all(bits(opt.steps()) == 250)
    opt.close()


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
def test_maximum_size_tensor_past_int32(fmt):
    """One bf16 tensor of 2^31 + 4099 elements (64-bit element offsets, 8.4M
    tiles, a 3-element final 8-bit block), bf16 grads, 2 calls; whole
    256-element blocks sampled around element 2^31, at both ends and at
    random, against the oracle."""
    _need_gpu()
    n = (1 << 31) + 4099
    say("case: maximum size", fmt, n)
    gen = torch.Generator(device=DEV).manual_seed(11)
    theta = (torch.randn(n, generator=gen, device=DEV) * 0.02).to(torch.bfloat16)
    grad = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    opt = GpuOpt([n], [W.BF16], [W.BF16], [0], 1, fmt)
    rng = np.random.default_rng(12)
    nblocks = (n + 255) // 256
    picks = sorted(set([0, 1, (1 << 23) - 1, 1 << 23, (1 << 23) + 1, nblocks - 2, nblocks - 1] +
                       rng.integers(0, nblocks, 40).tolist()))
    spans = [(b * 256, min(n, b * 256 + 256)) for b in picks]
    idx = torch.cat([torch.arange(lo, hi) for lo, hi in spans]).to(DEV)
    sizes = [hi - lo for lo, hi in spans]
    ref = oracle.OracleAdamW(sizes, [W.BF16] * len(sizes), [W.BF16] * len(sizes), [0] * len(sizes), fmt)
    th0 = bits(theta[idx])
    th_ref = np.split(th0, np.cumsum(sizes)[:-1])
    th_ref = [x.copy() for x in th_ref]
    groups = [W.Group(lr=1e-3, weight_decay=0.1)]
    for k in range(2):
        grad.copy_((torch.randn(n, generator=gen, device=DEV) * 1e-3).to(torch.bfloat16))
        opt.step(groups, [theta], [grad])
        gs = np.split(bits(grad[idx]), np.cumsum(sizes)[:-1])
        ref.step(th_ref, [x.copy() for x in gs], groups)
    torch.cuda.synchronize()
    got = np.split(bits(theta[idx]), np.cumsum(sizes)[:-1])
    m, v = opt.moments(0)
    gm = np.split(bits(m[idx]), np.cumsum(sizes)[:-1])
    gv = np.split(bits(v[idx]), np.cumsum(sizes)[:-1])
    for j, b in enumerate(picks):
        assert n_bit_mismatch(got[j], th_ref[j]) == 0, b
        assert n_bit_mismatch(gm[j], ref.m[j]) == 0 and n_bit_mismatch(gv[j], ref.v[j]) == 0, b
        if fmt == W.STATE_Q8:
            ms, vs = opt.scales(0)
            assert bits(ms[b:b + 1])[0] == ref.m_scale[j][0] and bits(vs[b:b + 1])[0] == ref.v_scale[j][0]
    assert list(bits(opt.steps())) == [2]
    opt.close()
    del theta, grad
    torch.cuda.empty_cache()


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_Q8])
def test_carried_step_restarts(fmt):
    """The carried step (the default launch mode) over 12 calls of a two-launch
    list, checked against the oracle after every call, through every event
    that starts its chain of bias corrections again or must leave it intact:
    a skipped call, a changed beta2, a switch to prepare + update and back,
    one dtype pair without any grad, step counters written by the caller
    followed by apexw_set_launch_mode, a call with no grad at all, and an
    import of a state exported five calls earlier."""
    _need_gpu()
    say("case: carried step restarts", fmt)
    sizes = [3000, 257, 4096, 1000, 513]
    pdt = [W.F32, W.F32, W.F32, W.BF16, W.BF16]
    gdt = [W.F32, W.F32, W.F32, W.BF16, W.BF16]
    group_of = [0, 1, 0, 1, 0]
    gen = torch.Generator().manual_seed(57)
    p_cpu = [(torch.randn(s, generator=gen) * 0.02).to(W.TORCH_DTYPE[d]) for s, d in zip(sizes, pdt)]
    params = [p.to(DEV) for p in p_cpu]
    th_ref = [bits(p) for p in p_cpu]
    opt = GpuOpt(sizes, pdt, gdt, group_of, 2, fmt)
    assert L.apexw_get_launch_mode(opt.h) == 3
    ref = oracle.OracleAdamW(sizes, pdt, gdt, group_of, fmt)
    fi = torch.zeros(1, device=DEV)
    blob = snap = None
    for k in range(1, 13):
        beta2 = 0.99 if k < 4 else 0.995
        groups = [W.Group(lr=1e-3, weight_decay=0.1), W.Group(lr=5e-4, beta1=0.8, beta2=beta2)]
        g_cpu = [(torch.randn(s, generator=gen) * 1e-3).to(W.TORCH_DTYPE[d]) for s, d in zip(sizes, gdt)]
        present = [True] * len(sizes)
        if k == 8:
            present[3] = present[4] = False          # the bf16 launch has nothing to do
        if k == 10:
            present = [False] * len(sizes)
        if k == 6:
            L.apexw_set_launch_mode(opt.h, 1)
        if k == 7:
            L.apexw_set_launch_mode(opt.h, 3)
        if k == 9:                                   # counters rewritten by the caller
            torch.cuda.synchronize()
            opt.steps().add_(5)
            ref.t[:len(sizes)] += 5
            L.apexw_set_launch_mode(opt.h, 0)
        if k == 11:
            L.apexw_import_state(opt.h, blob, 2, opt.stream)
            ref.t, ref.m, ref.v, ref.m_scale, ref.v_scale = snap
            snap = None
        skip = k == 3
        fi.fill_(1.0 if skip else 0.0)
        opt.step(groups, params, [g.to(DEV) if ok else None for g, ok in zip(g_cpu, present)],
                 found_inf=fi)
        ref.step(th_ref, [bits(g) if ok else None for g, ok in zip(g_cpu, present)], groups,
                 found_inf=skip)
        torch.cuda.synchronize()
        assert np.array_equal(bits(opt.steps()), ref.t), (k, bits(opt.steps()), ref.t)
        for i in range(len(sizes)):
            assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, (k, i)
            m, v = opt.moments(i)
            assert n_bit_mismatch(bits(m), ref.m[i]) == 0, (k, i)
            assert n_bit_mismatch(bits(v), ref.v[i]) == 0, (k, i)
            if fmt == W.STATE_Q8:
                ms, vs = opt.scales(i)
                assert n_bit_mismatch(bits(ms), ref.m_scale[i]) == 0, (k, i)
                assert n_bit_mismatch(bits(vs), ref.v_scale[i]) == 0, (k, i)
        if k == 5:
            blob = L.apexw_export_state(opt.h, L.make_groups(groups), 2, opt.stream)
            snap = (ref.t.copy(), [a.copy() for a in ref.m], [a.copy() for a in ref.v],
                    [None if a is None else a.copy() for a in ref.m_scale],
                    [None if a is None else a.copy() for a in ref.v_scale])
    assert list(ref.t) == [6, 6, 6, 6, 6]      # call 5 left t = 4; calls 11 and 12 follow the import
    opt.close()


def test_launch_mode_choice():
    """Which mode a step takes: the carried step needs a list without empty
    tensors (APEXW_EINVAL when forced otherwise, and the default falls back
    to the single launch); every list without one defaults to it, 8-bit or
    dense, small or streamed; forced modes are kept."""
    _need_gpu()
    say("case: launch mode choice")
    opt = GpuOpt([1000, 0, 77], [W.F32] * 3, [W.F32] * 3, [0, 0, 0], 1, W.STATE_F32)
    assert L.apexw_get_launch_mode(opt.h) == 2
    with pytest.raises(L.ApexwError) as e:
        L.apexw_set_launch_mode(opt.h, 3)
    assert e.value.code == L.APEXW_EINVAL
    assert L.apexw_get_launch_mode(opt.h) == 2
    opt.close()
    small = GpuOpt([4096, 300], [W.BF16] * 2, [W.BF16] * 2, [0, 0], 1, W.STATE_Q8)
    assert L.apexw_get_launch_mode(small.h) == 3
    L.apexw_set_cache_policy(small.h, 1)             # streaming
    assert L.apexw_get_launch_mode(small.h) == 3
    L.apexw_set_launch_mode(small.h, 1)
    assert L.apexw_get_launch_mode(small.h) == 1
    L.apexw_set_launch_mode(small.h, 2)
    assert L.apexw_get_launch_mode(small.h) == 2
    small.close()
    w = W.lora_q8()
    big = GpuOpt(w.numels, w.param_dtype, w.grad_dtype, w.group_of, len(w.groups), w.state_fmt)
    assert L.apexw_get_launch_mode(big.h) == 3       # 146 MB per step: streams
    big.close()
    fl = GpuOpt([1 << 22] * 4, [W.BF16] * 4, [W.F32] * 4, [0] * 4, 1, W.STATE_F32)
    assert L.apexw_get_launch_mode(fl.h) == 3        # streams too, dense moments
    fl.close()



# Tile kinds of the short-form boundary test: which quantity sits near which
# edge, and on which side (+1 inside the short forms' range, -1 outside).
_EDGE_KINDS = [("v_lo", +1), ("v_lo", -1), ("vhat_hi", +1), ("vhat_hi", -1),
               ("x_lo", +1), ("x_lo", -1), ("x_hi", +1), ("x_hi", -1), ("plain", 0)]


def _edge_state(n, rng, group, t0, beta1, beta2):
    """Moments (fp32, m signed) and grads for one tensor whose 256-element
    tiles each put one quantity of the first update just inside or just
    outside an edge of the short forms' range: v >= 2^-96, v / bc2 < 2^56,
    |lr * m_hat| >= 2^-96, |lr * m_hat| < 2^64 (within a factor 2^0.1 .. 2^3
    of the edge; boundary tiles get zero grads, so the moments only decay),
    or ordinary values.  Returns m, v, g and the kind of every tile."""
    bc1 = 1.0 - beta1 ** (t0 + 1)
    bc2 = 1.0 - beta2 ** (t0 + 1)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float64)
    v = np.abs(rng.standard_normal(n) * 1e-8)
    g = rng.standard_normal(n) * 1e-3
    kinds = []
    for t in range((n + 255) // 256):
        sl = slice(256 * t, min(n, 256 * t + 256))
        k = int(rng.integers(0, len(_EDGE_KINDS)))
        kinds.append(k)
        what, side = _EDGE_KINDS[k]
        if what == "plain":
            continue
        cnt = sl.stop - sl.start
        f = np.exp2(rng.uniform(0.1, 3.0, cnt))          # how far from the edge
        sign = np.where(rng.integers(0, 2, cnt) == 1, -1.0, 1.0)
        g[sl] = 0.0
        if what == "v_lo":           # v after the update = beta2 * v_old
            v[sl] = 2.0 ** -96 * f ** side / beta2
        elif what == "vhat_hi":      # v_hat = beta2 * v_old / bc2
            v[sl] = 2.0 ** 56 * f ** -side * bc2 / beta2
        elif what == "x_lo":         # x = lr * beta1 * m_old / bc1
            m[sl] = sign * 2.0 ** -96 * f ** side * bc1 / (group.lr * beta1)
        else:
            m[sl] = sign * 2.0 ** 64 * f ** -side * bc1 / (group.lr * beta1)
    return m.astype(np.float32), v.astype(np.float32), g.astype(np.float32), kinds


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
def test_short_form_range_boundaries_against_oracle(fmt):
    """The update takes short forms of v / bc2, its square root and the last
    division only inside a range (v >= 2^-96, v / bc2 < 2^56, 2^-96 <=
    |lr * m_hat| < 2^64, 0 <= eps <= 2^28), and a wave with any element
    outside it takes the IEEE operations.  Tiles whose moments lie just
    inside (the short forms at their edges) or just outside (the IEEE path)
    each edge, groups with eps = 2^28 and one ulp above it, eps = 0, lr = 1
    and 2^-30, step counters at 0 (bc1 < 1) and far along (bc1 rounded to
    1), three calls in every launch mode: every value bit-exact against the
    oracle."""
    _need_gpu()
    sizes = [256 * 40, 256 * 40 - 77, 256 * 30, 256 * 30 + 5]
    pdt = [W.F32, W.BF16, W.F32, W.F32]
    gdt = [W.F32, W.F32, W.BF16, W.F32]
    group_of = [0, 1, 2, 3]
    groups = [W.Group(lr=1e-3, weight_decay=0.1),
              W.Group(lr=1.0, eps=2.0 ** 28),
              W.Group(lr=1e-3, eps=float(np.nextafter(np.float32(2.0 ** 28), np.float32(np.inf)))),
              W.Group(lr=2.0 ** -30, eps=0.0, weight_decay=0.01)]
    to_dev = lambda h, d: (torch.from_numpy(h.view(np.int32) if d == W.F32 else h.view(np.int16))
                           .to(DEV).view(torch.float32 if d == W.F32 else torch.bfloat16))
    for t0 in (0, 10_000):
        for mode in (1, 2, 3):
            say("case: short-form boundaries", fmt, "t0", t0, "mode", mode)
            rng = np.random.default_rng(1234 + t0 + mode)
            th0 = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
            th_ref = [x.copy() if d == W.F32 else oracle.f32_to_bf16(x) for x, d in zip(th0, pdt)]
            params = [to_dev(h, d) for h, d in zip(th_ref, pdt)]
            opt = GpuOpt(sizes, pdt, gdt, group_of, len(groups), fmt)
            L.apexw_set_launch_mode(opt.h, mode)
            ref = oracle.OracleAdamW(sizes, pdt, gdt, group_of, fmt)
            grads = []
            for i, n in enumerate(sizes):
                G = groups[group_of[i]]
                m, v, g, _ = _edge_state(n, rng, G, t0, G.beta1, G.beta2)
                grads.append(g)
                if fmt == W.STATE_F32:
                    ref.m[i][:], ref.v[i][:] = m, v
                elif fmt == W.STATE_BF16:
                    ref.m[i][:], ref.v[i][:] = oracle.f32_to_bf16(m), oracle.f32_to_bf16(v)
                else:
                    # codes near the top of the range, scales from the block maxima
                    nb = (n + 255) // 256
                    pad = nb * 256 - n
                    am = np.abs(np.pad(m, (0, pad))).reshape(nb, 256).max(1)
                    av = np.pad(v, (0, pad)).reshape(nb, 256).max(1)
                    ref.m_scale[i][:] = (am / 127).astype(np.float32)
                    ref.v_scale[i][:] = (av / 255).astype(np.float32)
                    ref.m[i][:] = (np.sign(m) * rng.integers(64, 128, n)).astype(np.int8)
                    ref.v[i][:] = rng.integers(128, 256, n).astype(np.uint8)
                    ms, vs = opt.scales(i)
                    ms.copy_(torch.from_numpy(ref.m_scale[i].copy()))
                    vs.copy_(torch.from_numpy(ref.v_scale[i].copy()))
                dm, dv = opt.moments(i)
                dm.copy_(torch.from_numpy(ref.m[i].copy()).view(dm.dtype))
                dv.copy_(torch.from_numpy(ref.v[i].copy()).view(dv.dtype))
            if t0:
                opt.steps().copy_(torch.full((len(sizes),), t0, dtype=torch.int32))
                ref.t[:len(sizes)] = t0
            g_host = [g if d == W.F32 else oracle.f32_to_bf16(g) for g, d in zip(grads, gdt)]
            g_dev = [to_dev(h, d) for h, d in zip(g_host, gdt)]
            for k in range(3):
                opt.step(groups, params, g_dev)
                ref.step(th_ref, g_host, groups)
            torch.cuda.synchronize()
            f32 = lambda a: a.view(np.float32)
            for i in range(len(sizes)):
                as_p = f32 if pdt[i] == W.F32 else oracle.bf16_to_f32
                _same_bits_or_both_nan("theta%d" % i, bits(params[i]), th_ref[i], as_p)
                m, v = (bits(t) for t in opt.moments(i))
                if fmt == W.STATE_Q8:
                    assert np.array_equal(m, ref.m[i]) and np.array_equal(v, ref.v[i]), i
                    ms, vs = (bits(t) for t in opt.scales(i))
                    assert np.array_equal(ms.view(np.uint32), ref.m_scale[i].view(np.uint32)), i
                    assert np.array_equal(vs.view(np.uint32), ref.v_scale[i].view(np.uint32)), i
                else:
                    as_s = f32 if fmt == W.STATE_F32 else oracle.bf16_to_f32
                    _same_bits_or_both_nan("m%d" % i, m, ref.m[i], as_s)
                    _same_bits_or_both_nan("v%d" % i, v, ref.v[i], as_s)
            assert np.array_equal(bits(opt.steps()), ref.t[:len(sizes)])
            opt.close()


@pytest.mark.parametrize("cap", [0, 5])
def test_q8_tile_pairs_against_oracle(cap):
    """The uncapped 8-bit carried step gives each workgroup the tiles 2w and
    2w+1: two full blocks of one tensor, a full block and the tensor's
    partial last block, or two tiles of two tensors (odd tile counts, one-tile
    and 5-element tensors), and the launch's last tile alone; with a workgroup
    cap the grid-stride kernel takes the same list.  Five calls with absent
    grads and a skipped call: codes, scales, theta and counters bit-exact
    against the oracle."""
    _need_gpu()
    say("case: 8-bit tile pairs, cap", cap)
    sizes = [256 * 3, 256 * 2 + 100, 256, 5, 256 * 7 + 1, 256 * 4, 256 * 5 - 3]
    pdt = [W.F32, W.BF16, W.F32, W.BF16, W.BF16, W.F32, W.F32]
    gdt = [W.F32, W.BF16, W.F32, W.BF16, W.BF16, W.F32, W.F32]
    group_of = [0, 1, 0, 1, 0, 1, 0]
    groups = [W.Group(lr=1e-3, weight_decay=0.1), W.Group(lr=5e-4, eps=1e-6)]
    to_dev = lambda h, d: (torch.from_numpy(h.view(np.int32) if d == W.F32 else h.view(np.int16))
                           .to(DEV).view(torch.float32 if d == W.F32 else torch.bfloat16))
    rng = np.random.default_rng(77 + cap)
    th_ref = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
    th_ref = [x if d == W.F32 else oracle.f32_to_bf16(x) for x, d in zip(th_ref, pdt)]
    params = [to_dev(h, d) for h, d in zip(th_ref, pdt)]
    opt = GpuOpt(sizes, pdt, gdt, group_of, len(groups), W.STATE_Q8)
    if cap:
        L.apexw_set_workgroups(opt.h, cap)
    ref = oracle.OracleAdamW(sizes, pdt, gdt, group_of, W.STATE_Q8)
    flag = torch.zeros(1, dtype=torch.float32, device=DEV)
    for k in range(5):
        g32 = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in sizes]
        g_host = [g if d == W.F32 else oracle.f32_to_bf16(g) for g, d in zip(g32, gdt)]
        absent = {1, 3} if k == 2 else set()
        skip = k == 3
        flag.fill_(1.0 if skip else 0.0)
        opt.step(groups, params, [None if i in absent else to_dev(h, d)
                                  for i, (h, d) in enumerate(zip(g_host, gdt))], found_inf=flag)
        ref.step(th_ref, [None if i in absent else h for i, h in enumerate(g_host)], groups,
                 found_inf=skip)
    torch.cuda.synchronize()
    for i in range(len(sizes)):
        assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, i
        m, v = (bits(t) for t in opt.moments(i))
        assert np.array_equal(m, ref.m[i]) and np.array_equal(v, ref.v[i]), i
        ms, vs = (bits(t) for t in opt.scales(i))
        assert np.array_equal(ms.view(np.uint32), ref.m_scale[i].view(np.uint32)), i
        assert np.array_equal(vs.view(np.uint32), ref.v_scale[i].view(np.uint32)), i
    assert np.array_equal(bits(opt.steps()), ref.t[:len(sizes)])
    opt.close()


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
def test_few_tensor_launches_against_oracle(fmt):
    """A carried launch of at most 8 tensors, none empty, finds each tile's
    tensor from first-tile bounds in the kernel arguments (the unused entries
    repeat the last tensor); a larger launch reads the tile table.  Lists of
    1, 2, 7, 8 and 9 tensors of one dtype pair, and a mixed list whose
    fp32/fp32 launch holds 8 tensors and whose bf16/bf16 launch holds 9, in
    interleaved order; ragged sizes (1, 255, 256, 257 elements, several
    tiles); four calls with an absent grad and a skipped call: every value
    bit-exact against the oracle."""
    _need_gpu()
    pool = [257, 1, 256 * 3 + 7, 256, 255, 513, 3, 256 * 5, 1000]
    lists = [[(pool[j], W.F32, W.F32) for j in range(n)] for n in (1, 2, 7, 8, 9)]
    mixed = []
    for j in range(9):
        if j < 8:
            mixed.append((pool[j], W.F32, W.F32))
        mixed.append((pool[8 - j] + 11, W.BF16, W.BF16))
    lists.append(mixed)
    groups = [W.Group(lr=1e-3, weight_decay=0.1), W.Group(lr=5e-4, eps=1e-6)]
    to_dev = lambda h, d: (torch.from_numpy(h.view(np.int32) if d == W.F32 else h.view(np.int16))
                           .to(DEV).view(torch.float32 if d == W.F32 else torch.bfloat16))
    f32 = lambda a: a.view(np.float32)
    for li, spec in enumerate(lists):
        sizes = [s for s, _, _ in spec]
        pdt = [p for _, p, _ in spec]
        gdt = [g for _, _, g in spec]
        group_of = [i % 2 for i in range(len(spec))]
        say("case: few-tensor launches", fmt, "list", li, "tensors", len(spec))
        rng = np.random.default_rng(4242 + li)
        th_ref = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
        th_ref = [x if d == W.F32 else oracle.f32_to_bf16(x) for x, d in zip(th_ref, pdt)]
        params = [to_dev(h, d) for h, d in zip(th_ref, pdt)]
        opt = GpuOpt(sizes, pdt, gdt, group_of, len(groups), fmt)
        L.apexw_set_launch_mode(opt.h, 3)
        ref = oracle.OracleAdamW(sizes, pdt, gdt, group_of, fmt)
        flag = torch.zeros(1, dtype=torch.float32, device=DEV)
        for k in range(4):
            g32 = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in sizes]
            g_host = [g if d == W.F32 else oracle.f32_to_bf16(g) for g, d in zip(g32, gdt)]
            absent = {len(spec) - 1} if k == 1 else set()
            skip = k == 2
            flag.fill_(1.0 if skip else 0.0)
            opt.step(groups, params, [None if i in absent else to_dev(h, d)
                                      for i, (h, d) in enumerate(zip(g_host, gdt))], found_inf=flag)
            ref.step(th_ref, [None if i in absent else h for i, h in enumerate(g_host)], groups,
                     found_inf=skip)
        torch.cuda.synchronize()
        for i in range(len(sizes)):
            assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, (li, i)
            m, v = (bits(t) for t in opt.moments(i))
            if fmt == W.STATE_Q8:
                assert np.array_equal(m, ref.m[i]) and np.array_equal(v, ref.v[i]), (li, i)
                ms, vs = (bits(t) for t in opt.scales(i))
                assert np.array_equal(ms.view(np.uint32), ref.m_scale[i].view(np.uint32)), (li, i)
                assert np.array_equal(vs.view(np.uint32), ref.v_scale[i].view(np.uint32)), (li, i)
            else:
                as_s = f32 if fmt == W.STATE_F32 else oracle.bf16_to_f32
                _same_bits_or_both_nan("m%d" % i, m, ref.m[i], as_s)
                _same_bits_or_both_nan("v%d" % i, v, ref.v[i], as_s)
        assert np.array_equal(bits(opt.steps()), ref.t[:len(sizes)])
        opt.close()


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
def test_empty_list_and_lists_of_empty_tensors(fmt):
    """Degenerate lists: no tensor at all (every call succeeds and does
    nothing; the grad norm is 0 and the clip coefficient the oracle's; a
    checkpoint round-trips), and only empty tensors, with an absent grad and
    a skipped call: the step counters advance exactly as the oracle's (a
    present grad of no elements is a grad).  Such a list takes mode 1; modes
    2 and 3 are refused for it with APEXW_EINVAL, as documented, and the
    handle keeps its mode."""
    _need_gpu()
    groups = [W.Group(lr=1e-3, weight_decay=0.1)]
    gr = L.make_groups(groups)
    flag = torch.zeros(1, dtype=torch.float32, device=DEV)
    say("case: empty list", fmt)
    opt = GpuOpt([], [], [], [], 1, fmt)
    for _ in range(2):
        opt.step(groups, [], [], found_inf=flag)
    norm = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
    coef = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
    L.apexw_clip_grad_norm(opt.h, L.make_ptrs([]), 0, 1.0, 0, norm.data_ptr(), coef.data_ptr(),
                           opt.stream)
    L.apexw_unscale_check(opt.h, L.make_ptrs([]), 0, flag.data_ptr(), opt.stream)
    blob = L.apexw_export_state(opt.h, gr, 1, opt.stream)
    L.apexw_import_state(opt.h, blob, 1, opt.stream)
    torch.cuda.synchronize()
    assert norm.item() == 0.0 and flag.item() == 0.0
    assert coef.item() == oracle.OracleAdamW.clip_coef(0.0, 1.0)
    opt.close()
    for mode in (0, 1, 2, 3):
        say("case: only empty tensors", fmt, "mode", mode)
        sizes = [0, 0, 0]
        pdt, gdt = [W.F32, W.BF16, W.F32], [W.F32, W.BF16, W.BF16]
        opt = GpuOpt(sizes, pdt, gdt, [0, 0, 0], 1, fmt)
        if mode in (2, 3):
            with pytest.raises(L.ApexwError) as err:
                L.apexw_set_launch_mode(opt.h, mode)
            assert err.value.code == L.APEXW_EINVAL
        else:
            L.apexw_set_launch_mode(opt.h, mode)
        assert L.apexw_get_launch_mode(opt.h) == 1
        ref = oracle.OracleAdamW(sizes, pdt, gdt, [0, 0, 0], fmt)
        params = [torch.empty(0, device=DEV, dtype=torch.float32 if d == W.F32 else torch.bfloat16)
                  for d in pdt]
        th_ref = [np.zeros(0, np.float32) if d == W.F32 else np.zeros(0, np.uint16) for d in pdt]
        for k in range(5):
            absent = {1} if k == 1 else set()
            skip = k == 3
            flag.fill_(1.0 if skip else 0.0)
            g_dev = [None if i in absent else
                     torch.empty(0, device=DEV, dtype=torch.float32 if d == W.F32 else torch.bfloat16)
                     for i, d in enumerate(gdt)]
            g_host = [None if i in absent else
                      (np.zeros(0, np.float32) if d == W.F32 else np.zeros(0, np.uint16))
                      for i, d in enumerate(gdt)]
            opt.step(groups, params, g_dev, found_inf=flag)
            ref.step(th_ref, g_host, groups, found_inf=skip)
        torch.cuda.synchronize()
        assert np.array_equal(bits(opt.steps()), ref.t[:3]), (bits(opt.steps()), ref.t[:3])
        assert list(bits(opt.steps())) == [4, 3, 4]
        opt.close()


def test_refused_calls_write_nothing():
    """Every refused call (wrong group count, out-of-range hyperparameters,
    a NULL parameter pointer, out-of-range knobs) returns APEXW_EINVAL and
    leaves parameters, state and counters bit for bit as they were; the
    handle then steps on exactly as the oracle does."""
    _need_gpu()
    say("case: refused calls")
    sizes = [1000, 257, 4096]
    pdt, gdt = [W.F32, W.BF16, W.F32], [W.F32, W.F32, W.BF16]
    group_of = [0, 0, 0]
    good = [W.Group(lr=1e-3, weight_decay=0.1)]
    to_dev = lambda h, d: (torch.from_numpy(h.view(np.int32) if d == W.F32 else h.view(np.int16))
                           .to(DEV).view(torch.float32 if d == W.F32 else torch.bfloat16))
    rng = np.random.default_rng(5150)
    th_ref = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
    th_ref = [x if d == W.F32 else oracle.f32_to_bf16(x) for x, d in zip(th_ref, pdt)]
    params = [to_dev(h, d) for h, d in zip(th_ref, pdt)]
    opt = GpuOpt(sizes, pdt, gdt, group_of, 1, W.STATE_F32)
    ref = oracle.OracleAdamW(sizes, pdt, gdt, group_of, W.STATE_F32)

    def grads():
        g32 = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in sizes]
        g_host = [g if d == W.F32 else oracle.f32_to_bf16(g) for g, d in zip(g32, gdt)]
        return g_host, [to_dev(h, d) for h, d in zip(g_host, gdt)]

    g_host, g_dev = grads()
    opt.step(good, params, g_dev)
    ref.step(th_ref, g_host, good)
    torch.cuda.synchronize()
    before = [p.clone() for p in params], opt.state.clone()
    pa = L.make_ptrs([p.data_ptr() for p in params])
    ga = L.make_ptrs([g.data_ptr() for g in g_dev])
    bad_groups = [W.Group(lr=-1e-3), W.Group(lr=float("nan")), W.Group(lr=1e-3, eps=-1e-8),
                  W.Group(lr=1e-3, eps=float("inf")), W.Group(lr=1e-3, weight_decay=-0.1),
                  W.Group(lr=1e-3, beta1=1.0), W.Group(lr=1e-3, beta2=-0.5),
                  W.Group(lr=1e-3, beta1=float("nan"))]
    for g in bad_groups:
        with pytest.raises(L.ApexwError) as e:
            L.apexw_step(opt.h, L.make_groups([g]), 1, pa, ga, 0, opt.stream)
        assert e.value.code == L.APEXW_EINVAL, g
    with pytest.raises(L.ApexwError) as e:       # the handle was built for one group
        L.apexw_step(opt.h, L.make_groups(good * 2), 2, pa, ga, 0, opt.stream)
    assert e.value.code == L.APEXW_EINVAL
    with pytest.raises(L.ApexwError) as e:       # NULL pointer for a non-empty tensor
        L.apexw_step(opt.h, L.make_groups(good), 1,
                     L.make_ptrs([params[0].data_ptr(), 0, params[2].data_ptr()]), ga, 0,
                     opt.stream)
    assert e.value.code == L.APEXW_EINVAL
    for fn, arg in ((L.apexw_set_workgroups, -1), (L.apexw_set_occupancy, -2),
                    (L.apexw_set_cache_policy, 3), (L.apexw_set_launch_mode, 4)):
        with pytest.raises(L.ApexwError) as e:
            fn(opt.h, arg)
        assert e.value.code == L.APEXW_EINVAL, fn.__name__
    torch.cuda.synchronize()
    for p, q in zip(params, before[0]):
        assert torch.equal(p.view(torch.int16 if p.dtype == torch.bfloat16 else torch.int32),
                           q.view(torch.int16 if q.dtype == torch.bfloat16 else torch.int32))
    assert torch.equal(opt.state, before[1])
    g_host, g_dev = grads()
    opt.step(good, params, g_dev)
    ref.step(th_ref, g_host, good)
    torch.cuda.synchronize()
    for i in range(len(sizes)):
        assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, i
        m, v = (bits(t) for t in opt.moments(i))
        assert n_bit_mismatch(m, ref.m[i]) == 0 and n_bit_mismatch(v, ref.v[i]) == 0, i
    assert np.array_equal(bits(opt.steps()), ref.t[:len(sizes)])
    opt.close()


def test_two_threads_two_handles_on_two_streams():
    """The C ABI is thread-safe on distinct handles: two host threads step
    their own handles on their own streams at the same time (ctypes releases
    the interpreter lock for every call), twenty steps each, one of them
    with a failing call in between (its error stays on its thread); both
    end bit for bit at the oracle's results."""
    _need_gpu()
    import threading
    say("case: two threads, two handles")
    specs = [([5000, 300, 4096], [W.F32, W.BF16, W.F32], [W.F32, W.F32, W.BF16], W.STATE_F32),
             ([70000, 1], [W.BF16, W.BF16], [W.BF16, W.F32], W.STATE_Q8)]
    groups = [W.Group(lr=1e-3, weight_decay=0.1)]
    to_dev = lambda h, d: (torch.from_numpy(h.view(np.int32) if d == W.F32 else h.view(np.int16))
                           .to(DEV).view(torch.float32 if d == W.F32 else torch.bfloat16))
    jobs = []
    for t, (sizes, pdt, gdt, fmt) in enumerate(specs):
        rng = np.random.default_rng(600 + t)
        th0 = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
        th0 = [x if d == W.F32 else oracle.f32_to_bf16(x) for x, d in zip(th0, pdt)]
        gs = [[(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in sizes] for _ in range(20)]
        gs = [[x if d == W.F32 else oracle.f32_to_bf16(x) for x, d in zip(step, gdt)] for step in gs]
        params = [to_dev(h, d) for h, d in zip(th0, pdt)]
        grads = [[to_dev(h, d) for h, d in zip(step, gdt)] for step in gs]
        opt = GpuOpt(sizes, pdt, gdt, [0] * len(sizes), 1, fmt)
        jobs.append(dict(sizes=sizes, pdt=pdt, gdt=gdt, fmt=fmt, th0=th0, gs=gs, params=params,
                         grads=grads, opt=opt, stream=torch.cuda.Stream(), errors=[]))
    torch.cuda.synchronize()
    gr = L.make_groups(groups)

    def run(job, t):
        try:
            pa = L.make_ptrs([p.data_ptr() for p in job["params"]])
            s = job["stream"].cuda_stream
            for k in range(20):
                if t == 1 and k == 10:
                    try:                              # wrong group count: refused, this thread's error
                        L.apexw_step(job["opt"].h, gr, 2, pa, pa, 0, s)
                    except L.ApexwError:
                        job["errors"].append(L.apexw_last_error())
                ga = L.make_ptrs([g.data_ptr() for g in job["grads"][k]])
                L.apexw_step(job["opt"].h, gr, 1, pa, ga, 0, s)
        except Exception as e:                        # reported by the main thread
            job["errors"].append(repr(e))

    threads = [threading.Thread(target=run, args=(j, t)) for t, j in enumerate(jobs)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert jobs[0]["errors"] == [] and len(jobs[1]["errors"]) == 1, [j["errors"] for j in jobs]
    assert "group" in jobs[1]["errors"][0]
    for job in jobs:
        ref = oracle.OracleAdamW(job["sizes"], job["pdt"], job["gdt"], [0] * len(job["sizes"]),
                                 job["fmt"])
        th = [x.copy() for x in job["th0"]]
        for k in range(20):
            ref.step(th, job["gs"][k], groups)
        for i in range(len(job["sizes"])):
            assert n_bit_mismatch(bits(job["params"][i]), th[i]) == 0, (job["fmt"], i)
        assert np.array_equal(bits(job["opt"].steps()), ref.t[:len(job["sizes"])])
        job["opt"].close()
