"""GPU parity of global grad-norm clipping through the C ABI: the norm and
clip coefficient produced on the device, and the clipped AMP loop."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import GpuOpt, bits, n_bit_mismatch, norm_rel_bound, say, stable_max_norm
from tensor_adamw_optimizer_amd import _lib as L

pytestmark = pytest.mark.gpu
DEV = "cuda"

SIZES = [1, 255, 257, 4097, 70000, 0, 3]
PDT = [W.F32, W.BF16, W.F32, W.BF16, W.BF16, W.F32, W.F32]
GDT = [W.F32, W.F32, W.BF16, W.BF16, W.F32, W.F32, W.BF16]


def _ptrs(ts):
    return L.make_ptrs([0 if t is None else (t.data_ptr() or 16) for t in ts])


@pytest.mark.parametrize("inv", [1.0, 1.0 / 4096.0])
def test_norm_and_coefficient_match_oracle(inv):
    say("case: grad norm, inv", inv)
    n = len(SIZES)
    opt = GpuOpt(SIZES, PDT, GDT, [0] * n, 1, W.STATE_F32)
    ref = oracle.OracleAdamW(SIZES, PDT, GDT, [0] * n, "f32")
    gen = torch.Generator().manual_seed(41)
    inv_t = torch.tensor([inv], device=DEV)
    norm = torch.zeros(1, dtype=torch.float64, device=DEV)
    coef = torch.zeros(1, device=DEV)
    fi = torch.zeros(1, device=DEV)
    for trial in range(12):
        scale = float(np.exp(trial - 6))
        g_cpu = [(torch.randn(s, generator=gen) * scale / inv).to(W.TORCH_DTYPE[d]) for s, d in zip(SIZES, GDT)]
        absent = [(i + trial) % 5 == 0 for i in range(n)]
        g_dev = [None if a else g.to(DEV) for g, a in zip(g_cpu, absent)]
        g_np = [None if a else bits(g) for g, a in zip(g_cpu, absent)]
        want = ref.grad_norm(g_np, inv)
        rel = norm_rel_bound(g_np)
        max_norm = stable_max_norm(ref, want, rel, 1.0)
        fi.zero_()
        L.apexw_clip_grad_norm(opt.h, _ptrs(g_dev), inv_t.data_ptr(), max_norm, fi.data_ptr(),
                               norm.data_ptr(), coef.data_ptr(), opt.stream)
        torch.cuda.synchronize()
        assert abs(norm.item() - want) <= rel * want, (trial, norm.item(), want)
        assert coef.item() == ref.clip_coef(want, max_norm), trial
        assert fi.item() == 0.0
    # a NaN anywhere: the check inside the norm pass reports it
    g_dev = [torch.zeros(s, dtype=W.TORCH_DTYPE[d], device=DEV) for s, d in zip(SIZES, GDT)]
    g_dev[4][999] = float("nan")
    L.apexw_clip_grad_norm(opt.h, _ptrs(g_dev), 0, 1.0, fi.data_ptr(), 0, coef.data_ptr(), opt.stream)
    torch.cuda.synchronize()
    assert fi.item() == 1.0
    opt.close()


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
def test_clipped_amp_loop_matches_oracle(fmt):
    """zero found_inf -> clip_grad_norm (with the finite check) -> step_ex
    with inv_scale and clip_coef, 8 calls, the norm above and below
    max_norm, one overflow; everything on the device."""
    say("case: clipped amp loop", fmt)
    n = len(SIZES)
    groups = [W.Group(lr=1e-3, weight_decay=0.1)]
    gen = torch.Generator().manual_seed(42)
    p_cpu = [(torch.randn(s, generator=gen) * 0.02).to(W.TORCH_DTYPE[d]) for s, d in zip(SIZES, PDT)]
    params = [p.to(DEV) for p in p_cpu]
    opt = GpuOpt(SIZES, PDT, GDT, [0] * n, 1, fmt)
    ref = oracle.OracleAdamW(SIZES, PDT, GDT, [0] * n, fmt)
    th_ref = [bits(p) for p in p_cpu]
    fi = torch.zeros(1, device=DEV)
    coef = torch.zeros(1, device=DEV)
    inv = 1.0 / 1024.0
    inv_t = torch.tensor([inv], device=DEV)
    pa = _ptrs(params)
    ga = L.make_groups(groups)
    max_norm = 0.05
    coefs = []
    for k in range(1, 9):
        mag = 1e-4 if k % 2 else 1e-3
        g_cpu = [(torch.randn(s, generator=gen) * mag * 1024.0).to(W.TORCH_DTYPE[d])
                 for s, d in zip(SIZES, GDT)]
        if k == 5:
            g_cpu[2][3] = float("inf")
        g_dev = [g.to(DEV) for g in g_cpu]
        g_np = [bits(g) for g in g_cpu]
        found = ref.unscale_check(g_np, inv)
        want = ref.grad_norm(g_np, inv)
        mn = max_norm if found else stable_max_norm(ref, want, norm_rel_bound(g_np), max_norm)
        fi.zero_()
        L.apexw_clip_grad_norm(opt.h, _ptrs(g_dev), inv_t.data_ptr(), mn, fi.data_ptr(), 0,
                               coef.data_ptr(), opt.stream)
        L.apexw_step_ex(opt.h, ga, 1, pa, _ptrs(g_dev), inv_scale_ptr=inv_t.data_ptr(),
                        clip_coef_ptr=coef.data_ptr(), found_inf_ptr=fi.data_ptr(), stream=opt.stream)
        c = ref.clip_coef(want, mn)
        torch.cuda.synchronize()
        assert coef.item() == c or found, k
        coefs.append(c)
        ref.step(th_ref, g_np, groups, found_inf=found, inv_scale=inv, clip_coef=c)
    assert any(c < 1.0 for c in coefs) and any(c == 1.0 for c in coefs)
    assert np.array_equal(bits(opt.steps()), ref.t) and list(ref.t)[0] == 7
    for i in range(n):
        assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, i
        m, v = opt.moments(i)
        assert n_bit_mismatch(bits(m), ref.m[i]) == 0 and n_bit_mismatch(bits(v), ref.v[i]) == 0, i
        if fmt == W.STATE_Q8:
            ms, vs = opt.scales(i)
            assert n_bit_mismatch(bits(ms), ref.m_scale[i]) == 0, i
    opt.close()


def test_norm_deterministic_at_full_size():
    """Few-large grads (537M elements): the norm is the same on every call
    (fixed reduction order) and agrees with the oracle on the full list."""
    say("case: few_large norm")
    w = W.few_large()
    opt = GpuOpt(w.numels, w.param_dtype, w.grad_dtype, w.group_of, 1, w.state_fmt)
    g = W.grads_for_call(w, 1, DEV)
    norm = torch.zeros(1, dtype=torch.float64, device=DEV)
    coef = torch.zeros(1, device=DEV)
    seen = set()
    for _ in range(3):
        L.apexw_clip_grad_norm(opt.h, _ptrs(g), 0, 1.0, 0, norm.data_ptr(), coef.data_ptr(), opt.stream)
        torch.cuda.synchronize()
        seen.add(norm.item())
    assert len(seen) == 1
    ref = oracle.OracleAdamW(w.numels, w.param_dtype, w.grad_dtype, w.group_of, "f32")
    g_np = [bits(x) for x in g]
    want = ref.grad_norm(g_np, 1.0)
    # the oracle's running fp64 sum over 537M terms is itself only good to
    # about n*u (its rigorous bound); numpy's pairwise sum of the same fp64
    # squares is good to about log2(n)*u and pins the device result tightly
    assert abs(norm.item() - want) <= 0.5 * len(g_np) * w.numels[0] * 2.0 ** -53 * want
    pairwise = np.sqrt(sum(float(np.sum(x.astype(np.float64) ** 2)) for x in g_np))
    assert abs(norm.item() - pairwise) <= 1e-13 * pairwise
    assert coef.item() == ref.clip_coef(want, 1.0)
    opt.close()
