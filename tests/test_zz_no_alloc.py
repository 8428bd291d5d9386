"""apexw_clip_grad_norm_noalloc -- the grad-norm pass whose partial sums live
in the library's static device array -- against apexw_clip_grad_norm, through
the C ABI: norm, clip coefficient and overflow flag bit for bit, on two calls
in a row (a list that takes the two-stage reduction, then a smaller one that
sums its partials directly), and a list too large for the array refused
before anything is queued."""
import numpy as np
import pytest
import torch

import workloads as W
from gpu_helpers import GpuOpt, say
from tensor_adamw_optimizer_amd import _lib as L

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _grads(sizes, dts, seed, inf_at=None):
    gen = torch.Generator().manual_seed(seed)
    gs = [(torch.randn(n, generator=gen) * 1e-3).to(W.TORCH_DTYPE[d]).to(DEV)
          for n, d in zip(sizes, dts)]
    if inf_at is not None:
        gs[inf_at[0]][inf_at[1]] = float("inf")
    return gs


def _both(opt, gs, inv_scale, max_norm, absent=()):
    st = torch.cuda.current_stream().cuda_stream
    ga = L.make_ptrs([0 if i in absent else g.data_ptr() for i, g in enumerate(gs)])
    inv = torch.tensor([inv_scale], dtype=torch.float32, device=DEV)
    out = []
    for fn in (L.apexw_clip_grad_norm, L.apexw_clip_grad_norm_noalloc):
        fi = torch.zeros(1, device=DEV)
        norm = torch.full((1,), -1.0, dtype=torch.float64, device=DEV)
        coef = torch.full((1,), -1.0, dtype=torch.float32, device=DEV)
        fn(opt.h, ga, inv.data_ptr(), max_norm, fi.data_ptr(), norm.data_ptr(), coef.data_ptr(), st)
        torch.cuda.synchronize()
        out.append((norm.cpu().numpy().view(np.uint64)[0], coef.cpu().numpy().view(np.uint32)[0],
                    fi.item()))
    return out


def test_noalloc_norm_equals_workspace_norm_on_two_calls():
    # first call: about 36,500 tiles in two dtype pairs, more than 8192 read
    # groups, so the partials are reduced in two stages
    big = [3_000_000, 5_000_001, 1_234_567, 77]
    big_dt = [W.F32, W.BF16, W.F32, W.BF16]
    say("case: noalloc norm, large list", big)
    a = GpuOpt(big, [W.F32] * 4, big_dt, [0] * 4, 1, W.STATE_F32)
    gs = _grads(big, big_dt, 81)
    for inv_scale, max_norm, absent in ((1.0, 1.0, ()), (0.25, 1e-2, (1,)), (1.0, 1e9, ())):
        (n1, c1, f1), (n2, c2, f2) = _both(a, gs, inv_scale, max_norm, absent)
        assert n1 == n2 and c1 == c2 and f1 == f2 == 0.0, (inv_scale, max_norm)
        assert np.uint64(n1).view(np.float64) > 0
    gs_inf = _grads(big, big_dt, 82, inf_at=(2, 1_000_000))
    (n1, c1, f1), (n2, c2, f2) = _both(a, gs_inf, 1.0, 1.0)
    assert f1 == f2 == 1.0 and n1 == n2 and c1 == c2
    a.close()
    # second call, smaller: a few tiles, the partials summed directly; the
    # array still holds the first call's partials, which must not leak in
    small = [1000, 4097, 3]
    say("case: noalloc norm, small list", small)
    b = GpuOpt(small, [W.BF16, W.F32, W.F32], [W.BF16, W.F32, W.BF16], [0, 0, 0], 1, W.STATE_Q8)
    gs = _grads(small, [W.BF16, W.F32, W.BF16], 83)
    (n1, c1, f1), (n2, c2, f2) = _both(b, gs, 1.0, 1e-3)
    assert n1 == n2 and c1 == c2 and f1 == f2 == 0.0
    g64 = np.concatenate([g.float().cpu().numpy().astype(np.float64) for g in gs])
    assert abs(np.uint64(n2).view(np.float64) - np.sqrt(np.sum(g64 * g64))) <= \
        1e-12 * np.sqrt(np.sum(g64 * g64))
    b.close()


def test_noalloc_refuses_a_list_beyond_its_array():
    # 4.3 million tiles need more than 1,048,320 read groups: refused before
    # any work is queued (the grads are all absent: nothing would be read)
    n = 1_100_000_000
    say("case: noalloc norm refused, numel", n)
    opt = GpuOpt([n], [W.BF16], [W.BF16], [0], 1, W.STATE_Q8)
    coef = torch.zeros(1, device=DEV)
    with pytest.raises(L.ApexwError) as e:
        L.apexw_clip_grad_norm_noalloc(opt.h, L.make_ptrs([0]), 0, 1.0, 0, 0, coef.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream)
    assert e.value.code == L.APEXW_ENOSPC
    assert "static scratch" in str(e.value)
    opt.close()
    torch.cuda.empty_cache()
