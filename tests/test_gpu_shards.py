"""One GPU's share of a sharded (ZeRO-1 style) step, on one GPU: every
tensor split into N contiguous slices at 256-element boundaries, each of the
N shards stepped by its own handle over views of its slices (its own state,
counters and workspace).  Put together, the shards equal the oracle's
unsharded step bit for bit: the update is elementwise, and a slice that
starts on a 256-element boundary of its tensor has the same 8-bit blocks as
the whole tensor.  (The collectives around such a step -- grad
reduce-scatter, parameter all-gather, found_inf agreement -- need more than
one GPU and are not exercised.)"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import GpuOpt, bits, n_bit_mismatch, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def slice_bounds(n, ranks):
    """Rank r owns elements [b[r], b[r+1]) of a tensor of n elements; every
    bound but the last is a multiple of 256."""
    per = -(-n // ranks)
    per = -(-per // 256) * 256
    return [min(r * per, n) for r in range(ranks)] + [n]


@pytest.mark.parametrize("fmt", [W.STATE_F32, W.STATE_BF16, W.STATE_Q8])
def test_shards_of_a_list_equal_the_unsharded_step(fmt):
    say("case: shards", fmt)
    ranks = 4
    sizes = [70001, 3000, 256 * 37 + 5, 1000, 513, 8192]
    pdt = [W.BF16, W.F32, W.BF16, W.F32, W.F32, W.BF16]
    gdt = [W.F32, W.F32, W.BF16, W.BF16, W.F32, W.F32]
    group_of = [0, 1, 0, 1, 0, 1]
    groups = [W.Group(lr=1e-3, weight_decay=0.1), W.Group(lr=4e-3, beta1=0.8, beta2=0.99)]
    gen = torch.Generator().manual_seed(77)
    p_cpu = [(torch.randn(n, generator=gen) * 0.02).to(W.TORCH_DTYPE[d]) for n, d in zip(sizes, pdt)]
    params = [p.to(DEV) for p in p_cpu]
    bounds = [slice_bounds(n, ranks) for n in sizes]
    shards = []                                   # (opt, [(tensor, lo, hi)])
    for r in range(ranks):
        parts = [(i, b[r], b[r + 1]) for i, b in enumerate(bounds) if b[r + 1] > b[r]]
        opt = GpuOpt([hi - lo for _, lo, hi in parts], [pdt[i] for i, _, _ in parts],
                     [gdt[i] for i, _, _ in parts], [group_of[i] for i, _, _ in parts],
                     len(groups), fmt)
        shards.append((opt, parts))
    assert sum(len(parts) for _, parts in shards) > len(sizes)   # tensors really are split
    ref = oracle.OracleAdamW(sizes, pdt, gdt, group_of, fmt)
    th_ref = [bits(p) for p in p_cpu]
    fi = torch.zeros(1, device=DEV)
    for k in range(1, 7):
        g_cpu = [(torch.randn(n, generator=gen) * 1e-3).to(W.TORCH_DTYPE[d]) for n, d in zip(sizes, gdt)]
        present = [(i + k) % 4 != 0 for i in range(len(sizes))]
        g_dev = [g.to(DEV) if ok else None for g, ok in zip(g_cpu, present)]
        skip = k == 3
        fi.fill_(1.0 if skip else 0.0)
        for opt, parts in shards:
            opt.step(groups, [params[i][lo:hi] for i, lo, hi in parts],
                     [None if g_dev[i] is None else g_dev[i][lo:hi] for i, lo, hi in parts],
                     found_inf=fi)
        ref.step(th_ref, [bits(g) if ok else None for g, ok in zip(g_cpu, present)], groups,
                 found_inf=skip)
    torch.cuda.synchronize()
    for i in range(len(sizes)):
        assert n_bit_mismatch(bits(params[i]), th_ref[i]) == 0, i
    for opt, parts in shards:
        got_t = bits(opt.steps())
        for j, (i, lo, hi) in enumerate(parts):
            assert got_t[j] == ref.t[i], (i, lo)
            m, v = opt.moments(j)
            assert n_bit_mismatch(bits(m), ref.m[i][lo:hi]) == 0, (i, lo)
            assert n_bit_mismatch(bits(v), ref.v[i][lo:hi]) == 0, (i, lo)
            if fmt == W.STATE_Q8:
                ms, vs = opt.scales(j)
                assert n_bit_mismatch(bits(ms), ref.m_scale[i][lo // 256:-(-hi // 256)]) == 0, (i, lo)
                assert n_bit_mismatch(bits(vs), ref.v_scale[i][lo // 256:-(-hi // 256)]) == 0, (i, lo)
        opt.close()
