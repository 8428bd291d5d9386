"""Randomised runs of the torch wrapper against the oracle: random parameter
shapes and dtypes over one to three parameter groups, a random state format,
grad dtype and grad handling (per-parameter .grad, some absent, or flat
grads), learning rates changed between steps as a schedule would, and on
some runs a checkpoint through state_dict / torch.save / load_state_dict
into a fresh optimizer halfway.  Parameters, moments and step counters bit
for bit against the oracle after every step (NaNs compared as NaNs).
APEXW_WRAPPER_FUZZ_SEEDS asks for more runs than the default 12."""
import io
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import bits, n_bit_mismatch_nan_equal, say
from tensor_adamw_optimizer_amd import AdamW

pytestmark = pytest.mark.gpu
DEV = "cuda"
N_SEEDS = int(os.environ.get("APEXW_WRAPPER_FUZZ_SEEDS", "12"))
NAME = {torch.float32: W.F32, torch.bfloat16: W.BF16}


def _shape(rng):
    numel = int(np.exp(rng.uniform(0, np.log(6000))))
    dims = int(rng.integers(1, 4))
    if dims == 1:
        return (numel,)
    a = int(rng.integers(1, 65))
    if dims == 2:
        return (a, max(1, numel // a))
    b = int(rng.integers(1, 9))
    return (a, b, max(1, numel // (a * b)))


@pytest.mark.parametrize("seed", range(N_SEEDS))
def test_random_wrapper_run_against_oracle(seed):
    rng = np.random.default_rng(7000 + seed)
    gen = torch.Generator().manual_seed(8000 + seed)
    n = int(rng.integers(1, 12))
    shapes = [_shape(rng) for _ in range(n)]
    pdt = [torch.float32 if rng.random() < 0.5 else torch.bfloat16 for _ in range(n)]
    state = str(rng.choice(["f32", "bf16", "q8"]))
    flat = bool(rng.random() < 0.4)
    grad_dtype = [None, torch.float32, torch.bfloat16][int(rng.integers(0, 3))]
    n_groups = int(rng.integers(1, min(3, n) + 1))
    member = [i % n_groups for i in range(n)]
    rng.shuffle(member)
    hyper = [dict(lr=float(10 ** rng.uniform(-4, -2)),
                  betas=(float(rng.choice([0.0, 0.9, 0.95])), float(rng.choice([0.99, 0.999]))),
                  eps=float(rng.choice([1e-8, 1e-6])),
                  weight_decay=float(rng.choice([0.0, 0.01, 0.1]))) for _ in range(n_groups)]
    say("case: wrapper fuzz", seed, "n", n, "state", state, "flat", flat, "grad_dtype", grad_dtype,
        "groups", n_groups)
    p_cpu = [(torch.randn(s, generator=gen) * 0.02).to(d) for s, d in zip(shapes, pdt)]
    params = [torch.nn.Parameter(p.to(DEV)) for p in p_cpu]
    groups = [dict(params=[params[i] for i in range(n) if member[i] == g], **hyper[g])
              for g in range(n_groups)]
    order = [i for g in range(n_groups) for i in range(n) if member[i] == g]   # the wrapper's list

    def build():
        return AdamW(groups, state=state, grad_dtype=grad_dtype, flat_grads=flat)

    opt = build()
    gdt = [grad_dtype or pdt[i] for i in order]
    ref = oracle.OracleAdamW([params[i].numel() for i in order], [NAME[pdt[i]] for i in order],
                             [NAME[d] for d in gdt], [member[i] for i in order], state)
    th_ref = [bits(p_cpu[i].reshape(-1)) for i in order]
    checkpoint_at = int(rng.integers(1, 5)) if rng.random() < 0.5 else -1
    for k in range(6):
        if k == checkpoint_at:
            buf = io.BytesIO()
            torch.save(opt.state_dict(), buf)
            opt.close()
            opt = build()                             # a fresh optimizer, then the checkpoint
            buf.seek(0)
            opt.load_state_dict(torch.load(buf, weights_only=True))
        for g in opt.param_groups:                    # a schedule's change between steps
            if rng.random() < 0.3:
                g["lr"] = g["lr"] * 0.5
        g_np = []
        for j, i in enumerate(order):
            present = flat or rng.random() < 0.85
            g_cpu = (torch.randn(shapes[i], generator=gen) * 1e-3).to(gdt[j])
            if flat:
                params[i].grad.copy_(g_cpu.to(DEV))
            else:                                     # the optimizer set grad_dtype if it differs
                params[i].grad = g_cpu.to(DEV) if present else None
            g_np.append(bits(g_cpu.reshape(-1)) if present else None)
        grp = [W.Group(lr=float(g["lr"]), beta1=float(g["betas"][0]), beta2=float(g["betas"][1]),
                       eps=float(g["eps"]), weight_decay=float(g["weight_decay"]))
               for g in opt.param_groups]
        opt.step()
        ref.step(th_ref, g_np, grp)
        torch.cuda.synchronize()
        for j, i in enumerate(order):
            assert n_bit_mismatch_nan_equal(bits(params[i].detach().reshape(-1)), th_ref[j]) == 0, \
                (seed, k, i)
    for j in range(n):
        m, v = opt.moments(j)
        assert n_bit_mismatch_nan_equal(bits(m), ref.m[j]) == 0, (seed, j)
        assert n_bit_mismatch_nan_equal(bits(v), ref.v[j]) == 0, (seed, j)
    assert list(opt.read_steps()) == list(ref.t[:n])
    opt.close()
