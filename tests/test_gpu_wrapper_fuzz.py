"""Randomised runs of the torch wrapper against the oracle: random parameter
shapes and dtypes over one to three parameter groups, a random state format,
grad dtype and grad handling (per-parameter .grad, some absent, or flat
grads), learning rates changed between steps as a schedule would, on
some runs torch.amp.GradScaler driving the steps (a scale that is a power
of two or not, an overflowing grad now and then) or the global grad norm
clipped through clip_grad_norm, and on some runs a checkpoint through
state_dict / torch.save / load_state_dict into a fresh optimizer halfway.  Parameters, moments and step counters bit
for bit against the oracle after every step (NaNs compared as NaNs).
APEXW_WRAPPER_FUZZ_SEEDS asks for more runs than the default 12."""
import io
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_helpers import bits, n_bit_mismatch_nan_equal, norm_rel_bound, say, stable_max_norm
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
    drive = str(rng.choice(["plain", "amp", "clip"], p=[0.4, 0.3, 0.3]))
    if drive == "amp":              # GradScaler's own overflow check takes no bf16 grads
        grad_dtype = torch.float32
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
    scaler = (torch.amp.GradScaler("cuda", init_scale=float(rng.choice([2.0 ** 10, 3000.0])),
                                   growth_interval=1000) if drive == "amp" else None)
    say("  drive", drive, "checkpoint at", checkpoint_at)
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
        scale = 1.0
        if scaler is not None:
            scaler.scale(torch.ones((), device=DEV))      # as a training loop scales its loss
            scale = float(scaler.get_scale())
        overflow = scaler is not None and rng.random() < 0.2
        g_np = []
        for j, i in enumerate(order):
            # (GradScaler.update needs a grad somewhere: the first is present then)
            present = flat or rng.random() < 0.85 or (scaler is not None and j == 0)
            g_cpu = (torch.randn(shapes[i], generator=gen) * 1e-3 * scale).to(gdt[j])
            if overflow and j == 0 and present:
                g_cpu.view(-1)[0] = float("inf")
            if flat:
                params[i].grad.copy_(g_cpu.to(DEV))
            else:                                     # the optimizer set grad_dtype if it differs
                params[i].grad = g_cpu.to(DEV) if present else None
            g_np.append(bits(g_cpu.reshape(-1)) if present else None)
        overflow = overflow and g_np[0] is not None
        grp = [W.Group(lr=float(g["lr"]), beta1=float(g["betas"][0]), beta2=float(g["betas"][1]),
                       eps=float(g["eps"]), weight_decay=float(g["weight_decay"]))
               for g in opt.param_groups]
        if scaler is not None:
            scaler.step(opt)
            scaler.update()
            inv = float(np.float32(1.0 / np.float64(np.float32(scale))))   # fp64 reciprocal, once rounded
            ref.step(th_ref, g_np, grp, found_inf=overflow, inv_scale=inv)
            assert scaler.get_scale() == (scale / 2 if overflow else scale), (seed, k)
        elif drive == "clip" and rng.random() < 0.6:
            want = ref.grad_norm(g_np, 1.0)
            rel = norm_rel_bound(g_np)
            mn = stable_max_norm(ref, want, rel, float(10 ** rng.uniform(-3, 0)))
            norm_t, coef_t = opt.clip_grad_norm(mn)
            opt.step(clip_coef=coef_t)
            c = ref.clip_coef(want, mn)
            ref.step(th_ref, g_np, grp, clip_coef=c)
            torch.cuda.synchronize()
            assert abs(norm_t.item() - want) <= rel * want and coef_t.item() == c, (seed, k)
        else:
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
