"""Seeded synthetic workloads for the fused multi-tensor AdamW step.

This module only describes inputs: tensor shapes, dtypes, parameter groups,
hyperparameters, the found_inf / grad=None schedules, and seeded generators for
the initial parameters and the per-call gradients.  It holds none of the
optimizer's arithmetic, so both the oracle side (tests, CPU baseline) and the
HIP side (tests, bench) draw from it without sharing any update code.

Workloads (names used throughout tests and bench):

* ``tiny``       4 fp32 tensors [512,512], [1024], [256,1024], [3]; fp32 state;
                 20 calls; call 7 skipped by found_inf; the [3] tensor has no
                 grad on odd calls.
* ``few_large``  8 bf16 parameters [8192,8192] with fp32 grads, fp32 state,
                 10 calls.
* ``many_small`` 20,000 fp32 tensors, element counts log-uniform in
                 [64, 65536], 3 parameter groups round-robin, 10 calls.
* ``bf16_state`` the ``few_large`` tensor list with bf16 moments, 10 calls.
* ``lora_q8``    392 bf16 LoRA A/B tensors of a 28-layer model (hidden 3072,
                 kv 1024, MLP 8192, rank 16, on q,k,v,o,gate,up,down) with bf16
                 grads and 8-bit block-quantized moments, 250 calls.

The LoRA shapes stand in for the Llama-3.2-3B LoRA run reported on the page
"ApexW optimizer measured in Unsloth" (kongchang.com, test-setup section); no
weights or data of that run are used.

Reading of the unstated generator (documented with the design): parameters are
drawn as N(0, 0.02) in fp32 from ``torch.Generator().manual_seed(seed)`` tensor
by tensor in list order and cast (round-to-nearest-even) to the parameter
dtype; grads for 1-based call k are drawn as N(0, 1) fp32 from a generator
seeded ``seed * 1000 + k`` for every tensor in list order, scaled by 1e-3 and
cast to the grad dtype, then dropped where the schedule says "no grad".
"""
from __future__ import annotations

import dataclasses
import math
from typing import Callable, List, Optional, Sequence

import numpy as np
import torch

F32 = "f32"
BF16 = "bf16"

STATE_F32 = "f32"
STATE_BF16 = "bf16"
STATE_Q8 = "q8"

TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Group:
    lr: float
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0


@dataclasses.dataclass
class Workload:
    name: str
    shapes: List[tuple]
    param_dtype: List[str]
    grad_dtype: List[str]
    group_of: List[int]
    groups: List[Group]
    state_fmt: str
    steps: int
    seed: int = 0
    theta_std: float = 0.02
    grad_std: float = 1e-3
    # found_inf at 1-based call k (None: never)
    skip_rule: Optional[Callable[[int], bool]] = None
    # grad present for tensor i at 1-based call k (None: always)
    grad_rule: Optional[Callable[[int, int], bool]] = None

    def skip_call(self, k: int) -> bool:
        return bool(self.skip_rule(k)) if self.skip_rule else False

    def has_grad(self, i: int, k: int) -> bool:
        return bool(self.grad_rule(i, k)) if self.grad_rule else True

    @property
    def numels(self) -> List[int]:
        return [int(np.prod(s)) if len(s) else 1 for s in self.shapes]

    @property
    def n_params(self) -> int:
        return int(sum(self.numels))

    def describe(self) -> dict:
        return {
            "workload": self.name,
            "n_tensors": len(self.shapes),
            "n_params": self.n_params,
            "param_dtype": sorted(set(self.param_dtype)),
            "grad_dtype": sorted(set(self.grad_dtype)),
            "state": self.state_fmt,
            "n_groups": len(self.groups),
            "steps": self.steps,
        }


# ---------------------------------------------------------------- shapes

def lora_shapes(layers: int = 28, hidden: int = 3072, kv: int = 1024,
                mlp: int = 8192, rank: int = 16) -> List[tuple]:
    """LoRA A [r, in] and B [out, r] for q,k,v,o,gate,up,down of each layer,
    in that order, A before B."""
    mods = [  # (in, out)
        (hidden, hidden),  # q
        (hidden, kv),      # k
        (hidden, kv),      # v
        (hidden, hidden),  # o
        (hidden, mlp),     # gate
        (hidden, mlp),     # up
        (mlp, hidden),     # down
    ]
    out = []
    for _ in range(layers):
        for fan_in, fan_out in mods:
            out.append((rank, fan_in))
            out.append((fan_out, rank))
    return out


def log_uniform_sizes(n: int, lo: int, hi: int, seed: int) -> List[int]:
    """Element counts exp(U(ln lo, ln hi)) rounded to the nearest integer."""
    rng = np.random.default_rng(seed)
    x = np.exp(rng.uniform(math.log(lo), math.log(hi), size=n))
    return [int(min(hi, max(lo, round(float(v))))) for v in x]


# ---------------------------------------------------------------- configs

def tiny(seed: int = 0) -> Workload:
    shapes = [(512, 512), (1024,), (256, 1024), (3,)]
    n = len(shapes)
    return Workload(
        name="tiny", shapes=shapes, param_dtype=[F32] * n, grad_dtype=[F32] * n,
        group_of=[0] * n, groups=[Group(lr=1e-3, weight_decay=0.01)],
        state_fmt=STATE_F32, steps=20, seed=seed,
        skip_rule=lambda k: k == 7,
        grad_rule=lambda i, k: not (i == 3 and k % 2 == 1),
    )


def few_large(seed: int = 0, n_tensors: int = 8, dim: int = 8192,
              state_fmt: str = STATE_F32) -> Workload:
    shapes = [(dim, dim)] * n_tensors
    return Workload(
        name="few_large" if state_fmt == STATE_F32 else "bf16_state",
        shapes=shapes, param_dtype=[BF16] * n_tensors,
        grad_dtype=[F32] * n_tensors, group_of=[0] * n_tensors,
        groups=[Group(lr=2e-4, weight_decay=0.1)], state_fmt=state_fmt,
        steps=10, seed=seed,
    )


def few_large_shard(seed: int = 0, ranks: int = 8, n_tensors: int = 8, dim: int = 8192) -> Workload:
    """One rank's share of the few-large list under ZeRO-1 ownership over
    `ranks` GPUs: a contiguous slice of dim/ranks rows of every tensor (a
    multiple of 256 elements), the same dtypes and hyperparameters."""
    w = few_large(seed, n_tensors, dim)
    w.name = "few_large_shard%d" % ranks
    w.shapes = [(dim // ranks, dim)] * n_tensors
    return w


def bf16_state(seed: int = 0, n_tensors: int = 8, dim: int = 8192) -> Workload:
    return few_large(seed, n_tensors, dim, state_fmt=STATE_BF16)


def many_small(seed: int = 0, n_tensors: int = 20000) -> Workload:
    sizes = log_uniform_sizes(n_tensors, 64, 65536, seed)
    groups = [Group(lr=1e-3, weight_decay=0.1), Group(lr=5e-4, weight_decay=0.0),
              Group(lr=1e-4, weight_decay=0.01)]
    return Workload(
        name="many_small", shapes=[(s,) for s in sizes],
        param_dtype=[F32] * n_tensors, grad_dtype=[F32] * n_tensors,
        group_of=[i % 3 for i in range(n_tensors)], groups=groups,
        state_fmt=STATE_F32, steps=10, seed=seed,
    )


def lora_q8(seed: int = 0, layers: int = 28) -> Workload:
    shapes = lora_shapes(layers=layers)
    n = len(shapes)
    return Workload(
        name="lora_q8", shapes=shapes, param_dtype=[BF16] * n,
        grad_dtype=[BF16] * n, group_of=[0] * n,
        groups=[Group(lr=2e-4, weight_decay=0.01)], state_fmt=STATE_Q8,
        steps=250, seed=seed,
    )


WORKLOADS = {
    "tiny": tiny,
    "few_large": few_large,
    "many_small": many_small,
    "bf16_state": bf16_state,
    "lora_q8": lora_q8,
    "few_large_shard8": few_large_shard,
}


# ---------------------------------------------------------------- generators

def init_params(w: Workload, device="cpu") -> List[torch.Tensor]:
    """theta ~ N(0, theta_std) in fp32, cast to each parameter dtype."""
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    out = []
    for shape, dt in zip(w.shapes, w.param_dtype):
        x = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
        x.mul_(w.theta_std)
        out.append(x.to(TORCH_DTYPE[dt]))
    return out


def grads_for_call(w: Workload, k: int, device="cpu",
                   out: Optional[Sequence[torch.Tensor]] = None
                   ) -> List[Optional[torch.Tensor]]:
    """Grads of 1-based call k.  Every tensor is drawn in list order so the
    stream stays aligned; tensors without a grad at call k come back as None.
    With ``out`` the values are written into those tensors (stable addresses).
    """
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed * 1000 + k)
    res: List[Optional[torch.Tensor]] = []
    for i, (shape, dt) in enumerate(zip(w.shapes, w.grad_dtype)):
        x = torch.randn(shape, generator=gen, device=dev, dtype=torch.float32)
        x.mul_(w.grad_std)
        if not w.has_grad(i, k):
            res.append(None)
            continue
        if out is not None and out[i] is not None:
            out[i].copy_(x)
            res.append(out[i])
        else:
            res.append(x.to(TORCH_DTYPE[dt]))
    return res


def found_inf_for_call(w: Workload, k: int) -> bool:
    return bool(w.skip_call(k))


# ---------------------------------------------------------------- numpy views

def to_numpy_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy as numpy: fp32 as float32, bf16 as its uint16 bit pattern."""
    t = t.detach().contiguous().cpu().reshape(-1)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    if t.dtype == torch.float32:
        return t.numpy().copy()
    return t.numpy().copy()
