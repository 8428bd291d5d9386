"""Helpers of the GPU parity tests: drive the HIP library through its C ABI
(ctypes binding) with torch-allocated device buffers, and run the oracle on
the same inputs copied to the host."""
from __future__ import annotations

from typing import List, Optional, Sequence

import numpy as np
import torch

import oracle
import workloads as W
from tensor_adamw_optimizer_amd import _lib as L

DT = {W.F32: L.APEXW_F32, W.BF16: L.APEXW_BF16}
FMT = {W.STATE_F32: L.APEXW_STATE_F32, W.STATE_BF16: L.APEXW_STATE_BF16,
       W.STATE_Q8: L.APEXW_STATE_Q8}
MOMENT_DTYPE = {W.STATE_F32: (torch.float32, torch.float32),
                W.STATE_BF16: (torch.bfloat16, torch.bfloat16),
                W.STATE_Q8: (torch.int8, torch.uint8)}


def say(*a):
    print(*a, flush=True)


class GpuOpt:
    """One library handle over caller-owned torch tensors."""

    def __init__(self, numels: Sequence[int], param_dtype: Sequence[str],
                 grad_dtype: Sequence[str], group_of: Sequence[int], n_groups: int,
                 state_fmt: str, device="cuda"):
        self.numels = list(numels)
        self.state_fmt = state_fmt
        fmt = FMT[state_fmt]
        self.state_bytes = L.apexw_state_bytes(self.numels, fmt)
        self.layout, self.steps_off = L.apexw_state_layout(self.numels, fmt)
        self.ws_bytes = L.apexw_workspace_bytes(self.numels)
        # garbage in the buffers: create must zero the state itself
        self.state = torch.full((self.state_bytes + 256,), 0x5A, dtype=torch.uint8,
                                device=device)
        self.ws = torch.full((self.ws_bytes,), 0xA5, dtype=torch.uint8, device=device)
        self.stream = torch.cuda.current_stream().cuda_stream
        self.h = L.apexw_create(self.numels, [DT[d] for d in param_dtype],
                                [DT[d] for d in grad_dtype], list(group_of), n_groups,
                                fmt, self.state.data_ptr(), self.state_bytes,
                                self.ws.data_ptr(), self.ws_bytes, self.stream)

    def step(self, groups, params: Sequence[Optional[torch.Tensor]],
             grads: Sequence[Optional[torch.Tensor]],
             found_inf: Optional[torch.Tensor] = None):
        pa = L.make_ptrs([0 if p is None else p.data_ptr() for p in params])
        ga = L.make_ptrs([0 if g is None else (g.data_ptr() or 16) for g in grads])
        L.apexw_step(self.h, L.make_groups(groups), len(groups), pa, ga,
                     0 if found_inf is None else found_inf.data_ptr(), self.stream)

    def moments(self, i: int):
        m_off, v_off, _, _ = self.layout[i]
        dm, dv = MOMENT_DTYPE[self.state_fmt]
        n = self.numels[i]
        return (self.state[m_off:m_off + n * dm.itemsize].view(dm),
                self.state[v_off:v_off + n * dv.itemsize].view(dv))

    def scales(self, i: int):
        _, _, ms, vs = self.layout[i]
        nb = (self.numels[i] + 255) // 256
        return (self.state[ms:ms + 4 * nb].view(torch.float32),
                self.state[vs:vs + 4 * nb].view(torch.float32))

    def steps(self) -> torch.Tensor:
        n = len(self.numels)
        return self.state[self.steps_off:self.steps_off + 4 * n].view(torch.int32)

    def close(self):
        if self.h:
            L.apexw_destroy(self.h)
            self.h = 0


def bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy copy: fp32 -> float32, bf16 -> uint16 bits, ints as is."""
    return W.to_numpy_bits(t)


def as_f32(a: np.ndarray) -> np.ndarray:
    return oracle.bf16_to_f32(a) if a.dtype == np.uint16 else a.astype(np.float32)


def rel_err_elementwise(a: np.ndarray, b: np.ndarray) -> float:
    """max |a-b| / |b| over elements (0 where a == b)."""
    a = as_f32(a).astype(np.float64)
    b = as_f32(b).astype(np.float64)
    d = np.abs(a - b)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(d == 0, 0.0, d / np.abs(b))
    return float(np.max(r)) if r.size else 0.0


def normwise_err(a: np.ndarray, b: np.ndarray) -> float:
    a = as_f32(a).astype(np.float64)
    b = as_f32(b).astype(np.float64)
    den = np.max(np.abs(b)) if b.size else 0.0
    return float(np.max(np.abs(a - b)) / den) if den > 0 else float(np.max(np.abs(a - b), initial=0))


def n_bit_mismatch(a: np.ndarray, b: np.ndarray) -> int:
    assert a.dtype == b.dtype and a.shape == b.shape, (a.dtype, b.dtype, a.shape, b.shape)
    return int(np.count_nonzero(a.view(np.uint8).reshape(a.size, -1) !=
                                b.view(np.uint8).reshape(b.size, -1)) if a.size else 0)


def _nan_mask(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.float32:
        return np.isnan(a)
    if a.dtype == np.uint16:                              # bf16 bit patterns
        return (a & 0x7FFF) > 0x7F80
    return np.zeros(a.shape, dtype=bool)


def n_bit_mismatch_nan_equal(a: np.ndarray, b: np.ndarray) -> int:
    """Elements whose bits differ, except where both are NaN: IEEE 754 leaves
    the sign and payload of a NaN that an invalid operation makes (0/0,
    inf - inf, 0 * inf) unspecified, and the host's x86 default NaN has the
    sign set where gfx950's has it clear.  Every other value, and where the
    NaNs are, must agree bit for bit."""
    assert a.dtype == b.dtype and a.shape == b.shape, (a.dtype, b.dtype, a.shape, b.shape)
    if not a.size:
        return 0
    diff = (a.view(np.uint8).reshape(a.size, -1) != b.view(np.uint8).reshape(b.size, -1)).any(1)
    return int(np.count_nonzero(diff & ~(_nan_mask(a) & _nan_mask(b))))


def norm_rel_bound(grads) -> float:
    """Bound on |device norm - oracle norm| / oracle norm.  Both sum the same
    N squares (u*u of fp32 values u, exact in fp64) in different orders; any
    order of N - 1 additions of non-negative terms errs by at most
    gamma(N-1) = (N-1)u/(1-(N-1)u) of the sum (u = 2^-53), so the two sums
    differ by at most twice that, and the square roots (each rounded once)
    by at most gamma(N-1) + 2u relative."""
    n = sum(g.size for g in grads if g is not None)
    u = 2.0 ** -53
    return (n * u / (1.0 - n * u)) + 2.0 * u


def stable_max_norm(ref, want: float, rel: float, max_norm: float) -> float:
    """max_norm, nudged up until the fp32 clip coefficient is the same for
    every norm within rel of want: a coefficient on an fp32 rounding edge
    could then differ between two correct norms (a choice made from the
    oracle's norm alone)."""
    lo, hi = want * (1.0 - rel), want * (1.0 + rel)
    while ref.clip_coef(lo, max_norm) != ref.clip_coef(hi, max_norm):
        max_norm *= 1.0 + 2.0 ** -12
    return max_norm


def assert_fp32_state_parity(name, gpu, ref, rtol=1e-5):
    """fp32 bar: elementwise relative error <= rtol (expected: bitwise)."""
    e = rel_err_elementwise(gpu, ref)
    nb = n_bit_mismatch(gpu, ref)
    if e > 0 or nb:
        say("  %-10s max_rel=%.3g bit_mismatch=%d/%d" % (name, e, nb, gpu.size))
    assert e <= rtol, (name, e, nb)
    return nb
