"""torch-facing wrapper of the HIP fused AdamW library.

``AdamW`` takes CUDA (ROCm) tensors or torch-style parameter-group dicts,
allocates the optimizer state and the library workspace as torch uint8
buffers, and on ``step()`` hands the current grads, the group
hyperparameters and the device ``found_inf`` flag to ``apexw_step`` on
torch's current stream.  torch is only the allocator and the stream here;
the whole update runs in the library's kernels.
"""
from __future__ import annotations

from typing import Dict, Iterable, List, Optional

import torch

from . import _lib as L

_DT = {torch.float32: L.APEXW_F32, torch.bfloat16: L.APEXW_BF16}
_FMT = {"f32": L.APEXW_STATE_F32, "bf16": L.APEXW_STATE_BF16, "q8": L.APEXW_STATE_Q8}
_MOMENT_DTYPE = {"f32": (torch.float32, torch.float32),
                 "bf16": (torch.bfloat16, torch.bfloat16),
                 "q8": (torch.int8, torch.uint8)}


class _GroupView:
    __slots__ = ("lr", "beta1", "beta2", "eps", "weight_decay")

    def __init__(self, g: Dict):
        self.lr = float(g["lr"])
        self.beta1, self.beta2 = (float(b) for b in g["betas"])
        self.eps = float(g["eps"])
        self.weight_decay = float(g["weight_decay"])


class AdamW:
    """Fused multi-tensor AdamW (decoupled decay, scalar bias correction).

    state: "f32", "bf16" (round-to-nearest-even moments) or "q8" (int8 m /
    uint8 v codes with one fp32 absmax scale per 256-element block).
    grad_dtype: dtype the grads will have (default: each parameter's dtype).
    """

    def __init__(self, params: Iterable, lr: float = 1e-3, betas=(0.9, 0.999),
                 eps: float = 1e-8, weight_decay: float = 0.0, state: str = "f32",
                 grad_dtype: Optional[torch.dtype] = None):
        if state not in _FMT:
            raise ValueError("state must be one of %s" % sorted(_FMT))
        defaults = dict(lr=lr, betas=tuple(betas), eps=eps, weight_decay=weight_decay)
        params = list(params)
        if params and isinstance(params[0], dict):
            groups = [dict(defaults, **{k: v for k, v in g.items()}) for g in params]
        else:
            groups = [dict(defaults, params=params)]
        self.param_groups: List[Dict] = []
        self._params: List[torch.Tensor] = []
        group_of: List[int] = []
        for gi, g in enumerate(groups):
            g["params"] = list(g["params"])
            self.param_groups.append(g)
            for p in g["params"]:
                if not isinstance(p, torch.Tensor) or p.device.type != "cuda":
                    raise ValueError("parameters must be GPU tensors")
                if p.dtype not in _DT:
                    raise TypeError("parameter dtype %s is not float32 or bfloat16" % p.dtype)
                if not p.is_contiguous():
                    raise ValueError("parameters must be contiguous")
                self._params.append(p)
                group_of.append(gi)
        if not self._params:
            raise ValueError("no parameters")
        self.device = self._params[0].device
        self.state_fmt = state
        self._numel = [p.numel() for p in self._params]
        self._pdt = [_DT[p.dtype] for p in self._params]
        self._gdtype = [grad_dtype or p.dtype for p in self._params]
        self._gdt = [_DT[d] for d in self._gdtype]
        fmt = _FMT[state]
        self.state_bytes = L.apexw_state_bytes(self._numel, fmt)
        self._layout, self._steps_off = L.apexw_state_layout(self._numel, fmt)
        ws_bytes = L.apexw_workspace_bytes(self._numel)
        with torch.cuda.device(self.device):
            self.state = torch.empty(self.state_bytes, dtype=torch.uint8, device=self.device)
            self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
            stream = torch.cuda.current_stream(self.device).cuda_stream
            self._h = L.apexw_create(self._numel, self._pdt, self._gdt, group_of,
                                     len(self.param_groups), fmt, self.state.data_ptr(),
                                     self.state_bytes, self.workspace.data_ptr(), ws_bytes,
                                     stream)
        self._params_arr = L.make_ptrs([p.data_ptr() for p in self._params])

    # ------------------------------------------------------------ stepping
    def step(self, found_inf: Optional[torch.Tensor] = None) -> None:
        """One update; a parameter whose .grad is None is left untouched.
        found_inf: optional one-element float32 GPU tensor; nonzero skips the
        step on the device."""
        ptrs = []
        for p, gdt in zip(self._params, self._gdtype):
            g = p.grad
            if g is None:
                ptrs.append(0)
                continue
            if g.is_sparse:
                raise RuntimeError("sparse gradients are not supported")
            if g.dtype != gdt or g.shape != p.shape or not g.is_contiguous() \
                    or g.device != p.device:
                raise ValueError("grad must be a contiguous %s tensor shaped like its "
                                 "parameter on %s" % (gdt, p.device))
            # an empty grad has no storage; any non-null pointer marks "present"
            ptrs.append(g.data_ptr() or 16)
        self.step_pointers(L.make_ptrs(ptrs), found_inf)

    def step_pointers(self, grads_arr, found_inf: Optional[torch.Tensor] = None) -> None:
        """Step with a prepared void*[] of grad pointers (see _lib.make_ptrs)."""
        fi = 0
        if found_inf is not None:
            if found_inf.dtype != torch.float32 or found_inf.device != self.device \
                    or found_inf.numel() < 1:
                raise ValueError("found_inf must be a float32 tensor on the parameters' device")
            fi = found_inf.data_ptr()
        groups = [_GroupView(g) for g in self.param_groups]
        with torch.cuda.device(self.device):
            stream = torch.cuda.current_stream(self.device).cuda_stream
            L.apexw_step(self._h, L.make_groups(groups), len(groups), self._params_arr,
                         grads_arr, fi, stream)

    # ------------------------------------------------------------ state views
    def moments(self, i: int):
        """(m, v) of parameter i as views into the state buffer (format dtype)."""
        m_off, v_off, _, _ = self._layout[i]
        dm, dv = _MOMENT_DTYPE[self.state_fmt]
        n = self._numel[i]
        m = self.state[m_off:m_off + n * dm.itemsize].view(dm)
        v = self.state[v_off:v_off + n * dv.itemsize].view(dv)
        return m, v

    def scales(self, i: int):
        """(m_scale, v_scale) fp32 views of parameter i (8-bit state only)."""
        _, _, ms, vs = self._layout[i]
        if ms < 0:
            raise ValueError("only the 8-bit state has block scales")
        nb = (self._numel[i] + L.APEXW_Q8_BLOCK - 1) // L.APEXW_Q8_BLOCK
        return (self.state[ms:ms + 4 * nb].view(torch.float32),
                self.state[vs:vs + 4 * nb].view(torch.float32))

    def steps(self) -> torch.Tensor:
        """int32 step counter of every parameter (view)."""
        n = len(self._params)
        return self.state[self._steps_off:self._steps_off + 4 * n].view(torch.int32)

    def launch_info(self):
        return L.apexw_launch_info(self._h)

    def set_workgroups(self, wg: int) -> None:
        L.apexw_set_workgroups(self._h, wg)

    def close(self) -> None:
        if getattr(self, "_h", None):
            L.apexw_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
