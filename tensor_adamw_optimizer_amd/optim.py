"""torch-facing wrapper of the HIP fused AdamW library.

``AdamW`` is a torch.optim.Optimizer over CUDA (ROCm) tensors or
parameter-group dicts.  It allocates the optimizer state and the library
workspace as torch uint8 buffers, and on ``step()`` hands the current grads,
the group hyperparameters and the device ``found_inf`` flag to the library
on torch's current stream.  torch is only the allocator and the stream here;
the whole update runs in the library's kernels.
"""
from __future__ import annotations

import contextlib
from array import array
from typing import Dict, Iterable, List, Optional

import torch
import torch.optim.optimizer as _torch_optimizer

from . import _lib as L

# torch's current stream as a raw pointer: the query torch's own kernels
# launch with (a fraction of torch.cuda.current_stream's cost); the public
# form where a build lacks it
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)

# torch's registries of global optimizer step hooks (module-level dicts in
# torch.optim.optimizer); a build without them is treated as having hooks,
# so every step takes the hooked path
_NO_HOOKS: Dict = {}
_ALWAYS: Dict = {None: None}


def _global_pre_hooks() -> Dict:
    return getattr(_torch_optimizer, "_global_optimizer_pre_hooks", _ALWAYS)


def _global_post_hooks() -> Dict:
    return getattr(_torch_optimizer, "_global_optimizer_post_hooks", _NO_HOOKS)


def _profiling() -> bool:
    return bool(getattr(torch.autograd.profiler, "_is_profiler_enabled", True))

_DT = {torch.float32: L.APEXW_F32, torch.bfloat16: L.APEXW_BF16}
_FMT = {"f32": L.APEXW_STATE_F32, "fp32": L.APEXW_STATE_F32, "bf16": L.APEXW_STATE_BF16,
        "q8": L.APEXW_STATE_Q8}
_MOMENT_DTYPE = {"f32": (torch.float32, torch.float32), "fp32": (torch.float32, torch.float32),
                 "bf16": (torch.bfloat16, torch.bfloat16),
                 "q8": (torch.int8, torch.uint8)}


class _GroupView:
    __slots__ = ("lr", "beta1", "beta2", "eps", "weight_decay")

    def __init__(self, g: Dict):
        self.lr = float(g["lr"])
        self.beta1, self.beta2 = (float(b) for b in g["betas"])
        self.eps = float(g["eps"])
        self.weight_decay = float(g["weight_decay"])


class AdamW(torch.optim.Optimizer):
    """Fused multi-tensor AdamW (decoupled decay, scalar bias correction).

    A torch.optim.Optimizer: parameter groups, learning-rate schedulers and
    zero_grad work as usual, and torch.amp.GradScaler hands over its scale
    and overflow flag (the update unscales the grads itself and skips the
    step on the device, no host sync).  The tensor list is fixed at
    construction (add_param_group afterwards is refused).

    state: "f32" (or "fp32"), "bf16" (round-to-nearest-even moments) or "q8" (int8 m /
    uint8 v codes with one fp32 absmax scale per 256-element block).
    grad_dtype: dtype the grads will have (default: each parameter's dtype);
    a parameter of another dtype gets its grad_dtype attribute set to it, the
    torch rule for such grads (backward then produces them in that dtype).
    flat_grads: give every parameter a .grad that is a view into one flat
    buffer per grad dtype (each view 64-byte aligned), made here, zero-filled.
    Autograd then accumulates into these views in place, and step() hands the
    library the same pointer table every time instead of reading 'p.grad' of
    every parameter: O(1) host work per step besides one pass over the
    parameter pointers.  The contract: the .grad attributes stay these views
    (do not assign or delete them; zero_grad() of this optimizer zeroes the
    buffers in place whatever set_to_none says), so every parameter has a
    grad on every step -- a parameter that received none gets a zero grad,
    which decays it and counts a step, as torch does with set_to_none=False.
    flat_grads_intact() tells whether the contract still holds; step() looks
    at two parameters' .grad each time and raises once it finds a broken one
    (a whole list at the next step, a single one within a pass over the list).
    """

    # torch.amp.GradScaler: set grad_scale / found_inf on the optimizer and
    # call step() directly instead of unscaling the grads first
    _step_supports_amp_scaling = True

    def __init__(self, params: Iterable, lr: float = 1e-3, betas=(0.9, 0.999),
                 eps: float = 1e-8, weight_decay: float = 0.0, state: str = "f32",
                 grad_dtype: Optional[torch.dtype] = None, flat_grads: bool = False):
        if state not in _FMT:
            raise ValueError("state must be one of %s" % sorted(_FMT))
        self._h = None
        defaults = dict(lr=lr, betas=tuple(betas), eps=eps, weight_decay=weight_decay)
        super().__init__(params, defaults)
        self._params: List[torch.Tensor] = []
        group_of: List[int] = []
        for gi, g in enumerate(self.param_groups):
            for p in g["params"]:
                if p.device.type != "cuda":
                    raise ValueError("parameters must be GPU tensors")
                if p.dtype not in _DT:
                    raise TypeError("parameter dtype %s is not float32 or bfloat16" % p.dtype)
                if not p.is_contiguous():
                    raise ValueError("parameters must be contiguous")
                self._params.append(p)
                group_of.append(gi)
        self.device = self._params[0].device
        self.state_fmt = state
        self._numel = [p.numel() for p in self._params]
        self._pdt = [_DT[p.dtype] for p in self._params]
        self._gdtype = [grad_dtype or p.dtype for p in self._params]
        # torch accepts a .grad of another dtype than its parameter only
        # where the parameter's grad_dtype says so; autograd then produces
        # grads of that dtype
        for p, d in zip(self._params, self._gdtype):
            if d != p.dtype and hasattr(p, "grad_dtype"):
                p.grad_dtype = d
        self._gdt = [_DT[d] for d in self._gdtype]
        fmt = _FMT[state]
        self.state_bytes = L.apexw_state_bytes(self._numel, fmt)
        self._layout, self._steps_off = L.apexw_state_layout(self._numel, fmt)
        ws_bytes = L.apexw_workspace_bytes(self._numel)
        with torch.cuda.device(self.device):
            self.state_buffer = torch.empty(self.state_bytes, dtype=torch.uint8, device=self.device)
            self.workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=self.device)
            stream = torch.cuda.current_stream(self.device).cuda_stream
            self._h = L.apexw_create(self._numel, self._pdt, self._gdt, group_of,
                                     len(self.param_groups), fmt, self.state_buffer.data_ptr(),
                                     self.state_bytes, self.workspace.data_ptr(), ws_bytes,
                                     stream)
        self._param_ptrs = list(map(torch.Tensor.data_ptr, self._params))
        self._params_arr = L.make_ptrs(self._param_ptrs)
        # the groups' hyperparameters as the library reads them, refreshed in
        # place every step (the group count is fixed with the tensor list)
        self._groups_arr = (L.apexw_group * len(self.param_groups))()
        self._inv_buf: Optional[torch.Tensor] = None
        self._flat_bufs: List[torch.Tensor] = []
        self._flat_views: List[torch.Tensor] = []
        self._flat_arr = None
        if flat_grads:
            self._make_flat_grads()

    def _make_flat_grads(self) -> None:
        align = 64
        offsets, total = [], {}
        for n, d in zip(self._numel, self._gdtype):
            off = total.get(d, 0)
            offsets.append(off)
            total[d] = off + (n * d.itemsize + align - 1) // align * align
        bufs = {d: torch.zeros(max(b, align), dtype=torch.uint8, device=self.device)
                for d, b in total.items()}
        for p, n, d, off in zip(self._params, self._numel, self._gdtype, offsets):
            p.grad = bufs[d][off:off + n * d.itemsize].view(d).view(p.shape)
            self._flat_views.append(p.grad)
        self._flat_bufs = list(bufs.values())
        self._flat_arr = L.make_ptrs([g.data_ptr() or 16 for g in self._flat_views])
        self._flat_probe = 0

    def _flat_table(self):
        """The flat buffers' pointer table, after a look at two parameters'
        .grad (the first and one in rotation): a .grad removed or replaced
        behind this optimizer's back (Module.zero_grad with set_to_none, an
        assignment) would leave the step reading buffers that no longer
        receive the grads.  A list-wide break is found on the next step, one
        replaced .grad within one pass over the list."""
        k = self._flat_probe
        for i in (0, k):
            if self._params[i].grad is not self._flat_views[i]:
                raise RuntimeError(
                    "flat_grads: the .grad of parameter %d is no longer the view this optimizer "
                    "made; zero the grads with this optimizer's zero_grad() and never assign or "
                    "delete .grad" % i)
        self._flat_probe = k + 1 if k + 1 < len(self._params) else 0
        return self._flat_arr

    def flat_grads_intact(self) -> bool:
        """True while every .grad is still the view flat_grads made."""
        return bool(self._flat_views) and all(
            p.grad is g for p, g in zip(self._params, self._flat_views))

    def zero_grad(self, set_to_none: bool = True) -> None:
        if self._flat_bufs:
            for b in self._flat_bufs:       # the views stay in place
                b.zero_()
            return
        super().zero_grad(set_to_none=set_to_none)

    def _check_params(self) -> None:
        """Re-read the parameter pointers (one pass of cheap calls); a storage
        that moved -- 'p.data = ...', a re-materialised parameter -- gets a new
        pointer table, and a change of size, dtype, device or layout is refused."""
        ptrs = list(map(torch.Tensor.data_ptr, self._params))
        if ptrs == self._param_ptrs:
            return
        for i, p in enumerate(self._params):
            if (p.numel() != self._numel[i] or _DT.get(p.dtype) != self._pdt[i]
                    or p.device != self.device or not p.is_contiguous()):
                raise ValueError("parameter %d changed size, dtype, device or layout since the "
                                 "optimizer was built" % i)
        self._param_ptrs = ptrs
        self._params_arr = L.make_ptrs(ptrs)

    def add_param_group(self, param_group: Dict) -> None:
        if getattr(self, "_h", None) is not None:
            raise NotImplementedError(
                "the tensor list of this optimizer is fixed at construction; build a new "
                "one (state_dict / load_state_dict carry the state of the common tensors)")
        super().add_param_group(param_group)

    # ------------------------------------------------------------ stepping
    def _grads_arr(self):
        """The grad-pointer table of this step (0: no grad).  One pass of
        cheap per-tensor calls: torch itself guarantees that a .grad has its
        parameter's shape and device (and its dtype unless the parameter's
        grad_dtype says otherwise); sparse grads, which have no data pointer,
        and non-contiguous grads are refused."""
        gs = [p.grad for p in self._params]
        try:
            ptrs = array("Q", [0 if g is None else (g.data_ptr() or 16) for g in gs])
        except RuntimeError:
            if any(g is not None and g.layout is not torch.strided for g in gs):
                raise L.ApexwError(L.APEXW_ESPARSE, "AdamW.step",
                                   "sparse gradients are not supported") from None
            raise
        if not all(g is None or (g.is_contiguous() and g.dtype is d)
                   for g, d in zip(gs, self._gdtype)):
            bad = next(i for i, (g, d) in enumerate(zip(gs, self._gdtype))
                       if g is not None and not (g.is_contiguous() and g.dtype is d))
            raise ValueError("grad %d must be a contiguous %s tensor shaped like its parameter"
                             % (bad, self._gdtype[bad]))
        return L.ptr_table(ptrs)

    def _dev_ptr(self, t: Optional[torch.Tensor], name: str, dtype=torch.float32) -> int:
        if t is None:
            return 0
        if t.dtype != dtype or t.device != self.device or t.numel() < 1:
            raise ValueError("%s must be a %s tensor on the parameters' device" % (name, dtype))
        return t.data_ptr()

    def _stream(self) -> int:
        if _raw_stream is not None:
            return int(_raw_stream(self.device.index))
        return torch.cuda.current_stream(self.device).cuda_stream

    def _on_device(self):
        """The parameters' device made current for a library call (nothing to
        do when it already is)."""
        if torch.cuda.current_device() == self.device.index:
            return contextlib.nullcontext()
        return torch.cuda.device(self.device)

    def step(self, closure=None, found_inf: Optional[torch.Tensor] = None,
             inv_scale: Optional[torch.Tensor] = None,
             clip_coef: Optional[torch.Tensor] = None):
        """One update; a parameter whose .grad is None is left untouched.
        found_inf: one-element float32 GPU tensor, nonzero skips the step on
        the device.  inv_scale: grads are unscaled by it first.  clip_coef:
        then multiplied by it (see clip_grad_norm).  Under a GradScaler the
        scaler's grad_scale and found_inf are used when these are not given.

        Step pre- and post-hooks (this optimizer's and the global ones) and
        the profiler's record of the step work as with torch's optimizers;
        this class calls them itself (torch's own step wrapper costs several
        microseconds of host time per call even when none is registered)."""
        if (self._optimizer_step_pre_hooks or self._optimizer_step_post_hooks
                or _global_pre_hooks() or _global_post_hooks() or _profiling()):
            return self._step_hooked(closure, found_inf, inv_scale, clip_coef)
        return self._step(closure, found_inf, inv_scale, clip_coef)

    # torch.optim.Optimizer wraps a subclass's step with its hook runner
    # unless the step says it runs the hooks itself
    step.hooked = True

    def _step_hooked(self, closure, found_inf, inv_scale, clip_coef):
        """step() with hooks or the profiler, as torch's own step wrapper runs
        them: pre-hooks (which may replace the arguments), the step, then
        post-hooks, inside a record_function named as torch names it."""
        args = (self,)
        kwargs = dict(closure=closure, found_inf=found_inf, inv_scale=inv_scale,
                      clip_coef=clip_coef)
        name = "Optimizer.step#%s.step" % self.__class__.__name__
        with torch.autograd.profiler.record_function(name):
            glob_pre = _global_pre_hooks()
            for pre_hook in [h for h in glob_pre.values() if h is not None] + \
                    list(self._optimizer_step_pre_hooks.values()):
                result = pre_hook(self, args, kwargs)
                if result is not None:
                    if isinstance(result, tuple) and len(result) == 2:
                        args, kwargs = result
                    else:
                        raise RuntimeError("a step pre-hook must return None or a tuple "
                                           "(new_args, new_kwargs), got %r" % (result,))
            out = self._step(*args[1:], **kwargs)
            self._optimizer_step_code()
            for post_hook in list(self._optimizer_step_post_hooks.values()) + \
                    list(_global_post_hooks().values()):
                post_hook(self, args, kwargs)
        return out

    def _step(self, closure=None, found_inf: Optional[torch.Tensor] = None,
              inv_scale: Optional[torch.Tensor] = None,
              clip_coef: Optional[torch.Tensor] = None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        scaler_scale = getattr(self, "grad_scale", None)
        scaler_inf = getattr(self, "found_inf", None)
        if found_inf is None and torch.is_tensor(scaler_inf):
            # (a step in which no parameter has a grad gets the plain number
            # 0 from the scaler: nothing to check, nothing to skip)
            found_inf = scaler_inf.to(torch.float32).reshape(1)
        if inv_scale is None and scaler_scale is not None:
            inv_scale = self.inv_scale_of(scaler_scale)
        self.step_pointers(self._flat_table() if self._flat_arr is not None else self._grads_arr(),
                           found_inf, inv_scale, clip_coef)
        return loss

    def inv_scale_of(self, scale: torch.Tensor) -> torch.Tensor:
        """The unscaling factor for a loss scale held on the device, formed by
        the library as the fp64 reciprocal of the scale rounded once to fp32
        (a one-element float32 tensor this optimizer reuses)."""
        scale = scale.to(torch.float32).reshape(1)
        if self._inv_buf is None:
            self._inv_buf = torch.empty(1, dtype=torch.float32, device=self.device)
        with self._on_device():
            L.apexw_inv_scale(self._dev_ptr(scale, "grad_scale"), self._inv_buf.data_ptr(),
                              self._stream())
        return self._inv_buf

    def step_pointers(self, grads_arr, found_inf: Optional[torch.Tensor] = None,
                      inv_scale: Optional[torch.Tensor] = None,
                      clip_coef: Optional[torch.Tensor] = None) -> None:
        """Step with a prepared void*[] of grad pointers (_lib.make_ptrs or
        _lib.ptr_table), or with None: the grad table of the previous call on
        this optimizer -- for grad buffers that persist across steps, with no
        per-tensor work on the host."""
        arr = self._groups_arr
        for a, g in zip(arr, self.param_groups):    # a schedule may have changed them
            a.lr = float(g["lr"])
            b1, b2 = g["betas"]
            a.beta1 = float(b1)
            a.beta2 = float(b2)
            a.eps = float(g["eps"])
            a.weight_decay = float(g["weight_decay"])
        self._check_params()
        with self._on_device():
            L.apexw_step_ex(self._h, arr, len(arr), self._params_arr,
                            grads_arr, self._dev_ptr(inv_scale, "inv_scale"),
                            self._dev_ptr(clip_coef, "clip_coef"),
                            self._dev_ptr(found_inf, "found_inf"), 0, self._stream())

    def unscale_check(self, inv_scale: Optional[torch.Tensor], found_inf: torch.Tensor) -> None:
        """Set found_inf to 1 if any grad times inv_scale is not finite (never
        clears it); grads are not rewritten -- pass inv_scale to step()."""
        with self._on_device():
            L.apexw_unscale_check(self._h, self._grads_arr(), self._dev_ptr(inv_scale, "inv_scale"),
                                  self._dev_ptr(found_inf, "found_inf"), self._stream())

    def clip_grad_norm(self, max_norm: float, inv_scale: Optional[torch.Tensor] = None,
                       found_inf: Optional[torch.Tensor] = None):
        """Global norm of the (unscaled) grads and the clip coefficient, both
        on the device: returns (norm fp64 tensor, coef fp32 tensor); pass coef
        to step(clip_coef=...).  With found_inf the finite check runs too."""
        norm = torch.empty(1, dtype=torch.float64, device=self.device)
        coef = torch.empty(1, dtype=torch.float32, device=self.device)
        with self._on_device():
            L.apexw_clip_grad_norm(self._h, self._grads_arr(), self._dev_ptr(inv_scale, "inv_scale"),
                                   float(max_norm), self._dev_ptr(found_inf, "found_inf"),
                                   norm.data_ptr(), coef.data_ptr(), self._stream())
        return norm, coef

    # ------------------------------------------------------------ checkpoint
    def state_dict(self) -> Dict:
        """The optimizer checkpoint: the library's blob (format, tensor list,
        recipe, moments, scales, step counters) as a CPU uint8 tensor, plus
        the parameter-group hyperparameters; loadable with
        torch.load(weights_only=True)."""
        groups = [_GroupView(g) for g in self.param_groups]
        with self._on_device():
            blob = L.apexw_export_state(self._h, L.make_groups(groups), len(groups), self._stream())
        return {
            "apexw_blob": torch.frombuffer(bytearray(blob), dtype=torch.uint8),
            "param_groups": [{"lr": g["lr"], "betas": list(g["betas"]), "eps": g["eps"],
                              "weight_decay": g["weight_decay"]} for g in self.param_groups],
        }

    def load_state_dict(self, sd: Dict) -> None:
        blob = bytes(sd["apexw_blob"].cpu().numpy().tobytes())
        with self._on_device():
            L.apexw_import_state(self._h, blob, len(self.param_groups), self._stream())
        for g, h in zip(self.param_groups, sd["param_groups"]):
            g["lr"], g["betas"] = h["lr"], tuple(h["betas"])
            g["eps"], g["weight_decay"] = h["eps"], h["weight_decay"]

    # ------------------------------------------------------------ state views
    def moments(self, i: int):
        """(m, v) of parameter i as views into the state buffer (format dtype)."""
        m_off, v_off, _, _ = self._layout[i]
        dm, dv = _MOMENT_DTYPE[self.state_fmt]
        n = self._numel[i]
        m = self.state_buffer[m_off:m_off + n * dm.itemsize].view(dm)
        v = self.state_buffer[v_off:v_off + n * dv.itemsize].view(dv)
        return m, v

    def scales(self, i: int):
        """(m_scale, v_scale) fp32 views of parameter i (8-bit state only)."""
        _, _, ms, vs = self._layout[i]
        if ms < 0:
            raise ValueError("only the 8-bit state has block scales")
        nb = (self._numel[i] + L.APEXW_Q8_BLOCK - 1) // L.APEXW_Q8_BLOCK
        return (self.state_buffer[ms:ms + 4 * nb].view(torch.float32),
                self.state_buffer[vs:vs + 4 * nb].view(torch.float32))

    def steps(self) -> torch.Tensor:
        """int32 step counter of every parameter (view)."""
        n = len(self._params)
        return self.state_buffer[self._steps_off:self._steps_off + 4 * n].view(torch.int32)

    def read_steps(self):
        """Step counters copied to the host (synchronises the current stream)."""
        with self._on_device():
            return L.apexw_read_steps(self._h, len(self._params), self._stream())

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
