"""ctypes binding of the C ABI in include/apexw.h -- argument marshalling only.

Each function has the name of the C entry point it wraps.  Sizes come back as
Python ints; a nonzero return code raises :class:`ApexwError` carrying the
code and ``apexw_last_error()``.  Device pointers and streams are plain ints
(``tensor.data_ptr()``, ``stream.cuda_stream``).  Every step of the optimizer
runs in the HIP library; nothing here computes.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libapexw.so")

APEXW_OK = 0
APEXW_EINVAL = -1
APEXW_EDTYPE = -2
APEXW_ENOSPC = -3
APEXW_EHIP = -4
APEXW_ENOMEM = -5
APEXW_ESPARSE = -6

APEXW_F32 = 0
APEXW_BF16 = 1

APEXW_STATE_F32 = 0
APEXW_STATE_BF16 = 1
APEXW_STATE_Q8 = 2

APEXW_Q8_BLOCK = 256
APEXW_MAX_GROUPS = 32

# the entry points include/apexw.h declares
ENTRY_POINTS = (
    "apexw_state_bytes", "apexw_state_layout", "apexw_workspace_bytes",
    "apexw_create", "apexw_step", "apexw_step_scaled", "apexw_inv_scale", "apexw_unscale_check",
    "apexw_step_device", "apexw_step_ex", "apexw_clip_grad_norm", "apexw_clip_grad_norm_noalloc",
    "apexw_export_bytes", "apexw_export_state", "apexw_import_state",
    "apexw_read_steps", "apexw_launch_info", "apexw_set_workgroups",
    "apexw_set_occupancy", "apexw_get_occupancy", "apexw_set_cache_policy",
    "apexw_set_launch_mode", "apexw_get_launch_mode", "apexw_destroy", "apexw_last_error",
)


class ApexwError(RuntimeError):
    def __init__(self, code: int, where: str, message: str):
        super().__init__("%s failed (%d): %s" % (where, code, message))
        self.code = code


class apexw_group(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double)]


class apexw_step_options(ctypes.Structure):
    _fields_ = [("inv_scale", ctypes.c_void_p), ("clip_coef", ctypes.c_void_p),
                ("found_inf", ctypes.c_void_p), ("groups_dev", ctypes.c_void_p)]


class apexw_tensor_state(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int64), ("v", ctypes.c_int64),
                ("m_scale", ctypes.c_int64), ("v_scale", ctypes.c_int64)]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libapexw.so; a missing build is an error, never a fallback."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                "libapexw.so is not built (expected at %s); build it with "
                "`python -m tensor_adamw_optimizer_amd.build` or "
                "__graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.apexw_state_bytes.argtypes = [I32, P, I32, ctypes.POINTER(SZ)]
        L.apexw_state_layout.argtypes = [I32, P, I32, P, ctypes.POINTER(ctypes.c_int64)]
        L.apexw_workspace_bytes.argtypes = [I32, P, ctypes.POINTER(SZ)]
        L.apexw_create.argtypes = [I32, P, P, P, P, I32, I32, P, SZ, P, SZ, P,
                                   ctypes.POINTER(P)]
        L.apexw_step.argtypes = [P, P, I32, P, P, P, P]
        L.apexw_step_scaled.argtypes = [P, P, I32, P, P, P, P, P]
        L.apexw_inv_scale.argtypes = [P, P, P]
        L.apexw_unscale_check.argtypes = [P, P, P, P, P]
        L.apexw_step_device.argtypes = [P, P, I32, P, P, P, P, P]
        L.apexw_step_ex.argtypes = [P, P, I32, P, P, P, P]
        L.apexw_clip_grad_norm.argtypes = [P, P, P, ctypes.c_double, P, P, P, P]
        L.apexw_clip_grad_norm_noalloc.argtypes = [P, P, P, ctypes.c_double, P, P, P, P]
        L.apexw_export_bytes.argtypes = [P, ctypes.POINTER(SZ)]
        L.apexw_export_state.argtypes = [P, P, I32, P, SZ, P]
        L.apexw_import_state.argtypes = [P, P, SZ, P, I32, P]
        L.apexw_read_steps.argtypes = [P, P, P]
        L.apexw_launch_info.argtypes = [P, ctypes.POINTER(I32), ctypes.POINTER(I32),
                                        ctypes.POINTER(I32)]
        L.apexw_set_workgroups.argtypes = [P, I32]
        L.apexw_set_occupancy.argtypes = [P, I32]
        L.apexw_get_occupancy.argtypes = [P, ctypes.POINTER(I32)]
        L.apexw_set_cache_policy.argtypes = [P, I32]
        L.apexw_set_launch_mode.argtypes = [P, I32]
        L.apexw_get_launch_mode.argtypes = [P, ctypes.POINTER(I32)]
        L.apexw_destroy.argtypes = [P]
        L.apexw_last_error.argtypes = []
        L.apexw_last_error.restype = ctypes.c_char_p
        for name in ENTRY_POINTS[:-1]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, where: str) -> None:
    if rc != APEXW_OK:
        msg = lib().apexw_last_error().decode(errors="replace")
        raise ApexwError(rc, where, msg)


def _i64(values: Sequence[int]):
    return (ctypes.c_int64 * max(1, len(values)))(*values)


def _i32(values: Sequence[int]):
    return (ctypes.c_int32 * max(1, len(values)))(*values)


def apexw_last_error() -> str:
    return lib().apexw_last_error().decode(errors="replace")


def apexw_state_bytes(numel: Sequence[int], fmt: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().apexw_state_bytes(len(numel), _i64(numel), fmt, ctypes.byref(out)),
           "apexw_state_bytes")
    return out.value


def apexw_state_layout(numel: Sequence[int], fmt: int):
    """Returns ([(m, v, m_scale, v_scale) byte offsets per tensor], steps offset)."""
    arr = (apexw_tensor_state * max(1, len(numel)))()
    steps = ctypes.c_int64(0)
    _check(lib().apexw_state_layout(len(numel), _i64(numel), fmt, arr, ctypes.byref(steps)),
           "apexw_state_layout")
    return [(a.m, a.v, a.m_scale, a.v_scale) for a in arr[:len(numel)]], steps.value


def apexw_workspace_bytes(numel: Sequence[int]) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().apexw_workspace_bytes(len(numel), _i64(numel), ctypes.byref(out)),
           "apexw_workspace_bytes")
    return out.value


def apexw_create(numel: Sequence[int], param_dtype: Sequence[int], grad_dtype: Sequence[int],
                 group_of: Sequence[int], n_groups: int, fmt: int, state_ptr: int,
                 state_bytes: int, workspace_ptr: int, workspace_bytes: int,
                 stream: int = 0) -> int:
    h = ctypes.c_void_p(0)
    _check(lib().apexw_create(len(numel), _i64(numel), _i32(param_dtype), _i32(grad_dtype),
                              _i32(group_of), n_groups, fmt, state_ptr, state_bytes,
                              workspace_ptr, workspace_bytes, stream, ctypes.byref(h)),
           "apexw_create")
    return h.value


def make_groups(groups) -> ctypes.Array:
    """ctypes apexw_group[] from objects with lr/beta1/beta2/eps/weight_decay."""
    arr = (apexw_group * max(1, len(groups)))()
    for i, g in enumerate(groups):
        arr[i] = apexw_group(g.lr, g.beta1, g.beta2, g.eps, g.weight_decay)
    return arr


def make_ptrs(ptrs: Sequence[int]) -> ctypes.Array:
    """ctypes void*[] from ints (0 = NULL)."""
    return (ctypes.c_void_p * max(1, len(ptrs)))(*[p or None for p in ptrs])


class ptr_table:
    """A void*[] over an array('Q') of addresses (0 = NULL), passed to the
    library without a per-element conversion; keeps the array alive."""

    def __init__(self, ptrs: "array"):
        if ptrs.itemsize != 8:
            raise TypeError("ptr_table needs 64-bit addresses")
        self._a = ptrs if len(ptrs) else type(ptrs)("Q", [0])
        self._as_parameter_ = ctypes.c_void_p(self._a.buffer_info()[0])


def apexw_step(handle: int, groups_arr, n_groups: int, params_arr, grads_arr,
               found_inf_ptr: int = 0, stream: int = 0) -> None:
    """groups_arr / params_arr / grads_arr: arrays from make_groups / make_ptrs."""
    _check(lib().apexw_step(handle, groups_arr, n_groups, params_arr, grads_arr,
                            found_inf_ptr or None, stream or None), "apexw_step")


def apexw_step_scaled(handle: int, groups_arr, n_groups: int, params_arr, grads_arr,
                      inv_scale_ptr: int = 0, found_inf_ptr: int = 0, stream: int = 0) -> None:
    _check(lib().apexw_step_scaled(handle, groups_arr, n_groups, params_arr, grads_arr,
                                   inv_scale_ptr or None, found_inf_ptr or None, stream or None),
           "apexw_step_scaled")


def apexw_inv_scale(scale_ptr: int, inv_scale_ptr: int, stream: int = 0) -> None:
    """Device float at inv_scale_ptr = fp64 reciprocal of the one at scale_ptr."""
    _check(lib().apexw_inv_scale(scale_ptr or None, inv_scale_ptr or None, stream or None),
           "apexw_inv_scale")


def apexw_unscale_check(handle: int, grads_arr, inv_scale_ptr: int, found_inf_ptr: int,
                        stream: int = 0) -> None:
    _check(lib().apexw_unscale_check(handle, grads_arr, inv_scale_ptr or None,
                                     found_inf_ptr or None, stream or None),
           "apexw_unscale_check")


def apexw_step_device(handle: int, groups_dev_ptr: int, n_groups: int, params_arr, grads_arr,
                      inv_scale_ptr: int = 0, found_inf_ptr: int = 0, stream: int = 0) -> None:
    """groups_dev_ptr: device address of n_groups apexw_group records."""
    _check(lib().apexw_step_device(handle, groups_dev_ptr, n_groups, params_arr, grads_arr,
                                   inv_scale_ptr or None, found_inf_ptr or None, stream or None),
           "apexw_step_device")


def apexw_step_ex(handle: int, groups_arr, n_groups: int, params_arr, grads_arr,
                  inv_scale_ptr: int = 0, clip_coef_ptr: int = 0, found_inf_ptr: int = 0,
                  groups_dev_ptr: int = 0, stream: int = 0) -> None:
    """groups_arr may be None when groups_dev_ptr is given."""
    o = apexw_step_options(inv_scale_ptr or None, clip_coef_ptr or None, found_inf_ptr or None,
                           groups_dev_ptr or None)
    _check(lib().apexw_step_ex(handle, groups_arr, n_groups, params_arr, grads_arr,
                               ctypes.byref(o), stream or None), "apexw_step_ex")


def apexw_clip_grad_norm(handle: int, grads_arr, inv_scale_ptr: int, max_norm: float,
                         found_inf_ptr: int, norm_out_ptr: int, clip_coef_ptr: int,
                         stream: int = 0) -> None:
    _check(lib().apexw_clip_grad_norm(handle, grads_arr, inv_scale_ptr or None, max_norm,
                                      found_inf_ptr or None, norm_out_ptr or None,
                                      clip_coef_ptr or None, stream or None),
           "apexw_clip_grad_norm")


def apexw_clip_grad_norm_noalloc(handle: int, grads_arr, inv_scale_ptr: int, max_norm: float,
                                 found_inf_ptr: int, norm_out_ptr: int, clip_coef_ptr: int,
                                 stream: int = 0) -> None:
    _check(lib().apexw_clip_grad_norm_noalloc(handle, grads_arr, inv_scale_ptr or None, max_norm,
                                              found_inf_ptr or None, norm_out_ptr or None,
                                              clip_coef_ptr or None, stream or None),
           "apexw_clip_grad_norm_noalloc")


def apexw_export_bytes(handle: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().apexw_export_bytes(handle, ctypes.byref(out)), "apexw_export_bytes")
    return out.value


def apexw_export_state(handle: int, groups_arr, n_groups: int, stream: int = 0) -> bytes:
    """The checkpoint blob as bytes."""
    size = apexw_export_bytes(handle)
    buf = ctypes.create_string_buffer(size)
    _check(lib().apexw_export_state(handle, groups_arr, n_groups, buf, size, stream or None),
           "apexw_export_state")
    return buf.raw


def apexw_import_state(handle: int, blob: bytes, n_groups: int, stream: int = 0):
    """Load a blob; returns the recipe as a list of apexw_group records."""
    groups = (apexw_group * max(1, n_groups))()
    _check(lib().apexw_import_state(handle, blob, len(blob), groups, n_groups, stream or None),
           "apexw_import_state")
    return list(groups[:n_groups])


def apexw_read_steps(handle: int, n_tensors: int, stream: int = 0):
    """The int32 step counter of every tensor, copied to the host (syncs)."""
    out = (ctypes.c_int32 * max(1, n_tensors))()
    _check(lib().apexw_read_steps(handle, out, stream or None), "apexw_read_steps")
    return list(out)[:n_tensors]


def apexw_launch_info(handle: int):
    te, nt, wg = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    _check(lib().apexw_launch_info(handle, ctypes.byref(te), ctypes.byref(nt), ctypes.byref(wg)),
           "apexw_launch_info")
    return te.value, nt.value, wg.value


def apexw_set_workgroups(handle: int, workgroups: int) -> None:
    _check(lib().apexw_set_workgroups(handle, workgroups), "apexw_set_workgroups")


def apexw_set_occupancy(handle: int, workgroups_per_cu: int) -> None:
    _check(lib().apexw_set_occupancy(handle, workgroups_per_cu), "apexw_set_occupancy")


def apexw_get_occupancy(handle: int) -> int:
    out = ctypes.c_int32(0)
    _check(lib().apexw_get_occupancy(handle, ctypes.byref(out)), "apexw_get_occupancy")
    return out.value


def apexw_set_cache_policy(handle: int, policy: int) -> None:
    _check(lib().apexw_set_cache_policy(handle, policy), "apexw_set_cache_policy")


def apexw_set_launch_mode(handle: int, mode: int) -> None:
    _check(lib().apexw_set_launch_mode(handle, mode), "apexw_set_launch_mode")


def apexw_get_launch_mode(handle: int) -> int:
    m = ctypes.c_int32(0)
    _check(lib().apexw_get_launch_mode(handle, ctypes.byref(m)), "apexw_get_launch_mode")
    return m.value


def apexw_destroy(handle: int) -> None:
    _check(lib().apexw_destroy(handle), "apexw_destroy")
