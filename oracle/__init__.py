"""The oracle -- TEST INFRASTRUCTURE ONLY.

A ctypes wrapper around ``apexw_oracle.c``, the plain scalar CPU definition of
the fused multi-tensor AdamW step, plus ``ref64`` (an fp64 restatement used to
pin it).  Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package.  It shares no code with the HIP
library, and the HIP library never calls it.

Arrays are numpy: fp32 values as ``float32``, bf16 values as their ``uint16``
bit patterns, 8-bit codes as ``int8`` (m) / ``uint8`` (v), block scales as
``float32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Optional, Sequence

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "apexw_oracle.c")
LIB_PATH = os.path.join(HERE, "liboracle.so")
# the same source built with OpenMP: a timing build for the host baseline
OMP_LIB_PATH = os.path.join(HERE, "liboracle_omp.so")

F32, BF16 = 0, 1
STATE_F32, STATE_BF16, STATE_Q8 = 0, 1, 2
BLOCK = 256

DTYPE_CODE = {"f32": F32, "bf16": BF16}
STATE_CODE = {"f32": STATE_F32, "bf16": STATE_BF16, "q8": STATE_Q8}


class Group(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("beta1", ctypes.c_double),
                ("beta2", ctypes.c_double), ("eps", ctypes.c_double),
                ("weight_decay", ctypes.c_double)]


def _compile(path: str, extra, force: bool) -> str:
    if force or not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
        tmp = path + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off",
                               "-fno-fast-math", "-fPIC", "-shared", "-Wall",
                               *extra, "-o", tmp, SRC, "-lm"])
        os.replace(tmp, path)
    return path


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no contraction, no fast-math): the
    single-threaded parity build, and the OpenMP timing build of the same
    source."""
    _compile(OMP_LIB_PATH, ["-fopenmp"], force)
    return _compile(LIB_PATH, ["-Wno-unknown-pragmas"], force)


_lib = None


def load(path: str) -> ctypes.CDLL:
    """Open a build of the oracle at ``path`` and declare its signatures."""
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    L.oracle_bf16_to_f32.restype = ctypes.c_float
    L.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    L.oracle_f32_to_bf16.restype = ctypes.c_uint16
    L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
    L.oracle_f32_to_bf16_array.restype = None
    L.oracle_f32_to_bf16_array.argtypes = [ctypes.c_int64, P, P]
    L.oracle_pow_int.restype = ctypes.c_double
    L.oracle_pow_int.argtypes = [ctypes.c_double, ctypes.c_int32]
    for name in ("oracle_quantize_signed", "oracle_quantize_unsigned"):
        getattr(L, name).restype = None
        getattr(L, name).argtypes = [ctypes.c_int64, P, P, P]
    for name in ("oracle_dequantize_signed", "oracle_dequantize_unsigned"):
        getattr(L, name).restype = None
        getattr(L, name).argtypes = [ctypes.c_int64, P, ctypes.c_float, P]
    L.oracle_adamw_step.restype = ctypes.c_int32
    L.oracle_adamw_step.argtypes = [
        ctypes.c_int32, P, P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32,
        P, P, P, P, P, ctypes.c_int32]
    L.oracle_adamw_step_scaled.restype = ctypes.c_int32
    L.oracle_adamw_step_scaled.argtypes = [
        ctypes.c_int32, P, P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32,
        P, P, P, P, P, ctypes.c_float, ctypes.c_int32]
    L.oracle_adamw_step_clipped.restype = ctypes.c_int32
    L.oracle_adamw_step_clipped.argtypes = [
        ctypes.c_int32, P, P, P, P, P, P, P, ctypes.c_int32, ctypes.c_int32,
        P, P, P, P, P, ctypes.c_float, ctypes.c_float, ctypes.c_int32]
    L.oracle_grad_norm.restype = ctypes.c_double
    L.oracle_grad_norm.argtypes = [ctypes.c_int32, P, P, P, ctypes.c_float]
    L.oracle_clip_coef.restype = ctypes.c_float
    L.oracle_clip_coef.argtypes = [ctypes.c_double, ctypes.c_double]
    L.oracle_unscale_check.restype = ctypes.c_int32
    L.oracle_unscale_check.argtypes = [ctypes.c_int32, P, P, P, ctypes.c_float]
    L.oracle_threads.restype = ctypes.c_int32
    L.oracle_threads.argtypes = []
    L.oracle_adamw_step_three_loops.restype = ctypes.c_int32
    L.oracle_adamw_step_three_loops.argtypes = [
        ctypes.c_int32, P, P, P, P, P, ctypes.c_int32, P, P, P,
        ctypes.c_int32]
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        _lib = load(LIB_PATH)
    return _lib


_omp_lib = None


def omp_lib():
    """The OpenMP timing build (same source, same results)."""
    global _omp_lib
    if _omp_lib is None:
        if not os.path.exists(OMP_LIB_PATH):
            build()
        _omp_lib = load(OMP_LIB_PATH)
    return _omp_lib


def _ptr(a: Optional[np.ndarray]) -> int:
    return 0 if a is None else a.ctypes.data


def _ptr_array(arrs: Sequence[Optional[np.ndarray]]):
    # a present but empty array still needs a non-NULL pointer ("present")
    return (ctypes.c_void_p * max(1, len(arrs)))(
        *[None if a is None else (_ptr(a) or 16) for a in arrs])


def _groups(groups) -> ctypes.Array:
    arr = (Group * max(1, len(groups)))()
    for i, g in enumerate(groups):
        arr[i] = Group(g.lr, g.beta1, g.beta2, g.eps, g.weight_decay)
    return arr


# ---------------------------------------------------------------- scalars

def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    out = np.zeros(x.size, dtype=np.uint16)
    lib().oracle_f32_to_bf16_array(x.size, _ptr(x), _ptr(out))
    return out


def pow_int(base: float, e: int) -> float:
    return lib().oracle_pow_int(base, e)


def quantize_signed(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.zeros(x.size, dtype=np.int8)
    s = np.zeros(1, dtype=np.float32)
    lib().oracle_quantize_signed(x.size, _ptr(x), _ptr(q), _ptr(s))
    return q, float(s[0])


def quantize_unsigned(x: np.ndarray):
    x = np.ascontiguousarray(x, dtype=np.float32)
    q = np.zeros(x.size, dtype=np.uint8)
    s = np.zeros(1, dtype=np.float32)
    lib().oracle_quantize_unsigned(x.size, _ptr(x), _ptr(q), _ptr(s))
    return q, float(s[0])


def dequantize_signed(q: np.ndarray, scale: float) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.int8)
    x = np.zeros(q.size, dtype=np.float32)
    lib().oracle_dequantize_signed(q.size, _ptr(q), scale, _ptr(x))
    return x


def dequantize_unsigned(q: np.ndarray, scale: float) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8)
    x = np.zeros(q.size, dtype=np.float32)
    lib().oracle_dequantize_unsigned(q.size, _ptr(q), scale, _ptr(x))
    return x


# ---------------------------------------------------------------- optimizer

class OracleAdamW:
    """Multi-tensor AdamW state held on the host, updated by the C oracle.

    ``numels``, ``param_dtype``/``grad_dtype`` ("f32"/"bf16" per tensor),
    ``group_of`` (group index per tensor) and ``state_fmt`` ("f32", "bf16",
    "q8") fix the layout.  State starts at zero (m = v = 0, t = 0; 8-bit codes
    and scales 0).
    """

    def __init__(self, numels: Sequence[int], param_dtype: Sequence[str],
                 grad_dtype: Sequence[str], group_of: Sequence[int],
                 state_fmt: str, threaded: bool = False):
        # threaded: step with the OpenMP timing build (bitwise the same)
        self._threaded = threaded
        self.numels = [int(n) for n in numels]
        self.n = len(self.numels)
        self.param_dtype = list(param_dtype)
        self.grad_dtype = list(grad_dtype)
        self.group_of = list(group_of)
        self.state_fmt = state_fmt
        self.t = np.zeros(max(1, self.n), dtype=np.int32)
        self.m: List[np.ndarray] = []
        self.v: List[np.ndarray] = []
        self.m_scale: List[Optional[np.ndarray]] = []
        self.v_scale: List[Optional[np.ndarray]] = []
        for n in self.numels:
            nb = (n + BLOCK - 1) // BLOCK
            if state_fmt == "f32":
                self.m.append(np.zeros(n, np.float32))
                self.v.append(np.zeros(n, np.float32))
                self.m_scale.append(None)
                self.v_scale.append(None)
            elif state_fmt == "bf16":
                self.m.append(np.zeros(n, np.uint16))
                self.v.append(np.zeros(n, np.uint16))
                self.m_scale.append(None)
                self.v_scale.append(None)
            elif state_fmt == "q8":
                self.m.append(np.zeros(n, np.int8))
                self.v.append(np.zeros(n, np.uint8))
                self.m_scale.append(np.zeros(nb, np.float32))
                self.v_scale.append(np.zeros(nb, np.float32))
            else:
                raise ValueError(state_fmt)
        self._numel = np.array(self.numels or [0], dtype=np.int64)
        self._pdt = np.array([DTYPE_CODE[d] for d in self.param_dtype] or [0],
                             dtype=np.int32)
        self._gdt = np.array([DTYPE_CODE[d] for d in self.grad_dtype] or [0],
                             dtype=np.int32)
        self._grp = np.array(self.group_of or [0], dtype=np.int32)

    def moments_f32(self, i: int):
        """Decoded (m, v) of tensor i as fp32 arrays."""
        if self.state_fmt == "f32":
            return self.m[i].copy(), self.v[i].copy()
        if self.state_fmt == "bf16":
            return bf16_to_f32(self.m[i]), bf16_to_f32(self.v[i])
        n = self.numels[i]
        m = np.zeros(n, np.float32)
        v = np.zeros(n, np.float32)
        for b in range((n + BLOCK - 1) // BLOCK):
            lo, hi = b * BLOCK, min(n, (b + 1) * BLOCK)
            m[lo:hi] = dequantize_signed(self.m[i][lo:hi], float(self.m_scale[i][b]))
            v[lo:hi] = dequantize_unsigned(self.v[i][lo:hi], float(self.v_scale[i][b]))
        return m, v

    def unscale_check(self, grads: Sequence[Optional[np.ndarray]],
                      inv_scale: float) -> bool:
        """True if any present grad value times inv_scale (fp32) is not finite."""
        assert len(grads) == self.n
        return bool(lib().oracle_unscale_check(self.n, _ptr(self._numel), _ptr(self._gdt),
                                               _ptr_array(grads), inv_scale))

    def grad_norm(self, grads: Sequence[Optional[np.ndarray]], inv_scale: float = 1.0) -> float:
        """Euclidean norm of the unscaled present grads (fp64 accumulation)."""
        assert len(grads) == self.n
        return lib().oracle_grad_norm(self.n, _ptr(self._numel), _ptr(self._gdt),
                                      _ptr_array(grads), inv_scale)

    @staticmethod
    def clip_coef(norm: float, max_norm: float) -> float:
        return lib().oracle_clip_coef(norm, max_norm)

    def step(self, thetas: Sequence[np.ndarray],
             grads: Sequence[Optional[np.ndarray]], groups,
             found_inf: bool = False, inv_scale: Optional[float] = None,
             clip_coef: Optional[float] = None) -> None:
        """Update ``thetas`` (in place) and the held state by one call; with
        ``inv_scale`` the grads are unscaled (g * inv_scale in fp32) first,
        with ``clip_coef`` the unscaled grads are then multiplied by it."""
        assert len(thetas) == self.n and len(grads) == self.n
        for i, th in enumerate(thetas):
            want = np.uint16 if self.param_dtype[i] == "bf16" else np.float32
            assert th.dtype == want and th.flags.c_contiguous and th.size == self.numels[i]
            g = grads[i]
            if g is not None:
                want = np.uint16 if self.grad_dtype[i] == "bf16" else np.float32
                assert g.dtype == want and g.flags.c_contiguous and g.size == self.numels[i]
        args = (self.n, _ptr(self._numel), _ptr(self._pdt), _ptr_array(thetas),
                _ptr(self._gdt), _ptr_array(grads), _ptr(self._grp),
                _groups(groups), len(groups), STATE_CODE[self.state_fmt],
                _ptr_array(self.m), _ptr_array(self.v), _ptr_array(self.m_scale),
                _ptr_array(self.v_scale), _ptr(self.t))
        L = omp_lib() if self._threaded else lib()
        if inv_scale is None and clip_coef is None:
            rc = L.oracle_adamw_step(*args, int(bool(found_inf)))
        elif clip_coef is None:
            rc = L.oracle_adamw_step_scaled(*args, inv_scale, int(bool(found_inf)))
        else:
            rc = L.oracle_adamw_step_clipped(
                *args, 1.0 if inv_scale is None else inv_scale, clip_coef, int(bool(found_inf)))
        if rc != 0:
            raise ValueError("oracle_adamw_step rejected its arguments")

    def step_three_loops(self, thetas, grads, groups, found_inf=False) -> None:
        """fp32-only three-separate-loops form of the same step."""
        assert self.state_fmt == "f32"
        assert all(d == "f32" for d in self.param_dtype + self.grad_dtype)
        rc = lib().oracle_adamw_step_three_loops(
            self.n, _ptr(self._numel), _ptr_array(thetas), _ptr_array(grads),
            _ptr(self._grp), _groups(groups), len(groups), _ptr_array(self.m),
            _ptr_array(self.v), _ptr(self.t), int(bool(found_inf)))
        if rc != 0:
            raise ValueError("oracle_adamw_step_three_loops rejected its arguments")
