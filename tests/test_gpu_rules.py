"""Hardware rules the library relies on, checked exhaustively on the GPU.

tests/rules/bf16_all.hip: the bf16 narrowing of theta and of bf16 moments is
one v_cvt_pk_bf16_f32 per pair of values (pack_bf16x2 in the kernel header);
the check runs that function on every one of the 2^32 fp32 bit patterns and
counts the results that differ from round-to-nearest-even (and, for a NaN,
from the quiet NaN with the input's sign and top payload bits) -- the rule
the oracle implements on the host.

tests/rules/rcp_sqrt_all.hip: the update's square root (sqrt_rn: v_sqrt_f32
plus one residual correction with v_rsq_f32) on every fp32 input in [2^-96,
2^64) and its reciprocal (rcp_rn: v_rcp_f32 plus one Newton step) on every
fp32 input in [2^-126, 2^126], each against an exact fp64 test of the
nearest result, and v_rcp_f32 alone within one ulp on that range (the 8-bit
encoding's tie guard assumes it); and the short division by that reciprocal against IEEE
division on 2^32 hashed operand pairs of the ranges the update admits.
"""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RULES = os.path.join(ROOT, "tests", "rules")


def _lib(name):
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.init()
    path = os.path.join(RULES, name)
    if not os.path.exists(path):
        raise RuntimeError("tests/rules/%s is not built; run __graft_entry__.build()" % name)
    return ctypes.CDLL(path)


def test_bf16_conversion_matches_round_to_nearest_even_on_every_input():
    lib = _lib("libbf16_all.so")
    lib.bf16_check_all.restype = ctypes.c_int
    lib.bf16_check_all.argtypes = [ctypes.POINTER(ctypes.c_ulonglong)] * 3
    print("case: bf16 conversion of all 2^32 fp32 inputs", flush=True)
    count, first, seen = ctypes.c_ulonglong(7), ctypes.c_ulonglong(0), ctypes.c_ulonglong(0)
    rc = lib.bf16_check_all(ctypes.byref(count), ctypes.byref(first), ctypes.byref(seen))
    assert rc == 0, "HIP error %d" % rc
    assert seen.value == 1 << 32
    assert count.value == 0, "%d inputs differ, the first 0x%08x" % (count.value, first.value)


def test_sqrt_reciprocal_and_short_division_are_correctly_rounded():
    lib = _lib("librcp_sqrt_all.so")
    lib.rcp_sqrt_check_all.restype = ctypes.c_int
    lib.rcp_sqrt_check_all.argtypes = [ctypes.POINTER(ctypes.c_ulonglong)]
    print("case: sqrt_rn on [2^-96, 2^64), rcp_rn on [2^-126, 2^126], 2^32 short divisions",
          flush=True)
    out = (ctypes.c_ulonglong * 11)()
    rc = lib.rcp_sqrt_check_all(out)
    assert rc == 0, "HIP error %d" % rc
    sqrt_bad, sqrt_seen, rcp_bad, rcp_seen, div_bad, div_seen, raw_bad = list(out)[:7]
    assert sqrt_seen == 0x5F800000 - 0x0F800000          # every input of [2^-96, 2^64)
    assert rcp_seen == 0x7E800000 - 0x00800000 + 1       # every input of [2^-126, 2^126]
    assert div_seen == 1 << 32
    assert sqrt_bad == 0, "sqrt_rn: %d inputs differ, the first 0x%08x" % (sqrt_bad, out[7])
    assert rcp_bad == 0, "rcp_rn: %d inputs differ, the first 0x%08x" % (rcp_bad, out[8])
    assert div_bad == 0, "short division: %d pairs differ, the first pair %d" % (div_bad, out[9])
    assert raw_bad == 0, "v_rcp_f32: %d inputs an ulp or more off, the first 0x%08x" % (raw_bad, out[10])
