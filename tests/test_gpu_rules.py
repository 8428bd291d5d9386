"""Hardware rules the library relies on, checked exhaustively on the GPU.

The bf16 narrowing of theta and of bf16 moments is one v_cvt_pk_bf16_f32 per
pair of values (pack_bf16x2 in the kernel header).  tests/rules/bf16_all.hip
runs that function on every one of the 2^32 fp32 bit patterns and counts
the results that differ from round-to-nearest-even (and, for a NaN, from the
quiet NaN with the input's sign and top payload bits) -- the rule the oracle
implements on the host.
"""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "tests", "rules", "libbf16_all.so")


def test_bf16_conversion_matches_round_to_nearest_even_on_every_input():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    torch.cuda.init()
    if not os.path.exists(LIB):
        raise RuntimeError("tests/rules/libbf16_all.so is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB)
    lib.bf16_check_all.restype = ctypes.c_int
    lib.bf16_check_all.argtypes = [ctypes.POINTER(ctypes.c_ulonglong)] * 3
    print("case: bf16 conversion of all 2^32 fp32 inputs", flush=True)
    count, first, seen = ctypes.c_ulonglong(7), ctypes.c_ulonglong(0), ctypes.c_ulonglong(0)
    rc = lib.bf16_check_all(ctypes.byref(count), ctypes.byref(first), ctypes.byref(seen))
    assert rc == 0, "HIP error %d" % rc
    assert seen.value == 1 << 32
    assert count.value == 0, "%d inputs differ, the first 0x%08x" % (count.value, first.value)
