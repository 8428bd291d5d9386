"""The launch plan on the CPU (no GPU): tests/plan/plan_check.cpp, compiled
with g++ against the library's plan header under AddressSanitizer and
UndefinedBehaviorSanitizer, checks on random tensor lists -- empty lists,
empty and 1-element tensors, every mix of dtype pairs, and a 20,000-tensor
list -- that the tiles cover every element exactly once, that the XCD-major
table position is one-to-one onto the padded stripes, that every read
group's 4-entry load stays inside the reserved table, and that the 8-bit
kernel's workgroup-to-pair order takes every pair once, in runs per XCD."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "plan", "plan_check.cpp")
CSRC = os.path.join(ROOT, "tensor_adamw_optimizer_amd", "csrc")


def _build(tmp_path, sanitize: bool) -> str:
    if shutil.which("g++") is None:
        pytest.skip("g++ is not installed")
    exe = str(tmp_path / ("plan_check_san" if sanitize else "plan_check"))
    flags = ["-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-I", CSRC]
    if sanitize:
        flags += ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                  "-fno-omit-frame-pointer"]
    subprocess.check_call(["g++", *flags, "-o", exe, SRC])
    return exe


@pytest.mark.parametrize("seed", [1, 2])
def test_plan_under_sanitizers(tmp_path, seed):
    exe = _build(tmp_path, sanitize=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe, "300", str(seed)], stdout=subprocess.PIPE,
                         stderr=subprocess.STDOUT, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout[-4000:]
    assert res.stdout.strip().endswith("ok"), res.stdout[-2000:]


@pytest.mark.parametrize("old, new", [
    # the table position drops the stride: stripes collide
    ("return table_begin + (int64_t)(uk % kXcds) * stride + (int64_t)(uk / kXcds);",
     "return table_begin + (int64_t)(uk % kXcds) + (int64_t)(uk / kXcds);"),
    # the pair order drops the position within a run: pairs taken twice
    ("return w - r + (r % (uint32_t)kXcds) * kQ8PairRun + r / (uint32_t)kXcds;",
     "return w - r + (r % (uint32_t)kXcds) * kQ8PairRun;"),
    # the pair order is the identity: one-to-one, but no runs per XCD
    ("if (w >= P / W * W) return w;", "return w;"),
])
def test_plan_check_detects_a_broken_plan(tmp_path, old, new):
    """The checker itself: a plan header with one of these mistakes must fail it."""
    broken = tmp_path / "apexw_plan.hpp"
    text = open(os.path.join(CSRC, "apexw_plan.hpp")).read()
    assert text.count(old) == 1
    broken.write_text(text.replace(old, new))
    exe = str(tmp_path / "plan_check_broken")
    subprocess.check_call(["g++", "-std=c++17", "-O1", "-I", str(tmp_path), "-o", exe, SRC])
    res = subprocess.run([exe, "50", "3"], stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                         text=True, timeout=300)
    assert res.returncode != 0 and "FAIL" in res.stdout
