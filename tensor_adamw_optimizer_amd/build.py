"""Build step of the HIP library: compiles csrc/apexw.hip for gfx950 into
``libapexw.so`` next to this file (in-tree, so it travels with the sources).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "apexw.hip")
DEPS = [SRC, os.path.join(HERE, "csrc", "apexw_kernels.hpp"),
        os.path.join(HERE, "csrc", "apexw_plan.hpp"), os.path.join(ROOT, "include", "apexw.h")]
LIB = os.path.join(HERE, "libapexw.so")
ARCH = os.environ.get("APEXW_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    "--offload-arch=" + ARCH,
    # every fp32 operation separately rounded: no FMA contraction, correctly
    # rounded division and square root, denormals kept
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    # packed fp32 instructions are not generated
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", *FLAGS, "-I", os.path.join(ROOT, "include"), "-o", tmp, SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops" not in l)   # host pass: unknown feature
    if res.returncode != 0:
        if os.path.exists(tmp):
            os.remove(tmp)
        raise RuntimeError("hipcc failed:\n" + out)
    if out.strip() and verbose:
        print(out)
    os.replace(tmp, LIB)
    return LIB


RULES = os.path.join(ROOT, "tests", "rules")
CHECKS = [(os.path.join(RULES, src), os.path.join(RULES, lib))
          for src, lib in (("bf16_all.hip", "libbf16_all.so"),
                           ("rcp_sqrt_all.hip", "librcp_sqrt_all.so"))]


def build_checks(verbose: bool = False) -> list:
    """The test-only device checks of the kernel header's conversion,
    square root, reciprocal and short division (tests/rules), each its own
    library (each includes the kernel header), built with the library's
    flags."""
    built = []
    for src, lib in CHECKS:
        tmp = lib + ".tmp%d" % os.getpid()
        cmd = ["hipcc", *FLAGS, "-I", os.path.join(ROOT, "include"), "-I",
               os.path.join(HERE, "csrc"), "-o", tmp, src]
        if verbose:
            print(" ".join(cmd), flush=True)
        res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if res.returncode != 0:
            if os.path.exists(tmp):
                os.remove(tmp)
            raise RuntimeError("hipcc failed:\n" + res.stdout)
        os.replace(tmp, lib)
        built.append(lib)
    return built


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(d) > t for d in DEPS)


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
