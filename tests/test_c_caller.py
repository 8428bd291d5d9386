"""The C ABI from a plain C99 program (tests/c_abi/caller.c, built with gcc
against include/apexw.h and libapexw.so, no C++ and no Python in the
caller).  CPU: sizes and error codes agree with the Python binding.  GPU:
the program runs a mixed-dtype list for several steps in each state format;
its recorded inputs go through the oracle and every result bit must match."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import workloads as W
from tensor_adamw_optimizer_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "caller.c")
LIBDIR = os.path.join(ROOT, "tensor_adamw_optimizer_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")

NUMEL = [1000, 4096, 77, 2560]
PDT = [W.F32, W.BF16, W.F32, W.BF16]
GDT = [W.F32, W.F32, W.BF16, W.BF16]
GROUP = [0, 1, 0, 1]
GROUPS = [W.Group(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
          W.Group(lr=3e-3, beta1=0.8, beta2=0.99, eps=1e-6, weight_decay=0.0)]
FMT = {0: W.STATE_F32, 1: W.STATE_BF16, 2: W.STATE_Q8}


def build_caller(tmp_path) -> str:
    L.lib()                                   # the library must be built
    exe = str(tmp_path / "caller")
    cmd = ["gcc", "-std=c99", "-O1", "-Wall", "-Wextra", "-Werror", "-pedantic-errors",
           "-I", os.path.join(ROOT, "include"), "-isystem", os.path.join(ROCM, "include"),
           "-D__HIP_PLATFORM_AMD__", SRC, "-o", exe, "-L", LIBDIR, "-lapexw",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath," + LIBDIR, "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout
    return exe


def test_c_caller_host_functions(tmp_path):
    exe = build_caller(tmp_path)
    out = subprocess.run([exe, "host"], stdout=subprocess.PIPE, text=True, timeout=60, check=True)
    kv = dict(line.split("=", 1) for line in out.stdout.splitlines())
    assert int(kv["state_bytes_q8"]) == L.apexw_state_bytes(NUMEL, L.APEXW_STATE_Q8)
    assert int(kv["state_bytes_f32"]) == L.apexw_state_bytes(NUMEL, L.APEXW_STATE_F32)
    assert int(kv["workspace_bytes"]) == L.apexw_workspace_bytes(NUMEL)
    assert int(kv["bad_fmt_rc"]) == L.APEXW_EDTYPE and "format" in kv["bad_fmt_msg"]
    assert int(kv["null_destroy_rc"]) == L.APEXW_EINVAL


def _read(f, n, dt):
    if dt == W.F32:
        return np.frombuffer(f.read(4 * n), dtype=np.float32).copy()
    return np.frombuffer(f.read(2 * n), dtype=np.uint16).copy()


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_c_caller_steps_match_the_oracle(tmp_path, fmt):
    exe = build_caller(tmp_path)
    steps = 5
    path = str(tmp_path / "run.bin")
    print("case: C caller fmt", fmt, flush=True)
    subprocess.run([exe, "gpu", path, str(fmt), str(steps)], timeout=120, check=True)
    code = {0: L.APEXW_STATE_F32, 1: L.APEXW_STATE_BF16, 2: L.APEXW_STATE_Q8}[fmt]
    sb = L.apexw_state_bytes(NUMEL, code)
    layout, steps_off = L.apexw_state_layout(NUMEL, code)
    ref = oracle.OracleAdamW(NUMEL, PDT, GDT, GROUP, FMT[fmt])
    with open(path, "rb") as f:
        th = [_read(f, n, d) for n, d in zip(NUMEL, PDT)]
        for _ in range(steps):
            g = [_read(f, n, d) for n, d in zip(NUMEL, GDT)]
            ref.step(th, g, GROUPS)
        th_gpu = [_read(f, n, d) for n, d in zip(NUMEL, PDT)]
        blob = np.frombuffer(f.read(sb), dtype=np.uint8)
        t = np.frombuffer(f.read(4 * len(NUMEL)), dtype=np.int32)
    for i in range(len(NUMEL)):
        assert np.array_equal(th_gpu[i].view(np.uint8), th[i].view(np.uint8)), i
        m_off, v_off, ms, vs = layout[i]
        eb = {0: 4, 1: 2, 2: 1}[fmt]
        m = blob[m_off:m_off + NUMEL[i] * eb]
        v = blob[v_off:v_off + NUMEL[i] * eb]
        assert np.array_equal(m, ref.m[i].view(np.uint8)), i
        assert np.array_equal(v, ref.v[i].view(np.uint8)), i
        if fmt == 2:
            nb = (NUMEL[i] + 255) // 256
            assert np.array_equal(blob[ms:ms + 4 * nb], ref.m_scale[i].view(np.uint8)), i
            assert np.array_equal(blob[vs:vs + 4 * nb], ref.v_scale[i].view(np.uint8)), i
    assert np.array_equal(blob[steps_off:steps_off + 4 * len(NUMEL)].view(np.int32), ref.t)
    assert list(t) == [steps] * len(NUMEL)
