"""CPU checks of the rounding shortcuts the update kernel takes instead of a
correctly rounded division or square root per element (code_value,
div_uniform and sqrt_rn in csrc/apexw_kernels.hpp), written out with IEEE
fp32 arithmetic (numpy, or C with libm's fmaf for the fused multiply-adds)
and checked against the definitions.  The hardware approximations they start
from (v_rcp_f32, v_sqrt_f32, v_rsq_f32: within one ulp) are modelled by
trying the correctly rounded value and both of its neighbours.  (The device
checks of tests/test_gpu_rules.py cover the hardware's own outputs, and the
GPU parity tests the kernel itself bit for bit against the oracle.)"""
import os
import subprocess

import numpy as np

F32 = np.float32


# the float just above 1/2 - 2.5e-4f (kTieBound in the kernel)
TIE_BOUND = np.array([0x3EFFDF3C], np.uint32).view(F32)[0]


def test_tie_bound_is_the_distance_test():
    """|d - 1/2| > 2.5e-4f (d = |r - rint(r)| in [0, 1/2], computed in fp32)
    holds exactly when d < TIE_BOUND, for every float d in [0, 1/2]."""
    d = np.arange(0, 0x3F000001, 61, dtype=np.uint32).view(F32)      # [0, 1/2], every 61st
    d = np.concatenate([d, np.array([0x3EFFDF3B, 0x3EFFDF3C, 0x3EFFDF3D, 0x3F000000],
                                    np.uint32).view(F32)])
    assert np.array_equal(np.abs(d - F32(0.5)) > F32(2.5e-4), d < TIE_BOUND)


def _neighbours(a):
    return (np.nextafter(a, F32(-np.inf)), a, np.nextafter(a, F32(np.inf)))


# ------------------------------------------------------------ 8-bit codes

def code_rule(x, s, inv, lo, hi):
    """The kernel's rule: r = x*inv rounded to even, unless the block scale
    is not a normal number or r is within 2.5e-4 of a half-integer (or NaN),
    tested as |r - rint(r)| < TIE_BOUND; then the correctly rounded
    quotient, rounded and clamped."""
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        fast = (s >= F32(2.0 ** -126)) & (s <= F32(2.0 ** 126))
        r = x * inv
        q = np.rint(r)
        exact = ~fast | ~(np.abs(r - q) < TIE_BOUND)
        slow = np.where(s == 0, F32(0), np.clip(np.rint(x / s), lo, hi))
        return np.where(exact, slow, q), exact


def code_definition(x, s, lo, hi):
    """The quantizer's definition (the oracle's): round-half-even of the
    correctly rounded quotient, clamped; scale 0 gives code 0."""
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        return np.where(s == 0, F32(0), np.clip(np.rint(x / s), lo, hi))


def check_codes(x, s, lo, hi):
    want = code_definition(x, s, lo, hi)
    frac = []
    with np.errstate(over="ignore", divide="ignore"):
        inv0 = (F32(1.0) / s).astype(F32)
    for inv in _neighbours(inv0):
        got, exact = code_rule(x, s, inv, lo, hi)
        assert np.array_equal(got, want)
        frac.append(exact.mean())
    return max(frac)


def test_random_blocks_match_the_definition():
    rng = np.random.default_rng(0)
    total_slow = 0.0
    for rep in range(10):
        n = 1_000_000
        amax = np.float32(np.exp(rng.uniform(-80, 80, n))).astype(F32)
        for levels, lo in ((F32(127.0), F32(-127.0)), (F32(255.0), F32(0.0))):
            s = (amax / levels).astype(F32)
            x = (amax * rng.uniform(-1, 1, n).astype(F32)).astype(F32)
            if lo == 0:
                x = np.abs(x)
            x[:1000] = amax[:1000]                         # the block maximum itself
            total_slow += check_codes(x, s, lo, levels)
    assert total_slow / 20 < 0.01


def test_near_ties_and_degenerate_scales_match_the_definition():
    rng = np.random.default_rng(1)
    n = 1_000_000
    s = np.float32(np.exp(rng.uniform(-60, 60, n))).astype(F32)
    k = rng.integers(-127, 127, n).astype(F32) + F32(0.5)
    x = (k.astype(np.float64) * s.astype(np.float64)).astype(F32)
    # walk a few ulps either side of each near-tie
    for step in range(-3, 4):
        xs = x
        for _ in range(abs(step)):
            xs = np.nextafter(xs, F32(np.inf) if step > 0 else F32(-np.inf))
        check_codes(xs, s, F32(-127.0), F32(127.0))
    # zero, denormal, tiny, huge and infinite scales, every code value
    for sv in (0.0, 1e-45, 1e-40, 1e-38, 3e-39, 1.2e-38, 1e38, 3e36, np.inf):
        with np.errstate(over="ignore"):     # 1e38 * code passes FLT_MAX: inf, on purpose
            xv = (np.float32(sv if np.isfinite(sv) else 1.0) * np.arange(-127, 128, dtype=F32)).astype(F32)
        check_codes(xv, np.full_like(xv, F32(sv)), F32(-127.0), F32(127.0))
        check_codes(np.abs(xv), np.full_like(xv, F32(sv)), F32(0.0), F32(255.0))


# ------------------------------------------------------------ square root

def test_sqrt_and_reciprocal_correction_models(tmp_path):
    """sqrt_rn: one correction fma(fma(-s, s, x), t/2, s) of s = v_sqrt_f32(x)
    with t = v_rsq_f32(x); rcp_rn: one Newton step y + y*(1 - b*y) of
    y = v_rcp_f32(b).  On the host, for every x of two binades and every b of
    one: exact from correctly rounded inputs; from one-ulp inputs, exact for
    all but a handful.  So neither rule is exact for every one-ulp
    approximation, and their exactness on gfx950 rests on the hardware's own
    outputs, which the device check (tests/test_gpu_rules.py, every input of
    the kernel's ranges) covers."""
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "rules", "rcp_sqrt_rule.c")
    exe = str(tmp_path / "rcp_sqrt_rule")
    subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-Wall", "-o", exe, src, "-lm"],
                   check=True)
    out = subprocess.run([exe], stdout=subprocess.PIPE, text=True, timeout=300, check=True).stdout
    bad = {line.split()[0]: [int(k) for k in line.split()[1:]] for line in out.strip().splitlines()}
    assert set(bad) == {"s-1", "s+0", "s+1", "rcp"}, out
    assert bad["s+0"][1] == 0 and bad["rcp"][1] == 0, out     # correctly rounded inputs: exact
    total = sum(sum(bad[k]) for k in ("s-1", "s+0", "s+1"))
    assert 0 < total < 100, out                          # one-ulp inputs: a handful of x fail
    assert 0 < sum(bad["rcp"]) < 100, out


def test_uniform_divisor_rule_against_ieee_division(tmp_path):
    """m/bc1 and v/bc2: y = 1/b correctly rounded, q = x*y, one correction
    with the exact residual; in range (2^-100 <= |x| < 2^64, b in
    [2^-60, 1]) it equals IEEE division on every significand of x in a
    binade (both signs) and on samples at the range ends, for bias
    corrections of common betas and random divisors; outside the range the
    short form differs for some x (zero's sign, subnormals, inf), which is
    why the kernel tests the range."""
    src = os.path.join(os.path.dirname(os.path.abspath(__file__)), "rules", "div_rule.c")
    exe = str(tmp_path / "div_rule")
    subprocess.run(["gcc", "-std=c99", "-O2", "-ffp-contract=off", "-Wall", "-o", exe, src, "-lm"],
                   check=True)
    out = subprocess.run([exe], stdout=subprocess.PIPE, text=True, timeout=300, check=True).stdout
    lines = dict(line.split(" ", 1) for line in out.strip().splitlines())
    checked, _, mismatches = lines["checked"].split()
    assert int(checked) > 4e8 and int(mismatches) == 0, out
    outside, _, differ = lines["outside"].split()
    assert int(differ) > 0, out
