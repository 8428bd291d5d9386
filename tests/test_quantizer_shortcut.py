"""CPU checks of the rounding shortcuts the update kernel takes instead of a
correctly rounded division or square root per element (code_value, sqrt_rn
and div_uniform in csrc/apexw_kernels.hpp), written out with IEEE fp32
arithmetic (numpy, or C with libm's fmaf for the fused multiply-adds) and
checked against the definitions.  The hardware approximations two of them
start from (v_rcp_f32, v_sqrt_f32: within one ulp) are modelled by trying
the correctly rounded value and both of its neighbours.  (The GPU parity
tests check the kernel itself bit for bit against the oracle.)"""
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
        xv = (np.float32(sv if np.isfinite(sv) else 1.0) * np.arange(-127, 128, dtype=F32)).astype(F32)
        check_codes(xv, np.full_like(xv, F32(sv)), F32(-127.0), F32(127.0))
        check_codes(np.abs(xv), np.full_like(xv, F32(sv)), F32(0.0), F32(255.0))


# ------------------------------------------------------------ square root

def sqrt_rule(x, s0):
    """The kernel's selection from an approximation s0 >= 0: the lower neighbour
    if x <= lo*s0, the upper one if x > hi*s0 (signs of the fma residuals,
    exact here: lo*s0 is exact in float64 and the float64 difference keeps
    its sign)."""
    lo = (s0.view(np.uint32) - np.uint32(1)).view(F32)      # the kernel steps the bits
    hi = (s0.view(np.uint32) + np.uint32(1)).view(F32)      # (at 0: lo is a NaN)
    x64 = x.astype(np.float64)
    with np.errstate(invalid="ignore"):
        r = np.where(x64 - lo.astype(np.float64) * s0.astype(np.float64) <= 0, lo, s0)
        r = np.where(x64 - hi.astype(np.float64) * s0.astype(np.float64) > 0, hi, r)
    return r


def check_sqrt(x):
    want = np.sqrt(x)                       # IEEE: correctly rounded
    for s0 in _neighbours(want):
        got = sqrt_rule(x, s0)
        ok = (got == want) | (np.isnan(got) & np.isnan(want))
        assert ok.all(), x[~ok][:5]


def test_sqrt_selection_on_every_mantissa_of_two_binades():
    m = np.arange(1 << 23, dtype=np.uint32)
    for exp_bits in (127, 128):             # [1, 2) and [2, 4): both exponent parities
        check_sqrt(((np.uint32(exp_bits) << 23) | m).view(F32))


def test_sqrt_selection_over_the_range_it_is_used_on():
    rng = np.random.default_rng(2)
    x = np.exp2(rng.uniform(-96, 128, 5_000_000)).astype(F32)
    x = x[np.isfinite(x)]
    check_sqrt(x)
    edges = np.array([2.0 ** -96, np.nextafter(F32(2.0 ** -96), F32(1)), 1.0, 4.0,
                      np.finfo(F32).max, np.finfo(F32).tiny * 2 ** 30], F32)
    check_sqrt(edges)
    # zero and +inf come through the rule unchanged
    for v in (F32(0.0), F32(np.inf)):
        s0 = np.array([v], F32)
        assert sqrt_rule(np.array([v], F32), s0)[0] == v


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
