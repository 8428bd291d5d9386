"""The update kernel encodes 8-bit codes as rint(x * RN(1/s)) with a guard
that falls back to rint(RN(x/s)) near half-integers (round_quotient in
csrc/apexw_kernels.hpp).  This CPU test checks that rule, written out with
numpy's IEEE fp32 arithmetic, against the definition rint(RN(x/s)) on ten
million random pairs and on constructed near-ties.  (The GPU parity tests
check the kernel itself bit for bit against the oracle.)"""
import numpy as np


def shortcut(x, s):
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        inv = np.float32(1.0) / s
        r = x * inv
        q = np.rint(r)
        dist = np.abs(np.abs(r - q) - np.float32(0.5))
        slow = ~(np.abs(r) <= np.float32(256.0)) | ~(dist > np.float32(2.5e-4))
        return np.where(slow, np.rint(x / s), q), slow


def check(x, s):
    got, slow = shortcut(x, s)
    want = np.rint(x / s)
    assert np.array_equal(got, want)
    return slow.mean()


def test_random_blocks_match_the_definition():
    rng = np.random.default_rng(0)
    total_slow = 0.0
    for rep in range(10):
        n = 1_000_000
        amax = np.float32(np.exp(rng.uniform(-80, 80, n))).astype(np.float32)
        for div in (np.float32(127.0), np.float32(255.0)):
            s = (amax / div).astype(np.float32)
            x = (amax * rng.uniform(-1, 1, n).astype(np.float32)).astype(np.float32)
            if div == 255.0:
                x = np.abs(x)
            x[:1000] = amax[:1000]                         # the block maximum itself
            total_slow += check(x, s)
    assert total_slow / 20 < 0.01


def test_near_ties_match_the_definition():
    rng = np.random.default_rng(1)
    n = 1_000_000
    s = np.float32(np.exp(rng.uniform(-60, 60, n))).astype(np.float32)
    k = rng.integers(-127, 127, n).astype(np.float32) + np.float32(0.5)
    x = (k.astype(np.float64) * s.astype(np.float64)).astype(np.float32)
    # walk a few ulps either side of each near-tie
    for step in range(-3, 4):
        xs = np.nextafter(x, np.float32(np.inf) if step > 0 else np.float32(-np.inf))
        for _ in range(abs(step) - 1):
            xs = np.nextafter(xs, np.float32(np.inf) if step > 0 else np.float32(-np.inf))
        check(xs if step else x, s)
    # tiny and denormal scales, zero values
    s2 = np.array([1e-45, 1e-40, 1e-38, 3e-39, 1e38], np.float32)
    for sv in s2:
        xv = (np.float32(sv) * np.arange(-127, 128, dtype=np.float32)).astype(np.float32)
        check(xv, np.full_like(xv, sv))
