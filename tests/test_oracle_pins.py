"""Pins of the oracle against what the pages and the mathematics fix (CPU only).

Each test ties the scalar C oracle to something other than itself: the worked
example printed in "Fused optimizers and state precision" (ai-infra-kb M041)
section 02, closed forms of the update (first step, zero gradient, constant
gradient), an fp64 brute force on tiny inputs, exact rational arithmetic for
beta^t, torch's own bf16 rounding, and the properties of the section 05 block
quantizer.  A dropped term, a wrong sign, an off-by-one step count, eps inside
the square root, a coupled-L2 decay or a wrong rounding rule fails at least one
of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import OracleAdamW, ref64
from workloads import Group

HERE = os.path.dirname(os.path.abspath(__file__))


def f32(x):
    return np.asarray(x, dtype=np.float32)


def run_f32(theta, grads_per_step, group, skips=()):
    """Run the fp32 oracle on one tensor; returns theta, m, v, t after each call."""
    o = OracleAdamW([theta.size], ["f32"], ["f32"], [0], "f32")
    th = f32(theta).copy()
    out = []
    for k, g in enumerate(grads_per_step, start=1):
        o.step([th], [None if g is None else f32(g)], [group], found_inf=k in skips)
        m, v = o.moments_f32(0)
        out.append((th.copy(), m, v, int(o.t[0])))
    return out


# ------------------------------------------------------------ worked example

def test_worked_example_page_values():
    d = json.load(open(os.path.join(HERE, "golden", "worked_example.json")))
    grp = Group(lr=d["lr"], beta1=d["beta1"], beta2=d["beta2"], eps=d["eps"],
                weight_decay=d["weight_decay"])
    (th, m, v, t), = run_f32(f32(d["theta0"]), [f32(d["g"])], grp)
    assert t == 1
    np.testing.assert_allclose(m, d["m1"], rtol=1e-6)
    np.testing.assert_allclose(v, d["v1"], rtol=1e-6)
    # m_hat = g and v_hat = g^2 at the first step
    g = np.array(d["g"])
    np.testing.assert_allclose(m / (1 - d["beta1"]), g, rtol=1e-6)
    np.testing.assert_allclose(v / (1 - d["beta2"]), g * g, rtol=1e-5)
    # theta printed to 3 decimals
    half_unit = 0.5 * 10.0 ** (-d["theta1_printed_digits"])
    assert np.all(np.abs(th - np.array(d["theta1_approx"])) <= half_unit)
    np.testing.assert_allclose(th, d["theta1_approx"], atol=2e-6)


# ------------------------------------------------------------ closed forms

@pytest.mark.parametrize("lr,wd,eps", [(1e-3, 0.01, 1e-8), (0.01, 0.1, 1e-3),
                                       (0.05, 0.0, 5e-4), (2e-4, 0.5, 1e-8)])
def test_first_step_closed_form(lr, wd, eps):
    rng = np.random.default_rng(1)
    theta = f32(rng.normal(0, 0.02, 4099))
    g = f32(rng.normal(0, 1e-3, 4099))
    g[:7] = 0.0
    grp = Group(lr=lr, beta1=0.9, beta2=0.999, eps=eps, weight_decay=wd)
    (th, m, v, t), = run_f32(theta, [g], grp)
    g64, th64 = g.astype(np.float64), theta.astype(np.float64)
    np.testing.assert_allclose(m, 0.1 * g64, rtol=2e-7, atol=0)
    np.testing.assert_allclose(v, 0.001 * g64 * g64, rtol=4e-7, atol=0)
    want = th64 * (1 - lr * wd) - lr * g64 / (np.abs(g64) + eps)
    # fp32 rounding: theta*decay, the decay constant and the final subtraction
    # each contribute at most about half an ulp of theta; the step term is
    # exact to a few ulps of lr.
    bound = 2.0 * np.spacing(np.abs(want).astype(np.float32)) + 1e-6 * lr
    assert np.all(np.abs(th - want) <= bound)
    assert t == 1


def test_zero_grad_is_pure_decay():
    rng = np.random.default_rng(2)
    theta = f32(rng.normal(0, 0.02, 1000))
    lr, wd = 1e-2, 0.3
    steps = run_f32(theta, [np.zeros(1000, np.float32)] * 12,
                    Group(lr=lr, weight_decay=wd))
    for k, (th, m, v, t) in enumerate(steps, start=1):
        assert t == k
        assert not m.any() and not v.any()
        np.testing.assert_allclose(th, theta.astype(np.float64) * (1 - lr * wd) ** k,
                                   rtol=2e-6 * k, atol=0)


@pytest.mark.parametrize("beta1,beta2", [(0.9, 0.999), (0.8, 0.95)])
def test_constant_grad_closed_form(beta1, beta2):
    """g = c at every call: m_k = c(1-b1^k), v_k = c^2(1-b2^k), m_hat = c,
    v_hat = c^2, so theta_k = theta_{k-1}(1-lr wd) - lr c/(|c|+eps)."""
    rng = np.random.default_rng(3)
    n, K = 2000, 40
    theta = f32(rng.normal(0, 0.02, n))
    c = f32(rng.normal(0, 1e-3, n))
    lr, wd, eps = 1e-3, 0.05, 1e-4
    steps = run_f32(theta, [c] * K, Group(lr=lr, beta1=beta1, beta2=beta2,
                                          eps=eps, weight_decay=wd))
    c64 = c.astype(np.float64)
    th = theta.astype(np.float64)
    u = lr * c64 / (np.abs(c64) + eps)
    for k, (th_k, m_k, v_k, t) in enumerate(steps, start=1):
        assert t == k
        np.testing.assert_allclose(m_k, c64 * (1 - beta1 ** k), rtol=2e-6 * k)
        np.testing.assert_allclose(v_k, c64 * c64 * (1 - beta2 ** k), rtol=3e-6 * k)
        th = th * (1 - lr * wd) - u
        np.testing.assert_allclose(th_k, th, rtol=0, atol=1e-8 * k)


# ------------------------------------------------------------ brute force

def test_multi_step_against_fp64_brute_force():
    """Three tiny tensors, 20 calls, random grads, call 5 skipped, tensor 2
    without grad on even calls: fp32 oracle vs an fp64 evaluation."""
    rng = np.random.default_rng(4)
    sizes = [5, 17, 259]
    groups = [Group(lr=1e-2, weight_decay=0.1), Group(lr=3e-3, eps=1e-6, weight_decay=0.0)]
    group_of = [0, 1, 0]
    o = OracleAdamW(sizes, ["f32"] * 3, ["f32"] * 3, group_of, "f32")
    th32 = [f32(rng.normal(0, 0.02, n)) for n in sizes]
    st64 = [[x.astype(np.float64), np.zeros(n), np.zeros(n), 0]
            for x, n in zip(th32, sizes)]
    for k in range(1, 21):
        gs = [f32(rng.normal(0, 1e-3, n)) for n in sizes]
        if k % 2 == 0:
            gs[2] = None
        skip = k == 5
        o.step(th32, gs, groups, found_inf=skip)
        if skip:
            continue
        for i, g in enumerate(gs):
            if g is None:
                continue
            gr = groups[group_of[i]]
            th64, m64, v64, t64 = st64[i]
            st64[i] = list(ref64.adamw_fp64(th64, g.astype(np.float64), m64, v64,
                                            t64, gr.lr, gr.beta1, gr.beta2,
                                            gr.eps, gr.weight_decay))
    for i in range(3):
        th64, m64, v64, t64 = st64[i]
        m, v = o.moments_f32(i)
        assert o.t[i] == t64
        for a, b in ((th32[i], th64), (m, m64), (v, v64)):
            err = np.max(np.abs(a - b)) / np.max(np.abs(b))
            assert err <= 1e-5, err
    assert list(o.t) == [19, 19, 9]   # odd calls minus the skipped call 5


def test_three_loops_equal_one_pass_bitwise():
    rng = np.random.default_rng(5)
    sizes = [1000, 33, 4097]
    groups = [Group(lr=1e-3, weight_decay=0.01), Group(lr=5e-4)]
    a = OracleAdamW(sizes, ["f32"] * 3, ["f32"] * 3, [0, 1, 0], "f32")
    b = OracleAdamW(sizes, ["f32"] * 3, ["f32"] * 3, [0, 1, 0], "f32")
    tha = [f32(rng.normal(0, 0.02, n)) for n in sizes]
    thb = [x.copy() for x in tha]
    for k in range(1, 8):
        gs = [f32(rng.normal(0, 1e-3, n)) for n in sizes]
        if k == 3:
            gs[1] = None
        a.step(tha, gs, groups, found_inf=(k == 4))
        b.step_three_loops(thb, gs, groups, found_inf=(k == 4))
    for i in range(3):
        assert np.array_equal(tha[i].view(np.uint32), thb[i].view(np.uint32))
        assert np.array_equal(a.m[i].view(np.uint32), b.m[i].view(np.uint32))
        assert np.array_equal(a.v[i].view(np.uint32), b.v[i].view(np.uint32))
    assert np.array_equal(a.t, b.t)


def test_coupled_l2_is_a_different_update():
    """Adding the decay into g (coupled L2) is not AdamW; the oracle follows
    the decoupled form."""
    rng = np.random.default_rng(6)
    n = 512
    theta = f32(rng.normal(0, 0.5, n))
    grp = Group(lr=1e-2, weight_decay=0.2)
    gs = [f32(rng.normal(0, 1e-3, n)) for _ in range(5)]
    th_o = run_f32(theta, gs, grp)[-1][0].astype(np.float64)
    dec = [theta.astype(np.float64), np.zeros(n), np.zeros(n), 0]
    cpl = [theta.astype(np.float64), np.zeros(n), np.zeros(n), 0]
    for g in gs:
        args = (grp.lr, grp.beta1, grp.beta2, grp.eps, grp.weight_decay)
        dec = ref64.adamw_fp64(dec[0], g.astype(np.float64), dec[1], dec[2], dec[3], *args)
        cpl = ref64.adam_l2_fp64(cpl[0], g.astype(np.float64), cpl[1], cpl[2], cpl[3], *args)
    assert np.max(np.abs(th_o - dec[0])) < 1e-6
    assert np.max(np.abs(th_o - cpl[0])) > 1e-3


# ------------------------------------------------------------ skip / None

@pytest.mark.parametrize("fmt", ["f32", "bf16", "q8"])
def test_found_inf_and_missing_grad_change_nothing(fmt):
    rng = np.random.default_rng(7)
    sizes = [300, 1024]
    pdt = ["bf16", "f32"]
    o = OracleAdamW(sizes, pdt, ["f32", "bf16"], [0, 0], fmt)
    th = [oracle.f32_to_bf16(f32(rng.normal(0, 0.02, 300))),
          f32(rng.normal(0, 0.02, 1024))]
    grp = [Group(lr=1e-3, weight_decay=0.1)]

    def grads():
        return [f32(rng.normal(0, 1e-3, 300)),
                oracle.f32_to_bf16(f32(rng.normal(0, 1e-3, 1024)))]

    for _ in range(3):
        o.step(th, grads(), grp)

    def snap():
        return ([x.copy() for x in th], [x.copy() for x in o.m], [x.copy() for x in o.v],
                [None if s is None else s.copy() for s in o.m_scale],
                [None if s is None else s.copy() for s in o.v_scale], [o.t.copy()])

    before = snap()
    o.step(th, grads(), grp, found_inf=True)
    after = snap()
    for x, y in zip(before, after):
        for a, b in zip(x, y):
            assert (a is None and b is None) or np.array_equal(
                np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    # grad None on tensor 0 only: tensor 0 untouched, tensor 1 advances
    g = grads()
    o.step(th, [None, g[1]], grp)
    assert np.array_equal(th[0], before[0][0]) and np.array_equal(o.m[0], before[1][0])
    assert list(o.t) == [3, 4]


def test_zero_grad_is_not_missing_grad():
    rng = np.random.default_rng(8)
    theta = f32(rng.normal(0, 0.02, 64))
    g1 = f32(rng.normal(0, 1e-3, 64))
    grp = Group(lr=1e-2, weight_decay=0.1)
    zero = run_f32(theta, [g1, np.zeros(64, np.float32)], grp)
    none = run_f32(theta, [g1, None], grp)
    th1, m1, v1, _ = zero[0]
    thz, mz, vz, tz = zero[1]
    thn, mn, vn, tn = none[1]
    assert tn == 1 and tz == 2
    assert np.array_equal(thn, th1) and np.array_equal(mn, m1) and np.array_equal(vn, v1)
    np.testing.assert_allclose(mz, 0.9 * m1.astype(np.float64), rtol=1e-6)
    np.testing.assert_allclose(vz, 0.999 * v1.astype(np.float64), rtol=1e-6)
    assert not np.array_equal(thz, th1)


# ------------------------------------------------------------ scalars

def _round_to_f32(fr: Fraction) -> np.float32:
    """Nearest float32 to an exact rational, ties to even."""
    c = np.float32(float(fr))
    cands = [np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))]
    best = min(cands, key=lambda x: (abs(Fraction(float(x)) - fr),
                                     int(np.array(x).view(np.uint32)) & 1))
    return best


@pytest.mark.parametrize("beta", [0.9, 0.999, 0.95, 0.5, 0.9999])
def test_pow_int_against_exact_rationals(beta):
    b = Fraction(beta)  # the exact double value
    ts = list(range(1, 301)) + [1000, 4096, 65535, 100000]
    mism = 0
    for t in ts:
        exact = b ** t
        got = oracle.pow_int(beta, t)
        # each squaring doubles the relative error carried so far, so the
        # error of square-and-multiply grows at most linearly in t
        if exact < Fraction(2.0 ** -1000):        # underflow: only "tiny"
            assert got < 2.0 ** -1000
        else:
            bound = (t + 2 * t.bit_length()) * Fraction(1, 2 ** 53) * exact
            assert abs(Fraction(got) - exact) <= bound, t
        bc = np.float32(1.0 - got)
        mism += int(bc != _round_to_f32(1 - exact))
    assert mism == 0


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(9)
    x = f32(rng.normal(0, 1, 20000) * np.exp(rng.uniform(-30, 30, 20000)))
    bits = x.view(np.uint32).copy()
    bits[:4000] = (bits[:4000] & 0xFFFF0000) | 0x8000       # exact ties
    bits[4000:5000] = (bits[4000:5000] & 0xFFFF0000) | 0x7FFF
    bits[5000:6000] = (bits[5000:6000] & 0xFFFF0000) | 0x8001
    x = bits.view(np.float32)
    x[6000:6004] = [np.inf, -np.inf, 0.0, -0.0]
    x[6004] = np.float32(3.3895314e38)                      # rounds to inf
    ours = oracle.f32_to_bf16(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = oracle.bf16_to_f32(ours)
    ref_back = torch.from_numpy(ours.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    assert np.array_equal(back.view(np.uint32), ref_back.view(np.uint32))


def test_bf16_rounding_of_nans():
    """A NaN stays a NaN (torch agrees on the class; a signalling NaN whose
    payload sits in the low 16 bits must not round up into an infinity), comes
    out quiet (IEEE 754, section 6.2: an operation on a signalling NaN delivers
    a quiet one), and keeps its sign and the top 7 bits of its payload."""
    rng = np.random.default_rng(14)
    sign = rng.integers(0, 2, 4000).astype(np.uint32) << 31
    payload = rng.integers(1, 1 << 23, 4000).astype(np.uint32)
    payload[:500] &= 0xFFFF                                    # low payload only
    payload[:500] |= 1
    payload[500:1000] |= 0x400000                              # already quiet
    bits = sign | 0x7F800000 | payload
    x = bits.view(np.float32)
    assert np.isnan(x).all()
    ours = oracle.f32_to_bf16(x)
    theirs = torch.from_numpy(x.copy()).to(torch.bfloat16).float().numpy()
    assert np.isnan(theirs).all()
    wide = oracle.bf16_to_f32(ours)
    assert np.isnan(wide).all()
    assert np.all((ours & 0x7F80) == 0x7F80)                   # exponent all ones
    assert np.all(ours & 0x0040)                               # quiet bit
    assert np.array_equal(ours >> 15, (bits >> 31).astype(np.uint16))
    assert np.array_equal(ours & 0x3F, ((bits >> 16) & 0x3F).astype(np.uint16))


# ------------------------------------------------------------ quantizer

def test_quantizer_all_zero_block():
    q, s = oracle.quantize_signed(np.zeros(256, np.float32))
    assert s == 0.0 and not q.any()
    q, s = oracle.quantize_unsigned(np.zeros(256, np.float32))
    assert s == 0.0 and not q.any()
    assert not oracle.dequantize_signed(q.astype(np.int8), 0.0).any()


def test_quantizer_ties_round_half_even():
    q, s = oracle.quantize_signed(f32([127, 2.5, 3.5, -2.5, 0.5, -0.5, 1.5, -126.5]))
    assert s == 1.0
    assert list(q) == [127, 2, 4, -2, 0, 0, 2, -126]
    q, s = oracle.quantize_unsigned(f32([255, 0.5, 1.5, 2.5, 254.5, 0]))
    assert s == 1.0
    assert list(q) == [255, 0, 2, 2, 254, 0]


def test_quantizer_absmax_and_error_bound():
    rng = np.random.default_rng(10)
    for trial in range(2000):
        n = 256 if trial % 5 else int(rng.integers(1, 256))
        scale_mag = float(np.exp(rng.uniform(-40, 5)))
        x = f32(rng.normal(0, 1, n) * scale_mag)
        q, s = oracle.quantize_signed(x)
        amax = np.max(np.abs(x))
        assert s == np.float32(amax) / np.float32(127) or amax == 0
        assert np.abs(q[np.argmax(np.abs(x))]) == 127
        back = oracle.dequantize_signed(q, s)
        assert np.all(np.abs(back.astype(np.float64) - x) <= s * (0.5 + 256 * 2.0 ** -24))
        # re-encoding the decoded block keeps the codes
        q2, s2 = oracle.quantize_signed(back)
        assert np.array_equal(q, q2)
        assert abs(s2 - s) <= np.spacing(np.float32(s))
        y = np.abs(x) * np.abs(x)
        qv, sv = oracle.quantize_unsigned(y)
        assert qv[np.argmax(y)] == 255
        backv = oracle.dequantize_unsigned(qv, sv)
        assert np.all(np.abs(backv.astype(np.float64) - y) <= sv * (0.5 + 512 * 2.0 ** -24))


def test_q8_partial_block_has_own_scale_and_blocks_stay_in_tensor():
    rng = np.random.default_rng(11)
    sizes = [300, 40]
    o = OracleAdamW(sizes, ["f32", "f32"], ["f32", "f32"], [0, 0], "q8")
    th = [f32(rng.normal(0, 0.02, n)) for n in sizes]
    g = [f32(rng.normal(0, 1e-3, n)) for n in sizes]
    g[0][256:] *= 100.0          # the tail block has a much larger scale
    o.step(th, g, [Group(lr=1e-3)])
    assert o.m_scale[0].size == 2 and o.m_scale[1].size == 1
    m_true = 0.1 * g[0].astype(np.float64)
    assert math.isclose(o.m_scale[0][1], np.max(np.abs(m_true[256:])) / 127, rel_tol=1e-6)
    assert math.isclose(o.m_scale[0][0], np.max(np.abs(m_true[:256])) / 127, rel_tol=1e-6)
    assert math.isclose(o.m_scale[1][0], np.max(np.abs(0.1 * g[1])) / 127, rel_tol=1e-6)


# ------------------------------------------------------------ compact state

def test_q8_step_is_decode_update_encode():
    """theta uses this step's fp32 moments; storage is re-encoded afterwards."""
    rng = np.random.default_rng(12)
    n = 1000
    grp = [Group(lr=1e-3, weight_decay=0.01)]
    q = OracleAdamW([n], ["bf16"], ["bf16"], [0], "q8")
    th = oracle.f32_to_bf16(f32(rng.normal(0, 0.02, n)))
    for k in range(1, 9):
        g = oracle.f32_to_bf16(f32(rng.normal(0, 1e-3, n)))
        m_dec, v_dec = q.moments_f32(0)
        ref = OracleAdamW([n], ["bf16"], ["bf16"], [0], "f32")
        ref.m[0][:] = m_dec
        ref.v[0][:] = v_dec
        ref.t[0] = q.t[0]
        th_ref = th.copy()
        ref.step([th_ref], [g], grp)
        q.step([th], [g], grp)
        assert np.array_equal(th, th_ref)
        for b in range((n + 255) // 256):
            lo, hi = b * 256, min(n, b * 256 + 256)
            qm, sm = oracle.quantize_signed(ref.m[0][lo:hi])
            qv, sv = oracle.quantize_unsigned(ref.v[0][lo:hi])
            assert np.array_equal(qm, q.m[0][lo:hi]) and sm == q.m_scale[0][b]
            assert np.array_equal(qv, q.v[0][lo:hi]) and sv == q.v_scale[0][b]
        assert q.t[0] == k


def test_bf16_state_is_fp32_update_rounded():
    rng = np.random.default_rng(13)
    n = 777
    grp = [Group(lr=1e-3, weight_decay=0.1)]
    b = OracleAdamW([n], ["bf16"], ["f32"], [0], "bf16")
    th = oracle.f32_to_bf16(f32(rng.normal(0, 0.02, n)))
    for k in range(1, 6):
        g = f32(rng.normal(0, 1e-3, n))
        ref = OracleAdamW([n], ["bf16"], ["f32"], [0], "f32")
        ref.m[0][:], ref.v[0][:] = b.moments_f32(0)
        ref.t[0] = b.t[0]
        th_ref = th.copy()
        ref.step([th_ref], [g], grp)
        b.step([th], [g], grp)
        assert np.array_equal(th, th_ref)
        assert np.array_equal(b.m[0], oracle.f32_to_bf16(ref.m[0]))
        assert np.array_equal(b.v[0], oracle.f32_to_bf16(ref.v[0]))


# ------------------------------------------------------------ unscale / check

def _run_fmt(fmt, sizes, pdt, gdt, grads_per_call, group, inv_scale=None, seed=20):
    rng = np.random.default_rng(seed)
    o = OracleAdamW(sizes, pdt, gdt, [0] * len(sizes), fmt)
    th = []
    for n, d in zip(sizes, pdt):
        x = f32(rng.normal(0, 0.02, n))
        th.append(oracle.f32_to_bf16(x) if d == "bf16" else x)
    for gs in grads_per_call:
        o.step(th, gs, [group], inv_scale=inv_scale)
    return th, o


def _as_dtype(x, d):
    return oracle.f32_to_bf16(x) if d == "bf16" else f32(x)


@pytest.mark.parametrize("fmt", ["f32", "bf16", "q8"])
def test_unscale_by_power_of_two_is_exact(fmt):
    """Grads stored multiplied by 2^k and unscaled by 2^-k give bit for bit the
    plain step on the unscaled grads (the scaling is exact), and inv_scale = 1
    is the plain step; a multiply placed anywhere else would differ."""
    rng = np.random.default_rng(21)
    sizes, pdt, gdt = [700, 300], ["bf16", "f32"], ["f32", "bf16"]
    grp = Group(lr=1e-3, weight_decay=0.05)
    calls = [[f32(rng.normal(0, 1e-3, n)) for n in sizes] for _ in range(4)]
    plain = [[_as_dtype(g, d) for g, d in zip(c, gdt)] for c in calls]
    scaled = [[_as_dtype(g * 65536.0, d) for g, d in zip(c, gdt)] for c in calls]
    th_a, a = _run_fmt(fmt, sizes, pdt, gdt, plain, grp)
    th_b, b = _run_fmt(fmt, sizes, pdt, gdt, scaled, grp, inv_scale=1.0 / 65536.0)
    th_c, c = _run_fmt(fmt, sizes, pdt, gdt, plain, grp, inv_scale=1.0)
    for i in range(2):
        for other_th, other in ((th_b, b), (th_c, c)):
            assert np.array_equal(th_a[i], other_th[i])
            assert np.array_equal(a.m[i], other.m[i]) and np.array_equal(a.v[i], other.v[i])


def test_unscale_general_factor_against_fp64():
    rng = np.random.default_rng(22)
    n, inv = 513, 1.0 / 3.0
    grp = Group(lr=1e-2, weight_decay=0.1)
    theta = f32(rng.normal(0, 0.02, n))
    o = OracleAdamW([n], ["f32"], ["f32"], [0], "f32")
    th = theta.copy()
    st = [theta.astype(np.float64), np.zeros(n), np.zeros(n), 0]
    for _ in range(10):
        g = f32(rng.normal(0, 3e-3, n))
        o.step([th], [g], [grp], inv_scale=inv)
        g64 = (g * np.float32(inv)).astype(np.float64)
        st = list(ref64.adamw_fp64(st[0], g64, st[1], st[2], st[3], grp.lr, grp.beta1,
                                   grp.beta2, grp.eps, grp.weight_decay))
    assert np.max(np.abs(th - st[0])) / np.max(np.abs(st[0])) <= 1e-5
    m, v = o.moments_f32(0)
    assert np.max(np.abs(m - st[1])) / np.max(np.abs(st[1])) <= 1e-5


@pytest.mark.parametrize("inv", [1.0 / 65536.0, 1.0, 4.0, 3.0e30])
def test_unscale_check_matches_numpy_isfinite(inv):
    rng = np.random.default_rng(23)
    sizes, gdt = [1000, 257, 64], ["f32", "bf16", "f32"]
    o = OracleAdamW(sizes, ["f32"] * 3, gdt, [0, 0, 0], "f32")
    for trial in range(30):
        gs = [f32(rng.normal(0, 1.0, n) * np.exp(rng.uniform(-10, 10, n))) for n in sizes]
        if trial % 3 == 1:
            t = rng.integers(0, 3)
            gs[t][rng.integers(0, sizes[t])] = [np.inf, -np.inf, np.nan][trial % 3]
        if trial % 5 == 4:
            gs[0][5] = np.float32(3.0e38)          # finite, overflows when inv > 1
        absent = trial % 4 == 2
        stored = [_as_dtype(g, d) for g, d in zip(gs, gdt)]
        if absent:
            stored[0] = None
        want = False
        for g, d in zip(stored, gdt):
            if g is None:
                continue
            v = oracle.bf16_to_f32(g) if d == "bf16" else g
            with np.errstate(over="ignore", invalid="ignore"):
                want |= bool(np.any(~np.isfinite(v * np.float32(inv))))
        assert o.unscale_check(stored, inv) == want


def test_amp_recipe_skip_on_overflow():
    """Scale 2^16: grads arrive scaled; an overflow in any tensor makes the
    check report it and the step with that flag change nothing."""
    rng = np.random.default_rng(24)
    sizes = [400, 90]
    grp = Group(lr=1e-3, weight_decay=0.1)
    o = OracleAdamW(sizes, ["f32", "f32"], ["f32", "f32"], [0, 0], "f32")
    th = [f32(rng.normal(0, 0.02, n)) for n in sizes]
    scale = 65536.0
    for k in range(1, 7):
        gs = [f32(rng.normal(0, 1e-3, n) * scale) for n in sizes]
        if k == 4:
            gs[1][7] = np.inf
        found = o.unscale_check(gs, 1.0 / scale)
        assert found == (k == 4)
        before = [x.copy() for x in th] + [o.t.copy()]
        o.step(th, gs, [grp], found_inf=found, inv_scale=1.0 / scale)
        if found:
            after = [x.copy() for x in th] + [o.t.copy()]
            assert all(np.array_equal(a, b) for a, b in zip(before, after))
    assert list(o.t) == [5, 5]


# ------------------------------------------------------------ clipping

def test_grad_norm_against_exact_sum():
    """The oracle's fp64 running sum against the exactly rounded sum of the
    same fp32 products (math.fsum)."""
    rng = np.random.default_rng(30)
    sizes, gdt = [5000, 777, 1], ["f32", "bf16", "f32"]
    o = OracleAdamW(sizes, ["f32"] * 3, gdt, [0, 0, 0], "f32")
    for inv in (1.0, 1.0 / 1024.0, 1.0 / 3.0):
        gs = [f32(rng.normal(0, 1, n) * np.exp(rng.uniform(-5, 5, n))) for n in sizes]
        stored = [_as_dtype(g, d) for g, d in zip(gs, gdt)]
        stored[2] = None if inv == 1.0 else stored[2]
        u = []
        for g, d in zip(stored, gdt):
            if g is None:
                continue
            v = oracle.bf16_to_f32(g) if d == "bf16" else g
            u.append((v * np.float32(inv)).astype(np.float64))
        u = np.concatenate(u)
        exact = math.sqrt(math.fsum((u * u).tolist()))
        got = o.grad_norm(stored, inv)
        assert abs(got - exact) <= 1e-13 * exact


def test_clip_coef_cases():
    c = OracleAdamW.clip_coef
    assert c(0.0, 1.0) == 1.0                      # no grads: nothing to clip
    assert c(0.5, 1.0) == 1.0 and c(1.0, 1.0) == 1.0
    assert c(4.0, 1.0) == 0.25
    assert c(3.0, 1.0) == np.float32(1.0 / 3.0)
    assert c(float("nan"), 1.0) == 1.0
    assert c(float("inf"), 1.0) == 0.0


def test_clipped_step_scales_the_direction_only_through_g():
    """With clip 2^-k (exact) the clipped step equals the plain step on grads
    multiplied by 2^-k; a zero-grad-free first step is invariant to any clip
    (m_hat / sqrt(v_hat) = sign(g)), which a clip applied to theta, m or the
    update would break."""
    rng = np.random.default_rng(31)
    n = 900
    grp = [Group(lr=1e-2, weight_decay=0.1)]
    th0 = f32(rng.normal(0, 0.02, n))
    g = f32(rng.normal(0, 1e-3, n))
    a = OracleAdamW([n], ["f32"], ["f32"], [0], "f32")
    b = OracleAdamW([n], ["f32"], ["f32"], [0], "f32")
    tha, thb = th0.copy(), th0.copy()
    a.step([tha], [g * np.float32(0.125)], grp)
    b.step([thb], [g], grp, clip_coef=0.125)
    assert np.array_equal(tha, thb) and np.array_equal(a.m[0], b.m[0])
    grp0 = [Group(lr=1e-2, weight_decay=0.1, eps=0.0)]
    c = OracleAdamW([n], ["f32"], ["f32"], [0], "f32")
    thc = th0.copy()
    c.step([thc], [g], grp0, clip_coef=0.3)
    plain = OracleAdamW([n], ["f32"], ["f32"], [0], "f32")
    thp = th0.copy()
    plain.step([thp], [g], grp0)
    # first step with eps = 0: the direction is sign(g) (to a few ulps),
    # whatever the clip
    assert np.max(np.abs(thc.astype(np.float64) - thp)) < 1e-8
    assert not np.array_equal(c.m[0], plain.m[0])


def test_clipped_amp_loop_against_fp64():
    rng = np.random.default_rng(32)
    n, inv, max_norm = 2000, 1.0 / 512.0, 0.02
    grp = Group(lr=1e-2, weight_decay=0.01)
    o = OracleAdamW([n], ["f32"], ["f32"], [0], "f32")
    th = f32(rng.normal(0, 0.02, n))
    st = [th.astype(np.float64), np.zeros(n), np.zeros(n), 0]
    clipped = 0
    for _ in range(12):
        g = f32(rng.normal(0, 1e-3, n) * 512.0 * rng.uniform(0.2, 2.0))
        norm = o.grad_norm([g], inv)
        coef = OracleAdamW.clip_coef(norm, max_norm)
        clipped += coef < 1.0
        o.step([th], [g], [grp], inv_scale=inv, clip_coef=coef)
        u = (g * np.float32(inv)).astype(np.float64)
        un = np.sqrt(np.sum(u * u))
        u64 = u * (max_norm / un if un > max_norm else 1.0)
        st = list(ref64.adamw_fp64(st[0], u64, st[1], st[2], st[3], grp.lr, grp.beta1, grp.beta2,
                                   grp.eps, grp.weight_decay))
    assert 0 < clipped < 12
    assert np.max(np.abs(th - st[0])) / np.max(np.abs(st[0])) <= 1e-5


# ------------------------------------------------------------ timing build

@pytest.mark.parametrize("fmt", ["f32", "bf16", "q8"])
def test_threaded_timing_build_is_bitwise_the_parity_build(fmt):
    """The OpenMP build of the same oracle source (the host baseline's timing
    build) splits each tensor's elements or 8-bit blocks over threads; every
    value must come out exactly as in the single-threaded parity build."""
    assert oracle.omp_lib().oracle_threads() >= 1
    rng = np.random.default_rng(15)
    sizes = [200_003, 65_536, 1000, 3]
    pdt = ["bf16", "f32", "bf16", "f32"]
    gdt = ["f32", "f32", "bf16", "f32"]
    groups = [Group(lr=1e-3, weight_decay=0.1), Group(lr=5e-4, beta1=0.8, eps=1e-6)]
    gof = [0, 1, 0, 1]
    runs = []
    for threaded in (False, True):
        r = np.random.default_rng(16)
        o = OracleAdamW(sizes, pdt, gdt, gof, fmt, threaded=threaded)
        th = [oracle.f32_to_bf16(f32(r.normal(0, 0.02, n))) if d == "bf16" else f32(r.normal(0, 0.02, n))
              for n, d in zip(sizes, pdt)]
        for k in range(1, 6):
            gs = [oracle.f32_to_bf16(f32(r.normal(0, 1e-3, n))) if d == "bf16" else f32(r.normal(0, 1e-3, n))
                  for n, d in zip(sizes, gdt)]
            if k == 3:
                gs[2] = None
            o.step(th, gs, groups, found_inf=(k == 4), inv_scale=0.5 if k == 5 else None)
        runs.append((th, o))
    (th_a, a), (th_b, b) = runs
    assert np.array_equal(a.t, b.t)
    for i in range(len(sizes)):
        assert np.array_equal(th_a[i].view(np.uint8), th_b[i].view(np.uint8)), i
        assert np.array_equal(a.m[i].view(np.uint8), b.m[i].view(np.uint8)), i
        assert np.array_equal(a.v[i].view(np.uint8), b.v[i].view(np.uint8)), i
        if fmt == "q8":
            assert np.array_equal(a.m_scale[i].view(np.uint32), b.m_scale[i].view(np.uint32)), i
            assert np.array_equal(a.v_scale[i].view(np.uint32), b.v_scale[i].view(np.uint32)), i
