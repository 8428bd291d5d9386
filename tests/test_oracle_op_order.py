"""Bit-level pin of the oracle's order of operations (CPU only).

The update box of "Fused optimizers and state precision" (ai-infra-kb M041),
section 02, is written in Python.  Read with that language's own rules --
binary operators of equal precedence group from the left, `*` and `/` bind
tighter than `+` and `-`, `**` tighter still -- every expression in it names
one sequence of rounded operations.  The functions below evaluate the box
exactly that way with numpy: theta, g, m and v are float32 arrays, the
hyperparameters are Python floats (float64) that numpy rounds to float32 where
they meet an array, beta**t is taken on Python floats, and sqrt is np.sqrt
(correctly rounded).  In particular the box fixes

    v     = (beta2*v) + (((1-beta2)*g)*g)
    theta = (theta*(1-lr*weight_decay)) - ((lr*m_hat)/(sqrt(v_hat)+eps))

and nothing in the oracle's C source is consulted.  bf16 storage is wrapped
around the box with torch's own round-to-nearest-even conversion; 8-bit storage
with the section 05 block quantizer written here in numpy (scale = block absmax
/ 127 or / 255, codes round-half-even, an all-zero block gets scale 0 and
codes 0).  The oracle must agree bit for bit, over many steps, with skipped
calls and absent grads.  A different grouping -- (1-beta2)*(g*g),
lr*(m_hat/den) -- or a contracted multiply-add in the oracle changes some
float32 results and fails here; the last test builds such variants of the
oracle and shows it.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from oracle import OracleAdamW
from workloads import Group


# ------------------------------------------------------------ the literal box

def literal_box(theta, g, m, v, t, lr, beta1, beta2, eps, weight_decay):
    """M041 section 02, one step, on float32 arrays (t already advanced)."""
    m = beta1*m + (1-beta1)*g
    v = beta2*v + (1-beta2)*g*g
    m_hat = m / (1-beta1**t)
    v_hat = v / (1-beta2**t)
    theta = theta*(1-lr*weight_decay) - lr*m_hat/(np.sqrt(v_hat)+eps)
    return theta, m, v


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def _to_bf16_bits(x):
    """torch's float32 -> bfloat16 conversion (round to nearest even)."""
    return torch.from_numpy(_f32(x).copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _from_bf16_bits(b):
    return torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).float().numpy()


def _block_starts(n):
    return np.arange(0, n, 256)


def quantize_literal(x, levels, signed):
    """M041 section 05 per 256-element block of one tensor: scale = max|x| /
    levels, q = round(x / scale) (half to even), clamped to the code range;
    an all-zero block is handled on its own (scale 0, codes 0)."""
    starts = _block_starts(x.size)
    amax = np.maximum.reduceat(np.abs(x) if signed else x, starts)
    scale = amax / levels                               # float32 / int -> float32
    per = np.repeat(scale, np.diff(np.append(starts, x.size)))
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.round(x / per)
    q = np.where(per == 0, 0, q)
    lo, hi = (-levels, levels) if signed else (0, levels)
    q = np.clip(q, lo, hi)
    return q.astype(np.int8 if signed else np.uint8), scale.astype(np.float32)


def dequantize_literal(q, scale):
    starts = _block_starts(q.size)
    per = np.repeat(scale, np.diff(np.append(starts, q.size)))
    return q * per                                      # int * float32 -> float32


# ------------------------------------------------------------ a workload

SIZES = [100_003, 31_000, 7, 256 * 40]
GROUPS = [Group(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
          Group(lr=3e-4, beta1=0.85, beta2=0.995, eps=1e-6, weight_decay=0.1)]
GROUP_OF = [0, 1, 0, 1]


def _grads(rng, k, absent):
    out = []
    for i, n in enumerate(SIZES):
        g = _f32(rng.normal(0.0, 1e-3, n))
        g[:: 97] = 0.0                                   # exact zeros among them
        out.append(None if (i, k) in absent else g)
    return out


def _check_beta_powers(steps):
    # beta**t on Python floats and the oracle's square-and-multiply give the
    # same float32 bias correction at every count used here, so the box's
    # "**" reads the same whichever way the power is formed
    for G in GROUPS:
        for t in range(1, steps + 1):
            for b in (G.beta1, G.beta2):
                assert np.float32(1 - b**t) == np.float32(1 - oracle.pow_int(b, t))


def _run_literal_dense(steps, skips, absent, state, seed):
    rng = np.random.default_rng(seed)
    th0 = [_f32(rng.normal(0.0, 0.02, n)) for n in SIZES]
    grads = [_grads(rng, k, absent) for k in range(1, steps + 1)]
    # literal side
    th = [x.copy() for x in th0]
    m = [np.zeros(n, np.float32) for n in SIZES]
    v = [np.zeros(n, np.float32) for n in SIZES]
    t = [0] * len(SIZES)
    for k in range(1, steps + 1):
        if k in skips:
            continue
        for i in range(len(SIZES)):
            g = grads[k - 1][i]
            if g is None:
                continue
            t[i] += 1
            G = GROUPS[GROUP_OF[i]]
            th[i], mi, vi = literal_box(th[i], g, m[i], v[i], t[i], G.lr, G.beta1, G.beta2,
                                        G.eps, G.weight_decay)
            assert th[i].dtype == mi.dtype == vi.dtype == np.float32
            if state == "bf16":
                mi = _from_bf16_bits(_to_bf16_bits(mi))
                vi = _from_bf16_bits(_to_bf16_bits(vi))
            m[i], v[i] = mi, vi
    # oracle side
    o = OracleAdamW(SIZES, ["f32"] * len(SIZES), ["f32"] * len(SIZES), GROUP_OF, state)
    th_o = [x.copy() for x in th0]
    for k in range(1, steps + 1):
        o.step(th_o, grads[k - 1], GROUPS, found_inf=k in skips)
    return th, m, v, t, o, th_o


@pytest.mark.parametrize("state", ["f32", "bf16"])
def test_oracle_is_the_literal_box_bit_for_bit(state):
    steps = 20 if state == "f32" else 10
    skips = {7}
    absent = {(2, k) for k in range(1, steps + 1, 2)} | {(1, 4)}
    _check_beta_powers(steps)
    th, m, v, t, o, th_o = _run_literal_dense(steps, skips, absent, state, seed=31)
    assert list(o.t[:len(SIZES)]) == t
    for i in range(len(SIZES)):
        mo, vo = o.moments_f32(i)
        assert np.array_equal(th_o[i].view(np.uint32), th[i].view(np.uint32)), i
        assert np.array_equal(mo.view(np.uint32), m[i].view(np.uint32)), i
        assert np.array_equal(vo.view(np.uint32), v[i].view(np.uint32)), i


def test_bf16_params_are_widened_updated_and_rounded_once():
    steps = 10
    rng = np.random.default_rng(32)
    n = 70_001
    G = GROUPS[0]
    th_bits = _to_bf16_bits(rng.normal(0.0, 0.02, n))
    o = OracleAdamW([n], ["bf16"], ["bf16"], [0], "f32")
    th_o = th_bits.copy()
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    for k in range(1, steps + 1):
        g_bits = _to_bf16_bits(rng.normal(0.0, 1e-3, n))
        th, m, v = literal_box(_from_bf16_bits(th_bits), _from_bf16_bits(g_bits), m, v, k,
                               G.lr, G.beta1, G.beta2, G.eps, G.weight_decay)
        th_bits = _to_bf16_bits(th)
        o.step([th_o], [g_bits], [G])
    assert np.array_equal(th_o, th_bits)
    assert np.array_equal(o.m[0].view(np.uint32), m.view(np.uint32))
    assert np.array_equal(o.v[0].view(np.uint32), v.view(np.uint32))


def test_q8_is_decode_literal_box_encode_for_250_steps():
    steps = 250
    _check_beta_powers(steps)
    rng = np.random.default_rng(33)
    sizes = [256 * 96, 16 * 3072 + 100, 5]
    G = Group(lr=2e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    o = OracleAdamW(sizes, ["bf16"] * 3, ["bf16"] * 3, [0] * 3, "q8")
    th_bits = [_to_bf16_bits(rng.normal(0.0, 0.02, n)) for n in sizes]
    th_o = [b.copy() for b in th_bits]
    qm = [np.zeros(n, np.int8) for n in sizes]
    qv = [np.zeros(n, np.uint8) for n in sizes]
    sm = [np.zeros((n + 255) // 256, np.float32) for n in sizes]
    sv = [np.zeros((n + 255) // 256, np.float32) for n in sizes]
    t = [0] * 3
    for k in range(1, steps + 1):
        gs = [_to_bf16_bits(rng.normal(0.0, 1e-3, n)) for n in sizes]
        if k % 50 == 17:
            gs[1] = None
        skip = k == 101
        o.step(th_o, gs, [G], found_inf=skip)
        if skip:
            continue
        for i in range(3):
            if gs[i] is None:
                continue
            t[i] += 1
            mf = dequantize_literal(qm[i], sm[i])
            vf = dequantize_literal(qv[i], sv[i])
            th, mf, vf = literal_box(_from_bf16_bits(th_bits[i]), _from_bf16_bits(gs[i]), mf, vf,
                                     t[i], G.lr, G.beta1, G.beta2, G.eps, G.weight_decay)
            th_bits[i] = _to_bf16_bits(th)
            qm[i], sm[i] = quantize_literal(mf, 127, signed=True)
            qv[i], sv[i] = quantize_literal(vf, 255, signed=False)
    assert list(o.t[:3]) == t
    for i in range(3):
        assert np.array_equal(o.m[i], qm[i]), i
        assert np.array_equal(o.v[i], qv[i]), i
        assert np.array_equal(o.m_scale[i].view(np.uint32), sm[i].view(np.uint32)), i
        assert np.array_equal(o.v_scale[i].view(np.uint32), sv[i].view(np.uint32)), i
        assert np.array_equal(th_o[i], th_bits[i]), i


# ------------------------------------------------------------ the pin bites

V_EXPR = "(s->one_minus_beta2 * g) * g"
TH_EXPR = "(s->lr * m_hat) / denom"
MUTANTS = {
    "v with (1-beta2)*(g*g)": [(V_EXPR, "s->one_minus_beta2 * (g * g)")],
    "theta with lr*(m_hat/den)": [(TH_EXPR, "s->lr * (m_hat / denom)")],
}


def _build_variant(tmp_path, name, edits, extra_flags=()):
    src = open(oracle.SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, "the oracle no longer holds %r" % old
        src = src.replace(old, new)
    c = tmp_path / (name + ".c")
    c.write_text(src)
    so = tmp_path / (name + ".so")
    flags = list(extra_flags) or ["-ffp-contract=off"]
    subprocess.check_call(["gcc", "-O2", "-std=c11", *flags, "-fno-fast-math", "-fPIC",
                           "-shared", "-o", str(so), str(c), "-lm"])
    return str(so)


def _mismatch_under(monkeypatch, path):
    monkeypatch.setattr(oracle, "_lib", oracle.load(path))
    try:
        test_oracle_is_the_literal_box_bit_for_bit("f32")
    except AssertionError:
        return True
    finally:
        monkeypatch.undo()
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_regrouped_oracle_fails_the_pin(tmp_path, monkeypatch, name):
    path = _build_variant(tmp_path, "v%d" % sorted(MUTANTS).index(name), MUTANTS[name])
    assert _mismatch_under(monkeypatch, path), name


def test_contracted_oracle_fails_the_pin(tmp_path, monkeypatch):
    if os.uname().machine != "x86_64":
        pytest.skip("the contraction variant is built with x86 FMA")
    path = _build_variant(tmp_path, "fma", [], extra_flags=["-mfma", "-ffp-contract=fast"])
    assert _mismatch_under(monkeypatch, path)


def test_unchanged_rebuild_passes_the_pin(tmp_path, monkeypatch):
    path = _build_variant(tmp_path, "same", [])
    assert not _mismatch_under(monkeypatch, path)
