"""The activation-row oracle (gate_l2_rows, swiglu_l2_rows) against what
fixes it independently: hand-derived closed forms
(tests/golden/activation_closed_forms.json), scipy's logistic function,
exact rational arithmetic with 60-digit exponentials, invariants, and
planted mistakes.
"""
import numpy as np
import pytest
from scipy.special import expit

import golden_cases as gc
from oracle import brute
from oracle.bf16 import bf16_rne, bf16_value
from oracle.rows import (_l2_of_values, _sigmoid64, eps_as_passed, gate_gated_row, gate_l2_rows,
                         swiglu_l2_rows, swiglu_product_row)
from test_oracle_brute import _frac_row_to_bits

CASES = gc.load("activation_closed_forms.json")


def _bits(v):
    return bf16_rne(np.asarray(v, dtype=np.float64))


def _vec(case, key, cols):
    if key in case:
        return gc.row(case[key], cols).astype(np.float32)
    return np.ones(cols, np.float32)


def _run(case, gate_fn=gate_l2_rows, swiglu_fn=swiglu_l2_rows):
    cols = case["cols"]
    if case["op"] == "gate_l2_rows":
        o = _bits(gc.row(case["o"], cols))[None]
        g = _bits(gc.row(case["g"], cols))[None]
        return gate_fn(o, g, _vec(case, "sg", cols), 1e-6)[0]
    g = _bits(gc.row(case["g"], cols))[None]
    u = _bits(gc.row(case["u"], cols))[None]
    return swiglu_fn(g, u, _vec(case, "sug", cols), _vec(case, "suu", cols), 1e-6)[0]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] + "-" + c["op"] for c in CASES])
def test_closed_form(case):
    got = bf16_value(_run(case))
    assert np.array_equal(got, gc.expected(case["expect"], case["cols"])), got[:4]


def test_sigmoid_matches_scipy():
    x = np.concatenate([np.linspace(-120, 120, 20001), np.random.default_rng(3).normal(0, 8, 10000)])
    assert np.allclose(_sigmoid64(x), expit(x), rtol=4e-16, atol=0)


# ------------------------------------------------------------ exact arithmetic

def _act_rows(rng, n, cols_choices):
    for k in range(n):
        cols = int(rng.choice(cols_choices))
        kind = k % 5
        if kind == 0:
            a, b = rng.standard_normal(cols), rng.standard_normal(cols)
        elif kind == 1:                                   # large gate arguments: saturation
            a, b = rng.standard_normal(cols) * 40, rng.standard_normal(cols)
        elif kind == 2:                                   # wide dynamic range
            a = rng.standard_normal(cols) * np.exp2(rng.integers(-30, 8, cols))
            b = rng.standard_normal(cols) * np.exp2(rng.integers(-40, 40, cols))
        elif kind == 3:                                   # small integers (the pages' gate 4)
            a, b = rng.integers(-8, 9, cols).astype(float), rng.integers(-64, 65, cols).astype(float)
        else:
            a, b = rng.standard_normal(cols) * 3, rng.standard_normal(cols) * 1e-3
        s1 = rng.uniform(0.25, 4.0, cols).astype(np.float32)
        s2 = rng.uniform(0.25, 4.0, cols).astype(np.float32)
        yield bf16_rne(a), bf16_rne(b), s1, s2


def test_gate_matches_exact():
    rng = np.random.default_rng(606)
    flagged = 0
    for k, (g, o, sg, _) in enumerate(_act_rows(rng, 150, [8, 16, 40])):
        eps = [1e-6, 0.0, 0.5][k % 3]
        if eps == 0.0 and not bf16_value(gate_gated_row(o[None], g[None], sg)).any():
            continue
        got = gate_l2_rows(o[None], g[None], sg, eps)[0]
        want, near = brute.gate_row(o, g, sg, float(np.float32(eps)))
        wb = _frac_row_to_bits(want)
        diff = (got != wb) & ~((bf16_value(got) == 0) & (bf16_value(wb) == 0))
        assert not (diff & ~np.array(near)).any(), (k, np.nonzero(diff)[0])
        flagged += int(any(near))
    assert flagged <= 8


def test_swiglu_matches_exact():
    rng = np.random.default_rng(707)
    flagged = 0
    for k, (g, u, sug, suu) in enumerate(_act_rows(rng, 150, [8, 16, 40])):
        eps = [1e-6, 0.0, 0.5][k % 3]
        if eps == 0.0 and not bf16_value(swiglu_product_row(g[None], u[None], sug, suu)).any():
            continue
        got = swiglu_l2_rows(g[None], u[None], sug, suu, eps)[0]
        want, near = brute.swiglu_row(g, u, sug, suu, float(np.float32(eps)))
        wb = _frac_row_to_bits(want)
        diff = (got != wb) & ~((bf16_value(got) == 0) & (bf16_value(wb) == 0))
        assert not (diff & ~np.array(near)).any(), (k, np.nonzero(diff)[0])
        flagged += int(any(near))
    assert flagged <= 8


# ------------------------------------------------------------------ invariants

@pytest.fixture(scope="module")
def rows():
    rng = np.random.default_rng(808)
    a = bf16_rne(rng.standard_normal((16, 256)))
    b = bf16_rne(rng.standard_normal((16, 256)))
    s1 = rng.uniform(0.5, 2, 256).astype(np.float32)
    s2 = rng.uniform(0.5, 2, 256).astype(np.float32)
    return a, b, s1, s2


def test_gate_integer_rows_halve_exactly(rows):
    """The pages' gate-4 rows: g = 0 halves integer rows exactly."""
    o = bf16_rne(np.random.default_rng(9).integers(-64, 65, (4, 256)).astype(float))
    t = bf16_value(gate_gated_row(o, np.zeros_like(o), rows[2]))
    assert np.array_equal(t, bf16_value(o) / 2)


def test_power_of_two_scale_invariance(rows):
    g, o, sg, s2 = rows
    base = gate_l2_rows(o, g, sg, 0.0)
    for k in (-7, 5):
        assert np.array_equal(gate_l2_rows(bf16_rne(bf16_value(o) * 2.0 ** k), g, sg, 0.0), base)
    base = swiglu_l2_rows(g, o, sg, s2, 0.0)
    assert np.array_equal(swiglu_l2_rows(g, o, sg, s2 * np.float32(8), 0.0), base)


def test_signs(rows):
    g, o, sg, s2 = rows
    flip = np.uint16(0x8000)
    assert np.array_equal(bf16_value(gate_l2_rows(o ^ flip, g, sg)), -bf16_value(gate_l2_rows(o, g, sg)))
    assert np.array_equal(bf16_value(swiglu_l2_rows(g, o ^ flip, sg, s2)),
                          -bf16_value(swiglu_l2_rows(g, o, sg, s2)))


def test_sigmoid_symmetry_in_the_gate(rows):
    """sigmoid(-x) = 1 - sigmoid(x): the gated rows of g and -g add up to o."""
    g, o, sg, _ = rows
    t1 = bf16_value(gate_gated_row(o, g, sg))
    t2 = bf16_value(gate_gated_row(o, g ^ np.uint16(0x8000), sg))
    # each gated value is rounded to bf16 once: the sum is o within two half-ulps
    ov = bf16_value(o)
    assert np.all(np.abs(t1 + t2 - ov) <= 2.0 ** -8 * (np.abs(t1) + np.abs(t2)) + 1e-30)


def test_row_independence_and_permutation(rows):
    g, o, sg, s2 = rows
    y = swiglu_l2_rows(g, o, sg, s2)
    assert np.array_equal(swiglu_l2_rows(g[3:7], o[3:7], sg, s2), y[3:7])
    perm = np.random.default_rng(10).permutation(256)
    yp = bf16_value(swiglu_l2_rows(g[:, perm], o[:, perm], sg[perm], s2[perm]))
    assert np.allclose(yp, bf16_value(y)[:, perm], rtol=2 ** -7, atol=0)


# ------------------------------------------------------------ planted mistakes

def _gate_variant(kind):
    def fn(o_bits, g_bits, sg, eps):
        o = bf16_value(o_bits)
        if kind == "scale_on_o":
            o = o * sg
            x = bf16_value(g_bits)
        else:
            x = (bf16_value(g_bits).astype(np.float32) * sg).astype(np.float64)
        sig = 1.0 / (1.0 + np.exp(x if kind == "sign" else -x))
        t = o * sig if kind == "unrounded" else bf16_value(bf16_rne(o * sig))
        return bf16_rne(_l2_of_values(t, eps_as_passed(eps)))
    return fn


def _swiglu_variant(kind):
    def fn(g_bits, u_bits, sug, suu, eps):
        a = bf16_value(bf16_rne((bf16_value(g_bits).astype(np.float32) * sug).astype(np.float64)))
        b = bf16_value(bf16_rne((bf16_value(u_bits).astype(np.float32)
                                 * (sug if kind == "swapped" else suu)).astype(np.float64)))
        sig = 1.0 / (1.0 + np.exp(-a))
        silu = sig if kind == "sigmoid_only" else a * sig
        p = bf16_value(bf16_rne(silu * b))
        return bf16_rne(_l2_of_values(p, eps_as_passed(eps)))
    return fn


def test_planted_mistakes_fail_closed_forms():
    def fails(gate_fn=gate_l2_rows, swiglu_fn=swiglu_l2_rows):
        return any(not np.array_equal(bf16_value(_run(c, gate_fn, swiglu_fn)),
                                      gc.expected(c["expect"], c["cols"])) for c in CASES)
    assert not fails(gate_fn=_gate_variant("faithful"), swiglu_fn=_swiglu_variant("faithful"))
    for kind in ("sign", "scale_on_o"):
        assert fails(gate_fn=_gate_variant(kind)), kind
    for kind in ("sigmoid_only", "swapped"):
        assert fails(swiglu_fn=_swiglu_variant(kind)), kind
