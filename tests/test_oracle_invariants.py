"""Invariants of the row ops, checked on the oracle.

Properties fixed by the mathematics of the definitions (TensorFold PR #1260's
row kernels, the DragonScale README's W_eff), independent of how the oracle
computes them: unit length, gain-scaled length, the step-0 identity, alpha = 0
and alpha = 1, res == out, sign and operand symmetry, scale invariance,
column-permutation equivariance and row independence.
"""
import numpy as np
import pytest

from oracle.bf16 import bf16_rne, bf16_value
from oracle.rows import (l2_rows, slerp_rows, slerp_rows_detail,
                         weight_rownorm_gain)
from scale_invariant_row_amd import inputs


@pytest.fixture(scope="module")
def l2in():
    return inputs.l2_case(48, 1024, 77, residual=True)


@pytest.fixture(scope="module")
def slin():
    return inputs.slerp_case(32, 768, 78)


def test_unit_length(l2in):
    y = bf16_value(l2_rows(l2in.x, l2in.r, 1e-6))
    n = np.sqrt((y ** 2).sum(axis=1))
    # each element is rounded by at most half a bf16 ulp (2**-9 relative)
    assert np.all(np.abs(n - 1) <= 2 ** -8)


def test_residual_is_commutative(l2in):
    assert np.array_equal(l2_rows(l2in.x, l2in.r), l2_rows(l2in.r, l2in.x))


def test_odd_symmetry(l2in):
    neg = l2in.x ^ np.uint16(0x8000)
    assert np.array_equal(l2_rows(neg), l2_rows(l2in.x) ^ np.uint16(0x8000))


def test_power_of_two_scale_invariance(l2in):
    x = bf16_value(l2in.x)
    for k in (-20, -3, 5, 30):
        xs = bf16_rne(x * 2.0 ** k)
        # eps = 0: exactly invariant
        assert np.array_equal(l2_rows(xs, None, 0.0), l2_rows(l2in.x, None, 0.0))
        if k < -3:
            continue        # there S << eps: eps rightly dominates
        # eps = 1e-6 only moves values by eps/S (< 1e-7 here): at most one ulp
        a = bf16_value(l2_rows(xs, None, 1e-6))
        b = bf16_value(l2_rows(l2in.x, None, 1e-6))
        assert np.all(np.abs(a - b) <= np.abs(b) * 2 ** -7)


def test_column_permutation_equivariance(l2in):
    perm = np.random.default_rng(5).permutation(l2in.cols)
    y = l2_rows(l2in.x, l2in.r)
    yp = l2_rows(l2in.x[:, perm], l2in.r[:, perm])
    assert np.array_equal(yp, y[:, perm])


def test_row_independence(l2in):
    y = l2_rows(l2in.x, l2in.r)
    assert np.array_equal(l2_rows(l2in.x[7:19], l2in.r[7:19]), y[7:19])


def test_slerp_alpha_zero_gives_a(slin):
    a, _, u, h = slerp_rows_detail(slin.res, slin.out, np.zeros(slin.cols, np.float32))
    assert np.array_equal(u, bf16_value(a).astype(np.float32))
    assert np.array_equal(h, l2_rows(a, None, 1e-6))


def test_slerp_alpha_one_gives_b_when_exact(slin):
    a, b, u, h = slerp_rows_detail(slin.res, slin.out, np.ones(slin.cols, np.float32))
    av, bv = bf16_value(a), bf16_value(b)
    exact = (bv - av).astype(np.float32).astype(np.float64) == bv - av
    assert exact.all()      # differences of bf16 values of similar size are exact
    assert np.array_equal(h, l2_rows(b, None, 1e-6))


def test_slerp_equal_inputs_for_any_alpha(slin):
    alpha = np.random.default_rng(9).uniform(-3, 3, slin.cols).astype(np.float32)
    a, _, _, h = slerp_rows_detail(slin.res, slin.res, alpha)
    assert np.array_equal(h, l2_rows(a, None, 1e-6))


def test_slerp_alpha_sign(slin):
    assert np.array_equal(slerp_rows(slin.res, slin.out, slin.alpha),
                          slerp_rows(slin.res, slin.out, -slin.alpha))


def test_slerp_unit_length(slin):
    h = bf16_value(slerp_rows(slin.res, slin.out, slin.alpha))
    assert np.all(np.abs(np.sqrt((h ** 2).sum(axis=1)) - 1) <= 2 ** -8)


def test_rownorm_gain_scaled_length():
    case = inputs.rownorm_case([(40, 96), (24, 256)], 79)
    norms, weffs = weight_rownorm_gain(case.w, case.gain, case.radius)
    for w, g, n, we in zip(case.w, case.gain, norms, weffs):
        ref = np.sqrt((w.astype(np.float64) ** 2).sum(axis=1))
        assert np.allclose(n, ref, rtol=1e-7, atol=0)
        length = np.sqrt((bf16_value(we) ** 2).sum(axis=1))
        assert np.all(np.abs(length / g - 1) <= 2 ** -8)


def test_rownorm_step0_identity():
    """g = ||W_i|| gives W_eff = bf16(W) (same output at step 0).

    DragonScale README, "Patching options": init=preserve sets the gain to the
    row length.  The identity is exact up to float64 rounding of g w / n, so
    elements of w within 2**-40 (relative) of a bf16 midpoint are excluded.
    """
    case = inputs.rownorm_case([(64, 128)], 80)
    w = case.w[0]
    n = np.sqrt((w.astype(np.float64) ** 2).sum(axis=1))
    norms, weffs = weight_rownorm_gain([w], [n], [1.0])
    want = bf16_rne(w.astype(np.float64))
    wv = w.astype(np.float64)
    lo = bf16_value(bf16_rne(wv * (1 - 2.0 ** -40)))
    hi = bf16_value(bf16_rne(wv * (1 + 2.0 ** -40)))
    clear = lo == hi
    assert clear.mean() > 0.999
    assert np.array_equal(weffs[0][clear], want[clear])


def test_rownorm_radius_scales_linearly():
    case = inputs.rownorm_case([(16, 64)], 81)
    _, w1 = weight_rownorm_gain(case.w, case.gain, [1.0])
    _, w4 = weight_rownorm_gain(case.w, case.gain, [4.0])
    assert np.array_equal(bf16_value(w4[0]), 4 * bf16_value(w1[0]))


# ---- planted mistakes: a plausible slip in the oracle must fail a pin -------

def _l2_variant(x_bits, eps, *, drop_eps=False, drop_sqrt=False, sign=1.0):
    x = bf16_value(x_bits)
    s2 = (x ** 2).sum(axis=1, keepdims=True)
    d = s2 if drop_sqrt else np.sqrt(s2 + (0.0 if drop_eps else float(np.float32(eps))))
    return bf16_rne(sign * x / d)


def test_planted_mistakes_fail_closed_forms():
    import golden_cases as gc
    cases = {c["name"]: c for c in gc.load()}
    eps_case = cases["eps_pin"]
    x = bf16_rne(gc.row(eps_case["x"], eps_case["cols"]))[None]
    want = gc.expected(eps_case["expect"], eps_case["cols"])
    assert np.array_equal(bf16_value(_l2_variant(x, 1e-6))[0], want)
    assert not np.array_equal(bf16_value(_l2_variant(x, 1e-6, drop_eps=True))[0], want)
    tf = cases["three_four"]
    x = bf16_rne(gc.row(tf["x"], tf["cols"]))[None]
    want = gc.expected(tf["expect"], tf["cols"])
    assert not np.array_equal(bf16_value(_l2_variant(x, 1e-6, drop_sqrt=True))[0], want)
    assert not np.array_equal(bf16_value(_l2_variant(x, 1e-6, sign=-1.0))[0], want)


def test_planted_lerp_mistakes_fail_alpha_pins(slin):
    """alpha instead of |alpha|, or (a - b) for (b - a), break the alpha pins."""
    a, b, _, h = slerp_rows_detail(slin.res, slin.out, slin.alpha)
    av = bf16_value(a).astype(np.float32)
    bv = bf16_value(b).astype(np.float32)
    wrong_sign = av + slin.alpha * (bv - av)          # alpha not made absolute
    swapped = av + np.abs(slin.alpha) * (av - bv)     # operands transposed
    for u in (wrong_sign, swapped):
        hw = l2_rows(bf16_rne(u.astype(np.float64)), None, 1e-6)
        assert not np.array_equal(hw, h)
