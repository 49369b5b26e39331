"""The strict checks in their RMSNorm mode: a faithful fp32 run of rms_rows
and of its gradient passes; plausible mistakes fail.

numpy fp32 models of a kernel (tests/kernel_models.py) stand in for one.
Controls: the sum not divided by the row's length (l2_rows), eps added to
the sum before the division, the residual sum left unrounded, an fp16
accumulator on integer rows; for the gradient, P left undivided and eps
dropped on zero rows.
"""
import numpy as np
import pytest

import kernel_models as km
from oracle.bf16 import bf16_rne, bf16_value
from oracle.check import admissible_l2_backward, admissible_l2_rows, contract_bf16, \
    contract_grad, l2_grad_terms
from oracle.rows import eps_as_passed, rms_rows, rms_rows_backward
from scale_invariant_row_amd import inputs


@pytest.fixture(scope="module")
def case():
    c = inputs.l2_case(96, 768, 331, residual=True)
    dy = bf16_rne(np.random.default_rng(332).standard_normal(c.x.shape))
    return c, dy


@pytest.fixture(scope="module")
def small():
    """Rows of size ~1e-3, where mean(s^2) is comparable to eps."""
    rng = np.random.default_rng(333)
    x = bf16_rne(rng.standard_normal((64, 512)) * 1e-3)
    return x, bf16_rne(rng.standard_normal((64, 512)))


@pytest.fixture(scope="module")
def stress():
    c = inputs.stress_l2_case(rows=300, cols=2048, seed=334)
    dy = bf16_rne(np.random.default_rng(335).standard_normal(c.x.shape))
    return c, dy


def test_faithful_forward_passes(case, small, stress):
    for x, r in ((case[0].x, case[0].r), (small[0], None), (stress[0].x, stress[0].r)):
        y = km.l2_model(x, r, mean=True)
        rep = admissible_l2_rows(y, x, r, mean=True)
        assert rep.ok and rep.loose == 0, str(rep)
        assert contract_bf16(y, rms_rows(x, r)).all()


@pytest.mark.parametrize("ctl", ["no_mean", "unrounded_s"])
def test_forward_controls_fail(case, ctl):
    c, _ = case
    kw = {"no_mean": dict(mean=False), "unrounded_s": dict(mean=True, round_s=False)}[ctl]
    rep = admissible_l2_rows(km.l2_model(c.x, c.r, **kw), c.x, c.r, mean=True)
    assert rep.outside > 100, str(rep)


def test_eps_on_sum_fails_on_small_rows(small):
    x, _ = small
    rep = admissible_l2_rows(km.l2_model(x, None, mean=True, eps_on_sum=True), x, None, mean=True)
    assert rep.outside > 0.5 * x.size, str(rep)


def test_fp16_accumulator_fails_on_integer_rows(stress):
    c, _ = stress
    rows = c.meta["int_rows"]
    y = km.l2_model(c.x[rows], c.r[rows], mean=True, acc="f16")
    rep = admissible_l2_rows(y, c.x[rows], c.r[rows], mean=True)
    assert rep.outside > 0.5 * y.size, str(rep)


def test_faithful_backward_passes(case, small, stress):
    for x, r, dy in ((case[0].x, case[0].r, case[1]), (small[0], None, small[1]),
                     (stress[0].x, stress[0].r, stress[1])):
        ds = km.l2_backward_model(x, r, dy, mean=True)
        rep = admissible_l2_backward(ds, x, r, dy, mean=True)
        assert rep.ok, str(rep)
        xs = bf16_value(x)
        s = xs if r is None else bf16_value(bf16_rne(xs + bf16_value(r)))
        terms = l2_grad_terms(s, bf16_value(dy), eps_as_passed(1e-6), mean=True)
        assert contract_grad(ds, rms_rows_backward(x, r, dy), terms).all()


def test_backward_controls_fail(case, stress):
    c, dy = case
    rep = admissible_l2_backward(km.l2_backward_model(c.x, c.r, dy, mean=True, k_mean=False),
                                 c.x, c.r, dy, mean=True)
    assert rep.outside > 100, str(rep)
    rep = admissible_l2_backward(km.l2_backward_model(c.x, c.r, dy, mean=False),
                                 c.x, c.r, dy, mean=True)
    assert rep.outside > 100, str(rep)
    s, sdy = stress
    rows = s.meta["zero_rows"]
    ds = km.l2_backward_model(s.x[rows], s.r[rows], sdy[rows], mean=True, use_eps=False)
    rep = admissible_l2_backward(ds, s.x[rows], s.r[rows], sdy[rows], mean=True)
    assert rep.outside > 0.9 * ds.size, str(rep)
