"""The gradient checks themselves: a faithful fp32 run passes, plausible
mistakes fail.

numpy fp32 models of a backward kernel (tests/kernel_models.py) stand in for
one: the faithful model must meet both the contract and the strict interval
check; each control (an unrounded residual sum, the projection taken on the
rounded forward output, a bf16 accumulator, eps left out) must fail the
strict check.
"""
import numpy as np
import pytest

import kernel_models as km
from oracle.bf16 import bf16_rne, bf16_value
from oracle.check import (admissible_l2_backward, admissible_rownorm_backward,
                          contract_grad, l2_grad_terms, rownorm_grad_terms)
from oracle.rows import (eps_as_passed, l2_rows_backward, weight_rownorm_gain_backward)
from scale_invariant_row_amd import inputs


def _dy(shape, seed):
    return bf16_rne(np.random.default_rng(seed).standard_normal(shape))


@pytest.fixture(scope="module")
def l2in():
    c = inputs.l2_case(96, 4096, 311, residual=True)
    return c, _dy(c.x.shape, 312)


@pytest.fixture(scope="module")
def stress():
    c = inputs.stress_l2_case(rows=300, cols=2048, seed=313)
    return c, _dy(c.x.shape, 314)


def _s(c):
    return bf16_value(bf16_rne(bf16_value(c.x) + bf16_value(c.r)))


def test_faithful_l2_backward_passes(l2in):
    c, dy = l2in
    ds = km.l2_backward_model(c.x, c.r, dy)
    rep = admissible_l2_backward(ds, c.x, c.r, dy)
    assert rep.ok, str(rep)
    assert rep.wide < 0.002 * rep.n, str(rep)       # the check stays sharp
    want = l2_rows_backward(c.x, c.r, dy)
    terms = l2_grad_terms(_s(c), bf16_value(dy), eps_as_passed(1e-6))
    assert contract_grad(ds, want, terms).all()


def test_faithful_l2_backward_passes_stress(stress):
    c, dy = stress
    ds = km.l2_backward_model(c.x, c.r, dy)
    rep = admissible_l2_backward(ds, c.x, c.r, dy)
    assert rep.ok, str(rep)
    want = l2_rows_backward(c.x, c.r, dy)
    terms = l2_grad_terms(_s(c), bf16_value(dy), eps_as_passed(1e-6))
    assert contract_grad(ds, want, terms).all()


@pytest.mark.parametrize("ctl", ["unrounded_s", "project_on_y", "bf16_acc"])
def test_l2_backward_controls_fail(l2in, ctl):
    c, dy = l2in
    kw = {"unrounded_s": dict(round_s=False), "project_on_y": dict(proj="y"),
          "bf16_acc": dict(acc="bf16")}[ctl]
    ds = km.l2_backward_model(c.x, c.r, dy, **kw)
    rep = admissible_l2_backward(ds, c.x, c.r, dy)
    assert rep.outside > 100, str(rep)


def test_l2_backward_no_eps_fails_on_zero_rows(stress):
    c, dy = stress
    rows = stress[0].meta["zero_rows"]
    ds = km.l2_backward_model(c.x[rows], c.r[rows], dy[rows], use_eps=False)
    rep = admissible_l2_backward(ds, c.x[rows], c.r[rows], dy[rows])
    assert rep.outside > 0.9 * ds.size, str(rep)


@pytest.fixture(scope="module")
def wcase():
    c = inputs.rownorm_case([(64, 768), (32, 3072)], 315)
    de = [_dy(w.shape, 316 + i) for i, w in enumerate(c.w)]
    return c, de


def test_faithful_rownorm_backward_passes(wcase):
    c, de = wcase
    want_dw, want_dg = weight_rownorm_gain_backward(c.w, c.gain, c.radius, de)
    for i, w in enumerate(c.w):
        dw, dg = km.rownorm_backward_model(w, c.gain[i], c.radius[i], de[i])
        rw, rg = admissible_rownorm_backward(dw, dg, w, c.gain[i], c.radius[i], de[i])
        assert rw.ok and rg.ok, (str(rw), str(rg))
        tw, tg = rownorm_grad_terms(w.astype(np.float64), c.gain[i].astype(np.float64),
                                    float(np.float32(c.radius[i])), bf16_value(de[i]))
        assert contract_grad(dw, want_dw[i], tw, "f32").all()
        assert contract_grad(dg, want_dg[i], tg, "f32").all()


@pytest.mark.parametrize("ctl", ["bf16_acc", "project_on_weff"])
def test_rownorm_backward_controls_fail(wcase, ctl):
    c, de = wcase
    kw = {"bf16_acc": dict(acc="bf16"), "project_on_weff": dict(proj="weff")}[ctl]
    dw, dg = km.rownorm_backward_model(c.w[0], c.gain[0], c.radius[0], de[0], **kw)
    rw, rg = admissible_rownorm_backward(dw, dg, c.w[0], c.gain[0], c.radius[0], de[0])
    assert rw.outside > 100 and rg.outside > 10, (str(rw), str(rg))


def test_rownorm_backward_zero_row_and_exact_zeros(wcase):
    c, de = wcase
    w = c.w[0].copy()
    w[5] = 0
    dw, dg = km.rownorm_backward_model(w, c.gain[0], c.radius[0], de[0])
    rw, rg = admissible_rownorm_backward(dw, dg, w, c.gain[0], c.radius[0], de[0])
    assert rw.ok and rg.ok
    dw[5, 3] = 1e-30                                   # a zero row must stay exactly zero
    rw, _ = admissible_rownorm_backward(dw, dg, w, c.gain[0], c.radius[0], de[0])
    assert rw.outside == 1
