"""The tolerance checks themselves: sharp enough to catch a dropped rounding
point, loose enough to pass a faithful fp32 run.

TensorFold PR #1260's controls: each drops one rounding point (the sum before
the norm, the slerp's a, its b) and must go red; an fp16 sum on integer rows
must overflow to zero outputs.  Here they are numpy fp32 models of a kernel
(tests/kernel_models.py).
"""
import numpy as np
import pytest

import kernel_models as km
from oracle.bf16 import bf16_rne, bf16_value
from oracle.check import (admissible_l2_rows, admissible_rownorm,
                          admissible_slerp_rows, contract_bf16, contract_rel)
from oracle.rows import l2_rows, slerp_rows, weight_rownorm_gain
from scale_invariant_row_amd import inputs


@pytest.fixture(scope="module")
def l2in():
    return inputs.l2_case(128, 4096, 301, residual=True)


@pytest.fixture(scope="module")
def stress():
    return inputs.stress_l2_case(rows=400, cols=2048, seed=302)


@pytest.fixture(scope="module")
def slin():
    return inputs.slerp_case(96, 4096, 303)


def test_faithful_l2_passes(l2in):
    y = km.l2_model(l2in.x, l2in.r)
    rep = admissible_l2_rows(y, l2in.x, l2in.r)
    assert rep.ok, str(rep)
    assert contract_bf16(y, l2_rows(l2in.x, l2in.r)).all()


def test_faithful_l2_passes_stress(stress):
    y = km.l2_model(stress.x, stress.r)
    rep = admissible_l2_rows(y, stress.x, stress.r)
    assert rep.ok, str(rep)


def test_control_unrounded_sum_fails(l2in):
    y = km.l2_model(l2in.x, l2in.r, round_s=False)
    rep = admissible_l2_rows(y, l2in.x, l2in.r)
    assert rep.outside > 100, str(rep)


def test_control_fp16_sum_fails_on_integer_rows(stress):
    rows = stress.meta["int_rows"]
    x, r = stress.x[rows], stress.r[rows]
    y = km.l2_model(x, r, acc="f16")
    assert not bf16_value(y).any()            # the fp16 sum overflowed: zero rows
    rep = admissible_l2_rows(y, x, r)
    assert rep.outside > 0.9 * y.size
    y32 = km.l2_model(x, r)
    assert admissible_l2_rows(y32, x, r).ok
    # integer rows: every fp32 partial sum is an exact integer < 2**24
    assert admissible_l2_rows(y32, x, r, depth=0).ok


def test_control_bf16_sum_fails(l2in):
    y = km.l2_model(l2in.x, l2in.r, acc="bf16")
    rep = admissible_l2_rows(y, l2in.x, l2in.r)
    assert rep.outside > 1000, str(rep)


def test_faithful_slerp_passes(slin):
    h = km.slerp_model(slin.res, slin.out, slin.alpha)
    rep = admissible_slerp_rows(h, slin.res, slin.out, slin.alpha)
    assert rep.ok, str(rep)
    assert contract_bf16(h, slerp_rows(slin.res, slin.out, slin.alpha)).all()


@pytest.mark.parametrize("drop", ["a", "b"])
def test_control_unrounded_a_or_b_fails(slin, drop):
    h = km.slerp_model(slin.res, slin.out, slin.alpha,
                       round_a=(drop != "a"), round_b=(drop != "b"))
    rep = admissible_slerp_rows(h, slin.res, slin.out, slin.alpha)
    assert rep.outside > 100, str(rep)


def test_faithful_rownorm_passes():
    case = inputs.rownorm_case([(300, 768), (100, 3072)], 304)
    for w, g in zip(case.w, case.gain):
        n, we = km.rownorm_model(w, g)
        rn, rw = admissible_rownorm(n, we, w, g)
        assert rn.ok and rw.ok, (str(rn), str(rw))
        ref_n, ref_w = weight_rownorm_gain([w], [g], [1.0])
        assert contract_rel(n, ref_n[0]).all()
        assert contract_bf16(we, ref_w[0], zero_sign=False).all()


def test_rownorm_control_wrong_gain_fails():
    case = inputs.rownorm_case([(200, 768)], 305)
    w, g = case.w[0], case.gain[0]
    n, we = km.rownorm_model(w, g * np.float32(1.01))
    _, rw = admissible_rownorm(n, we, w, g)
    assert rw.outside > 1000


def test_contract_flags_two_ulp_error(l2in):
    y = l2_rows(l2in.x, l2in.r)
    bad = y.copy()
    bad[3, 10] = bad[3, 10] + 2                 # two bf16 ulps away
    ok = contract_bf16(bad, y)
    assert not ok[3, 10] and ok.sum() == y.size - 1
    one = y.copy()
    one[5, 5] = one[5, 5] + 1
    assert contract_bf16(one, y).all()
    rep = admissible_l2_rows(bad, l2in.x, l2in.r)
    assert rep.outside >= 1


def test_contract_special_values():
    nan, inf, ninf = 0x7FC0, 0x7F80, 0xFF80
    want = np.array([nan, inf, 0x0000, 0x8000, 0x3F80], np.uint16)
    assert contract_bf16(want, want).all()
    got = np.array([0x3F80, ninf, 0x8000, 0x8000, 0x3F81], np.uint16)
    assert list(contract_bf16(got, want)) == [False, False, False, True, True]
    assert contract_bf16(got[2:4], want[2:4], zero_sign=False).all()


def test_nonfinite_rows_exact_pattern():
    x = bf16_rne(np.random.default_rng(3).standard_normal((3, 64)))
    x[0, 5] = 0x7F80            # +inf: finite elements -> 0, the inf -> NaN
    x[1, 9] = 0x7FC0            # NaN: the whole row NaN
    y = l2_rows(x)
    assert np.isnan(bf16_value(y[0, 5])) and not bf16_value(np.delete(y[0], 5)).any()
    assert np.isnan(bf16_value(y[1])).all()
    assert admissible_l2_rows(y, x).ok
    bad = y.copy()
    bad[0, 0] = 0x3F80
    assert not admissible_l2_rows(bad, x).ok
