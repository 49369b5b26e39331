"""The activation-row checks themselves: a faithful fp32 run passes, and each
of the pages' controls (TensorFold PR #1260's activation-row commit: drop the
gated row's rounding, the scaled gate's, the scaled up's, or the product's)
fails the strict check."""
import numpy as np
import pytest

import kernel_models as km
from oracle.bf16 import bf16_rne, bf16_value
from oracle.check import (act_unique_mask, admissible_act_rows, contract_bf16, gate_candidates,
                          swiglu_candidates)
from oracle.rows import gate_l2_rows, swiglu_l2_rows


@pytest.fixture(scope="module")
def gate_in():
    rng = np.random.default_rng(321)
    o = bf16_rne(rng.standard_normal((64, 4096)))
    g = bf16_rne(rng.standard_normal((64, 4096)) * 2)
    sg = rng.uniform(0.5, 2.0, 4096).astype(np.float32)
    return o, g, sg


@pytest.fixture(scope="module")
def swiglu_in():
    rng = np.random.default_rng(322)
    g = bf16_rne(rng.standard_normal((48, 7168)))
    u = bf16_rne(rng.standard_normal((48, 7168)))
    sug = rng.uniform(0.5, 3.0, 7168).astype(np.float32)
    suu = rng.uniform(0.5, 3.0, 7168).astype(np.float32)
    return g, u, sug, suu


def test_faithful_gate_passes(gate_in):
    o, g, sg = gate_in
    y = km.gate_model(o, g, sg)
    lo, hi = gate_candidates(o, g, sg)
    rep = admissible_act_rows(y, lo, hi)
    assert rep.ok, str(rep)
    uniq = act_unique_mask(lo, hi)
    assert uniq.mean() > 0.99
    assert contract_bf16(y, gate_l2_rows(o, g, sg))[uniq].all()


def test_gate_control_fails(gate_in):
    o, g, sg = gate_in
    y = km.gate_model(o, g, sg, round_t=False)
    lo, hi = gate_candidates(o, g, sg)
    rep = admissible_act_rows(y, lo, hi)
    assert rep.outside > 100, str(rep)


def test_faithful_swiglu_passes(swiglu_in):
    g, u, sug, suu = swiglu_in
    y = km.swiglu_model(g, u, sug, suu)
    lo, hi = swiglu_candidates(g, u, sug, suu)
    rep = admissible_act_rows(y, lo, hi)
    assert rep.ok, str(rep)
    uniq = act_unique_mask(lo, hi)
    assert uniq.mean() > 0.99
    assert contract_bf16(y, swiglu_l2_rows(g, u, sug, suu))[uniq].all()


@pytest.mark.parametrize("drop", ["round_a", "round_b", "round_p"])
def test_swiglu_controls_fail(swiglu_in, drop):
    g, u, sug, suu = swiglu_in
    y = km.swiglu_model(g, u, sug, suu, **{drop: False})
    lo, hi = swiglu_candidates(g, u, sug, suu)
    rep = admissible_act_rows(y, lo, hi)
    assert rep.outside > 100, str(rep)


def test_saturated_gate_admits_fp32_zero():
    """exp beyond fp32's range: fp32 gives sigmoid 0, float64 a subnormal; both pass."""
    o = bf16_rne(np.full((1, 64), 3.0e38))
    g = bf16_rne(np.full((1, 64), -88.8))
    sg = np.ones(64, np.float32)
    lo, hi = gate_candidates(o, g, sg)
    assert (lo[0] == 0).all() and (hi[0] > 0).all()


def test_gate_fp16_sum_control_fails_on_half_integer_rows():
    """The pages' gate 4 for the gate: with g = 0, sigmoid is 1/2 and each
    gated row holds halves of integers, exact in fp32, so the fp32 sums are
    exact (depth 0 passes); an fp16 sum overflows to zero outputs and fails."""
    rng = np.random.default_rng(323)
    o = bf16_rne(rng.integers(-64, 65, (16, 4096)).astype(float))
    g = bf16_rne(np.zeros((16, 4096)))
    sg = rng.uniform(0.5, 2.0, 4096).astype(np.float32)
    lo, hi = gate_candidates(o, g, sg)
    assert (lo == hi).all() and (lo == bf16_value(o) / 2).all()
    y32 = km.gate_model(o, g, sg)
    assert admissible_act_rows(y32, lo, hi, depth=0).ok
    y16 = km.gate_model(o, g, sg, acc="f16")
    assert not bf16_value(y16).any()                 # the fp16 sum overflowed: zero rows
    rep = admissible_act_rows(y16, lo, hi)
    assert rep.outside > 0.9 * y16.size, str(rep)


def test_swiglu_fp16_sum_control_fails():
    """The pages' gate 4 for SwiGLU: its squares are not integers, so the fp32
    sums are checked against the depth bound; an fp16 sum overflows on rows of
    the MLP width whose squares add past fp16's range, and fails."""
    rng = np.random.default_rng(324)
    g = bf16_rne(rng.standard_normal((16, 7168)) * 4)
    u = bf16_rne(rng.standard_normal((16, 7168)) * 4)
    sug = rng.uniform(0.5, 2.0, 7168).astype(np.float32)
    suu = rng.uniform(0.5, 2.0, 7168).astype(np.float32)
    lo, hi = swiglu_candidates(g, u, sug, suu)
    assert admissible_act_rows(km.swiglu_model(g, u, sug, suu), lo, hi).ok
    y16 = km.swiglu_model(g, u, sug, suu, acc="f16")
    assert not bf16_value(y16).any()
    rep = admissible_act_rows(y16, lo, hi)
    assert rep.outside > 0.9 * y16.size, str(rep)
