"""The rescale method's row ops (DragonScale README, "Optimizer") on the
oracle, against hand-derived closed forms, exact arithmetic, the reduction
to the weight gradient's tangent projection, invariants and planted mistakes."""
import math

import numpy as np
import pytest

import golden_cases as gc
from oracle import brute
from oracle.bf16 import bf16_rne
from oracle.rows import (rescale_after_step, rescale_project, rescale_project_values,
                         rownorm_backward_values)

CASES = gc.load("rescale_closed_forms.json")


def _f32(spec, cols):
    return gc.row(spec, cols).astype(np.float32)[None]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_closed_form(case):
    cols = case["cols"]
    w = _f32(case["w"], cols)
    if "expect_v" in case:
        got = rescale_project([w], [_f32(case["v"], cols)])[0][0]
        assert np.array_equal(got, gc.expected(case["expect_v"], cols).astype(np.float32)), got[:4]
    if "expect_w" in case:
        ws, _ = rescale_after_step([w], [None], [case["rho"]])
        want = gc.expected(case["expect_w"], cols).astype(np.float32)
        assert np.array_equal(ws[0][0], want), ws[0][0][:4]


def _rows(seed, rows=12, cols=96):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((rows, cols)) * 0.02).astype(np.float32)
    v = (rng.standard_normal((rows, cols)) * 1e-3).astype(np.float32)
    return w, v


def test_matches_exact():
    rng = np.random.default_rng(610)
    flagged = 0
    for k in range(120):
        cols = int(rng.choice([8, 12, 32]))
        scale = float(np.exp2(rng.integers(-60, 60))) if k % 3 == 0 else 0.02
        w = (rng.standard_normal(cols) * scale).astype(np.float32)
        v = (rng.standard_normal(cols) * np.exp2(rng.integers(-20, 5))).astype(np.float32)
        if k % 7 == 0:
            v = (w * np.float32(3.0) + rng.standard_normal(cols).astype(np.float32) * 1e-4 * scale).astype(np.float32)
        rho = [1.0, 2.0, float(np.sqrt(np.float32(cols)))][k % 3]
        ws, ms = rescale_after_step([w[None]], [v[None]], [rho])
        w_ex, v_ex, near = brute.rescale_row(w, v, rho)
        want_w = np.array([float(x) for x in w_ex], np.float32)
        want_v = np.array([float(x) for x in v_ex], np.float32)
        nr = np.array(near)
        assert not ((ws[0][0] != want_w) & ~nr).any(), k
        assert not ((ms[0][0] != want_v) & ~nr).any(), k
        flagged += int(nr.sum())
    assert flagged <= 10


def test_projection_is_the_weight_gradients_tangent_projection():
    """(I - w_hat w_hat^T) v is the unit-row weight gradient with g = ||w||, r = 1."""
    w, v = _rows(611)
    w64, v64 = w.astype(np.float64), v.astype(np.float64)
    n = np.sqrt((w64 ** 2).sum(axis=1))
    dw, _ = rownorm_backward_values(w64, n, 1.0, v64)
    assert np.allclose(rescale_project_values(w64, v64), dw, rtol=1e-13, atol=1e-18)


def test_tangent_and_idempotent():
    w, v = _rows(612)
    p = rescale_project([w], [v])[0]
    for i in range(w.shape[0]):
        terms = np.abs(w[i].astype(np.float64) * p[i])
        assert abs(math.fsum(w[i].astype(np.float64) * p[i])) <= 2.0 ** -22 * math.fsum(terms) + 1e-40
    p2 = rescale_project([w], [p])[0]
    assert np.allclose(p2, p, rtol=0, atol=2.0 ** -22 * np.abs(v).max())


def test_rescaled_rows_have_the_radius_and_keep_direction():
    w, _ = _rows(613)
    for rho in (1.0, 27.7128, 0.5):
        ws, _ = rescale_after_step([w], [None], [rho])
        n = np.sqrt((ws[0].astype(np.float64) ** 2).sum(axis=1))
        assert np.all(np.abs(n - np.float32(rho)) <= 4 * 2.0 ** -24 * np.float32(rho))
        cos = (ws[0].astype(np.float64) * w).sum(1) / (n * np.sqrt((w.astype(np.float64) ** 2).sum(1)))
        assert np.all(np.abs(cos - 1) <= 1e-12)


def test_scale_invariance():
    w, v = _rows(614)
    for k in (-40, 7):
        ws = (w * np.float32(2.0 ** k)).astype(np.float32)
        assert np.array_equal(rescale_project([ws], [v])[0], rescale_project([w], [v])[0])
        assert np.array_equal(rescale_after_step([ws], [None], [1.0])[0][0],
                              rescale_after_step([w], [None], [1.0])[0][0])


def _variant(kind):
    def project(w, v):
        out = []
        for wm, vm in zip(w, v):
            w64, v64 = wm.astype(np.float64), vm.astype(np.float64)
            o = v64.copy()
            for i in range(w64.shape[0]):
                ss = math.fsum(w64[i] ** 2)
                if ss == 0:
                    continue
                p = math.fsum(w64[i] * v64[i])
                k = p / math.sqrt(ss) if kind == "over_norm" else p / ss
                o[i] = v64[i] + w64[i] * k if kind == "plus" else v64[i] - w64[i] * k
            out.append(o.astype(np.float32))
        return out
    return project


def test_planted_mistakes_fail_closed_forms():
    def fails(fn):
        for c in CASES:
            if "expect_v" not in c:
                continue
            got = fn([_f32(c["w"], c["cols"])], [_f32(c["v"], c["cols"])])[0][0]
            if not np.array_equal(got, gc.expected(c["expect_v"], c["cols"]).astype(np.float32)):
                return True
        return False
    assert not fails(_variant("faithful"))
    assert fails(_variant("plus")) and fails(_variant("over_norm"))
