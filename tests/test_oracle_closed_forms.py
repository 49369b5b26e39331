"""The oracle against hand-derived closed forms (tests/golden/closed_forms.json)."""
import numpy as np
import pytest

import golden_cases as gc
from oracle.bf16 import bf16_rne, bf16_value
from oracle.rows import l2_rows, slerp_rows, weight_rownorm_gain

CASES = gc.load()


def _bits(v):
    return bf16_rne(np.asarray(v, dtype=np.float64))


@pytest.mark.parametrize("case", CASES, ids=[c["name"] + "-" + c["op"] for c in CASES])
def test_closed_form(case):
    cols = case["cols"]
    exp = case["expect"]
    if case["op"] == "l2_rows":
        x = _bits(gc.row(case["x"], cols))[None]
        r = _bits(gc.row(case["r"], cols))[None] if "r" in case else None
        got = l2_rows(x, r, 1e-6)[0]
    elif case["op"] == "slerp_rows":
        res = _bits(gc.row(case["res"], cols))[None]
        out = _bits(gc.row(case["out"], cols))[None]
        alpha = gc.row(case["alpha"], cols).astype(np.float32)
        got = slerp_rows(res, out, alpha, 1e-6)[0]
    else:
        w = gc.row(case["w"], cols).astype(np.float32)[None]
        g = np.array([case["g"]], np.float32)
        norms, weffs = weight_rownorm_gain([w], [g], [case["rho"]])
        assert norms[0][0] == np.float32(exp["norm"])
        got = weffs[0][0]
    want = gc.expected(exp, cols)
    assert np.array_equal(bf16_value(got), want)
    if "bits" in exp:
        assert (got == int(exp["bits"], 16)).all()
    if want.min() == 0 and case["op"] != "rownorm":
        # zeros produced from +0 inputs are +0
        assert not np.signbit(bf16_value(got)[want == 0]).any()
