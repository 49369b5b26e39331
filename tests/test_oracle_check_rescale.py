"""The rescale checks themselves: a faithful fp32 run passes; a projection
dividing by ||w|| instead of ||w||^2, or none at all, fails."""
import numpy as np
import pytest

import kernel_models as km
from oracle.check import admissible_rescale, contract_grad, contract_rel, rescale_terms
from oracle.rows import rescale_after_step


@pytest.fixture(scope="module")
def wv():
    rng = np.random.default_rng(341)
    w = (rng.standard_normal((64, 768)) * 0.02).astype(np.float32)
    w[3] = 0
    v = (rng.standard_normal((64, 768)) * 1e-3).astype(np.float32)
    return w, v


def test_faithful_passes(wv):
    w, v = wv
    for rho in (1.0, 27.7):
        gw, gv = km.rescale_model(w, v, rho)
        rw, rv = admissible_rescale(gw, gv, w, v, rho)
        assert rw.ok and rv.ok, (str(rw), str(rv))
        ws, ms = rescale_after_step([w], [v], [rho])
        assert contract_rel(gw, ws[0]).all()
        terms = rescale_terms(w.astype(np.float64), v.astype(np.float64))
        assert contract_grad(gv, ms[0], terms, "f32").all()


@pytest.mark.parametrize("ctl", [dict(k_over_norm=True), dict(project=False)])
def test_controls_fail(wv, ctl):
    w, v = wv
    gw, gv = km.rescale_model(w, v, 1.0, **ctl)
    _, rv = admissible_rescale(gw, gv, w, v, 1.0)
    assert rv.outside > 1000, str(rv)
