"""The seeded workload generators: deterministic, shaped and structured as stated."""
import numpy as np

from oracle.bf16 import bf16_value
from scale_invariant_row_amd import inputs


def test_deterministic():
    a = inputs.l2_case(16, 512, 5)
    b = inputs.l2_case(16, 512, 5)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.r, b.r)
    c = inputs.l2_case(16, 512, 6)
    assert not np.array_equal(a.x, c.x)
    s1 = inputs.slerp_case(4, 256, 9)
    s2 = inputs.slerp_case(4, 256, 9)
    assert np.array_equal(s1.alpha, s2.alpha) and np.array_equal(s1.out, s2.out)


def test_distributions():
    s = inputs.slerp_case(256, 1024, 10)
    res, out = bf16_value(s.res), bf16_value(s.out)
    assert abs(res.std() - 1) < 0.01 and abs(out.std() - 2) < 0.02
    assert s.alpha.dtype == np.float32 and np.abs(s.alpha).max() <= 0.2
    w = inputs.rownorm_case([(512, 768)], 11)
    assert abs(w.w[0].std() - 0.02) < 2e-4
    assert w.gain[0].min() >= 0.5 and w.gain[0].max() <= 2.0


def test_transformer_shapes():
    shapes = inputs.transformer_linears()
    assert len(shapes) == 48
    assert sum(r for r, _ in shapes) == 82944
    assert sum(r * c for r, c in shapes) == 84934656
    assert shapes[:4] == [(2304, 768), (768, 768), (3072, 768), (768, 3072)]


def test_stress_structure():
    c = inputs.stress_l2_case(rows=1000, cols=512, seed=12)
    x, r = bf16_value(c.x), bf16_value(c.r)
    z, ir = c.meta["zero_rows"], c.meta["int_rows"]
    assert len(z) == 10 and len(ir) == 10 and not set(z) & set(ir)
    assert not x[z].any() and not r[z].any()
    assert not r[ir].any()
    xi = x[ir]
    assert np.array_equal(xi, np.round(xi)) and np.abs(xi).max() <= 64
    assert ((xi ** 2).sum(axis=1) < 2 ** 24).all()
    normal = np.setdiff1d(np.arange(1000), np.concatenate([z, ir]))
    big = (np.abs(x[normal]) > 50).mean()
    assert 0.005 < big < 0.015
