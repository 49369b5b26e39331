"""The backward oracle against what fixes it independently of its own formulas.

* hand-derived closed forms (tests/golden/backward_closed_forms.json);
* torch autograd in float64 through the forward definitions: the Jacobian is
  derived mechanically from y = s / sqrt(sum s^2 + eps) and from
  W_eff = g r w / ||w|| (DragonScale README, "What DragonScale changes"), not
  from the oracle's hand-derived projection;
* central finite differences of the forward;
* invariants: <ds, s> = <s, dy> eps / D^3, <dW, w> = 0, g dg = <dWe, W_eff>,
  power-of-two homogeneity, sign symmetries, the residual fan-out;
* exact rational arithmetic on tiny rows (oracle.brute);
* plausible slips planted in a copy of the backward fail one of these.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import golden_cases as gc
from oracle import brute
from oracle.bf16 import bf16_rne, bf16_value
from oracle.rows import (_l2_of_values, eps_as_passed, l2_backward_values, l2_rows_backward,
                         rownorm_backward_values, weight_rownorm_gain_backward)
from test_oracle_brute import _frac_row_to_bits, _rows

CASES = gc.load("backward_closed_forms.json")


def _bits(v):
    return bf16_rne(np.asarray(v, dtype=np.float64))


def _f32(v):
    return np.asarray(v, dtype=np.float64).astype(np.float32)


# ------------------------------------------------------------ closed forms

def _run_case(case, l2_fn=None, rn_fn=None):
    """(got, want) value arrays for one fixture; the fns replace the oracle's."""
    cols = case["cols"]
    exp = case["expect"]
    if case["op"] == "l2_rows_backward":
        s = _bits(gc.row(case["s"], cols))[None]
        dy = _bits(gc.row(case["dy"], cols))[None]
        if l2_fn is None:
            got = bf16_value(l2_rows_backward(s, None, dy, 1e-6))[0]
        else:
            got = bf16_value(bf16_rne(l2_fn(bf16_value(s), bf16_value(dy),
                                            eps_as_passed(1e-6))))[0]
        return [got], [gc.expected(exp, cols)]
    w = _f32(gc.row(case["w"], cols))[None]
    g = np.array([case["g"]], np.float32)
    de = _bits(gc.row(case["dwe"], cols))[None]
    if rn_fn is None:
        dws, dgs = weight_rownorm_gain_backward([w], [g], [case["rho"]], [de])
        dw, dg = dws[0][0], dgs[0][0]
    else:
        dw, dg = rn_fn(w.astype(np.float64), g.astype(np.float64),
                       float(np.float32(case["rho"])), bf16_value(de))
        dw, dg = dw.astype(np.float32)[0], np.float32(dg[0])
    want_dw = _f32(gc.expected(exp["dw"], cols))
    return [dw, np.array([dg])], [want_dw, np.array([np.float32(exp["dg"])])]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] + "-" + c["op"] for c in CASES])
def test_closed_form(case):
    for got, want in zip(*_run_case(case)):
        assert np.array_equal(np.asarray(got, np.float64), np.asarray(want, np.float64)), \
            (case["name"], got[:4], want[:4])


def test_l2_zero_gradients_are_positive_zero():
    case = next(c for c in CASES if c["name"] == "three_four")
    s = _bits(gc.row(case["s"], 64))[None]
    dy = _bits(gc.row(case["dy"], 64))[None]
    got = bf16_value(l2_rows_backward(s, None, dy, 1e-6))[0]
    assert not np.signbit(got[2:]).any()


# ------------------------------------------------------------- autograd

def _random_rows(rng, rows, cols, kind):
    if kind == "normal":
        v = rng.standard_normal((rows, cols))
    elif kind == "tiny":                         # eps dominates the norm
        v = rng.standard_normal((rows, cols)) * 2.0 ** -12
    elif kind == "wide":
        v = rng.standard_normal((rows, cols)) * np.exp2(rng.integers(-20, 20, (rows, cols)))
    else:                                        # sparse
        v = rng.standard_normal((rows, cols)) * (rng.random((rows, cols)) < 0.1)
    return bf16_value(bf16_rne(v))


def _l2_scale(s, dy, eps64):
    """Per element, the size of the terms whose difference forms ds."""
    d2 = (s ** 2).sum(axis=1, keepdims=True) + eps64
    a = np.abs(s * dy).sum(axis=1, keepdims=True)
    return (np.abs(dy) + np.abs(s) * a / d2) / np.sqrt(d2)


@pytest.mark.parametrize("kind", ["normal", "tiny", "wide", "sparse"])
@pytest.mark.parametrize("eps", [1e-6, 0.0, 0.5])
def test_l2_backward_matches_autograd(kind, eps):
    rng = np.random.default_rng(zlib.crc32(f"{kind} {eps}".encode()))
    s = _random_rows(rng, 24, 96, kind)
    dy = bf16_value(bf16_rne(rng.standard_normal(s.shape)))
    eps64 = eps_as_passed(eps)
    if eps64 == 0.0:
        s[:, 0] = np.where((s == 0).all(axis=1), 1.0, s[:, 0])
    st = torch.tensor(s, dtype=torch.float64, requires_grad=True)
    y = st / torch.sqrt((st * st).sum(dim=1, keepdim=True) + eps64)
    y.backward(torch.tensor(dy, dtype=torch.float64))
    want = st.grad.numpy()
    got = l2_backward_values(s, dy, eps64)
    assert np.all(np.abs(got - want) <= 1e-13 * _l2_scale(s, dy, eps64))


@pytest.mark.parametrize("scale", [0.02, 2.0 ** 40, 2.0 ** -40])
def test_rownorm_backward_matches_autograd(scale):
    rng = np.random.default_rng(int(math.log2(scale) + 100))
    w = _f32(rng.standard_normal((20, 80)) * scale).astype(np.float64)
    w[3] = 0.0
    g = _f32(rng.uniform(-2, 2, 20)).astype(np.float64)
    rho = float(np.float32(math.sqrt(80)))
    de = bf16_value(bf16_rne(rng.standard_normal(w.shape)))
    wt = torch.tensor(w, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    ss = (wt * wt).sum(dim=1, keepdim=True)
    n = torch.sqrt(torch.where(ss == 0, torch.ones_like(ss), ss))
    weff = gt[:, None] * rho * wt / n
    # the zero row is scaled by the constant 0: no gradient
    weff = torch.where(torch.tensor(w == 0).all(dim=1, keepdim=True), 0 * weff, weff)
    weff.backward(torch.tensor(de))
    dw, dg = rownorm_backward_values(w, g, rho, de)
    nrm = np.sqrt((w ** 2).sum(axis=1, keepdims=True))
    nrm[3] = 1.0
    sc = np.abs(g * rho)[:, None] / nrm * (
        np.abs(de) + np.abs(w) * np.abs(w * de).sum(axis=1, keepdims=True) / nrm ** 2)
    assert np.all(np.abs(dw - wt.grad.numpy()) <= 1e-13 * sc)
    assert np.allclose(dg, gt.grad.numpy(), rtol=1e-13, atol=0)
    assert not dw[3].any() and dg[3] == 0


# --------------------------------------------------- finite differences

def test_l2_backward_finite_differences():
    rng = np.random.default_rng(7)
    eps64 = eps_as_passed(1e-6)
    s = _random_rows(rng, 12, 64, "normal")
    dy = bf16_value(bf16_rne(rng.standard_normal(s.shape)))
    ds = l2_backward_values(s, dy, eps64)
    for _ in range(3):
        v = rng.standard_normal(s.shape)
        h = 1e-6
        fd = ((_l2_of_values(s + h * v, eps64) - _l2_of_values(s - h * v, eps64)) * dy
              ).sum(axis=1) / (2 * h)
        an = (ds * v).sum(axis=1)
        assert np.allclose(fd, an, rtol=1e-7, atol=1e-9)


def _weff_values(w, g, rho):
    n = np.sqrt((w ** 2).sum(axis=1, keepdims=True))
    return g[:, None] * rho * w / n


def test_rownorm_backward_finite_differences():
    rng = np.random.default_rng(8)
    w = _f32(rng.standard_normal((10, 48)) * 0.02).astype(np.float64)
    g = _f32(rng.uniform(0.5, 2, 10)).astype(np.float64)
    de = bf16_value(bf16_rne(rng.standard_normal(w.shape)))
    dw, dg = rownorm_backward_values(w, g, 1.0, de)
    h = 1e-9
    for _ in range(3):
        v = rng.standard_normal(w.shape)
        fd = ((_weff_values(w + h * v, g, 1.0) - _weff_values(w - h * v, g, 1.0)) * de
              ).sum(axis=1) / (2 * h)
        assert np.allclose(fd, (dw * v).sum(axis=1), rtol=1e-6, atol=1e-6)
    hg = 1e-6
    fdg = ((_weff_values(w, g + hg, 1.0) - _weff_values(w, g - hg, 1.0)) * de).sum(axis=1) / (2 * hg)
    assert np.allclose(fdg, dg, rtol=1e-8, atol=1e-10)


# ------------------------------------------------------------ invariants

def test_l2_backward_radial_component():
    """<ds, s> = <s, dy> eps / D^3: the gradient is tangent up to eps."""
    rng = np.random.default_rng(9)
    for eps in (1e-6, 0.25, 0.0):
        eps64 = eps_as_passed(eps)
        s = _random_rows(rng, 16, 128, "normal")
        dy = bf16_value(bf16_rne(rng.standard_normal(s.shape)))
        ds = l2_backward_values(s, dy, eps64)
        for i in range(s.shape[0]):
            d2 = math.fsum(s[i] ** 2) + eps64
            p = math.fsum(s[i] * dy[i])
            lhs = math.fsum(ds[i] * s[i])
            assert abs(lhs - p * eps64 / d2 ** 1.5) <= 1e-14 * math.fsum(np.abs(ds[i] * s[i])) \
                + 1e-14 * abs(p) / math.sqrt(d2)


def test_rownorm_backward_tangent_and_gain_identity():
    rng = np.random.default_rng(10)
    w = _f32(rng.standard_normal((16, 96)) * 0.02).astype(np.float64)
    g = _f32(rng.uniform(0.5, 2, 16)).astype(np.float64)
    rho = 3.0
    de = bf16_value(bf16_rne(rng.standard_normal(w.shape)))
    dw, dg = rownorm_backward_values(w, g, rho, de)
    weff = _weff_values(w, g, rho)
    for i in range(16):
        assert abs(math.fsum(dw[i] * w[i])) <= 1e-14 * math.fsum(np.abs(dw[i] * w[i]))
        assert abs(g[i] * dg[i] - math.fsum(de[i] * weff[i])) <= \
            1e-14 * math.fsum(np.abs(de[i] * weff[i]))


def test_power_of_two_homogeneity():
    rng = np.random.default_rng(11)
    x = bf16_rne(rng.standard_normal((8, 64)))
    dy = bf16_rne(rng.standard_normal((8, 64)))
    base = bf16_value(l2_rows_backward(x, None, dy, 0.0))
    for k in (-9, -2, 3, 17):
        xs = bf16_rne(bf16_value(x) * 2.0 ** k)
        got = bf16_value(l2_rows_backward(xs, None, dy, 0.0))
        assert np.array_equal(got, base * 2.0 ** -k)
    w = _f32(rng.standard_normal((8, 64)) * 0.02)
    g = _f32(rng.uniform(0.5, 2, 8))
    dws, dgs = weight_rownorm_gain_backward([w], [g], [1.0], [dy])
    for k in (-30, 5):
        dws2, dgs2 = weight_rownorm_gain_backward([w * np.float32(2.0 ** k)], [g], [1.0], [dy])
        assert np.array_equal(dws2[0], dws[0] * np.float32(2.0 ** -k))
        assert np.array_equal(dgs2[0], dgs[0])
    dws3, dgs3 = weight_rownorm_gain_backward([w], [g * 2], [1.0], [dy])
    assert np.array_equal(dws3[0], dws[0] * 2) and np.array_equal(dgs3[0], dgs[0])


def test_sign_symmetries_and_residual_fan_out():
    rng = np.random.default_rng(12)
    x = bf16_rne(rng.standard_normal((8, 64)))
    r = bf16_rne(rng.standard_normal((8, 64)))
    dy = bf16_rne(rng.standard_normal((8, 64)))
    base = l2_rows_backward(x, r, dy)
    assert np.array_equal(base, l2_rows_backward(r, x, dy))
    flip = np.uint16(0x8000)
    # y(-s) = -y(s): the Jacobian is even in s
    assert np.array_equal(bf16_value(l2_rows_backward(x ^ flip, r ^ flip, dy)), bf16_value(base))
    # linear in dy
    assert np.array_equal(bf16_value(l2_rows_backward(x, r, dy ^ flip)), -bf16_value(base))


# ------------------------------------------------------- exact arithmetic

def test_l2_backward_matches_exact():
    rng = np.random.default_rng(404)
    disagree = 0
    for k, x in enumerate(_rows(rng, 300, [8, 16, 24, 40, 64])):
        eps = [1e-6, 0.0, 1.0, 3e-4][k % 4]
        use_r = k % 2 == 1
        r = bf16_rne(rng.standard_normal(x.size)) if use_r else None
        dy = bf16_rne(rng.standard_normal(x.size) * np.exp2(rng.integers(-10, 10)))
        if k % 7 == 3:          # dy nearly radial: ds cancels
            dy = bf16_rne(bf16_value(x) * 1.5 + 1e-3 * rng.standard_normal(x.size))
        s = bf16_value(x) if r is None else bf16_value(bf16_rne(bf16_value(x) + bf16_value(r)))
        if not np.isfinite(s).all() or (eps == 0.0 and not s.any()):
            continue
        got = l2_rows_backward(x[None], None if r is None else r[None], dy[None], eps)[0]
        want, near = brute.l2_backward_row(x, r, dy, float(np.float32(eps)))
        want_bits = _frac_row_to_bits(want)
        diff = (got != want_bits) & ~((bf16_value(got) == 0) & (bf16_value(want_bits) == 0))
        assert not (diff & ~np.array(near)).any(), (k, np.nonzero(diff)[0])
        disagree += int(diff.sum())
    assert disagree <= 3


def test_rownorm_backward_matches_exact():
    rng = np.random.default_rng(505)
    flagged = 0
    for k in range(200):
        cols = int(rng.choice([8, 12, 32, 48]))
        scale = float(np.exp2(rng.integers(-60, 60))) if k % 3 == 0 else 0.02
        w = _f32(rng.standard_normal(cols) * scale)
        g = np.float32(rng.uniform(-2.0, 2.0))
        rho = [1.0, 1.0, float(np.sqrt(np.float32(cols)))][k % 3]
        de = bf16_rne(rng.standard_normal(cols) * np.exp2(rng.integers(-8, 8)))
        dws, dgs = weight_rownorm_gain_backward([w[None]], [np.array([g])], [rho], [de[None]])
        want_dw, want_dg, near, near_g = brute.rownorm_backward_row(w, float(g), rho, de)
        assert near_g or dgs[0][0] == np.float32(float(want_dg)), k
        want = np.array([float(v) for v in want_dw], np.float32)
        diff = dws[0][0] != want
        assert not (diff & ~np.array(near)).any(), (k, np.nonzero(diff)[0])
        flagged += int(np.sum(near)) + int(near_g)
    assert flagged <= 20


# ------------------------------------------------------- planted mistakes

def _l2_mutant(kind):
    def fn(s, dy, eps64):
        out = np.empty_like(s)
        for i in range(s.shape[0]):
            d2 = math.fsum(s[i] ** 2) + (0.0 if kind == "drop_eps" else eps64)
            p = math.fsum(s[i] * dy[i])
            d = math.sqrt(d2)
            if kind == "k_over_D":
                out[i] = (dy[i] - s[i] * (p / d)) / d
            elif kind == "plus":
                out[i] = (dy[i] + s[i] * (p / d2)) / d
            elif kind == "no_final_div":
                out[i] = dy[i] - s[i] * (p / d2)
            elif kind == "div_D2":
                out[i] = (dy[i] - s[i] * (p / d2)) / d2
            else:
                out[i] = (dy[i] - s[i] * (p / d2)) / d
        return out
    return fn


def _rn_mutant(kind):
    def fn(w, g, rho, de):
        dw = np.zeros_like(w)
        dg = np.zeros(w.shape[0])
        for i in range(w.shape[0]):
            ss = math.fsum(w[i] ** 2)
            n = math.sqrt(ss)
            if n == 0:
                continue
            p = math.fsum(w[i] * de[i])
            dg[i] = {"dg_gain": g[i] * p / n, "dg_no_norm": rho * p}.get(kind, rho * p / n)
            coef = g[i] / n if kind == "no_radius" else g[i] * rho / n
            proj = p / n if kind == "proj_over_n" else p / ss
            dw[i] = coef * (de[i] - w[i] * proj)
        return dw, dg
    return fn


def _fails_some_case(l2_fn=None, rn_fn=None):
    for case in CASES:
        if (case["op"] == "l2_rows_backward") != (l2_fn is not None):
            continue
        for got, want in zip(*_run_case(case, l2_fn, rn_fn)):
            if not np.array_equal(np.asarray(got, np.float64), np.asarray(want, np.float64)):
                return True
    return False


def test_planted_mistakes_fail_closed_forms():
    assert not _fails_some_case(l2_fn=_l2_mutant("faithful"))
    assert not _fails_some_case(rn_fn=_rn_mutant("faithful"))
    for kind in ("drop_eps", "k_over_D", "plus", "no_final_div", "div_D2"):
        assert _fails_some_case(l2_fn=_l2_mutant(kind)), kind
    for kind in ("dg_gain", "dg_no_norm", "no_radius", "proj_over_n"):
        assert _fails_some_case(rn_fn=_rn_mutant(kind)), kind
