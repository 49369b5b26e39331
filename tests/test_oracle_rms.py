"""The RMSNorm oracle (the ternary/8-bit GPT model page's parameter-free
rms_norm) against what fixes it independently of its own formulas.

* hand-derived closed forms (tests/golden/rms_closed_forms.json);
* torch's own rms_norm in float64, and autograd through it for the gradient;
* l2_rows with eps scaled by n: at n = 4^k the two must agree bit for bit up
  to the exact factor 2^k (y = sqrt(n) s / sqrt(sum s^2 + n eps));
* exact rational arithmetic on tiny rows (oracle.brute);
* central finite differences, <ds, s> = <s, dy> eps / D^3, power-of-two
  homogeneity, sign symmetry, the residual fan-out, column permutations;
* plausible slips planted in copies of the definitions fail the closed forms.
"""
import math

import numpy as np
import pytest
import torch

import golden_cases as gc
from oracle import brute
from oracle.bf16 import bf16_rne, bf16_value
from oracle.rows import (_rms_of_values, eps_as_passed, l2_rows, rms_backward_values, rms_rows,
                         rms_rows_backward)
from test_oracle_brute import _frac_row_to_bits, _rows

CASES = gc.load("rms_closed_forms.json")
FWD = [c for c in CASES if c["op"] == "rms_rows"]
BWD = [c for c in CASES if c["op"] == "rms_rows_backward"]


def _bits(v):
    return bf16_rne(np.asarray(v, dtype=np.float64))


def _normal_bits(rng, shape, scale=1.0):
    return _bits(rng.standard_normal(shape) * scale)


# ------------------------------------------------------------ closed forms

def _fwd_case(case, fn=None):
    s = _bits(gc.row(case["s"], case["cols"]))[None]
    if fn is None:
        got = bf16_value(rms_rows(s, None, 1e-6))[0]
    else:
        got = bf16_value(bf16_rne(fn(bf16_value(s), eps_as_passed(1e-6))))[0]
    return got, gc.expected(case["expect"], case["cols"])


def _bwd_case(case, fn=None):
    cols = case["cols"]
    s = _bits(gc.row(case["s"], cols))[None]
    dy = _bits(gc.row(case["dy"], cols))[None]
    if fn is None:
        got = bf16_value(rms_rows_backward(s, None, dy, 1e-6))[0]
    else:
        got = bf16_value(bf16_rne(fn(bf16_value(s), bf16_value(dy), eps_as_passed(1e-6))))[0]
    return got, gc.expected(case["expect"], cols)


@pytest.mark.parametrize("case", FWD, ids=[c["name"] for c in FWD])
def test_forward_closed_form(case):
    got, want = _fwd_case(case)
    assert np.array_equal(got, want), (case["name"], got[:4], want[:4])
    assert not np.signbit(got[want == 0]).any()


@pytest.mark.parametrize("case", BWD, ids=[c["name"] for c in BWD])
def test_backward_closed_form(case):
    got, want = _bwd_case(case)
    assert np.array_equal(got, want), (case["name"], got[:4], want[:4])


# ------------------------------------------------------- torch's rms_norm

def _near_midpoint(v, rel=2.0 ** -40):
    """float64 values within rel of a bf16 rounding midpoint."""
    with np.errstate(all="ignore"):
        return bf16_rne(v * (1 - rel)) != bf16_rne(v * (1 + rel))


@pytest.mark.parametrize("eps", [1e-6, 0.0, 0.25])
@pytest.mark.parametrize("cols", [8, 320, 768, 1000])
def test_forward_matches_torch_rms_norm(eps, cols):
    rng = np.random.default_rng(cols * 7 + int(eps * 100))
    x = _normal_bits(rng, (16, cols))
    x[3] = _normal_bits(rng, cols, 2.0 ** -12)           # eps dominates the mean
    x[5] = _bits(rng.integers(-64, 65, cols).astype(float))
    eps64 = eps_as_passed(eps)
    t = torch.nn.functional.rms_norm(torch.tensor(bf16_value(x)), (cols,), eps=eps64).numpy()
    got = rms_rows(x, None, eps)
    want = bf16_rne(t)
    diff = got != want
    assert not (diff & ~_near_midpoint(t)).any(), np.argwhere(diff)[:4]
    assert diff.sum() <= 2


def test_backward_matches_torch_autograd():
    rng = np.random.default_rng(21)
    for eps in (1e-6, 0.0, 0.5):
        eps64 = eps_as_passed(eps)
        for kind_scale in (1.0, 2.0 ** -12, 2.0 ** 30):
            s = bf16_value(_normal_bits(rng, (12, 96), kind_scale))
            dy = bf16_value(_normal_bits(rng, s.shape))
            st = torch.tensor(s, requires_grad=True)
            torch.nn.functional.rms_norm(st, (96,), eps=eps64).backward(torch.tensor(dy))
            got = rms_backward_values(s, dy, eps64)
            d2 = (s ** 2).mean(axis=1, keepdims=True) + eps64
            sc = (np.abs(dy) + np.abs(s) * np.abs(s * dy).sum(axis=1, keepdims=True)
                  / (96 * d2)) / np.sqrt(d2)
            assert np.all(np.abs(got - st.grad.numpy()) <= 1e-13 * sc), (eps, kind_scale)


# -------------------------------------------------- l2_rows with eps * n

@pytest.mark.parametrize("k", [1, 3, 5, 6])
def test_l2_with_eps_scaled_by_n(k):
    """n = 4^k: rms(s, eps) = 2^k l2(s, n eps), exactly, before and after rounding."""
    n = 4 ** k
    rng = np.random.default_rng(300 + k)
    x = _normal_bits(rng, (24, n))
    x[2] = _normal_bits(rng, n, 2.0 ** -12)
    r = _normal_bits(rng, (24, n))
    eps32 = float(np.float32(1e-6))
    ln = l2_rows(x, r, eps32 * n)                      # n eps32 is an fp32 value
    want = bf16_value(ln) * 2.0 ** k
    assert np.array_equal(bf16_value(rms_rows(x, r, eps32)), want)


# ---------------------------------------------------------- exact values

def test_forward_matches_exact():
    rng = np.random.default_rng(606)
    disagree = 0
    for k, x in enumerate(_rows(rng, 300, [8, 12, 24, 40, 64])):
        eps = [1e-6, 0.0, 1.0, 3e-4][k % 4]
        r = _normal_bits(rng, x.size) if k % 2 else None
        s = bf16_value(x) if r is None else bf16_value(bf16_rne(bf16_value(x) + bf16_value(r)))
        if not np.isfinite(s).all() or (eps == 0.0 and not s.any()):
            continue
        got = rms_rows(x[None], None if r is None else r[None], eps)[0]
        want, near = brute.rms_row(x, r, float(np.float32(eps)))
        wb = _frac_row_to_bits(want)
        zero = (bf16_value(got) == 0) & (bf16_value(wb) == 0)
        assert np.array_equal(np.signbit(bf16_value(got))[zero], np.signbit(s)[zero]), k
        diff = (got != wb) & ~zero
        assert not (diff & ~np.array(near)).any(), (k, np.nonzero(diff)[0])
        disagree += int(diff.sum())
    assert disagree <= 3


def test_backward_matches_exact():
    rng = np.random.default_rng(707)
    disagree = 0
    for k, x in enumerate(_rows(rng, 300, [8, 16, 24, 40, 64])):
        eps = [1e-6, 0.0, 1.0, 3e-4][k % 4]
        r = _normal_bits(rng, x.size) if k % 2 else None
        dy = _bits(rng.standard_normal(x.size) * np.exp2(rng.integers(-10, 10)))
        if k % 7 == 3:                                  # dy nearly radial: ds cancels
            dy = _bits(bf16_value(x) * 1.5 + 1e-3 * rng.standard_normal(x.size))
        s = bf16_value(x) if r is None else bf16_value(bf16_rne(bf16_value(x) + bf16_value(r)))
        if not (np.isfinite(s).all() and np.isfinite(bf16_value(dy)).all()) or \
                (eps == 0.0 and not s.any()):
            continue
        got = rms_rows_backward(x[None], None if r is None else r[None], dy[None], eps)[0]
        want, near = brute.rms_backward_row(x, r, dy, float(np.float32(eps)))
        wb = _frac_row_to_bits(want)
        diff = (got != wb) & ~((bf16_value(got) == 0) & (bf16_value(wb) == 0))
        assert not (diff & ~np.array(near)).any(), (k, np.nonzero(diff)[0])
        disagree += int(diff.sum())
    assert disagree <= 3


# ------------------------------------------------------------- invariants

def test_backward_finite_differences():
    rng = np.random.default_rng(23)
    eps64 = eps_as_passed(1e-6)
    s = bf16_value(_normal_bits(rng, (12, 64)))
    dy = bf16_value(_normal_bits(rng, s.shape))
    ds = rms_backward_values(s, dy, eps64)
    for _ in range(3):
        v = rng.standard_normal(s.shape)
        h = 1e-6
        fd = ((_rms_of_values(s + h * v, eps64) - _rms_of_values(s - h * v, eps64)) * dy
              ).sum(axis=1) / (2 * h)
        assert np.allclose(fd, (ds * v).sum(axis=1), rtol=1e-7, atol=1e-8)


def test_backward_radial_component():
    """<ds, s> = <s, dy> eps / D^3 with D^2 = mean(s^2) + eps."""
    rng = np.random.default_rng(24)
    for eps in (1e-6, 0.25, 0.0):
        eps64 = eps_as_passed(eps)
        s = bf16_value(_normal_bits(rng, (16, 128)))
        dy = bf16_value(_normal_bits(rng, s.shape))
        ds = rms_backward_values(s, dy, eps64)
        for i in range(16):
            d2 = math.fsum(s[i] ** 2) / 128 + eps64
            p = math.fsum(s[i] * dy[i])
            lhs = math.fsum(ds[i] * s[i])
            assert abs(lhs - p * eps64 / d2 ** 1.5) <= 1e-14 * math.fsum(np.abs(ds[i] * s[i])) \
                + 1e-14 * abs(p) / math.sqrt(d2)


def test_homogeneity_symmetry_fan_out_permutation():
    rng = np.random.default_rng(25)
    x = _normal_bits(rng, (8, 64))
    r = _normal_bits(rng, (8, 64))
    dy = _normal_bits(rng, (8, 64))
    y0 = bf16_value(rms_rows(x, None, 0.0))
    g0 = bf16_value(rms_rows_backward(x, None, dy, 0.0))
    for k in (-9, 3, 17):
        xs = _bits(bf16_value(x) * 2.0 ** k)
        assert np.array_equal(bf16_value(rms_rows(xs, None, 0.0)), y0)
        assert np.array_equal(bf16_value(rms_rows_backward(xs, None, dy, 0.0)), g0 * 2.0 ** -k)
    flip = np.uint16(0x8000)
    base = rms_rows(x, r)
    assert np.array_equal(bf16_value(rms_rows(x ^ flip, r ^ flip)), -bf16_value(base))
    assert np.array_equal(rms_rows(r, x), base)
    gb = rms_rows_backward(x, r, dy)
    assert np.array_equal(rms_rows_backward(r, x, dy), gb)
    assert np.array_equal(bf16_value(rms_rows_backward(x, r, dy ^ flip)), -bf16_value(gb))
    perm = rng.permutation(64)
    assert np.array_equal(rms_rows(x[:, perm], r[:, perm]), base[:, perm])
    assert np.array_equal(rms_rows(x[2:5], r[2:5]), base[2:5])


# ------------------------------------------------------- planted mistakes

def _fwd_mutant(kind):
    def fn(s, eps64):
        out = np.empty_like(s)
        n = s.shape[1]
        for i in range(s.shape[0]):
            ss = math.fsum(s[i] ** 2)
            t = {"no_mean": ss + eps64, "eps_on_sum": (ss + eps64) / n,
                 "n_minus_1": ss / (n - 1) + eps64, "no_eps": ss / n}.get(kind, ss / n + eps64)
            out[i] = s[i] / (t if kind == "no_sqrt" else math.sqrt(t))
        return out
    return fn


def _bwd_mutant(kind):
    def fn(s, dy, eps64):
        out = np.empty_like(s)
        n = s.shape[1]
        for i in range(s.shape[0]):
            d2 = math.fsum(s[i] ** 2) / n + (0.0 if kind == "drop_eps" else eps64)
            p = math.fsum(s[i] * dy[i])
            k = p / d2 if kind == "k_without_n" else p / (n * d2)
            d = math.sqrt(d2)
            out[i] = (dy[i] - s[i] * k) / (d ** 3 if kind == "div_D3" else d)
        return out
    return fn


def test_planted_mistakes_fail_closed_forms():
    def fwd_fails(fn):
        return any(not np.array_equal(*_fwd_case(c, fn)) for c in FWD)

    def bwd_fails(fn):
        return any(not np.array_equal(*_bwd_case(c, fn)) for c in BWD)

    assert not fwd_fails(_fwd_mutant("faithful")) and not bwd_fails(_bwd_mutant("faithful"))
    for kind in ("no_mean", "eps_on_sum", "n_minus_1", "no_eps", "no_sqrt"):
        assert fwd_fails(_fwd_mutant(kind)), kind
    for kind in ("drop_eps", "k_without_n", "div_D3"):
        assert bwd_fails(_bwd_mutant(kind)), kind
