"""The float64 oracle against exact rational arithmetic on tiny rows.

oracle.brute computes the same definitions with exact sums, 60-digit square
roots and integer rounding.  The two must agree on every element, except
where the exact value lies within 1e-12 (relative) of a rounding midpoint,
which the brute force flags: there float64's own rounding may decide.
"""
import numpy as np
import pytest

from oracle import brute
from oracle.bf16 import bf16_rne, bf16_value
from oracle.rows import l2_rows, slerp_rows, weight_rownorm_gain


def _frac_row_to_bits(vals):
    out = []
    for v in vals:
        if abs(v) >= 2 ** 128:
            out.append(0x7F80 if v > 0 else 0xFF80)
        else:
            out.append(int(bf16_rne(np.array([float(v)]))[0]))
    return np.array(out, np.uint16)


def _rows(rng, n, cols_choices):
    """Random tiny bf16 rows with varied magnitudes and structure."""
    for k in range(n):
        cols = int(rng.choice(cols_choices))
        kind = k % 6
        if kind == 0:
            v = rng.standard_normal(cols)
        elif kind == 1:                                   # small integers
            v = rng.integers(-64, 65, cols).astype(float)
        elif kind == 2:                                   # wide dynamic range
            v = rng.standard_normal(cols) * np.exp2(rng.integers(-60, 60, cols))
        elif kind == 3:                                   # tiny rows: eps dominates
            v = rng.standard_normal(cols) * 2.0 ** -12
        elif kind == 4:                                   # sparse
            v = rng.standard_normal(cols) * (rng.random(cols) < 0.2)
        else:                                             # subnormal and huge
            v = rng.standard_normal(cols) * np.exp2(rng.choice([-130, -20, 0, 40, 100], cols))
        yield bf16_rne(v)


EPS_CHOICES = [1e-6, 0.0, 1.0, 3e-4]


def test_l2_rows_matches_exact():
    rng = np.random.default_rng(101)
    disagree = 0
    for k, x in enumerate(_rows(rng, 600, [8, 16, 24, 40, 64])):
        eps = EPS_CHOICES[k % len(EPS_CHOICES)]
        use_r = k % 2 == 1
        r = bf16_rne(rng.standard_normal(x.size)) if use_r else None
        if eps == 0.0 and not bf16_value(x).any() and (r is None or not bf16_value(r).any()):
            continue
        got = l2_rows(x[None], None if r is None else r[None], eps)[0]
        want, near = brute.l2_row(x, r, float(np.float32(eps)))
        want_bits = _frac_row_to_bits(want)
        diff = got != want_bits
        # +0/-0 agree in value; signs are checked separately below
        diff &= ~((bf16_value(got) == 0) & (bf16_value(want_bits) == 0))
        assert not (diff & ~np.array(near)).any(), (k, np.nonzero(diff)[0])
        disagree += int(diff.sum())
    assert disagree <= 3


def test_slerp_rows_matches_exact():
    rng = np.random.default_rng(202)
    flagged = 0
    n = 0
    for k, res in enumerate(_rows(rng, 240, [8, 16, 32])):
        n += 1
        out = bf16_rne(2.0 * rng.standard_normal(res.size))
        alpha = rng.uniform(-0.2, 0.2, res.size).astype(np.float32)
        if k % 5 == 0:
            alpha = rng.uniform(-1.5, 1.5, res.size).astype(np.float32)
        eps = EPS_CHOICES[k % 3]
        if eps == 0.0 and not bf16_value(res).any():
            continue
        got = slerp_rows(res[None], out[None], alpha, eps)[0]
        want, near = brute.slerp_row(res, out, alpha, float(np.float32(eps)))
        want_bits = _frac_row_to_bits(want)
        same = (got == want_bits) | ((bf16_value(got) == 0) & (bf16_value(want_bits) == 0))
        if near:
            flagged += 1
            continue
        assert same.all(), (k, np.nonzero(~same)[0])
    assert flagged <= n // 20


def test_rownorm_matches_exact():
    rng = np.random.default_rng(303)
    for k in range(300):
        cols = int(rng.choice([8, 12, 32, 48]))
        scale = float(np.exp2(rng.integers(-70, 70))) if k % 3 == 0 else 0.02
        w = (rng.standard_normal(cols) * scale).astype(np.float32)
        g = np.float32(rng.uniform(0.5, 2.0))
        rho = [1.0, 1.0, float(np.sqrt(np.float32(cols)))][k % 3]
        norms, weffs = weight_rownorm_gain([w[None]], [np.array([g])], [rho])
        n32, want, near = brute.rownorm_row(w, float(g), rho)
        if near:
            continue
        assert norms[0][0] == np.float32(float(n32)), k
        want_bits = _frac_row_to_bits(want)
        same = (weffs[0][0] == want_bits) | ((bf16_value(weffs[0][0]) == 0) & (bf16_value(want_bits) == 0))
        assert same.all(), (k, np.nonzero(~same)[0])


def test_brute_finds_known_ties():
    """The rounding helper flags exact midpoints and rounds them to even."""
    from fractions import Fraction
    r, near = brute.bf16_of(Fraction(257, 256))        # 1 + 2**-8: midpoint of 1 and 1+2**-7
    assert r == 1 and near
    r, near = brute.bf16_of(Fraction(259, 256))        # 1 + 3 * 2**-8: rounds up to even
    assert r == Fraction(260, 256) and near
    r, near = brute.fp32_of(Fraction(1) + Fraction(1, 2 ** 24))
    assert r == 1 and near
