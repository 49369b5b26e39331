"""Pins of the oracle's bf16 rounding against two independent references.

* torch's float32 -> bfloat16 cast (a library routine, round to nearest even),
  for every value that float32 can hold;
* exact rational rounding (oracle.brute.round_fraction, integer arithmetic),
  for float64 values that float32 cannot hold.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle.bf16 import BF16_MAX, bf16_rne, bf16_ulp, bf16_value
from oracle.brute import bf16_of


def torch_bf16_bits(v32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def all_finite_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_value(b)
    return b[np.isfinite(v)], v[np.isfinite(v)]


def test_every_pattern_round_trips():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bf16_value(b)
    back = bf16_rne(v)
    fin = ~np.isnan(v)
    assert np.array_equal(back[fin], b[fin])
    assert np.isnan(bf16_value(back[~fin])).all()


def test_midpoints_round_to_even():
    b, v = all_finite_bf16()
    pos = v[(v >= 0)]
    pos = np.unique(pos)
    mids = (pos[:-1] + pos[1:]) / 2            # exact in float64 and float32
    for sign in (1.0, -1.0):
        m = sign * mids
        got = bf16_rne(m)
        assert np.array_equal(got, torch_bf16_bits(m.astype(np.float32)))
        # the chosen neighbour has an even significand (last bit 0)
        assert ((got & 1) == 0).all()


def test_midpoint_neighbours_go_to_nearer_value():
    _, v = all_finite_bf16()
    pos = np.unique(v[v >= 0])
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    for m in (up, dn, -up, -dn):
        assert np.array_equal(bf16_rne(m.astype(np.float64)), torch_bf16_bits(m))


def test_random_float32_matches_torch():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, 1_000_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    assert np.array_equal(bf16_rne(v.astype(np.float64)), torch_bf16_bits(v))


def test_overflow_threshold():
    top = BF16_MAX
    mid = (top + 2.0 ** 128) / 2                 # (2 - 2**-8) * 2**127
    assert bf16_value(bf16_rne(np.array([top])))[0] == top
    assert np.isinf(bf16_value(bf16_rne(np.array([mid]))))[0]
    below = np.nextafter(mid, 0.0)
    assert bf16_value(bf16_rne(np.array([below])))[0] == top
    assert bf16_value(bf16_rne(np.array([-mid])))[0] == -np.inf
    assert np.array_equal(bf16_rne(np.array([1e300, -1e300])), [0x7F80, 0xFF80])


def test_signed_zero_and_nan():
    assert bf16_rne(np.array([0.0]))[0] == 0x0000
    assert bf16_rne(np.array([-0.0]))[0] == 0x8000
    assert bf16_rne(np.array([-1e-300]))[0] == 0x8000   # underflows to -0
    assert np.isnan(bf16_value(bf16_rne(np.array([np.nan]))))[0]


def test_float64_values_match_exact_rounding():
    """float64 inputs (not float32-representable) against rational rounding."""
    rng = np.random.default_rng(11)
    exps = rng.integers(-140, 128, 4000)
    v = rng.uniform(1.0, 2.0, 4000) * np.exp2(exps.astype(np.float64))
    v *= rng.choice([-1.0, 1.0], 4000)
    # also values within a float64 ulp or two of bf16 midpoints
    _, fb = all_finite_bf16()
    pos = np.unique(fb[fb > 0])
    pick = rng.integers(0, pos.size - 1, 2000)
    mids = (pos[pick] + pos[pick + 1]) / 2
    v = np.concatenate([v, np.nextafter(mids, np.inf), np.nextafter(mids, 0.0)])
    got = bf16_rne(v)
    for x, g in zip(v, got):
        r, _ = bf16_of(Fraction(float(x)))
        want = float(r) if abs(r) < 2 ** 128 else np.copysign(np.inf, x)
        assert bf16_value(np.array([g]))[0] == want, x


def test_subnormal_spacing():
    assert bf16_ulp(np.array([0.0]))[0] == 2.0 ** -133
    assert bf16_ulp(np.array([2.0 ** -130]))[0] == 2.0 ** -133
    assert bf16_ulp(np.array([1.0]))[0] == 2.0 ** -7
    assert bf16_ulp(np.array([1.5]))[0] == 2.0 ** -7
    assert bf16_ulp(np.array([-0.75]))[0] == 2.0 ** -8
    # the smallest subnormal rounds from its half to even (0) and above it up
    assert bf16_rne(np.array([2.0 ** -134]))[0] == 0
    assert bf16_rne(np.array([2.0 ** -134 * 1.0000001]))[0] == 1
