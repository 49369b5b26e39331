"""The q/k row oracle (qk_rows_l2) against what fixes it independently:
hand-derived closed forms (tests/golden/qk_closed_forms.json), exact
arithmetic with 50-digit cos and sin (mpmath), invariants, and planted
mistakes."""
import math

import numpy as np
import pytest

import golden_cases as gc
from oracle import brute
from oracle.bf16 import bf16_rne, bf16_value
from oracle.rows import (_l2_of_values, eps_as_passed, l2_rows, qk_rotated_heads, qk_rows_l2,
                         rope_angles)
from test_oracle_brute import _frac_row_to_bits

CASES = gc.load("qk_closed_forms.json")


def _run(case, fn=qk_rows_l2):
    hd = case["head_dim"]
    qw = 2 * hd if case["name"] == "two_heads_k_unscaled" else hd
    q = bf16_rne(gc.row(case["q"], qw))[None]
    inv = gc.row(case["inv_freq"], hd // 2).astype(np.float32)
    sc = gc.row(case["q_scale"], qw).astype(np.float32)
    k = bf16_rne(gc.row(case["k"], hd))[None] if "k" in case else None
    return fn(q, k, np.array([case["pos"]]), inv, sc, hd, 1e-6), qw


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_closed_form(case):
    (qo, ko), qw = _run(case)
    assert np.array_equal(bf16_value(qo)[0], gc.expected(case["expect_q"], qw))
    if "k" in case:
        assert np.array_equal(bf16_value(ko)[0], gc.expected(case["expect_k"], case["head_dim"]))


def test_angles_are_fp32_products():
    pos = np.array([0, 1, 199_801, 5000])
    inv = (10000.0 ** (-np.arange(0, 256, 2) / 256)).astype(np.float32)
    th = rope_angles(pos, inv)
    assert th.dtype == np.float64
    assert np.array_equal(th, (pos.astype(np.float32)[:, None] * inv).astype(np.float64))


def _inputs(seed, rows=6, nq=2, nk=1, hd=32):
    rng = np.random.default_rng(seed)
    q = bf16_rne(rng.standard_normal((rows, nq * hd)))
    k = bf16_rne(rng.standard_normal((rows, nk * hd)))
    pos = rng.integers(0, 250_000, rows)
    pos[0] = 0
    inv = (10000.0 ** (-np.arange(0, hd, 2) / hd)).astype(np.float32)
    sc = rng.uniform(0.5, 4, nq * hd).astype(np.float32)
    return q, k, pos, inv, sc, hd


def test_matches_exact():
    flagged = 0
    for seed in range(12):
        q, k, pos, inv, sc, hd = _inputs(900 + seed, rows=3, nq=2, nk=1, hd=16)
        qo, ko = qk_rows_l2(q, k, pos, inv, sc, hd)
        for r in range(q.shape[0]):
            for h in range(2):
                n, out, near = brute.qk_head(q[r, h * hd:(h + 1) * hd], pos[r], inv,
                                             sc[h * hd:(h + 1) * hd], float(np.float32(1e-6)))
                if near:
                    flagged += 1
                    continue
                got = qo[r, h * hd:(h + 1) * hd]
                want = _frac_row_to_bits(out)
                same = (got == want) | ((bf16_value(got) == 0) & (bf16_value(want) == 0))
                assert same.all(), (seed, r, h)
            n, _, near = brute.qk_head(k[r], pos[r], inv, np.ones(hd, np.float32),
                                       float(np.float32(1e-6)))
            if not near:
                want = _frac_row_to_bits(n)
                same = (ko[r] == want) | ((bf16_value(ko[r]) == 0) & (bf16_value(want) == 0))
                assert same.all(), (seed, r, "k")
    assert flagged <= 6


def test_position_zero_is_l2_per_head():
    q, k, pos, inv, sc, hd = _inputs(950)
    z = np.zeros_like(pos)
    qo, ko = qk_rows_l2(q, k, z, inv, np.ones_like(sc), hd)
    per_head = l2_rows(q.reshape(-1, hd)).reshape(q.shape)
    assert np.array_equal(qo, per_head)
    assert np.array_equal(ko, l2_rows(k.reshape(-1, hd)).reshape(k.shape))


def test_rotation_keeps_length():
    q, k, pos, inv, sc, hd = _inputs(951, rows=20)
    r = bf16_value(qk_rotated_heads(q, rope_angles(pos, inv), hd)).reshape(-1, hd)
    x = bf16_value(q).reshape(-1, hd)
    nr, nx = np.sqrt((r ** 2).sum(1)), np.sqrt((x ** 2).sum(1))
    assert np.all(np.abs(nr - nx) <= 2.0 ** -8 * nx)


def test_relative_position():
    """<R(p) q, R(p') k> depends on p - p' alone (angles exact: inv powers of two)."""
    hd = 16
    rng = np.random.default_rng(952)
    q = bf16_rne(rng.standard_normal((1, hd)))
    k = bf16_rne(rng.standard_normal((1, hd)))
    inv = np.exp2(-np.arange(hd // 2, dtype=np.float64)).astype(np.float32)

    def dot(p, pk):
        rq = bf16_value(qk_rotated_heads(q, rope_angles(np.array([p]), inv), hd))
        rk = bf16_value(qk_rotated_heads(k, rope_angles(np.array([pk]), inv), hd))
        return float((rq * rk).sum())
    ref = dot(3, 0)
    for p, pk in ((10, 7), (103, 100), (5003, 5000)):
        assert abs(dot(p, pk) - ref) <= 2.0 ** -6 * float(np.abs(bf16_value(q)).sum() * np.abs(bf16_value(k)).max() * 2)


def test_heads_and_rows_independent():
    q, k, pos, inv, sc, hd = _inputs(953, rows=8, nq=3)
    qo, ko = qk_rows_l2(q, k, pos, inv, sc, hd)
    q2 = q.copy()
    q2[:, hd:2 * hd] = bf16_rne(np.ones((8, hd)))
    qo2, _ = qk_rows_l2(q2, k, pos, inv, sc, hd)
    assert np.array_equal(qo2[:, :hd], qo[:, :hd]) and np.array_equal(qo2[:, 2 * hd:], qo[:, 2 * hd:])
    qo3, ko3 = qk_rows_l2(q[2:5], k[2:5], pos[2:5], inv, sc, hd)
    assert np.array_equal(qo3, qo[2:5]) and np.array_equal(ko3, ko[2:5])


# ------------------------------------------------------------ planted mistakes

def _variant(kind):
    def fn(q_bits, k_bits, positions, inv_freq, q_scale, hd, eps):
        th = rope_angles(positions, inv_freq)
        x = bf16_value(q_bits).reshape(q_bits.shape[0], -1, hd)
        c, s = np.cos(th)[:, None, :], np.sin(th)[:, None, :]
        if kind == "interleaved":
            x1, x2 = x[..., 0::2], x[..., 1::2]
            rot = np.empty_like(x)
            rot[..., 0::2], rot[..., 1::2] = x1 * c - x2 * s, x2 * c + x1 * s
        else:
            x1, x2 = x[..., :hd // 2], x[..., hd // 2:]
            sgn = -1.0 if kind == "sign" else 1.0
            rot = np.concatenate([x1 * c - sgn * x2 * s, x2 * c + sgn * x1 * s], axis=-1)
        r = bf16_value(bf16_rne(rot)).reshape(-1, hd)
        n = _l2_of_values(r, eps_as_passed(eps))
        if kind != "scale_before_round":
            n = bf16_value(bf16_rne(n))
        qo = bf16_rne((n.reshape(q_bits.shape).astype(np.float32) * q_scale).astype(np.float64))
        return qo, None
    return fn


def test_planted_mistakes_fail_closed_forms():
    def fails(fn):
        for c in CASES:
            if "k" in c:
                continue
            (qo, _), qw = _run(c, fn)
            if not np.array_equal(bf16_value(qo)[0], gc.expected(c["expect_q"], qw)):
                return True
        return False
    assert not fails(_variant("faithful"))
    for kind in ("sign", "interleaved", "scale_before_round"):
        assert fails(_variant(kind)), kind
