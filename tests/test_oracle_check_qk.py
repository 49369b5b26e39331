"""The q/k check itself: a faithful fp32 run passes; the pages' two controls
(TensorFold PR #1260's q/k commit: drop the rotated head's rounding, or q's
normalized head's) fail the strict check."""
import numpy as np
import pytest

import kernel_models as km
from oracle.bf16 import bf16_rne, bf16_value
from oracle.check import admissible_qk_rows, contract_bf16
from oracle.rows import qk_rows_l2


@pytest.fixture(scope="module")
def qk_in():
    rng = np.random.default_rng(331)
    hd, rows = 256, 24
    q = bf16_rne(rng.standard_normal((rows, 4 * hd)))
    k = bf16_rne(rng.standard_normal((rows, 1 * hd)))
    pos = np.concatenate([np.arange(16), 199_800 + np.arange(8)])
    inv = (10000.0 ** (-np.arange(0, hd, 2) / hd)).astype(np.float32)
    sc = rng.uniform(0.5, 3.0, 4 * hd).astype(np.float32)
    return q, k, pos, inv, sc, hd


def test_faithful_passes(qk_in):
    q, k, pos, inv, sc, hd = qk_in
    qo, ko = km.qk_model(q, k, pos, inv, sc, hd)
    rq, rk, uq, uk = admissible_qk_rows(qo, ko, q, k, pos, inv, sc, hd)
    assert rq.ok and rk.ok, (str(rq), str(rk))
    assert uq.mean() > 0.97 and uk.mean() > 0.97
    wq, wk = qk_rows_l2(q, k, pos, inv, sc, hd)
    assert contract_bf16(qo, wq)[uq].all() and contract_bf16(ko, wk)[uk].all()


@pytest.mark.parametrize("drop", ["round_r", "round_n"])
def test_controls_fail(qk_in, drop):
    q, k, pos, inv, sc, hd = qk_in
    qo, ko = km.qk_model(q, k, pos, inv, sc, hd, **{drop: False})
    rq, rk, _, _ = admissible_qk_rows(qo, ko, q, k, pos, inv, sc, hd)
    assert rq.outside > 100, str(rq)


def test_integer_heads_at_position_zero_are_exact():
    """The pages' gate 4 for q/k: integer heads, no rotation, exact fp32 sums."""
    rng = np.random.default_rng(332)
    hd = 128
    q = bf16_rne(rng.integers(-64, 65, (4, 2 * hd)).astype(float))
    pos = np.zeros(4, np.int64)
    inv = np.ones(hd // 2, np.float32)
    sc = np.ones(2 * hd, np.float32)
    qo, _ = km.qk_model(q, None, pos, inv, sc, hd)
    rq, _, uq, _ = admissible_qk_rows(qo, None, q, None, pos, inv, sc, hd, depth=0)
    assert rq.ok, str(rq)


def test_integer_heads_fp16_sum_control_fails():
    """The pages' gate 4 for q/k: integer heads with no rotation (position 0)
    overflow an fp16 sum to a zero output, which fails the strict check."""
    rng = np.random.default_rng(333)
    hd = 256
    q = bf16_rne(rng.integers(-64, 65, (6, 4 * hd)).astype(float))
    k = bf16_rne(rng.integers(-64, 65, (6, hd)).astype(float))
    pos = np.zeros(6, np.int64)
    inv = (10000.0 ** (-np.arange(0, hd, 2) / hd)).astype(np.float32)
    sc = rng.uniform(0.5, 2.0, 4 * hd).astype(np.float32)
    qo, ko = km.qk_model(q, k, pos, inv, sc, hd)
    rq, rk, _, _ = admissible_qk_rows(qo, ko, q, k, pos, inv, sc, hd, depth=0)
    assert rq.ok and rk.ok, (str(rq), str(rk))
    qo16, ko16 = km.qk_model(q, k, pos, inv, sc, hd, acc="f16")
    assert not bf16_value(qo16).any() and not bf16_value(ko16).any()
    rq, rk, _, _ = admissible_qk_rows(qo16, ko16, q, k, pos, inv, sc, hd)
    assert rq.outside > 0.9 * qo16.size and rk.outside > 0.9 * ko16.size, (str(rq), str(rk))
