"""The weight op's gain modes and layouts on the oracle (DragonScale README,
"Patching options" and "Supported layers"), against what fixes them
independently of the oracle's own formulas:

* hand-derived closed forms (tests/golden/weight_modes_closed_forms.json):
  unit mode, a scalar gain and its gradient, an odd conv width, GPT-2's
  Conv1D and a ConvTranspose as column blocks;
* torch's own weight normalisation (torch._weight_norm, g v / ||v|| with the
  norm over every dimension but one) in float64, which fixes which values
  form a row for Linear/Conv (dim 0), Conv1D and ConvTranspose (dim 1);
* torch autograd for a scalar gain's gradient;
* exact rational arithmetic at odd widths (oracle.brute);
* planted mistakes in the layout mapping (the transposed reading of a
  column block) fail the closed forms.
"""
import math
import zlib

import numpy as np
import pytest
import torch

import golden_cases as gc
from oracle import brute
from oracle.bf16 import bf16_rne, bf16_value
from oracle.rows import (column_block_rows, gains_of, to_column_block, weight_rownorm_gain,
                         weight_rownorm_scalar_gain_backward)

CASES = gc.load("weight_modes_closed_forms.json")
FWD = [c for c in CASES if "expect" in c]


def _f32(v):
    return np.asarray(v, dtype=np.float64).astype(np.float32)


def weff_stored(stored, gain, rho, layout, units=None, seg=None, rows_fn=column_block_rows):
    """W_eff (bf16 values) of a stored weight under a layout, through the oracle."""
    w = _f32(stored)
    g = None if gain is None else _f32(gain)
    if layout == "rows":
        return bf16_value(weight_rownorm_gain([w], [g], [rho])[1][0])
    rows = rows_fn(w, units, seg)
    eff = bf16_value(weight_rownorm_gain([rows], [g], [rho])[1][0])
    return to_column_block(eff, w.shape, seg)


@pytest.mark.parametrize("case", FWD, ids=[c["name"] for c in FWD])
def test_closed_form(case):
    got = weff_stored(case["stored"], case["gain"], case["rho"], case["layout"],
                      case.get("units"), case.get("seg"))
    assert np.array_equal(got, np.array(case["expect"], np.float64)), got


def test_scalar_gain_gradient_closed_form():
    c = next(c for c in CASES if c["name"] == "scalar_gain_gradient")
    dw, dg = weight_rownorm_scalar_gain_backward(_f32(c["stored"]), _f32(c["gain"]), c["rho"],
                                                 bf16_rne(np.array(c["dweff"], np.float64)))
    assert np.array_equal(dw, _f32(c["expect_dw"]))
    assert dg == np.float32(c["expect_dg"])
    dw0, dg0 = weight_rownorm_scalar_gain_backward(_f32(c["stored"]), None, 1.0,
                                                   bf16_rne(np.array(c["dweff"], np.float64)))
    assert dg0 is None and np.array_equal(dw0, _f32(c["expect_dw"]) / 2)


def test_transposed_block_reading_fails():
    """Reading a column block as stored[u*seg:(u+1)*seg, :] (the wrong axis)
    must break the Conv1D and ConvTranspose closed forms."""
    def wrong(stored, units, seg):
        a = np.asarray(stored)
        return np.stack([a.reshape(-1)[u * a.size // units:(u + 1) * a.size // units]
                         for u in range(units)])
    for name in ("conv1d_gpt2", "conv_transpose"):
        c = next(c for c in CASES if c["name"] == name)
        got = weff_stored(c["stored"], c["gain"], c["rho"], c["layout"], c["units"], c["seg"],
                          rows_fn=wrong)
        assert not np.array_equal(got, np.array(c["expect"], np.float64)), name


# --------------------------------------------------- torch's weight_norm

def _near_mid(v, rel=2.0 ** -40):
    with np.errstate(all="ignore"):
        return bf16_rne(v * (1 - rel)) != bf16_rne(v * (1 + rel))


@pytest.mark.parametrize("kind", ["linear", "conv2d", "conv1d_gpt2", "conv_transpose2d",
                                  "conv_transpose1d_groups"])
def test_layouts_match_torch_weight_norm(kind):
    rng = np.random.default_rng(zlib.crc32(kind.encode()))
    if kind == "linear":
        v, dim = rng.standard_normal((24, 40)) * 0.02, 0
    elif kind == "conv2d":
        v, dim = rng.standard_normal((16, 3, 7, 7)) * 0.02, 0          # 147 = odd width
    elif kind == "conv1d_gpt2":
        v, dim = rng.standard_normal((48, 72)) * 0.02, 1               # [in, out]
    elif kind == "conv_transpose2d":
        v, dim = rng.standard_normal((12, 10, 3, 3)) * 0.02, 1         # [in, out, kh, kw]
    else:
        v, dim = rng.standard_normal((8, 6, 5)) * 0.02, 1              # [in, out/groups, k], 2 groups
    v = v.astype(np.float32)
    groups = 2 if kind == "conv_transpose1d_groups" else 1
    units_pg = v.shape[dim]
    g = rng.uniform(0.5, 2, units_pg * groups).astype(np.float32)
    k = int(np.prod(v.shape[2:])) if v.ndim > 2 else 1
    if dim == 0:
        w2 = v.reshape(v.shape[0], -1)
        eff = bf16_value(weight_rownorm_gain([w2], [g], [1.0])[1][0]).reshape(v.shape)
        want = torch._weight_norm(torch.tensor(v, dtype=torch.float64),
                                  torch.tensor(g, dtype=torch.float64).reshape(-1, *[1] * (v.ndim - 1)),
                                  0).numpy()
    else:
        in_pg = v.shape[0] // groups
        eff = np.empty(v.shape)
        want = np.empty(v.shape)
        for grp in range(groups):
            vg = v[grp * in_pg:(grp + 1) * in_pg]
            stored = vg.reshape(in_pg, units_pg * k)                   # [A, ld]
            gg = g[grp * units_pg:(grp + 1) * units_pg]
            rows = column_block_rows(stored, units_pg, k)
            e = bf16_value(weight_rownorm_gain([rows], [gg], [1.0])[1][0])
            eff[grp * in_pg:(grp + 1) * in_pg] = to_column_block(e, stored.shape, k).reshape(vg.shape)
            shape = [1] * v.ndim
            shape[1] = units_pg
            want[grp * in_pg:(grp + 1) * in_pg] = torch._weight_norm(
                torch.tensor(vg, dtype=torch.float64),
                torch.tensor(gg, dtype=torch.float64).reshape(shape), 1).numpy()
    diff = bf16_rne(want) != bf16_rne(eff)
    assert not (diff & ~_near_mid(want)).any(), np.argwhere(diff)[:4]


# --------------------------------------------------------- scalar gain

@pytest.mark.parametrize("scale", [0.02, 2.0 ** 30])
def test_scalar_gain_gradient_matches_autograd(scale):
    rng = np.random.default_rng(int(math.log2(scale)) + 50)
    w = _f32(rng.standard_normal((30, 44)) * scale)
    w[4] = 0.0
    g = np.float32(1.7)
    rho = float(np.float32(math.sqrt(44)))
    de = bf16_rne(rng.standard_normal(w.shape))
    wt = torch.tensor(w.astype(np.float64), requires_grad=True)
    gt = torch.tensor(float(g), dtype=torch.float64, requires_grad=True)
    ss = (wt * wt).sum(dim=1, keepdim=True)
    n = torch.sqrt(torch.where(ss == 0, torch.ones_like(ss), ss))
    zero = torch.tensor((w == 0).all(axis=1)[:, None])
    weff = torch.where(zero, 0 * wt, gt * rho * wt / n)
    weff.backward(torch.tensor(bf16_value(de)))
    dw, dg = weight_rownorm_scalar_gain_backward(w, np.array([g]), rho, de)
    assert abs(float(dg) - gt.grad.item()) <= 2.0 ** -23 * abs(gt.grad.item()) + 1e-30
    nz = ~zero.numpy()[:, 0]
    assert np.allclose(dw[nz], wt.grad.numpy()[nz].astype(np.float32), rtol=2e-6, atol=1e-30)
    assert not dw[~nz].any()


def test_gains_of_modes():
    assert np.array_equal(gains_of(None, 3), np.ones(3))
    assert np.array_equal(gains_of(np.array([2.5], np.float32), 3), np.full(3, 2.5))
    assert np.array_equal(gains_of(np.array([1, 2, 3], np.float32), 3), [1, 2, 3])


# ------------------------------------------------------- exact, odd widths

def test_odd_widths_match_exact():
    rng = np.random.default_rng(818)
    flagged = 0
    for k in range(120):
        cols = int(rng.choice([1, 3, 5, 7, 27, 75, 147]))
        scale = float(np.exp2(rng.integers(-60, 60))) if k % 3 == 0 else 0.02
        w = _f32(rng.standard_normal(cols) * scale)
        g = np.float32(rng.uniform(-2.0, 2.0))
        rho = [1.0, float(np.sqrt(np.float32(cols)))][k % 2]
        norms, weffs = weight_rownorm_gain([w[None]], [np.array([g])], [rho])
        want_n, want_e, near = brute.rownorm_row(w, float(g), rho)
        if near:
            flagged += 1
            continue
        assert norms[0][0] == np.float32(float(want_n)), k
        assert np.array_equal(bf16_value(weffs[0][0]), np.array([float(v) for v in want_e])), k
    assert flagged <= 5
