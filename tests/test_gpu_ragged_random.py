"""Randomised ragged weight calls on the GPU: a matrix's bits do not depend on
its neighbours.

Seeded random batches mix every kind of matrix the weight calls take: widths
whose rows take one, two, four or eight waves, single-element rows (widths
that are not a multiple of 4), column blocks (GPT-2 Conv1D and ConvTranspose
layouts), a gain per row, one per matrix or none, small classes (which share
a mixed-shape launch) and a large one (its own launch), and more than 48
matrices (a staged descriptor table).  Every output of a call equals, bit
for bit, the output of the same matrix called alone, and sampled rows of the
forward meet the oracle's contracts.
"""
import numpy as np
import pytest

from gpu_util import announce, dev_bits, dev_f32, host_bits
from oracle.check import contract_bf16, contract_rel
from oracle.rows import column_block_rows, gains_of, weight_rownorm_gain
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu

WIDTHS = [4, 44, 64, 147, 256, 480, 576, 768, 1152, 2048, 2304, 3072, 4608, 5000, 9216]


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


def batch(seed, n, big=False):
    """n random matrices: (stored fp32 w, gain or None, seg or None, bf16
    dL/dW_eff bits, fp32 v), drawn from one seeded generator."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        if rng.random() < 0.15:                    # a column block
            seg = int(rng.choice([1, 2, 4, 9]))
            units = int(rng.integers(1, 150))
            stored = (int(rng.integers(1, 300)), units * seg)
            rows = units
        else:
            seg = None
            cols = int(rng.choice(WIDTHS))
            rows = int(rng.integers(1, max(2, min(400, 600_000 // cols))))
            stored = (rows, cols)
        if big and i == 0:                         # a class large enough for its own launch
            seg, rows, stored = None, 40_000, (40_000, 768)
        w = (0.02 * rng.standard_normal(stored)).astype(np.float32)
        if rng.random() < 0.1:
            w[0] *= np.float32(2.0 ** 100)         # a rescued unit
        mode = rng.choice(["row", "scalar", "none"])
        g = (rng.uniform(0.5, 2.0, rows).astype(np.float32) if mode == "row" else
             np.array([rng.uniform(0.5, 2.0)], np.float32) if mode == "scalar" else None)
        de = inputs.to_bf16_bits(rng.standard_normal(stored))
        v = (1e-3 * rng.standard_normal(stored)).astype(np.float32)
        out.append((w, g, seg, de, v))
    return out


def _dev_gain(g, rows):
    """A gain per row as [rows], one per matrix as a 0-dim tensor, or None."""
    if g is None:
        return None
    t = dev_f32(g)
    return t.reshape(()) if g.size == 1 and rows != 1 else t


CASES = [(2200, 30, False), (2201, 70, False), (2202, 40, True)]


@pytest.mark.parametrize("seed,n,big", CASES)
def test_forward_and_gradient(B, seed, n, big):
    import torch
    mats = batch(seed, n, big)
    announce("ragged random", seed, n, big)
    ws = [dev_f32(m[0]) for m in mats]
    gs = [_dev_gain(m[1], m[0].shape[1] // m[2] if m[2] else m[0].shape[0]) for m in mats]
    segs = [m[2] for m in mats]
    des = [dev_bits(m[3]) for m in mats]
    n_all, e_all = B.ds_weight_rownorm_gain(ws, gs, segs=segs)
    dw_all, dg_all = B.ds_weight_rownorm_gain_backward(ws, gs, des, segs=segs)
    torch.cuda.synchronize()
    for i, (w, g, seg, de, _) in enumerate(mats):
        n1, e1 = B.ds_weight_rownorm_gain([ws[i]], [gs[i]], segs=[seg])
        dw1, dg1 = B.ds_weight_rownorm_gain_backward([ws[i]], [gs[i]], [des[i]], segs=[seg])
        torch.cuda.synchronize()
        label = f"seed {seed} matrix {i}: {w.shape}, seg {seg}, gain {None if g is None else g.size}"
        assert torch.equal(n1[0], n_all[i]), label
        assert torch.equal(e1[0].view(torch.int16), e_all[i].view(torch.int16)), label
        assert torch.equal(dw1[0], dw_all[i]), label
        if dg1[0] is not None:
            assert torch.equal(dg1[0], dg_all[i]), label
        # the forward against the oracle on a few unit rows
        units = w.shape[1] // seg if seg else w.shape[0]
        rows = column_block_rows(w, units, seg) if seg else w
        got_e = host_bits(e_all[i])
        erows = column_block_rows(got_e, units, seg) if seg else got_e
        idx = np.unique(np.r_[0, units - 1, np.random.default_rng(seed + i).integers(0, units, 4)])
        gv = gains_of(g, units)
        gsel = None if g is None else gv[idx].astype(np.float32)
        n_ref, e_ref = weight_rownorm_gain([rows[idx]], [gsel], [1.0])
        assert contract_rel(n_all[i].cpu().numpy()[idx], n_ref[0]).all(), label
        assert contract_bf16(erows[idx], e_ref[0], zero_sign=False).all(), label


@pytest.mark.parametrize("seed,n,big", CASES[:2])
def test_rescale(B, seed, n, big):
    import torch
    mats = batch(seed + 50, n, big)
    announce("ragged random rescale", seed, n)
    segs = [m[2] for m in mats]
    for after_step in (False, True):
        call = B.ds_rescale_after_step if after_step else B.ds_rescale_project
        ws, vs = [dev_f32(m[0]) for m in mats], [dev_f32(m[4]) for m in mats]
        call(ws, vs, segs=segs)
        torch.cuda.synchronize()
        for i, m in enumerate(mats):
            w1, v1 = dev_f32(m[0]), dev_f32(m[4])
            call([w1], [v1], segs=[m[2]])
            torch.cuda.synchronize()
            assert torch.equal(w1, ws[i]) and torch.equal(v1, vs[i]), (after_step, seed, i)
