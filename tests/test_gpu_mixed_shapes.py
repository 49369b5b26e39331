"""Every shape of the mixed-shape weight kernels, in one ragged call.

The small classes of a ragged weight call that share a workgroup size run in
one mixed-shape launch, whose kernel switches on each task's shape key to
that shape's row body.  Here one matrix of every shape those kernels hold
(16-byte rows of one, two, four and eight waves; single-element rows, widths
that are not a multiple of 4) goes into one call of each weight op: the
forward, the gradient and the two rescale calls.  Every output must equal,
bit for bit, the same matrix's output called alone (its own shape's kernel),
and meet the oracle's contracts on every row.  Row counts that leave the
last item of a one-wave shape part-empty, a rescued row (scaled by 2^100), a
tiny one (2^-120) and a zero row are in every matrix.  A second call holds
three matrices of each shape: more than fit in the kernel arguments, so its
task table is staged in device memory.
"""
import os
import re
import sys

import numpy as np
import pytest

from gpu_util import announce, depth_for, dev_bits, dev_f32, host_bits
from oracle.bf16 import bf16_value
from oracle.check import (admissible_rownorm, contract_bf16, contract_grad, contract_rel,
                          rescale_terms, rownorm_grad_terms)
from oracle.rows import rescale_after_step, weight_rownorm_gain, weight_rownorm_gain_backward
from scale_invariant_row_amd import inputs

CSRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                    "scale_invariant_row_amd", "csrc")
sys.path.insert(0, CSRC)
import gen_instances as gen  # noqa: E402

pytestmark = pytest.mark.gpu


def mixed_keys(name):
    """Shape keys (NE * 10000 + G * 100 + V) the mixed kernels of a launcher switch on."""
    text = open(os.path.join(CSRC, name)).read()
    return sorted({int(k) for k in re.findall(r"case (\d+): \w+_item<", text)})


def width_of(key):
    """The narrowest row width whose weight shape is `key` (launch.hpp's
    pick_weight_shape: 16-byte vectors for a multiple of 4, else single
    elements)."""
    lim = gen.limits()
    ne, G, V = key // 10000, key // 100 % 100, key % 100
    for cols in range(1, gen.MAX_ELEM_COLS + 1):
        shape = gen.rownorm_shape(cols // 4, lim) if cols % 4 == 0 else gen.elem_shape(cols, lim)
        if (4 if cols % 4 == 0 else 1, ) + tuple(shape) == (ne, G, V):
            return cols
    raise AssertionError(f"no width has shape {key}")


def test_mixed_kernels_hold_the_same_shapes():
    keys = mixed_keys("inst_rownorm.hip")
    assert keys == mixed_keys("inst_rownorm_bwd.hip") == mixed_keys("inst_rescale.hip")
    assert len(keys) >= 20


def matrices(copies, seed):
    """`copies` matrices of each mixed shape: shapes (rows, width), in key order."""
    rng = np.random.default_rng(seed)
    shapes = []
    for key in mixed_keys("inst_rownorm.hip"):
        cols = width_of(key)
        for _ in range(copies):
            shapes.append((int(rng.integers(5, 12)), cols))
    return shapes


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


def case(copies, seed):
    shapes = matrices(copies, seed)
    c = inputs.rownorm_grad_case(shapes, seed)
    for w in c.w:
        w[1] *= np.float32(2.0 ** 100)       # a rescued row
        w[2] *= np.float32(2.0 ** -120)      # a tiny one
        w[3] = 0.0                           # a zero row
    v = inputs.rescale_case(shapes, seed + 1).v
    return c, v


CASES = [(1, 3100), (3, 3101)]


@pytest.mark.parametrize("copies,seed", CASES)
def test_forward(B, copies, seed):
    import torch
    c, _ = case(copies, seed)
    announce("mixed shapes forward", len(c.w), "matrices")
    ws, gs = [dev_f32(w) for w in c.w], [dev_f32(g) for g in c.gain]
    n_all, e_all = B.ds_weight_rownorm_gain(ws, gs, [1.0] * len(ws))
    torch.cuda.synchronize()
    for i, (w, g) in enumerate(zip(c.w, c.gain)):
        n1, e1 = B.ds_weight_rownorm_gain([ws[i]], [gs[i]], [1.0])
        torch.cuda.synchronize()
        assert torch.equal(n1[0], n_all[i]), f"matrix {i} {w.shape}: norms differ alone"
        assert torch.equal(e1[0].view(torch.int16), e_all[i].view(torch.int16)), (i, w.shape)
        got_n, got_e = n_all[i].cpu().numpy(), host_bits(e_all[i])
        n_ref, e_ref = weight_rownorm_gain([w], [g], [1.0])
        assert contract_rel(got_n, n_ref[0]).all(), (i, w.shape)
        assert contract_bf16(got_e, e_ref[0], zero_sign=False).all(), (i, w.shape)
        rn, rw = admissible_rownorm(got_n, got_e, w, g, 1.0, depth=depth_for(w.shape[1]))
        assert rn.ok and rw.ok, f"matrix {i} {w.shape}: {rn} / {rw}"


@pytest.mark.parametrize("copies,seed", CASES)
def test_backward(B, copies, seed):
    import torch
    c, _ = case(copies, seed)
    announce("mixed shapes backward", len(c.w), "matrices")
    ws, gs = [dev_f32(w) for w in c.w], [dev_f32(g) for g in c.gain]
    des = [dev_bits(d) for d in c.dwe]
    dw_all, dg_all = B.ds_weight_rownorm_gain_backward(ws, gs, des, [1.0] * len(ws))
    torch.cuda.synchronize()
    for i, (w, g, de) in enumerate(zip(c.w, c.gain, c.dwe)):
        dw1, dg1 = B.ds_weight_rownorm_gain_backward([ws[i]], [gs[i]], [des[i]], [1.0])
        torch.cuda.synchronize()
        assert torch.equal(dw1[0], dw_all[i]) and torch.equal(dg1[0], dg_all[i]), (i, w.shape)
        got_dw, got_dg = dw_all[i].cpu().numpy(), dg_all[i].cpu().numpy()
        want_dw, want_dg = weight_rownorm_gain_backward([w], [g], [1.0], [de])
        tw, tg = rownorm_grad_terms(w.astype(np.float64), g.astype(np.float64), 1.0,
                                    bf16_value(de))
        assert contract_grad(got_dw, want_dw[0], tw, "f32").all(), (i, w.shape)
        assert contract_grad(got_dg, want_dg[0], tg, "f32").all(), (i, w.shape)


@pytest.mark.parametrize("copies,seed", CASES)
@pytest.mark.parametrize("after_step", [False, True])
def test_rescale(B, copies, seed, after_step):
    import torch
    c, v = case(copies, seed)
    announce("mixed shapes rescale", "after step" if after_step else "project", len(c.w))
    call = B.ds_rescale_after_step if after_step else B.ds_rescale_project
    ws, vs = [dev_f32(w) for w in c.w], [dev_f32(x) for x in v]
    call(ws, vs)
    torch.cuda.synchronize()
    for i, (w, vv) in enumerate(zip(c.w, v)):
        w1, v1 = dev_f32(w), dev_f32(vv)
        call([w1], [v1])
        torch.cuda.synchronize()
        assert torch.equal(w1, ws[i]) and torch.equal(v1, vs[i]), (after_step, i, w.shape)
        got_w, got_v = ws[i].cpu().numpy(), vs[i].cpu().numpy()
        terms = rescale_terms(w.astype(np.float64), vv.astype(np.float64))
        w_ref, v_ref = rescale_after_step([w], [vv], [1.0])
        assert contract_grad(got_v, v_ref[0], terms, "f32").all(), (after_step, i, w.shape)
        if after_step:
            assert contract_rel(got_w, w_ref[0]).all(), (i, w.shape)
        else:
            assert np.array_equal(got_w, w), (i, w.shape)
