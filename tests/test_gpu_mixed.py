"""Mixed-shape launches of the ragged weight calls on the GPU.

Small classes of rows that share a workgroup size run in one launch whose
kernel picks each task's row body by its shape key.  A matrix's bits must
not depend on that: every output of a mixed call equals, bit for bit, the
output of the same matrix called alone (its own shape's kernel), and
sampled rows meet the oracle's contracts.  The classes here are sized just
under the mixing bound and together exceed one pass of the grid (64
workgroups per compute unit, the library's cap, held here through
DS_ROWS_TEST_MAX_GROUPS whatever the environment says), so each workgroup
runs items of one-wave rows and of four-wave rows in turn (their LDS combines
must still alternate), with rescued rows among them; a class of two-wave rows
(128-thread workgroups) runs in a launch of its own.
"""
import os

import numpy as np
import pytest

from gpu_util import announce, depth_for, dev_bits, dev_f32, host_bits
from oracle.check import (admissible_rownorm, admissible_rownorm_backward, contract_bf16,
                          contract_grad, contract_rel, rescale_terms, rownorm_grad_terms)
from oracle.bf16 import bf16_value
from oracle.rows import rescale_after_step, weight_rownorm_gain, weight_rownorm_gain_backward
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu

ITEMS_PER_CU = 31          # just under the library's mixing bound of 32 per CU


@pytest.fixture(scope="module", autouse=True)
def grid_of_64_per_cu():
    """Every launch of this module on a grid of at most 64 workgroups per CU."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    old = os.environ.get("DS_ROWS_TEST_MAX_GROUPS")
    os.environ["DS_ROWS_TEST_MAX_GROUPS"] = str(64 * cus)
    yield
    if old is None:
        del os.environ["DS_ROWS_TEST_MAX_GROUPS"]
    else:
        os.environ["DS_ROWS_TEST_MAX_GROUPS"] = old


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


@pytest.fixture(scope="module")
def case():
    """Three small classes of 256-thread workgroups: one-wave rows of 64 and
    of 480 values (four rows an item) and four-wave rows of 4,608 (one row an
    item), each of ITEMS_PER_CU items per compute unit, and two-wave rows of
    2,048 (an odd count); a few rows of each scaled far out of fp32's
    comfortable range."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = ITEMS_PER_CU * cus
    shapes = [(4 * n, 64), (4 * n, 480), (n - 1, 2048), (n, 4608)]
    c = inputs.rownorm_grad_case(shapes, 2100)
    for i, w in enumerate(c.w):
        w[5] *= np.float32(2.0 ** 100)
        w[9] *= np.float32(2.0 ** -120)
        w[w.shape[0] - 1] = 0.0
    v = inputs.rescale_case(shapes, 2101).v
    return c, v


def _sample(rows, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.r_[0, 5, 9, rows - 1, rng.integers(0, rows, 24)])


def test_forward_mixed_equals_single(B, case):
    import torch
    c, _ = case
    announce("mixed forward", [w.shape for w in c.w])
    ws = [dev_f32(w) for w in c.w]
    gs = [dev_f32(g) for g in c.gain]
    n_all, e_all = B.ds_weight_rownorm_gain(ws, gs, [1.0] * len(ws))
    torch.cuda.synchronize()
    for i in range(len(c.w)):
        n1, e1 = B.ds_weight_rownorm_gain([ws[i]], [gs[i]], [1.0])
        torch.cuda.synchronize()
        assert torch.equal(n1[0], n_all[i]), f"matrix {i}: norms differ from the single call"
        assert torch.equal(e1[0].view(torch.int16), e_all[i].view(torch.int16)), i
        idx = _sample(c.w[i].shape[0], 2102 + i)
        w, g = c.w[i][idx], c.gain[i][idx]
        got_n, got_e = n_all[i].cpu().numpy()[idx], host_bits(e_all[i])[idx]
        n_ref, e_ref = weight_rownorm_gain([w], [g], [1.0])
        assert contract_rel(got_n, n_ref[0]).all(), i
        assert contract_bf16(got_e, e_ref[0], zero_sign=False).all(), i
        rn, rw = admissible_rownorm(got_n, got_e, w, g, 1.0, depth=depth_for(w.shape[1]))
        assert rn.ok and rw.ok, f"matrix {i}: {rn} / {rw}"


def test_backward_mixed_equals_single(B, case):
    import torch
    c, _ = case
    announce("mixed backward", [w.shape for w in c.w])
    ws = [dev_f32(w) for w in c.w]
    gs = [dev_f32(g) for g in c.gain]
    des = [dev_bits(d) for d in c.dwe]
    dw_all, dg_all = B.ds_weight_rownorm_gain_backward(ws, gs, des, [1.0] * len(ws))
    torch.cuda.synchronize()
    for i in range(len(c.w)):
        dw1, dg1 = B.ds_weight_rownorm_gain_backward([ws[i]], [gs[i]], [des[i]], [1.0])
        torch.cuda.synchronize()
        assert torch.equal(dw1[0], dw_all[i]) and torch.equal(dg1[0], dg_all[i]), i
        idx = _sample(c.w[i].shape[0], 2103 + i)
        w, g, de = c.w[i][idx], c.gain[i][idx], c.dwe[i][idx]
        got_dw, got_dg = dw_all[i].cpu().numpy()[idx], dg_all[i].cpu().numpy()[idx]
        want_dw, want_dg = weight_rownorm_gain_backward([w], [g], [1.0], [de])
        tw, tg = rownorm_grad_terms(w.astype(np.float64), g.astype(np.float64), 1.0,
                                    bf16_value(de))
        assert contract_grad(got_dw, want_dw[0], tw, "f32").all(), i
        assert contract_grad(got_dg, want_dg[0], tg, "f32").all(), i
        rw, rg = admissible_rownorm_backward(got_dw, got_dg, w, g, 1.0, de,
                                             depth=depth_for(w.shape[1]))
        assert rw.ok and rg.ok, f"matrix {i}: {rw} / {rg}"


def test_rescale_mixed_equals_single(B, case):
    import torch
    c, v = case
    announce("mixed rescale", [w.shape for w in c.w])
    for after_step in (False, True):
        ws, vs = [dev_f32(w) for w in c.w], [dev_f32(x) for x in v]
        call = B.ds_rescale_after_step if after_step else B.ds_rescale_project
        call(ws, vs)
        torch.cuda.synchronize()
        for i in range(len(c.w)):
            w1, v1 = dev_f32(c.w[i]), dev_f32(v[i])
            call([w1], [v1])
            torch.cuda.synchronize()
            assert torch.equal(w1, ws[i]) and torch.equal(v1, vs[i]), (after_step, i)
            idx = _sample(c.w[i].shape[0], 2104 + i)
            w, vv = c.w[i][idx], v[i][idx]
            got_w, got_v = ws[i].cpu().numpy()[idx], vs[i].cpu().numpy()[idx]
            terms = rescale_terms(w.astype(np.float64), vv.astype(np.float64))
            w_ref, v_ref = rescale_after_step([w], [vv], [1.0])
            assert contract_grad(got_v, v_ref[0], terms, "f32").all(), (after_step, i)
            if after_step:
                assert contract_rel(got_w, w_ref[0]).all(), i
            else:
                assert np.array_equal(got_w, w), i
