"""The staging path's failure handling, with the failures forced from the host.

A ragged weight call with more than 48 matrices of one width stages its
matrix table through a ring of 8 library-owned slots.  DS_ROWS_TEST_FAIL
makes one step fail as if the runtime had refused it (no kernel is made to
fail).  A refused slot allocation or table upload must enqueue nothing and
return the slot at once (the owner's note on TensorFold PR #1260: refund
failed upload ownership); a refused launch returns its slot behind an event
once the upload has run.  More failures than the ring has slots, followed by
a call that succeeds, show that no slot was lost.
"""
import numpy as np
import pytest

from gpu_util import announce, dev_f32, host_bits
from oracle.check import contract_bf16
from oracle.rows import weight_rownorm_gain
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu

SHAPES = [(8, 64)] * 60          # one width class of 60 matrices: a staged table


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


@pytest.fixture(scope="module")
def case():
    return inputs.rownorm_case(SHAPES, 2100)


def call(B, case):
    """One staged call on outputs holding a sentinel; returns (error or None,
    norms, W_eff bits)."""
    import torch
    ws = [dev_f32(w) for w in case.w]
    gs = [dev_f32(g) for g in case.gain]
    norms = [torch.full((w.shape[0],), float("nan"), device="cuda:0") for w in case.w]
    weffs = [torch.full(w.shape, 0x7FC1, dtype=torch.int16, device="cuda:0") for w in case.w]
    err = None
    try:
        B.ds_weight_rownorm_gain(ws, gs, case.radius, norm_out=norms, w_eff=weffs)
    except RuntimeError as e:
        err = str(e)
    torch.cuda.synchronize()
    return err, [n.cpu().numpy() for n in norms], [host_bits(w) for w in weffs]


def untouched(norms, weffs):
    return all(np.isnan(n).all() for n in norms) and all((w == 0x7FC1).all() for w in weffs)


def correct(case, norms, weffs):
    n_ref, w_ref = weight_rownorm_gain(case.w, case.gain, case.radius)
    return all(contract_bf16(w, r, zero_sign=False).all() for w, r in zip(weffs, w_ref)) and \
        all(np.allclose(n, r, rtol=2e-6, atol=0) for n, r in zip(norms, n_ref))


@pytest.mark.parametrize("what,code", [("alloc", "DS_ERR_ALLOC"), ("copy", "DS_ERR_LAUNCH"),
                                       ("launch", "DS_ERR_LAUNCH")])
def test_refused_step_enqueues_nothing_and_loses_no_slot(B, case, monkeypatch, what, code):
    announce("staging failure", what)
    err, norms, weffs = call(B, case)
    assert err is None and correct(case, norms, weffs)          # the path works
    monkeypatch.setenv("DS_ROWS_TEST_FAIL", what)
    for _ in range(12):                                          # more than the ring's 8 slots
        err, norms, weffs = call(B, case)
        assert err is not None and code in err, err
        assert untouched(norms, weffs)                           # no kernel ran
    monkeypatch.delenv("DS_ROWS_TEST_FAIL")
    for _ in range(12):
        err, norms, weffs = call(B, case)
        assert err is None, err
        assert correct(case, norms, weffs)


def test_unknown_failure_name_is_ignored(B, case, monkeypatch):
    monkeypatch.setenv("DS_ROWS_TEST_FAIL", "nothing")
    err, norms, weffs = call(B, case)
    assert err is None and correct(case, norms, weffs)
