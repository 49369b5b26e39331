"""The allocation-free weight gradient against the allocating one, through
the C ABI: bit-identical dL/dW, per-row dL/dg and scalar-gain totals, on two
calls in a row, the second smaller (the library's scratch keeps the first
call's shares; nothing may leak into the second)."""
import ctypes

import numpy as np
import pytest

from gpu_util import announce, dev_bits, dev_f32
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


def descs_for(B, case, modes, dev_w, dev_g, dev_de, outs, shares):
    """ds_rownorm_grad_desc per matrix; `shares[i]` is the scalar gain's
    per-row buffer for the allocating call, None for the allocation-free one."""
    arr = (B.RownormGradDesc * len(case.w))()
    for i, m in enumerate(modes):
        dw, dg, tot = outs[i]
        rows, cols = case.w[i].shape
        per_row = dg if m == B.DS_GAIN_ROW else shares[i]
        arr[i] = B.RownormGradDesc(
            dev_w[i].data_ptr(), None if m == B.DS_GAIN_NONE else dev_g[i].data_ptr(), 1.0,
            dev_de[i].data_ptr(), dw.data_ptr(),
            None if per_row is None else per_row.data_ptr(), rows, cols, m,
            None if tot is None else tot.data_ptr(), 0, 0)
    return arr


def outputs(case, modes, fill):
    import torch
    outs = []
    for i, m in enumerate(modes):
        rows, cols = case.w[i].shape
        dw = torch.full((rows, cols), fill, dtype=torch.float32, device="cuda:0")
        dg = torch.full((rows,), fill, dtype=torch.float32, device="cuda:0") \
            if m == 0 else None
        tot = torch.full((1,), fill, dtype=torch.float32, device="cuda:0") if m == 1 else None
        outs.append((dw, dg, tot))
    return outs


def one_case(B, shapes, modes, seed):
    """Both entry points on one ragged call; returns nothing, asserts bits."""
    import torch
    L = B.lib()
    case = inputs.rownorm_grad_case(shapes, seed)
    dev_w = [dev_f32(w) for w in case.w]
    dev_g = [dev_f32(g if m == B.DS_GAIN_ROW else g[:1]) for g, m in zip(case.gain, modes)]
    dev_de = [dev_bits(d) for d in case.dwe]
    shares = [torch.empty(w.shape[0], dtype=torch.float32, device="cuda:0") if m == 1 else None
              for w, m in zip(case.w, modes)]
    ref = outputs(case, modes, 0.0)
    new = outputs(case, modes, float("nan"))
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    n = len(case.w)
    announce("noalloc weight gradient", n, "matrices", sum(w.shape[0] for w in case.w), "rows")
    st = L.ds_weight_rownorm_gain_backward(descs_for(B, case, modes, dev_w, dev_g, dev_de, ref,
                                                     shares), n, sp)
    assert st == B.DS_OK, B.ds_status_string(st)
    st = L.ds_weight_rownorm_gain_backward_noalloc(
        descs_for(B, case, modes, dev_w, dev_g, dev_de, new, [None] * n), n, sp)
    assert st == B.DS_OK, B.ds_status_string(st)
    torch.cuda.synchronize()
    for i, m in enumerate(modes):
        for a, b, what in zip(ref[i], new[i], ("dW", "dg", "total")):
            if a is None:
                continue
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), (i, m, what)
        if m == 1:      # the total against a float64 sum of the allocating call's shares
            exact = shares[i].double().sum().item()
            assert abs(ref[i][2].item() - exact) <= 1e-5 * max(1.0, abs(exact)), i


def test_noalloc_matches_allocating_call_twice(B):
    # call 1: 60 scalar-gain matrices of one width (more than one launch's
    # inline table), gains per row and none at two other widths
    shapes = [(64, 768)] * 60 + [(33, 3072)] * 6 + [(17, 147)] * 5
    modes = [1] * 60 + [0] * 6 + [2] * 5
    one_case(B, shapes, modes, 4100)
    # call 2, smaller: fewer scalar-gain rows land where call 1's shares were
    shapes = [(40, 768), (9, 3072), (5, 768), (1, 147)]
    modes = [1, 1, 0, 1]
    one_case(B, shapes, modes, 4101)


def test_noalloc_refuses_beyond_scratch(B):
    import torch
    L = B.lib()
    n = B.DS_SCRATCH_FLOATS + 1
    w = torch.zeros(n, 4, device="cuda:0")
    de = torch.zeros(n, 4, dtype=torch.int16, device="cuda:0")
    g = torch.ones(1, device="cuda:0")
    dw = torch.empty_like(w)
    tot = torch.empty(1, device="cuda:0")
    arr = (B.RownormGradDesc * 1)()
    arr[0] = B.RownormGradDesc(w.data_ptr(), g.data_ptr(), 1.0, de.data_ptr(), dw.data_ptr(),
                               None, n, 4, B.DS_GAIN_SCALAR, tot.data_ptr(), 0, 0)
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert L.ds_weight_rownorm_gain_backward_noalloc(arr, 1, sp) == B.DS_ERR_SCRATCH


def test_noalloc_binding(B):
    """The binding's wrapper, with the transformer's 48 linears and scalar gains."""
    import torch
    case = inputs.make("rownorm_gain_bwd_12x4_d768")
    ws = [dev_f32(w) for w in case.w]
    gs = [dev_f32(g[:1]).reshape(()) for g in case.gain]
    des = [dev_bits(d) for d in case.dwe]
    announce("noalloc binding, 48 linears")
    dw0, dg0 = B.ds_weight_rownorm_gain_backward(ws, gs, des, case.radius)
    dw1, dg1 = B.ds_weight_rownorm_gain_backward_noalloc(ws, gs, des, case.radius)
    torch.cuda.synchronize()
    for i in range(len(ws)):
        assert torch.equal(dw0[i], dw1[i]) and torch.equal(dg0[i], dg1[i]), i
