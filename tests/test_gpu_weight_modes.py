"""The weight ops' gain modes and widths on the GPU against the CPU oracle:
one gain for the whole matrix and no gain (mode "unit"), forward and
backward, in ragged calls that mix them with gains per row; rows whose width
is not a multiple of 4 (a convolution's 3 x 7 x 7) in the forward, gradient
and rescale calls; ResNet-50's convolutions and a vocabulary embedding at
radius sqrt(768).

Forward outputs meet the 1-ulp / 2e-6 contract and the strict interval; dW
meets the gradient contract and interval; a scalar gain's gradient (the sum
of the rows' shares) is within 2e-6 relative plus 2^-16 of the sum of the
shares' magnitudes of the float64 value.
"""
import numpy as np
import pytest

from gpu_util import announce, depth_for, dev_bits, dev_f32, host_bits
from oracle.bf16 import bf16_value
from oracle.check import (admissible_rownorm, admissible_rownorm_backward, contract_bf16,
                          contract_grad, contract_rel, rownorm_grad_terms)
from oracle.rows import gains_of, weight_rownorm_gain, weight_rownorm_gain_backward, \
    weight_rownorm_scalar_gain_backward
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


SHAPES = [(33, 768), (7, 3072), (100, 44), (5, 12288)]
MODES = ["row", "scalar", "none", "scalar", "none", "row", "scalar", "none"]


def _case(seed):
    shapes = [SHAPES[i % len(SHAPES)] for i in range(len(MODES))]
    case = inputs.rownorm_grad_case(shapes, seed, radius=1.0)
    gains = []
    for m, g in zip(MODES, case.gain):
        gains.append(g if m == "row" else (g[:1].copy() if m == "scalar" else None))
    return case, gains


def _dev_gain(g, mode):
    import torch
    if g is None:
        return None
    t = dev_f32(g)
    return t.reshape(()) if mode == "scalar" else t


def test_forward_modes(B):
    import torch
    case, gains = _case(1400)
    announce("rownorm gain modes forward", MODES)
    ws = [dev_f32(w) for w in case.w]
    gs = [_dev_gain(g, m) for g, m in zip(gains, MODES)]
    rho = [1.0, 27.712812921102035] * 4
    norms, weffs = B.ds_weight_rownorm_gain(ws, gs, rho)
    torch.cuda.synchronize()
    for i, (w, g) in enumerate(zip(case.w, gains)):
        n_ref, e_ref = weight_rownorm_gain([w], [g], [rho[i]])
        got_n = norms[i].cpu().numpy()
        got_e = host_bits(weffs[i])
        assert contract_rel(got_n, n_ref[0]).all(), i
        assert contract_bf16(got_e, e_ref[0], zero_sign=False).all(), i
        rn, rw = admissible_rownorm(got_n, got_e, w, gains_of(g, w.shape[0]).astype(np.float32),
                                    rho[i], depth=depth_for(w.shape[1]))
        assert rn.ok and rw.ok, f"{i} {MODES[i]}: {rn} / {rw}"


def test_backward_modes(B):
    import torch
    case, gains = _case(1401)
    announce("rownorm gain modes backward", MODES)
    ws = [dev_f32(w) for w in case.w]
    gs = [_dev_gain(g, m) for g, m in zip(gains, MODES)]
    des = [dev_bits(d) for d in case.dwe]
    dws, dgs = B.ds_weight_rownorm_gain_backward(ws, gs, des, case.radius)
    dws2, dgs2 = B.ds_weight_rownorm_gain_backward(ws, gs, des, case.radius)
    torch.cuda.synchronize()
    for i, (w, g, de) in enumerate(zip(case.w, gains, case.dwe)):
        mode = MODES[i]
        rho = case.radius[i]
        g_rows = gains_of(g, w.shape[0]).astype(np.float32)
        dw = dws[i].cpu().numpy()
        assert np.array_equal(dw, dws2[i].cpu().numpy())
        want_dw, want_dg = weight_rownorm_gain_backward([w], [g_rows], [rho], [de])
        tw, tg = rownorm_grad_terms(w.astype(np.float64), g_rows.astype(np.float64),
                                    float(np.float32(rho)), bf16_value(de))
        assert contract_grad(dw, want_dw[0], tw, "f32").all(), f"{i} {mode}: dW"
        rw, _ = admissible_rownorm_backward(dw, want_dg[0], w, g_rows, rho, de,
                                            depth=depth_for(w.shape[1]))
        assert rw.ok, f"{i} {mode}: {rw}"
        if mode == "none":
            assert dgs[i] is None
        elif mode == "row":
            assert contract_grad(dgs[i].cpu().numpy(), want_dg[0], tg, "f32").all(), i
        else:
            got = dgs[i].cpu().numpy()
            assert got.shape == () and np.array_equal(got, dgs2[i].cpu().numpy())
            _, total = weight_rownorm_scalar_gain_backward(w, g, rho, de)
            assert contract_grad(np.array([got]), np.array([total]), np.array([tg.sum()]),
                                 "f32").all(), f"{i}: scalar gain {got} vs {total}"


def test_scalar_gain_on_the_transformer_workload(B):
    """The 48 linears, each with one gain: dL/dg per matrix on the device."""
    import torch
    case = inputs.make("rownorm_gain_bwd_12x4_d768")
    announce("rownorm scalar gains, 48 linears")
    ws = [dev_f32(w) for w in case.w]
    gs = [dev_f32(g[:1]).reshape(()) for g in case.gain]
    des = [dev_bits(d) for d in case.dwe]
    _, dgs = B.ds_weight_rownorm_gain_backward(ws, gs, des, case.radius)
    torch.cuda.synchronize()
    for i, (w, g, de) in enumerate(zip(case.w, case.gain, case.dwe)):
        wd, dd = ws[i].double(), des[i].double()
        n = wd.pow(2).sum(dim=1).sqrt()
        exact = ((wd * dd).sum(dim=1) / n).sum().item()
        mag = ((wd * dd).abs().sum(dim=1) / n).sum().item()
        got = dgs[i].item()
        assert abs(got - exact) <= 2e-6 * abs(exact) + 2.0 ** -16 * mag, (i, got, exact)


def test_scalar_gain_backward_on_a_side_stream(B):
    """On a stream other than the current one, a scalar gain's temporary row
    shares belong to that stream: the results equal the default stream's bit
    for bit, also when the current stream allocates and writes memory while
    the side stream's kernels still run."""
    import torch
    case = inputs.make("rownorm_gain_bwd_12x4_d768")
    announce("rownorm scalar gains on a side stream")
    ws = [dev_f32(w) for w in case.w]
    gs = [dev_f32(g[:1]).reshape(()) for g in case.gain]
    des = [dev_bits(d) for d in case.dwe]
    dw0, dg0 = B.ds_weight_rownorm_gain_backward(ws, gs, des, case.radius)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for handle in (side, side.cuda_stream):
        side.wait_stream(torch.cuda.current_stream())
        dw1, dg1 = B.ds_weight_rownorm_gain_backward(ws, gs, des, case.radius, stream=handle)
        # current-stream work that would reuse a freed block at once
        junk = [torch.full((w.shape[0],), float("nan"), device="cuda:0") for w in case.w]
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        del junk
        for i in range(len(ws)):
            assert torch.equal(dw1[i], dw0[i]), i
            assert torch.equal(dg1[i], dg0[i]), (i, dg1[i].item(), dg0[i].item())


# ------------------------------------------------ widths not a multiple of 4

from test_gpu_backward import check_rn, run_rn                       # noqa: E402
from test_gpu_rescale import check as check_rescale, run as run_rescale  # noqa: E402
from test_gpu_rownorm import check_matrix, run as run_fwd           # noqa: E402

ODD = [1, 3, 27, 75, 147, 1001, 1025, 4097, 16383]


@pytest.mark.parametrize("cols", ODD)
def test_odd_widths(B, cols):
    rows = 37 if cols <= 4097 else 5
    announce("weights, single-element rows", rows, cols)
    fc = inputs.rownorm_case([(rows, cols)], 1500 + cols % 71)
    n, w = run_fwd(B, fc)
    check_matrix(n[0], w[0], fc.w[0], fc.gain[0], 1.0, np.arange(rows), f"fwd {rows}x{cols}")
    gc_ = inputs.rownorm_grad_case([(rows, cols)], 1600 + cols % 71)
    dw, dg = run_rn(B, gc_)
    check_rn(dw[0], dg[0], gc_.w[0], gc_.gain[0], 1.0, gc_.dwe[0], np.arange(rows),
             f"bwd {rows}x{cols}")
    rc = inputs.rescale_case([(rows, cols)], 1700 + cols % 71, radius=2.0)
    for after in (False, True):
        gw, gv = run_rescale(B, rc, after)
        check_rescale(gw[0], gv[0], rc.w[0], rc.v[0], 2.0, after, np.arange(rows),
                      f"rescale {'after' if after else 'project'} {rows}x{cols}")


def test_mixed_widths_ragged_equals_single(B):
    """Element-path and vector-path matrices in one call: each matrix's bits
    are those of a call holding it alone."""
    shapes = [(40, 147), (33, 768), (9, 27), (64, 4096), (5, 1001)]
    case = inputs.rownorm_case(shapes, 1501)
    announce("weights, mixed widths ragged")
    n_all, w_all = run_fwd(B, case)
    for i in range(len(shapes)):
        one = inputs.RownormCase("one", [case.w[i]], [case.gain[i]], [case.radius[i]])
        n1, w1 = run_fwd(B, one)
        assert np.array_equal(n1[0], n_all[i]) and np.array_equal(w1[0], w_all[i]), shapes[i]


def test_empty_matrix_scalar_gain(B):
    """A scalar gain's gradient over an empty matrix is 0 (the sum over no
    rows), written even though there are no shares; a neighbour with rows is
    unaffected."""
    import torch
    dev = "cuda:0"
    announce("empty matrix, scalar gain")
    case = inputs.rownorm_grad_case([(33, 768)], 1410)
    w0 = torch.empty(0, 768, device=dev)
    de0 = torch.empty(0, 768, dtype=torch.bfloat16, device=dev)
    g = torch.tensor(1.5, device=dev)
    w1, de1 = dev_f32(case.w[0]), dev_bits(case.dwe[0])
    g1 = dev_f32(case.gain[0][:1].copy()).reshape(())
    dg = [torch.full((), float("nan"), device=dev), torch.full((), float("nan"), device=dev)]
    _, dgs = B.ds_weight_rownorm_gain_backward([w0, w1], [g, g1], [de0, de1], dgain=dg)
    torch.cuda.synchronize()
    assert dgs[0].item() == 0.0
    want = float(weight_rownorm_scalar_gain_backward(case.w[0], case.gain[0][:1].copy(), 1.0,
                                                     case.dwe[0])[1])
    assert abs(dgs[1].item() - want) <= 1e-5 * (1.0 + abs(want))


def test_resnet50_workload(B):
    """ResNet-50's convolutions and classifier, forward and backward, sampled rows."""
    case = inputs.make("rownorm_gain_resnet50")
    announce("weights", case.name, len(case.w))
    n, w = run_fwd(B, case)
    for i, (wm, gm) in enumerate(zip(case.w, case.gain)):
        exact = np.sqrt((wm.astype(np.float64) ** 2).sum(axis=1))
        assert contract_rel(n[i], exact).all(), f"matrix {i}"
        rows = np.unique(np.r_[0, wm.shape[0] - 1, np.arange(0, wm.shape[0], 97)])
        check_matrix(n[i], w[i], wm, gm, 1.0, rows, f"conv {i} {wm.shape}")
    gcase = inputs.make("rownorm_gain_bwd_resnet50")
    dw, dg = run_rn(B, gcase)
    for i, (wm, gm, de) in enumerate(zip(gcase.w, gcase.gain, gcase.dwe)):
        rows = np.unique(np.r_[0, wm.shape[0] - 1, np.arange(0, wm.shape[0], 131)])
        check_rn(dw[i], dg[i], wm, gm, 1.0, de, rows, f"conv {i} {wm.shape}")


def test_embedding_workload(B):
    """A 50304 x 768 vocabulary embedding at radius sqrt(768)."""
    case = inputs.make("rownorm_gain_embedding_50304x768")
    announce("weights", case.name)
    n, w = run_fwd(B, case)
    wm, gm, rho = case.w[0], case.gain[0], case.radius[0]
    exact = np.sqrt((wm.astype(np.float64) ** 2).sum(axis=1))
    assert contract_rel(n[0], exact).all()
    rows = np.unique(np.r_[0, wm.shape[0] - 1, np.arange(0, wm.shape[0], 509)])
    check_matrix(n[0], w[0], wm, gm, rho, rows, case.name)
    # every row: |W_eff_i| = g_i rho within bf16 rounding
    le = np.sqrt((bf16_value(w[0]) ** 2).sum(axis=1))
    assert np.all(np.abs(le - np.abs(gm.astype(np.float64)) * rho) <=
                  2.0 ** -8 * np.abs(gm) * rho)
