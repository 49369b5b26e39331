"""Column-block weights on the GPU against the CPU oracle: GPT-2's Conv1D
([in, out], each output unit a column, seg 1) and ConvTranspose groups
([in, out * k], seg = k), through the forward, gradient and rescale calls.

The oracle gathers each unit's values into a row (oracle.rows.column_block_rows),
runs the row definitions and scatters the result back; the GPU output must
meet the same contracts and strict intervals as contiguous rows, with the
column-block kernel's own sum-tree depth.
"""
import math

import numpy as np
import pytest

from gpu_util import announce, dev_bits, dev_f32, host_bits
from oracle.bf16 import bf16_value
from oracle.check import (admissible_rescale, admissible_rownorm, admissible_rownorm_backward,
                          contract_bf16, contract_grad, contract_rel, rescale_terms,
                          rownorm_grad_terms)
from oracle.rows import (column_block_rows, rescale_after_step, rescale_project,
                         to_column_block, weight_rownorm_gain, weight_rownorm_gain_backward)
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


# The seg-1 kernel's single-pass tiles, per op (the library's rule): vectors
# per lane K and lanes per stored row.
SINGLE_PASS = {"fwd": (12, 16), "bwd": (12, 16), "rescale": (6, 8)}


def single_pass_lanes(A, units, seg, op, ld=None, aligned=True):
    """Lanes per stored row of the single-pass column-block tile for this
    layout, or 0 when a two-pass tile runs: seg 1, units and ld multiples of
    4, 16-byte-aligned buffers, A within the tile's 1024 K / lanes stored rows
    and 32-bit offsets over them."""
    ld = units * seg if ld is None else ld
    if seg != 1 or units % 4 or ld % 4 or not aligned:
        return 0
    k, lanes = SINGLE_PASS[op]
    cap = 1024 * k // lanes
    if A > cap or cap * ld * 4 + 256 > 2 ** 31 - 1:
        return 0
    return lanes


def tree_adds(n):
    """Additions along the deepest path of the single-pass kernel's per-lane
    tree over n values (pairs: a product and an fma; then pairwise)."""
    if n <= 1:
        return 0
    if n == 2:
        return 1
    return 1 + max(tree_adds(n // 2), tree_adds(n - n // 2))


def depth_col(stored_rows, seg, op=None, units=None, ld=None):
    """Additions along any path of the column-block sum tree.  Two-pass
    kernel: a chain of ceil(A / 128) terms, the eight chains and sixteen waves
    pairwise, a unit's seg columns pairwise (plus one for the chain's first
    addition).  Single-pass kernel (when `op` and `units` say it runs): the
    lane's K values pairwise, the 64 / lanes row slots and the sixteen waves
    pairwise."""
    two_pass = -(-stored_rows // 128) + 1 + 3 + 4 + (math.ceil(math.log2(seg)) if seg > 1 else 0)
    lanes = single_pass_lanes(stored_rows, units, seg, op, ld) if op and units else 0
    if not lanes:
        return two_pass
    return tree_adds(SINGLE_PASS[op][0]) + int(math.log2(64 // lanes)) + 4


def rows_of(stored, seg):
    return column_block_rows(stored, stored.shape[1] // seg, seg)


def check_forward(norm, weff_bits, w, g, rho, seg, label, sample=None):
    units = w.shape[1] // seg
    rows = rows_of(w, seg)
    got_e = rows_of(weff_bits, seg)
    idx = np.arange(units) if sample is None else sample
    n_ref, e_ref = weight_rownorm_gain([rows[idx]], [g[idx]], [rho])
    assert contract_rel(norm[idx], n_ref[0]).all(), f"{label}: norms"
    ok = contract_bf16(got_e[idx], e_ref[0], zero_sign=False)
    assert ok.all(), f"{label}: W_eff beyond 1 ulp at {np.argwhere(~ok)[:4]}"
    rn, rw = admissible_rownorm(norm[idx], got_e[idx], rows[idx], g[idx], rho,
                                depth=depth_col(w.shape[0], seg, "fwd", units))
    assert rn.ok and rw.ok, f"{label}: {rn} / {rw}"


def check_backward(dw, dg, w, g, rho, de, seg, label, sample=None):
    units = w.shape[1] // seg
    rows, drows, derows = rows_of(w, seg), rows_of(dw, seg), rows_of(de, seg)
    idx = np.arange(units) if sample is None else sample
    want_dw, want_dg = weight_rownorm_gain_backward([rows[idx]], [g[idx]], [rho], [derows[idx]])
    tw, tg = rownorm_grad_terms(rows[idx].astype(np.float64), g[idx].astype(np.float64),
                                float(np.float32(rho)), bf16_value(derows[idx]))
    assert contract_grad(drows[idx], want_dw[0], tw, "f32").all(), f"{label}: dW"
    assert contract_grad(dg[idx], want_dg[0], tg, "f32").all(), f"{label}: dg"
    rw, rg = admissible_rownorm_backward(drows[idx], dg[idx], rows[idx], g[idx], rho, derows[idx],
                                         depth=depth_col(w.shape[0], seg, "bwd", units))
    assert rw.ok and rg.ok, f"{label}: {rw} / {rg}"


def run_forward(B, ws, gs, segs, rho=None):
    import torch
    norms, weffs = B.ds_weight_rownorm_gain([dev_f32(w) for w in ws], [dev_f32(g) for g in gs],
                                            rho or [1.0] * len(ws), segs=segs)
    torch.cuda.synchronize()
    return [n.cpu().numpy() for n in norms], [host_bits(e) for e in weffs]


def run_backward(B, ws, gs, des, segs, rho=None):
    import torch
    dws, dgs = B.ds_weight_rownorm_gain_backward(
        [dev_f32(w) for w in ws], [dev_f32(g) for g in gs], [dev_bits(d) for d in des],
        rho or [1.0] * len(ws), segs=segs)
    torch.cuda.synchronize()
    return [d.cpu().numpy() for d in dws], [d.cpu().numpy() for d in dgs]


# (stored rows A, units, seg): GPT-2 Conv1D shapes and ConvTranspose groups
SHAPES = [(768, 96, 1), (40, 130, 1), (1, 77, 1), (12, 10, 9), (7, 33, 16), (5, 9, 27),
          (3, 4, 64), (33, 70, 5), (2, 3, 3)]


@pytest.mark.parametrize("A,units,seg", SHAPES)
def test_shapes(B, A, units, seg):
    announce("colblock", A, units, seg)
    c = inputs.colblock_grad_case([(A, units * seg)], seg, 1800 + A + seg)
    w, g, de = c.w[0], c.gain[0], c.dwe[0]
    n, e = run_forward(B, [w], [g], [seg], [2.0])
    check_forward(n[0], e[0], w, g, 2.0, seg, f"fwd {A}x{units}x{seg}")
    dw, dg = run_backward(B, [w], [g], [de], [seg], [2.0])
    check_backward(dw[0], dg[0], w, g, 2.0, de, seg, f"bwd {A}x{units}x{seg}")
    # rescale: the gradient, then the momentum and the rows after a step
    import torch
    v = (1e-3 * np.random.default_rng(A + seg).standard_normal(w.shape)).astype(np.float32)
    wd, vd = dev_f32(w), dev_f32(v)
    B.ds_rescale_project([wd], [vd], segs=[seg])
    torch.cuda.synchronize()
    rows, vrows = rows_of(w, seg), rows_of(v, seg)
    want_v = rescale_project([rows], [vrows])[0]
    got_v = rows_of(vd.cpu().numpy(), seg)
    terms = rescale_terms(rows.astype(np.float64), vrows.astype(np.float64))
    assert contract_grad(got_v, want_v, terms, "f32").all(), "project"
    assert np.array_equal(wd.cpu().numpy(), w)
    depth = depth_col(A, seg, "rescale", units)
    _, rv = admissible_rescale(rows, got_v, rows, vrows, 1.0, False, depth=depth)
    assert rv.ok, f"project: {rv}"
    wd, vd = dev_f32(w), dev_f32(v)
    B.ds_rescale_after_step([wd], [vd], [3.0], segs=[seg])
    torch.cuda.synchronize()
    ws_ref, vs_ref = rescale_after_step([rows], [vrows], [3.0])
    got_w, got_v = rows_of(wd.cpu().numpy(), seg), rows_of(vd.cpu().numpy(), seg)
    assert contract_rel(got_w, ws_ref[0]).all(), "after step: w"
    assert contract_grad(got_v, vs_ref[0], terms, "f32").all(), "after step: v"
    rw, rv = admissible_rescale(got_w, got_v, rows, vrows, 3.0, True, depth=depth)
    assert rw.ok and rv.ok, f"after step: {rw} / {rv}"


@pytest.mark.parametrize("A,units,seg", [(768, 96, 1), (33, 70, 5), (3, 4, 64)])
def test_after_step_without_momentum(B, A, units, seg):
    """After a step with no momentum only the weight is rescaled; a zero unit
    is left as it is."""
    import torch
    announce("colblock after_step, no momentum", A, units, seg)
    rng = np.random.default_rng(1806 + A + seg)
    w = rng.standard_normal((A, units * seg)).astype(np.float32)
    w[:, seg:2 * seg] = 0.0                            # unit 1 is zero
    wd = dev_f32(w)
    B.ds_rescale_after_step([wd], None, [1.5], segs=[seg])
    torch.cuda.synchronize()
    rows = rows_of(w, seg)
    got = rows_of(wd.cpu().numpy(), seg)
    want, _ = rescale_after_step([rows], [None], [1.5])
    assert contract_rel(got, want[0]).all(), "after step: w"
    assert np.array_equal(got[1], rows[1]), "zero unit"
    rw, _ = admissible_rescale(got, None, rows, None, 1.5, True,
                               depth=depth_col(A, seg, "rescale", units))
    assert rw.ok, f"after step: {rw}"


def test_outputs_keep_the_layout(B):
    """Values outside the units' columns (ld > units * seg) are not touched, and
    W_eff lands where each unit's values sit."""
    import torch
    A, units, seg, ld = 6, 5, 3, 20
    rng = np.random.default_rng(1801)
    stored = (0.02 * rng.standard_normal((A, ld))).astype(np.float32)
    g = rng.uniform(0.5, 2, units).astype(np.float32)
    wd = dev_f32(stored)
    weff = torch.full((A, ld), 7.0, dtype=torch.bfloat16, device="cuda:0")
    norms = torch.empty(units, dtype=torch.float32, device="cuda:0")
    # a column block over the first units * seg columns of each stored row
    gd = dev_f32(g)
    d = (B.RownormDesc * 1)()
    d[0] = B.RownormDesc(wd.data_ptr(), gd.data_ptr(), 1.0, norms.data_ptr(),
                         weff.data_ptr(), units, A * seg, 0, seg, ld)
    assert B.lib().ds_weight_rownorm_gain(d, 1, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    got = host_bits(weff)
    assert (bf16_value(got[:, units * seg:]) == 7.0).all()
    rows = column_block_rows(stored, units, seg)
    _, e_ref = weight_rownorm_gain([rows], [g], [1.0])
    want = to_column_block(e_ref[0], (A, units * seg), seg)
    assert contract_bf16(got[:, :units * seg], want, zero_sign=False).all()


def test_ragged_mix_equals_single(B):
    """Column-block and contiguous matrices in one call: bits as when alone."""
    c1 = inputs.colblock_grad_case([(64, 200), (9, 90)], 1, 1802)
    c2 = inputs.colblock_grad_case([(8, 60)], 4, 1803)
    c3 = inputs.rownorm_grad_case([(50, 768), (7, 147)], 1804)
    ws = c1.w + c2.w + c3.w
    gs = c1.gain + c2.gain + c3.gain
    des = c1.dwe + c2.dwe + c3.dwe
    segs = [1, 1, 4, None, None]
    announce("colblock ragged mix")
    n_all, e_all = run_forward(B, ws, gs, segs)
    dw_all, dg_all = run_backward(B, ws, gs, des, segs)
    for i in range(len(ws)):
        n1, e1 = run_forward(B, [ws[i]], [gs[i]], [segs[i]])
        dw1, dg1 = run_backward(B, [ws[i]], [gs[i]], [des[i]], [segs[i]])
        assert np.array_equal(n1[0], n_all[i]) and np.array_equal(e1[0], e_all[i]), i
        assert np.array_equal(dw1[0], dw_all[i]) and np.array_equal(dg1[0], dg_all[i]), i


def test_edge_units(B):
    """Zero units, units far outside fp32's comfortable range (rescued), a unit
    holding an infinity."""
    A, units, seg = 40, 64, 2
    rng = np.random.default_rng(1805)
    w = rng.standard_normal((A, units * seg))
    scale = np.ones(units)
    scale[[1, 2, 3, 4, 5]] = [0.0, 2.0 ** 100, 2.0 ** -120, 2.0 ** -140, 2.0 ** 60]
    w = (w * np.repeat(scale, seg)[None, :]).astype(np.float32)
    g = rng.uniform(0.5, 2, units).astype(np.float32)
    de_f = rng.standard_normal(w.shape) * np.where(np.arange(units * seg) // seg == 7, 2.0 ** 100, 1)
    from oracle.bf16 import bf16_rne
    de = bf16_rne(de_f)
    announce("colblock edge units")
    n, e = run_forward(B, [w], [g], [seg])
    check_forward(n[0], e[0], w, g, 1.0, seg, "edge fwd")
    dw, dg = run_backward(B, [w], [g], [de], [seg])
    check_backward(dw[0], dg[0], w, g, 1.0, de, seg, "edge bwd")
    wi = w.copy()
    wi[3, 2 * 9] = np.inf                             # unit 9 holds an infinity
    n, e = run_forward(B, [wi], [g], [seg])
    got = bf16_value(rows_of(e[0], seg))
    assert np.isnan(got[9]).any() and np.isfinite(got[np.arange(units) != 9]).all()


def test_gpt2_conv1d_workload(B):
    """GPT-2 small's 48 Conv1D weights, forward and backward, sampled units,
    every unit's length and the gradient's tangency on the device."""
    import torch
    c = inputs.make("rownorm_gain_gpt2_conv1d")
    announce("colblock", c.name, len(c.w))
    segs = [1] * len(c.w)
    n, e = run_forward(B, c.w, c.gain, segs)
    dw, dg = run_backward(B, c.w, c.gain, c.dwe, segs)
    for i, (w, g, de) in enumerate(zip(c.w, c.gain, c.dwe)):
        exact = np.sqrt((w.astype(np.float64) ** 2).sum(axis=0))
        assert contract_rel(n[i], exact).all(), f"matrix {i}: norms"
        wt = torch.from_numpy(w).to("cuda:0").double()
        dwt = torch.from_numpy(dw[i]).to("cuda:0").double()
        rad = (wt * dwt).sum(dim=0).abs()
        assert bool((rad <= 1e-5 * (wt * dwt).abs().sum(dim=0) + 1e-30).all().item()), i
        sample = np.unique(np.r_[0, w.shape[1] - 1, np.arange(0, w.shape[1], 61)])
        check_forward(n[i], e[i], w, g, 1.0, 1, f"matrix {i}", sample)
        check_backward(dw[i], dg[i], w, g, 1.0, de, 1, f"matrix {i}", sample)


def test_graph_replays_match_eager(B):
    """RMS rows and their gradient, a scalar-gain gradient (its row-share total
    kernel), single-element rows and column blocks, captured in one graph:
    each replay, with inputs rewritten eagerly between replays, equals eager
    calls bit for bit."""
    import torch
    dev = "cuda:0"
    gen = torch.Generator(device=dev).manual_seed(1900)
    x = torch.randn(512, 768, device=dev, generator=gen).to(torch.bfloat16)
    dy = torch.randn(512, 768, device=dev, generator=gen).to(torch.bfloat16)
    cb = inputs.colblock_grad_case([(96, 320), (12, 90)], 1, 1901)
    el = inputs.rownorm_grad_case([(40, 147)], 1902)
    ws = [torch.from_numpy(m).to(dev) for m in cb.w + el.w]
    gs = [torch.from_numpy(cb.gain[0]).to(dev), torch.from_numpy(cb.gain[1][:1]).to(dev).reshape(()),
          torch.from_numpy(el.gain[0]).to(dev)]
    des = [dev_bits(d) for d in cb.dwe + el.dwe]
    segs = [1, 1, None]
    y, dx = torch.empty_like(x), torch.empty_like(x)
    weff = [torch.empty(m.shape, dtype=torch.bfloat16, device=dev) for m in ws]
    norms = [torch.empty(m.shape[1] if s else m.shape[0], device=dev) for m, s in zip(ws, segs)]
    dws = [torch.empty_like(m) for m in ws]
    dgs = [torch.empty(ws[0].shape[1], device=dev), torch.empty((), device=dev),
           torch.empty(ws[2].shape[0], device=dev)]

    def step():
        B.ds_rms_rows(x, None, 1e-6, out=y)
        B.ds_rms_rows_backward(x, None, dy, 1e-6, out=dx)
        B.ds_weight_rownorm_gain(ws, gs, None, norm_out=norms, w_eff=weff, segs=segs)
        B.ds_weight_rownorm_gain_backward(ws, gs, des, dw=dws, dgain=dgs, segs=segs)

    announce("graph capture: rms, scalar gain, element rows, column blocks")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        g2 = torch.Generator(device=dev).manual_seed(1950 + rep)
        x.copy_(torch.randn(512, 768, device=dev, generator=g2).to(torch.bfloat16))
        for m in ws:
            m.mul_(0.5 + rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ye = B.ds_rms_rows(x, None, 1e-6)
        dxe = B.ds_rms_rows_backward(x, None, dy, 1e-6)
        ne, ee = B.ds_weight_rownorm_gain(ws, gs, None, segs=segs)
        dwe, dge = B.ds_weight_rownorm_gain_backward(ws, gs, des, segs=segs)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), ye.view(torch.int16)), rep
        assert torch.equal(dx.view(torch.int16), dxe.view(torch.int16)), rep
        for i in range(3):
            assert torch.equal(norms[i], ne[i]) and torch.equal(weff[i].view(torch.int16),
                                                                ee[i].view(torch.int16)), (rep, i)
            assert torch.equal(dws[i], dwe[i]) and torch.equal(dgs[i], dge[i]), (rep, i)
