"""ds_rescale_project and ds_rescale_after_step on the GPU against the oracle.

The projected rows meet the gradient contract (2e-6 relative plus 2^-16 of
their cancelling terms) and the strict interval; rescaled rows are within
2e-6 and inside their interval.  The 48-matrix workload is checked on
sampled rows and, on every row, through the properties the method exists
for: rescaled rows have the radius, projected rows are tangent.
"""
import math

import numpy as np
import pytest

from gpu_util import announce, depth_for, dev_f32, sample_rows
from oracle.check import admissible_rescale, contract_grad, contract_rel, rescale_terms
from oracle.rows import rescale_after_step, rescale_project
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


def run(B, case, after_step, with_v=True):
    import torch
    ws = [dev_f32(w) for w in case.w]
    vs = [dev_f32(v) for v in case.v] if with_v else None
    if after_step:
        B.ds_rescale_after_step(ws, vs, case.radius)
    else:
        B.ds_rescale_project(ws, vs)
    torch.cuda.synchronize()
    return [w.cpu().numpy() for w in ws], (None if vs is None else [v.cpu().numpy() for v in vs])


def check(gw, gv, w, v, rho, after_step, rows, label):
    w, gw = w[rows], gw[rows]
    v = None if v is None else v[rows]
    gv = None if gv is None else gv[rows]
    if after_step:
        ws, ms = rescale_after_step([w], [v], [rho])
        ok = contract_rel(gw, ws[0])
        assert ok.all(), f"{label}: w beyond 2e-6: {np.argwhere(~ok)[:4]}"
    else:
        ms = rescale_project([w], [v])
        assert np.array_equal(gw, w), f"{label}: project changed w"
    if v is not None:
        terms = rescale_terms(w.astype(np.float64), v.astype(np.float64))
        ok = contract_grad(gv, ms[0], terms, "f32")
        assert ok.all(), f"{label}: v beyond the contract: {np.argwhere(~ok)[:4]}"
    rw, rv = admissible_rescale(gw, gv, w, v, rho, after_step, depth=depth_for(w.shape[1]))
    assert rv.ok and (rw.ok or not after_step), f"{label}: {rw} / {rv}"


@pytest.mark.parametrize("after_step", [False, True])
@pytest.mark.parametrize("cols", [4, 8, 44, 768, 1028, 3072, 4096, 5000, 12288, 65536])
def test_widths(B, cols, after_step):
    rows = 33 if cols <= 4096 else 5
    case = inputs.rescale_case([(rows, cols)], 1800 + cols % 71, radius=1.5)
    announce("rescale", "after_step" if after_step else "project", rows, cols)
    gw, gv = run(B, case, after_step)
    check(gw[0], gv[0], case.w[0], case.v[0], 1.5, after_step, np.arange(rows), f"{rows}x{cols}")


def test_after_step_without_momentum(B):
    case = inputs.rescale_case([(40, 768), (9, 3072)], 1801, radius=2.0)
    announce("rescale after_step, no momentum")
    gw, _ = run(B, case, True, with_v=False)
    for i in range(2):
        check(gw[i], None, case.w[i], None, 2.0, True, np.arange(case.w[i].shape[0]), f"m{i}")


def test_workload(B):
    import torch
    case = inputs.make("rescale_12x4_d768")
    announce("rescale workload", case.name, len(case.w))
    for after_step in (False, True):
        gw, gv = run(B, case, after_step)
        for i, (w, v) in enumerate(zip(case.w, case.v)):
            w64 = torch.from_numpy(gw[i]).double()
            v64 = torch.from_numpy(gv[i]).double()
            ref = torch.from_numpy(w).double() if not after_step else w64
            rad = (ref * v64).sum(1).abs()
            bound = 2.0 ** -16 * (ref.abs() * torch.from_numpy(
                rescale_terms(w.astype(np.float64), v.astype(np.float64)))).sum(1) + 1e-30
            assert bool((rad <= bound).all()), f"matrix {i}: projection not tangent"
            if after_step:
                n = w64.pow(2).sum(1).sqrt()
                assert bool(((n - 1).abs() <= 4 * 2.0 ** -24).all()), f"matrix {i}: radius"
            rows = sample_rows(w.shape[0], 8, 1802 + i)
            check(gw[i], gv[i], w, v, 1.0, after_step, rows, f"matrix {i} {w.shape}")


def test_edge_rows(B):
    rng = np.random.default_rng(1803)
    cols = 768
    w = (0.02 * rng.standard_normal((8, cols))).astype(np.float32)
    v = (1e-3 * rng.standard_normal((8, cols))).astype(np.float32)
    w[0] = 0                                              # zero row: left as it is
    w[1] *= np.float32(2.0 ** 100)                        # S overflows
    w[2] *= np.float32(2.0 ** -70)                        # S underflows
    w[3] *= np.float32(2.0 ** 30)
    v[3] = (rng.standard_normal(cols) * 2.0 ** 100).astype(np.float32)   # P overflows
    v[4] = (w[4] * np.float32(5.0)).astype(np.float32)                   # radial: v -> ~0
    v[5] = 0
    for after_step in (False, True):
        case = inputs.RescaleCase("edge", [w], [v], [3.0])
        announce("rescale edge rows", after_step)
        gw, gv = run(B, case, after_step)
        assert np.array_equal(gv[0][0], v[0]) and np.array_equal(gw[0][0], w[0])
        check(gw[0], gv[0], w, v, 3.0, after_step, np.arange(1, 8), f"edge {after_step}")


def test_ragged_equals_single_and_staged(B):
    case = inputs.rescale_case([(5, 64)] * 52 + [(7, 3072), (3, 44)], 1804)
    announce("rescale staged", len(case.w))
    gw, gv = run(B, case, True)
    for i in (0, 51, 52, 53):
        one = inputs.RescaleCase("one", [case.w[i]], [case.v[i]], [case.radius[i]])
        w1, v1 = run(B, one, True)
        assert np.array_equal(w1[0], gw[i]) and np.array_equal(v1[0], gv[i]), i


def test_graph_replays_match_eager(B):
    import torch
    case = inputs.rescale_case([(96, 768), (24, 3072)], 1805)
    dev = "cuda:0"
    ws = [torch.from_numpy(w).to(dev) for w in case.w]
    gs = [torch.from_numpy(v).to(dev) for v in case.v]
    ms = [torch.from_numpy(v * 3).to(dev) for v in case.v]
    w0 = [w.clone() for w in ws]

    def step():
        B.ds_rescale_project(ws, gs)
        for w, g in zip(ws, gs):
            w.sub_(g, alpha=0.1)                          # an SGD step between the two
        B.ds_rescale_after_step(ws, ms, [1.0, 1.0])

    announce("rescale graph capture")
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
        gen = torch.Generator(device=dev).manual_seed(1900 + rep)
        for w, g, m, w_init in zip(ws, gs, ms, w0):
            w.copy_(w_init * (1 + rep))
            g.copy_(torch.randn(g.shape, device=dev, generator=gen) * 1e-3)
            m.copy_(torch.randn(m.shape, device=dev, generator=gen) * 1e-3)
        snap = [t.clone() for t in ws + gs + ms]
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        out = [t.clone() for t in ws + gs + ms]
        for t, s_ in zip(ws + gs + ms, snap):
            t.copy_(s_)
        torch.cuda.synchronize()
        step()
        torch.cuda.synchronize()
        for a, b in zip(out, ws + gs + ms):
            assert torch.equal(a, b), f"replay {rep}"
