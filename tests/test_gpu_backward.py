"""The gradients on the GPU against the CPU oracle: ds_l2_rows_backward and
ds_weight_rownorm_gain_backward.

Every compared element must meet the gradient contract (one bf16 ulp, or
2e-6 relative for fp32, plus 2^-16 of the size of the two terms whose
difference forms it) and lie inside the strict interval of an fp32 run with
the kernels' own sum-tree depth.  Full-size workloads are checked on sampled
rows against the oracle, and on every row through properties that hold at
any size (the gradient is tangent to the row; the gain gradient against a
float64 reduction on the device).
"""
import math

import numpy as np
import pytest

from gpu_util import announce, depth_for, dev_bits, dev_f32, host_bits, sample_rows
from oracle.bf16 import bf16_rne, bf16_value
from oracle.check import (admissible_l2_backward, admissible_rownorm_backward, contract_grad,
                          l2_grad_terms, rownorm_grad_terms)
from oracle.rows import eps_as_passed, l2_rows_backward, weight_rownorm_gain_backward
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


# ------------------------------------------------------------ l2_rows

def run_l2(B, x, r, dy, eps=1e-6):
    import torch
    dx = B.ds_l2_rows_backward(dev_bits(x), None if r is None else dev_bits(r), dev_bits(dy), eps)
    torch.cuda.synchronize()
    return host_bits(dx)


def s_values(x, r):
    xv = bf16_value(x)
    if r is None:
        return xv
    with np.errstate(all="ignore"):
        return bf16_value(bf16_rne(xv + bf16_value(r)))


def check_l2(got, x, r, dy, eps, rows, label):
    xs = x[rows]
    rs = None if r is None else r[rows]
    want = l2_rows_backward(xs, rs, dy[rows], eps)
    terms = l2_grad_terms(s_values(xs, rs), bf16_value(dy[rows]), eps_as_passed(eps))
    ok = contract_grad(got[rows], want, terms)
    assert ok.all(), f"{label}: {np.count_nonzero(~ok)} beyond the contract, e.g. {np.argwhere(~ok)[:4]}"
    rep = admissible_l2_backward(got[rows], xs, rs, dy[rows], eps, depth=depth_for(x.shape[1]),
                                 row_ids=rows)
    assert rep.ok, f"{label}: {rep}"
    return rep


WIDTHS = [8, 64, 512, 520, 1024, 4096, 4104, 7168, 8192, 8200, 16392, 32776, 65536]


@pytest.mark.parametrize("residual", [True, False])
@pytest.mark.parametrize("cols", WIDTHS)
def test_l2_widths(B, cols, residual):
    rows = 37 if cols <= 8200 else 5
    c = inputs.l2_grad_case(rows, cols, 1100 + cols % 97, residual=residual)
    announce("l2_rows_backward", rows, cols, "residual" if residual else "")
    got = run_l2(B, c.x, c.r, c.dy)
    check_l2(got, c.x, c.r, c.dy, 1e-6, np.arange(rows), f"{rows}x{cols}")


def _radial_property(x, r, dy, dx):
    """|<ds, s>| stays within the bf16 rounding of ds of its exact value
    <s, dy> eps / D^3, on every row (float64 on the device)."""
    import torch
    s = x.double() if r is None else (x.float() + r.float()).to(torch.bfloat16).double()
    d = dy.double()
    g = dx.double()
    d2 = (s * s).sum(dim=1) + eps_as_passed(1e-6)
    p = (s * d).sum(dim=1)
    lhs = (g * s).sum(dim=1)
    exact = p * eps_as_passed(1e-6) / d2 ** 1.5
    tol = 2.0 ** -7 * (g * s).abs().sum(dim=1) + 1e-30
    return bool(((lhs - exact).abs() <= tol).all().item())


def test_l2_full_workload(B):
    import torch
    c = inputs.make("l2_rows_res_bwd_8192x4096")
    announce("l2_rows_backward full", c.name)
    xd, rd, dyd = dev_bits(c.x), dev_bits(c.r), dev_bits(c.dy)
    dx = B.ds_l2_rows_backward(xd, rd, dyd, 1e-6)
    dx2 = B.ds_l2_rows_backward(xd, rd, dyd, 1e-6)
    part = B.ds_l2_rows_backward(xd[100:613], rd[100:613], dyd[100:613], 1e-6)
    torch.cuda.synchronize()
    got = host_bits(dx)
    assert np.array_equal(got, host_bits(dx2))
    assert np.array_equal(got[100:613], host_bits(part))       # rows do not see the batch
    assert _radial_property(xd, rd, dyd, dx)
    rows = sample_rows(8192, 48, 1101)
    check_l2(got, c.x, c.r, c.dy, 1e-6, rows, c.name)


def test_l2_stress_workload(B):
    import torch
    c = inputs.make("l2_rows_res_stress_32768x8192")
    dy = inputs.grad_bits(c.x.shape, 1102)
    announce("l2_rows_backward stress", c.name)
    xd, rd, dyd = dev_bits(c.x), dev_bits(c.r), dev_bits(dy)
    dx = B.ds_l2_rows_backward(xd, rd, dyd, 1e-6)
    torch.cuda.synchronize()
    assert _radial_property(xd, rd, dyd, dx)
    got = host_bits(dx)
    del xd, rd, dyd, dx
    zr, ir = c.meta["zero_rows"], c.meta["int_rows"]
    rows = sample_rows(c.x.shape[0], 24, 1103, must=list(zr[:8]) + list(ir[:8]))
    check_l2(got, c.x, c.r, dy, 1e-6, rows, c.name)


def test_l2_in_place(B):
    import torch
    c = inputs.l2_grad_case(300, 4096, 1104)
    want = run_l2(B, c.x, c.r, c.dy)
    for target in ("dy", "x", "r"):
        xd, rd, dyd = dev_bits(c.x), dev_bits(c.r), dev_bits(c.dy)
        out = {"dy": dyd, "x": xd, "r": rd}[target]
        announce("l2_rows_backward in place, dx =", target)
        B.ds_l2_rows_backward(xd, rd, dyd, 1e-6, out=out)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), want), target


def test_l2_extremes(B):
    """Rows whose fp32 sums overflow or underflow are rescaled, not lost."""
    rng = np.random.default_rng(1105)
    cols = 1024
    xs, dys = [], []
    for e_s, e_d in ((120, 0), (64, 0), (20, 100), (0, 120), (-20, 0), (-60, -60),
                     (-126, 0), (-133, 30), (10, -120), (0, 0)):
        xs.append(rng.standard_normal(cols) * 2.0 ** e_s)
        dys.append(rng.standard_normal(cols) * 2.0 ** e_d)
    big = np.zeros(cols); big[5] = 3.0e38; big[77] = -1.0e38
    xs.append(big); dys.append(rng.standard_normal(cols))
    sub = np.zeros(cols); sub[:7] = 2.0 ** -133 * np.arange(1, 8)
    xs.append(sub); dys.append(rng.standard_normal(cols))
    radial = rng.standard_normal(cols)
    xs.append(radial); dys.append(radial * 3.0)                   # dy parallel to s
    xs.append(np.zeros(cols)); dys.append(rng.standard_normal(cols))   # zero row
    x = bf16_rne(np.array(xs))
    dy = bf16_rne(np.array(dys))
    for eps in (1e-6, 0.0, 1.0, 2.0 ** -140):
        keep = np.array([bf16_value(x[i]).any() or eps > 0 for i in range(len(xs))])
        announce("l2_rows_backward extremes eps", eps)
        got = run_l2(B, x[keep], None, dy[keep], eps)
        check_l2(got, x[keep], None, dy[keep], eps, np.arange(int(keep.sum())), f"eps={eps}")


def test_l2_nonfinite(B):
    rng = np.random.default_rng(1106)
    x = bf16_rne(rng.standard_normal((7, 512)))
    r = bf16_rne(rng.standard_normal((7, 512)))
    dy = bf16_rne(rng.standard_normal((7, 512)))
    x[0, 3] = 0x7F80             # +inf in s
    x[1, 9] = 0x7FC0             # NaN in s
    dy[2, 5] = 0x7F80            # +inf in dy
    dy[3, 5], dy[3, 6] = 0x7F80, 0xFF80
    dy[4, 0] = 0x7FC0            # NaN in dy
    x[5, :] = 0
    r[5, :] = 0
    announce("l2_rows_backward non-finite")
    got = run_l2(B, x, r, dy)
    want = l2_rows_backward(x, r, dy)
    g, w = bf16_value(got), bf16_value(want)
    assert np.array_equal(np.isnan(g), np.isnan(w))
    fin = ~np.isnan(g)
    assert np.array_equal(np.isinf(g[fin]), np.isinf(w[fin]))
    assert np.array_equal(g[np.isinf(g)], w[np.isinf(w)])
    check_l2(got, x, r, dy, 1e-6, np.array([5, 6]), "finite rows")
    z = run_l2(B, x[5:6], r[5:6], dy[5:6], 0.0)                # eps = 0, zero row: 0/0
    assert np.isnan(bf16_value(z)).all()


def test_l2_empty(B):
    import torch
    e = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda:0")
    out = B.ds_l2_rows_backward(e, None, e, 1e-6)
    assert out.shape == (0, 64)


# ------------------------------------------------------------ weights

def run_rn(B, case, radius=None, want_dgain=True):
    import torch
    ws = [dev_f32(w) for w in case.w]
    gs = [dev_f32(g) for g in case.gain]
    des = [dev_bits(d) for d in case.dwe]
    dws, dgs = B.ds_weight_rownorm_gain_backward(ws, gs, des, radius or case.radius,
                                                 want_dgain=want_dgain)
    torch.cuda.synchronize()
    return ([d.cpu().numpy() for d in dws],
            [None if d is None else d.cpu().numpy() for d in dgs])


def check_rn(dw, dg, w, g, rho, de, rows, label):
    want_dw, want_dg = weight_rownorm_gain_backward([w[rows]], [g[rows]], [rho], [de[rows]])
    tw, tg = rownorm_grad_terms(w[rows].astype(np.float64), g[rows].astype(np.float64),
                                float(np.float32(rho)), bf16_value(de[rows]))
    ok = contract_grad(dw[rows], want_dw[0], tw, "f32")
    assert ok.all(), f"{label}: dW beyond the contract: {np.count_nonzero(~ok)} {np.argwhere(~ok)[:4]}"
    okg = contract_grad(dg[rows], want_dg[0], tg, "f32")
    assert okg.all(), f"{label}: dg beyond the contract: {np.argwhere(~okg)[:4]}"
    rw, rg = admissible_rownorm_backward(dw[rows], dg[rows], w[rows], g[rows], rho, de[rows],
                                         depth=depth_for(w.shape[1]))
    assert rw.ok and rg.ok, f"{label}: {rw} / {rg}"


@pytest.mark.parametrize("cols", [4, 8, 44, 768, 1028, 3072, 4096, 5000, 12288, 65536])
def test_rownorm_widths(B, cols):
    rows = 33 if cols <= 4096 else 5
    case = inputs.rownorm_grad_case([(rows, cols)], 1200 + cols % 89)
    announce("rownorm_backward single", rows, cols)
    dw, dg = run_rn(B, case)
    check_rn(dw[0], dg[0], case.w[0], case.gain[0], 1.0, case.dwe[0], np.arange(rows),
             f"{rows}x{cols}")


def _device_properties(B, case, dws, dgs):
    """Every row: dg against a float64 reduction on the device, and <dW, w> = 0."""
    import torch
    for i, (w, g, de) in enumerate(zip(case.w, case.gain, case.dwe)):
        wd = torch.from_numpy(w).to("cuda:0").double()
        gd = torch.from_numpy(g).to("cuda:0").double()
        dd = dev_bits(de).double()
        rho = float(np.float32(case.radius[i]))
        n = wd.pow(2).sum(dim=1).sqrt()
        p = (wd * dd).sum(dim=1)
        a = (wd * dd).abs().sum(dim=1)
        dg_exact = rho * p / n
        dg = torch.from_numpy(dgs[i]).to("cuda:0").double()
        tol = 2e-6 * dg_exact.abs() + 2.0 ** -16 * rho * a / n
        assert bool(((dg - dg_exact).abs() <= tol).all().item()), f"matrix {i}: dg"
        dw = torch.from_numpy(dws[i]).to("cuda:0").double()
        terms = (gd * rho).abs()[:, None] / n[:, None] * (dd.abs() + wd.abs() * (a / n ** 2)[:, None])
        rad = (dw * wd).sum(dim=1).abs()
        bound = 2.0 ** -16 * (wd.abs() * terms).sum(dim=1) + 4e-6 * (dw * wd).abs().sum(dim=1)
        assert bool((rad <= bound).all().item()), f"matrix {i}: dW not tangent"


def test_rownorm_transformer_workload(B):
    case = inputs.make("rownorm_gain_bwd_12x4_d768")
    announce("rownorm_backward full", case.name, len(case.w), case.total_rows)
    dw, dg = run_rn(B, case)
    dw2, dg2 = run_rn(B, case)
    for i in range(len(case.w)):
        assert np.array_equal(dw[i], dw2[i]) and np.array_equal(dg[i], dg2[i])
    _device_properties(B, case, dw, dg)
    for i, (w, g, de) in enumerate(zip(case.w, case.gain, case.dwe)):
        rows = sample_rows(w.shape[0], 12, 1300 + i)
        check_rn(dw[i], dg[i], w, g, 1.0, de, rows, f"matrix {i} {w.shape}")


def test_rownorm_pages_shape(B):
    case = inputs.make("rownorm_gain_bwd_11008x4096")
    announce("rownorm_backward", case.name)
    dw, dg = run_rn(B, case)
    _device_properties(B, case, dw, dg)
    rows = sample_rows(11008, 24, 1301)
    check_rn(dw[0], dg[0], case.w[0], case.gain[0], 1.0, case.dwe[0], rows, case.name)


def test_rownorm_ragged_equals_single(B):
    case = inputs.rownorm_grad_case([(100, 768), (7, 3072), (33, 44), (64, 768)], 1302)
    announce("rownorm_backward ragged vs single")
    dw, dg = run_rn(B, case)
    for i in range(len(case.w)):
        one = inputs.RownormGradCase("one", [case.w[i]], [case.gain[i]], [case.radius[i]],
                                     [case.dwe[i]])
        dw1, dg1 = run_rn(B, one)
        assert np.array_equal(dw1[0], dw[i]) and np.array_equal(dg1[0], dg[i])
    _, dg_none = run_rn(B, case, want_dgain=False)
    assert all(d is None for d in dg_none)


def test_rownorm_edge_rows(B):
    rng = np.random.default_rng(1303)
    cols = 768
    w = (0.02 * rng.standard_normal((12, cols))).astype(np.float32)
    w[0] = 0                                                     # zero row
    w[1] *= np.float32(2.0 ** 100)                               # S overflows
    w[2] *= np.float32(2.0 ** -70)                               # S underflows
    w[3, :] = 0
    w[3, 7] = np.float32(1e-42)                                  # one subnormal
    w[4, :] = 0
    w[4, :3] = [3, 4, 0]                                         # closed-form row
    g = rng.uniform(-2, 2, 12).astype(np.float32)
    de = bf16_rne(rng.standard_normal((12, cols)))
    w[5] *= np.float32(2.0 ** 20)
    de[5] = bf16_rne(rng.standard_normal(cols) * 2.0 ** 115)     # P overflows
    de[6] = bf16_rne(rng.standard_normal(cols) * 2.0 ** -120)    # P underflows
    de[7] = bf16_rne(w[7].astype(np.float64) * 50)               # radial dWe: dW ~ 0
    de[0, 3] = 0x7FC0                                            # NaN into a zero row
    for rho in (1.0, math.sqrt(768.0)):
        case = inputs.RownormGradCase("edge", [w], [g], [rho], [de])
        announce("rownorm_backward edge rows rho", rho)
        dw, dg = run_rn(B, case)
        assert not dw[0][0].any() and dg[0][0] == 0                # zero row: exact zeros
        check_rn(dw[0], dg[0], w, g, rho, de, np.arange(1, 12), f"edge rho={rho}")


def test_rownorm_nonfinite(B):
    rng = np.random.default_rng(1304)
    w = (0.02 * rng.standard_normal((4, 64))).astype(np.float32)
    g = rng.uniform(0.5, 2, 4).astype(np.float32)
    de = bf16_rne(rng.standard_normal((4, 64)))
    w[0, 1] = np.inf
    g[1] = np.nan
    de[2, 2] = 0x7FC0
    case = inputs.RownormGradCase("nonfinite", [w], [g], [1.0], [de])
    announce("rownorm_backward non-finite")
    dw, dg = run_rn(B, case)
    want_dw, want_dg = weight_rownorm_gain_backward([w], [g], [1.0], [de])
    for got, want in ((dw[0], want_dw[0]), (dg[0], want_dg[0])):
        assert np.array_equal(np.isnan(got), np.isnan(want))
    check_rn(dw[0], dg[0], w, g, 1.0, de, np.array([3]), "finite row")


def test_rownorm_staged_table(B):
    """More than 48 matrices of one width: the staged descriptor table."""
    shapes = [(5, 64)] * 60 + [(3, 768)] * 5
    case = inputs.rownorm_grad_case(shapes, 1305)
    announce("rownorm_backward staged", len(shapes))
    dw, dg = run_rn(B, case)
    for i in (0, 31, 59, 60, 64):
        check_rn(dw[i], dg[i], case.w[i], case.gain[i], 1.0, case.dwe[i],
                 np.arange(case.w[i].shape[0]), f"matrix {i}")


def test_backward_graph_replays_match_eager(B):
    """Both gradient calls (inline tables) captured in a graph: each replay, with
    new inputs written eagerly between replays, equals eager calls bit for bit."""
    import torch
    dev = "cuda:0"
    gen = torch.Generator(device=dev).manual_seed(1306)
    x = torch.randn(256, 4096, device=dev, generator=gen).to(torch.bfloat16)
    r = torch.randn(256, 4096, device=dev, generator=gen).to(torch.bfloat16)
    dy = torch.randn(256, 4096, device=dev, generator=gen).to(torch.bfloat16)
    case = inputs.rownorm_grad_case([(96, 768), (48, 3072)], 1307)
    ws = [torch.from_numpy(m).to(dev) for m in case.w]
    gs = [torch.from_numpy(v).to(dev) for v in case.gain]
    des = [dev_bits(d) for d in case.dwe]
    dx = torch.empty_like(x)
    dws = [torch.empty_like(m) for m in ws]
    dgs = [torch.empty(m.shape[0], device=dev) for m in ws]

    def step():
        B.ds_l2_rows_backward(x, r, dy, 1e-6, out=dx)
        B.ds_weight_rownorm_gain_backward(ws, gs, des, dw=dws, dgain=dgs)

    announce("graph capture: both gradients")
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
        g2 = torch.Generator(device=dev).manual_seed(1400 + rep)
        dy.copy_(torch.randn(256, 4096, device=dev, generator=g2).to(torch.bfloat16))
        x.copy_(torch.randn(256, 4096, device=dev, generator=g2).to(torch.bfloat16))
        for m in ws:
            m.mul_(0.75)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        dxe = B.ds_l2_rows_backward(x, r, dy, 1e-6)
        dwe, dge = B.ds_weight_rownorm_gain_backward(ws, gs, des)
        torch.cuda.synchronize()
        assert torch.equal(dx.view(torch.int16), dxe.view(torch.int16)), f"replay {rep}: l2"
        for i in range(len(ws)):
            assert torch.equal(dws[i], dwe[i]) and torch.equal(dgs[i], dge[i]), \
                f"replay {rep}: weights {i}"
