"""ds_rms_rows and ds_rms_rows_backward on the GPU against the CPU oracle.

Element by element at sizes the oracle finishes in seconds, over every side of
the shape policy's classes with and without a residual; sampled rows plus
properties that hold at any size (unit RMS of every output row; the gradient's
radial part <ds, s> = <s, dy> eps / D^3) at the full workload sizes.
Tolerances: one bf16 ulp for the forward, the gradient contract (one bf16
ulp plus 2^-16 of the size of its two terms) for the backward, and the strict
admissible sets of an fp32 run with the mean.
"""
import numpy as np
import pytest

from gpu_util import announce, depth_for, dev_bits, host_bits, sample_rows
from oracle.bf16 import bf16_rne, bf16_value
from oracle.check import admissible_l2_backward, admissible_l2_rows, contract_bf16, \
    contract_grad, l2_grad_terms
from oracle.rows import eps_as_passed, rms_rows, rms_rows_backward
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


def s_values(x, r):
    xv = bf16_value(x)
    if r is None:
        return xv
    with np.errstate(all="ignore"):
        return bf16_value(bf16_rne(xv + bf16_value(r)))


def fwd(B, x, r, eps=1e-6):
    import torch
    y = B.ds_rms_rows(dev_bits(x), None if r is None else dev_bits(r), eps)
    torch.cuda.synchronize()
    return host_bits(y)


def bwd(B, x, r, dy, eps=1e-6):
    import torch
    dx = B.ds_rms_rows_backward(dev_bits(x), None if r is None else dev_bits(r), dev_bits(dy), eps)
    torch.cuda.synchronize()
    return host_bits(dx)


def check_fwd(got, x, r, eps, label):
    ok = contract_bf16(got, rms_rows(x, r, eps))
    assert ok.all(), f"{label}: {np.count_nonzero(~ok)} beyond 1 ulp, e.g. {np.argwhere(~ok)[:4]}"
    rep = admissible_l2_rows(got, x, r, eps, depth=depth_for(x.shape[1]), mean=True)
    assert rep.ok, f"{label}: {rep}"


def check_bwd(got, x, r, dy, eps, label):
    terms = l2_grad_terms(s_values(x, r), bf16_value(dy), eps_as_passed(eps), mean=True)
    ok = contract_grad(got, rms_rows_backward(x, r, dy, eps), terms)
    assert ok.all(), f"{label}: {np.count_nonzero(~ok)} beyond the contract, e.g. {np.argwhere(~ok)[:4]}"
    rep = admissible_l2_backward(got, x, r, dy, eps, depth=depth_for(x.shape[1]), mean=True)
    assert rep.ok, f"{label}: {rep}"


# the pages' d_model widths and every side of the shape classes
WIDTHS = [8, 64, 256, 320, 384, 512, 520, 768, 1024, 1032, 2048, 4096, 4104, 7168, 8192, 8200,
          16392, 32776, 65536]


@pytest.mark.parametrize("residual", [False, True])
@pytest.mark.parametrize("cols", WIDTHS)
def test_widths(B, cols, residual):
    rows = 37 if cols <= 8200 else 5
    c = inputs.l2_grad_case(rows, cols, 1200 + cols % 89, residual=residual)
    announce("rms_rows fwd+bwd", rows, cols, "residual" if residual else "")
    check_fwd(fwd(B, c.x, c.r), c.x, c.r, 1e-6, f"fwd {rows}x{cols}")
    check_bwd(bwd(B, c.x, c.r, c.dy), c.x, c.r, c.dy, 1e-6, f"bwd {rows}x{cols}")


def _rms_one(y, tol=2.0 ** -7):
    """Every output row has mean square 1 within tol (on the device)."""
    ms = y.double().pow(2).mean(dim=1)
    return bool(((ms - 1).abs() <= tol).all().item())


def _radial_ok(s, dy, dx, eps):
    """|<ds, s> - <s, dy> eps / D^3| within the bf16 rounding of ds (device, float64)."""
    n = s.shape[1]
    d2 = s.pow(2).sum(dim=1) / n + eps_as_passed(eps)
    p = (s * dy).sum(dim=1)
    lhs = (dx * s).sum(dim=1)
    tol = 2.0 ** -7 * (dx * s).abs().sum(dim=1) + 1e-30
    return bool(((lhs - p * eps_as_passed(eps) / d2 ** 1.5).abs() <= tol).all().item())


def test_workload(B):
    import torch
    c = inputs.make("rms_rows_bwd_16384x768")
    announce("rms_rows full", c.name)
    xd, dyd = dev_bits(c.x), dev_bits(c.dy)
    y = B.ds_rms_rows(xd, None, 1e-6)
    y2 = B.ds_rms_rows(xd, None, 1e-6)
    dx = B.ds_rms_rows_backward(xd, None, dyd, 1e-6)
    part = B.ds_rms_rows_backward(xd[999:2040], None, dyd[999:2040], 1e-6)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert _rms_one(y)
    assert _radial_ok(xd.double(), dyd.double(), dx.double(), 1e-6)
    gy, gdx = host_bits(y), host_bits(dx)
    assert np.array_equal(gdx[999:2040], host_bits(part))        # rows do not see the batch
    rows = sample_rows(c.x.shape[0], 64, 1201)
    check_fwd(gy[rows], c.x[rows], None, 1e-6, c.name)
    check_bwd(gdx[rows], c.x[rows], None, c.dy[rows], 1e-6, c.name)


def test_stress_workload(B):
    import torch
    c = inputs.make("l2_rows_res_stress_32768x8192")
    dy = inputs.grad_bits(c.x.shape, 1202)
    announce("rms_rows stress", c.name)
    xd, rd, dyd = dev_bits(c.x), dev_bits(c.r), dev_bits(dy)
    y = B.ds_rms_rows(xd, rd, 1e-6)
    dx = B.ds_rms_rows_backward(xd, rd, dyd, 1e-6)
    torch.cuda.synchronize()
    zr, ir = c.meta["zero_rows"], c.meta["int_rows"]
    gy, gdx = host_bits(y), host_bits(dx)
    del xd, rd, dyd, y, dx
    rows = sample_rows(c.x.shape[0], 24, 1203, must=list(zr[:8]) + list(ir[:8]))
    check_fwd(gy[rows], c.x[rows], c.r[rows], 1e-6, c.name)
    check_bwd(gdx[rows], c.x[rows], c.r[rows], dy[rows], 1e-6, c.name)


def test_extremes(B):
    """Rows whose fp32 sums overflow or underflow are rescaled, not lost."""
    rng = np.random.default_rng(1204)
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
    xs.append(radial); dys.append(radial * 3.0)
    xs.append(np.zeros(cols)); dys.append(rng.standard_normal(cols))
    x = bf16_rne(np.array(xs))
    dy = bf16_rne(np.array(dys))
    for eps in (1e-6, 0.0, 1.0, 2.0 ** -140):
        keep = np.array([bf16_value(x[i]).any() or eps > 0 for i in range(len(xs))])
        announce("rms_rows extremes eps", eps)
        check_fwd(fwd(B, x[keep], None, eps), x[keep], None, eps, f"fwd eps={eps}")
        check_bwd(bwd(B, x[keep], None, dy[keep], eps), x[keep], None, dy[keep], eps,
                  f"bwd eps={eps}")


def test_nonfinite_and_zero_rows(B):
    rng = np.random.default_rng(1205)
    x = bf16_rne(rng.standard_normal((6, 512)))
    dy = bf16_rne(rng.standard_normal((6, 512)))
    x[0, 3] = 0x7F80             # +inf
    x[1, 9] = 0x7FC0             # NaN
    dy[2, 5] = 0x7F80
    x[3, :] = 0                  # zero row: y = 0, dx = dy / sqrt(eps)
    announce("rms_rows non-finite")
    gy = fwd(B, x, None)
    gdx = bwd(B, x, None, dy)
    check_fwd(gy, x, None, 1e-6, "non-finite fwd")
    assert np.array_equal(bf16_value(gdx[3]), bf16_value(rms_rows_backward(x[3:4], None, dy[3:4]))[0])
    want = rms_rows_backward(x, None, dy)
    gv, wv = bf16_value(gdx), bf16_value(want)
    assert np.array_equal(np.isnan(gv), np.isnan(wv))
    assert np.array_equal(gv[~np.isnan(wv)] == np.inf, wv[~np.isnan(wv)] == np.inf)


def test_in_place(B):
    import torch
    c = inputs.l2_grad_case(200, 768, 1206)
    want_y = fwd(B, c.x, c.r)
    want_dx = bwd(B, c.x, c.r, c.dy)
    for target in ("x", "r"):
        xd, rd = dev_bits(c.x), dev_bits(c.r)
        out = xd if target == "x" else rd
        announce("rms_rows in place, y =", target)
        B.ds_rms_rows(xd, rd, 1e-6, out=out)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), want_y), target
    for target in ("dy", "x", "r"):
        xd, rd, dyd = dev_bits(c.x), dev_bits(c.r), dev_bits(c.dy)
        out = {"dy": dyd, "x": xd, "r": rd}[target]
        announce("rms_rows_backward in place, dx =", target)
        B.ds_rms_rows_backward(xd, rd, dyd, 1e-6, out=out)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(out), want_dx), target


def test_against_l2_with_eps_scaled_by_n(B):
    """At n = 4^k, rms(s, eps) and 2^k l2(s, n eps) agree within one bf16 ulp."""
    import torch
    c = inputs.l2_case(64, 4096, 1207)
    xd, rd = dev_bits(c.x), dev_bits(c.r)
    announce("rms_rows vs l2_rows at 4096")
    y_rms = B.ds_rms_rows(xd, rd, 1e-6)
    y_l2 = B.ds_l2_rows(xd, rd, float(np.float32(1e-6)) * 4096)
    torch.cuda.synchronize()
    scaled = bf16_rne(bf16_value(host_bits(y_l2)) * 64.0)
    assert contract_bf16(host_bits(y_rms), scaled).all()


def test_empty(B):
    import torch
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda:0")
    assert B.ds_rms_rows(x).shape == (0, 64)
    assert B.ds_rms_rows_backward(x, None, x).shape == (0, 64)
