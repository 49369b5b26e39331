"""ds_l2_rows on the GPU against the CPU oracle.

Element-by-element at sizes the oracle finishes in seconds (several vector
groups and ragged tails); sampled rows plus size-independent properties at
the full workload sizes, in the launch configuration the benchmark times.
Tolerances: the 1-bf16-ulp contract and the strict admissible set.
"""
import numpy as np
import pytest

from gpu_util import announce, depth_for, dev_bits, host_bits, sample_rows, unit_norm_ok
from oracle.bf16 import bf16_rne, bf16_value
from oracle.check import admissible_l2_rows, contract_bf16
from oracle.rows import l2_rows as l2_ref
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


def run(B, x, r=None, eps=1e-6):
    import torch
    xd = dev_bits(x)
    rd = None if r is None else dev_bits(r)
    y = B.ds_l2_rows(xd, rd, eps)
    torch.cuda.synchronize()
    return host_bits(y)


def full_check(got, x, r, eps, label):
    want = l2_ref(x, r, eps)
    ok = contract_bf16(got, want)
    assert ok.all(), f"{label}: {np.count_nonzero(~ok)} elements beyond 1 ulp, first {np.argwhere(~ok)[:5]}"
    rep = admissible_l2_rows(got, x, r, eps, depth=depth_for(np.shape(x)[-1]))
    assert rep.ok, f"{label}: {rep}"


# every side of the shape policy's class boundaries (64, 128, 256, 512, 1024,
# 2048 and 4096 vectors of 8 columns), the widths of the pages, and the limit
COLS = [8, 64, 512, 520, 1024, 1032, 2048, 2056, 4096, 4104, 7168, 8192, 8200, 12296,
        16384, 16392, 32768, 32776, 65528, 65536]


@pytest.mark.parametrize("cols", COLS)
@pytest.mark.parametrize("residual", [False, True])
def test_small_shapes(B, cols, residual):
    rows = 37 if cols <= 8192 else 5
    c = inputs.l2_case(rows, cols, 500 + cols % 97, residual=residual)
    announce("l2_rows small", rows, cols, residual)
    got = run(B, c.x, c.r)
    full_check(got, c.x, c.r, 1e-6, f"{rows}x{cols}")


def test_workload_64x1024(B):
    c = inputs.make("l2_rows_64x1024")
    announce("l2_rows", c.name)
    got = run(B, c.x, c.r, c.eps)
    full_check(got, c.x, c.r, c.eps, c.name)
    assert np.array_equal(got, l2_ref(c.x, c.r, c.eps))   # no near-tie moved here


def _big(B, c, nsample, must=()):
    import torch
    announce("l2_rows full size", c.name, c.rows, c.cols)
    xd = dev_bits(c.x)
    rd = None if c.r is None else dev_bits(c.r)
    y = B.ds_l2_rows(xd, rd, c.eps)
    y2 = B.ds_l2_rows(xd, rd, c.eps)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "repeat run differs"
    idx = sample_rows(c.rows, nsample, 7, must)
    got = host_bits(y)[idx]
    xs, rs = c.x[idx], None if c.r is None else c.r[idx]
    full_check(got, xs, rs, c.eps, c.name)
    # rows [a:b] alone give the same bits as inside the full batch
    a, b = c.rows // 3, c.rows // 3 + 1000
    ys = B.ds_l2_rows(xd[a:b].contiguous(), None if rd is None else rd[a:b].contiguous(), c.eps)
    torch.cuda.synchronize()
    assert torch.equal(ys.view(torch.int16), y[a:b].view(torch.int16))
    return xd, rd, y


def test_workload_8192x4096_residual(B):
    import torch
    c = inputs.make("l2_rows_res_8192x4096")
    xd, rd, y = _big(B, c, 512)
    assert unit_norm_ok(y)
    # the residual add is symmetric, and l2 is odd
    y_sw = B.ds_l2_rows(rd, xd, c.eps)
    neg = B.ds_l2_rows((xd.view(torch.int16) ^ -32768).view(torch.bfloat16),
                       (rd.view(torch.int16) ^ -32768).view(torch.bfloat16), c.eps)
    torch.cuda.synchronize()
    assert torch.equal(y_sw.view(torch.int16), y.view(torch.int16))
    # odd symmetry, bit for bit, except that an exact cancellation x + r = 0
    # is +0 for either sign of the inputs (IEEE round-to-nearest)
    nz = y.float() != 0
    assert torch.equal(neg.view(torch.int16)[nz], (y.view(torch.int16) ^ -32768)[nz])
    assert (neg.float()[~nz] == 0).all()


def test_workload_stress_32768x8192(B):
    import torch
    c = inputs.make("l2_rows_res_stress_32768x8192")
    zero, ints = c.meta["zero_rows"], c.meta["int_rows"]
    must = np.concatenate([zero[:40], ints[:60]])
    xd, rd, y = _big(B, c, 700, must)
    # zero rows -> +0 rows; every other row unit length
    assert not y[torch.as_tensor(zero, device=y.device)].view(torch.int16).any().item()
    assert unit_norm_ok(y, skip_rows=zero)
    # integer rows: every fp32 partial sum is exact, so the sum tree is exact
    got = host_bits(y)[ints[:100]]
    rep = admissible_l2_rows(got, c.x[ints[:100]], c.r[ints[:100]], c.eps, depth=0)
    assert rep.ok, str(rep)
    # the same workload without the residual
    y0 = B.ds_l2_rows(xd, None, c.eps)
    torch.cuda.synchronize()
    idx = sample_rows(c.rows, 200, 8, must)
    full_check(host_bits(y0)[idx], c.x[idx], None, c.eps, c.name + " r=NULL")


def test_more_rows_than_one_launch(B, monkeypatch):
    """l2_rows, rms_rows and their gradients over several launches
    (DS_ROWS_TEST_MAX_GROUPS lowers the cap of 64 workgroups per compute
    unit): the bits equal one launch's, at one row per workgroup and at
    four."""
    import torch
    for rows, cols, cap in ((301, 4096, "64"), (301, 768, "10")):
        c = inputs.l2_case(rows, cols, 631 + cols, residual=True)
        announce("l2/rms rows in pieces", rows, cols, cap)
        xd, rd = dev_bits(c.x), dev_bits(c.r)
        dy = dev_bits(inputs.l2_case(rows, cols, 632 + cols).x)
        calls = (lambda: B.ds_l2_rows(xd, rd, c.eps), lambda: B.ds_rms_rows(xd, rd, c.eps),
                 lambda: B.ds_l2_rows_backward(xd, rd, dy, c.eps),
                 lambda: B.ds_rms_rows_backward(xd, rd, dy, c.eps))
        one = [f() for f in calls]
        monkeypatch.setenv("DS_ROWS_TEST_MAX_GROUPS", cap)
        pieces = [f() for f in calls]
        monkeypatch.delenv("DS_ROWS_TEST_MAX_GROUPS")
        torch.cuda.synchronize()
        for a, b in zip(one, pieces):
            assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (rows, cols)
        full_check(host_bits(pieces[0]), c.x, c.r, c.eps, f"pieces {rows}x{cols}")


def test_zero_rows_enqueue_nothing(B):
    import torch
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda:0")
    y = B.ds_l2_rows(x)
    assert y.shape == (0, 64)


def test_in_place(B):
    import torch
    c = inputs.l2_case(300, 4096, 601)
    want = l2_ref(c.x, c.r)
    xd, rd = dev_bits(c.x), dev_bits(c.r)
    announce("l2_rows in place y=x, y=r")
    B.ds_l2_rows(xd, rd, 1e-6, out=xd)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(xd), run(B, c.x, c.r))
    xd = dev_bits(c.x)
    B.ds_l2_rows(xd, rd, 1e-6, out=rd)
    torch.cuda.synchronize()
    assert contract_bf16(host_bits(rd), want).all()


def test_extreme_magnitudes_and_eps(B):
    """Rows whose fp32 sum overflows or underflows are rescaled, not lost."""
    rng = np.random.default_rng(602)
    cols = 1024
    rows = []
    for e in (120, 100, 64, 63, 20, -20, -60, -63, -64, -80, -110, -126, -133):
        rows.append(rng.standard_normal(cols) * 2.0 ** e)
    big = np.zeros(cols); big[5] = 3.0e38; big[77] = -1.0e38          # squares overflow
    rows.append(big)
    sub = np.zeros(cols); sub[:7] = 2.0 ** -133 * np.arange(1, 8)       # bf16 subnormals
    rows.append(sub)
    rows.append(np.zeros(cols))                                         # eps alone
    x = bf16_rne(np.array(rows))
    for eps in (1e-6, 0.0, 2.0 ** -140, 1.0, 3.0e38):
        announce("l2_rows extremes eps", eps)
        got = run(B, x, None, eps)
        keep = np.array([bf16_value(x[i]).any() or eps > 0 for i in range(len(rows))])
        full_check(got[keep], x[keep], None, eps, f"extremes eps={eps}")


def test_nonfinite_propagation(B):
    rng = np.random.default_rng(603)
    x = bf16_rne(rng.standard_normal((6, 512)))
    r = bf16_rne(rng.standard_normal((6, 512)))
    x[0, 3] = 0x7F80           # +inf
    x[1, 9] = 0xFF80           # -inf
    x[2, 100] = 0x7FC0         # NaN
    r[3, 0] = 0x7FC0
    x[4, 1], r[4, 1] = 0x7F80, 0xFF80       # inf + -inf = NaN
    announce("l2_rows non-finite")
    got = run(B, x, r)
    want = l2_ref(x, r)
    g, w = bf16_value(got), bf16_value(want)
    assert np.array_equal(np.isnan(g), np.isnan(w))
    assert np.array_equal(g[~np.isnan(g)], w[~np.isnan(w)])
    assert np.array_equal(np.signbit(g[~np.isnan(g)]), np.signbit(w[~np.isnan(w)]))
    assert (got[5] == run(B, x[5:6], r[5:6])[0]).all()


def test_signed_zero_and_cancellation(B):
    x = np.zeros((2, 64), np.uint16)
    r = np.zeros((2, 64), np.uint16)
    x[0, :4] = bf16_rne(np.array([1.5, -2.0, 3.0, -0.0]))
    r[0, :4] = bf16_rne(np.array([-1.5, 2.0, 1.0, -0.0]))
    x[1, :] = 0x8000           # -0 row, no residual part
    r[1, :] = 0x8000
    announce("l2_rows signed zeros")
    got = run(B, x, r)
    assert np.array_equal(got, l2_ref(x, r))
    assert got[0, 3] == 0x8000 and (got[1] == 0x8000).all()
