"""The seg-1 column-block kernel (units and ld multiples of 4; 16-byte-aligned
buffers) against the CPU oracle: single-pass tiles (64 units for the forward
and the gradient, 32 for the rescale calls) with stored-row counts that fill
the lanes' K vectors exactly or leave them ragged, a ragged last tile, a gap
between the units' columns and the next stored row (ld > units), units out
of fp32's range and zero units (the rescue path); two-pass tiles in the same
launch for taller matrices; a ragged call mixing both equal to each matrix
alone; and the layouts that fall back to the two-pass kernel (a unit count
or ld not a multiple of 4, a misaligned buffer) giving the same contract.

Each case runs the forward, the gradient and both rescale calls through the
C ABI and checks the 1-ulp contract and the strict interval at the depth of
the kernel that ran (tests/test_gpu_colblock.py: single_pass_lanes)."""
import numpy as np
import pytest

from gpu_util import announce, dev_bits, dev_f32, host_bits
from oracle.bf16 import bf16_rne, bf16_value
from oracle.check import (admissible_rescale, admissible_rownorm, admissible_rownorm_backward,
                          contract_bf16, contract_grad, contract_rel, rescale_terms,
                          rownorm_grad_terms)
from oracle.rows import (column_block_rows, rescale_after_step, rescale_project,
                         weight_rownorm_gain, weight_rownorm_gain_backward)
from test_gpu_colblock import depth_col, single_pass_lanes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


def call_forward(B, wd, gd, units, A, ld, weff, norms, radius=1.0):
    import torch
    d = (B.RownormDesc * 1)()
    d[0] = B.RownormDesc(wd.data_ptr(), gd.data_ptr(), radius, norms.data_ptr(), weff.data_ptr(),
                         units, A, 0, 1, ld)
    st = B.lib().ds_weight_rownorm_gain(d, 1, torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().ds_status_string(st)


def call_backward(B, wd, gd, ded, units, A, ld, dw, dg, radius=1.0):
    import torch
    d = (B.RownormGradDesc * 1)()
    d[0] = B.RownormGradDesc(wd.data_ptr(), gd.data_ptr(), radius, ded.data_ptr(), dw.data_ptr(),
                             dg.data_ptr(), units, A, 0, None, 1, ld)
    st = B.lib().ds_weight_rownorm_gain_backward(d, 1, torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().ds_status_string(st)


def call_rescale(B, wd, vd, units, A, ld, after_step, radius=1.0):
    import torch
    d = (B.RescaleDesc * 1)()
    d[0] = B.RescaleDesc(wd.data_ptr(), 0 if vd is None else vd.data_ptr(), radius, units, A, 1, ld)
    fn = B.lib().ds_rescale_after_step if after_step else B.lib().ds_rescale_project
    st = fn(d, 1, torch.cuda.current_stream().cuda_stream)
    assert st == 0, B.lib().ds_status_string(st)


def run_all(B, w, g, de, v, units, ld, label, offset=0):
    """Forward, gradient and both rescale calls on stored [A, ld] matrices
    (units columns used), with every buffer starting `offset` elements into
    its allocation; checks every unit."""
    import torch
    A = w.shape[0]
    dev = "cuda:0"

    def place(a, dtype):
        flat = torch.zeros(a.size + offset + 8, dtype=dtype, device=dev)
        view = flat[offset:offset + a.size].view(a.shape)
        if dtype == torch.bfloat16:
            view.copy_(dev_bits(a))
        else:
            view.copy_(torch.from_numpy(np.ascontiguousarray(a)).to(dev))
        return view

    aligned = offset % 4 == 0
    wd, gd = place(w, torch.float32), dev_f32(g)
    rows = column_block_rows(w, units, 1)
    g64 = g
    # forward
    weff = place(np.full(w.shape, 0x40e0, dtype=np.uint16), torch.bfloat16)   # 7.0 outside
    norms = torch.empty(units, dtype=torch.float32, device=dev)
    call_forward(B, wd, gd, units, A, ld, weff, norms)
    torch.cuda.synchronize()
    got = host_bits(weff)
    assert (bf16_value(got[:, units:]) == 7.0).all(), f"{label}: values past the units"
    got_rows = column_block_rows(got, units, 1)
    n_ref, e_ref = weight_rownorm_gain([rows], [g64], [1.0])
    n = norms.cpu().numpy()
    assert contract_rel(n, n_ref[0]).all(), f"{label}: norms"
    ok = contract_bf16(got_rows, e_ref[0], zero_sign=False)
    assert ok.all(), f"{label}: W_eff beyond 1 ulp at {np.argwhere(~ok)[:4]}"
    depth = depth_col(A, 1, "fwd", units, ld) if aligned else depth_col(A, 1)
    rn, rw = admissible_rownorm(n, got_rows, rows, g64, 1.0, depth=depth)
    assert rn.ok and rw.ok, f"{label}: {rn} / {rw}"
    # gradient
    ded = place(de, torch.bfloat16)
    dw = place(np.zeros(w.shape, np.float32), torch.float32)
    dg = torch.empty(units, dtype=torch.float32, device=dev)
    call_backward(B, wd, gd, ded, units, A, ld, dw, dg)
    torch.cuda.synchronize()
    dwr = column_block_rows(dw.cpu().numpy(), units, 1)
    derows = column_block_rows(de, units, 1)
    want_dw, want_dg = weight_rownorm_gain_backward([rows], [g64], [1.0], [derows])
    tw, tg = rownorm_grad_terms(rows.astype(np.float64), g64.astype(np.float64), 1.0,
                                bf16_value(derows))
    assert contract_grad(dwr, want_dw[0], tw, "f32").all(), f"{label}: dW"
    assert contract_grad(dg.cpu().numpy(), want_dg[0], tg, "f32").all(), f"{label}: dg"
    depth = depth_col(A, 1, "bwd", units, ld) if aligned else depth_col(A, 1)
    rw_, rg = admissible_rownorm_backward(dwr, dg.cpu().numpy(), rows, g64, 1.0, derows,
                                          depth=depth)
    assert rw_.ok and rg.ok, f"{label}: {rw_} / {rg}"
    assert (dw.cpu().numpy()[:, units:] == 0).all(), f"{label}: dW past the units"
    # rescale calls
    depth = depth_col(A, 1, "rescale", units, ld) if aligned else depth_col(A, 1)
    vrows = column_block_rows(v, units, 1)
    terms = rescale_terms(rows.astype(np.float64), vrows.astype(np.float64))
    wd2, vd2 = place(w, torch.float32), place(v, torch.float32)
    call_rescale(B, wd2, vd2, units, A, ld, False)
    torch.cuda.synchronize()
    got_v = column_block_rows(vd2.cpu().numpy(), units, 1)
    assert contract_grad(got_v, rescale_project([rows], [vrows])[0], terms, "f32").all(), \
        f"{label}: project"
    assert np.array_equal(wd2.cpu().numpy(), w), f"{label}: project wrote w"
    assert np.array_equal(vd2.cpu().numpy()[:, units:], v[:, units:]), f"{label}: v past the units"
    _, rv = admissible_rescale(rows, got_v, rows, vrows, 1.0, False, depth=depth)
    assert rv.ok, f"{label}: project {rv}"
    wd2, vd2 = place(w, torch.float32), place(v, torch.float32)
    call_rescale(B, wd2, vd2, units, A, ld, True, 3.0)
    torch.cuda.synchronize()
    ws_ref, vs_ref = rescale_after_step([rows], [vrows], [3.0])
    got_w = column_block_rows(wd2.cpu().numpy(), units, 1)
    got_v = column_block_rows(vd2.cpu().numpy(), units, 1)
    assert contract_rel(got_w, ws_ref[0]).all(), f"{label}: after step w"
    assert contract_grad(got_v, vs_ref[0], terms, "f32").all(), f"{label}: after step v"
    assert np.array_equal(wd2.cpu().numpy()[:, units:], w[:, units:]), f"{label}: w past the units"
    rw2, rv2 = admissible_rescale(got_w, got_v, rows, vrows, 3.0, True, depth=depth)
    assert rw2.ok and rv2.ok, f"{label}: after step {rw2} / {rv2}"
    return rows


def make(A, units, ld, seed, scales=None):
    rng = np.random.default_rng(seed)
    w = (0.02 * rng.standard_normal((A, ld))).astype(np.float32)
    if scales is not None:
        w[:, :units] = (w[:, :units].astype(np.float64) * scales[None, :]).astype(np.float32)
    g = rng.uniform(0.5, 2.0, units).astype(np.float32)
    de = bf16_rne(rng.standard_normal((A, ld)))
    v = (1e-3 * rng.standard_normal((A, ld))).astype(np.float32)
    return w, g, de, v


# (A, units, ld): single-pass tiles up to 768 stored rows, two-pass tiles
# (same launch) beyond; ld > units leaves a gap the calls must not touch
CASES = [
    (768, 96, 96),      # single-pass, K filled; a ragged last tile (64 + 32 units)
    (700, 132, 136),    # K not filled; gap of 4
    (1, 4, 4),          # one stored row, one unit group
    (64, 200, 200),     # short; a tile of 8 units last
    (769, 16, 16),      # one stored row past the capacity: two-pass tiles
    (3072, 36, 44),     # GPT-2's MLP projection height: two-pass tiles; gap of 8
    (2000, 72, 72),     # two-pass, a stored-row count that is not a multiple of 128
    (3073, 8, 8),       # one stored row past 3,072
]


@pytest.mark.parametrize("A,units,ld", CASES)
def test_single_pass_layouts(B, A, units, ld):
    announce("colblock single pass", A, units, ld,
             [single_pass_lanes(A, units, 1, op, ld) for op in ("fwd", "bwd", "rescale")])
    w, g, de, v = make(A, units, ld, 2100 + A + units)
    run_all(B, w, g, de, v, units, ld, f"{A}x{units} ld {ld}")


@pytest.mark.parametrize("A,units,ld,offset", [(768, 96, 96, 1), (768, 96, 96, 2),
                                               (300, 30, 30, 0), (300, 32, 34, 0)])
def test_fallback_layouts(B, A, units, ld, offset):
    """A misaligned buffer, a unit count or an ld not a multiple of 4: the
    two-pass kernel runs, to the same contract."""
    announce("colblock fallback", A, units, ld, offset)
    w, g, de, v = make(A, units, ld, 2200 + A + units + offset)
    run_all(B, w, g, de, v, units, ld, f"{A}x{units} ld {ld} +{offset}", offset)


@pytest.mark.parametrize("A", [768, 3072])
def test_rescue_units(B, A):
    """Units out of fp32's comfortable range (rescued), a zero unit, a unit
    holding an infinity, next to ordinary units in the same tiles."""
    units = 40
    scales = np.ones(units)
    scales[[1, 2, 3, 4, 5, 9]] = [0.0, 2.0 ** 100, 2.0 ** -120, 2.0 ** -140, 2.0 ** 60, 1.0]
    announce("colblock single pass rescue", A, units)
    w, g, de, v = make(A, units, units, 2300 + A, scales)
    rows = run_all(B, w, g, de, v, units, units, f"rescue {A}")
    # the zero unit: the rescale calls leave it (and its v) as they are
    assert (rows[1] == 0).all()
    import torch
    wi = w.copy()
    wi[3, 9] = np.inf                                  # unit 9 holds an infinity
    wd, gd = dev_f32(wi), dev_f32(g)
    weff = torch.empty(wi.shape, dtype=torch.bfloat16, device="cuda:0")
    norms = torch.empty(units, dtype=torch.float32, device="cuda:0")
    call_forward(B, wd, gd, units, A, units, weff, norms)
    torch.cuda.synchronize()
    got = bf16_value(column_block_rows(host_bits(weff), units, 1))
    assert np.isnan(got[9]).any() and np.isfinite(got[np.arange(units) != 9]).all()
    n_ref, e_ref = weight_rownorm_gain([column_block_rows(w, units, 1)[np.arange(units) != 9]],
                                       [g[np.arange(units) != 9]], [1.0])
    ok = contract_bf16(host_bits(weff)[:, np.arange(units) != 9].T, e_ref[0], zero_sign=False)
    assert ok.all(), "units beside the infinity"


def test_ragged_mix_equals_single(B):
    """Single-pass and two-pass tiles of the seg-1 kernel in one call (short
    and tall matrices): each matrix's outputs equal a call of it alone."""
    import torch
    shapes = [(3072, 64), (768, 128), (700, 132), (769, 16)]
    rng = np.random.default_rng(2500)
    ws = [(0.02 * rng.standard_normal(s)).astype(np.float32) for s in shapes]
    gs = [rng.uniform(0.5, 2, s[1]).astype(np.float32) for s in shapes]
    des = [bf16_rne(rng.standard_normal(s)) for s in shapes]
    segs = [1] * len(shapes)
    announce("colblock seg-1 ragged mix", shapes)

    def fwd(idx):
        n, e = B.ds_weight_rownorm_gain([dev_f32(ws[i]) for i in idx], [dev_f32(gs[i]) for i in idx],
                                        [1.0] * len(idx), segs=[1] * len(idx))
        d, g = B.ds_weight_rownorm_gain_backward([dev_f32(ws[i]) for i in idx],
                                                 [dev_f32(gs[i]) for i in idx],
                                                 [dev_bits(des[i]) for i in idx], [1.0] * len(idx),
                                                 segs=[1] * len(idx))
        torch.cuda.synchronize()
        return ([x.cpu().numpy() for x in n], [host_bits(x) for x in e],
                [x.cpu().numpy() for x in d], [x.cpu().numpy() for x in g])

    allr = fwd(list(range(len(shapes))))
    for i in range(len(shapes)):
        one = fwd([i])
        for k in range(4):
            assert np.array_equal(one[k][0].view(np.uint8), allr[k][i].view(np.uint8)), (i, k)


def test_zero_unit_kept_by_rescale(B):
    """The rescale calls leave a zero unit's w and v bits as they are (the
    single-pass kernel writes them back)."""
    import torch
    A, units = 768, 64
    w, g, de, v = make(A, units, units, 2400)
    w[:, 5] = 0.0
    w[:, 6] = -0.0
    v[:, 6] = np.float32(np.nan)
    for after in (False, True):
        wd, vd = dev_f32(w), dev_f32(v)
        call_rescale(B, wd, vd, units, A, units, after, 2.0)
        torch.cuda.synchronize()
        gw, gv = wd.cpu().numpy(), vd.cpu().numpy()
        for u in (5, 6):
            assert np.array_equal(gw[:, u].view(np.uint32), w[:, u].view(np.uint32)), (after, u)
            assert np.array_equal(gv[:, u].view(np.uint32), v[:, u].view(np.uint32)), (after, u)
