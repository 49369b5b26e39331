"""ds_slerp_rows on the GPU against the CPU oracle (contract + strict set)."""
import numpy as np
import pytest

from gpu_util import announce, depth_for, dev_bits, dev_f32, host_bits, sample_rows, unit_norm_ok
from oracle.bf16 import bf16_rne, bf16_value
from oracle.check import admissible_slerp_rows, contract_bf16, slerp_unique_mask
from oracle.rows import l2_rows as l2_ref
from oracle.rows import slerp_rows as slerp_ref
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


def run(B, res, out, alpha, eps=1e-6):
    import torch
    h = B.ds_slerp_rows(dev_bits(res), dev_bits(out), dev_f32(alpha), eps)
    torch.cuda.synchronize()
    return host_bits(h)


def full_check(got, res, out, alpha, eps, label):
    """1-ulp contract where a and b are unique; the admissible set everywhere.

    Where a_j or b_j is at a near-tie both bf16 values are correct and the
    lerp may amplify the difference, so h_j is not unique there.
    """
    want = slerp_ref(res, out, alpha, eps)
    ok = contract_bf16(got, want)
    depth = depth_for(np.shape(res)[-1])
    uniq = slerp_unique_mask(res, out, eps, depth)
    bad = ~ok & uniq
    assert not bad.any(), f"{label}: {np.count_nonzero(bad)} beyond 1 ulp, first {np.argwhere(bad)[:5]}"
    assert uniq.mean() > 0.97, f"{label}: too few unique elements ({uniq.mean():.4f})"
    rep = admissible_slerp_rows(got, res, out, alpha, eps, depth)
    assert rep.ok, f"{label}: {rep}"


@pytest.mark.parametrize("cols", [8, 64, 520, 1024, 1032, 2056, 4096, 4104, 7168, 8192, 8200,
                                  16392, 32776, 65536])
def test_small_shapes(B, cols):
    rows = 29 if cols <= 8192 else 4
    c = inputs.slerp_case(rows, cols, 700 + cols % 89)
    announce("slerp_rows small", rows, cols)
    full_check(run(B, c.res, c.out, c.alpha), c.res, c.out, c.alpha, 1e-6, f"{rows}x{cols}")


@pytest.mark.parametrize("name", ["slerp_rows_8192x4096", "slerp_rows_8192x7168"])
def test_workloads(B, name):
    import torch
    c = inputs.make(name)
    announce("slerp_rows full size", name)
    rd, od, ad = dev_bits(c.res), dev_bits(c.out), dev_f32(c.alpha)
    h = B.ds_slerp_rows(rd, od, ad, c.eps)
    h2 = B.ds_slerp_rows(rd, od, ad, c.eps)
    hn = B.ds_slerp_rows(rd, od, -ad, c.eps)           # only |alpha| enters
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16))
    assert torch.equal(h.view(torch.int16), hn.view(torch.int16))
    assert unit_norm_ok(h)
    idx = sample_rows(c.rows, 400, 9)
    full_check(host_bits(h)[idx], c.res[idx], c.out[idx], c.alpha, c.eps, name)
    a, b = 5000, 5300
    hs = B.ds_slerp_rows(rd[a:b].contiguous(), od[a:b].contiguous(), ad, c.eps)
    torch.cuda.synchronize()
    assert torch.equal(hs.view(torch.int16), h[a:b].view(torch.int16))


def test_more_rows_than_one_launch(B, monkeypatch):
    """A call with more row groups than one launch takes runs as several
    launches (DS_ROWS_TEST_MAX_GROUPS lowers the cap of 64 workgroups per
    compute unit so small calls take that path): the bits equal one
    launch's, and rows on both sides of each seam meet the oracle."""
    import torch
    c = inputs.slerp_case(300, 4096, 7171)              # one row per workgroup
    rd, od, ad = dev_bits(c.res), dev_bits(c.out), dev_f32(c.alpha)
    announce("slerp_rows in one launch and in pieces of 64 rows", 300, 4096)
    one = B.ds_slerp_rows(rd, od, ad, c.eps)
    monkeypatch.setenv("DS_ROWS_TEST_MAX_GROUPS", "64")
    pieces = B.ds_slerp_rows(rd, od, ad, c.eps)
    small = inputs.slerp_case(301, 1024, 7172)         # four rows per workgroup
    one_s = B.ds_slerp_rows(dev_bits(small.res), dev_bits(small.out), dev_f32(small.alpha), small.eps)
    monkeypatch.delenv("DS_ROWS_TEST_MAX_GROUPS")
    one_s2 = B.ds_slerp_rows(dev_bits(small.res), dev_bits(small.out), dev_f32(small.alpha), small.eps)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int16), pieces.view(torch.int16))
    assert torch.equal(one_s.view(torch.int16), one_s2.view(torch.int16))
    idx = np.r_[0, 62:66, 126:130, 254:258, 298:300]
    full_check(host_bits(pieces)[idx], c.res[idx], c.out[idx], c.alpha, c.eps, "pieces")
    full_check(host_bits(one_s), small.res, small.out, small.alpha, small.eps, "pieces, 1024")


def test_alpha_special_cases(B):
    """alpha = 0 (h = l2(a)), alpha = 1 (h = l2(b)), res == out (h = l2(a))."""
    c = inputs.slerp_case(40, 4096, 701)
    announce("slerp_rows alpha 0 / 1 / res==out")
    zeros = np.zeros(c.cols, np.float32)
    ones = np.ones(c.cols, np.float32)
    wild = np.random.default_rng(1).uniform(-3, 3, c.cols).astype(np.float32)
    for res, out, alpha, label in ((c.res, c.out, zeros, "alpha 0"), (c.res, c.out, ones, "alpha 1"),
                                   (c.res, c.res, wild, "res == out")):
        full_check(run(B, res, out, alpha), res, out, alpha, 1e-6, label)
    # the oracle's identity, on the same inputs
    assert np.array_equal(slerp_ref(c.res, c.out, zeros), l2_ref(l2_ref(c.res), None))


def test_in_place_and_nonfinite(B):
    import torch
    c = inputs.slerp_case(64, 2048, 702)
    rd, od = dev_bits(c.res), dev_bits(c.out)
    announce("slerp_rows in place h=res")
    B.ds_slerp_rows(rd, od, dev_f32(c.alpha), 1e-6, h=rd)
    torch.cuda.synchronize()
    full_check(host_bits(rd), c.res, c.out, c.alpha, 1e-6, "in place")
    res, out, alpha = c.res.copy(), c.out.copy(), c.alpha.copy()
    res[0, 5] = 0x7F80
    out[1, 7] = 0x7FC0
    alpha[11] = np.inf
    announce("slerp_rows non-finite")
    got = run(B, res, out, alpha)
    w = bf16_value(slerp_ref(res, out, alpha))
    g = bf16_value(got)
    assert np.array_equal(np.isnan(g), np.isnan(w))
    assert np.array_equal(g[~np.isnan(g)], w[~np.isnan(w)])


def test_extreme_alpha_rescaled(B):
    """|alpha| large enough that the fp32 sum of u^2 overflows: rescaled."""
    c = inputs.slerp_case(8, 1024, 703)
    alpha = np.full(c.cols, 3.0e37, np.float32)
    announce("slerp_rows huge alpha")
    full_check(run(B, c.res, c.out, alpha), c.res, c.out, alpha, 1e-6, "huge alpha")


def test_zero_rows_tiny_eps(B):
    """All-zero res/out rows with eps far below 2^-96 (down to fp32
    subnormals): the inverse lengths come from eps alone, after rescaling."""
    c = inputs.slerp_case(6, 512, 704)
    res, out = c.res.copy(), c.out.copy()
    res[0] = 0
    out[1] = 0
    res[2] = 0
    out[2] = 0
    for eps in (2.0 ** -100, 2.0 ** -140, 1e-6):
        announce("slerp_rows zero rows eps", eps)
        full_check(run(B, res, out, c.alpha, eps), res, out, c.alpha, eps, f"eps={eps}")
