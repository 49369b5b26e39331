"""ds_qk_rows_l2 on the GPU against the CPU oracle.

Every element must lie in the strict admissible set (an fp32 run with the
device sincosf within COSF_ULPS); elements whose admissible output is a
single bf16 value must also be within 1 ulp of the oracle.  The full-size
workload is checked on sampled rows and, on every row, through unit-length
k heads.
"""
import numpy as np
import pytest

from gpu_util import announce, host_bits, sample_rows
from oracle.bf16 import bf16_rne, bf16_value
from oracle.check import admissible_qk_rows, contract_bf16
from oracle.rows import qk_rows_l2
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


def _dev(c):
    import torch
    d = torch.device("cuda:0")
    bits = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(d).view(torch.bfloat16)
    return (bits(c.q), None if c.k is None else bits(c.k), torch.from_numpy(c.pos.astype(np.int32)).to(d),
            torch.from_numpy(c.inv_freq).to(d), torch.from_numpy(c.q_scale).to(d))


def run(B, c, eps=1e-6):
    import torch
    q, k, pos, inv, sc = _dev(c)
    qo, ko = B.ds_qk_rows_l2(q, k, pos, inv, sc, c.head_dim, eps)
    torch.cuda.synchronize()
    return host_bits(qo), None if ko is None else host_bits(ko)


def check(qo, ko, c, rows, label, eps=1e-6, min_unique=0.97):
    q, k, pos = c.q[rows], None if c.k is None else c.k[rows], c.pos[rows]
    rq, rk, uq, uk = admissible_qk_rows(qo[rows], None if ko is None else ko[rows], q, k, pos,
                                        c.inv_freq, c.q_scale, c.head_dim, eps, depth=16)
    assert rq.ok and rk.ok, f"{label}: q {rq} / k {rk}"
    wq, wk = qk_rows_l2(q, k, pos, c.inv_freq, c.q_scale, c.head_dim, eps)
    for got, want, u, name in ((qo[rows], wq, uq, "q"), (None if ko is None else ko[rows], wk, uk, "k")):
        if got is None or u is None:
            continue
        bad = ~contract_bf16(got, want, zero_sign=False) & u
        assert not bad.any(), f"{label} {name}: {np.count_nonzero(bad)} beyond 1 ulp"
        assert u.mean() >= min_unique, f"{label} {name}: unique {u.mean():.4f}"


@pytest.mark.parametrize("hd", [256, 128])
@pytest.mark.parametrize("nq,nk", [(16, 4), (3, 1), (1, 0), (5, 3)])
def test_shapes(B, hd, nq, nk):
    c = inputs.qk_case(37, nq, nk, hd, 1700 + hd + nq * 7 + nk)
    announce("qk_rows_l2", hd, nq, nk)
    qo, ko = run(B, c)
    check(qo, ko, c, np.arange(37), f"hd={hd} nq={nq} nk={nk}")


def test_workload(B):
    import torch
    c = inputs.make("qk_rows_l2_8192_h16x4_d256")
    announce("qk_rows_l2 full", c.name)
    q, k, pos, inv, sc = _dev(c)
    qo, ko = B.ds_qk_rows_l2(q, k, pos, inv, sc, 256)
    qo2, ko2 = B.ds_qk_rows_l2(q, k, pos, inv, sc, 256)
    part_q, part_k = B.ds_qk_rows_l2(q[300:1400], k[300:1400], pos[300:1400], inv, sc, 256)
    torch.cuda.synchronize()
    assert torch.equal(qo.view(torch.int16), qo2.view(torch.int16))
    assert torch.equal(qo[300:1400].view(torch.int16), part_q.view(torch.int16))
    assert torch.equal(ko[300:1400].view(torch.int16), part_k.view(torch.int16))
    n = ko.float().view(8192, 4, 256).pow(2).sum(-1).sqrt()
    assert bool(((n - 1).abs() <= 2 ** -7).all().item())          # every k head unit length
    gq, gk = host_bits(qo), host_bits(ko)
    rows = sample_rows(8192, 24, 1701, must=[5460, 5461, 8191])
    check(gq, gk, c, rows, c.name)


def test_more_rows_than_one_launch(B, monkeypatch):
    """A call with more row groups than one launch takes runs as several
    launches (DS_ROWS_TEST_MAX_GROUPS lowers the cap of 64 workgroups per
    compute unit): strided views and in-place outputs move with each piece,
    the bits equal one launch's, and rows on both sides of each seam meet
    the oracle."""
    import torch
    rows = 333                                          # pieces of 2 x 50 rows
    c = inputs.qk_case(rows, 3, 2, 128, 1703)
    announce("qk_rows_l2 in pieces", rows)
    want_q, want_k = run(B, c)
    d = torch.device("cuda:0")
    fused = torch.zeros(rows, 6 * 128 + 64, dtype=torch.int16, device=d)     # q | k | v
    fused[:, :384] = torch.from_numpy(c.q.view(np.int16)).to(d)
    fused[:, 384:640] = torch.from_numpy(c.k.view(np.int16)).to(d)
    fused = fused.view(torch.bfloat16)
    _, _, pos, inv, sc = _dev(c)
    qv, kv = fused[:, :384], fused[:, 384:640]
    monkeypatch.setenv("DS_ROWS_TEST_MAX_GROUPS", "50")
    B.ds_qk_rows_l2(qv, kv, pos, inv, sc, 128, q_out=qv, k_out=kv)
    torch.cuda.synchronize()
    monkeypatch.delenv("DS_ROWS_TEST_MAX_GROUPS")
    assert np.array_equal(host_bits(qv.contiguous()), want_q)
    assert np.array_equal(host_bits(kv.contiguous()), want_k)
    assert not fused[:, 640:].view(torch.int16).any()
    check(want_q, want_k, c, np.arange(rows), "pieces")


def test_strided_views_and_in_place(B):
    """q and k as slices of one fused projection row; outputs in place."""
    import torch
    c = inputs.qk_case(64, 16, 4, 256, 1702)
    want_q, want_k = run(B, c)
    d = torch.device("cuda:0")
    qkv = torch.zeros(64, 6144, dtype=torch.int16, device=d)
    qkv[:, :4096] = torch.from_numpy(c.q.view(np.int16)).to(d)
    qkv[:, 4096:5120] = torch.from_numpy(c.k.view(np.int16)).to(d)
    qkv = qkv.view(torch.bfloat16)
    _, _, pos, inv, sc = _dev(c)
    qv, kv = qkv[:, :4096], qkv[:, 4096:5120]
    announce("qk_rows_l2 strided, in place")
    B.ds_qk_rows_l2(qv, kv, pos, inv, sc, 256, q_out=qv, k_out=kv)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(qv.contiguous()), want_q)
    assert np.array_equal(host_bits(kv.contiguous()), want_k)
    assert not qkv[:, 5120:].view(torch.int16).any()                  # v untouched


def test_extremes(B):
    rng = np.random.default_rng(1703)
    hd = 256
    q = rng.standard_normal((8, 2 * hd))
    q[0, :hd] = 0.0                                   # zero head: eps alone
    q[1, :hd] *= 2.0 ** 100                           # squares overflow fp32
    q[2, :hd] *= 2.0 ** -100                          # ... and underflow
    q[3, hd:] = rng.integers(-64, 65, hd)             # integer head
    c = inputs.QkCase("extremes", bf16_rne(q), None,
                      np.array([0, 1, -5, 2 ** 24 + 1, 7, 199_999, 1_000_000, 3], np.int32),
                      inputs.rope_inv_freq(hd), rng.uniform(0.5, 2, 2 * hd).astype(np.float32), hd)
    for eps in (1e-6, 0.0):
        keep = np.arange(8) if eps > 0 else np.arange(1, 8)
        cc = inputs.QkCase("x", c.q[keep], None, c.pos[keep], c.inv_freq, c.q_scale, hd)
        announce("qk_rows_l2 extremes eps", eps)
        qo, _ = run(B, cc, eps)
        check(qo, None, cc, np.arange(len(keep)), f"extremes eps={eps}", eps, min_unique=0.9)


def test_nonfinite(B):
    rng = np.random.default_rng(1704)
    hd = 128
    q = bf16_rne(rng.standard_normal((3, 2 * hd)))
    q[0, 5] = 0x7FC0
    q[1, hd + 3] = 0x7F80
    c = inputs.QkCase("nf", q, None, np.array([3, 4, 5], np.int32), inputs.rope_inv_freq(hd),
                      np.ones(2 * hd, np.float32), hd)
    announce("qk_rows_l2 non-finite")
    qo, _ = run(B, c)
    want, _ = qk_rows_l2(c.q, None, c.pos, c.inv_freq, c.q_scale, hd)
    g, w = bf16_value(qo), bf16_value(want)
    assert np.array_equal(np.isnan(g), np.isnan(w))
    check(qo, None, c, np.array([2]), "finite row")
