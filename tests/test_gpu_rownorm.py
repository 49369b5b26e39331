"""ds_weight_rownorm_gain on the GPU against the CPU oracle."""
import numpy as np
import pytest

from gpu_util import announce, depth_for, dev_f32, host_bits, sample_rows
from oracle.bf16 import bf16_rne, bf16_value
from oracle.check import admissible_rownorm, contract_bf16, contract_rel
from oracle.rows import weight_rownorm_gain as ref
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


def run(B, case, radius=None):
    import torch
    ws = [dev_f32(w) for w in case.w]
    gs = [dev_f32(g) for g in case.gain]
    norms, weffs = B.ds_weight_rownorm_gain(ws, gs, radius or case.radius)
    torch.cuda.synchronize()
    return [n.cpu().numpy() for n in norms], [host_bits(w) for w in weffs]


def check_matrix(n_got, w_got, w, g, rho, rows, label):
    n_ref, w_ref = ref([w[rows]], [g[rows]], [rho])
    okn = contract_rel(n_got[rows], n_ref[0])
    assert okn.all(), f"{label}: norms beyond 2e-6: {np.argwhere(~okn)[:5]}"
    okw = contract_bf16(w_got[rows], w_ref[0], zero_sign=False)
    assert okw.all(), f"{label}: W_eff beyond 1 ulp: {np.count_nonzero(~okw)}"
    rn, rw = admissible_rownorm(n_got[rows], w_got[rows], w[rows], g[rows], rho,
                                depth=depth_for(w.shape[1]))
    assert rn.ok and rw.ok, f"{label}: {rn} / {rw}"


@pytest.mark.parametrize("cols", [4, 8, 44, 768, 1028, 3072, 4096, 5000, 12288, 65536])
def test_single_matrix_shapes(B, cols):
    rows = 33 if cols <= 4096 else 5
    case = inputs.rownorm_case([(rows, cols)], 800 + cols % 83)
    announce("rownorm single", rows, cols)
    n, w = run(B, case)
    check_matrix(n[0], w[0], case.w[0], case.gain[0], 1.0, np.arange(rows), f"{rows}x{cols}")


def test_transformer_workload(B):
    case = inputs.make("rownorm_gain_12x4_d768")
    announce("rownorm full", case.name, len(case.w), case.total_rows)
    n, w = run(B, case)
    n2, w2 = run(B, case)
    for i, (wm, gm) in enumerate(zip(case.w, case.gain)):
        assert np.array_equal(n[i], n2[i]) and np.array_equal(w[i], w2[i])
        # every row length against float64 (vectorised), sampled rows in full
        exact = np.sqrt((wm.astype(np.float64) ** 2).sum(axis=1))
        assert contract_rel(n[i], exact).all(), f"matrix {i}"
        rows = sample_rows(wm.shape[0], 24, 100 + i)
        check_matrix(n[i], w[i], wm, gm, 1.0, rows, f"matrix {i} {wm.shape}")


def test_ragged_equals_single(B):
    """A matrix's bits do not depend on the other matrices in the call."""
    case = inputs.rownorm_case([(100, 768), (7, 3072), (33, 44), (64, 768)], 810)
    announce("rownorm ragged vs single")
    n_all, w_all = run(B, case)
    for i in range(len(case.w)):
        one = inputs.RownormCase("one", [case.w[i]], [case.gain[i]], [case.radius[i]])
        n1, w1 = run(B, one)
        assert np.array_equal(n1[0], n_all[i]) and np.array_equal(w1[0], w_all[i])
    rev = inputs.RownormCase("rev", case.w[::-1], case.gain[::-1], case.radius[::-1])
    n_r, w_r = run(B, rev)
    for i in range(len(case.w)):
        assert np.array_equal(w_r[len(case.w) - 1 - i], w_all[i])


def test_grid_stride_equals_one_item_each(B, monkeypatch):
    """With the per-launch cap of 64 workgroups per compute unit lowered
    (the DS_ROWS_TEST_MAX_GROUPS hook) the ragged kernels' grid-stride loops run
    several items per workgroup: forward, gradient and both rescale calls
    give the bits of one item per workgroup, over every launch kind (a large
    class of its own, mixed small classes, single-element rows, column
    blocks)."""
    import torch
    shapes = [(900, 768), (37, 3072), (33, 44), (64, 147), (300, 4096)]
    c = inputs.rownorm_grad_case(shapes, 811)
    cb = inputs.colblock_grad_case([(96, 320), (12, 90)], 1, 812)
    announce("weights on a grid of 7 workgroups against one item each")

    def calls():
        ws = [dev_f32(w) for w in c.w] + [dev_f32(w) for w in cb.w]
        gs = [dev_f32(g) for g in c.gain] + [dev_f32(g) for g in cb.gain]
        des = [torch.from_numpy(np.ascontiguousarray(d).view(np.int16)).to("cuda:0").view(torch.bfloat16)
               for d in c.dwe + cb.dwe]
        segs = [None] * len(c.w) + [1] * len(cb.w)
        n, e = B.ds_weight_rownorm_gain(ws, gs, None, segs=segs)
        dw, dg = B.ds_weight_rownorm_gain_backward(ws, gs, des, segs=segs)
        vs = [0.01 * torch.ones_like(w) for w in ws]
        B.ds_rescale_project(ws, vs, segs=segs)
        B.ds_rescale_after_step(ws, vs, segs=segs)
        torch.cuda.synchronize()
        return [t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)
                for t in n + e + dw + dg + vs + ws]

    one = calls()
    monkeypatch.setenv("DS_ROWS_TEST_MAX_GROUPS", "7")
    loop = calls()
    monkeypatch.delenv("DS_ROWS_TEST_MAX_GROUPS")
    assert len(one) == len(loop)
    for i, (a, b) in enumerate(zip(one, loop)):
        assert torch.equal(a, b), i


def test_step0_identity_and_radius(B):
    """g = ||W_i|| (the gain init that keeps the output) gives W_eff = bf16(W)."""
    case = inputs.rownorm_case([(256, 768)], 811)
    announce("rownorm step-0 identity")
    n, _ = run(B, case)
    same = inputs.RownormCase("id", case.w, [n[0].astype(np.float32)], [1.0])
    _, w = run(B, same)
    want = bf16_rne(case.w[0].astype(np.float64))
    ok = contract_bf16(w[0], want, zero_sign=False)
    assert ok.all()
    assert (w[0] == want).mean() > 0.999
    emb = inputs.RownormCase("emb", case.w, case.gain, [float(np.sqrt(768.0))])
    n_e, w_e = run(B, emb)
    check_matrix(n_e[0], w_e[0], case.w[0], case.gain[0], float(np.sqrt(np.float32(768.0))),
                 np.arange(256), "radius sqrt(768)")


def test_zero_tiny_huge_and_nonfinite_rows(B):
    rng = np.random.default_rng(812)
    w = (rng.standard_normal((10, 768)) * 0.02).astype(np.float32)
    w[0] = 0.0                                         # zero row -> zero row, norm 0
    w[1] *= np.float32(2.0 ** -100)                    # squares underflow: rescaled
    w[2] = (w[2] * np.float32(2.0 ** 100) * np.float32(2.0 ** 20)).astype(np.float32)  # squares overflow
    w[3, :] = 0.0
    w[3, 5] = np.float32(1.4e-45)                      # one fp32 subnormal
    w[4, 3] = np.inf
    w[5, 9] = np.nan
    g = rng.uniform(0.5, 2.0, 10).astype(np.float32)
    g[6] = 0.0
    g[7] = -1.5
    case = inputs.RownormCase("edge", [w], [g], [1.0])
    announce("rownorm edge rows")
    n, we = run(B, case)
    n_ref, w_ref = ref([w], [g], [1.0])
    finite = [0, 1, 2, 3, 6, 7, 8, 9]
    assert contract_rel(n[0][finite], n_ref[0][finite]).all()
    assert contract_bf16(we[0][finite], w_ref[0][finite], zero_sign=False).all()
    assert not bf16_value(we[0][0]).any() and n[0][0] == 0
    g4, r4 = bf16_value(we[0][4]), bf16_value(w_ref[0][4])
    assert np.array_equal(np.isnan(g4), np.isnan(r4)) and np.isinf(n[0][4])
    assert np.isnan(bf16_value(we[0][5])).all() and np.isnan(n[0][5])


def test_staged_table_many_matrices(B):
    """More than 48 matrices of one width go through the staged device table."""
    shapes = [(17 + i % 5, 768) for i in range(60)] + [(9, 256)] * 5
    case = inputs.rownorm_case(shapes, 813)
    announce("rownorm staged table", len(shapes))
    n, w = run(B, case)
    for i, (wm, gm) in enumerate(zip(case.w, case.gain)):
        check_matrix(n[i], w[i], wm, gm, 1.0, np.arange(wm.shape[0]), f"staged {i}")
    for i in (0, 31, 59, 62):
        one = inputs.RownormCase("one", [case.w[i]], [case.gain[i]], [1.0])
        n1, w1 = run(B, one)
        assert np.array_equal(n1[0], n[i]) and np.array_equal(w1[0], w[i])
