"""Every output element of every full-size workload against the oracle.

Each workload runs on the GPU once, in the launch configuration the benchmark
times (one call over all its rows), and every element of the result is then
checked on the CPU, in chunks of rows spread over worker processes
(``fullsize_jobs``):

* the contract: one bf16 ulp at the oracle value's binade for bf16 outputs,
  2e-6 relative for fp32 row lengths (for the gradients, the gradient
  contract: one ulp or 2e-6 plus 2^-16 of the size of the cancelling terms);
  for slerp, q/k and the activation rows it applies where the admissible set
  has one value (an intermediate at a near-tie may round either way, and both
  roundings are correct);
* the strict admissible set (the float64 value at the bf16 rounding points
  as a range over an fp32 run's spread, the method of TensorFold PR #1260's
  kernel-contract check), on every element, with the kernels' sum-tree depth.

Each test prints its counts (elements, bits differing from the oracle's
rounding, the largest distance in bf16 steps, near-ties, and for slerp the
elements whose a or b may round either way) and, when DS_FULLSIZE_REPORT
names a file, appends them to it as JSON lines.
"""
import json
import os
import time

import numpy as np
import pytest

import fullsize_jobs as J
from gpu_util import KERNEL_DEPTH, announce, depth_for, dev_bits, dev_f32, host_bits
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


def report(name, counts, t0):
    counts = dict(counts)
    counts["workload"] = name
    counts["seconds"] = round(time.perf_counter() - t0, 1)
    counts["workers"] = J.workers()
    line = json.dumps(counts)
    print("[fullsize]", line, flush=True)
    path = os.environ.get("DS_FULLSIZE_REPORT")
    if path:
        with open(path, "a") as f:
            f.write(line + "\n")
    return counts


def assert_clean(name, c):
    assert c["beyond"] == 0, f"{name}: {c['beyond']} elements beyond the contract, e.g. {c['first_bad']}"
    assert c["outside"] == 0, f"{name}: {c['outside']} elements outside the admissible set, e.g. {c['first_bad']}"


def l2_workload(B, c, name, r, mean=False):
    import torch
    t0 = time.perf_counter()
    announce("full-size l2", name, c.rows, c.cols, "r" if r is not None else "r=NULL")
    xd = dev_bits(c.x)
    rd = None if r is None else dev_bits(r)
    fn = B.ds_rms_rows if mean else B.ds_l2_rows
    y = fn(xd, rd, c.eps)
    torch.cuda.synchronize()
    got = host_bits(y)
    del xd, rd, y
    depth = depth_for(c.cols)
    jobs = [(got[a:b], c.x[a:b], None if r is None else r[a:b], c.eps, depth, a, mean)
            for a, b in J.chunks(c.rows)]
    counts = report(name, J.merge(J.run_pool(J.l2_job, jobs)), t0)
    assert counts["n"] == c.rows * c.cols
    assert_clean(name, counts)
    return counts


def test_l2_64x1024(B):
    c = inputs.make("l2_rows_64x1024")
    l2_workload(B, c, c.name, c.r)


def test_l2_res_8192x4096(B):
    c = inputs.make("l2_rows_res_8192x4096")
    l2_workload(B, c, c.name, c.r)


@pytest.fixture(scope="module")
def stress():
    return inputs.make("l2_rows_res_stress_32768x8192")


def test_l2_stress_32768x8192(B, stress):
    counts = l2_workload(B, stress, stress.name, stress.r)
    # the zero rows (eps path) and the integer rows are inside the workload;
    # every element counted
    assert counts["n"] == 32768 * 8192


def test_l2_stress_32768x8192_no_residual(B, stress):
    l2_workload(B, stress, stress.name + "_r_null", None)


@pytest.mark.parametrize("name", ["slerp_rows_8192x4096", "slerp_rows_8192x7168"])
def test_slerp(B, name):
    import torch
    c = inputs.make(name)
    t0 = time.perf_counter()
    announce("full-size slerp", name)
    h = B.ds_slerp_rows(dev_bits(c.res), dev_bits(c.out), dev_f32(c.alpha), c.eps)
    torch.cuda.synchronize()
    got = host_bits(h)
    del h
    depth = depth_for(c.cols)
    jobs = [(got[a:b], c.res[a:b], c.out[a:b], c.alpha, c.eps, depth, a)
            for a, b in J.chunks(c.rows)]
    counts = report(name, J.merge(J.run_pool(J.slerp_job, jobs)), t0)
    assert counts["n"] == c.rows * c.cols
    assert_clean(name, counts)
    # a or b at a near-tie: both roundings are correct; such elements stay rare
    assert counts["nonunique"] <= 0.03 * counts["n"]


def test_rownorm_12x4_d768(B):
    import torch
    case = inputs.make("rownorm_gain_12x4_d768")
    t0 = time.perf_counter()
    announce("full-size rownorm", case.name, len(case.w), case.total_rows)
    norms, weffs = B.ds_weight_rownorm_gain([dev_f32(w) for w in case.w],
                                            [dev_f32(g) for g in case.gain], case.radius)
    torch.cuda.synchronize()
    got_n = [n.cpu().numpy() for n in norms]
    got_w = [host_bits(w) for w in weffs]
    jobs = []
    for i, (w, g) in enumerate(zip(case.w, case.gain)):
        depth = depth_for(w.shape[1])
        for a, b in J.chunks(w.shape[0]):
            jobs.append((got_n[i][a:b], got_w[i][a:b], w[a:b], g[a:b], case.radius[i], depth, a))
    counts = report(case.name, J.merge(J.run_pool(J.rownorm_job, jobs)), t0)
    assert counts["n"] == case.total_elems and counts["norms"] == case.total_rows
    assert counts["norms_beyond"] == 0
    assert_clean(case.name, counts)


def test_qk_8192_h16x4_d256(B):
    import torch
    c = inputs.make("qk_rows_l2_8192_h16x4_d256")
    t0 = time.perf_counter()
    announce("full-size qk", c.name)
    d = torch.device("cuda:0")
    qo, ko = B.ds_qk_rows_l2(dev_bits(c.q), dev_bits(c.k),
                             torch.from_numpy(c.pos.astype(np.int32)).to(d),
                             torch.from_numpy(c.inv_freq).to(d), torch.from_numpy(c.q_scale).to(d),
                             c.head_dim, c.eps)
    torch.cuda.synchronize()
    gq, gk = host_bits(qo), host_bits(ko)
    rows = c.q.shape[0]
    jobs = [(gq[a:b], gk[a:b], c.q[a:b], c.k[a:b], c.pos[a:b], c.inv_freq, c.q_scale,
             c.head_dim, c.eps, 16, a) for a, b in J.chunks(rows, 256)]
    counts = report(c.name, J.merge(J.run_pool(J.qk_job, jobs)), t0)
    assert counts["n"] == rows * (c.q.shape[1] + c.k.shape[1])
    assert_clean(c.name, counts)


@pytest.mark.parametrize("name", ["gate_l2_rows_8192x4096", "swiglu_l2_rows_8192x7168"])
def test_activation_rows(B, name):
    import torch
    c = inputs.make(name)
    t0 = time.perf_counter()
    announce("full-size activation rows", name)
    kind = "gate" if name.startswith("gate") else "swiglu"
    if kind == "gate":
        y = B.ds_gate_l2_rows(dev_bits(c.a), dev_bits(c.b), dev_f32(c.s0), c.eps)
    else:
        y = B.ds_swiglu_l2_rows(dev_bits(c.a), dev_bits(c.b), dev_f32(c.s0), dev_f32(c.s1), c.eps)
    torch.cuda.synchronize()
    got = host_bits(y)
    rows, cols = got.shape
    jobs = [(kind, got[a:b], c.a[a:b], c.b[a:b], c.s0, c.s1, c.eps, depth_for(cols), a)
            for a, b in J.chunks(rows)]
    counts = report(name, J.merge(J.run_pool(J.act_job, jobs)), t0)
    assert counts["n"] == rows * cols
    assert_clean(name, counts)


@pytest.mark.parametrize("name", ["l2_rows_res_bwd_8192x4096", "rms_rows_bwd_16384x768"])
def test_l2_backward(B, name):
    import torch
    c = inputs.make(name)
    mean = name.startswith("rms")
    t0 = time.perf_counter()
    announce("full-size gradient", name)
    fn = B.ds_rms_rows_backward if mean else B.ds_l2_rows_backward
    dx = fn(dev_bits(c.x), None if c.r is None else dev_bits(c.r), dev_bits(c.dy), c.eps)
    torch.cuda.synchronize()
    got = host_bits(dx)
    rows, cols = got.shape
    jobs = [(got[a:b], c.x[a:b], None if c.r is None else c.r[a:b], c.dy[a:b], c.eps,
             min(depth_for(cols), KERNEL_DEPTH), a, mean) for a, b in J.chunks(rows)]
    counts = report(name, J.merge(J.run_pool(J.l2_backward_job, jobs)), t0)
    assert counts["n"] == rows * cols
    assert_clean(name, counts)


def test_rownorm_backward_12x4_d768(B):
    import torch
    case = inputs.make("rownorm_gain_bwd_12x4_d768")
    t0 = time.perf_counter()
    announce("full-size weight gradient", case.name)
    dws, dgs = B.ds_weight_rownorm_gain_backward([dev_f32(w) for w in case.w],
                                                 [dev_f32(g) for g in case.gain],
                                                 [dev_bits(d) for d in case.dwe], case.radius)
    torch.cuda.synchronize()
    dws = [d.cpu().numpy() for d in dws]
    dgs = [d.cpu().numpy() for d in dgs]
    jobs = []
    for i, (w, g, de) in enumerate(zip(case.w, case.gain, case.dwe)):
        depth = depth_for(w.shape[1])
        for a, b in J.chunks(w.shape[0]):
            jobs.append((dws[i][a:b], dgs[i][a:b], w[a:b], g[a:b], case.radius[i], de[a:b],
                         depth, a))
    counts = report(case.name, J.merge(J.run_pool(J.rownorm_backward_job, jobs)), t0)
    assert counts["n"] == case.total_elems and counts["dg"] == case.total_rows
    assert counts["dg_beyond"] == 0
    assert_clean(case.name, counts)


# ---------------------------------------------------- the other workloads


def test_rms_rows_16384x768(B):
    g = inputs.make("rms_rows_bwd_16384x768")        # its x: the forward's input
    c = inputs.L2Case("rms_rows_16384x768", g.x, None, g.eps)
    l2_workload(B, c, c.name, None, mean=True)


def _weights_forward(B, name, case, depth_of=None):
    import torch
    t0 = time.perf_counter()
    announce("full-size weights", name, len(case.w))
    norms, weffs = B.ds_weight_rownorm_gain([dev_f32(w) for w in case.w],
                                            [dev_f32(g) for g in case.gain], case.radius)
    torch.cuda.synchronize()
    got_n = [n.cpu().numpy() for n in norms]
    got_w = [host_bits(w) for w in weffs]
    jobs = []
    for i, (w, g) in enumerate(zip(case.w, case.gain)):
        depth = depth_for(w.shape[1])
        for a, b in J.chunks(w.shape[0]):
            jobs.append((got_n[i][a:b], got_w[i][a:b], w[a:b], g[a:b], case.radius[i], depth, a))
    counts = report(name, J.merge(J.run_pool(J.rownorm_job, jobs)), t0)
    assert counts["n"] == case.total_elems and counts["norms"] == case.total_rows
    assert counts["norms_beyond"] == 0
    assert_clean(name, counts)


def _weights_backward(B, name, case):
    import torch
    t0 = time.perf_counter()
    announce("full-size weight gradient", name, len(case.w))
    dws, dgs = B.ds_weight_rownorm_gain_backward([dev_f32(w) for w in case.w],
                                                 [dev_f32(g) for g in case.gain],
                                                 [dev_bits(d) for d in case.dwe], case.radius)
    torch.cuda.synchronize()
    dws = [d.cpu().numpy() for d in dws]
    dgs = [d.cpu().numpy() for d in dgs]
    jobs = []
    for i, (w, g, de) in enumerate(zip(case.w, case.gain, case.dwe)):
        depth = depth_for(w.shape[1])
        for a, b in J.chunks(w.shape[0]):
            jobs.append((dws[i][a:b], dgs[i][a:b], w[a:b], g[a:b], case.radius[i], de[a:b],
                         depth, a))
    counts = report(name, J.merge(J.run_pool(J.rownorm_backward_job, jobs)), t0)
    assert counts["n"] == case.total_elems and counts["dg"] == case.total_rows
    assert counts["dg_beyond"] == 0
    assert_clean(name, counts)


@pytest.mark.parametrize("name", ["rownorm_gain_resnet50", "rownorm_gain_embedding_50304x768"])
def test_weights_forward(B, name):
    _weights_forward(B, name, inputs.make(name))


def test_weights_11008x4096(B):
    case = inputs.make("rownorm_gain_bwd_11008x4096")
    _weights_forward(B, "rownorm_gain_11008x4096", case)
    _weights_backward(B, case.name, case)


def test_weights_backward_resnet50(B):
    _weights_backward(B, "rownorm_gain_bwd_resnet50", inputs.make("rownorm_gain_bwd_resnet50"))


def test_gpt2_conv1d_column_blocks(B):
    """GPT-2's 48 Conv1D weights stored [in, out]: every unit (a stored column)
    gathered into a row, forward and gradient, at the sum-tree depth of the
    column-block kernel that runs (single-pass for these layouts)."""
    import torch
    from oracle.rows import column_block_rows
    from test_gpu_colblock import depth_col
    c = inputs.make("rownorm_gain_gpt2_conv1d")
    t0 = time.perf_counter()
    announce("full-size column blocks", c.name, len(c.w))
    segs = [1] * len(c.w)
    norms, weffs = B.ds_weight_rownorm_gain([dev_f32(w) for w in c.w],
                                            [dev_f32(g) for g in c.gain], [1.0] * len(c.w),
                                            segs=segs)
    dws, dgs = B.ds_weight_rownorm_gain_backward([dev_f32(w) for w in c.w],
                                                 [dev_f32(g) for g in c.gain],
                                                 [dev_bits(d) for d in c.dwe], [1.0] * len(c.w),
                                                 segs=segs)
    torch.cuda.synchronize()
    rows = lambda a: column_block_rows(a, a.shape[1], 1)
    fwd, bwd = [], []
    for i, (w, g, de) in enumerate(zip(c.w, c.gain, c.dwe)):
        wr, er = rows(w), rows(host_bits(weffs[i]))
        dwr, der = rows(dws[i].cpu().numpy()), rows(de)
        n, dg = norms[i].cpu().numpy(), dgs[i].cpu().numpy()
        depth_f = depth_col(w.shape[0], 1, "fwd", w.shape[1])
        depth_b = depth_col(w.shape[0], 1, "bwd", w.shape[1])
        for a, b in J.chunks(wr.shape[0]):
            fwd.append((n[a:b], er[a:b], wr[a:b], g[a:b], 1.0, depth_f, a))
            bwd.append((dwr[a:b], dg[a:b], wr[a:b], g[a:b], 1.0, der[a:b], depth_b, a))
    cf = report(c.name, J.merge(J.run_pool(J.rownorm_job, fwd)), t0)
    cb = report(c.name + "_bwd", J.merge(J.run_pool(J.rownorm_backward_job, bwd)), t0)
    el = sum(w.size for w in c.w)
    assert cf["n"] == el and cb["n"] == el
    assert cf["norms_beyond"] == 0 and cb["dg_beyond"] == 0
    assert_clean(c.name, cf)
    assert_clean(c.name + " gradient", cb)


@pytest.mark.parametrize("after_step", [False, True])
def test_rescale_12x4_d768(B, after_step):
    import torch
    case = inputs.make("rescale_12x4_d768")
    name = case.name + ("_after_step" if after_step else "_project")
    t0 = time.perf_counter()
    announce("full-size rescale", name)
    ws = [dev_f32(w) for w in case.w]
    vs = [dev_f32(v) for v in case.v]
    if after_step:
        B.ds_rescale_after_step(ws, vs, case.radius)
    else:
        B.ds_rescale_project(ws, vs)
    torch.cuda.synchronize()
    gw = [w.cpu().numpy() for w in ws]
    gv = [v.cpu().numpy() for v in vs]
    jobs = []
    for i, (w, v) in enumerate(zip(case.w, case.v)):
        depth = depth_for(w.shape[1])
        for a, b in J.chunks(w.shape[0]):
            jobs.append((gw[i][a:b], gv[i][a:b], w[a:b], v[a:b], case.radius[i], after_step,
                         depth, a))
    counts = report(name, J.merge(J.run_pool(J.rescale_job, jobs)), t0)
    assert counts["n"] == sum(w.size for w in case.w)
    assert_clean(name, counts)
