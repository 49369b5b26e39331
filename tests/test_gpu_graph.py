"""The entry points inside a captured HIP graph: every replay matches eager calls.

Between replays the test writes new inputs eagerly and synchronises, then
compares each replay's outputs bit for bit with the same library calls made
eagerly on the same inputs.  A ragged weight call that would stage its
descriptor table (more than 48 matrices of one width) splits into launches
that carry their tables in the kernel arguments when its stream is being
captured; captured, its replays match eager calls too.
"""
import numpy as np
import pytest

from gpu_util import announce
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


def _bits(t):
    import torch
    return t.view(torch.int16)


def test_graph_replays_match_eager(B):
    import torch
    dev = "cuda:0"
    rows, cols = 512, 4096
    g0 = torch.Generator(device=dev).manual_seed(5)
    x = torch.randn(rows, cols, device=dev, generator=g0).to(torch.bfloat16)
    r = torch.randn(rows, cols, device=dev, generator=g0).to(torch.bfloat16)
    res = torch.randn(rows, cols, device=dev, generator=g0).to(torch.bfloat16)
    out = (2 * torch.randn(rows, cols, device=dev, generator=g0)).to(torch.bfloat16)
    alpha = (torch.rand(cols, device=dev, generator=g0) - 0.5) * 0.4
    case = inputs.rownorm_case([(96, 768), (32, 768), (48, 3072)], 901)
    ws = [torch.from_numpy(m).to(dev) for m in case.w]
    gs = [torch.from_numpy(v).to(dev) for v in case.gain]
    y = torch.empty_like(x)
    h = torch.empty_like(res)
    ns = [torch.empty(m.shape[0], device=dev) for m in ws]
    es = [torch.empty(m.shape, dtype=torch.bfloat16, device=dev) for m in ws]

    def step():
        B.ds_l2_rows(x, r, 1e-6, out=y)
        B.ds_slerp_rows(res, out, alpha, 1e-6, h=h)
        B.ds_weight_rownorm_gain(ws, gs, norm_out=ns, w_eff=es)

    announce("graph capture: l2 + slerp + rownorm (inline tables)")
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
        # new inputs, written eagerly, then one replay
        gen = torch.Generator(device=dev).manual_seed(100 + rep)
        x.copy_(torch.randn(rows, cols, device=dev, generator=gen).to(torch.bfloat16))
        res.copy_(torch.randn(rows, cols, device=dev, generator=gen).to(torch.bfloat16))
        alpha.copy_((torch.rand(cols, device=dev, generator=gen) - 0.5) * 0.4)
        for m in ws:
            m.mul_(1.5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ye = B.ds_l2_rows(x, r, 1e-6)
        he = B.ds_slerp_rows(res, out, alpha, 1e-6)
        ne, ee = B.ds_weight_rownorm_gain(ws, gs)
        torch.cuda.synchronize()
        assert torch.equal(_bits(y), _bits(ye)), f"replay {rep}: l2_rows"
        assert torch.equal(_bits(h), _bits(he)), f"replay {rep}: slerp_rows"
        for i in range(len(ws)):
            assert torch.equal(ns[i], ne[i]) and torch.equal(_bits(es[i]), _bits(ee[i])), \
                f"replay {rep}: rownorm {i}"


@pytest.mark.parametrize("shapes", [
    [(8, 256)] * 50,                                               # one class of 50
    # four small classes: three share a 256-thread mixed launch of 75 matrices
    [(3 + i % 7, (256, 768, 147, 3072)[i % 4]) for i in range(100)],
])
def test_staged_ragged_calls_capture(B, shapes):
    """Ragged calls whose eager form stages a table (forward, gradient and the
    two rescale calls), captured into one graph and replayed three times."""
    import torch
    dev = "cuda:0"
    case = inputs.rownorm_grad_case(shapes, 902)
    v0 = inputs.rescale_case(shapes, 903).v
    ws = [torch.from_numpy(m).to(dev) for m in case.w]
    # a gain per row; in the mixed batch also one gain per matrix (its
    # gradient a sum of row shares) and no gain
    mode = [("row", "scalar", "none")[i % 3] if len(shapes) == 100 else "row"
            for i in range(len(shapes))]
    gs = [torch.from_numpy(g).to(dev) if m == "row" else
          torch.tensor(float(g[0]), device=dev) if m == "scalar" else None
          for g, m in zip(case.gain, mode)]
    des = [torch.from_numpy(d.view(np.int16)).to(dev).view(torch.bfloat16) for d in case.dwe]
    w2 = [m.clone() for m in ws]                       # the rescale calls' own rows
    vs = [torch.from_numpy(v).to(dev) for v in v0]
    ns = [torch.empty(m.shape[0], device=dev) for m in ws]
    es = [torch.empty(m.shape, dtype=torch.bfloat16, device=dev) for m in ws]
    dws = [torch.empty_like(m) for m in ws]
    dgs = [torch.empty(m.shape[0], device=dev) if md == "row" else
           torch.empty((), device=dev) if md == "scalar" else None for m, md in zip(ws, mode)]

    def step():
        B.ds_weight_rownorm_gain(ws, gs, norm_out=ns, w_eff=es)
        B.ds_weight_rownorm_gain_backward(ws, gs, des, dw=dws, dgain=dgs)
        B.ds_rescale_project(ws, vs)
        B.ds_rescale_after_step(w2, vs)

    announce("graph capture of staged ragged calls:", len(shapes), "matrices")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                         # eager, staged
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(3):
        gen = torch.Generator(device=dev).manual_seed(200 + rep)
        for m, m2 in zip(ws, w2):
            m.copy_(0.02 * torch.randn(m.shape, device=dev, generator=gen))
            m2.copy_(m)
        for v in vs:
            v.copy_(1e-3 * torch.randn(v.shape, device=dev, generator=gen))
        w_in = [m.clone() for m in ws]
        v_in = [v.clone() for v in vs]
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ne, ee = B.ds_weight_rownorm_gain(w_in, gs)
        dwe, dge = B.ds_weight_rownorm_gain_backward(w_in, gs, des)
        ve = [v.clone() for v in v_in]
        B.ds_rescale_project(w_in, ve)
        w2e = [m.clone() for m in w_in]
        B.ds_rescale_after_step(w2e, ve)
        torch.cuda.synchronize()
        for i in range(len(ws)):
            assert torch.equal(ns[i], ne[i]) and torch.equal(_bits(es[i]), _bits(ee[i])), \
                f"replay {rep}: forward {i}"
            assert torch.equal(dws[i], dwe[i]), f"replay {rep}: gradient {i}"
            assert (dgs[i] is None and dge[i] is None) or torch.equal(dgs[i], dge[i]), \
                f"replay {rep}: gain gradient {i} ({mode[i]})"
            assert torch.equal(vs[i], ve[i]) and torch.equal(w2[i], w2e[i]), \
                f"replay {rep}: rescale {i}"
