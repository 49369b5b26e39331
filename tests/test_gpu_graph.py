"""The entry points inside a captured HIP graph: every replay matches eager calls.

Between replays the test writes new inputs eagerly and synchronises, then
compares each replay's outputs bit for bit with the same library calls made
eagerly on the same inputs.  A ragged weight call that would need the staged
descriptor table (more than 48 matrices of one width) refuses to be captured.
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


def test_staged_ragged_call_refuses_capture(B):
    import torch
    dev = "cuda:0"
    case = inputs.rownorm_case([(8, 256)] * 50, 902)
    ws = [torch.from_numpy(m).to(dev) for m in case.w]
    gs = [torch.from_numpy(v).to(dev) for v in case.gain]
    ns = [torch.empty(m.shape[0], device=dev) for m in ws]
    es = [torch.empty(m.shape, dtype=torch.bfloat16, device=dev) for m in ws]
    B.ds_weight_rownorm_gain(ws, gs, norm_out=ns, w_eff=es)     # eager: fine
    torch.cuda.synchronize()
    announce("graph capture refusal: 50 matrices of one width")
    graph = torch.cuda.CUDAGraph()
    with pytest.raises(RuntimeError, match="DS_ERR_CAPTURE"):
        with torch.cuda.graph(graph):
            B.ds_weight_rownorm_gain(ws, gs, norm_out=ns, w_eff=es)
    torch.cuda.synchronize()
    # the library and the device still work
    n2, e2 = B.ds_weight_rownorm_gain(ws, gs)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(ns, n2))
