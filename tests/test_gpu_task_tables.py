"""The weight kernels' task tables at their boundaries, on the GPU.

Each workgroup of a ragged weight launch finds the matrix (task) that owns
its work item: from the table in the kernel arguments (at most 48 tasks,
read with scalar loads) or from a table staged in device memory (more than
48).  Here the same batches run with 1, 47, 48 and 49 matrices, of one width
(one kernel) and of mixed widths (a mixed-shape launch), and with the grid
held to a few workgroups per launch (the test hook DS_ROWS_TEST_MAX_GROUPS),
so that every workgroup walks many items and crosses from one matrix to the
next inside its loop.  Every output of the forward, the gradient and both
rescale calls must equal, bit for bit, the same matrix called alone on the
full grid.
"""
import os

import numpy as np
import pytest

from gpu_util import announce, dev_bits, dev_f32
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


def shapes(n, mixed, seed):
    rng = np.random.default_rng(seed)
    widths = (768, 147, 2048, 256) if mixed else (768,)
    return [(int(rng.integers(1, 30)), widths[i % len(widths)]) for i in range(n)]


def run_all(B, w, g, d, v):
    """Forward, gradient and both rescale calls over the matrices w (fp32),
    gains g, bf16 dL/dW_eff bits d and fp32 v."""
    import torch
    ws, gs, des = [dev_f32(x) for x in w], [dev_f32(x) for x in g], [dev_bits(x) for x in d]
    n, e = B.ds_weight_rownorm_gain(ws, gs)
    dw, dg = B.ds_weight_rownorm_gain_backward(ws, gs, des)
    vp = [dev_f32(x) for x in v]
    B.ds_rescale_project(ws, vp)
    w2, va = [dev_f32(x) for x in w], [dev_f32(x) for x in v]
    B.ds_rescale_after_step(w2, va)
    torch.cuda.synchronize()
    return n, e, dw, dg, vp, w2, va


@pytest.mark.parametrize("count", [1, 47, 48, 49])
@pytest.mark.parametrize("mixed", [False, True])
def test_tables_and_item_loops(B, count, mixed):
    import torch
    sh = shapes(count, mixed, 3300 + count)
    c = inputs.rownorm_grad_case(sh, 3300 + count)
    v = inputs.rescale_case(sh, 3400 + count).v
    refs = [run_all(B, [c.w[i]], [c.gain[i]], [c.dwe[i]], [v[i]]) for i in range(count)]
    announce("task tables:", count, "matrices", "mixed widths" if mixed else "one width",
             "on a grid of 3 workgroups per launch")
    old = os.environ.get("DS_ROWS_TEST_MAX_GROUPS")
    os.environ["DS_ROWS_TEST_MAX_GROUPS"] = "3"
    try:
        got = run_all(B, c.w, c.gain, c.dwe, v)
    finally:
        if old is None:
            del os.environ["DS_ROWS_TEST_MAX_GROUPS"]
        else:
            os.environ["DS_ROWS_TEST_MAX_GROUPS"] = old
    names = ("norms", "w_eff", "dW", "dg", "projected v", "rescaled w", "after-step v")
    for i in range(count):
        for name, a, b in zip(names, got, refs[i]):
            x, y = a[i], b[0]
            if x.dtype == torch.bfloat16:
                x, y = x.view(torch.int16), y.view(torch.int16)
            assert torch.equal(x, y), f"matrix {i} {sh[i]}: {name} differs from the matrix alone"
