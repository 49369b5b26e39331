"""Ragged weight calls from several host threads at once, each on its own stream.

A ragged call of more than 48 matrices stages its task table through the
library's per-device ring of eight pinned-host and device slots: the table
is written into a free slot's host buffer, copied on the caller's stream, and
the slot is handed out again only after an event behind the call's launches
has completed.  The ring is shared by every thread of the process and
guarded by one mutex; this checks that threads calling at once, on streams
of their own, never see each other's tables.  Each of four threads makes
alternate forward and gradient calls over its own batch of 60 matrices
(more calls in all than the ring has slots, so slots are reused while other
threads' copies are in flight); every output must equal, bit for bit, the
same call made alone before the threads start.  The ctypes calls release the
GIL, so the library calls do run at once.
"""
import threading

import numpy as np
import pytest

from gpu_util import announce, dev_bits, dev_f32
from scale_invariant_row_amd import inputs

pytestmark = pytest.mark.gpu

THREADS = 4
ROUNDS = 6
MATRICES = 60           # more than the 48 a call carries in its kernel arguments


@pytest.fixture(scope="module")
def B():
    from scale_invariant_row_amd import binding
    binding.lib()
    return binding


def batch(seed):
    rng = np.random.default_rng(seed)
    shapes = [(int(rng.integers(1, 40)), int(rng.choice([64, 147, 768, 1028, 3072])))
              for _ in range(MATRICES)]
    c = inputs.rownorm_grad_case(shapes, seed)
    return ([dev_f32(w) for w in c.w], [dev_f32(g) for g in c.gain],
            [dev_bits(d) for d in c.dwe])


def test_threads_on_their_own_streams(B):
    import torch
    announce("concurrent staged calls", THREADS, "threads x", ROUNDS, "rounds")
    data = [batch(3200 + i) for i in range(THREADS)]
    ref = []
    for ws, gs, des in data:
        n, e = B.ds_weight_rownorm_gain(ws, gs)
        dw, dg = B.ds_weight_rownorm_gain_backward(ws, gs, des)
        torch.cuda.synchronize()
        ref.append((n, e, dw, dg))

    errors = []
    start = threading.Barrier(THREADS)

    def worker(i):
        try:
            ws, gs, des = data[i]
            n0, e0, dw0, dg0 = ref[i]
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                start.wait(timeout=60)
                for r in range(ROUNDS):
                    if r % 2 == 0:
                        n, e = B.ds_weight_rownorm_gain(ws, gs, stream=st)
                        st.synchronize()
                        for k in range(MATRICES):
                            if not (torch.equal(n[k], n0[k]) and
                                    torch.equal(e[k].view(torch.int16), e0[k].view(torch.int16))):
                                errors.append(f"thread {i} round {r}: forward matrix {k}")
                                return
                    else:
                        dw, dg = B.ds_weight_rownorm_gain_backward(ws, gs, des, stream=st)
                        st.synchronize()
                        for k in range(MATRICES):
                            if not (torch.equal(dw[k], dw0[k]) and torch.equal(dg[k], dg0[k])):
                                errors.append(f"thread {i} round {r}: gradient matrix {k}")
                                return
        except Exception as exc:            # reported below, in the main thread
            errors.append(f"thread {i}: {exc!r}")

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(THREADS)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    assert not errors, errors
