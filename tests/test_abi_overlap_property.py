"""The ragged weight calls' overlap rule, as a property over random layouts.

Every matrix of a ragged call runs concurrently with the others, so the
library refuses (DS_ERR_ARG) a call in which any output byte range shares a
byte with another output or with any input of the call, and accepts every
other well-formed call.  Descriptors here are well formed (aligned, shaped,
non-null) and placed at random in a small fake address space; the
library's decision is compared with a direct model of the rule.  Accepted
calls stop at the device lookup, so this runs only where no HIP device
exists (the addresses are never dereferenced).
"""
import os

import pytest
from hypothesis import given, settings, strategies as st

from scale_invariant_row_amd import binding as B

pytestmark = [
    pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="library not built"),
    pytest.mark.skipif("__import__('torch').cuda.device_count() > 0",
                       reason="accepted calls would launch on fake addresses"),
]

BASE = 0x100000
SLOTS = 64            # 256-byte slots of the fake address space


def overlaps(a, b):
    return a[0] < b[1] and b[0] < a[1]


def expected(ranges_in, ranges_out):
    outs = [r for r in ranges_out if r[1] > r[0]]
    ins = [r for r in ranges_in if r[1] > r[0]]
    for i, o in enumerate(outs):
        if any(overlaps(o, p) for p in outs[i + 1:]) or any(overlaps(o, p) for p in ins):
            return B.DS_ERR_ARG
    return B.DS_ERR_DEVICE


matrix = st.tuples(st.integers(1, 4),                     # rows
                   st.sampled_from([4, 8, 12, 16, 20]),    # cols (16-byte vector path)
                   st.integers(0, SLOTS - 4),              # slot of w
                   st.integers(0, SLOTS - 4),              # slot of gain
                   st.integers(0, SLOTS - 4),              # slot of w_eff
                   st.one_of(st.none(), st.integers(0, SLOTS - 4)))   # slot of norm_out


@settings(max_examples=300, deadline=None)
@given(st.lists(matrix, min_size=1, max_size=5))
def test_forward_overlap_rule(mats):
    L = B.lib()
    descs = (B.RownormDesc * len(mats))()
    ins, outs = [], []
    for i, (rows, cols, sw, sg, se, sn) in enumerate(mats):
        w, g, e = BASE + 256 * sw, BASE + 256 * sg, BASE + 256 * se
        n = None if sn is None else BASE + 256 * sn
        descs[i] = B.RownormDesc(w, g, 1.0, n, e, rows, cols, 0, 0, 0)
        ins += [(w, w + rows * cols * 4), (g, g + rows * 4)]
        outs.append((e, e + rows * cols * 2))
        if n is not None:
            outs.append((n, n + rows * 4))
    assert L.ds_weight_rownorm_gain(descs, len(mats), None) == expected(ins, outs)


@settings(max_examples=300, deadline=None)
@given(st.lists(st.tuples(st.integers(1, 4), st.sampled_from([4, 8, 16]),
                          st.integers(0, SLOTS - 4), st.integers(0, SLOTS - 4)),
                min_size=1, max_size=5),
       st.booleans())
def test_rescale_overlap_rule(mats, after_step):
    """Project reads w and writes v; after a step both are written."""
    L = B.lib()
    descs = (B.RescaleDesc * len(mats))()
    ins, outs = [], []
    for i, (rows, cols, sw, sv) in enumerate(mats):
        w, v = BASE + 256 * sw, BASE + 256 * sv
        descs[i] = B.RescaleDesc(w, v, 1.0, rows, cols, 0, 0)
        nb = rows * cols * 4
        (outs if after_step else ins).append((w, w + nb))
        outs.append((v, v + nb))
    fn = L.ds_rescale_after_step if after_step else L.ds_rescale_project
    assert fn(descs, len(mats), None) == expected(ins, outs)


@settings(max_examples=200, deadline=None)
@given(st.lists(st.tuples(st.integers(1, 3), st.sampled_from([1, 2, 3]), st.integers(1, 3),
                          st.integers(0, SLOTS - 8), st.integers(0, SLOTS - 8)),
                min_size=1, max_size=4))
def test_column_block_spans(mats):
    """A column block's span runs from its first value to one past its last:
    (A - 1) * ld + rows * seg values; outputs use the same layout."""
    L = B.lib()
    descs = (B.RownormDesc * len(mats))()
    ins, outs = [], []
    for i, (units, seg, A, sw, se) in enumerate(mats):
        ld = units * seg + 2
        w, e = BASE + 256 * sw + 4, BASE + 256 * se + 2
        g = BASE + 256 * SLOTS + 64 * i                  # gains kept apart
        descs[i] = B.RownormDesc(w, g, 1.0, None, e, units, A * seg, 0, seg, ld)
        span = (A - 1) * ld + units * seg
        ins += [(w, w + span * 4), (g, g + units * 4)]
        outs.append((e, e + span * 2))
    assert L.ds_weight_rownorm_gain(descs, len(mats), None) == expected(ins, outs)
