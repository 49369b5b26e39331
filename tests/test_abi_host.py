"""The C ABI without a GPU: symbols, status strings and argument validation.

Every refused call returns before its first HIP call, so these run anywhere
(fake pointer values are never dereferenced).  Calls with valid arguments are
made only where no HIP device exists, where they must stop at DS_ERR_DEVICE.
"""
import ctypes
import os

import pytest

from scale_invariant_row_amd import binding as B

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH),
                                reason="library not built (python -m scale_invariant_row_amd.build)")


def no_device():
    import torch
    return torch.cuda.device_count() == 0


@pytest.fixture(scope="module")
def L():
    return B.lib()


def test_exports_every_declared_function(L):
    names = B.header_functions()
    assert set(names) == {"ds_l2_rows", "ds_slerp_rows", "ds_weight_rownorm_gain",
                          "ds_l2_rows_backward", "ds_weight_rownorm_gain_backward",
                          "ds_weight_rownorm_gain_backward_noalloc",
                          "ds_gate_l2_rows", "ds_swiglu_l2_rows", "ds_qk_rows_l2",
                          "ds_rescale_project", "ds_rescale_after_step",
                          "ds_rms_rows", "ds_rms_rows_backward",
                          "ds_status_string", "ds_version"}
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strings(L):
    assert B.ds_version() == 10900
    for code in range(0, -10, -1):
        s = B.ds_status_string(code)
        assert s.startswith("DS_"), s
    assert "unknown" in B.ds_status_string(42)


A = 0x10000          # fake, 16-byte aligned addresses; never dereferenced
Bp = 0x20000000
C = 0x40000000


NORM = ["ds_l2_rows", "ds_rms_rows"]
NORM_BWD = ["ds_l2_rows_backward", "ds_rms_rows_backward"]


@pytest.mark.parametrize("name", NORM)
@pytest.mark.parametrize("rows,cols,code", [
    (-1, 64, B.DS_ERR_SHAPE), (4, 0, B.DS_ERR_SHAPE), (4, 12, B.DS_ERR_SHAPE),
    (4, 65544, B.DS_ERR_SHAPE), (4, 4, B.DS_ERR_SHAPE), (1 << 60, 64, B.DS_ERR_SHAPE)])
def test_l2_shape(L, name, rows, cols, code):
    assert getattr(L, name)(A, None, Bp, rows, cols, 1e-6, None) == code


@pytest.mark.parametrize("name", NORM)
def test_l2_eps(L, name):
    for eps in (-1e-6, float("nan"), float("inf")):
        assert getattr(L, name)(A, None, Bp, 4, 64, eps, None) == B.DS_ERR_ARG


@pytest.mark.parametrize("name", NORM)
def test_l2_pointers(L, name):
    f = getattr(L, name)
    assert f(None, None, Bp, 4, 64, 1e-6, None) == B.DS_ERR_NULL
    assert f(A, None, None, 4, 64, 1e-6, None) == B.DS_ERR_NULL
    assert f(A + 8, None, Bp, 4, 64, 1e-6, None) == B.DS_ERR_ALIGN
    assert f(A, A + 2, Bp, 4, 64, 1e-6, None) == B.DS_ERR_ALIGN
    assert f(A, None, Bp + 4, 4, 64, 1e-6, None) == B.DS_ERR_ALIGN
    # y partly overlapping x or r
    assert f(A, None, A + 16, 4, 64, 1e-6, None) == B.DS_ERR_ARG
    assert f(A, C, C + 256, 4, 64, 1e-6, None) == B.DS_ERR_ARG


@pytest.mark.parametrize("name", NORM)
def test_l2_zero_rows_is_noop(L, name):
    assert getattr(L, name)(None, None, None, 0, 64, 1e-6, None) == B.DS_OK


@pytest.mark.skipif("not no_device()")
@pytest.mark.parametrize("name", NORM)
def test_l2_valid_args_reach_device_lookup(L, name):
    f = getattr(L, name)
    assert f(A, None, Bp, 4, 64, 1e-6, None) == B.DS_ERR_DEVICE
    assert f(A, C, A, 4, 64, 1e-6, None) == B.DS_ERR_DEVICE     # y == x is allowed
    assert L.ds_slerp_rows(A, Bp, C, A, 4, 64, 1e-6, None) == B.DS_ERR_DEVICE


def test_slerp_validation(L):
    f = L.ds_slerp_rows
    assert f(A, Bp, None, C, 4, 64, 1e-6, None) == B.DS_ERR_NULL
    assert f(A, Bp, C + 4, C + 4096, 4, 64, 1e-6, None) == B.DS_ERR_ALIGN
    assert f(A, Bp, C, C + 64, 4, 64, 1e-6, None) == B.DS_ERR_ARG     # alpha overlaps h
    assert f(A, Bp, C, A + 32, 4, 64, 1e-6, None) == B.DS_ERR_ARG     # h partly over res
    assert f(A, Bp, C, C + 4096, 4, 60, 1e-6, None) == B.DS_ERR_SHAPE
    assert f(A, Bp, C, C + 4096, 4, 64, -1.0, None) == B.DS_ERR_ARG
    assert f(None, None, None, None, 0, 64, 1e-6, None) == B.DS_OK


def _descs(*items):
    arr = (B.RownormDesc * len(items))()
    for i, d in enumerate(items):
        arr[i] = B.RownormDesc(*d)
    return arr


def test_rownorm_validation(L):
    f = L.ds_weight_rownorm_gain
    good = (A, Bp, 1.0, Bp + 4096, C, 16, 64)
    assert f(_descs(good), -1, None) == B.DS_ERR_ARG
    assert f(None, 0, None) == B.DS_OK
    assert f(None, 2, None) == B.DS_ERR_NULL
    assert f(_descs((A, Bp, 1.0, None, C, 16, 0)), 1, None) == B.DS_ERR_SHAPE
    # a width that is not a multiple of 4 takes single elements, up to 16,384
    assert f(_descs((A, Bp, 1.0, None, C, 16, 16387)), 1, None) == B.DS_ERR_SHAPE
    # ... with 4-byte fp32 and 2-byte bf16 alignment (16 on the vector path)
    assert f(_descs((A + 2, Bp, 1.0, None, C, 16, 147)), 1, None) == B.DS_ERR_ALIGN
    assert f(_descs((A + 4, Bp, 1.0, None, C + 1, 16, 147)), 1, None) == B.DS_ERR_ALIGN
    assert f(_descs((A + 4, Bp, 1.0, None, C, 16, 148)), 1, None) == B.DS_ERR_ALIGN
    assert f(_descs((A, Bp, float("inf"), None, C, 16, 64)), 1, None) == B.DS_ERR_ARG
    assert f(_descs((A, None, 1.0, None, C, 16, 64)), 1, None) == B.DS_ERR_NULL
    assert f(_descs((A + 4, Bp, 1.0, None, C, 16, 64)), 1, None) == B.DS_ERR_ALIGN
    assert f(_descs((A, Bp, 1.0, Bp + 4098, C, 16, 64)), 1, None) == B.DS_ERR_ALIGN
    assert f(_descs((A, Bp, 1.0, None, A + 64, 16, 64)), 1, None) == B.DS_ERR_ARG   # w_eff over w
    # two matrices writing the same bytes
    assert f(_descs(good, (A, Bp, 1.0, None, C + 512, 16, 64)), 2, None) == B.DS_ERR_ARG
    # a bad descriptor anywhere refuses the whole call
    assert f(_descs(good, (A, Bp, 1.0, None, C + 65536, -3, 64)), 2, None) == B.DS_ERR_SHAPE
    # zero-row descriptors are skipped, pointers unchecked
    assert f(_descs((None, None, 1.0, None, None, 0, 64)), 1, None) == B.DS_OK


@pytest.mark.skipif("not no_device()")
def test_rownorm_valid_args_reach_device_lookup(L):
    good = (A, Bp, 1.0, Bp + 4096, C, 16, 64)
    shared_w = (A, Bp, 1.0, None, C + 65536, 16, 64)      # tied weights: same w, two outputs
    assert L.ds_weight_rownorm_gain(_descs(good, shared_w), 2, None) == B.DS_ERR_DEVICE


@pytest.mark.parametrize("name", NORM_BWD)
def test_l2_backward_validation(L, name):
    f = getattr(L, name)
    assert f(None, None, C, Bp, 4, 64, 1e-6, None) == B.DS_ERR_NULL
    assert f(A, None, None, Bp, 4, 64, 1e-6, None) == B.DS_ERR_NULL
    assert f(A, None, C, None, 4, 64, 1e-6, None) == B.DS_ERR_NULL
    assert f(A, None, C + 2, Bp, 4, 64, 1e-6, None) == B.DS_ERR_ALIGN
    assert f(A, Bp + 8, C, Bp, 4, 64, 1e-6, None) == B.DS_ERR_ALIGN
    assert f(A, None, C, C + 16, 4, 64, 1e-6, None) == B.DS_ERR_ARG      # dx partly over dy
    assert f(A, None, C, A + 256, 4, 64, 1e-6, None) == B.DS_ERR_ARG     # dx partly over x
    assert f(A, None, C, Bp, 4, 60, 1e-6, None) == B.DS_ERR_SHAPE
    assert f(A, None, C, Bp, 4, 64, float("nan"), None) == B.DS_ERR_ARG
    assert f(None, None, None, None, 0, 64, 1e-6, None) == B.DS_OK


@pytest.mark.skipif("not no_device()")
@pytest.mark.parametrize("name", NORM_BWD)
def test_l2_backward_valid_args_reach_device_lookup(L, name):
    f = getattr(L, name)
    assert f(A, None, C, Bp, 4, 64, 1e-6, None) == B.DS_ERR_DEVICE
    assert f(A, Bp, C, C, 4, 64, 1e-6, None) == B.DS_ERR_DEVICE          # dx == dy
    assert f(A, Bp, C, A, 4, 64, 1e-6, None) == B.DS_ERR_DEVICE          # dx == x


def _gdescs(*items):
    arr = (B.RownormGradDesc * len(items))()
    for i, d in enumerate(items):
        arr[i] = B.RownormGradDesc(*d)
    return arr


def test_rownorm_backward_validation(L):
    f = L.ds_weight_rownorm_gain_backward
    # w, gain, radius, dw_eff, dw, dgain, rows, cols
    good = (A, Bp, 1.0, C, C + 65536, Bp + 4096, 16, 64)
    assert f(_gdescs(good), -1, None) == B.DS_ERR_ARG
    assert f(None, 0, None) == B.DS_OK
    assert f(None, 1, None) == B.DS_ERR_NULL
    assert f(_gdescs((A, Bp, 1.0, C, C + 65536, None, 16, 0)), 1, None) == B.DS_ERR_SHAPE
    assert f(_gdescs((A, Bp, 1.0, C, C + 65536, None, 16, 65537)), 1, None) == B.DS_ERR_SHAPE
    assert f(_gdescs((A, Bp, 1.0, C + 1, C + 65536, None, 16, 147)), 1, None) == B.DS_ERR_ALIGN
    assert f(_gdescs((A, Bp, float("nan"), C, C + 65536, None, 16, 64)), 1, None) == B.DS_ERR_ARG
    assert f(_gdescs((A, Bp, 1.0, None, C + 65536, None, 16, 64)), 1, None) == B.DS_ERR_NULL
    assert f(_gdescs((A, Bp, 1.0, C, None, None, 16, 64)), 1, None) == B.DS_ERR_NULL
    assert f(_gdescs((A, Bp, 1.0, C + 8, C + 65536, None, 16, 64)), 1, None) == B.DS_ERR_ALIGN
    assert f(_gdescs((A, Bp, 1.0, C, C + 65536, Bp + 4098, 16, 64)), 1, None) == B.DS_ERR_ALIGN
    # dw over dw_eff, dgain over gain, dw over w
    assert f(_gdescs((A, Bp, 1.0, C, C + 512, None, 16, 64)), 1, None) == B.DS_ERR_ARG
    assert f(_gdescs((A, Bp, 1.0, C, C + 65536, Bp + 16, 16, 64)), 1, None) == B.DS_ERR_ARG
    assert f(_gdescs((A, Bp, 1.0, C, A, None, 16, 64)), 1, None) == B.DS_ERR_ARG
    # one matrix's output over another matrix's input
    other = (A + 8192, Bp + 1024, 1.0, C + 8192, A + 2048, None, 16, 64)
    assert f(_gdescs(good, other), 2, None) == B.DS_ERR_ARG
    assert f(_gdescs((None, None, 1.0, None, None, None, 0, 64)), 1, None) == B.DS_OK


def test_gain_mode_validation(L):
    f = L.ds_weight_rownorm_gain
    # w, gain, radius, norm_out, w_eff, rows, cols, gain_mode
    assert f(_descs((A, Bp, 1.0, None, C, 16, 64, 3)), 1, None) == B.DS_ERR_ARG
    assert f(_descs((A, Bp, 1.0, None, C, 16, 64, -1)), 1, None) == B.DS_ERR_ARG
    assert f(_descs((A, None, 1.0, None, C, 16, 64, B.DS_GAIN_SCALAR)), 1, None) == B.DS_ERR_NULL
    assert f(_descs((A, Bp + 2, 1.0, None, C, 16, 64, B.DS_GAIN_SCALAR)), 1, None) == B.DS_ERR_ALIGN
    # a gain per row over W_eff's first bytes
    assert f(_descs((A, C - 4, 1.0, None, C, 16, 64, B.DS_GAIN_ROW)), 1, None) == B.DS_ERR_ARG
    g = L.ds_weight_rownorm_gain_backward
    # w, gain, radius, dw_eff, dw, dgain, rows, cols, gain_mode, dgain_total
    tot = Bp + 8192
    assert g(_gdescs((A, Bp, 1.0, C, C + 65536, Bp + 4096, 16, 64, B.DS_GAIN_ROW, tot)), 1,
             None) == B.DS_ERR_ARG                       # a total needs a scalar gain
    assert g(_gdescs((A, Bp, 1.0, C, C + 65536, None, 16, 64, B.DS_GAIN_SCALAR, tot)), 1,
             None) == B.DS_ERR_ARG                       # and the shares it sums
    assert g(_gdescs((A, None, 1.0, C, C + 65536, Bp + 4096, 16, 64, B.DS_GAIN_NONE)), 1,
             None) == B.DS_ERR_ARG                       # no gain, no gain gradient
    assert g(_gdescs((A, Bp, 1.0, C, C + 65536, Bp + 4096, 16, 64, B.DS_GAIN_SCALAR, tot + 2)),
             1, None) == B.DS_ERR_ALIGN
    assert g(_gdescs((A, Bp, 1.0, C, C + 65536, Bp + 4096, 16, 64, B.DS_GAIN_SCALAR,
                      Bp + 4096 + 60)), 1, None) == B.DS_ERR_ARG   # total over the shares
    # an empty matrix's total (0) needs no shares, but is still checked and placed
    assert g(_gdescs((None, None, 1.0, None, None, None, 0, 64, B.DS_GAIN_SCALAR, tot + 2)),
             1, None) == B.DS_ERR_ALIGN
    assert g(_gdescs((A, Bp, 1.0, C, C + 65536, Bp + 4096, 16, 64, B.DS_GAIN_SCALAR, tot),
                     (None, None, 1.0, None, None, None, 0, 64, B.DS_GAIN_SCALAR, tot)),
             2, None) == B.DS_ERR_ARG                    # two totals in one place


@pytest.mark.skipif("not no_device()")
def test_empty_matrix_total_is_accepted(L):
    """rows = 0 with a scalar gain and no shares buffer passes validation and
    stops at the device lookup for the total's launch."""
    g = L.ds_weight_rownorm_gain_backward
    st = g(_gdescs((None, None, 1.0, None, None, None, 0, 64, B.DS_GAIN_SCALAR, Bp + 8192)), 1,
           None)
    assert st == B.DS_ERR_DEVICE


def test_column_block_validation(L):
    f = L.ds_weight_rownorm_gain
    # w, gain, radius, norm_out, w_eff, rows (units), cols (A * seg), gain_mode, seg, ld
    assert f(_descs((A, Bp, 1.0, None, C, 16, 130, 0, 65, 2000)), 1, None) == B.DS_ERR_SHAPE
    assert f(_descs((A, Bp, 1.0, None, C, 16, 10, 0, 3, 2000)), 1, None) == B.DS_ERR_SHAPE
    assert f(_descs((A, Bp, 1.0, None, C, 16, 12, 0, 3, 47)), 1, None) == B.DS_ERR_SHAPE
    assert f(_descs((A, Bp, 1.0, None, C, 16, 12, 0, -3, 48)), 1, None) == B.DS_ERR_SHAPE
    assert f(_descs((A + 2, Bp, 1.0, None, C, 16, 12, 0, 3, 48)), 1, None) == B.DS_ERR_ALIGN
    assert f(_descs((A, Bp, 1.0, None, C + 1, 16, 12, 0, 3, 48)), 1, None) == B.DS_ERR_ALIGN
    # W_eff over the last stored row of w: the span is (A - 1) * ld + rows * seg values
    assert f(_descs((A, Bp, 1.0, None, A + 4 * (3 * 48 + 40), 16, 12, 0, 3, 48)), 1,
             None) == B.DS_ERR_ARG
    g = L.ds_weight_rownorm_gain_backward
    assert g(_gdescs((A, Bp, 1.0, C, C + 65536, None, 16, 12, 0, None, 70, 48)), 1,
             None) == B.DS_ERR_SHAPE
    r = L.ds_rescale_project
    assert r(_rdescs((A, C, 1.0, 16, 12, 4, 40)), 1, None) == B.DS_ERR_SHAPE    # ld < rows * seg


@pytest.mark.skipif("not no_device()")
def test_column_blocks_reach_device_lookup(L):
    f = L.ds_weight_rownorm_gain
    assert f(_descs((A + 4, Bp, 1.0, None, C + 2, 16, 12, 0, 3, 48)), 1, None) == B.DS_ERR_DEVICE
    assert f(_descs((A, Bp, 1.0, None, C, 2304, 768, 0, 1, 2304)), 1, None) == B.DS_ERR_DEVICE
    assert L.ds_rescale_after_step(_rdescs((A, None, 1.0, 16, 12, 3, 48)), 1,
                                   None) == B.DS_ERR_DEVICE


@pytest.mark.skipif("not no_device()")
def test_odd_widths_reach_device_lookup(L):
    assert L.ds_weight_rownorm_gain(_descs((A + 4, Bp, 1.0, None, C + 2, 16, 147)), 1,
                                    None) == B.DS_ERR_DEVICE
    assert L.ds_weight_rownorm_gain_backward(
        _gdescs((A + 4, Bp, 1.0, C + 2, C + 65540, None, 16, 27)), 1, None) == B.DS_ERR_DEVICE
    assert L.ds_rescale_project(_rdescs((A + 4, C + 4, 1.0, 16, 16383)), 1, None) == B.DS_ERR_DEVICE


@pytest.mark.skipif("not no_device()")
def test_gain_modes_reach_device_lookup(L):
    f = L.ds_weight_rownorm_gain
    assert f(_descs((A, None, 1.0, None, C, 16, 64, B.DS_GAIN_NONE)), 1, None) == B.DS_ERR_DEVICE
    assert f(_descs((A, Bp, 1.0, None, C, 16, 64, B.DS_GAIN_SCALAR)), 1, None) == B.DS_ERR_DEVICE
    # a scalar gain spans 4 bytes: W_eff right after it does not overlap it
    assert f(_descs((A, C - 4, 1.0, None, C, 16, 64, B.DS_GAIN_SCALAR)), 1, None) == B.DS_ERR_DEVICE
    g = L.ds_weight_rownorm_gain_backward
    assert g(_gdescs((A, Bp, 1.0, C, C + 65536, Bp + 4096, 16, 64, B.DS_GAIN_SCALAR, Bp + 8192)),
             1, None) == B.DS_ERR_DEVICE
    assert g(_gdescs((A, None, 1.0, C, C + 65536, None, 16, 64, B.DS_GAIN_NONE)), 1,
             None) == B.DS_ERR_DEVICE


@pytest.mark.skipif("not no_device()")
def test_rownorm_backward_valid_args_reach_device_lookup(L):
    good = (A, Bp, 1.0, C, C + 65536, Bp + 4096, 16, 64)
    tied = (A, Bp, 1.0, C, C + 131072, None, 16, 64)       # same inputs, other outputs
    assert L.ds_weight_rownorm_gain_backward(_gdescs(good, tied), 2, None) == B.DS_ERR_DEVICE


def test_rownorm_output_over_other_input_refused(L):
    good = (A, Bp, 1.0, Bp + 4096, C, 16, 64)
    over = (A + 8192, Bp + 1024, 1.0, None, A, 16, 64)     # its W_eff over the first w
    assert L.ds_weight_rownorm_gain(_descs(good, over), 2, None) == B.DS_ERR_ARG


def test_activation_validation(L):
    gate, sw = L.ds_gate_l2_rows, L.ds_swiglu_l2_rows
    S1, S2 = C + 0x100000, C + 0x200000
    assert gate(A, Bp, None, C, 4, 64, 1e-6, None) == B.DS_ERR_NULL
    assert gate(A, None, S1, C, 4, 64, 1e-6, None) == B.DS_ERR_NULL
    assert gate(A, Bp, S1 + 4, C, 4, 64, 1e-6, None) == B.DS_ERR_ALIGN
    assert gate(A, Bp, S1, C + 8, 4, 64, 1e-6, None) == B.DS_ERR_ALIGN
    assert gate(A, Bp, S1, A + 64, 4, 64, 1e-6, None) == B.DS_ERR_ARG       # y partly over o
    assert gate(A, Bp, C + 256, C, 4, 64, 1e-6, None) == B.DS_ERR_ARG       # sg inside y
    assert gate(A, Bp, S1, C, 4, 12, 1e-6, None) == B.DS_ERR_SHAPE
    assert gate(A, Bp, S1, C, 4, 64, -1.0, None) == B.DS_ERR_ARG
    assert gate(None, None, None, None, 0, 64, 1e-6, None) == B.DS_OK
    assert sw(A, Bp, S1, None, C, 4, 64, 1e-6, None) == B.DS_ERR_NULL
    assert sw(A, Bp, S1, S2 + 8, C, 4, 64, 1e-6, None) == B.DS_ERR_ALIGN
    assert sw(A, Bp, S1, C + 64, C, 4, 64, 1e-6, None) == B.DS_ERR_ARG      # suu inside y
    assert sw(A, Bp, S1, S2, Bp + 32, 4, 64, 1e-6, None) == B.DS_ERR_ARG    # y partly over u
    assert sw(None, None, None, None, None, 0, 64, 1e-6, None) == B.DS_OK


@pytest.mark.skipif("not no_device()")
def test_activation_valid_args_reach_device_lookup(L):
    S1, S2 = C + 0x100000, C + 0x200000
    assert L.ds_gate_l2_rows(A, Bp, S1, A, 4, 64, 1e-6, None) == B.DS_ERR_DEVICE      # y == o
    assert L.ds_swiglu_l2_rows(A, Bp, S1, S2, Bp, 4, 64, 1e-6, None) == B.DS_ERR_DEVICE  # y == u


def _qk(L, q=A, ldq=4096, k=Bp, ldk=1024, pos=C, inv=C + 0x10000, sc=C + 0x20000,
        qo=C + 0x100000, ldqo=4096, ko=C + 0x4000000, ldko=1024, rows=4, nq=16, nk=4, hd=256,
        eps=1e-6):
    return L.ds_qk_rows_l2(q, ldq, k, ldk, pos, inv, sc, qo, ldqo, ko, ldko, rows, nq, nk, hd,
                           eps, None)


def test_qk_validation(L):
    assert _qk(L, hd=64) == B.DS_ERR_SHAPE
    assert _qk(L, nq=-1) == B.DS_ERR_SHAPE
    assert _qk(L, ldq=4000) == B.DS_ERR_SHAPE                   # stride below the width
    assert _qk(L, ldk=1028) == B.DS_ERR_SHAPE                   # stride not a multiple of 8
    assert _qk(L, eps=-1.0) == B.DS_ERR_ARG
    assert _qk(L, pos=None) == B.DS_ERR_NULL
    assert _qk(L, sc=None) == B.DS_ERR_NULL
    assert _qk(L, ko=None) == B.DS_ERR_NULL
    assert _qk(L, inv=C + 0x10008) == B.DS_ERR_ALIGN
    assert _qk(L, qo=C + 0x100008) == B.DS_ERR_ALIGN
    assert _qk(L, qo=A + 64) == B.DS_ERR_ARG                    # q_out partly over q
    assert _qk(L, ko=A + 2048) == B.DS_ERR_ARG                  # k_out over q
    assert _qk(L, qo=A, ldqo=4104) == B.DS_ERR_ARG              # same base, other stride
    assert _qk(L, rows=0, q=None, k=None, pos=None, inv=None) == B.DS_OK
    assert _qk(L, nq=0, nk=0) == B.DS_OK


@pytest.mark.skipif("not no_device()")
def test_qk_fused_views_reach_device_lookup(L):
    """q and k as column slices of one [rows, 6144] projection, updated in place."""
    base = 0x60000000
    q, k = base, base + 4096 * 2
    assert _qk(L, q=q, ldq=6144, k=k, ldk=6144, qo=q, ldqo=6144, ko=k, ldko=6144) == \
        B.DS_ERR_DEVICE
    # writing q's output over k's slice is refused
    assert _qk(L, q=q, ldq=6144, k=k, ldk=6144, qo=k - 2048, ldqo=6144, ko=k, ldko=6144) == \
        B.DS_ERR_ARG


def _rdescs(*items):
    arr = (B.RescaleDesc * len(items))()
    for i, d in enumerate(items):
        arr[i] = B.RescaleDesc(*d)
    return arr


def test_rescale_validation(L):
    pr, af = L.ds_rescale_project, L.ds_rescale_after_step
    good = (A, C, 1.0, 16, 64)                        # w, v, radius, rows, cols
    assert pr(_rdescs(good), -1, None) == B.DS_ERR_ARG
    assert pr(None, 0, None) == B.DS_OK and af(None, 0, None) == B.DS_OK
    assert pr(None, 1, None) == B.DS_ERR_NULL
    assert pr(_rdescs((A, None, 1.0, 16, 64)), 1, None) == B.DS_ERR_NULL      # project needs v
    assert pr(_rdescs((A, C, 1.0, 16, 0)), 1, None) == B.DS_ERR_SHAPE
    assert pr(_rdescs((A, C, 1.0, 16, 20001)), 1, None) == B.DS_ERR_SHAPE
    assert pr(_rdescs((A, C + 2, 1.0, 16, 147)), 1, None) == B.DS_ERR_ALIGN
    assert pr(_rdescs((A + 8, C, 1.0, 16, 64)), 1, None) == B.DS_ERR_ALIGN
    assert pr(_rdescs((A, A + 1024, 1.0, 16, 64)), 1, None) == B.DS_ERR_ARG   # v over w
    assert af(_rdescs((A, C, float("inf"), 16, 64)), 1, None) == B.DS_ERR_ARG
    # after a step w is written too: two matrices sharing w are refused
    assert af(_rdescs(good, (A, C + 65536, 1.0, 16, 64)), 2, None) == B.DS_ERR_ARG
    assert af(_rdescs((None, None, 1.0, 0, 64)), 1, None) == B.DS_OK


@pytest.mark.skipif("not no_device()")
def test_rescale_valid_args_reach_device_lookup(L):
    good = (A, C, 1.0, 16, 64)
    tied = (A, C + 65536, 1.0, 16, 64)               # project: w shared (read only), two v
    assert L.ds_rescale_project(_rdescs(good, tied), 2, None) == B.DS_ERR_DEVICE
    assert L.ds_rescale_after_step(_rdescs((A, None, 2.0, 16, 64)), 1, None) == B.DS_ERR_DEVICE


def test_binding_raises_on_missing_library(monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", "/nonexistent/libdsrows.so")
    with pytest.raises(RuntimeError, match="missing"):
        B.lib()


# ------------------------------------------- the allocation-free weight gradient

BIG = 1 << 36        # fake addresses far apart for matrices of a million rows


def test_noalloc_validation(L):
    g = L.ds_weight_rownorm_gain_backward_noalloc
    tot = Bp + 8192
    # w, gain, radius, dw_eff, dw, dgain, rows, cols, gain_mode, dgain_total
    assert g(None, 0, None) == B.DS_OK
    assert g(None, 1, None) == B.DS_ERR_NULL
    # the shares live in the library's scratch: a scalar gain's dgain must be NULL
    assert g(_gdescs((A, Bp, 1.0, C, C + 65536, Bp + 4096, 16, 64, B.DS_GAIN_SCALAR, tot)), 1,
             None) == B.DS_ERR_ARG
    assert g(_gdescs((A, Bp, 1.0, C, C + 65536, Bp + 4096, 16, 64, B.DS_GAIN_SCALAR)), 1,
             None) == B.DS_ERR_ARG
    # the other checks are the allocating call's
    assert g(_gdescs((A, Bp, 1.0, C, C + 65536, None, 16, 64, B.DS_GAIN_ROW, tot)), 1,
             None) == B.DS_ERR_ARG
    assert g(_gdescs((A, Bp, 1.0, C + 8, C + 65536, None, 16, 64)), 1, None) == B.DS_ERR_ALIGN


def _big_scalar(i, rows):
    base = (i + 1) * BIG
    # w, gain, radius, dw_eff, dw, dgain, rows, cols, gain_mode, dgain_total
    return (base, base + BIG // 2, 1.0, base + BIG // 4, base + 3 * BIG // 4, None, rows, 8,
            B.DS_GAIN_SCALAR, base + BIG // 2 + 64)


def test_noalloc_scratch_limit(L):
    g = L.ds_weight_rownorm_gain_backward_noalloc
    n = B.DS_SCRATCH_FLOATS
    assert g(_gdescs(_big_scalar(0, n + 1)), 1, None) == B.DS_ERR_SCRATCH
    # the limit is over the call's scalar-gain rows together
    assert g(_gdescs(_big_scalar(0, n // 2), _big_scalar(1, n // 2 + 1)), 2,
             None) == B.DS_ERR_SCRATCH
    # rows with a gain per row need no scratch
    per_row = (5 * BIG, 5 * BIG + BIG // 2, 1.0, 5 * BIG + BIG // 4, 5 * BIG + 3 * BIG // 4,
               5 * BIG + BIG // 2 + 4 * n + 64, n, 8)
    st = g(_gdescs(_big_scalar(0, n), per_row), 2, None)
    assert st != B.DS_ERR_SCRATCH and st != B.DS_ERR_ARG
    assert "DS_SCRATCH_FLOATS" in B.ds_status_string(B.DS_ERR_SCRATCH)


@pytest.mark.skipif("not no_device()")
def test_noalloc_valid_args_reach_device_lookup(L):
    g = L.ds_weight_rownorm_gain_backward_noalloc
    n = B.DS_SCRATCH_FLOATS
    assert g(_gdescs(_big_scalar(0, n)), 1, None) == B.DS_ERR_DEVICE
    assert g(_gdescs(_big_scalar(0, n // 2), _big_scalar(1, n // 2)), 2, None) == B.DS_ERR_DEVICE
