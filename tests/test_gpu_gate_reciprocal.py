"""The gate's fast reciprocal against IEEE division, exhaustively.

The gate row computes sigmoid = 1 / b with b = 1 + exp(-x) in [1, +inf] as
gfx950's v_rcp_f32 estimate plus one fma correction, and takes the IEEE
division only for b >= 2^126, +inf or NaN (TensorFold PR #1260's activation
commit: sigmoid is torch's fp32 form with IEEE division).  That shortcut is
exact only if the two agree bit for bit on every b it is used for: this runs
the device code over every fp32 value from 1 up to 2^126 (2^30 values) and
checks that none differs, and that from 2^126 on they do (the quotient is
subnormal there and the estimate flushes it), which is why the kernel
switches to the division at that point.
"""
import ctypes
import struct

import pytest

from scale_invariant_row_amd import binding as B

pytestmark = pytest.mark.gpu


def bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


@pytest.fixture(scope="module")
def check():
    import torch
    B.lib()
    L = ctypes.CDLL(B.LIB_PATH.replace("libdsrows.so", "libdsbench.so"))
    L.dsb_recip_check.argtypes = [ctypes.c_uint32, ctypes.c_uint32, ctypes.c_void_p,
                                  ctypes.c_void_p]
    L.dsb_recip_check.restype = ctypes.c_int

    def run(first: int, last: int):
        out = torch.tensor([0, -1], dtype=torch.int32, device="cuda:0")
        st = torch.cuda.current_stream().cuda_stream
        assert L.dsb_recip_check(first, last - first, out.data_ptr(), st) == 0
        torch.cuda.synchronize()
        n, lowest = out.cpu().tolist()
        return n, lowest & 0xFFFFFFFF
    return run


def test_equal_to_ieee_division_on_every_b_below_2_to_126(check):
    n, lowest = check(bits(1.0), bits(2.0 ** 126))
    assert n == 0, f"{n} values differ, the smallest bits {lowest:#x}"


def test_differs_from_2_to_126_on(check):
    # (2^126, max]: the quotient is subnormal and the estimate flushes it
    # (2^126 itself has the normal quotient 2^-126)
    first, last = bits(2.0 ** 126), 0x7F800000
    n, lowest = check(first, last)
    assert n >= (last - first) - 1 and lowest in (first, first + 1), (n, hex(lowest))
