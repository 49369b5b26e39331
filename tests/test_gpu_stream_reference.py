"""The benchmark's stream references do the traffic they stand for.

bench.py quotes two plain stream kernels (libdsbench.so) as the rate a
kernel of the row ops' launch can reach: y = x ^ r over bf16 rows with
l2_rows' launch, and y = bf16(x) over fp32 rows with the weight op's launch.
A reference that skipped work would flatter every fraction quoted against
it, so each is checked here on every element, at the benchmark's shapes and
at widths whose rows leave lanes idle: the XOR bit for bit, the fp32 to bf16
rounding against torch's (round to nearest even).
"""
import ctypes

import pytest

from gpu_util import announce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def BL():
    from scale_invariant_row_amd import binding
    binding.lib()
    lib = ctypes.CDLL(binding.LIB_PATH.replace("libdsrows.so", "libdsbench.so"))
    lib.dsb_stream_rows.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 2 + [ctypes.c_void_p]
    lib.dsb_stream_rows.restype = ctypes.c_int
    lib.dsb_stream_f32_rows.argtypes = [ctypes.c_void_p] * 2 + [ctypes.c_int64] * 2 + [ctypes.c_void_p]
    lib.dsb_stream_f32_rows.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("rows,cols", [(8192, 4096), (1000, 1024), (77, 520), (5, 8192)])
def test_xor_stream(BL, rows, cols):
    import torch
    announce("stream reference x ^ r", rows, cols)
    g = torch.Generator(device="cuda:0").manual_seed(rows + cols)
    x = torch.randint(-32768, 32767, (rows, cols), dtype=torch.int16, device="cuda:0", generator=g)
    r = torch.randint(-32768, 32767, (rows, cols), dtype=torch.int16, device="cuda:0", generator=g)
    y = torch.full_like(x, 0x5555)
    st = torch.cuda.current_stream().cuda_stream
    assert BL.dsb_stream_rows(x.data_ptr(), r.data_ptr(), y.data_ptr(), rows, cols, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(y, x ^ r)


@pytest.mark.parametrize("rows,cols", [(11008, 4096), (73728, 768), (333, 1028), (9, 2304), (3, 20)])
def test_fp32_to_bf16_stream(BL, rows, cols):
    import torch
    announce("stream reference bf16(x)", rows, cols)
    g = torch.Generator(device="cuda:0").manual_seed(rows * 7 + cols)
    x = torch.randn(rows, cols, device="cuda:0", generator=g) * 0.02
    y = torch.full((rows, cols), 0x5555, dtype=torch.int16, device="cuda:0")
    st = torch.cuda.current_stream().cuda_stream
    assert BL.dsb_stream_f32_rows(x.data_ptr(), y.data_ptr(), rows, cols, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(y, x.to(torch.bfloat16).view(torch.int16))


def test_unsupported_widths_are_refused(BL):
    import torch
    st = torch.cuda.current_stream().cuda_stream
    assert BL.dsb_stream_rows(None, None, None, 1, 12, st) == -1          # not a multiple of 8
    assert BL.dsb_stream_f32_rows(None, None, 1, 6, st) == -1              # not a multiple of 4
    assert BL.dsb_stream_f32_rows(None, None, 0, 4096, st) == 0            # nothing to do
