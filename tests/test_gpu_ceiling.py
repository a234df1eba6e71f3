"""The benchmark's streaming-ceiling kernel (libopq_ceiling.so) moves exactly
the bytes it is asked to: every 16-byte unit of the output rows is written,
nothing past them, whatever the tile and row split."""
import ctypes

import pytest

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes past the output that must stay untouched


def _lib():
    from w4a16_linear_amd import build as B
    lib = ctypes.CDLL(B.CEILING_LIB)
    f = lib.opq_ceiling_stream_rows
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_void_p]
    return f


# (rows, read bytes per row, written bytes per row): the quantize and
# dequantize mixes of a 3840-wide row, rows longer than a tile, rows that
# only write, and counts that leave a partial last tile.
CASES = [(1000, 7680, 2416), (37, 2416, 7680), (5, 32768, 16), (3, 0, 48),
         (20481, 48, 16), (2, 16, 65536)]


@pytest.mark.parametrize("rows,rd,wr", CASES)
def test_stream_ceiling_writes_exactly_its_rows(gpu_lib, rows, rd, wr):
    import torch
    f = _lib()
    dev = torch.device("cuda:0")
    src = torch.randint(0, 256, (max(rows * rd, 16),), dtype=torch.uint8, device=dev)
    dst = torch.full((rows * wr + GUARD,), 0xAB, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    assert f(src.data_ptr(), dst.data_ptr(), rows, rd, wr, stream) == 0
    torch.cuda.synchronize()
    out = dst.cpu()
    assert bool((out[rows * wr:] == 0xAB).all()), "wrote past the output rows"
    # each written unit is (xor of the tile's reads, unit index, tile, 0): its
    # last word is zero wherever the kernel wrote
    units = out[:rows * wr].view(torch.int32).view(-1, 4)
    assert bool((units[:, 3] == 0).all()), "an output unit was not written"
