"""The streaming-read reference the benchmark quotes beside HBM peak reads
every byte of its buffer: each thread's XOR of its 16-byte pieces (grid-stride
order) matches the same fold computed on the host, for every launch shape
the benchmark tries and for a length that leaves a ragged last trip."""

import ctypes
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def stream_lib():
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_asymmetric_head_amd", "libdiffkv_stream.so"))
    lib.diffkv_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_void_p]
    lib.diffkv_stream_read.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("blocks,unroll", [(512, 4), (512, 8), (2048, 8), (8192, 4)])
def test_every_piece_is_read(blocks, unroll):
    lib = stream_lib()
    rng = np.random.default_rng(blocks + unroll)
    n16 = blocks * 256 * 3 + 12345            # several trips and a ragged tail
    host = rng.integers(0, 2 ** 32, size=(n16, 4), dtype=np.uint32)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(blocks * 256, dtype=torch.int32, device="cuda")
    print(f"[gpu] stream_read blocks={blocks} unroll={unroll} bytes={n16 * 16}", flush=True)
    st = lib.diffkv_stream_read(src.data_ptr(), n16 * 16, sink.data_ptr(), blocks, unroll,
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    stride = blocks * 256
    fold = np.bitwise_xor.reduce(host, axis=1)
    padded = np.zeros(-(-n16 // stride) * stride, dtype=np.uint32)
    padded[:n16] = fold
    expect = np.bitwise_xor.reduce(padded.reshape(-1, stride), axis=0)
    got = sink.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, expect)
