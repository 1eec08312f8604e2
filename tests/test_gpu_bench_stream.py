"""The measured-ceiling kernels of bench.py (bench_stream.so) move the bytes
they claim: every source byte they are timed on is read and every destination
byte written, checked against the same arithmetic on the host. A ceiling from
a kernel that skipped traffic would flatter every fraction computed from it.
"""
import ctypes
import os

import numpy as np
import pytest

from conftest import ROOT
from gpu_util import to_dev, to_host

pytestmark = pytest.mark.gpu

GROUPS = 5


@pytest.fixture(scope="module")
def so(dev):
    # loaded after torch (the dev fixture), so that both use torch's HIP runtime
    path = os.path.join(ROOT, "bench_stream.so")
    if not os.path.exists(path):
        pytest.fail(f"{path} is not built: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.bench_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_void_p]
    lib.bench_stream.restype = ctypes.c_int
    return lib


def run(so, kind, src, dst_bytes):
    import torch

    s = to_dev(src, torch.device("cuda:0"))
    d = torch.zeros(dst_bytes, dtype=torch.uint8, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert so.bench_stream(kind, s.data_ptr(), d.data_ptr(), GROUPS, stream) == 0
    torch.cuda.synchronize()
    return to_host(d)


def test_read4_write1(so):
    rng = np.random.Generator(np.random.PCG64(1))
    src = rng.integers(0, 256, GROUPS * 32768, dtype=np.uint8)
    got = run(so, 0, src, GROUPS * 8192).view(np.uint32).reshape(GROUPS, 512, 4)
    v = src.view(np.uint32).reshape(GROUPS, 4, 512, 4)  # group, quarter, thread, word
    assert np.array_equal(got, v[:, 0] ^ v[:, 1] ^ v[:, 2] ^ v[:, 3])


def test_read1_write4(so):
    rng = np.random.Generator(np.random.PCG64(2))
    src = rng.integers(0, 256, GROUPS * 8192, dtype=np.uint8)
    got = run(so, 1, src, GROUPS * 32768).view(np.uint32).reshape(GROUPS, 2, 4, 256, 4)
    v = src.view(np.uint32).reshape(GROUPS, 2, 256, 4)  # group, half, thread, word
    for j in range(4):
        assert np.array_equal(got[:, :, j], v ^ np.uint32(j))


def test_read_only_writes_nothing(so):
    # quarter q of group g holds the byte 4g + q + 1: a thread's four vectors
    # XOR to the byte (4g+1)^(4g+2)^(4g+3)^(4g+4), never 0xFF, so no word of
    # theirs has all bits set and the all-ones key never matches
    src = np.repeat(np.arange(GROUPS * 4, dtype=np.uint8) + 1, 8192)
    assert all((4 * g + 1) ^ (4 * g + 2) ^ (4 * g + 3) ^ (4 * g + 4) != 0xFF for g in range(GROUPS))
    got = run(so, 2, src, GROUPS * 16)
    assert not got.any()


def test_rejects_bad_arguments(so):
    assert so.bench_stream(0, None, None, GROUPS, None) != 0
    assert so.bench_stream(3, 16, 16, GROUPS, None) != 0
    assert so.bench_stream(0, 16, 16, 0, None) != 0
    assert so.bench_stream(0, 8, 16, GROUPS, None) != 0
