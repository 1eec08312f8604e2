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
    lib.bench_stream_grid.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.bench_stream_grid.restype = ctypes.c_int
    return lib


def run(so, kind, src, dst_bytes, grid=1):
    import torch

    s = to_dev(src, torch.device("cuda:0"))
    d = torch.zeros(dst_bytes, dtype=torch.uint8, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if kind <= 2:
        assert so.bench_stream(kind, s.data_ptr(), d.data_ptr(), GROUPS, stream) == 0
    else:
        assert so.bench_stream_grid(kind, s.data_ptr(), d.data_ptr(), GROUPS, grid, stream) == 0
    torch.cuda.synchronize()
    return to_host(d)


# the persistent kinds on grids smaller than, equal to and larger than the
# group count (each workgroup walks several groups, one, or none)
GRIDS = (1, 2, GROUPS, 64)


@pytest.mark.parametrize("grid", GRIDS)
def test_read4_write1(so, grid):
    rng = np.random.Generator(np.random.PCG64(1))
    src = rng.integers(0, 256, GROUPS * 32768, dtype=np.uint8)
    got = run(so, 0, src, GROUPS * 8192).view(np.uint32).reshape(GROUPS, 512, 4)
    v = src.view(np.uint32).reshape(GROUPS, 4, 512, 4)  # group, quarter, thread, word
    assert np.array_equal(got, v[:, 0] ^ v[:, 1] ^ v[:, 2] ^ v[:, 3])
    # persistent form: 256 threads, 8 reads and 2 writes each per group
    got = run(so, 3, src, GROUPS * 8192, grid).view(np.uint32).reshape(GROUPS, 2, 256, 4)
    v = src.view(np.uint32).reshape(GROUPS, 8, 256, 4)
    x = np.bitwise_xor.reduce(v, axis=1)
    for j in range(2):
        assert np.array_equal(got[:, j], x ^ np.uint32(j))


@pytest.mark.parametrize("grid", GRIDS)
def test_read1_write4(so, grid):
    rng = np.random.Generator(np.random.PCG64(2))
    src = rng.integers(0, 256, GROUPS * 8192, dtype=np.uint8)
    got = run(so, 1, src, GROUPS * 32768).view(np.uint32).reshape(GROUPS, 2, 4, 256, 4)
    v = src.view(np.uint32).reshape(GROUPS, 2, 256, 4)  # group, half, thread, word
    for j in range(4):
        assert np.array_equal(got[:, :, j], v ^ np.uint32(j))
    # persistent form: 2 reads and 8 writes per thread and group
    got = run(so, 4, src, GROUPS * 32768, grid).view(np.uint32).reshape(GROUPS, 8, 256, 4)
    x = v[:, 0] ^ v[:, 1]
    for j in range(8):
        assert np.array_equal(got[:, j], x ^ np.uint32(j))


@pytest.mark.parametrize("grid", GRIDS)
def test_read_only_writes_nothing(so, grid):
    # quarter q of group g holds the byte 4g + q + 1: a thread's four vectors
    # XOR to the byte (4g+1)^(4g+2)^(4g+3)^(4g+4), never 0xFF, so no word of
    # theirs has all bits set and the all-ones key never matches
    src = np.repeat(np.arange(GROUPS * 4, dtype=np.uint8) + 1, 8192)
    assert all((4 * g + 1) ^ (4 * g + 2) ^ (4 * g + 3) ^ (4 * g + 4) != 0xFF for g in range(GROUPS))
    got = run(so, 2, src, GROUPS * 16)
    assert not got.any()
    # persistent form: eighths of a group hold the bytes of its quarters
    # twice, so its 8 vectors XOR to 0, never all ones
    got = run(so, 5, src, GROUPS * 16, grid)
    assert not got.any()


def test_rejects_bad_arguments(so):
    assert so.bench_stream(0, None, None, GROUPS, None) != 0
    assert so.bench_stream(3, 16, 16, GROUPS, None) != 0
    assert so.bench_stream(0, 16, 16, 0, None) != 0
    assert so.bench_stream(0, 8, 16, GROUPS, None) != 0
    assert so.bench_stream_grid(3, 16, 16, GROUPS, 0, None) != 0
    assert so.bench_stream_grid(4, 16, 16, GROUPS, 65537, None) != 0


def test_mfma_ceiling_computes_its_products(so):
    """bench_mfma issues the MFMAs it is timed for: one workgroup, two
    iterations, against the same products in float64 on the host."""
    import torch

    so.bench_mfma.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                              ctypes.c_void_p]
    so.bench_mfma.restype = ctypes.c_int
    rng = np.random.Generator(np.random.PCG64(3))
    vals = rng.standard_normal(4 * 16 * 64 * 8).astype(np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)  # bf16 by truncation: exact operands
    src = to_dev(bits, torch.device("cuda:0"))
    dst = torch.zeros(4 * 4096, dtype=torch.float32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert so.bench_mfma(src.data_ptr(), dst.data_ptr(), 1, 2, stream) == 0
    torch.cuda.synchronize()
    got = to_host(dst).reshape(4, 4, 16, 64)  # wave, tile, register, lane
    op = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(4, 16, 64, 8)
    lane = np.arange(64)
    for wv in range(4):
        # operand set i as a 32 x 16 matrix: lane l holds row l % 32, k = 8 (l / 32) + e
        def mat(i):
            m = np.zeros((32, 16))
            for l in range(64):
                m[l % 32, 8 * (l // 32): 8 * (l // 32) + 8] = op[wv, i, l]
            return m
        A = [mat(i) for i in range(8)]
        B = [mat(8 + i) for i in range(8)]
        want = np.zeros((4, 32, 32))
        for _ in range(2):
            for m in range(64):
                want[m % 4] += A[m % 8] @ B[(m // 8 + m) % 8].T
        for t in range(4):
            for v in range(16):
                rows = 8 * (v // 4) + 4 * (lane // 32) + v % 4
                np.testing.assert_allclose(got[wv, t, v], want[t, rows, lane % 32], rtol=2e-5,
                                           atol=2e-4)
    assert so.bench_mfma(src.data_ptr(), dst.data_ptr(), 0, 1, stream) != 0
