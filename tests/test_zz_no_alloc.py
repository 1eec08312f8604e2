"""The allocation-free linear forward (nf4_linear_forward_noalloc) against
the existing entry point (nf4_linear_forward with a caller workspace): the
same kernels in the same order, so the outputs must be identical, bit for
bit. Two calls in a row share the library's static scratch, the second with
a smaller input; a shape whose workspace would not fit is rejected.

Inputs are seeded synthetic tensors.
"""
import ctypes

import numpy as np
import pytest

import nf4_quantize_amd as nq
import workloads
from gpu_util import log, to_dev, to_host

pytestmark = pytest.mark.gpu


def case(dev, m, N, K, r, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.standard_normal(N * K, dtype=np.float32) * np.float32(0.02)
    wt = nq.quantize(to_dev(w, dev), double_quant=True)
    wt = nq.NF4Tensor(wt.codes, None, wt.absmax_q, wt.absmax_scale, (N, K))
    x = to_dev(workloads.to_bf16_bits(rng.standard_normal((m, K), dtype=np.float32)), dev)
    a = b = None
    if r:
        a = to_dev(workloads.to_bf16_bits(rng.standard_normal((K, r), dtype=np.float32)
                                          * np.float32(0.01)), dev)
        b = to_dev(workloads.to_bf16_bits(rng.standard_normal((r, N), dtype=np.float32)
                                          * np.float32(0.01)), dev)
    return wt, x, a, b


def test_noalloc_forward_equals_workspace_forward(dev):
    import torch

    for m, N, K, r, seed in ((1024, 2048, 4096, 64, 1),   # first call: the larger input
                             (100, 512, 1024, 16, 2),     # second call: smaller
                             (4096, 512, 512, 192, 3),    # the largest rank that fits at m = 4096
                             (7, 320, 512, 0, 4)):        # no adapter: no scratch used
        log(f"no-alloc forward m={m} N={N} K={K} r={r}")
        wt, x, a, b = case(dev, m, N, K, r, seed)
        want = nq.linear_forward(x, wt, a, b, 2.0)
        torch.cuda.synchronize()
        got = nq.nf4_linear_forward_noalloc(x, wt, a, b, 2.0)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(got), to_host(want)), (m, N, K, r)


def test_noalloc_rejects_oversized_scratch(dev):
    m, N, K, r = 4096, 256, 512, 256
    assert nq.nf4_linear_workspace_size(m, r) > nq.NF4_NOALLOC_SCRATCH_BYTES
    wt, x, a, b = case(dev, 8, N, K, r, 5)
    ws = wt.weight_struct()
    y = x.new_empty((m, N))
    xx = x.new_empty((m, K))
    st = nq.lib().nf4_linear_forward_noalloc(xx.data_ptr(), m, ctypes.byref(ws), a.data_ptr(),
                                             b.data_ptr(), r, 2.0, y.data_ptr(), None)
    assert st == 2  # NF4_ERR_SIZE: nothing launched
