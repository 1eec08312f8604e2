"""GPU parity of the adapter gradients ("QLoRA: Mathematical Foundations ...",
"Gradient Computation"): dA = s X^T (dY B^T) and dB = s (X A)^T dY against
the oracle's double-precision sums.

Tolerance: max_i |g_i - r_i| / max(|r_i|, rms(r)) <= 2e-2 (bf16 operands and
bf16 X.A, dY.B^T; fp32 token sums; the reference keeps every product exact).
Inputs are seeded synthetic bf16 tensors; nothing the oracle reads comes from
the GPU.
"""
import numpy as np
import pytest

import nf4_quantize_amd as nq
import oracle
import workloads
from gpu_util import log, rel_err_metric, to_dev, to_host

pytestmark = pytest.mark.gpu

TOL = 2e-2


def case(seed, m, k, n, r, sigma=0.05):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = workloads.to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    dy = workloads.to_bf16_bits(rng.standard_normal((m, n), dtype=np.float32))
    a = workloads.to_bf16_bits(rng.standard_normal((k, r), dtype=np.float32) * np.float32(sigma))
    b = workloads.to_bf16_bits(rng.standard_normal((r, n), dtype=np.float32) * np.float32(sigma))
    return x, dy, a, b


def host_f32(t):
    import torch

    if t.dtype == torch.bfloat16:
        return (to_host(t).astype(np.uint32) << 16).view(np.float32)
    return t.detach().cpu().numpy()


CASES = [
    # (m, K, N, r): one tile and several, ragged token counts, a rank that is
    # not a multiple of 64, the widest rank, token sums split over workgroups
    (64, 256, 128, 16),
    (37, 192, 320, 8),
    (130, 512, 256, 64),
    (70, 320, 192, 256),
    (1, 64, 64, 8),
    (300, 1024, 512, 40),
    (257, 2048, 128, 72),
    (1000, 128, 640, 24),
]


@pytest.mark.parametrize("m,k,n,r", CASES)
@pytest.mark.parametrize("dt", ["float32", "bfloat16"])
def test_lora_grads_full(dev, m, k, n, r, dt):
    import torch

    log(f"lora grads m={m} K={k} N={n} r={r} {dt}")
    x, dy, a, b = case(m + 3 * k + n + r, m, k, n, r)
    gdt = getattr(torch, dt)
    ga, gb = nq.lora_backward(to_dev(x, dev), to_dev(dy, dev), to_dev(a, dev), to_dev(b, dev), 2.0,
                              grad_dtype=gdt)
    torch.cuda.synchronize()
    ra, rb = oracle.lora_grads(x, dy, a, b, 2.0)
    ea, _ = rel_err_metric(host_f32(ga), ra)
    eb, _ = rel_err_metric(host_f32(gb), rb)
    log(f"  dA err {ea:.3e}, dB err {eb:.3e}")
    assert ga.shape == (k, r) and gb.shape == (r, n)
    assert ea <= TOL and eb <= TOL


def test_lora_grads_one_side_and_no_tokens(dev):
    import torch

    m, k, n, r = 96, 256, 192, 32
    x, dy, a, b = case(9, m, k, n, r)
    args = (to_dev(x, dev), to_dev(dy, dev), to_dev(a, dev), to_dev(b, dev), 2.0)
    ga, gb = nq.lora_backward(*args, grad_b=False)
    gb2 = torch.full((r, n), 7.0, device=dev)
    ga2, gb2r = nq.lora_backward(*args, grad_a=False, grad_b=gb2)
    torch.cuda.synchronize()
    assert gb is None and ga2 is None and gb2r is gb2
    ra, rb = oracle.lora_grads(x, dy, a, b, 2.0)
    assert rel_err_metric(host_f32(ga), ra)[0] <= TOL
    assert rel_err_metric(host_f32(gb2), rb)[0] <= TOL
    # no tokens: both sums are empty, the gradients are zero (outputs prefilled)
    z = torch.empty((0, k), dtype=torch.bfloat16, device=dev)
    zy = torch.empty((0, n), dtype=torch.bfloat16, device=dev)
    oa = torch.full((k, r), 5.0, device=dev)
    ob = torch.full((r, n), 5.0, device=dev)
    nq.lora_backward(z, zy, args[2], args[3], 2.0, grad_a=oa, grad_b=ob)
    torch.cuda.synchronize()
    assert float(oa.abs().max()) == 0.0 and float(ob.abs().max()) == 0.0


def test_lora_grads_qlora_shape_sampled(dev):
    """4096 tokens, K = N = 8192, r = 64 (the QLoRA linear's shape): sampled
    rows of dA and columns of dB against the oracle."""
    import torch

    d = workloads.linear_inputs()
    s = workloads.LIN_SCALE
    ga, gb = nq.lora_backward(to_dev(d["x"], dev), to_dev(d["dy"], dev), to_dev(d["a"], dev),
                              to_dev(d["b"], dev), s)
    torch.cuda.synchronize()
    K, N = d["x"].shape[1], d["dy"].shape[1]
    rows = np.array([0, 1, 63, 64, 777, 4095, 4096, 6000, K - 1])
    cols = np.array([0, 5, 64, 1000, 4097, 8000, N - 1])
    log("oracle adapter gradients at 4096 x 8192 x 8192, r = 64 (sampled)")
    ra, rb = oracle.lora_grads(d["x"], d["dy"], d["a"], d["b"], s, a_rows=rows, b_cols=cols)
    ea, _ = rel_err_metric(host_f32(ga)[rows], ra)
    eb, _ = rel_err_metric(host_f32(gb)[:, cols], rb)
    log(f"  dA err {ea:.3e}, dB err {eb:.3e}")
    assert ea <= TOL and eb <= TOL


@pytest.mark.parametrize("m,k,n,r", [(1000, 128, 640, 24), (300, 1024, 512, 40), (1, 64, 64, 8)])
def test_lora_grads_reused_dirty_workspace(dev, m, k, n, r):
    """The workspace holds the products X.A, dY.B^T and the split partial
    sums of both products, then of both gradients, at once: a workspace full
    of non-zero bytes, used by two calls in a row, gives the same gradients
    both times, equal to those of a fresh workspace and within the tolerance
    of the oracle."""
    import torch

    log(f"lora grads, reused dirty workspace m={m} K={k} N={n} r={r}")
    x, dy, a, b = case(40 + m, m, k, n, r)
    args = (to_dev(x, dev), to_dev(dy, dev), to_dev(a, dev), to_dev(b, dev), 2.0)
    size = nq.nf4_lora_backward_workspace_size(m, k, n, r)
    ws = torch.full((size,), 0x7F, dtype=torch.uint8, device=dev)
    out = []
    for _ in range(2):
        ga = torch.empty((k, r), dtype=torch.float32, device=dev)
        gb = torch.empty((r, n), dtype=torch.float32, device=dev)
        nq.lora_backward(*args, grad_a=ga, grad_b=gb, workspace=ws)
        out.append((ga, gb))
    fa, fb = nq.lora_backward(*args)
    torch.cuda.synchronize()
    for ga, gb in out:
        assert torch.equal(ga.view(torch.int32), fa.view(torch.int32))
        assert torch.equal(gb.view(torch.int32), fb.view(torch.int32))
    ra, rb = oracle.lora_grads(x, dy, a, b, 2.0)
    assert rel_err_metric(host_f32(fa), ra)[0] <= TOL
    assert rel_err_metric(host_f32(fb), rb)[0] <= TOL
