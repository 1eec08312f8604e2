"""The differentiable QLoRA linear (nf4_lora_linear / NF4LoRALinear): forward,
dX and the adapter gradients through torch autograd, against the oracle's
double-precision linear and adapter gradients ("QLoRA: Mathematical
Foundations ...", "Forward Pass Computation" and "Gradient Computation").
The packed weight is the oracle's quantization of a seeded weight, uploaded;
nothing the oracle reads comes from the GPU. Tolerance: the linear's 2e-2
rule (rel_err_metric).
"""
import numpy as np
import pytest

import nf4_quantize_amd as nq
import oracle
import workloads
from gpu_util import log, rel_err_metric, to_dev, to_host
from test_gpu_linear import oracle_wdeq, upload_weight

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _f32(t):
    import torch

    return (to_host(t.detach().contiguous()).astype(np.uint32) << 16).view(np.float32) \
        if t.dtype == torch.bfloat16 else t.detach().cpu().numpy()


@pytest.mark.parametrize("lead,K,N,r", [((2, 48), 512, 384, 16), ((130,), 1024, 256, 64)])
def test_lora_linear_autograd(dev, lead, K, N, r):
    import torch

    log(f"autograd QLoRA linear lead={lead} K={K} N={N} r={r}")
    rng = np.random.Generator(np.random.PCG64(sum(lead) + K + N + r))
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    m = int(np.prod(lead))
    x = workloads.to_bf16_bits(rng.standard_normal((m, K), dtype=np.float32))
    dy = workloads.to_bf16_bits(rng.standard_normal((m, N), dtype=np.float32))
    a = workloads.to_bf16_bits(rng.standard_normal((K, r), dtype=np.float32) * np.float32(0.05))
    b = workloads.to_bf16_bits(rng.standard_normal((r, N), dtype=np.float32) * np.float32(0.05))
    wt, host = upload_weight(w, dev)
    wd = oracle_wdeq(host, (N, K))

    Layer = nq.make_lora_linear_module()
    layer = Layer(wt, r=r, alpha=2.0 * r)  # scale alpha / r = 2
    # B starts at zero: the layer is the quantized base alone
    xt = to_dev(x, dev).reshape(*lead, K)
    y0 = layer(xt)
    torch.cuda.synchronize()
    assert y0.shape == (*lead, N)
    assert rel_err_metric(_f32(y0).reshape(m, N), oracle.linear_forward(x, wd))[0] <= TOL

    with torch.no_grad():
        layer.lora_a.copy_(to_dev(a, dev))
        layer.lora_b.copy_(to_dev(b, dev))
    xg = to_dev(x, dev).reshape(*lead, K).requires_grad_()
    y = layer(xg)
    y.backward(to_dev(dy, dev).reshape(*lead, N))
    torch.cuda.synchronize()
    s = layer.scale
    e_y = rel_err_metric(_f32(y).reshape(m, N), oracle.linear_forward(x, wd, a, b, s))[0]
    e_dx = rel_err_metric(_f32(xg.grad).reshape(m, K), oracle.linear_backward_input(dy, wd, a, b, s))[0]
    ra, rb = oracle.lora_grads(x, dy, a, b, s)
    e_da = rel_err_metric(_f32(layer.lora_a.grad), ra)[0]
    e_db = rel_err_metric(_f32(layer.lora_b.grad), rb)[0]
    log(f"  y {e_y:.2e}, dX {e_dx:.2e}, dA {e_da:.2e}, dB {e_db:.2e}")
    assert layer.lora_a.grad.dtype == torch.bfloat16 and layer.lora_b.grad.shape == (r, N)
    assert max(e_y, e_dx, e_da, e_db) <= TOL


def test_lora_linear_frozen_input_and_merge(dev):
    """No gradient asked for X: only the adapter's are computed. The merged
    layer's weight dequantizes to the oracle's merge of the same adapter."""
    import torch

    K, N, r = 256, 128, 8
    rng = np.random.Generator(np.random.PCG64(77))
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)
    x = workloads.to_bf16_bits(rng.standard_normal((64, K), dtype=np.float32))
    wt, host = upload_weight(w, dev)
    layer = nq.make_lora_linear_module()(wt, r=r, alpha=16.0)
    y = layer(to_dev(x, dev))
    y.float().sum().backward()
    torch.cuda.synchronize()
    assert layer.lora_a.grad is not None and layer.lora_b.grad is not None
    # B = 0: dA = s X^T (dY B^T) = 0 exactly
    assert float(layer.lora_a.grad.abs().max()) == 0.0
    merged = layer.merged()
    a = to_host(layer.lora_a.detach())
    b = to_host(layer.lora_b.detach())
    # (B = 0: the delta is exactly zero, so the merge is a plain re-quantization)
    codes, _, q8, sc, _ = oracle.merge_lora(host["codes"], (N, K), a, b, layer.scale, q=host["q"],
                                            scale=host["scale"])
    assert np.array_equal(to_host(merged.codes), codes)
    assert np.array_equal(to_host(merged.absmax_q), q8)
    assert np.array_equal(to_host(merged.absmax_scale).view(np.uint32), sc.view(np.uint32))
