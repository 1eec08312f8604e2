"""The library's calls under HIP graph capture: they allocate nothing, clear
nothing with memset nodes and take the caller's stream, so a captured storage
step (quantize + dequantize), decode GEMV (the allocation-free forward),
large-M forward and input gradient, adapter gradients and merge replay to the
eager results bit for bit.
Each replay follows eager work that clobbers every output, and is checked on
its own.
"""
import numpy as np
import pytest

import nf4_quantize_amd as nq
import workloads
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch

    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.uint8)


def test_graph_replays_match_eager(dev):
    import torch

    N, K, r = 1024, 4096, 16
    rng = np.random.Generator(np.random.PCG64(31))
    w = to_dev(workloads.to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02)), dev)
    x4 = to_dev(workloads.to_bf16_bits(rng.standard_normal((4, K), dtype=np.float32)), dev)
    X = to_dev(workloads.to_bf16_bits(rng.standard_normal((300, K), dtype=np.float32)), dev)
    dY = to_dev(workloads.to_bf16_bits(rng.standard_normal((300, N), dtype=np.float32)), dev)
    A = to_dev(workloads.to_bf16_bits(rng.standard_normal((K, r), dtype=np.float32) * np.float32(0.05)), dev)
    B = to_dev(workloads.to_bf16_bits(rng.standard_normal((r, N), dtype=np.float32) * np.float32(0.05)), dev)
    ws = torch.empty(nq.nf4_linear_workspace_size(300, r), dtype=torch.uint8, device=dev)
    lws = torch.empty(nq.nf4_lora_backward_workspace_size(300, K, N, r), dtype=torch.uint8, device=dev)
    mws = torch.empty(nq.nf4_merge_lora_workspace_size(N, K), dtype=torch.uint8, device=dev)

    def outputs():
        return dict(t=nq.empty_nf4((N, K), dev), wd=torch.empty_like(w),
                    y4=torch.empty((4, N), dtype=torch.bfloat16, device=dev),
                    Y=torch.empty((300, N), dtype=torch.bfloat16, device=dev),
                    dX=torch.empty((300, K), dtype=torch.bfloat16, device=dev),
                    gA=torch.empty((K, r), dtype=torch.float32, device=dev),
                    gB=torch.empty((r, N), dtype=torch.float32, device=dev),
                    merged=nq.empty_nf4((N, K), dev))

    def work(o):
        nq.quantize(w, out=o["t"])
        nq.dequantize(o["t"], out=o["wd"])
        nq.nf4_linear_forward_noalloc(x4, o["t"], out=o["y4"])
        nq.nf4_linear_forward(X, o["t"], A, B, 2.0, out=o["Y"], workspace=ws)
        nq.nf4_linear_backward_input(dY, o["t"], A, B, 2.0, out=o["dX"], workspace=ws)
        nq.nf4_lora_backward(X, dY, A, B, 2.0, grad_a=o["gA"], grad_b=o["gB"], workspace=lws)
        nq.nf4_merge_lora(o["t"], A, B, 2.0, o["merged"], workspace=mws)

    ref = outputs()
    work(ref)
    torch.cuda.synchronize()

    got = outputs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work(got)  # warm-up on a side stream, as torch asks before a capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        work(got)
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work between replays: clobber every output the graph writes
        for k, v in got.items():
            for part in ((v.codes, v.absmax_q, v.absmax_scale) if k in ("t", "merged") else (v,)):
                part.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"graph replay {rep}")
        for k in ("wd", "y4", "Y", "dX", "gA", "gB"):
            assert torch.equal(_bits(got[k]), _bits(ref[k])), (rep, k)
        for k in ("t", "merged"):
            for part in ("codes", "absmax_q", "absmax_scale"):
                assert torch.equal(_bits(getattr(got[k], part)), _bits(getattr(ref[k], part))), (rep, k, part)
