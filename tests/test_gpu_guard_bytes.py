"""Guard bytes around every device output of every entry point: each output
(and each workspace) sits between two 4 KiB canary regions, and after the
call every canary byte must be unchanged. The parity tests compare only the
documented ranges, so a store past the end of an output (a partial last
block or group, a ragged tile, the last entry of a batch) shows up here.

Inputs are seeded synthetic tensors; outputs are not compared with the
oracle here (the parity tests do that), only their surroundings.
"""
import numpy as np
import pytest

import nf4_quantize_amd as nq
import workloads
from gpu_util import log, to_dev

pytestmark = pytest.mark.gpu

PAD = 4096
CANARY = 0xA5
SIZES = (1, 2, 63, 64, 65, 1000, 16383, 16384, 16385, 3 * 16384 + 100, 64 * 257 + 7)


class Guarded:
    """Device buffers with canary pads; check() asserts every pad is intact."""

    def __init__(self, dev):
        self.dev = dev
        self.bufs = []

    def empty(self, n, dtype):
        import torch

        if n == 0:
            return None
        nbytes = n * torch.empty((), dtype=dtype).element_size()
        raw = torch.full((PAD + nbytes + (-nbytes) % 256 + PAD,), CANARY, dtype=torch.uint8,
                         device=self.dev)
        self.bufs.append((raw, nbytes))
        return raw[PAD:PAD + nbytes].view(dtype)

    def check(self, what):
        import torch

        torch.cuda.synchronize()
        for i, (raw, nbytes) in enumerate(self.bufs):
            h = raw.cpu().numpy()
            bad = np.count_nonzero(h[:PAD] != CANARY) + np.count_nonzero(h[PAD + nbytes:] != CANARY)
            assert bad == 0, f"{what}: buffer {i} ({nbytes} B): {bad} guard bytes overwritten"
        self.bufs.clear()


def nblocks(n, b=64):
    return (n + b - 1) // b


def storage(g, n, dq=True, keep_absmax=False, fmt=None):
    """An NF4Tensor whose buffers are all guarded."""
    import torch

    fmt = fmt or nq.NF4Format()
    nb = fmt.nblocks(n)
    return nq.NF4Tensor(g.empty((n + 1) // 2, torch.uint8),
                        g.empty(nb, torch.float32) if (keep_absmax or not dq) else None,
                        g.empty(nb, torch.uint8) if dq else None,
                        g.empty(fmt.ngroups(n), torch.float32) if dq else None, (n,), fmt=fmt,
                        absmax_offset=g.empty(1, torch.float32) if (dq and fmt.mean_offset) else None)


def weights(n, dtype, seed):
    w = workloads.gaussian_f32(seed, n, 0.02)
    return workloads.to_bf16_bits(w) if dtype == "bf16" else w


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_storage_path_guard_bytes(dev, dtype):
    import torch

    g = Guarded(dev)
    for n in SIZES:
        log(f"guard bytes: quantize / dequantize n={n} {dtype}")
        w = to_dev(weights(n, dtype, n), dev)
        for dq, keep in ((True, False), (True, True), (False, True)):
            t = storage(g, n, dq, keep)
            nq.nf4_quantize(w, t.codes, t.absmax, t.absmax_q, t.absmax_scale)
            for odt in (torch.float32, torch.bfloat16):
                out = g.empty(n, odt)
                nq.dequantize(t, out_dtype=odt, out=out)
            g.check(f"quantize/dequantize n={n} dq={dq} keep={keep}")
        amax = to_dev(np.abs(workloads.gaussian_f32(n + 1, nblocks(n), 0.05)), dev)
        q8, sc = g.empty(nblocks(n), torch.uint8), g.empty(nblocks(nblocks(n), 256), torch.float32)
        nq.nf4_double_quantize(amax, q8, sc)
        g.check(f"double_quantize nblocks={nblocks(n)}")


FORMATS = [
    nq.NF4Format(16, 64, "linear8", False),
    nq.NF4Format(128, 256, "e5m2", True),
    nq.NF4Format(1024, 4, "e4m3", True),
    nq.NF4Format(64, 256, "e4m3", False, "fp4"),
]


@pytest.mark.parametrize("fi", range(len(FORMATS)))
def test_format_variants_guard_bytes(dev, fi):
    import torch

    f = FORMATS[fi]
    g = Guarded(dev)
    for n in (1, 65, 16385, 3 * 16384 + 100, 5 * 1024 + 3):
        log(f"guard bytes: format {f} n={n}")
        w = to_dev(weights(n, "bf16", n + 7), dev)
        t = storage(g, n, True, True, fmt=f)
        ws = g.empty(max(1, nq.nf4_quantize_ex_workspace_size(n, f)), torch.uint8)
        nq.nf4_quantize_ex(w, f, t.codes, t.absmax, t.absmax_q, t.absmax_scale, t.absmax_offset,
                           workspace=ws)
        for odt in (torch.float32, torch.bfloat16):
            out = g.empty(n, odt)
            nq.nf4_dequantize_ex(t.codes, n, f, out, None, t.absmax_q, t.absmax_scale,
                                 t.absmax_offset)
        nb = f.nblocks(n)
        q, sc = g.empty(nb, torch.uint8), g.empty(f.ngroups(n), torch.float32)
        off = g.empty(1, torch.float32) if f.mean_offset else None
        ws = g.empty(max(1, nq.nf4_double_quantize_ex_workspace_size(nb, f)), torch.uint8)
        nq.nf4_double_quantize_ex(t.absmax, f, q, sc, off, workspace=ws)
        g.check(f"format {f} n={n}")


def test_batched_guard_bytes(dev):
    import torch

    g = Guarded(dev)
    sizes = [16384 * 3, 100, 16385, 64, 7 * 16384 + 1000, 1, 16384]
    sizes = sizes * 5  # 35 entries: two launches of entries, plus the tail launch
    ws = [to_dev(weights(n, "bf16", 50 + i), dev) for i, n in enumerate(sizes)]
    log(f"guard bytes: batched, {len(sizes)} entries")
    ts = [storage(g, n, dq=(i % 3 != 2), keep_absmax=(i % 3 == 2)) for i, n in enumerate(sizes)]
    nq.nf4_quantize_batched(ws, ts)
    outs = [g.empty(n, torch.bfloat16) for n in sizes]
    nq.nf4_dequantize_batched(ts, outs)
    g.check("batched")


LINEAR_SHAPES = [
    # m, N, K, r: decode GEMV, the fused GEMM kernels, the portable path
    (1, 320, 512, 0),
    (16, 192, 2048, 0),
    (3, 16 * 5 + 7, 4096, 0),   # the LDS-staged decode kernel, ragged last tile
    (2, 50, 8192, 0),
    (37, 320, 512, 8),
    (300, 256, 256, 16),
    (17, 64, 64, 0),
    (257, 576, 640, 64),
    (5, 100, 128, 3),
]


@pytest.mark.parametrize("shape", LINEAR_SHAPES)
def test_linear_guard_bytes(dev, shape):
    import torch

    m, N, K, r = shape
    log(f"guard bytes: linear m={m} N={N} K={K} r={r}")
    g = Guarded(dev)
    rng = np.random.Generator(np.random.PCG64(m * 7 + N))
    wt = nq.quantize(to_dev(weights(N * K, "bf16", N + K), dev), double_quant=True)
    wt = nq.NF4Tensor(wt.codes, None, wt.absmax_q, wt.absmax_scale, (N, K))
    x = to_dev(workloads.to_bf16_bits(rng.standard_normal((m, K), dtype=np.float32)), dev)
    dy = to_dev(workloads.to_bf16_bits(rng.standard_normal((m, N), dtype=np.float32)), dev)
    a = b = None
    if r:
        a = to_dev(workloads.to_bf16_bits(rng.standard_normal((K, r), dtype=np.float32) * 0.01), dev)
        b = to_dev(workloads.to_bf16_bits(rng.standard_normal((r, N), dtype=np.float32) * 0.01), dev)
    wsb = nq.nf4_linear_workspace_size(m, r)
    y = g.empty(m * N, torch.bfloat16).view(m, N)
    nq.linear_forward(x, wt, a, b, 2.0, out=y, workspace=g.empty(max(wsb, 1), torch.uint8))
    dx = g.empty(m * K, torch.bfloat16).view(m, K)
    nq.linear_backward_input(dy, wt, a, b, 2.0, out=dx,
                             workspace=g.empty(max(wsb, 1), torch.uint8))
    g.check(f"linear {shape}")
    if r and r % 8 == 0:
        for gdt in (torch.float32, torch.bfloat16):
            ga, gb = g.empty(K * r, gdt).view(K, r), g.empty(r * N, gdt).view(r, N)
            lw = nq.nf4_lora_backward_workspace_size(m, K, N, r)
            nq.lora_backward(x, dy, a, b, 2.0, grad_dtype=gdt, grad_a=ga, grad_b=gb,
                             workspace=g.empty(max(lw, 1), torch.uint8))
        g.check(f"lora_backward {shape}")
        for dq in (True, False):
            out = storage(g, N * K, dq=dq, keep_absmax=not dq)
            out = nq.NF4Tensor(out.codes, out.absmax, out.absmax_q, out.absmax_scale, (N, K))
            mw = nq.nf4_merge_lora_workspace_size(N, K)
            nq.nf4_merge_lora(wt, a, b, 2.0, out, workspace=g.empty(max(mw, 1), torch.uint8))
        g.check(f"merge {shape}")
