"""GPU parity of the storage-format variants (nf4_quantize_ex,
nf4_double_quantize_ex, nf4_dequantize_ex) against the CPU oracle: block
sizes 16..4096, DQ blocks 1..4096, E4M3 / E5M2 / linear 8-bit scale codes,
with and without the tensor-wide mean offset. Everything is integer or
decided in fp32 on both sides, so every output is compared bit for bit.

Inputs are seeded synthetic tensors; nothing the oracle reads comes from the
GPU.
"""
import numpy as np
import pytest

import nf4_quantize_amd as nq
import oracle
import workloads
from gpu_util import log, to_dev, to_host

pytestmark = pytest.mark.gpu

FMTS = ("e4m3", "e5m2", "linear8")


def nan_equal(a, b):
    a = np.asarray(a)
    b = np.asarray(b)
    na, nb_ = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb_) and np.array_equal(a[~na].view(np.uint32), b[~nb_].view(np.uint32))


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("off", [False, True])
def test_scale_decode_all_codes(dev, fmt, off):
    """Every 8-bit code through the variant dequantizer (level 15 = 1.0, group
    value 1.0, mu = 0): the hardware converts (fp8 / bf8) and the integer
    decode against the oracle's decode, NaN and infinity codes included."""
    import torch

    bs = 16
    n = 256 * bs
    f = nq.NF4Format(bs, 256, fmt, off)
    codes = torch.full((n // 2,), 0xFF, dtype=torch.uint8, device=dev)
    q = torch.arange(256, dtype=torch.uint8, device=dev)
    sc = torch.ones(1, dtype=torch.float32, device=dev)
    mu = torch.zeros(1, dtype=torch.float32, device=dev)
    out = torch.empty(n, dtype=torch.float32, device=dev)
    nq.nf4_dequantize_ex(codes, n, f, out, absmax_q=q, absmax_scale=sc,
                         absmax_offset=mu if off else None)
    torch.cuda.synchronize()
    got = to_host(out)[::bs]
    want = oracle.block_scales_ex(256, 256, fmt, q=np.arange(256, dtype=np.uint8),
                                  scale=np.ones(1, np.float32),
                                  offset=np.float32(0) if off else None)
    assert nan_equal(got, want)


def make_weights(seed, n, dtype, bs):
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.standard_normal(n, dtype=np.float32) * np.float32(workloads.SIGMA_W)
    idx = rng.choice(n, size=max(1, n // 1000), replace=False)
    w[idx] *= 10  # outliers
    w[: min(n, bs)] = 0.0  # an all-zero block
    return workloads.to_bf16_bits(w) if dtype == "bf16" else w


def check_variant(dev, w, f, keep_absmax=True, label=""):
    import torch

    n = w.size
    log(f"format parity {label}: n={n} {w.dtype} B1={f.blocksize} B2={f.dq_blocksize} "
        f"{f.dq_format} offset={f.mean_offset} absmax={keep_absmax}")
    t = nq.quantize(to_dev(w, dev), keep_absmax=keep_absmax, fmt=f)
    torch.cuda.synchronize()
    codes, amax = oracle.quantize_bs(w, f.blocksize)
    q, sc, mu = oracle.double_quantize_ex(amax, f.dq_blocksize, f.dq_format, f.mean_offset)
    assert np.array_equal(to_host(t.codes), codes), "codes differ"
    if keep_absmax:
        assert np.array_equal(to_host(t.absmax), amax), "absmax differs"
    assert np.array_equal(to_host(t.absmax_q), q), "8-bit scale codes differ"
    assert np.array_equal(to_host(t.absmax_scale).view(np.uint32), sc.view(np.uint32)), \
        "group values differ"
    if f.mean_offset:
        assert to_host(t.absmax_offset)[0].view(np.uint32) == np.float32(mu).view(np.uint32), \
            "mean offset differs"
    for odt, oname in ((torch.float32, oracle.F32), (torch.bfloat16, oracle.BF16)):
        out = nq.dequantize(t, out_dtype=odt)
        torch.cuda.synchronize()
        ref = oracle.dequantize_ex(codes, n, f.blocksize, f.dq_blocksize, f.dq_format, q=q,
                                   scale=sc, offset=mu, out_dtype=oname)
        got = to_host(out).ravel()
        assert np.array_equal(got.view(np.uint32) if odt == torch.float32 else got,
                              ref.view(np.uint32) if odt == torch.float32 else ref), \
            f"dequantized {odt} differs"
    # without double quantization: codes + absmax, dequantized from absmax
    if keep_absmax:
        t2 = nq.quantize(to_dev(w, dev), double_quant=False, fmt=f)
        out = nq.dequantize(t2, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert np.array_equal(to_host(t2.codes), codes)
        assert np.array_equal(to_host(t2.absmax), amax)
        ref = oracle.dequantize_ex(codes, n, f.blocksize, absmax=amax)
        assert np.array_equal(to_host(out).view(np.uint32), ref.view(np.uint32))


CASES = [
    # (B1, B2, format, mean offset)
    (64, 256, "e5m2", False),
    (64, 256, "linear8", False),
    (64, 256, "e4m3", True),
    (64, 256, "e5m2", True),
    (64, 256, "linear8", True),
    (16, 256, "e4m3", False),
    (32, 64, "e5m2", True),
    (128, 256, "e4m3", False),
    (128, 1, "linear8", True),
    (256, 16, "e4m3", True),
    (512, 4096, "e5m2", False),
    (1024, 2, "linear8", False),
    (2048, 128, "e4m3", True),
    (4096, 256, "linear8", True),
    (64, 32, "e4m3", False),
    (64, 1024, "e4m3", False),
]


@pytest.mark.parametrize("bs,dqb,fmt,off", CASES)
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_variant_parity(dev, bs, dqb, fmt, off, dtype):
    f = nq.NF4Format(bs, dqb, fmt, off)
    # several full units and groups plus a ragged tail (odd n: a half byte)
    n = 3 * max(16384, 4 * bs) + 2 * bs + 7
    check_variant(dev, make_weights(bs + dqb + len(fmt), n, dtype, bs), f, label="ragged")


@pytest.mark.parametrize("n", [1, 2, 15, 17, 64, 4095, 4096, 16384 + 3])
@pytest.mark.parametrize("bs", [16, 64, 512, 4096])
def test_variant_small_sizes(dev, n, bs):
    f = nq.NF4Format(bs, 4, "e5m2", True)
    check_variant(dev, make_weights(n, n, "bf16", bs), f, label="small")


def test_variant_workspace_path(dev):
    """Two-pass formats without an absmax output keep the block scales in the
    workspace."""
    for f in (nq.NF4Format(128, 256, "e4m3", False), nq.NF4Format(64, 256, "linear8", True)):
        check_variant(dev, make_weights(3, 70000, "bf16", f.blocksize), f, keep_absmax=False,
                      label="workspace")


def test_default_format_through_ex_matches(dev):
    """nf4_quantize_ex with {64, 256, E4M3, no offset} computes nf4_quantize."""
    import torch

    w = to_dev(make_weights(9, 100003, "bf16", 64), dev)
    f = nq.NF4Format()
    a = nq.quantize(w, keep_absmax=True)
    codes = torch.empty_like(a.codes)
    am = torch.empty_like(a.absmax)
    q = torch.empty_like(a.absmax_q)
    sc = torch.empty_like(a.absmax_scale)
    nq.nf4_quantize_ex(w, f, codes, am, q, sc)
    out = torch.empty(w.numel(), dtype=torch.bfloat16, device=dev)
    nq.nf4_dequantize_ex(codes, w.numel(), f, out, absmax_q=q, absmax_scale=sc)
    ref = nq.dequantize(a)
    torch.cuda.synchronize()
    for x, y in ((codes, a.codes), (am, a.absmax), (q, a.absmax_q), (sc, a.absmax_scale),
                 (out, ref.ravel())):
        assert torch.equal(x, y)


@pytest.mark.parametrize("nblocks", [1, 4096, 5000, 4096 * 4096 + 77])
def test_double_quantize_ex_mean_levels(dev, nblocks):
    """The mean offset over one, two and three levels of the pairwise sum."""
    import torch

    rng = np.random.Generator(np.random.PCG64(nblocks))
    amax = np.abs(rng.standard_normal(nblocks, dtype=np.float32)) + np.float32(0.5)
    for fmt in ("e4m3", "linear8"):
        f = nq.NF4Format(64, 256, fmt, True)
        log(f"double_quantize_ex nblocks={nblocks} {fmt} offset")
        q, sc, off = nq.double_quantize(to_dev(amax, dev), fmt=f)
        torch.cuda.synchronize()
        rq, rsc, rmu = oracle.double_quantize_ex(amax, 256, fmt, True)
        assert to_host(off)[0].view(np.uint32) == np.float32(rmu).view(np.uint32)
        assert np.array_equal(to_host(q), rq)
        assert np.array_equal(to_host(sc).view(np.uint32), rsc.view(np.uint32))


def test_variant_mlp_shape(dev):
    """11008 x 4096 bf16 with outliers (the MLP weight) in a variant format, all
    outputs compared in full."""
    w = workloads.weight_mlp_outliers_bf16()
    check_variant(dev, w.ravel(), nq.NF4Format(128, 256, "e5m2", True), label="mlp")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dqb", [1, 8, 64, 256, 4096])
def test_double_quantize_ex_standalone(dev, fmt, dqb):
    """nf4_double_quantize_ex on existing fp32 block scales (no mean offset),
    including a ragged last group and zero scales."""
    import torch

    rng = np.random.Generator(np.random.PCG64(dqb + len(fmt)))
    nb = 3 * max(dqb, 64) + 37
    amax = np.abs(rng.standard_normal(nb, dtype=np.float32)) * np.float32(0.05)
    amax[:5] = 0.0
    f = nq.NF4Format(64, dqb, fmt, False)
    q, sc = nq.double_quantize(to_dev(amax, dev), fmt=f)
    torch.cuda.synchronize()
    rq, rsc, _ = oracle.double_quantize_ex(amax, dqb, fmt, False)
    assert np.array_equal(to_host(q), rq)
    assert np.array_equal(to_host(sc).view(np.uint32), rsc.view(np.uint32))
