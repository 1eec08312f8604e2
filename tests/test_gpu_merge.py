"""GPU parity of nf4_merge_lora (merging the adapter into the quantized base and
re-quantizing) against the CPU oracle.

The base storage is made by the oracle, so nothing the oracle reads comes from
the GPU. Two kinds of adapter:
  - dyadic values (k * 2^-6, k * 2^-5 with |k| <= 3, scale 2): every sum over
    the rank is exact in fp32 in any order, so the merged weight and all
    outputs must be bit-exact;
  - Gaussian values: the matrix cores sum the rank in an order of their own,
    so the merged fp32 value may differ from the oracle's (exact sum, one
    rounding) by the fp32 summation bound. Where that interval straddles a
    decision point of the re-quantization, either neighbouring code is a
    correct result; every other code, scale code and scale must match the
    values the oracle derives, and the straddling elements must be rare.
"""
import numpy as np
import pytest

import nf4_quantize_amd as nq
import oracle
from gpu_util import log, to_dev, to_host
from workloads import to_bf16_bits

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def base_storage(seed, N, K, dq=True):
    rng = np.random.Generator(np.random.PCG64(seed))
    w = to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    codes, amax = oracle.quantize(w.ravel())
    if not dq:
        return codes, amax, None, None
    q, sc = oracle.double_quantize(amax)
    return codes, None, q, sc


def to_gpu_tensor(dev, shape, codes, amax, q, sc):
    return nq.NF4Tensor(to_dev(codes, dev), None if amax is None else to_dev(amax, dev),
                        None if q is None else to_dev(q, dev), None if sc is None else to_dev(sc, dev),
                        tuple(shape))


def dyadic(rng, shape, e):
    return to_bf16_bits((rng.integers(-3, 4, size=shape) * 2.0 ** e).astype(np.float32))


def gaussian(rng, shape, sigma):
    return to_bf16_bits(rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma))


def unpack(codes, n):
    return np.stack([codes & 15, codes >> 4], axis=1).ravel()[:n]


def gpu_merge(dev, shape, base, A, B, s, keep_absmax=True, dq=True):
    import torch

    w = to_gpu_tensor(dev, shape, *base)
    out = nq.merge_lora(w, to_dev(A, dev), to_dev(B, dev), s, double_quant=dq,
                        keep_absmax=keep_absmax)
    torch.cuda.synchronize()
    return out


EXACT_CASES = [
    # (N, K, r): one tile; K not a multiple of 256 and ragged N; rank not a
    # multiple of 32; the widest rank; a single row
    (64, 256, 64),
    (100, 320, 8),
    (37, 64, 72),
    (130, 1024, 256),
    (1, 128, 16),
    (200, 2112, 40),
]


@pytest.mark.parametrize("N,K,r", EXACT_CASES)
@pytest.mark.parametrize("dq", [True, False])
def test_merge_exact_adapter_bit_exact(dev, N, K, r, dq):
    log(f"merge exact adapter N={N} K={K} r={r} dq={dq}")
    rng = np.random.Generator(np.random.PCG64(N * 7 + K + r))
    base = base_storage(N + K, N, K, dq)
    A, B = dyadic(rng, (K, r), -6), dyadic(rng, (r, N), -5)
    out = gpu_merge(dev, (N, K), base, A, B, 2.0, keep_absmax=True, dq=dq)
    nc, na, nq8, nsc, _ = oracle.merge_lora(base[0], (N, K), A, B, 2.0, *base[1:], dq=dq)
    assert np.array_equal(to_host(out.codes), nc)
    assert np.array_equal(to_host(out.absmax).view(np.uint32), na.view(np.uint32))
    if dq:
        assert np.array_equal(to_host(out.absmax_q), nq8)
        assert np.array_equal(to_host(out.absmax_scale).view(np.uint32), nsc.view(np.uint32))


def test_merge_zero_adapter_is_identity(dev):
    import torch

    N, K, r = 96, 512, 32
    base = base_storage(4, N, K)
    A = np.zeros((K, r), np.uint16)
    B = gaussian(np.random.Generator(np.random.PCG64(1)), (r, N), 0.1)
    out = gpu_merge(dev, (N, K), base, A, B, 2.0, keep_absmax=False)
    assert np.array_equal(to_host(out.codes), base[0])
    assert np.array_equal(to_host(out.absmax_q), base[2])
    assert np.array_equal(to_host(out.absmax_scale), base[3])
    # in place: the base's own buffers receive the merged weight
    rng = np.random.Generator(np.random.PCG64(2))
    A, B = dyadic(rng, (K, r), -6), dyadic(rng, (r, N), -5)
    w = to_gpu_tensor(dev, (N, K), *base)
    nq.merge_lora(w, to_dev(A, dev), to_dev(B, dev), 2.0, out=w)
    torch.cuda.synchronize()
    nc, _, nq8, nsc, _ = oracle.merge_lora(base[0], (N, K), A, B, 2.0, *base[1:])
    assert np.array_equal(to_host(w.codes), nc)
    assert np.array_equal(to_host(w.absmax_q), nq8)
    assert np.array_equal(to_host(w.absmax_scale), nsc)


def check_valid(out, base, shape, A, B, s, rows, label):
    """Codes, block scales and DQ codes of `rows` (whole DQ groups) against
    the oracle's merged weight and the fp32 summation bound."""
    N, K = shape
    r = A.shape[1]
    wm = oracle.merged_weight(base[0], shape, A, B, s, *base[1:], rows=rows).astype(np.float64)
    af = np.abs(oracle.bf16_to_f32(A).astype(np.float64))
    bf = np.abs(oracle.bf16_to_f32(B).astype(np.float64))
    sab = (af @ bf[:, rows]).T  # sum_j |A[k][j] B[j][n]|, [rows x K]
    delta = 1.01 * abs(s) * (r + 2) * U * sab + 2.0 ** -22 * np.abs(wm) + 1e-37
    nbk = K // 64
    wmb = wm.reshape(len(rows), nbk, 64)
    db = delta.reshape(len(rows), nbk, 64)
    c1 = np.abs(wmb).max(axis=2)
    dc = db.max(axis=2)
    g_c1 = to_host(out.absmax).reshape(N, nbk)[rows]
    assert np.all(np.abs(g_c1 - c1) <= dc), f"{label}: block scales outside the bound"
    # code intervals: w in [wm - d, wm + d], c in [c1 - dc, c1 + dc]
    lo_w, hi_w = wmb - db, wmb + db
    lo_c = np.maximum(c1 - dc, 1e-38)[..., None]
    hi_c = (c1 + dc)[..., None]
    cands = np.stack([lo_w / lo_c, lo_w / hi_c, hi_w / lo_c, hi_w / hi_c])
    lo = cands.min(axis=0) * (1 - 2.0 ** -22) - 2.0 ** -40
    hi = cands.max(axis=0) * (1 + 2.0 ** -22) + 2.0 ** -40
    lo = np.clip(lo, -1.0, 1.0)
    hi = np.clip(hi, -1.0, 1.0)
    code_lo = oracle.nearest_code_array(np.nextafter(lo.astype(np.float32), -2)).reshape(lo.shape)
    code_hi = oracle.nearest_code_array(np.nextafter(hi.astype(np.float32), 2)).reshape(hi.shape)
    g_codes = unpack(to_host(out.codes), N * K).reshape(N, nbk, 64)[rows]
    assert np.all((g_codes >= code_lo) & (g_codes <= code_hi)), f"{label}: codes outside the interval"
    amb = np.mean(code_lo != code_hi)
    # codes that differ from those of the oracle's own merged weight (only
    # possible where the interval straddles a decision point)
    ref_codes = oracle.nearest_code_array(
        (wmb / c1[..., None]).astype(np.float32)).reshape(wmb.shape)
    ref_codes[np.broadcast_to(c1[..., None] == 0, wmb.shape)] = 7
    diff = np.mean(g_codes != ref_codes)
    log(f"  {label}: {np.mean(code_lo == code_hi) * 100:.4f}% of codes decided uniquely "
        f"(straddling: {amb * 100:.4f}%), all valid; {diff * 100:.5f}% differ from the "
        f"oracle's codes of its own merged weight")
    # the straddling share grows with the worst-case bound (r + 2) u
    assert amb < 1e-3 * max(1.0, r / 64)
    # double quantization of whole groups (256 blocks)
    if out.absmax_q is not None:
        flat = np.concatenate([np.arange(rw * nbk, (rw + 1) * nbk) for rw in rows])
        c1f, dcf = c1.ravel(), dc.ravel()
        gq = to_host(out.absmax_q)[flat]
        groups = flat // 256
        ug = np.unique(groups)
        c2 = np.array([c1f[groups == gi].max() for gi in ug])
        dg = np.array([dcf[groups == gi].max() for gi in ug])
        g_c2 = to_host(out.absmax_scale)[ug]
        assert np.all(np.abs(g_c2 - c2) <= dg)
        gi = np.searchsorted(ug, groups)
        rlo = (c1f - dcf) / (c2[gi] + dg[gi]) * (1 - 2.0 ** -22)
        rhi = (c1f + dcf) / np.maximum(c2[gi] - dg[gi], 1e-38) * (1 + 2.0 ** -22)
        qlo = oracle.e4m3_encode(np.clip(rlo, 0, 1).astype(np.float32))
        qhi = oracle.e4m3_encode(np.clip(rhi, 0, 1).astype(np.float32))
        assert np.all((gq >= qlo) & (gq <= qhi)), f"{label}: E4M3 scale codes outside the interval"


@pytest.mark.parametrize("N,K,r", [(128, 2048, 64), (100, 320, 24), (66, 4096, 256)])
def test_merge_gaussian_adapter_valid(dev, N, K, r):
    log(f"merge gaussian adapter N={N} K={K} r={r}")
    rng = np.random.Generator(np.random.PCG64(N + K + r))
    base = base_storage(N * K, N, K)
    # delta comparable to the weights (sigma 0.02): s * sqrt(r) * sa * sb ~ 0.02
    sab = (0.01 / np.sqrt(r)) ** 0.5
    A, B = gaussian(rng, (K, r), sab), gaussian(rng, (r, N), sab)
    out = gpu_merge(dev, (N, K), base, A, B, 2.0, keep_absmax=True)
    check_valid(out, base, (N, K), A, B, 2.0, np.arange(N), f"N={N} K={K} r={r}")


def test_merge_qlora_shape_sampled(dev):
    """W NF4+DQ [8192 x 8192], r = 64, s = 2 (the QLoRA linear's shape): row
    pairs (whole DQ groups of 2 x 128 blocks) against the oracle."""
    N = K = 8192
    r, s = 64, 2.0
    rng = np.random.Generator(np.random.PCG64(7))
    # the whole base is quantized by the oracle on the CPU and uploaded
    w = to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    log("oracle quantize of the 8192 x 8192 base")
    codes, amax = oracle.quantize(w.ravel())
    q, sc = oracle.double_quantize(amax)
    del w, amax
    base = (codes, None, q, sc)
    A, B = gaussian(rng, (K, r), 0.035), gaussian(rng, (r, N), 0.035)
    out = gpu_merge(dev, (N, K), base, A, B, s, keep_absmax=True)
    rows = np.array([0, 1, 2, 3, 1000, 1001, 4096, 4097, 8190, 8191])
    check_valid(out, base, (N, K), A, B, s, rows, "8192 x 8192 r=64")
