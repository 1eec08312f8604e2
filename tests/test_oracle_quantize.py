"""Pins of the oracle's blockwise quantization, double quantization, FP8 codec,
bf16 rounding and dequantization (CPU only).

Sources: "QLoRA: Mathematical Foundations of 4-Bit NormalFloat Quantization,
Double Quantization, and Paged Optimizers", sections "Block-Wise Quantization
Mechanics" (c1, argmin, reconstruction) and "Double Quantization (DQ)" (c2 and
the 8-bit code of c1/c2); "QLoRA in Production: 4-bit NormalFloat & Double
Quantization Deep Dive", the uniform-vs-NF4 toy comparison.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from workloads import gaussian_f32


def unpack(codes, n):
    lo = codes & 15
    hi = codes >> 4
    return np.stack([lo, hi], axis=1).ravel()[:n]


def brute_quantize(w32):
    """Brute force in numpy float32: per 64-block max|w|, w/c1, first argmin."""
    q = None
    import oracle

    q = oracle.codebook()
    n = w32.size
    out = np.zeros(n, np.uint8)
    absmax = []
    for b in range(0, n, 64):
        blk = w32[b:b + 64]
        c1 = np.max(np.abs(blk))
        absmax.append(c1)
        if c1 == 0:
            out[b:b + 64] = 7
            continue
        nrm = (blk / c1).astype(np.float32)
        out[b:b + blk.size] = np.argmin(np.abs(nrm[:, None] - q[None, :]), axis=1)
    return out, np.array(absmax, np.float32)


@pytest.mark.parametrize("n", [1, 2, 63, 64, 65, 127, 128, 1000, 4097])
def test_quantize_matches_brute_force(oracle_mod, n):
    w = gaussian_f32(100 + n, n, 0.02)
    codes, absmax = oracle_mod.quantize(w)
    want, want_absmax = brute_quantize(w)
    assert codes.size == (n + 1) // 2
    assert np.array_equal(unpack(codes, n), want)
    assert np.array_equal(absmax, want_absmax)
    if n % 2:
        assert codes[-1] >> 4 == 0  # odd n: last high nibble is zero


def test_quantize_bf16_input_is_widened_exactly(oracle_mod):
    w = gaussian_f32(7, 4096, 0.02)
    bits = torch.from_numpy(w).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    widened = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    c_bf, a_bf = oracle_mod.quantize(bits)
    c_32, a_32 = oracle_mod.quantize(widened)
    assert np.array_equal(c_bf, c_32) and np.array_equal(a_bf, a_32)


def test_absmax_is_block_max(oracle_mod):
    w = gaussian_f32(8, (37, 64 * 5), 1.0).ravel()
    _, absmax = oracle_mod.quantize(w)
    assert np.array_equal(absmax, np.abs(w).reshape(-1, 64).max(axis=1))


def test_special_blocks(oracle_mod):
    # all-zero block -> code 7 everywhere, c1 = 0
    z = np.zeros(64, np.float32)
    codes, absmax = oracle_mod.quantize(z)
    assert absmax[0] == 0 and np.all(unpack(codes, 64) == 7)
    # negative zeros as well
    codes, absmax = oracle_mod.quantize(-z)
    assert np.all(unpack(codes, 64) == 7)
    # single non-zero element -> 0 or 15, all others 7
    for sign, code in ((1.0, 15), (-1.0, 0)):
        w = np.zeros(64, np.float32)
        w[17] = sign * 0.3
        c = unpack(oracle_mod.quantize(w)[0], 64)
        assert c[17] == code and np.all(np.delete(c, 17) == 7)
    # elements at +-c1 map to the end levels
    w = np.array([0.5, -0.5] + [0.1] * 62, np.float32)
    c = unpack(oracle_mod.quantize(w)[0], 64)
    assert c[0] == 15 and c[1] == 0
    # tiny (subnormal) blocks are quantized like any other scale
    w = (gaussian_f32(9, 64, 1.0) * np.float32(1e-39)).astype(np.float32)
    c, a = oracle_mod.quantize(w)
    want, _ = brute_quantize(w)
    assert np.array_equal(unpack(c, 64), want)


def test_non_finite_rejected(oracle_mod):
    w = np.zeros(64, np.float32)
    w[3] = np.inf
    with pytest.raises(ValueError):
        oracle_mod.quantize(w)


# ---------------------------------------------------------------- FP8 E4M3FN

def test_e4m3_decode_matches_library(oracle_mod):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle_mod.e4m3_decode(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    both_nan = np.isnan(ours) & np.isnan(lib)
    assert np.all(both_nan | (ours == lib))
    assert oracle_mod.e4m3_decode([0x38])[0] == 1.0
    assert oracle_mod.e4m3_decode([0x7E])[0] == 448.0
    assert oracle_mod.e4m3_decode([0x01])[0] == 2.0 ** -9


def test_e4m3_encode_exhaustive_on_unit_interval(oracle_mod):
    """Every binary32 r in [0, 1] (about 1.07e9 values) against torch's CPU
    float8_e4m3fn cast (round to nearest even)."""
    chunk = 1 << 24
    spans = [(s, min(s + chunk, 0x3F800001)) for s in range(0, 0x3F800001, chunk)]

    def run(span):
        r = np.arange(span[0], span[1], dtype=np.uint32).view(np.float32)
        ours = oracle_mod.e4m3_encode(r)
        lib = torch.from_numpy(r).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        return int(np.count_nonzero(ours != lib))

    with ThreadPoolExecutor(max_workers=8) as ex:
        bad = sum(ex.map(run, spans))
    assert bad == 0


def test_e4m3_brute_force_nearest(oracle_mod):
    """Nearest of the 127 non-negative finite codes, ties to the even code, on
    values at and around every midpoint."""
    vals = oracle_mod.e4m3_decode(np.arange(127, dtype=np.uint8)).astype(np.float64)
    mids = (vals[:-1] + vals[1:]) / 2
    probe = []
    for m in mids[vals[1:] <= 1.0]:
        m32 = np.float32(m)
        probe += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(2))]
    probe = np.array(probe, np.float32)
    ours = oracle_mod.e4m3_encode(probe)
    d = np.abs(probe.astype(np.float64)[:, None] - vals[None, :])
    best = d.min(axis=1, keepdims=True)
    cands = d == best
    for i in range(probe.size):
        idx = np.nonzero(cands[i])[0]
        want = idx[0] if idx.size == 1 else idx[np.argmax(idx % 2 == 0)]
        assert ours[i] == want, (probe[i], ours[i], idx)


# ---------------------------------------------------------------- bf16

def test_bf16_rounding_matches_library(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(21))
    bits = rng.integers(0, 1 << 32, 4_000_000, dtype=np.uint64).astype(np.uint32)
    # force a share of exact halfway patterns and their neighbours
    bits[:100_000] = (bits[:100_000] & 0xFFFF0000) | 0x8000
    bits[100_000:200_000] = (bits[100_000:200_000] & 0xFFFF0000) | 0x7FFF
    x = bits.view(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < 3.0e38)]
    ours = oracle_mod.f32_to_bf16(x)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, lib)


# ---------------------------------------------------------------- DQ

def test_double_quantize_against_definition(oracle_mod):
    w = gaussian_f32(31, 64 * 256 * 3 + 64 * 17, 0.02)
    _, absmax = oracle_mod.quantize(w)
    q, scale = oracle_mod.double_quantize(absmax)
    nb = absmax.size
    assert q.size == nb and scale.size == (nb + 255) // 256
    for g in range(scale.size):
        grp = absmax[g * 256:(g + 1) * 256]
        assert scale[g] == np.max(np.abs(grp))  # c2 = max |c1| of the group
        ratio = (grp / scale[g]).astype(np.float32)  # correctly rounded fp32 division
        lib = torch.from_numpy(ratio).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q[g * 256:(g + 1) * 256], lib)
    assert q.max() <= 0x38  # ratios are in [0, 1]


def test_fp8_encoders_on_signed_values(oracle_mod):
    """Negative ratios and -0 against torch's CPU float8_e4m3fn and
    float8_e5m2 casts (round to nearest even, sign of zero kept): the sign
    bit on the magnitude's code."""
    rng = np.random.Generator(np.random.PCG64(17))
    r = -np.abs(rng.standard_normal(200000).astype(np.float32))
    r[::3] *= np.float32(1e-3)
    r[::7] *= np.float32(1e-6)                 # rounds to -0
    r[:4] = [-0.0, -1.0, -2.0 ** -10, -2.0 ** -17]
    r = np.concatenate([r, -r]).astype(np.float32)
    for enc, dt in ((oracle_mod.e4m3_encode, torch.float8_e4m3fn),
                    (oracle_mod.e5m2_encode, torch.float8_e5m2)):
        lib = torch.from_numpy(r).to(dt).view(torch.uint8).numpy()
        assert np.array_equal(enc(r), lib), dt
    assert oracle_mod.e4m3_encode(np.float32([-0.0]))[0] == 0x80


def test_double_quantize_signed_scales(oracle_mod):
    """c2 = max |c1| of the group; a negative c1 is the signed E4M3 code of
    fl32(c1 / c2) (torch's cast); the unsigned linear code rejects it."""
    rng = np.random.Generator(np.random.PCG64(18))
    a = (rng.standard_normal(700) * 0.05).astype(np.float32)
    a[::4] = -0.0
    q, scale = oracle_mod.double_quantize(a)
    for g in range(scale.size):
        grp = a[g * 256:(g + 1) * 256]
        assert scale[g] == np.max(np.abs(grp))
        lib = torch.from_numpy((grp / scale[g]).astype(np.float32)).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(q[g * 256:(g + 1) * 256], lib)
    with pytest.raises(Exception):
        oracle_mod.double_quantize_ex(a, 256, "linear8", False)
    oracle_mod.double_quantize_ex(np.abs(a), 256, "linear8", False)


def test_double_quantize_zero_group(oracle_mod):
    absmax = np.zeros(300, np.float32)
    absmax[260] = 0.5
    q, scale = oracle_mod.double_quantize(absmax)
    assert scale[0] == 0 and np.all(q[:256] == 0)
    assert scale[1] == 0.5 and q[260] == 0x38 and np.all(np.delete(q[256:], 4) == 0)


# ---------------------------------------------------------------- dequant

def test_dequantize_values_and_error_bound(oracle_mod):
    w = gaussian_f32(41, 64 * 512 + 33, 0.02)
    n = w.size
    codes, absmax = oracle_mod.quantize(w)
    deq = oracle_mod.dequantize(codes, n, absmax=absmax)
    q = oracle_mod.codebook()
    c = unpack(codes, n)
    blk_scale = np.repeat(absmax, 64)[:n]
    # the reconstruction is the product q[code] * c1, one fp32 rounding
    prod = q[c].astype(np.float64) * blk_scale.astype(np.float64)
    assert np.all(np.abs(deq - prod) <= np.spacing(np.abs(deq).astype(np.float32)) * 0.5 + 0)
    # error bound: at most half of the widest gap (q1 - q0) times c1
    half_gap = (q[1] - q[0]) / 2.0
    assert np.all(np.abs(w - deq) <= half_gap * blk_scale * (1 + 1e-6))
    # re-quantizing the reconstruction gives the same codes (absmax is kept)
    codes2, absmax2 = oracle_mod.quantize(deq)
    assert np.array_equal(absmax2, absmax)
    assert np.array_equal(codes2, codes)


def test_dequantize_dq_scale_error(oracle_mod):
    w = gaussian_f32(42, 64 * 256 * 4, 0.02)
    n = w.size
    codes, absmax = oracle_mod.quantize(w)
    q8, scale = oracle_mod.double_quantize(absmax)
    deq = oracle_mod.dequantize(codes, n, q=q8, scale=scale)
    ref = oracle_mod.dequantize(codes, n, absmax=absmax)
    # E4M3 keeps 3 mantissa bits: the reconstructed c1 is within 2^-4 relative
    # in the normal range, so every weight is too.
    rel = np.abs(deq - ref) / np.maximum(np.abs(ref), 1e-30)
    nz = ref != 0
    assert np.max(rel[nz]) <= 2.0 ** -4 * (1 + 1e-6)
    # c1' = decode(code8) * c2, as exact product of the library-decoded FP8 value
    dec = torch.from_numpy(q8).view(torch.float8_e4m3fn).float().numpy()
    c1p = (dec * np.repeat(scale, 256)[:dec.size]).astype(np.float32)
    for b in [0, 5, 300, 1023]:
        assert oracle_mod.lib().nf4ref_block_scale(
            b, None, q8.ctypes.data, scale.ctypes.data) == c1p[b]


def test_dequantize_bf16_is_rne_of_fp32(oracle_mod):
    w = gaussian_f32(43, 64 * 256 * 2 + 100, 0.02)
    n = w.size
    codes, absmax = oracle_mod.quantize(w)
    q8, scale = oracle_mod.double_quantize(absmax)
    f32 = oracle_mod.dequantize(codes, n, q=q8, scale=scale)
    b16 = oracle_mod.dequantize(codes, n, q=q8, scale=scale, out_dtype=oracle_mod.BF16)
    lib = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b16, lib)


def test_nf4_mse_below_uniform_4bit(oracle_mod):
    """The production blog's toy claim: on Gaussian data the NF4 codebook has a
    lower mean squared error than the uniform 4-bit absmax grid (levels
    (k + 1/2)/7.5). Both blockwise with the same 64-element absmax."""
    w = gaussian_f32(44, 64 * 4096, 0.02)
    codes, absmax = oracle_mod.quantize(w)
    nf4 = oracle_mod.dequantize(codes, w.size, absmax=absmax)
    blk = w.reshape(-1, 64).astype(np.float64)
    am = np.abs(blk).max(axis=1, keepdims=True)
    s = np.round(blk / am * 7.5 - 0.5)
    uni = ((s + 0.5) * am / 7.5).ravel()
    mse_nf4 = np.mean((w - nf4) ** 2)
    mse_uni = np.mean((w - uni) ** 2)
    assert mse_nf4 < mse_uni


def test_dequantize_range_equals_slice(oracle_mod):
    w = gaussian_f32(45, 64 * 256 * 3 + 50, 0.02)
    n = w.size
    codes, absmax = oracle_mod.quantize(w)
    q8, scale = oracle_mod.double_quantize(absmax)
    full = oracle_mod.dequantize(codes, n, q=q8, scale=scale)
    for start, count in [(0, 7), (16383, 3), (20000, 16384), (n - 9, 9)]:
        part = oracle_mod.dequantize_range(codes, n, start, count, q=q8, scale=scale)
        assert np.array_equal(part, full[start:start + count])
    rows = oracle_mod.dequantize_rows(codes, (n // 50, 50), [0, 3, 100], q=q8, scale=scale)
    assert np.array_equal(rows[1], full[150:200])
