"""Pins of the oracle's storage-format variants (CPU only): block sizes other
than 64 ("QLoRA: Mathematical Foundations ...", "Block-Wise Quantization
Mechanics": 64 is the typical size), the 8-bit code formats of double
quantization and its mean offset ("Double Quantization (DQ)": an 8-bit float
format that the page does not name, with an asymmetric bias / mean
subtraction in the prose).

Each pin comes from outside the oracle: numpy's IEEE half precision (E5M2 is
the upper byte of binary16), brute-force nearest-value searches in exact
arithmetic, numpy group maxima, closed forms of two-valued inputs, and sums
that are exact.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from workloads import to_bf16_bits


def unpack(codes, n):
    return np.stack([codes & 15, codes >> 4], axis=1).ravel()[:n]


def e5m2_from_half(c):
    """E5M2 code c as the binary16 whose upper byte is c (numpy's decoding)."""
    return (np.asarray(c, np.uint16) << 8).view(np.float16).astype(np.float32)


# ---- E5M2 ----

def test_e5m2_decode_is_the_upper_byte_of_binary16(oracle_mod):
    codes = np.arange(256)
    got = oracle_mod.e5m2_decode(codes)
    want = e5m2_from_half(codes)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert got[0x7B] == 57344.0 and np.isinf(got[0x7C])


def brute_e5m2(r):
    """Nearest finite E5M2 value by exhaustive search in exact arithmetic;
    on a tie the code with an even mantissa (even code) wins."""
    vals = e5m2_from_half(np.arange(256))
    best, best_d = None, None
    for c in range(256):
        v = vals[c]
        if not np.isfinite(v):
            continue
        if (v < 0) != (r < 0) and v != 0:
            continue
        d = abs(Fraction(float(r)) - Fraction(float(v)))
        if best is None or d < best_d or (d == best_d and c % 2 == 0 and best % 2 == 1):
            best, best_d = c, d
    return best


def test_e5m2_encode_is_the_nearest_value(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(5))
    vals = e5m2_from_half(np.arange(0, 0x3D))  # every code of [0, 1] and one above
    mids = (vals[:-1].astype(np.float64) + vals[1:]) / 2
    r = np.concatenate([
        rng.uniform(-1, 1, 300), rng.uniform(0, 2.0 ** -13, 100),
        mids, np.nextafter(mids.astype(np.float32), 2), np.nextafter(mids.astype(np.float32), -2),
        vals, -vals[1:],
    ]).astype(np.float32)
    got = oracle_mod.e5m2_encode(r)
    for x, c in zip(r, got):
        want = brute_e5m2(x)
        if x < 0 and (want & 0x7F) == 0:
            want = 0x80  # a negative value that rounds to zero keeps its sign
        assert c == want, (float(x), int(c), want)


def test_e5m2_round_trip(oracle_mod):
    vals = e5m2_from_half(np.arange(256))
    finite = np.isfinite(vals) & ~((np.arange(256) == 0x80))
    codes = np.arange(256)[finite]
    assert np.array_equal(oracle_mod.e5m2_encode(vals[finite]), codes)


# ---- pairwise sum ----

def test_pairwise_sum_tree_shape(oracle_mod):
    # 2^24 + 1 rounds back to 2^24 (tie to even) while 1 + 1 is exact: the
    # pairwise tree gives 2^24 + 2, a left-to-right sum would give 2^24.
    assert oracle_mod.pairwise_sum(np.array([2 ** 24, 1, 1, 1], np.float32)) == 2 ** 24 + 2
    # five values: padded to eight, ((2^24+1) + (1+1)) + ((1+0) + 0) = (2^24+2) + 1,
    # a tie between 2^24+2 and 2^24+4 that goes to the even significand
    assert oracle_mod.pairwise_sum(np.array([2 ** 24, 1, 1, 1, 1], np.float32)) == 2 ** 24 + 4
    assert oracle_mod.pairwise_sum(np.array([], np.float32)) == 0.0
    assert oracle_mod.pairwise_sum(np.array([3.5], np.float32)) == 3.5


@pytest.mark.parametrize("n", [1, 2, 3, 7, 64, 255, 256, 1000, 4097])
def test_pairwise_sum_exact_cases(oracle_mod, n):
    rng = np.random.Generator(np.random.PCG64(n))
    # small integers times a common power of two: every partial sum is exact
    x = (rng.integers(0, 1000, n) * 2.0 ** -7).astype(np.float32)
    assert oracle_mod.pairwise_sum(x) == math.fsum(x.astype(np.float64))


# ---- block sizes ----

def brute_codes(w32, blocksize, levels):
    """Codes by exhaustive search in numpy float32: per block max |w|, then
    the first index minimising |fl32(fl32(w / c1) - q_i)|."""
    n = w32.size
    out = np.zeros(n, np.uint8)
    amax = []
    for b in range(0, n, blocksize):
        blk = w32[b:b + blocksize]
        c1 = np.float32(np.max(np.abs(blk)))
        amax.append(c1)
        if c1 == 0:
            out[b:b + blocksize] = 7
            continue
        nrm = (blk / c1).astype(np.float32)
        d = np.abs((nrm[:, None] - levels[None, :].astype(np.float32)).astype(np.float32))
        out[b:b + blocksize] = np.argmin(d, axis=1)
    return out, np.array(amax, np.float32)


@pytest.mark.parametrize("blocksize", [16, 32, 128, 256, 1024, 4096])
@pytest.mark.parametrize("n", [5000, 4096 * 3 + 17])
def test_quantize_block_sizes_brute_force(oracle_mod, printed_codebook, blocksize, n):
    rng = np.random.Generator(np.random.PCG64(blocksize + n))
    w = rng.standard_normal(n, dtype=np.float32)
    w[:blocksize] = 0.0  # one all-zero block
    codes, amax = oracle_mod.quantize_bs(w, blocksize)
    bc, ba = brute_codes(w, blocksize, printed_codebook.astype(np.float32))
    assert np.array_equal(amax, ba)
    assert np.array_equal(unpack(codes, n), bc)


def test_quantize_block_size_doubling(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(21))
    n = 64 * 200
    w = to_bf16_bits(rng.standard_normal(n, dtype=np.float32))
    _, a64 = oracle_mod.quantize_bs(w, 64)
    _, a128 = oracle_mod.quantize_bs(w, 128)
    assert np.array_equal(a128, np.maximum(a64[0::2], a64[1::2]))
    # plant the same max |w| in both halves of every 128-block: the codes of
    # the two block sizes then agree
    wf = oracle_mod.bf16_to_f32(w).reshape(-1, 2, 64)
    peak = np.abs(wf).max(axis=(1, 2))
    wf[:, 0, 0] = peak
    wf[:, 1, 5] = -peak
    w2 = to_bf16_bits(wf.ravel())
    c64, _ = oracle_mod.quantize_bs(w2, 64)
    c128, _ = oracle_mod.quantize_bs(w2, 128)
    assert np.array_equal(c64, c128)


def test_dequantize_block_max_is_exact(oracle_mod):
    """The element of largest magnitude maps to a level of magnitude 1, so
    each block's largest |w'| equals its c1 exactly, for any block size."""
    rng = np.random.Generator(np.random.PCG64(4))
    for bs in (16, 128, 512, 4096):
        n = bs * 5 + 3
        w = rng.standard_normal(n, dtype=np.float32) * 3
        codes, amax = oracle_mod.quantize_bs(w, bs)
        out = oracle_mod.dequantize_ex(codes, n, blocksize=bs, absmax=amax)
        for b in range(len(amax)):
            assert np.max(np.abs(out[b * bs:(b + 1) * bs])) == amax[b]


# ---- double-quantization formats and the mean offset ----

def absmax_like(rng, nb):
    """Absmax values of Gaussian 64-blocks (positive, bunched around 2.4)."""
    return np.abs(rng.standard_normal((nb, 64), dtype=np.float32)).max(axis=1).astype(np.float32)


@pytest.mark.parametrize("dq_blocksize", [1, 2, 64, 256, 4096])
@pytest.mark.parametrize("fmt", ["e4m3", "e5m2", "linear8"])
def test_group_scale_is_the_group_max(oracle_mod, dq_blocksize, fmt):
    rng = np.random.Generator(np.random.PCG64(dq_blocksize))
    nb = 5 * dq_blocksize + 3
    a = absmax_like(rng, nb)
    _, sc, _ = oracle_mod.double_quantize_ex(a, dq_blocksize, fmt)
    pad = np.zeros(-nb % dq_blocksize, np.float32)
    gmax = np.concatenate([a, pad]).reshape(-1, dq_blocksize).max(axis=1)
    want = gmax if fmt != "linear8" else (gmax / np.float32(255)).astype(np.float32)
    assert np.array_equal(sc, want)


def test_linear8_code_is_the_nearest_step(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(8))
    a = absmax_like(rng, 4096)
    for off in (False, True):
        q, sc, mu = oracle_mod.double_quantize_ex(a, 256, "linear8", off)
        codes = q.view(np.int8).astype(np.int64) if off else q.astype(np.int64)
        near_tie = 0
        for b in range(a.size):
            x = Fraction(float(a[b])) - (Fraction(float(mu)) if off else 0)
            x = Fraction(float(np.float32(a[b] - mu))) if off else x
            t = x / Fraction(float(sc[b // 256]))
            k = math.floor(t + Fraction(1, 2))
            if abs(t - math.floor(t) - Fraction(1, 2)) < Fraction(1, 2 ** 18):
                near_tie += 1  # fl32(x / u) may round across the half-way point
                assert codes[b] in (math.floor(t), math.floor(t) + 1)
                continue
            assert codes[b] == k
        assert near_tie < 10


def test_mean_offset_two_valued_closed_form(oracle_mod):
    """Blocks alternating between a and b: mu = (a+b)/2, x = -+(b-a)/2, c2 =
    (b-a)/2, ratios -+1, and both FP8 formats hold 1 exactly, so every scale
    is reconstructed exactly. Without the offset, a/b = 0.6 is not an E4M3
    value and the smaller scale comes back wrong."""
    a, b = np.float32(0.75), np.float32(1.25)
    absmax = np.tile(np.array([a, b], np.float32), 512)
    for fmt in ("e4m3", "e5m2"):
        q, sc, mu = oracle_mod.double_quantize_ex(absmax, 256, fmt, True)
        assert mu == 1.0 and np.all(sc == 0.25)
        rec = oracle_mod.block_scales_ex(absmax.size, 256, fmt, q=q, scale=sc, offset=mu)
        assert np.array_equal(rec, absmax)
        # codes are signed: below the mean negative, above positive
        assert np.all(q[0::2] & 0x80) and not np.any(q[1::2] & 0x80)
    q, sc, _ = oracle_mod.double_quantize_ex(absmax, 256, "e4m3", False)
    rec = oracle_mod.block_scales_ex(absmax.size, 256, "e4m3", q=q, scale=sc)
    assert rec[0] == np.float32(0.625 * 1.25) and rec[1] == b
    # linear8 with the offset: code -127 / +127, scale within one rounding of each
    q, sc, mu = oracle_mod.double_quantize_ex(absmax, 256, "linear8", True)
    assert np.all(q.view(np.int8)[0::2] == -127) and np.all(q.view(np.int8)[1::2] == 127)
    rec = oracle_mod.block_scales_ex(absmax.size, 256, "linear8", q=q, scale=sc, offset=mu)
    assert np.max(np.abs(rec - absmax)) <= 2.0 ** -23


def test_mean_offset_constant_input(oracle_mod):
    """Every c1 equal: mu is that value, x = 0, c2 = 0, and the scale comes back exactly."""
    absmax = np.full(1000, 2.375, np.float32)
    for fmt in ("e4m3", "e5m2", "linear8"):
        q, sc, mu = oracle_mod.double_quantize_ex(absmax, 256, fmt, True)
        assert mu == np.float32(2.375) and np.all(sc == 0) and np.all(q == 0)
        rec = oracle_mod.block_scales_ex(absmax.size, 256, fmt, q=q, scale=sc, offset=mu)
        assert np.all(rec == absmax)


def test_mean_offset_value(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(12))
    # exact sum (multiples of 2^-10 below 2^13): mu is the correctly rounded mean
    a = (rng.integers(1, 4096, 3000) * 2.0 ** -10).astype(np.float32)
    _, _, mu = oracle_mod.double_quantize_ex(a, 256, "e4m3", True)
    assert mu == np.float32(Fraction(math.fsum(a.astype(np.float64))) / a.size)


# relative bound on |c1' - c1| / c2 per format: half a step of the format at
# the ratio (3 mantissa bits E4M3, 2 E5M2; 1/255 or 1/127 linear) plus the
# fp32 roundings of the ratio and the product (and of the offset sum)
@pytest.mark.parametrize("fmt,rel,absolute", [("e4m3", 2.0 ** -4, 2.0 ** -10),
                                              ("e5m2", 2.0 ** -3, 2.0 ** -17),
                                              ("linear8", 0.0, None)])
@pytest.mark.parametrize("off", [False, True])
def test_reconstruction_error_bound(oracle_mod, fmt, rel, absolute, off):
    rng = np.random.Generator(np.random.PCG64(31))
    a = absmax_like(rng, 256 * 40 + 7)
    a[::97] *= 8  # a few outliers
    q, sc, mu = oracle_mod.double_quantize_ex(a, 256, fmt, off)
    rec = oracle_mod.block_scales_ex(a.size, 256, fmt, q=q, scale=sc, offset=mu)
    x = (a - mu).astype(np.float64) if off else a.astype(np.float64)
    g = np.arange(a.size) // 256
    if fmt == "linear8":
        c2 = sc[g].astype(np.float64) * (127 if off else 255)
        bound = sc[g].astype(np.float64) / 2 + 4 * 2.0 ** -24 * (np.abs(a) + c2)
    else:
        c2 = sc[g].astype(np.float64)
        bound = rel * np.abs(x) + absolute * c2 + 4 * 2.0 ** -24 * (np.abs(a) + c2)
    assert np.all(np.abs(rec.astype(np.float64) - a) <= bound)
    # for the float formats the offset helps: the values near the mean get
    # the format's fine steps, and the mean error falls (the linear code
    # loses a level bit to the sign instead)
    if off and fmt != "linear8":
        q0, sc0, _ = oracle_mod.double_quantize_ex(a, 256, fmt, False)
        rec0 = oracle_mod.block_scales_ex(a.size, 256, fmt, q=q0, scale=sc0)
        assert np.mean(np.abs(rec - a)) < np.mean(np.abs(rec0 - a))


def test_variant_argument_checks(oracle_mod):
    a = np.ones(10, np.float32)
    with pytest.raises(ValueError):
        oracle_mod.double_quantize_ex(a, 3)
    with pytest.raises(ValueError):
        oracle_mod.double_quantize_ex(a, 8192)
    with pytest.raises(ValueError):
        oracle_mod.double_quantize_ex(a, 256, 7)
    with pytest.raises(ValueError):
        oracle_mod.quantize_bs(np.ones(10, np.float32), 8)
    with pytest.raises(ValueError):
        oracle_mod.quantize_bs(np.ones(10, np.float32), 96)


def test_variant_footprint_closed_forms(oracle_mod):
    """[MF] "Double Quantization (DQ)": 8 / B1 + 32 / (B1 B2) bits per parameter
    of scale data, with B1 and B2 as parameters; 32 / B1 without DQ."""
    n = 1 << 24
    for b1, b2 in ((64, 256), (128, 256), (32, 64), (256, 1024)):
        dq = oracle_mod.storage_bytes_ex(n, b1, b2, True)
        assert (dq - n // 2) * 8 / n == 8 / b1 + 32 / (b1 * b2)
        assert (oracle_mod.storage_bytes_ex(n, b1, b2, False) - n // 2) * 8 / n == 32 / b1
        assert oracle_mod.storage_bytes_ex(n, b1, b2, True, True) == dq + 4
    # the printed default: 0.127 bits of overhead (0.126953125 exactly)
    assert oracle_mod.storage_bytes_ex(n) == oracle_mod.storage_bytes(n, True)
    assert oracle_mod.storage_bytes_ex(10, 48) == -1
