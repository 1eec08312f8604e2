"""Pins of the oracle's codebook swaps (CPU only): the blockwise scheme with
the FP4 or Int4 levels in place of NF4's ("QLoRA: Mathematical Foundations
...", "Empirical Performance and Architectural Guidelines", finding 2: NF4
beats FP4 and Int4; "QLoRA in Production ...", "1. 4-bit NormalFloat (NF4)":
the numpy comparison with a naive uniform 4-bit quantizer).

Pins: the Int4 codebook reproduces the uniform quantizer of that comparison
(one block = its per-tensor absmax), exhaustive nearest-level search in
numpy for every codebook, and the pages' claim itself on Gaussian weights:
NF4's mean squared error is below FP4's and Int4's.
The FP4 codebook is OCP E2M1 in its own encoding with every value divided
by 6 (the pages name FP4 without defining it): pinned code by code to the
E2M1 table of the OCP Microscaling Formats specification
(tests/golden/fp4_e2m1.txt), and its nearest-code function to the
sign-magnitude form that encoding implies.
"""
import numpy as np
import pytest

from conftest import read_golden_column
from workloads import to_bf16_bits


def unpack(codes, n):
    return np.stack([codes & 15, codes >> 4], axis=1).ravel()[:n]


def test_int4_is_the_uniform_quantizer_of_the_comparison(oracle_mod):
    """One 64-block: x / absmax * 7.5 - 0.5 rounded gives k' in [-8, 7] and the
    value (k' + 0.5) * absmax / 7.5; the Int4 code is k' + 8, except at an
    exact half-way point (the toy's round-half-even against the lowest index)."""
    rng = np.random.Generator(np.random.PCG64(42))
    lv = oracle_mod.codebook_levels("int4").astype(np.float64)
    assert np.allclose(lv, (np.arange(-8, 8) + 0.5) / 7.5, rtol=0, atol=6e-8)
    for _ in range(50):
        x = rng.standard_normal(64).astype(np.float32)
        codes, amax = oracle_mod.quantize_cb(x, 64, "int4")
        t = x.astype(np.float64) / float(amax[0]) * 7.5 - 0.5
        kp = np.clip(np.round(t), -8, 7)
        got = unpack(codes, 64).astype(np.int64) - 8
        tie = np.abs(np.abs(t - np.floor(t)) - 0.5) < 1e-5
        assert np.all((got == kp) | tie)
        deq = oracle_mod.dequantize_cb(codes, 64, codebook="int4", absmax=amax).astype(np.float64)
        want = (kp + 0.5) * float(amax[0]) / 7.5
        assert np.all((np.abs(deq - want) <= 2e-7 * float(amax[0])) | tie)


@pytest.mark.parametrize("cb", ["nf4", "fp4", "int4"])
def test_codebook_brute_force(oracle_mod, cb):
    rng = np.random.Generator(np.random.PCG64(len(cb)))
    lv = oracle_mod.codebook_levels(cb)
    if cb == "fp4":
        # OCP order: +0 .. +1 at codes 0..7, -0 .. -1 at codes 8..15
        assert np.all(np.diff(lv[:8]) > 0) and np.all(np.diff(lv[8:]) < 0)
        assert lv[7] == 1 and lv[15] == -1
    else:
        assert np.all(np.diff(lv) > 0) and lv[0] == -1 and lv[-1] == 1
    n = 64 * 40 + 9
    w = rng.standard_normal(n, dtype=np.float32)
    w[:64] = 0.0
    codes, amax = oracle_mod.quantize_cb(w, 64, cb)
    got = unpack(codes, n)
    zero_code = int(np.argmin(np.abs(lv)))
    for b in range(0, n, 64):
        blk = w[b:b + 64]
        c1 = np.float32(np.max(np.abs(blk)))
        assert amax[b // 64] == c1
        if c1 == 0:
            assert np.all(got[b:b + 64] == zero_code)
            continue
        nrm = (blk / c1).astype(np.float32)
        d = np.abs((nrm[:, None] - lv[None, :]).astype(np.float32))
        assert np.array_equal(got[b:b + 64], np.argmin(d, axis=1))
    deq = oracle_mod.dequantize_cb(codes, n, codebook=cb, absmax=amax)
    assert np.array_equal(deq, (lv[got] * amax[np.arange(n) // 64]).astype(np.float32))


def test_nf4_codebook_path_equals_nf4(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(8))
    w = to_bf16_bits(rng.standard_normal(5000, dtype=np.float32))
    assert all(np.array_equal(a, b) for a, b in zip(oracle_mod.quantize_cb(w, 64, "nf4"),
                                                     oracle_mod.quantize(w)))


@pytest.mark.parametrize("bs", [64, 256])
def test_nf4_beats_fp4_and_int4_on_gaussian_weights(oracle_mod, bs):
    rng = np.random.Generator(np.random.PCG64(bs))
    w = (rng.standard_normal(1 << 16) * 0.02).astype(np.float32)
    mse = {}
    for cb in ("nf4", "fp4", "int4"):
        codes, amax = oracle_mod.quantize_cb(w, bs, cb)
        deq = oracle_mod.dequantize_cb(codes, w.size, blocksize=bs, codebook=cb, absmax=amax)
        mse[cb] = float(np.mean((deq.astype(np.float64) - w) ** 2))
    assert mse["nf4"] < mse["fp4"] and mse["nf4"] < mse["int4"], mse


def test_fp4_is_the_ocp_e2m1_encoding(oracle_mod):
    """Code c of the FP4 codebook is the E2M1 value of bit pattern c, divided
    by 6 (rounded once to fp32), sign of zero included."""
    rows = read_golden_column("fp4_e2m1.txt", col=None)
    assert len(rows) == 16
    lv = oracle_mod.codebook_levels("fp4")
    for code, sign, exp, man, val in rows:
        c, sgn, e, m = int(code), int(sign), int(exp), int(man)
        v = float(val)
        assert c == 8 * sgn + 2 * e + m  # the table's own bit fields
        mag = 0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + 0.5 * m)
        assert abs(v) == mag and bool(np.signbit(v)) == bool(sgn)
        assert lv[c] == np.float32(np.float32(v) / np.float32(6.0))
        assert bool(np.signbit(lv[c])) == bool(sgn)


def test_fp4_nearest_code_is_sign_magnitude(oracle_mod):
    """With the E2M1 encoding, the lowest-index nearest code of n is
    8 * sign(n) + the nearest magnitude index of |n|, except that every n
    nearest to zero gets +0 (code 0, the lower index of the +0 / -0 tie);
    -0 (code 8) is never chosen."""
    rng = np.random.Generator(np.random.PCG64(99))
    n = 64 * 200
    w = rng.standard_normal(n, dtype=np.float32)
    w[::97] = 0.0
    w[1::89] = -0.0
    w[2::83] *= np.float32(1e-3)                   # near the zero switch
    w[::64] = np.float32(4.0)                      # c1 = 4 in every block
    codes, amax = oracle_mod.quantize_cb(w, 64, "fp4")
    got = unpack(codes, n)
    assert not np.any(got == 8)
    pos, _ = oracle_mod.quantize_cb(np.abs(w), 64, "fp4")
    mag = unpack(pos, n)
    assert np.all(mag < 8)
    want = np.where((w < 0) & (mag > 0), mag + 8, mag)
    assert np.array_equal(got, want)
    assert np.all(got[w == 0] == 0)
