"""Pins of the oracle's adapter gradients (CPU only).

Source: "QLoRA: Mathematical Foundations of 4-Bit NormalFloat Quantization,
Double Quantization, and Paged Optimizers", "Gradient Computation": the
gradients of the two adapter matrices of the loss whose output gradient is dY.

The pin is the derivative itself, not the printed expressions: with the base
weight set to zero, the oracle's forward Y(A, B) = s (X A) B is linear in A for
a fixed B and in B for a fixed A, so for the scalar L = sum(G * Y) the change
of L under a unit step of one entry of A (or B) is exactly that entry of dL/dA
(or dL/dB), the gradient the oracle computes with dY = G. Integer-valued bf16
inputs keep every sum exact in double, so both sides agree exactly; a dropped
factor s, a transposed operand or a swapped A/B would not.
"""
import numpy as np
import pytest

from workloads import to_bf16_bits


def small_ints(rng, shape, lo=-3, hi=4):
    return rng.integers(lo, hi, size=shape).astype(np.float32)


def loss(oracle_mod, x, A, B, G, s):
    m, K = x.shape
    N = G.shape[1]
    wz = np.zeros((N, K), np.float32)
    y = oracle_mod.linear_forward(x, wz, A, B, s)
    return float(np.sum(y * G.astype(np.float64)))


@pytest.mark.parametrize("m,K,N,r,s", [(5, 7, 6, 3, 2.0), (4, 9, 5, 1, 0.5), (3, 4, 8, 2, 1.0)])
def test_lora_grads_equal_forward_differences(oracle_mod, m, K, N, r, s):
    rng = np.random.Generator(np.random.PCG64(1000 * m + K))
    xf, gf = small_ints(rng, (m, K)), small_ints(rng, (m, N))
    af, bf = small_ints(rng, (K, r)), small_ints(rng, (r, N))
    x, A, B = to_bf16_bits(xf), to_bf16_bits(af), to_bf16_bits(bf)
    G = to_bf16_bits(gf)
    da, db = oracle_mod.lora_grads(x, G, A, B, s)
    assert da.shape == (K, r) and db.shape == (r, N)
    L0 = loss(oracle_mod, x, A, B, gf, s)
    for k in range(K):
        for c in range(r):
            a1 = af.copy()
            a1[k, c] += 1.0
            assert loss(oracle_mod, x, to_bf16_bits(a1), B, gf, s) - L0 == da[k, c]
    for c in range(r):
        for n in range(N):
            b1 = bf.copy()
            b1[c, n] += 1.0
            assert loss(oracle_mod, x, A, to_bf16_bits(b1), gf, s) - L0 == db[c, n]


def test_lora_grads_row_and_column_selection(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(3))
    m, K, N, r = 6, 10, 12, 4
    x = to_bf16_bits(rng.standard_normal((m, K), dtype=np.float32))
    dy = to_bf16_bits(rng.standard_normal((m, N), dtype=np.float32))
    A = to_bf16_bits(rng.standard_normal((K, r), dtype=np.float32))
    B = to_bf16_bits(rng.standard_normal((r, N), dtype=np.float32))
    da, db = oracle_mod.lora_grads(x, dy, A, B, 2.0)
    rows, cols = np.array([9, 0, 4]), np.array([11, 3])
    da_s, db_s = oracle_mod.lora_grads(x, dy, A, B, 2.0, a_rows=rows, b_cols=cols)
    assert np.array_equal(da_s, da[rows]) and np.array_equal(db_s, db[:, cols])


def test_lora_grads_reject_bad_indices(oracle_mod):
    x = np.zeros((2, 3), np.uint16)
    dy = np.zeros((2, 4), np.uint16)
    A = np.zeros((3, 1), np.uint16)
    B = np.zeros((1, 4), np.uint16)
    with pytest.raises(ValueError):
        oracle_mod.lora_grads(x, dy, A, B, 1.0, a_rows=np.array([3]))
    with pytest.raises(ValueError):
        oracle_mod.lora_grads(x, dy, A, B, 1.0, b_cols=np.array([-1]))
