"""Pins of the oracle's adapter merge (CPU only): the merged weight
Wm = dequantize(W) + s (A B)^T that "QLoRA in Production ...", "Step 4:
Merging and Inference", folds into the base, re-quantized as "QLoRA:
quantising the part you are not training", "What it costs" (item 3), says a
merge into the quantized base must be.

Pins: a zero adapter leaves the stored weight unchanged (quantizing a
dequantized NF4 weight is the identity: its largest element per block is
+-c1' exactly); with adapters of small dyadic values, numpy's float64 matmul
gives the delta exactly; and the merged weight's forward equals the
adapter forward of the linear oracle up to the fp32 rounding of the merge.
"""
import numpy as np
import pytest

from workloads import to_bf16_bits


def base(seed, N, K, dq=True):
    import oracle

    rng = np.random.Generator(np.random.PCG64(seed))
    w = to_bf16_bits(rng.standard_normal((N, K), dtype=np.float32) * np.float32(0.02))
    codes, amax = oracle.quantize(w.ravel())
    if not dq:
        return codes, amax, None, None
    q, sc = oracle.double_quantize(amax)
    return codes, None, q, sc


def dyadic(rng, shape, scale_exp):
    """bf16 values k * 2^scale_exp, k in -3..3: products and their sums over the
    rank stay exact in fp32 and float64."""
    return to_bf16_bits((rng.integers(-3, 4, size=shape) * 2.0 ** scale_exp).astype(np.float32))


@pytest.mark.parametrize("dq", [True, False])
def test_zero_adapter_is_identity(oracle_mod, dq):
    N, K, r = 48, 320, 16
    codes, amax, q, sc = base(1, N, K, dq)
    A = np.zeros((K, r), np.uint16)
    B = to_bf16_bits(np.ones((r, N), np.float32))
    nc, na, nq8, nsc, wm = oracle_mod.merge_lora(codes, (N, K), A, B, 2.0, amax, q, sc, dq)
    deq = oracle_mod.dequantize(codes, N * K, amax, q, sc)
    assert np.array_equal(wm.ravel(), deq)
    assert np.array_equal(nc, codes)
    if dq:
        assert np.array_equal(nq8, q) and np.array_equal(nsc, sc)
    else:
        assert np.array_equal(na, amax)


@pytest.mark.parametrize("N,K,r,s", [(16, 128, 8, 2.0), (33, 192, 24, 0.5), (8, 64, 64, 1.0)])
def test_merged_weight_is_base_plus_scaled_product(oracle_mod, N, K, r, s):
    rng = np.random.Generator(np.random.PCG64(N + K + r))
    codes, _, q, sc = base(N, N, K)
    A = dyadic(rng, (K, r), -6)
    B = dyadic(rng, (r, N), -5)
    wm = oracle_mod.merged_weight(codes, (N, K), A, B, s, q=q, scale=sc)
    deq = oracle_mod.dequantize(codes, N * K, q=q, scale=sc).reshape(N, K)
    af = oracle_mod.bf16_to_f32(A).astype(np.float64)
    bf = oracle_mod.bf16_to_f32(B).astype(np.float64)
    delta = (s * (af @ bf)).T.astype(np.float32)  # exact: dyadic values, power-of-two s
    want = (deq + delta).astype(np.float32)       # one fp32 rounding of the sum
    assert np.array_equal(wm, want)
    # row selection
    rows = np.array([N - 1, 0, N // 2])
    assert np.array_equal(oracle_mod.merged_weight(codes, (N, K), A, B, s, q=q, scale=sc,
                                                   rows=rows), want[rows])


def test_merged_forward_equals_adapter_forward(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(77))
    N, K, r, m, s = 24, 256, 16, 5, 2.0
    codes, _, q, sc = base(5, N, K)
    A = to_bf16_bits(rng.standard_normal((K, r), dtype=np.float32) * np.float32(0.05))
    B = to_bf16_bits(rng.standard_normal((r, N), dtype=np.float32) * np.float32(0.05))
    x = to_bf16_bits(rng.standard_normal((m, K), dtype=np.float32))
    wm = oracle_mod.merged_weight(codes, (N, K), A, B, s, q=q, scale=sc)
    deq = oracle_mod.dequantize(codes, N * K, q=q, scale=sc).reshape(N, K)
    merged = oracle_mod.linear_forward(x, wm)
    lora = oracle_mod.linear_forward(x, deq, A, B, s)
    xf = np.abs(oracle_mod.bf16_to_f32(x).astype(np.float64))
    # each merged element carries at most two fp32 roundings (d and the sum)
    bound = xf @ (np.abs(wm.astype(np.float64)).T * 2.0 ** -22 + 1e-30)
    assert np.all(np.abs(merged - lora) <= bound)
    # and the adapter matters: without it the forward is far off
    plain = oracle_mod.linear_forward(x, deq)
    assert np.max(np.abs(plain - lora)) > 100 * np.max(bound)


def test_merge_changes_codes_and_rejects_bad_rows(oracle_mod):
    rng = np.random.Generator(np.random.PCG64(3))
    N, K, r = 16, 128, 8
    codes, _, q, sc = base(2, N, K)
    A = to_bf16_bits(rng.standard_normal((K, r), dtype=np.float32) * np.float32(0.1))
    B = to_bf16_bits(rng.standard_normal((r, N), dtype=np.float32) * np.float32(0.1))
    nc, _, nq8, nsc, wm = oracle_mod.merge_lora(codes, (N, K), A, B, 2.0, q=q, scale=sc)
    assert np.mean(nc != codes) > 0.2
    nc2, na2 = oracle_mod.quantize(wm.ravel())
    assert np.array_equal(nc, nc2)
    with pytest.raises(ValueError):
        oracle_mod.merged_weight(codes, (N, K), A, B, 1.0, q=q, scale=sc, rows=np.array([N]))
