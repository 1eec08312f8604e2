"""Pins of the oracle's storage sizes against the figures the pages print, and
of its matmul reference against library routines and the adjoint identity
(CPU only).

Sources: "Lesson 15. NF4 and Double Quantisation" ("Double quantisation"
tables); "QLoRA: Mathematical Foundations ..." ("Double Quantization (DQ)",
"Forward Pass Computation", "Gradient Computation"); "QLoRA in Production ..."
("2. Double Quantization (DQ)"); "QLoRA: quantising the part you are not
training" ("The idea in one line").
"""
import numpy as np
import pytest

from conftest import read_golden_column
from workloads import gaussian_f32, to_bf16_bits


def footprint_values(oracle_mod):
    n = 1 << 34  # a large multiple of 64*256: per-parameter figures are exact
    b_dq = oracle_mod.storage_bytes(n, True) / n
    b_nodq = oracle_mod.storage_bytes(n, False) / n
    scale_bits_dq = (oracle_mod.storage_bytes(n, True) - n // 2) * 8 / n
    scale_bits_nodq = (oracle_mod.storage_bytes(n, False) - n // 2) * 8 / n
    saving = scale_bits_nodq - scale_bits_dq

    def gb(params, dq=True):
        return oracle_mod.storage_bytes(params, dq) / 1e9

    p65 = 65_000_000_000
    p7 = 7_000_000_000
    blocks_7b = (oracle_mod.storage_bytes(p7, False) - (p7 + 1) // 2) // 4
    return {
        "bytes_per_param_no_dq": b_nodq,
        "bits_per_param_no_dq": 8 * b_nodq,
        "bytes_per_param_dq": b_dq,
        "bits_per_param_dq": 8 * b_dq,
        "scale_bits_no_dq": scale_bits_nodq,
        "scale_share_of_4bit": scale_bits_nodq / 4.0,
        "scale_bits_dq": scale_bits_dq,
        "dq_saving_bits": saving,
        "dq_saving_fraction": saving / scale_bits_nodq,
        "dq_saving_65b_gb": (oracle_mod.storage_bytes(p65, False)
                             - oracle_mod.storage_bytes(p65, True)) / 1e9,
        "blocks_7b_millions": blocks_7b / 1e6,
        "scale_mb_7b": 4 * blocks_7b / 1e6,
        "dq_bits_per_block": scale_bits_dq * 64,
        "nf4_gb_8b": gb(8_000_000_000),
        "nf4_gb_70b": gb(70_000_000_000),
    }


def test_footprint_matches_printed_figures(oracle_mod):
    got = footprint_values(oracle_mod)
    rows = read_golden_column("footprint.txt", col=None)
    assert len(rows) == len(got)
    for key, printed, tol, _src in rows:
        assert abs(got[key] - float(printed)) <= float(tol), (key, got[key], printed)


def test_footprint_exact_rationals(oracle_mod):
    # 0.5 + 1/64 + 4/(64*256) bytes per parameter, exactly
    assert oracle_mod.storage_bytes(1 << 20, True) == 540_928
    assert oracle_mod.storage_bytes(1 << 20, True) / (1 << 20) == 0.515869140625
    assert oracle_mod.storage_bytes(1 << 20, False) / (1 << 20) == 0.5625
    # partial blocks and groups round up
    assert oracle_mod.storage_bytes(1, True) == 1 + 1 + 4
    assert oracle_mod.storage_bytes(65, False) == 33 + 8
    assert oracle_mod.storage_bytes(64 * 256 + 1, True) == 8193 + 257 + 8


# ---------------------------------------------------------------- matmuls

def _small_linear(seed, m=7, k=192, n=40, r=5):
    rng = np.random.Generator(np.random.PCG64(seed))
    x = to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    dy = to_bf16_bits(rng.standard_normal((m, n), dtype=np.float32))
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    a = to_bf16_bits(rng.standard_normal((k, r), dtype=np.float32) * np.float32(0.1))
    b = to_bf16_bits(rng.standard_normal((r, n), dtype=np.float32) * np.float32(0.1))
    return x, dy, w, a, b


def _f(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_forward_reference_matches_library_matmul(oracle_mod):
    x, _, w, a, b = _small_linear(51)
    s = 2.0
    got = oracle_mod.linear_forward(x, w, a, b, s)
    want = _f(x) @ w.astype(np.float64).T + s * (_f(x) @ _f(a)) @ _f(b)
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))
    base = oracle_mod.linear_forward(x, w)
    assert np.max(np.abs(base - _f(x) @ w.astype(np.float64).T)) <= 1e-12 * np.max(np.abs(base))


def test_backward_reference_matches_library_matmul(oracle_mod):
    _, dy, w, a, b = _small_linear(52)
    s = 2.0
    got = oracle_mod.linear_backward_input(dy, w, a, b, s)
    want = _f(dy) @ w.astype(np.float64) + s * (_f(dy) @ _f(b).T) @ _f(a).T
    assert np.max(np.abs(got - want)) <= 1e-12 * np.max(np.abs(want))


def test_forward_backward_adjoint_identity(oracle_mod):
    """<dY, f(X)> == <g(dY), X> for the linear map f and its input gradient g:
    catches a transposed operand or a misplaced adapter factor in either."""
    x, dy, w, a, b = _small_linear(53, m=5, k=128, n=96, r=8)
    s = 2.0
    y = oracle_mod.linear_forward(x, w, a, b, s)
    dx = oracle_mod.linear_backward_input(dy, w, a, b, s)
    lhs = np.sum(_f(dy) * y)
    rhs = np.sum(dx * _f(x))
    assert abs(lhs - rhs) <= 1e-10 * max(abs(lhs), 1.0)


def test_row_and_column_selection(oracle_mod):
    x, dy, w, a, b = _small_linear(54)
    full = oracle_mod.linear_forward(x, w, a, b, 2.0)
    rows = np.array([6, 0, 3])
    cols = np.array([39, 1, 17, 17])
    sel = oracle_mod.linear_forward(x, w, a, b, 2.0, rows=rows, cols=cols)
    assert np.array_equal(sel, full[np.ix_(rows, cols)])
    fullb = oracle_mod.linear_backward_input(dy, w, a, b, 2.0)
    colsb = np.array([0, 191, 64])
    selb = oracle_mod.linear_backward_input(dy, w, a, b, 2.0, rows=rows, cols=colsb)
    assert np.array_equal(selb, fullb[np.ix_(rows, colsb)])


def test_lora_scale_enters_linearly(oracle_mod):
    x, _, w, a, b = _small_linear(55)
    y0 = oracle_mod.linear_forward(x, w, a, b, 0.0)
    y1 = oracle_mod.linear_forward(x, w, a, b, 1.0)
    y2 = oracle_mod.linear_forward(x, w, a, b, 2.0)
    assert np.allclose(y2 - y0, 2 * (y1 - y0), rtol=1e-12, atol=1e-14)
    assert np.max(np.abs(y1 - y0)) > 0
