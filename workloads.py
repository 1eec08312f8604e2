"""Seeded synthetic inputs shared by the tests and the benchmark.

This module only draws random numbers and lays them out; it holds none of the
quantization or matmul arithmetic. The weight distribution follows the premise
of "QLoRA: Mathematical Foundations of 4-Bit NormalFloat Quantization, Double
Quantization, and Paged Optimizers", section "4-Bit NormalFloat (NF4)": trained
weights are close to zero-mean Gaussians. Real checkpoints are not used.

Host arrays: numpy ``Generator(PCG64(seed))``. bf16 values are returned as
their uint16 bit patterns (torch's CPU fp32->bf16 cast, round to nearest even).
Large stacks are drawn on the device with a seeded ``torch.Generator``.
"""
import numpy as np

SIGMA_W = 0.02  # weight std of every workload


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x32):
    """fp32 numpy array -> bf16 bit patterns (uint16), round to nearest even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def gaussian_f32(seed, shape, sigma):
    rng = _rng(seed)
    return rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)


# ---- workload 1: one 1024x1024 fp32 matrix, N(0, 0.02^2), seed 1 ----
def weight_1024_f32(seed=1):
    return gaussian_f32(seed, (1024, 1024), SIGMA_W)


# ---- workload 2: 11008x4096 bf16, N(0, 0.02^2), 0.1% entries x10, seed 2 ----
MLP_SHAPE = (11008, 4096)


def weight_mlp_outliers_bf16(seed=2, shape=MLP_SHAPE, frac=0.001, factor=10.0):
    rng = _rng(seed)
    n = int(np.prod(shape))
    w = rng.standard_normal(n, dtype=np.float32) * np.float32(SIGMA_W)
    k = int(round(n * frac))
    idx = rng.choice(n, size=k, replace=False)
    w[idx] *= np.float32(factor)
    return to_bf16_bits(w).reshape(shape)


# ---- workload 3: a 32-layer 8B-shaped stack, bf16, drawn on the device ----
STACK_LAYERS = 32
STACK_MATRICES = (
    ("q", (4096, 4096)),
    ("k", (1024, 4096)),
    ("v", (1024, 4096)),
    ("o", (4096, 4096)),
    ("gate", (14336, 4096)),
    ("up", (14336, 4096)),
    ("down", (4096, 14336)),
)


def stack_seed(layer, matrix_index):
    return 3 + layer * 7 + matrix_index


def stack_matrix_bf16(layer, matrix_index, device, out=None):
    """Draws one stack matrix on `device` (torch bf16); same bits for the same seed."""
    import torch

    shape = STACK_MATRICES[matrix_index][1]
    g = torch.Generator(device=device)
    g.manual_seed(stack_seed(layer, matrix_index))
    w = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    w.mul_(SIGMA_W)
    if out is None:
        return w.to(torch.bfloat16)
    out.copy_(w.to(torch.bfloat16).view(-1))
    return out


def stack_params():
    return STACK_LAYERS * sum(a * b for _, (a, b) in STACK_MATRICES)


# ---- workload 4: decode GEMV, x bf16 [M x 8192], W [28672 x 8192], seed 4 ----
GEMV_N, GEMV_K = 28672, 8192
GEMV_MS = (1, 4, 16)


def gemv_inputs(seed=4, n=GEMV_N, k=GEMV_K, m_max=16):
    """Returns (w fp32 [n,k] ~ N(0, 0.02^2), x bf16 bits [m_max, k] ~ N(0,1))."""
    rng = _rng(seed)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(SIGMA_W)
    x = to_bf16_bits(rng.standard_normal((m_max, k), dtype=np.float32))
    return w, x


# ---- workload 5: QLoRA linear, X/dY [4096 x 8192], W [8192 x 8192], r = 64 ----
LIN_M, LIN_N, LIN_K, LIN_R, LIN_SCALE = 4096, 8192, 8192, 64, 2.0
SIGMA_LORA = 0.01


def linear_inputs(seed=5, m=LIN_M, n=LIN_N, k=LIN_K, r=LIN_R):
    """Returns dict: w fp32 [n,k]; x, dy bf16 bits [m,k], [m,n]; a [k,r], b [r,n] bf16 bits."""
    rng = _rng(seed)
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(SIGMA_W)
    x = to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    dy = to_bf16_bits(rng.standard_normal((m, n), dtype=np.float32))
    a = to_bf16_bits(rng.standard_normal((k, r), dtype=np.float32) * np.float32(SIGMA_LORA))
    b = to_bf16_bits(rng.standard_normal((r, n), dtype=np.float32) * np.float32(SIGMA_LORA))
    return {"w": w, "x": x, "dy": dy, "a": a, "b": b}
