"""GPU parity of the fused NF4 linear (forward and input gradient, with and
without the adapter) against the oracle's double-precision reference.

Tolerance: max_i |y_i - r_i| / max(|r_i|, rms(r)) <= 2e-2 (bf16 operands,
fp32 accumulation, bf16 output; the reference uses the oracle's fp32
dequantized weight and no intermediate rounding). The weight is quantized by
the oracle and uploaded, so no input of the reference comes from the GPU.
"""
import numpy as np
import pytest

import nf4_quantize_amd as nq
import oracle
import workloads
from gpu_util import log, plain_rel_err, rel_err_metric, to_dev, to_host

pytestmark = pytest.mark.gpu

TOL = 2e-2


def upload_weight(w32, dev, dq=True):
    """Quantize on the CPU oracle and upload the packed weight."""
    N, K = w32.shape
    codes, absmax = oracle.quantize(w32.ravel())
    q8, scale = oracle.double_quantize(absmax)
    t = nq.NF4Tensor(to_dev(codes, dev), None if dq else to_dev(absmax, dev),
                     to_dev(q8, dev) if dq else None, to_dev(scale, dev) if dq else None, (N, K))
    host = dict(codes=codes, absmax=None if dq else absmax, q=q8 if dq else None,
                scale=scale if dq else None)
    return t, host


def oracle_wdeq(host, shape, rows=None):
    N, K = shape
    if rows is None:
        return oracle.dequantize(host["codes"], N * K, absmax=host["absmax"], q=host["q"],
                                 scale=host["scale"]).reshape(N, K)
    return oracle.dequantize_rows(host["codes"], shape, rows, absmax=host["absmax"], q=host["q"],
                                  scale=host["scale"])


def small_case(seed, m, n, k, r, dq=True, sigma_lora=0.05):
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.standard_normal((n, k), dtype=np.float32) * np.float32(0.02)
    x = workloads.to_bf16_bits(rng.standard_normal((m, k), dtype=np.float32))
    dy = workloads.to_bf16_bits(rng.standard_normal((m, n), dtype=np.float32))
    a = b = None
    if r:
        a = workloads.to_bf16_bits(rng.standard_normal((k, r), dtype=np.float32) * np.float32(sigma_lora))
        b = workloads.to_bf16_bits(rng.standard_normal((r, n), dtype=np.float32) * np.float32(sigma_lora))
    return w, x, dy, a, b


CASES = [
    # (m, N, K, r)
    (64, 512, 256, 16),
    (1, 128, 64, 0),
    (4, 1024, 2048, 8),
    (16, 768, 1024, 0),
    (37, 100, 192, 5),     # ragged rows and columns
    (130, 96, 320, 64),
    (256, 256, 512, 64),
    (2, 4096, 128, 3),
    # large-M shapes (N % 64 == 0, r % 8 == 0): several output tiles, ragged
    # rows, rank not a multiple of the 64-wide K step, and the widest rank
    (512, 1024, 256, 16),
    (300, 512, 1024, 40),
    (257, 2048, 512, 32),
    (70, 320, 192, 256),
    (200, 64, 64, 8),
    # adapter down-projection split over K: slices of 3 and 6 steps (not a
    # multiple of the 4-slot ring), empty trailing slices, and a rank that
    # leaves the second 64-column group mostly padding
    (64, 1344, 1408, 24),
    (100, 640, 2880, 48),
    (96, 1024, 1024, 72),
    # decode-shaped (no adapter): ragged column counts and odd row counts
    (3, 100, 192, 0),
    (16, 200, 320, 0),
    (9, 48, 128, 0),
    (5, 16 * 37, 64 * 11, 0),
    (3, 100, 768, 0),       # decode path (K % 256 == 0), ragged N
    (9, 48, 512, 0),
    (1, 16 * 600 + 5, 256, 0),
    (16, 1000, 1280, 0),
    # decode path with each tile count per workgroup (the grid is about one
    # workgroup per CU, so the tile count follows from N)
    (2, 16 * 300, 512, 0),
    (1, 16 * 1000 + 3, 256, 0),
    (7, 16 * 1300, 256, 0),
    (16, 16 * 1500 + 7, 512, 0),
    (1, 16 * 1900, 256, 0),
    (4, 16 * 1792, 2304, 0),
    # one activation row with K a multiple of 2048 (the row-streaming
    # kernel): 1, 2 and 4 pieces per row, fewer rows than waves, and K = 6144
    # (3 pieces, which the 16-row kernel takes)
    (1, 1000, 2048, 0),
    (1, 300, 4096, 0),
    (1, 77, 8192, 0),
    (1, 5000, 8192, 0),
    (1, 640, 6144, 0),
    # rows dealt round-robin over the grid's waves: some waves take one row
    # more than others
    (1, 16 * 300 + 5, 2048, 0),
    (1, 9000, 4096, 0),
    # 2 <= m <= 16 with K = 2048, 4096 or 8192 (the LDS-staged decode
    # kernel): 1, 2 and 4 stages per tile, ragged last tiles, a last
    # workgroup whose second tile lies past N, and stage walks that end
    # part-way through the four-stage ring
    (2, 100, 2048, 0),
    (5, 16 * 37 + 3, 4096, 0),
    (16, 16 * 300 + 9, 8192, 0),
    (3, 16 * 1100, 2048, 0),
    (7, 16 * 257, 4096, 0),
    (16, 16 * 700 + 1, 8192, 0),
]


@pytest.mark.parametrize("m,n,k,r", CASES)
@pytest.mark.parametrize("dq", [True, False])
def test_linear_small_full(dev, m, n, k, r, dq):
    import torch

    log(f"linear full check m={m} N={n} K={k} r={r} dq={dq}")
    w, x, dy, a, b = small_case(m * 7 + n + k + r, m, n, k, r, dq)
    wt, host = upload_weight(w, dev, dq)
    wd = oracle_wdeq(host, (n, k))
    s = 2.0
    xa, dya = to_dev(x, dev), to_dev(dy, dev)
    aa = to_dev(a, dev) if r else None
    ba = to_dev(b, dev) if r else None
    y = nq.linear_forward(xa, wt, aa, ba, s)
    dx = nq.linear_backward_input(dya, wt, aa, ba, s)
    torch.cuda.synchronize()
    y_ref = oracle.linear_forward(x, wd, a, b, s)
    dx_ref = oracle.linear_backward_input(dy, wd, a, b, s)
    e_y, n_y = rel_err_metric(_bf16_to_f32(to_host(y)), y_ref)
    e_dx, n_dx = rel_err_metric(_bf16_to_f32(to_host(dx)), dx_ref)
    log(f"  fwd err {e_y:.3e} (normwise {n_y:.3e}); dx err {e_dx:.3e} (normwise {n_dx:.3e})")
    assert e_y <= TOL and e_dx <= TOL


def test_lora_path_is_present(dev):
    """With the adapter's contribution comparable to the base path, dropping it
    (or applying it with the wrong scale) would exceed the tolerance."""
    import torch

    m, n, k, r = 32, 256, 512, 16
    w, x, dy, a, b = small_case(5, m, n, k, r, sigma_lora=0.2)
    wt, host = upload_weight(w, dev)
    wd = oracle_wdeq(host, (n, k))
    y = nq.linear_forward(to_dev(x, dev), wt, to_dev(a, dev), to_dev(b, dev), 2.0)
    torch.cuda.synchronize()
    got = (to_host(y).astype(np.uint32) << 16).view(np.float32)
    ref = oracle.linear_forward(x, wd, a, b, 2.0)
    ref_half = oracle.linear_forward(x, wd, a, b, 1.0)
    assert rel_err_metric(got, ref)[0] <= TOL
    assert rel_err_metric(got, ref_half)[0] > 5 * TOL


def _bf16_to_f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


@pytest.mark.parametrize("m", workloads.GEMV_MS)
def test_decode_gemv_sampled(dev, m, gemv_case):
    """Decode shape: x [M x 8192] times the 28672 x 8192 NF4 weight; all M rows
    on 384 sampled output columns."""
    import torch

    wt, host, x = gemv_case
    N, K = wt.shape
    y = nq.linear_forward(to_dev(x[:m], dev), wt)
    torch.cuda.synchronize()
    cols = np.sort(np.random.Generator(np.random.PCG64(40 + m)).choice(N, 384, replace=False))
    wd_rows = oracle_wdeq(host, (N, K), rows=cols)
    ref = oracle.linear_forward(x[:m], wd_rows)  # columns of Y = rows of W
    got = _bf16_to_f32(to_host(y))[:, cols]
    e, nw = rel_err_metric(got, ref)
    log(f"gemv M={m}: err {e:.3e} normwise {nw:.3e}")
    assert e <= TOL


def test_decode_gemv_longest_rows_sampled(dev):
    """The 16-row decode kernel at its longest rows (K = 32768) with 8 tiles of
    16 rows per workgroup, where a workgroup's staged scale data is largest
    (more than 256 c2 groups). The packed weight is random storage: any code
    bytes, finite E4M3 scale codes and positive c2 values. Checked on sampled
    output columns (including the ragged last tile) against the oracle."""
    import torch

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    K = 32768
    N = 16 * (7 * cus + 1) + 5  # more than 7 tiles per CU: 8 per workgroup; ragged last tile
    rng = np.random.Generator(np.random.PCG64(77))
    codes = rng.integers(0, 256, size=N * K // 2, dtype=np.uint8)
    nblk = N * K // 64
    q8 = rng.integers(0x20, 0x7F, size=nblk, dtype=np.uint8)  # 0x7F would be NaN
    scale = (rng.random((nblk + 255) // 256, dtype=np.float32) * np.float32(0.05) + np.float32(0.01))
    log(f"gemv longest rows: N={N} K={K} ({N * K // 2} code bytes)")
    t = nq.NF4Tensor(to_dev(codes, dev), None, to_dev(q8, dev), to_dev(scale, dev), (N, K))
    host = dict(codes=codes, absmax=None, q=q8, scale=scale)
    cols = np.unique(np.concatenate([rng.choice(N, 250, replace=False), np.arange(N - 6, N)]))
    wd = oracle_wdeq(host, (N, K), rows=cols)
    for m in (4, 16):
        x = workloads.to_bf16_bits(rng.standard_normal((m, K), dtype=np.float32))
        y = nq.linear_forward(to_dev(x, dev), t)
        torch.cuda.synchronize()
        ref = oracle.linear_forward(x, wd)
        got = _bf16_to_f32(to_host(y))[:, cols]
        e, nw = rel_err_metric(got, ref)
        log(f"  M={m}: err {e:.3e} normwise {nw:.3e}")
        assert e <= TOL
    del t
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def gemv_case(dev):
    log("preparing 28672x8192 NF4 weight on the oracle")
    w, x = workloads.gemv_inputs()
    wt, host = upload_weight(w, dev)
    return wt, host, x


@pytest.fixture(scope="module")
def linear_case(dev):
    log("preparing 4096x8192x8192 r=64 case on the oracle")
    d = workloads.linear_inputs()
    wt, host = upload_weight(d["w"], dev)
    wd = oracle_wdeq(host, d["w"].shape)
    return d, wt, wd


def tile_rows(m, tile=256, seed=78):
    """One random row inside every `tile`-row band of an m-row output, plus
    the first and last rows: every output tile of the GEMM (each row band
    crossed with all columns) holds a checked row."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rows = [lo + int(rng.integers(0, min(tile, m - lo))) for lo in range(0, m, tile)]
    return np.unique(np.array(rows + [0, m - 1]))


def test_qlora_linear_forward_sampled(dev, linear_case):
    """4096 x 8192 x 8192, r = 64: one row in every 256-row tile band, all
    8192 columns."""
    import torch

    d, wt, wd = linear_case
    s = workloads.LIN_SCALE
    y = nq.linear_forward(to_dev(d["x"], dev), wt, to_dev(d["a"], dev), to_dev(d["b"], dev), s)
    torch.cuda.synchronize()
    rows = tile_rows(d["x"].shape[0])
    ref = oracle.linear_forward(d["x"], wd, d["a"], d["b"], s, rows=rows)
    got = _bf16_to_f32(to_host(y))[rows]
    e, nw = rel_err_metric(got, ref)
    pm, p999 = plain_rel_err(got, ref)
    log(f"qlora forward {rows.size} rows x all columns: err {e:.3e} normwise {nw:.3e} "
        f"plain max {pm:.3e} plain p99.9 {p999:.3e}")
    assert e <= TOL


def test_qlora_linear_backward_input_sampled(dev, linear_case):
    """dX of the same shape: one row in every 256-row tile band, all 8192
    columns."""
    import torch

    d, wt, wd = linear_case
    s = workloads.LIN_SCALE
    dx = nq.linear_backward_input(to_dev(d["dy"], dev), wt, to_dev(d["a"], dev),
                                  to_dev(d["b"], dev), s)
    torch.cuda.synchronize()
    rows = tile_rows(d["dy"].shape[0], seed=79)
    ref = oracle.linear_backward_input(d["dy"], wd, d["a"], d["b"], s, rows=rows)
    got = _bf16_to_f32(to_host(dx))[rows]
    e, nw = rel_err_metric(got, ref)
    pm, p999 = plain_rel_err(got, ref)
    log(f"qlora input-grad {rows.size} rows x all columns: err {e:.3e} normwise {nw:.3e} "
        f"plain max {pm:.3e} plain p99.9 {p999:.3e}")
    assert e <= TOL
