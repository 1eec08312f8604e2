"""ctypes wrapper around the CPU oracle ``libnf4ref.so``.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package. It shares no code
with the GPU library ``nf4_quantize_amd`` and never imports it.

Every function takes and returns numpy arrays on the host. The arithmetic lives
in ``nf4ref.c``; this module only marshals arguments.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libnf4ref.so")
_lib = None

BLOCK = 64
DQ_BLOCK = 256
F32, BF16 = 0, 1

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            _build.build()
        L = ctypes.CDLL(_LIB_PATH)
        L.nf4ref_codebook.argtypes = [_p]
        L.nf4ref_normal_quantile.argtypes = [ctypes.c_double]
        L.nf4ref_normal_quantile.restype = ctypes.c_double
        L.nf4ref_construct_codebook.argtypes = [ctypes.c_double, _p]
        L.nf4ref_solve_delta.argtypes = [ctypes.c_double]
        L.nf4ref_solve_delta.restype = ctypes.c_double
        L.nf4ref_nearest_code.argtypes = [ctypes.c_float]
        L.nf4ref_nearest_code_array.argtypes = [_p, _i64, _p]
        L.nf4ref_bf16_to_f32.argtypes = [ctypes.c_uint16]
        L.nf4ref_bf16_to_f32.restype = ctypes.c_float
        L.nf4ref_f32_to_bf16.argtypes = [ctypes.c_float]
        L.nf4ref_f32_to_bf16.restype = ctypes.c_uint16
        L.nf4ref_f32_to_bf16_array.argtypes = [_p, _i64, _p]
        L.nf4ref_quantize.argtypes = [_p, ctypes.c_int, _i64, _p, _p]
        L.nf4ref_e4m3_encode.argtypes = [ctypes.c_float]
        L.nf4ref_e4m3_encode.restype = ctypes.c_uint8
        L.nf4ref_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.nf4ref_e4m3_decode.restype = ctypes.c_float
        L.nf4ref_e4m3_encode_array.argtypes = [_p, _i64, _p]
        L.nf4ref_double_quantize.argtypes = [_p, _i64, _p, _p]
        L.nf4ref_block_scale.argtypes = [_i64, _p, _p, _p]
        L.nf4ref_block_scale.restype = ctypes.c_float
        L.nf4ref_dequantize.argtypes = [_p, _i64, _p, _p, _p, _p, ctypes.c_int]
        L.nf4ref_dequantize_range.argtypes = [_p, _i64, _i64, _i64, _p, _p, _p, _p, ctypes.c_int]
        L.nf4ref_storage_bytes.argtypes = [_i64, ctypes.c_int]
        L.nf4ref_storage_bytes.restype = _i64
        for name in ("nf4ref_linear_forward", "nf4ref_linear_backward_input"):
            getattr(L, name).argtypes = [_p, _i64, _i64, _i64, _p, _p, _p, _i32,
                                         ctypes.c_double, _p, _i64, _p, _i64, _p]
        L.nf4ref_quantize_bs.argtypes = [_p, ctypes.c_int, _i64, _i32, _p, _p]
        L.nf4ref_e5m2_encode.argtypes = [ctypes.c_float]
        L.nf4ref_e5m2_encode.restype = ctypes.c_uint8
        L.nf4ref_e5m2_decode.argtypes = [ctypes.c_uint8]
        L.nf4ref_e5m2_decode.restype = ctypes.c_float
        L.nf4ref_e5m2_encode_array.argtypes = [_p, _i64, _p]
        L.nf4ref_pairwise_sum.argtypes = [_p, _i64]
        L.nf4ref_pairwise_sum.restype = ctypes.c_float
        L.nf4ref_double_quantize_ex.argtypes = [_p, _i64, _i32, ctypes.c_int, ctypes.c_int, _p,
                                                _p, _p]
        L.nf4ref_block_scale_ex.argtypes = [_i64, _i32, ctypes.c_int, _p, _p, _p, _p]
        L.nf4ref_block_scale_ex.restype = ctypes.c_float
        L.nf4ref_dequantize_range_ex.argtypes = [_p, _i64, _i64, _i64, _i32, _i32, ctypes.c_int,
                                                 _p, _p, _p, _p, _p, ctypes.c_int]
        L.nf4ref_merged_weight.argtypes = [_p, _p, _p, _p, _i64, _i64, _p, _p, _i32,
                                           ctypes.c_float, _p, _i64, _p]
        L.nf4ref_codebook_levels.argtypes = [ctypes.c_int, _p]
        L.nf4ref_quantize_cb.argtypes = [_p, ctypes.c_int, _i64, _i32, ctypes.c_int, _p, _p]
        L.nf4ref_dequantize_range_cb.argtypes = [_p, _i64, _i64, _i64, _i32, _i32, ctypes.c_int,
                                                 ctypes.c_int, _p, _p, _p, _p, _p, ctypes.c_int]
        L.nf4ref_storage_bytes_ex.argtypes = [_i64, _i32, _i32, ctypes.c_int, ctypes.c_int]
        L.nf4ref_storage_bytes_ex.restype = _i64
        L.nf4ref_lora_grads.argtypes = [_p, _p, _i64, _i64, _i64, _p, _p, _i32, ctypes.c_double,
                                        _p, _i64, _p, _p, _i64, _p]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its input (status {rc})")


def _as_bits(w):
    """Returns (array, dtype code) for fp32 arrays or bf16 given as uint16 bits."""
    w = np.ascontiguousarray(w)
    if w.dtype == np.float32:
        return w, F32
    if w.dtype == np.uint16:
        return w, BF16
    raise TypeError("oracle inputs are float32 or bf16 bit patterns (uint16)")


def codebook():
    q = np.zeros(16, np.float32)
    lib().nf4ref_codebook(_ptr(q))
    return q


def construct_codebook(delta):
    out = np.zeros(16, np.float64)
    _check(lib().nf4ref_construct_codebook(float(delta), _ptr(out)), "construct_codebook")
    return out


def normal_quantile(p):
    return lib().nf4ref_normal_quantile(float(p))


def solve_delta(level14):
    return lib().nf4ref_solve_delta(float(level14))


def nearest_code(n):
    return int(lib().nf4ref_nearest_code(float(np.float32(n))))


def nearest_code_array(n):
    n = np.ascontiguousarray(n, dtype=np.float32)
    out = np.zeros(n.shape, np.uint8)
    _check(lib().nf4ref_nearest_code_array(_ptr(n), n.size, _ptr(out)), "nearest_code_array")
    return out


def f32_to_bf16(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.shape, np.uint16)
    _check(lib().nf4ref_f32_to_bf16_array(_ptr(x), x.size, _ptr(out)), "f32_to_bf16")
    return out


def bf16_to_f32(h):
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def nblocks(n):
    return (n + BLOCK - 1) // BLOCK


def ngroups(n):
    return (nblocks(n) + DQ_BLOCK - 1) // DQ_BLOCK


def quantize(w):
    """Blockwise NF4: returns (packed codes uint8[ceil(n/2)], absmax float32[ceil(n/64)])."""
    w, dt = _as_bits(w)
    n = w.size
    codes = np.zeros((n + 1) // 2, np.uint8)
    absmax = np.zeros(nblocks(n), np.float32)
    _check(lib().nf4ref_quantize(_ptr(w), dt, n, _ptr(codes), _ptr(absmax)), "quantize")
    return codes, absmax


def double_quantize(absmax):
    absmax = np.ascontiguousarray(absmax, dtype=np.float32)
    nb = absmax.size
    q = np.zeros(nb, np.uint8)
    scale = np.zeros((nb + DQ_BLOCK - 1) // DQ_BLOCK, np.float32)
    _check(lib().nf4ref_double_quantize(_ptr(absmax), nb, _ptr(q), _ptr(scale)),
           "double_quantize")
    return q, scale


def e4m3_encode(r):
    r = np.ascontiguousarray(r, dtype=np.float32)
    out = np.zeros(r.shape, np.uint8)
    _check(lib().nf4ref_e4m3_encode_array(_ptr(r), r.size, _ptr(out)), "e4m3_encode")
    return out


def e4m3_decode(c):
    f = lib().nf4ref_e4m3_decode
    return np.array([f(int(v)) for v in np.asarray(c).ravel()], np.float32)


def dequantize(codes, n, absmax=None, q=None, scale=None, out_dtype=F32):
    """Returns float32[n] (out_dtype F32) or bf16 bit patterns uint16[n] (BF16)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    absmax = None if absmax is None else np.ascontiguousarray(absmax, dtype=np.float32)
    q = None if q is None else np.ascontiguousarray(q, dtype=np.uint8)
    scale = None if scale is None else np.ascontiguousarray(scale, dtype=np.float32)
    out = np.zeros(n, np.float32 if out_dtype == F32 else np.uint16)
    _check(lib().nf4ref_dequantize(_ptr(codes), n, _ptr(absmax), _ptr(q), _ptr(scale),
                                   _ptr(out), out_dtype), "dequantize")
    return out


def dequantize_range(codes, n, start, count, absmax=None, q=None, scale=None, out_dtype=F32):
    """Elements [start, start+count) of the n-element tensor (global block indices)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    absmax = None if absmax is None else np.ascontiguousarray(absmax, dtype=np.float32)
    q = None if q is None else np.ascontiguousarray(q, dtype=np.uint8)
    scale = None if scale is None else np.ascontiguousarray(scale, dtype=np.float32)
    out = np.zeros(count, np.float32 if out_dtype == F32 else np.uint16)
    _check(lib().nf4ref_dequantize_range(_ptr(codes), n, start, count, _ptr(absmax), _ptr(q),
                                         _ptr(scale), _ptr(out), out_dtype), "dequantize_range")
    return out


def dequantize_rows(codes, shape, rows, absmax=None, q=None, scale=None):
    """fp32 rows of a dequantized [N x K] weight."""
    N, K = shape
    out = np.zeros((len(rows), K), np.float32)
    for i, r in enumerate(rows):
        out[i] = dequantize_range(codes, N * K, int(r) * K, K, absmax, q, scale)
    return out


# ---- variants of the storage format (block sizes, DQ code formats, mean offset) ----

DQ_FORMATS = {"e4m3": 0, "e5m2": 1, "linear8": 2}


def _fmt(f):
    if isinstance(f, str):
        return DQ_FORMATS[f]
    return int(f)


def quantize_bs(w, blocksize=BLOCK):
    """Blockwise NF4 with block size B1: (codes uint8[ceil(n/2)], absmax float32[ceil(n/B1)])."""
    w, dt = _as_bits(w)
    n = w.size
    codes = np.zeros((n + 1) // 2, np.uint8)
    absmax = np.zeros((n + blocksize - 1) // blocksize, np.float32)
    _check(lib().nf4ref_quantize_bs(_ptr(w), dt, n, int(blocksize), _ptr(codes), _ptr(absmax)),
           "quantize_bs")
    return codes, absmax


def e5m2_encode(r):
    r = np.ascontiguousarray(r, dtype=np.float32)
    out = np.zeros(r.shape, np.uint8)
    _check(lib().nf4ref_e5m2_encode_array(_ptr(r), r.size, _ptr(out)), "e5m2_encode")
    return out


def e5m2_decode(c):
    f = lib().nf4ref_e5m2_decode
    return np.array([f(int(v)) for v in np.asarray(c).ravel()], np.float32)


def pairwise_sum(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    return np.float32(lib().nf4ref_pairwise_sum(_ptr(x), x.size))


def double_quantize_ex(absmax, dq_blocksize=DQ_BLOCK, dq_format="e4m3", mean_offset=False):
    """Returns (q uint8[nblocks], scale float32[ceil(nblocks/B2)], offset float32 or None)."""
    absmax = np.ascontiguousarray(absmax, dtype=np.float32)
    nb = absmax.size
    q = np.zeros(nb, np.uint8)
    scale = np.zeros((nb + dq_blocksize - 1) // dq_blocksize, np.float32)
    off = np.zeros(1, np.float32)
    _check(lib().nf4ref_double_quantize_ex(_ptr(absmax), nb, int(dq_blocksize), _fmt(dq_format),
                                           1 if mean_offset else 0, _ptr(q), _ptr(scale),
                                           _ptr(off)), "double_quantize_ex")
    return q, scale, (off[0] if mean_offset else None)


def block_scales_ex(nblocks, dq_blocksize=DQ_BLOCK, dq_format="e4m3", absmax=None, q=None,
                    scale=None, offset=None):
    """The reconstructed scale of every block."""
    absmax = None if absmax is None else np.ascontiguousarray(absmax, dtype=np.float32)
    q = None if q is None else np.ascontiguousarray(q, dtype=np.uint8)
    scale = None if scale is None else np.ascontiguousarray(scale, dtype=np.float32)
    off = None if offset is None else np.array([offset], np.float32)
    f = lib().nf4ref_block_scale_ex
    return np.array([f(b, int(dq_blocksize), _fmt(dq_format), _ptr(absmax), _ptr(q), _ptr(scale),
                       _ptr(off)) for b in range(nblocks)], np.float32)


def dequantize_ex(codes, n, blocksize=BLOCK, dq_blocksize=DQ_BLOCK, dq_format="e4m3",
                  absmax=None, q=None, scale=None, offset=None, out_dtype=F32, start=0,
                  count=None):
    """Elements [start, start+count) of the n-element tensor under the variant."""
    count = n - start if count is None else count
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    absmax = None if absmax is None else np.ascontiguousarray(absmax, dtype=np.float32)
    q = None if q is None else np.ascontiguousarray(q, dtype=np.uint8)
    scale = None if scale is None else np.ascontiguousarray(scale, dtype=np.float32)
    off = None if offset is None else np.array([offset], np.float32)
    out = np.zeros(count, np.float32 if out_dtype == F32 else np.uint16)
    _check(lib().nf4ref_dequantize_range_ex(_ptr(codes), n, start, count, int(blocksize),
                                            int(dq_blocksize), _fmt(dq_format), _ptr(absmax),
                                            _ptr(q), _ptr(scale), _ptr(off), _ptr(out),
                                            out_dtype), "dequantize_range_ex")
    return out


# ---- merging the adapter into the quantized base ----

def merged_weight(codes, shape, A, B, s, absmax=None, q=None, scale=None, rows=None):
    """fp32 rows of Wm = dequantize(W) + s (A B)^T (see nf4ref_merged_weight)."""
    N, K = shape
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    absmax = None if absmax is None else np.ascontiguousarray(absmax, dtype=np.float32)
    q = None if q is None else np.ascontiguousarray(q, dtype=np.uint8)
    scale = None if scale is None else np.ascontiguousarray(scale, dtype=np.float32)
    A = np.ascontiguousarray(A, dtype=np.uint16)
    B = np.ascontiguousarray(B, dtype=np.uint16)
    r = A.shape[1]
    rows = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    nr = N if rows is None else rows.size
    out = np.zeros((nr, K), np.float32)
    _check(lib().nf4ref_merged_weight(_ptr(codes), _ptr(absmax), _ptr(q), _ptr(scale), N, K,
                                      _ptr(A), _ptr(B), r, float(np.float32(s)), _ptr(rows), nr,
                                      _ptr(out)), "merged_weight")
    return out


def merge_lora(codes, shape, A, B, s, absmax=None, q=None, scale=None, dq=True):
    """Merge and re-quantize: returns (codes, absmax, q, scale) of the merged
    weight (q and scale None when dq is False) and the fp32 merged weight."""
    wm = merged_weight(codes, shape, A, B, s, absmax, q, scale)
    nc, na = quantize(wm.ravel())
    if not dq:
        return nc, na, None, None, wm
    nq8, nsc = double_quantize(na)
    return nc, na, nq8, nsc, wm


# ---- codebook swaps ----

CODEBOOKS = {"nf4": 0, "fp4": 1, "int4": 2}


def _cb(c):
    return CODEBOOKS[c] if isinstance(c, str) else int(c)


def codebook_levels(codebook):
    q = np.zeros(16, np.float32)
    _check(lib().nf4ref_codebook_levels(_cb(codebook), _ptr(q)), "codebook_levels")
    return q


def quantize_cb(w, blocksize=BLOCK, codebook="nf4"):
    """Blockwise quantization to the codebook's 16 levels: (codes, absmax)."""
    w, dt = _as_bits(w)
    n = w.size
    codes = np.zeros((n + 1) // 2, np.uint8)
    absmax = np.zeros((n + blocksize - 1) // blocksize, np.float32)
    _check(lib().nf4ref_quantize_cb(_ptr(w), dt, n, int(blocksize), _cb(codebook), _ptr(codes),
                                    _ptr(absmax)), "quantize_cb")
    return codes, absmax


def dequantize_cb(codes, n, blocksize=BLOCK, dq_blocksize=DQ_BLOCK, dq_format="e4m3",
                  codebook="nf4", absmax=None, q=None, scale=None, offset=None, out_dtype=F32,
                  start=0, count=None):
    count = n - start if count is None else count
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    absmax = None if absmax is None else np.ascontiguousarray(absmax, dtype=np.float32)
    q = None if q is None else np.ascontiguousarray(q, dtype=np.uint8)
    scale = None if scale is None else np.ascontiguousarray(scale, dtype=np.float32)
    off = None if offset is None else np.array([offset], np.float32)
    out = np.zeros(count, np.float32 if out_dtype == F32 else np.uint16)
    _check(lib().nf4ref_dequantize_range_cb(_ptr(codes), n, start, count, int(blocksize),
                                            int(dq_blocksize), _fmt(dq_format), _cb(codebook),
                                            _ptr(absmax), _ptr(q), _ptr(scale), _ptr(off),
                                            _ptr(out), out_dtype), "dequantize_range_cb")
    return out


def storage_bytes_ex(n, blocksize=BLOCK, dq_blocksize=DQ_BLOCK, dq=True, mean_offset=False):
    return int(lib().nf4ref_storage_bytes_ex(int(n), int(blocksize), int(dq_blocksize),
                                             1 if dq else 0, 1 if mean_offset else 0))


def storage_bytes(n, dq):
    return int(lib().nf4ref_storage_bytes(int(n), 1 if dq else 0))


def _index(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int64)


def linear_forward(x, wdeq, A=None, B=None, s=1.0, rows=None, cols=None):
    """x: bf16 bits uint16 [m,K]; wdeq: float32 [N,K]; A: uint16 [K,r]; B: uint16 [r,N].
    Returns float64 [len(rows), len(cols)]."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    wdeq = np.ascontiguousarray(wdeq, dtype=np.float32)
    m, K = x.shape
    N = wdeq.shape[0]
    assert wdeq.shape[1] == K
    r = 0 if A is None else A.shape[1]
    A = None if A is None else np.ascontiguousarray(A, dtype=np.uint16)
    B = None if B is None else np.ascontiguousarray(B, dtype=np.uint16)
    rows, cols = _index(rows), _index(cols)
    nr = m if rows is None else rows.size
    nc = N if cols is None else cols.size
    out = np.zeros((nr, nc), np.float64)
    _check(lib().nf4ref_linear_forward(_ptr(x), m, K, N, _ptr(wdeq), _ptr(A), _ptr(B), r,
                                       float(s), _ptr(rows), nr, _ptr(cols), nc, _ptr(out)),
           "linear_forward")
    return out


def linear_backward_input(dy, wdeq, A=None, B=None, s=1.0, rows=None, cols=None):
    """dy: bf16 bits uint16 [m,N]; wdeq: float32 [N,K]. Returns float64 [len(rows), len(cols)]."""
    dy = np.ascontiguousarray(dy, dtype=np.uint16)
    wdeq = np.ascontiguousarray(wdeq, dtype=np.float32)
    m, N = dy.shape
    K = wdeq.shape[1]
    assert wdeq.shape[0] == N
    r = 0 if A is None else A.shape[1]
    A = None if A is None else np.ascontiguousarray(A, dtype=np.uint16)
    B = None if B is None else np.ascontiguousarray(B, dtype=np.uint16)
    rows, cols = _index(rows), _index(cols)
    nr = m if rows is None else rows.size
    nc = K if cols is None else cols.size
    out = np.zeros((nr, nc), np.float64)
    _check(lib().nf4ref_linear_backward_input(_ptr(dy), m, K, N, _ptr(wdeq), _ptr(A), _ptr(B),
                                              r, float(s), _ptr(rows), nr, _ptr(cols), nc,
                                              _ptr(out)), "linear_backward_input")
    return out


def lora_grads(x, dy, A, B, s=1.0, a_rows=None, b_cols=None):
    """Adapter gradients ([MF] "Gradient Computation"): dA = s X^T (dY B^T) and
    dB = s (X A)^T dY in double. x: uint16 bf16 bits [m,K]; dy: [m,N]; A: [K,r];
    B: [r,N]. Returns (dA [len(a_rows), r], dB [r, len(b_cols)]) as float64."""
    x = np.ascontiguousarray(x, dtype=np.uint16)
    dy = np.ascontiguousarray(dy, dtype=np.uint16)
    A = np.ascontiguousarray(A, dtype=np.uint16)
    B = np.ascontiguousarray(B, dtype=np.uint16)
    m, K = x.shape
    N = dy.shape[1]
    r = A.shape[1]
    assert dy.shape[0] == m and A.shape[0] == K and B.shape == (r, N)
    a_rows, b_cols = _index(a_rows), _index(b_cols)
    na = K if a_rows is None else a_rows.size
    nb = N if b_cols is None else b_cols.size
    da = np.zeros((na, r), np.float64)
    db = np.zeros((r, nb), np.float64)
    _check(lib().nf4ref_lora_grads(_ptr(x), _ptr(dy), m, K, N, _ptr(A), _ptr(B), r, float(s),
                                   _ptr(a_rows), na, _ptr(da), _ptr(b_cols), nb, _ptr(db)),
           "lora_grads")
    return da, db
