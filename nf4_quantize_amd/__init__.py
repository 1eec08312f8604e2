"""Python binding of ``libnf4.so``, the gfx950 NF4 / double-quantization /
fused NF4-linear library (C ABI in ``include/nf4.h``).

The functions named like the C entry points (``nf4_quantize`` ...) marshal
torch device tensors into pointers and call the library; every step of the
computation runs in the library's HIP kernels. torch supplies device memory
and the current HIP stream only. The convenience layer (``quantize``,
``dequantize``, ``linear_forward`` ...) allocates outputs with ``torch.empty``
and calls those functions.

The library must be built first (``python -m nf4_quantize_amd.build``); when
it is missing every call raises ``NF4LibraryMissing`` - there is no fallback.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnf4.so")

BLOCK = 64
DQ_BLOCK = 256
NF4_F32, NF4_BF16 = 0, 1

STATUS = {
    0: "NF4_OK",
    1: "NF4_ERR_NULL",
    2: "NF4_ERR_SIZE",
    3: "NF4_ERR_UNSUPPORTED",
    4: "NF4_ERR_ALIGN",
    5: "NF4_ERR_WORKSPACE",
    6: "NF4_ERR_LAUNCH",
}

# Every extern "C" function declared in include/nf4.h.
EXPORTS = (
    "nf4_status_string",
    "nf4_codebook",
    "nf4_codebook_levels",
    "nf4_storage_bytes",
    "nf4_quantize",
    "nf4_double_quantize",
    "nf4_dequantize",
    "nf4_linear_workspace_size",
    "nf4_linear_forward",
    "nf4_linear_forward_noalloc",
    "nf4_linear_backward_input",
    "nf4_linear_kernel_path",
    "nf4_lora_backward_workspace_size",
    "nf4_lora_backward",
    "nf4_quantize_ex_workspace_size",
    "nf4_quantize_ex",
    "nf4_double_quantize_ex_workspace_size",
    "nf4_double_quantize_ex",
    "nf4_dequantize_ex",
    "nf4_merge_lora_workspace_size",
    "nf4_merge_lora",
    "nf4_storage_bytes_ex",
    "nf4_quantize_batched",
    "nf4_dequantize_batched",
)

# nf4_dq_format: the 8-bit code of double quantization.
DQ_FORMATS = {"e4m3": 0, "e5m2": 1, "linear8": 2}
# nf4_codebook_id: the 16 levels of the 4-bit code.
CODEBOOKS = {"nf4": 0, "fp4": 1, "int4": 2}


class NF4LibraryMissing(RuntimeError):
    pass


class NF4Error(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what} failed: {STATUS.get(status, status)}")


class nf4_weight(ctypes.Structure):
    _fields_ = [
        ("codes", ctypes.c_void_p),
        ("absmax_q", ctypes.c_void_p),
        ("absmax_scale", ctypes.c_void_p),
        ("absmax", ctypes.c_void_p),
        ("n_out", ctypes.c_int64),
        ("k_in", ctypes.c_int64),
        ("blocksize", ctypes.c_int32),
        ("dq_blocksize", ctypes.c_int32),
    ]


class nf4_format(ctypes.Structure):
    _fields_ = [
        ("blocksize", ctypes.c_int32),
        ("dq_blocksize", ctypes.c_int32),
        ("dq_format", ctypes.c_int32),
        ("dq_mean_offset", ctypes.c_int32),
        ("codebook", ctypes.c_int32),
    ]


class nf4_batch_entry(ctypes.Structure):
    _fields_ = [
        ("w", ctypes.c_void_p),
        ("n", ctypes.c_int64),
        ("codes", ctypes.c_void_p),
        ("absmax", ctypes.c_void_p),
        ("absmax_q", ctypes.c_void_p),
        ("absmax_scale", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """Loads libnf4.so (once). Raises NF4LibraryMissing if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise NF4LibraryMissing(
            f"{LIB_PATH} is not built; run `python -m nf4_quantize_amd.build` (hipcc, gfx950)")
    # torch ships its own HIP runtime under the same soname as ROCm's. Loading
    # torch first makes libnf4.so bind to that copy; loaded the other way
    # round, a process would hold two HIP runtimes, and torch's device
    # pointers would be foreign to the library's launches.
    import torch  # noqa: F401

    L = ctypes.CDLL(LIB_PATH)
    p, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    L.nf4_status_string.argtypes = [ctypes.c_int]
    L.nf4_status_string.restype = ctypes.c_char_p
    L.nf4_codebook.argtypes = []
    L.nf4_codebook.restype = ctypes.POINTER(ctypes.c_float)
    L.nf4_codebook_levels.argtypes = [i32]
    L.nf4_codebook_levels.restype = ctypes.POINTER(ctypes.c_float)
    L.nf4_storage_bytes.argtypes = [i64, i32, i32, i32]
    L.nf4_storage_bytes.restype = i64
    L.nf4_quantize.argtypes = [p, ctypes.c_int, i64, i32, p, p, i32, p, p, p]
    L.nf4_quantize.restype = ctypes.c_int
    L.nf4_double_quantize.argtypes = [p, i64, i32, p, p, p]
    L.nf4_double_quantize.restype = ctypes.c_int
    L.nf4_dequantize.argtypes = [p, i64, i32, p, p, p, i32, p, ctypes.c_int, p]
    L.nf4_dequantize.restype = ctypes.c_int
    L.nf4_linear_workspace_size.argtypes = [i64, i32]
    L.nf4_linear_workspace_size.restype = ctypes.c_size_t
    L.nf4_linear_kernel_path.argtypes = [i64, i64, i64, i32, i32]
    L.nf4_linear_kernel_path.restype = i32
    for name in ("nf4_linear_forward", "nf4_linear_backward_input"):
        fn = getattr(L, name)
        fn.argtypes = [p, i64, ctypes.POINTER(nf4_weight), p, p, i32, f32, p, p,
                       ctypes.c_size_t, p]
        fn.restype = ctypes.c_int
    L.nf4_linear_forward_noalloc.argtypes = [p, i64, ctypes.POINTER(nf4_weight), p, p, i32, f32,
                                             p, p]
    L.nf4_linear_forward_noalloc.restype = ctypes.c_int
    L.nf4_lora_backward_workspace_size.argtypes = [i64, i64, i64, i32]
    L.nf4_lora_backward_workspace_size.restype = ctypes.c_size_t
    L.nf4_lora_backward.argtypes = [p, p, i64, i64, i64, p, p, i32, f32, p, p, ctypes.c_int, p,
                                    ctypes.c_size_t, p]
    L.nf4_lora_backward.restype = ctypes.c_int
    fmt_p = ctypes.POINTER(nf4_format)
    L.nf4_quantize_ex_workspace_size.argtypes = [i64, fmt_p]
    L.nf4_quantize_ex_workspace_size.restype = ctypes.c_size_t
    L.nf4_double_quantize_ex_workspace_size.argtypes = [i64, fmt_p]
    L.nf4_double_quantize_ex_workspace_size.restype = ctypes.c_size_t
    L.nf4_quantize_ex.argtypes = [p, ctypes.c_int, i64, fmt_p, p, p, p, p, p, p, ctypes.c_size_t, p]
    L.nf4_quantize_ex.restype = ctypes.c_int
    L.nf4_double_quantize_ex.argtypes = [p, i64, fmt_p, p, p, p, p, ctypes.c_size_t, p]
    L.nf4_double_quantize_ex.restype = ctypes.c_int
    L.nf4_dequantize_ex.argtypes = [p, i64, fmt_p, p, p, p, p, p, ctypes.c_int, p]
    L.nf4_dequantize_ex.restype = ctypes.c_int
    L.nf4_storage_bytes_ex.argtypes = [i64, fmt_p, i32]
    for fn in (L.nf4_quantize_batched, L.nf4_dequantize_batched):
        fn.argtypes = [ctypes.POINTER(nf4_batch_entry), i32, ctypes.c_int, p]
        fn.restype = ctypes.c_int
    L.nf4_storage_bytes_ex.restype = i64
    L.nf4_merge_lora_workspace_size.argtypes = [i64, i64]
    L.nf4_merge_lora_workspace_size.restype = ctypes.c_size_t
    L.nf4_merge_lora.argtypes = [ctypes.POINTER(nf4_weight), p, p, i32, f32, p, p, p, p, p,
                                 ctypes.c_size_t, p]
    L.nf4_merge_lora.restype = ctypes.c_int
    _lib = L
    return L


def _check(status, what):
    if status != 0:
        raise NF4Error(status, what)


# ------------------------------------------------------------------ marshalling

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt):
    import torch

    if dt == torch.float32:
        return NF4_F32
    if dt == torch.bfloat16:
        return NF4_BF16
    raise TypeError(f"unsupported dtype {dt}: float32 or bfloat16")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


# ------------------------------------------------------------- C-named calls

def nf4_codebook():
    cb = lib().nf4_codebook()
    return [cb[i] for i in range(16)]


def nf4_codebook_levels(codebook="nf4"):
    cb = lib().nf4_codebook_levels(CODEBOOKS[codebook] if isinstance(codebook, str) else codebook)
    if not cb:
        raise ValueError(f"unknown codebook {codebook!r}")
    return [cb[i] for i in range(16)]


def nf4_storage_bytes(n, double_quant=True, blocksize=BLOCK, dq_blocksize=DQ_BLOCK):
    return int(lib().nf4_storage_bytes(n, blocksize, dq_blocksize, 1 if double_quant else 0))


def nf4_quantize(w, codes, absmax=None, absmax_q=None, absmax_scale=None,
                 blocksize=BLOCK, dq_blocksize=DQ_BLOCK):
    """w: float32/bfloat16 device tensor (any shape, flattened). Outputs as in nf4.h."""
    _need_cuda(w, codes, absmax, absmax_q, absmax_scale)
    st = lib().nf4_quantize(_ptr(w), _dtype_code(w.dtype), w.numel(), blocksize, _ptr(codes),
                            _ptr(absmax), dq_blocksize, _ptr(absmax_q), _ptr(absmax_scale),
                            _stream(w.device))
    _check(st, "nf4_quantize")


def nf4_double_quantize(absmax, absmax_q, absmax_scale, dq_blocksize=DQ_BLOCK):
    _need_cuda(absmax, absmax_q, absmax_scale)
    st = lib().nf4_double_quantize(_ptr(absmax), absmax.numel(), dq_blocksize, _ptr(absmax_q),
                                   _ptr(absmax_scale), _stream(absmax.device))
    _check(st, "nf4_double_quantize")


def nf4_dequantize(codes, n, out, absmax=None, absmax_q=None, absmax_scale=None,
                   blocksize=BLOCK, dq_blocksize=DQ_BLOCK):
    _need_cuda(codes, out, absmax, absmax_q, absmax_scale)
    st = lib().nf4_dequantize(_ptr(codes), n, blocksize, _ptr(absmax), _ptr(absmax_q),
                              _ptr(absmax_scale), dq_blocksize, _ptr(out), _dtype_code(out.dtype),
                              _stream(codes.device))
    _check(st, "nf4_dequantize")


def nf4_linear_workspace_size(m, r):
    return int(lib().nf4_linear_workspace_size(m, r))


LINEAR_PATHS = {1: "decode", 2: "mfma", 3: "portable"}


def linear_kernel_path(m, n_out, k_in, r=0, backward=False):
    """Kernel family of a linear call of this shape (nf4_linear_kernel_path):
    "decode", "mfma", or "portable" (the fp32 fallback without matrix
    cores); None for a shape the calls reject."""
    return LINEAR_PATHS.get(int(lib().nf4_linear_kernel_path(m, n_out, k_in, r, 1 if backward else 0)))


def _addr(t):
    return None if t is None else t.data_ptr()


def _batch(ws, ts, what):
    """nf4_batch_entry array of (dense tensor, NF4Tensor) pairs, and their
    common dense dtype code."""
    if len(ws) != len(ts):
        raise ValueError(f"{what}: {len(ws)} dense tensors for {len(ts)} NF4 tensors")
    dts = {w.dtype for w in ws}
    if len(dts) > 1:
        raise ValueError(f"{what}: one dtype per call, got {sorted(map(str, dts))}")
    arr = (nf4_batch_entry * max(1, len(ws)))()
    for i, (w, t) in enumerate(zip(ws, ts)):
        _need_cuda(w, t.codes, t.absmax, t.absmax_q, t.absmax_scale)
        if not t.fmt.is_default:
            raise ValueError(f"{what}: batched calls take the default storage format")
        if w.numel() != t.numel:
            raise ValueError(f"{what}: entry {i} has {w.numel()} elements, its NF4 tensor {t.numel}")
        arr[i] = nf4_batch_entry(_addr(w), w.numel(), _addr(t.codes), _addr(t.absmax),
                                 _addr(t.absmax_q), _addr(t.absmax_scale))
    return arr, (_dtype_code(ws[0].dtype) if ws else NF4_BF16)


class NF4Batch:
    """A batched call prepared once: the nf4_batch_entry array pairing dense
    tensors ws[i] with NF4 tensors ts[i] is built here (the per-entry checks
    and marshalling cost microseconds per entry of host time) and reused by
    every quantize() / dequantize(). Holds references to all tensors."""

    def __init__(self, ws, ts):
        self._keep = (list(ws), list(ts))
        self.arr, self.dtype = _batch(self._keep[0], self._keep[1], "NF4Batch")
        self.count = len(self._keep[0])
        self.device = self._keep[1][0].codes.device if self.count else None

    def quantize(self):
        """nf4_quantize_batched: ws[i] -> ts[i]."""
        if self.count:
            _check(lib().nf4_quantize_batched(self.arr, self.count, self.dtype,
                                              _stream(self.device)), "nf4_quantize_batched")

    def dequantize(self):
        """nf4_dequantize_batched: ts[i] -> ws[i]."""
        if self.count:
            _check(lib().nf4_dequantize_batched(self.arr, self.count, self.dtype,
                                                _stream(self.device)), "nf4_dequantize_batched")


def nf4_quantize_batched(ws, outs):
    """nf4_quantize of ws[i] into outs[i] (NF4Tensor, default format) for
    every i, in few launches. All ws share one dtype and one device."""
    NF4Batch(ws, outs).quantize()


def nf4_dequantize_batched(ts, outs):
    """nf4_dequantize of ts[i] (NF4Tensor, default format) into outs[i] for
    every i, in few launches. All outs share one dtype and one device."""
    NF4Batch(outs, ts).dequantize()


@dataclass(frozen=True)
class NF4Format:
    """Storage-format variant (nf4_format in nf4.h): block size B1, DQ block
    B2, the 8-bit code format of double quantization ("e4m3", "e5m2",
    "linear8"), the tensor-wide mean offset, and the 4-bit codebook ("nf4",
    "fp4", "int4")."""
    blocksize: int = BLOCK
    dq_blocksize: int = DQ_BLOCK
    dq_format: str = "e4m3"
    mean_offset: bool = False
    codebook: str = "nf4"

    @property
    def is_default(self):
        return self == NF4Format()

    def struct(self):
        if self.dq_format not in DQ_FORMATS:
            raise ValueError(f"dq_format must be one of {sorted(DQ_FORMATS)}")
        if self.codebook not in CODEBOOKS:
            raise ValueError(f"codebook must be one of {sorted(CODEBOOKS)}")
        return nf4_format(self.blocksize, self.dq_blocksize, DQ_FORMATS[self.dq_format],
                          1 if self.mean_offset else 0, CODEBOOKS[self.codebook])

    def nblocks(self, n):
        return (n + self.blocksize - 1) // self.blocksize

    def ngroups(self, n):
        return (self.nblocks(n) + self.dq_blocksize - 1) // self.dq_blocksize


def _ws_size(fn, n, fmt):
    size = fn(n, ctypes.byref(fmt.struct()))
    if size == ctypes.c_size_t(-1).value:
        raise NF4Error(3, fn.__name__)
    return int(size)


def nf4_storage_bytes_ex(n, fmt: NF4Format, double_quant=True):
    return int(lib().nf4_storage_bytes_ex(n, ctypes.byref(fmt.struct()), 1 if double_quant else 0))


def nf4_quantize_ex_workspace_size(n, fmt: NF4Format):
    return _ws_size(lib().nf4_quantize_ex_workspace_size, n, fmt)


def nf4_double_quantize_ex_workspace_size(nblocks, fmt: NF4Format):
    return _ws_size(lib().nf4_double_quantize_ex_workspace_size, nblocks, fmt)


def _workspace(size, device):
    import torch

    return torch.empty(max(size, 1), dtype=torch.uint8, device=device) if size else None


def nf4_quantize_ex(w, fmt: NF4Format, codes, absmax=None, absmax_q=None, absmax_scale=None,
                    absmax_offset=None, workspace=None):
    _need_cuda(w, codes, absmax, absmax_q, absmax_scale, absmax_offset, workspace)
    if workspace is None and absmax_q is not None:
        workspace = _workspace(nf4_quantize_ex_workspace_size(w.numel(), fmt), w.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = lib().nf4_quantize_ex(_ptr(w), _dtype_code(w.dtype), w.numel(), ctypes.byref(fmt.struct()),
                               _ptr(codes), _ptr(absmax), _ptr(absmax_q), _ptr(absmax_scale),
                               _ptr(absmax_offset), _ptr(workspace), ws_bytes, _stream(w.device))
    _check(st, "nf4_quantize_ex")


def nf4_double_quantize_ex(absmax, fmt: NF4Format, absmax_q, absmax_scale, absmax_offset=None,
                           workspace=None):
    _need_cuda(absmax, absmax_q, absmax_scale, absmax_offset, workspace)
    if workspace is None:
        workspace = _workspace(nf4_double_quantize_ex_workspace_size(absmax.numel(), fmt),
                               absmax.device)
    ws_bytes = 0 if workspace is None else workspace.numel()
    st = lib().nf4_double_quantize_ex(_ptr(absmax), absmax.numel(), ctypes.byref(fmt.struct()),
                                      _ptr(absmax_q), _ptr(absmax_scale), _ptr(absmax_offset),
                                      _ptr(workspace), ws_bytes, _stream(absmax.device))
    _check(st, "nf4_double_quantize_ex")


def nf4_dequantize_ex(codes, n, fmt: NF4Format, out, absmax=None, absmax_q=None,
                      absmax_scale=None, absmax_offset=None):
    _need_cuda(codes, out, absmax, absmax_q, absmax_scale, absmax_offset)
    st = lib().nf4_dequantize_ex(_ptr(codes), n, ctypes.byref(fmt.struct()), _ptr(absmax),
                                 _ptr(absmax_q), _ptr(absmax_scale), _ptr(absmax_offset),
                                 _ptr(out), _dtype_code(out.dtype), _stream(codes.device))
    _check(st, "nf4_dequantize_ex")


# ------------------------------------------------------------- convenience

@dataclass
class NF4Config:
    """The four quantization knobs of the pages' configuration ("Lesson 15. NF4
    and Double Quantisation", "The configuration"), plus the block sizes.
    Only NF4 storage with bf16 compute is supported."""
    load_in_4bit: bool = True
    quant_type: str = "nf4"
    use_double_quant: bool = True
    compute_dtype: str = "bfloat16"
    blocksize: int = BLOCK
    dq_blocksize: int = DQ_BLOCK
    dq_format: str = "e4m3"
    dq_mean_offset: bool = False

    def validate(self):
        if not self.load_in_4bit:
            raise ValueError("only 4-bit storage is implemented")
        if self.quant_type != "nf4":
            raise ValueError("only quant_type='nf4' is implemented")
        if str(self.compute_dtype).replace("torch.", "") != "bfloat16":
            raise ValueError("only bfloat16 compute is implemented")
        self.format().struct()
        if self.blocksize not in (16, 32, 64, 128, 256, 512, 1024, 2048, 4096):
            raise ValueError("blocksize: a power of two in [16, 4096]")
        if self.dq_blocksize < 1 or self.dq_blocksize > 4096 or \
                self.dq_blocksize & (self.dq_blocksize - 1):
            raise ValueError("dq_blocksize: a power of two in [1, 4096]")
        return self

    def format(self):
        return NF4Format(self.blocksize, self.dq_blocksize, self.dq_format, self.dq_mean_offset)


@dataclass
class NF4Tensor:
    """Packed NF4 storage of a tensor of `shape` (row-major flattening)."""
    codes: "object"
    absmax: Optional["object"]
    absmax_q: Optional["object"]
    absmax_scale: Optional["object"]
    shape: Tuple[int, ...]
    fmt: NF4Format = NF4Format()
    absmax_offset: Optional["object"] = None

    @property
    def numel(self):
        n = 1
        for d in self.shape:
            n *= d
        return n

    @property
    def double_quant(self):
        return self.absmax_q is not None

    def storage_bytes(self):
        return sum(t.numel() * t.element_size() for t in
                   (self.codes, self.absmax, self.absmax_q, self.absmax_scale, self.absmax_offset)
                   if t is not None)

    def weight_struct(self):
        """nf4_weight view of a 2-D [N x K] weight (keep self alive while used)."""
        if len(self.shape) != 2:
            raise ValueError("a linear weight is 2-D [n_out x k_in]")
        if not self.fmt.is_default:
            raise ValueError("the fused linear kernels take the default storage format "
                             "(B1 = 64, B2 = 256, E4M3, no mean offset)")
        return nf4_weight(
            codes=self.codes.data_ptr(),
            absmax_q=self.absmax_q.data_ptr() if self.absmax_q is not None else None,
            absmax_scale=self.absmax_scale.data_ptr() if self.absmax_scale is not None else None,
            absmax=self.absmax.data_ptr() if self.absmax is not None else None,
            n_out=self.shape[0], k_in=self.shape[1], blocksize=BLOCK, dq_blocksize=DQ_BLOCK)


def nblocks(n):
    return (n + BLOCK - 1) // BLOCK


def ngroups(n):
    return (nblocks(n) + DQ_BLOCK - 1) // DQ_BLOCK


def empty_nf4(shape, device, double_quant=True, keep_absmax=False, fmt: NF4Format = None):
    import torch

    fmt = fmt or NF4Format()
    n = 1
    for d in shape:
        n *= d
    nb, ng = fmt.nblocks(n), fmt.ngroups(n)
    codes = torch.empty((n + 1) // 2, dtype=torch.uint8, device=device)
    absmax = (torch.empty(nb, dtype=torch.float32, device=device)
              if (keep_absmax or not double_quant) else None)
    q = torch.empty(nb, dtype=torch.uint8, device=device) if double_quant else None
    sc = torch.empty(ng, dtype=torch.float32, device=device) if double_quant else None
    off = (torch.empty(1, dtype=torch.float32, device=device)
           if (double_quant and fmt.mean_offset) else None)
    return NF4Tensor(codes, absmax, q, sc, tuple(shape), fmt, off)


def quantize(w, double_quant=True, keep_absmax=False, out: Optional[NF4Tensor] = None,
             fmt: NF4Format = None):
    """Blockwise NF4 (+ double quantization) of a float32/bfloat16 device tensor,
    in the default storage format or the variant `fmt`."""
    fmt = out.fmt if out is not None else (fmt or NF4Format())
    t = out if out is not None else empty_nf4(tuple(w.shape), w.device, double_quant, keep_absmax,
                                               fmt)
    if fmt.is_default:
        nf4_quantize(w.contiguous(), t.codes, t.absmax, t.absmax_q, t.absmax_scale)
    else:
        nf4_quantize_ex(w.contiguous(), fmt, t.codes, t.absmax, t.absmax_q, t.absmax_scale,
                        t.absmax_offset)
    return t


def quantize_batched(ws, double_quant=True, keep_absmax=False):
    """quantize() of every tensor of the list ws (one dtype, one device), in
    few launches; returns the list of NF4Tensor."""
    outs = [empty_nf4(tuple(w.shape), w.device, double_quant, keep_absmax) for w in ws]
    nf4_quantize_batched([w.contiguous() for w in ws], outs)
    return outs


def dequantize_batched(ts, out_dtype=None):
    """dequantize() of every NF4Tensor of the list ts, in few launches."""
    import torch

    out_dtype = out_dtype or torch.bfloat16
    outs = [torch.empty(t.shape, dtype=out_dtype, device=t.codes.device) for t in ts]
    nf4_dequantize_batched(ts, outs)
    return outs


def double_quantize(absmax, fmt: NF4Format = None):
    """Returns (absmax_q, absmax_scale), plus the offset tensor when fmt has
    the mean offset."""
    import torch

    fmt = fmt or NF4Format()
    nb = absmax.numel()
    q = torch.empty(nb, dtype=torch.uint8, device=absmax.device)
    sc = torch.empty((nb + fmt.dq_blocksize - 1) // fmt.dq_blocksize, dtype=torch.float32,
                     device=absmax.device)
    if fmt == NF4Format(blocksize=fmt.blocksize):
        nf4_double_quantize(absmax, q, sc)
        return q, sc
    off = torch.empty(1, dtype=torch.float32, device=absmax.device) if fmt.mean_offset else None
    nf4_double_quantize_ex(absmax, fmt, q, sc, off)
    return (q, sc, off) if fmt.mean_offset else (q, sc)


def dequantize(t: NF4Tensor, out_dtype=None, out=None):
    import torch

    out_dtype = out_dtype or torch.bfloat16
    if out is None:
        out = torch.empty(t.shape, dtype=out_dtype, device=t.codes.device)
    if not t.fmt.is_default:
        if t.double_quant:
            nf4_dequantize_ex(t.codes, t.numel, t.fmt, out, absmax_q=t.absmax_q,
                              absmax_scale=t.absmax_scale, absmax_offset=t.absmax_offset)
        else:
            nf4_dequantize_ex(t.codes, t.numel, t.fmt, out, absmax=t.absmax)
    elif t.double_quant:
        nf4_dequantize(t.codes, t.numel, out, absmax_q=t.absmax_q, absmax_scale=t.absmax_scale)
    else:
        nf4_dequantize(t.codes, t.numel, out, absmax=t.absmax)
    return out


def _linear(name, act, w: NF4Tensor, lora_a, lora_b, lora_scale, out_cols, out=None,
            workspace=None):
    import torch

    _need_cuda(act, lora_a, lora_b, out, workspace)
    if act.dtype != torch.bfloat16:
        raise TypeError("activations are bfloat16")
    m = act.shape[0]
    r = 0 if lora_a is None else lora_a.shape[1]
    if out is None:
        out = torch.empty((m, out_cols), dtype=torch.bfloat16, device=act.device)
    ws_bytes = nf4_linear_workspace_size(m, r)
    if workspace is None and ws_bytes:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=act.device)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    ws = w.weight_struct()
    st = getattr(lib(), name)(_ptr(act), m, ctypes.byref(ws), _ptr(lora_a), _ptr(lora_b), r,
                              float(lora_scale), _ptr(out), _ptr(workspace), ws_len,
                              _stream(act.device))
    _check(st, name)
    return out


def nf4_linear_forward(x, w: NF4Tensor, lora_a=None, lora_b=None, lora_scale=1.0, out=None,
                       workspace=None):
    """Y = X . dequantize(W)^T + lora_scale * (X . A) . B; x bf16 [m x K], W [N x K]."""
    return _linear("nf4_linear_forward", x, w, lora_a, lora_b, lora_scale, w.shape[0], out,
                   workspace)


NF4_NOALLOC_SCRATCH_BYTES = 32 << 20  # include/nf4.h


def nf4_linear_forward_noalloc(x, w: NF4Tensor, lora_a=None, lora_b=None, lora_scale=1.0,
                               out=None):
    """nf4_linear_forward without a workspace: the library's static device
    scratch stands in for it (nothing is allocated by the call when `out` is
    given). Calls that overlap on one GPU race on that scratch."""
    import torch

    _need_cuda(x, lora_a, lora_b, out)
    if x.dtype != torch.bfloat16:
        raise TypeError("activations are bfloat16")
    m = x.shape[0]
    r = 0 if lora_a is None else lora_a.shape[1]
    if out is None:
        out = torch.empty((m, w.shape[0]), dtype=torch.bfloat16, device=x.device)
    ws = w.weight_struct()
    st = lib().nf4_linear_forward_noalloc(_ptr(x), m, ctypes.byref(ws), _ptr(lora_a),
                                          _ptr(lora_b), r, float(lora_scale), _ptr(out),
                                          _stream(x.device))
    _check(st, "nf4_linear_forward_noalloc")
    return out


def nf4_linear_backward_input(dy, w: NF4Tensor, lora_a=None, lora_b=None, lora_scale=1.0,
                              out=None, workspace=None):
    """dX = dY . dequantize(W) + lora_scale * (dY . B^T) . A^T; dy bf16 [m x N]."""
    return _linear("nf4_linear_backward_input", dy, w, lora_a, lora_b, lora_scale, w.shape[1],
                   out, workspace)


def nf4_lora_backward_workspace_size(m, k_in, n_out, r):
    return int(lib().nf4_lora_backward_workspace_size(int(m), int(k_in), int(n_out), int(r)))


def nf4_lora_backward(x, dy, lora_a, lora_b, lora_scale=1.0, grad_dtype=None, grad_a=True,
                      grad_b=True, workspace=None):
    """Adapter gradients: dA = lora_scale * X^T (dY B^T) [K x r] and
    dB = lora_scale * (X A)^T dY [r x N]; x bf16 [m x K], dy bf16 [m x N],
    lora_a [K x r], lora_b [r x N]. grad_a / grad_b: True (allocate), False
    (skip) or an output tensor. Returns (dA or None, dB or None)."""
    import torch

    if grad_dtype is None:
        grad_dtype = torch.float32
    _need_cuda(x, dy, lora_a, lora_b, workspace)
    for t in (x, dy, lora_a, lora_b):
        if t.dtype != torch.bfloat16:
            raise TypeError("activations, gradients and adapters are bfloat16")
    m, K = x.shape
    N = dy.shape[1]
    r = lora_a.shape[1]
    dev = x.device

    def out(spec, shape):
        if spec is True:
            return torch.empty(shape, dtype=grad_dtype, device=dev)
        if spec is False or spec is None:
            return None
        _need_cuda(spec)
        return spec

    ga, gb = out(grad_a, (K, r)), out(grad_b, (r, N))
    for g in (ga, gb):
        if g is not None and g.dtype != grad_dtype:
            raise TypeError("gradient outputs must have grad_dtype")
    ws_bytes = nf4_lora_backward_workspace_size(m, K, N, r)
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    ws_len = workspace.numel() * workspace.element_size()
    st = lib().nf4_lora_backward(_ptr(x), _ptr(dy), m, K, N, _ptr(lora_a), _ptr(lora_b), r,
                                 float(lora_scale), _ptr(ga), _ptr(gb), _dtype_code(grad_dtype),
                                 _ptr(workspace), ws_len, _stream(dev))
    _check(st, "nf4_lora_backward")
    return ga, gb


linear_forward = nf4_linear_forward
linear_backward_input = nf4_linear_backward_input
lora_backward = nf4_lora_backward


# ------------------------------------------------- merging the adapter

def nf4_merge_lora_workspace_size(n_out, k_in):
    return int(lib().nf4_merge_lora_workspace_size(n_out, k_in))


def nf4_merge_lora(w: NF4Tensor, lora_a, lora_b, lora_scale, out: NF4Tensor, workspace=None):
    """W_out = quantize(dequantize(w) + lora_scale (A B)^T) into out's buffers
    (out may be w itself: an in-place merge)."""
    _need_cuda(lora_a, lora_b, out.codes, out.absmax, out.absmax_q, out.absmax_scale, workspace)
    if out.absmax_q is not None and out.absmax is None and workspace is None:
        workspace = _workspace(nf4_merge_lora_workspace_size(*w.shape), lora_a.device)
    ws = w.weight_struct()
    st = lib().nf4_merge_lora(ctypes.byref(ws), _ptr(lora_a), _ptr(lora_b), lora_a.shape[1],
                              float(lora_scale), _ptr(out.codes), _ptr(out.absmax),
                              _ptr(out.absmax_q), _ptr(out.absmax_scale), _ptr(workspace),
                              0 if workspace is None else workspace.numel(),
                              _stream(lora_a.device))
    _check(st, "nf4_merge_lora")
    return out


def merge_lora(w: NF4Tensor, lora_a, lora_b, lora_scale=1.0, out: Optional[NF4Tensor] = None,
               double_quant=None, keep_absmax=False, workspace=None):
    """Merges the adapter (A [K x r], B [r x N] bf16) into the NF4 weight w
    [N x K] and re-quantizes; returns the merged NF4Tensor (new buffers unless
    `out` is given; `out=w` merges in place)."""
    if out is None:
        dq = w.double_quant if double_quant is None else double_quant
        out = empty_nf4(w.shape, w.codes.device, dq, keep_absmax)
    return nf4_merge_lora(w, lora_a, lora_b, lora_scale, out, workspace)


lora_merge = merge_lora


# ------------------------------------------------- codebook comparison

def quantization_mse(w, fmt: NF4Format = None, double_quant=True):
    """Mean squared error of quantizing then dequantizing the device tensor w
    in format `fmt` (the codebook comparison of NF4 against FP4 and Int4).
    Quantization and dequantization run in the library's kernels; the error
    is reduced with torch on the device (float64)."""
    import torch

    t = quantize(w, double_quant=double_quant, fmt=fmt)
    d = dequantize(t, out_dtype=torch.float32)
    return float(((d.double() - w.double()) ** 2).mean())



# ------------------------------------------------------------ serialization

# The packed storage is its own file format: every part of an NF4Tensor is a
# tensor of the file, and the shape and storage format go into its metadata.
# Bytes are written and read back unchanged, so a loaded weight dequantizes to
# exactly what the saved one did ("QLoRA in Production: 4-bit NormalFloat &
# Double Quantization Deep Dive", "Step 4: Merging and Inference", keeps the
# quantized base on disk between training and serving).
_PARTS = ("codes", "absmax", "absmax_q", "absmax_scale", "absmax_offset")
_FILE_TAG = "nf4-packed-v1"


def _expected_parts(shape, fmt: NF4Format, parts):
    n = 1
    for d in shape:
        n *= d
    sizes = {"codes": (n + 1) // 2, "absmax": fmt.nblocks(n), "absmax_q": fmt.nblocks(n),
             "absmax_scale": fmt.ngroups(n), "absmax_offset": 1}
    dtypes = {"codes": "uint8", "absmax": "float32", "absmax_q": "uint8",
              "absmax_scale": "float32", "absmax_offset": "float32"}
    return {p: (sizes[p], dtypes[p]) for p in parts}


def save_nf4(path, tensors):
    """Write the dict {name: NF4Tensor} to the safetensors file `path`.
    Each present part is copied to host memory as it is; nothing is
    re-quantized."""
    import json
    from safetensors.torch import save_file

    if not tensors:
        raise ValueError("nothing to save")
    flat, meta = {}, {}
    for name, t in tensors.items():
        if "." in name:
            raise ValueError(f"tensor name {name!r}: '.' separates a name from its parts")
        parts = [p for p in _PARTS if getattr(t, p) is not None]
        for p in parts:
            flat[f"{name}.{p}"] = getattr(t, p).detach().contiguous().cpu()
        f = t.fmt
        meta[name] = {"shape": list(t.shape), "blocksize": f.blocksize,
                      "dq_blocksize": f.dq_blocksize, "dq_format": f.dq_format,
                      "mean_offset": bool(f.mean_offset), "codebook": f.codebook,
                      "parts": parts}
    save_file(flat, path, metadata={"format": _FILE_TAG, "nf4": json.dumps(meta)})


def load_nf4(path, device="cpu"):
    """Read a file written by save_nf4 into {name: NF4Tensor} on `device`.
    Raises ValueError when a part is missing or has the wrong size or type
    for the recorded shape and format."""
    import json
    from safetensors import safe_open

    out = {}
    with safe_open(path, framework="pt", device="cpu") as fh:
        md = fh.metadata() or {}
        if md.get("format") != _FILE_TAG:
            raise ValueError(f"{path}: not an NF4 packed file")
        meta = json.loads(md["nf4"])
        keys = set(fh.keys())
        for name, m in meta.items():
            fmt = NF4Format(m["blocksize"], m["dq_blocksize"], m["dq_format"],
                            bool(m["mean_offset"]), m["codebook"])
            fmt.struct()
            shape = tuple(int(d) for d in m["shape"])
            parts = {}
            for p, (size, dt) in _expected_parts(shape, fmt, m["parts"]).items():
                key = f"{name}.{p}"
                if key not in keys:
                    raise ValueError(f"{path}: {key} is missing")
                t = fh.get_tensor(key)
                if t.dim() != 1 or t.numel() != size or str(t.dtype) != f"torch.{dt}":
                    raise ValueError(f"{path}: {key} is {tuple(t.shape)} {t.dtype}, "
                                     f"expected ({size},) {dt}")
                parts[p] = t.to(device)
            if "codes" not in parts or (("absmax_q" in parts) != ("absmax_scale" in parts)) \
                    or ("absmax" not in parts and "absmax_q" not in parts):
                raise ValueError(f"{path}: {name} lacks the parts its scales need")
            out[name] = NF4Tensor(parts["codes"], parts.get("absmax"), parts.get("absmax_q"),
                                  parts.get("absmax_scale"), shape, fmt,
                                  parts.get("absmax_offset"))
    return out


# ------------------------------------------------------- autograd integration

# The QLoRA linear as a torch autograd function ("QLoRA: Mathematical
# Foundations of 4-Bit NormalFloat Quantization, Double Quantization, and
# Paged Optimizers", "Forward Pass Computation" and "Gradient Computation"):
# forward Y = X W'^T + s (X A) B with W' the dequantized frozen base, backward
# dX from nf4_linear_backward_input and dA, dB from nf4_lora_backward. The base
# gets no gradient. Every product runs in the library's kernels; this layer
# only reshapes and routes tensors.
def _autograd_function():
    import torch

    class NF4LoRALinearFunction(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x, lora_a, lora_b, weight, lora_scale):
            lead = x.shape[:-1]
            x2 = x.reshape(-1, x.shape[-1]).contiguous()
            y = nf4_linear_forward(x2, weight, lora_a, lora_b, lora_scale)
            ctx.save_for_backward(x2, lora_a, lora_b)
            ctx.weight, ctx.lora_scale, ctx.lead = weight, lora_scale, lead
            return y.reshape(*lead, y.shape[-1])

        @staticmethod
        def backward(ctx, dy):
            x2, lora_a, lora_b = ctx.saved_tensors
            dy2 = dy.reshape(-1, dy.shape[-1]).to(torch.bfloat16).contiguous()
            dx = da = db = None
            if ctx.needs_input_grad[0]:
                dx = nf4_linear_backward_input(dy2, ctx.weight, lora_a, lora_b, ctx.lora_scale)
                dx = dx.reshape(*ctx.lead, dx.shape[-1])
            want_a, want_b = ctx.needs_input_grad[1], ctx.needs_input_grad[2]
            if want_a or want_b:
                da, db = nf4_lora_backward(x2, dy2, lora_a, lora_b, ctx.lora_scale, grad_dtype=lora_a.dtype,
                                           grad_a=want_a, grad_b=want_b)
            return dx, da, db, None, None

    return NF4LoRALinearFunction


_FN = None


def nf4_lora_linear(x, weight: NF4Tensor, lora_a, lora_b, lora_scale=1.0):
    """Differentiable QLoRA linear: x bf16 [..., K], weight NF4 [N x K] (frozen),
    lora_a bf16 [K x r], lora_b bf16 [r x N]; returns bf16 [..., N]. Gradients
    flow to x, lora_a and lora_b."""
    global _FN
    if _FN is None:
        _FN = _autograd_function()
    return _FN.apply(x, lora_a, lora_b, weight, float(lora_scale))


def make_lora_linear_module():
    """torch.nn.Module class of a QLoRA linear layer (created on first use so
    that importing this package does not import torch)."""
    import math

    import torch

    class NF4LoRALinear(torch.nn.Module):
        """A linear layer whose weight is stored in NF4 (+ double quantization)
        and frozen, with a trainable low-rank adapter: y = x W'^T + (alpha / r)
        (x A) B. A starts random (Kaiming-uniform bound), B at zero, so the
        layer starts as the quantized base alone."""

        def __init__(self, weight, r=64, alpha=16.0, generator=None):
            super().__init__()
            if not isinstance(weight, NF4Tensor):
                weight = quantize(weight.to(torch.bfloat16).contiguous())
            n_out, k_in = weight.shape
            dev = weight.codes.device
            self.weight = weight
            self.r, self.scale = r, float(alpha) / r
            bound = 1.0 / math.sqrt(k_in)
            a = (torch.rand((k_in, r), generator=generator, device=dev) * 2 - 1) * bound
            self.lora_a = torch.nn.Parameter(a.to(torch.bfloat16))
            self.lora_b = torch.nn.Parameter(torch.zeros((r, n_out), dtype=torch.bfloat16, device=dev))

        def forward(self, x):
            return nf4_lora_linear(x, self.weight, self.lora_a, self.lora_b, self.scale)

        def merged(self):
            """The adapter merged into the base and re-quantized (nf4_merge_lora)."""
            return merge_lora(self.weight, self.lora_a.detach(), self.lora_b.detach(), self.scale)

    return NF4LoRALinear
