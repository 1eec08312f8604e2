"""The C-ABI library loads and exports every function include/nf4.h declares,
and its host-side validation rejects bad arguments before any HIP call
(CPU only: no call here reaches a kernel launch).
"""
import ctypes
import os
import re

import numpy as np
import pytest

from conftest import ROOT

import nf4_quantize_amd as nq

FAKE = 0x10000  # a 16-byte-aligned, never dereferenced address


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nq.LIB_PATH):
        from nf4_quantize_amd import build

        build.build()
    return nq.lib()


def header_functions():
    text = open(os.path.join(ROOT, "include", "nf4.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(nf4_[a-z_0-9]+)\s*\(", text)
    return sorted(set(names))


def test_exports_match_header(L):
    declared = header_functions()
    assert declared == sorted(nq.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name
    out = os.popen(f"nm -D --defined-only {nq.LIB_PATH}").read()
    exported = sorted(set(re.findall(r"\b(nf4_[a-z_0-9]+)\b", out)))
    assert exported == declared


def test_codebook_is_printed_table(L, printed_codebook):
    assert np.array_equal(np.array(nq.nf4_codebook(), np.float64), printed_codebook)


def test_storage_bytes(L):
    assert nq.nf4_storage_bytes(1 << 20) == 540_928
    assert nq.nf4_storage_bytes(1 << 20, double_quant=False) == (1 << 19) + 4 * (1 << 14)
    assert nq.nf4_storage_bytes(11008 * 4096) / (11008 * 4096) == 0.515869140625
    assert L.nf4_storage_bytes(-1, 64, 256, 1) == -1
    assert L.nf4_storage_bytes(64, 32, 256, 1) == -1
    assert L.nf4_storage_bytes(64, 64, 128, 1) == -1


def test_status_strings(L):
    for code, name in nq.STATUS.items():
        assert L.nf4_status_string(code).decode().startswith(name)


def q(L, w=FAKE, dt=1, n=128, bs=64, codes=FAKE, absmax=None, dq=256, aq=FAKE, asc=FAKE):
    return L.nf4_quantize(w, dt, n, bs, codes, absmax, dq, aq, asc, None)


def test_quantize_validation(L):
    assert q(L, n=0) == 0  # empty: OK, nothing launched
    assert q(L, n=-1) == 2
    assert q(L, n=(1 << 37) + 1) == 2
    assert q(L, bs=32) == 3
    assert q(L, dq=128) == 3
    assert q(L, dt=7) == 3
    assert q(L, w=None) == 1
    assert q(L, codes=None) == 1
    assert q(L, aq=None) == 1  # only one of the DQ outputs
    assert q(L, aq=None, asc=None) == 1  # no scale output at all
    assert q(L, w=FAKE + 8) == 4
    assert q(L, codes=FAKE + 4) == 4
    assert q(L, asc=FAKE + 2) == 4
    assert q(L, aq=None, asc=None, absmax=FAKE + 1) == 4


def test_double_quantize_validation(L):
    f = L.nf4_double_quantize
    assert f(FAKE, 0, 256, FAKE, FAKE, None) == 0
    assert f(FAKE, -3, 256, FAKE, FAKE, None) == 2
    assert f(FAKE, 10, 64, FAKE, FAKE, None) == 3
    assert f(None, 10, 256, FAKE, FAKE, None) == 1
    assert f(FAKE, 10, 256, None, FAKE, None) == 1
    assert f(FAKE + 2, 10, 256, FAKE, FAKE, None) == 4


def test_dequantize_validation(L):
    f = L.nf4_dequantize
    assert f(FAKE, 0, 64, None, FAKE, FAKE, 256, FAKE, 1, None) == 0
    assert f(FAKE, -1, 64, None, FAKE, FAKE, 256, FAKE, 1, None) == 2
    assert f(FAKE, 100, 16, None, FAKE, FAKE, 256, FAKE, 1, None) == 3
    assert f(FAKE, 100, 64, None, FAKE, FAKE, 256, FAKE, 5, None) == 3
    assert f(None, 100, 64, None, FAKE, FAKE, 256, FAKE, 1, None) == 1
    assert f(FAKE, 100, 64, None, None, None, 256, FAKE, 1, None) == 1  # no scales at all
    assert f(FAKE, 100, 64, None, FAKE, None, 256, FAKE, 1, None) == 1
    assert f(FAKE, 100, 64, None, FAKE, FAKE, 256, FAKE + 8, 1, None) == 4


def _w(n=256, k=512, codes=FAKE, aq=FAKE, asc=FAKE, am=None, bs=64, dq=256):
    return nq.nf4_weight(codes=codes, absmax_q=aq, absmax_scale=asc, absmax=am, n_out=n, k_in=k,
                         blocksize=bs, dq_blocksize=dq)


@pytest.mark.parametrize("fn", ["nf4_linear_forward", "nf4_linear_backward_input"])
def test_linear_validation(L, fn):
    f = getattr(L, fn)
    ws = nq.nf4_linear_workspace_size(64, 16)
    assert ws == 64 * 64 * 2 + 8 * 64 * 64 * 4

    def call(act=FAKE, m=64, w=None, a=FAKE, b=FAKE, r=16, out=FAKE, wsp=FAKE, wsb=ws):
        w = w if w is not None else _w()
        return f(act, m, ctypes.byref(w), a, b, r, 2.0, out, wsp, wsb, None)

    assert f(FAKE, 64, None, FAKE, FAKE, 16, 2.0, FAKE, FAKE, ws, None) == 1
    assert call(m=0) == 0
    assert call(m=-1) == 2
    assert call(w=_w(k=100)) == 2  # K % 64 != 0
    assert call(r=300) == 2
    assert call(w=_w(bs=32)) == 3
    assert call(w=_w(dq=64)) == 3
    assert call(act=None) == 1
    assert call(out=None) == 1
    assert call(w=_w(codes=None)) == 1
    assert call(w=_w(aq=None, asc=None)) == 1
    assert call(a=None) == 1  # r > 0 without A
    assert call(b=None) == 1
    # r == 0 needs no adapter and no workspace: validation goes on to the alignment check
    assert call(a=None, b=None, r=0, wsp=None, wsb=0, act=FAKE + 2) == 4
    assert call(act=FAKE + 2) == 4
    assert call(w=_w(codes=FAKE + 4)) == 4
    assert call(wsp=None) == 5
    assert call(wsb=ws - 1) == 5


def test_linear_forward_noalloc_validation(L):
    """The allocation-free forward validates like nf4_linear_forward and
    rejects a shape whose workspace exceeds its scratch, before any HIP call."""
    f = L.nf4_linear_forward_noalloc

    def call(act=FAKE, m=64, w=None, a=FAKE, b=FAKE, r=16, out=FAKE):
        w = w if w is not None else _w()
        return f(act, m, ctypes.byref(w), a, b, r, 2.0, out, None)

    assert f(FAKE, 64, None, FAKE, FAKE, 16, 2.0, FAKE, None) == 1
    assert call(m=0) == 0
    assert call(m=-1) == 2
    assert call(r=300) == 2
    assert call(w=_w(bs=32)) == 3
    assert call(act=None) == 1
    assert call(a=None) == 1
    assert call(act=FAKE + 2) == 4
    text = open(os.path.join(ROOT, "include", "nf4.h")).read()
    mac = re.search(r"#define NF4_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert mac and int(mac.group(1)) << int(mac.group(2)) == nq.NF4_NOALLOC_SCRATCH_BYTES
    big = nq.nf4_linear_workspace_size(4096, 256)
    assert big > nq.NF4_NOALLOC_SCRATCH_BYTES >= nq.nf4_linear_workspace_size(4096, 192)
    assert call(m=4096, r=256) == 2  # scratch too small: NF4_ERR_SIZE, nothing launched


def test_workspace_size(L):
    # bf16 product [m x rp] padded to 256 bytes, then 8 fp32 partials [8 x m x rp]
    assert nq.nf4_linear_workspace_size(4096, 64) == 4096 * 64 * 2 + 8 * 4096 * 64 * 4
    assert nq.nf4_linear_workspace_size(3, 5) == 512 + 8 * 3 * 64 * 4
    assert nq.nf4_linear_workspace_size(10, 65) == 10 * 128 * 2 + 8 * 10 * 128 * 4
    assert nq.nf4_linear_workspace_size(100, 0) == 0


def test_linear_kernel_path(L):
    """Which kernel family a linear shape runs, without a device: the decode
    kernels only forward with r = 0, 1 <= m <= 16 and K % 256 == 0 up to
    32768; the MFMA GEMM for N % 64 == 0 and r % 8 == 0; the portable fp32
    kernel otherwise; -1 for rejected sizes."""
    p = nq.linear_kernel_path
    assert p(4, 28672, 8192) == "decode"
    assert p(16, 28672, 8192) == "decode"
    assert p(1, 100, 256) == "decode"                 # any N on the decode path
    assert p(17, 28672, 8192) == "mfma"               # more rows than the decode kernels take
    assert p(4, 28672, 8192, backward=True) == "mfma"  # the input gradient has no decode path
    assert p(4, 28672, 8192, r=64) == "mfma"          # an adapter leaves the decode path
    assert p(16, 4096, 32768 + 256) == "mfma"         # longer rows than the decode kernels take
    assert p(4096, 8192, 8192, r=64) == "mfma"
    assert p(37, 100, 192, r=5) == "portable"         # N % 64 != 0
    assert p(64, 512, 256, r=12) == "portable"        # r % 8 != 0
    assert p(64, 512, 256, r=12, backward=True) == "portable"
    assert p(4, 100, 192) == "portable"               # decode-shaped but K % 256 != 0
    for bad in ((-1, 64, 64, 0), (4, 0, 64, 0), (4, 64, 96, 0), (4, 64, 64, 257), (4, 64, 64, -1)):
        assert L.nf4_linear_kernel_path(*bad, 0) == -1
    assert p(4, 64, 96) is None


def test_config_surface():
    nq.NF4Config().validate()
    for bad in (dict(quant_type="fp4"), dict(compute_dtype="float32"), dict(blocksize=96),
                dict(load_in_4bit=False), dict(dq_format="int8")):
        with pytest.raises(ValueError):
            nq.NF4Config(**bad).validate()


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(nq, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(nq, "_lib", None)
    with pytest.raises(nq.NF4LibraryMissing):
        nq.lib()


def test_lora_backward_validation(L):
    f = L.nf4_lora_backward
    ws = nq.nf4_lora_backward_workspace_size(64, 512, 256, 16)
    # X.A and dY.B^T as bf16, stored transposed [64 x 128] (64 tokens rounded
    # up to a step of 64, plus one padding step), then 8 fp32 partial sums of
    # the larger of 2 x [64 x 64] and [512 x 16] + [16 x 256]
    assert ws == 2 * 64 * 128 * 2 + 8 * (512 * 16 + 16 * 256) * 4
    assert nq.nf4_lora_backward_workspace_size(64, 512, 256, 0) == 0
    assert nq.nf4_lora_backward_workspace_size(-1, 512, 256, 16) == 0

    def call(x=FAKE, dy=FAKE, m=64, k=512, n=256, a=FAKE, b=FAKE, r=16, ga=FAKE, gb=FAKE, dt=0,
             wsp=FAKE, wsb=ws):
        return f(x, dy, m, k, n, a, b, r, 2.0, ga, gb, dt, wsp, wsb, None)

    assert call(m=-1) == 2
    assert call(k=100) == 2  # k_in % 64 != 0
    assert call(n=96) == 2   # n_out % 64 != 0
    assert call(r=12) == 2   # r % 8 != 0
    assert call(r=264) == 2
    assert call(r=0) == 2
    assert call(dt=7) == 3
    assert call(ga=None, gb=None) == 0  # nothing asked: OK, nothing launched
    assert call(x=None) == 1
    assert call(dy=None) == 1
    assert call(a=None) == 1
    assert call(b=None) == 1
    assert call(x=FAKE + 2) == 4
    assert call(gb=FAKE + 4) == 4
    assert call(wsp=None) == 5
    assert call(wsb=ws - 1) == 5
    assert call(wsp=FAKE + 16) == 4  # the workspace is 256-byte aligned


def _fmt(bs=64, dq=256, f=0, off=0, cb=0):
    return ctypes.byref(nq.nf4_format(bs, dq, f, off, cb))


def test_format_variant_validation(L):
    """nf4_quantize_ex / nf4_double_quantize_ex / nf4_dequantize_ex reject bad
    formats, sizes, pointers, alignment and workspace before any HIP call."""
    q = L.nf4_quantize_ex
    ok = dict(w=FAKE, dt=nq.NF4_BF16, n=1024, codes=FAKE, am=None, aq=FAKE, asc=FAKE, off=FAKE,
              ws=FAKE, wsb=1 << 20)

    def call_q(fmt, **kw):
        a = dict(ok, **kw)
        return q(a["w"], a["dt"], a["n"], fmt, a["codes"], a["am"], a["aq"], a["asc"], a["off"],
                 a["ws"], a["wsb"], None)

    assert call_q(None) == 1
    for bad in (_fmt(bs=8), _fmt(bs=96), _fmt(bs=8192), _fmt(dq=0), _fmt(dq=3), _fmt(dq=8192),
                _fmt(f=3), _fmt(f=-1), _fmt(off=2), _fmt(cb=3), _fmt(cb=-1)):
        assert call_q(bad) == 3
    assert call_q(_fmt(), n=-1) == 2
    assert call_q(_fmt(), dt=7) == 3
    assert call_q(_fmt(bs=128), n=0) == 0
    assert call_q(_fmt(), w=None) == 1
    assert call_q(_fmt(), aq=None) == 1  # one of the two DQ outputs missing
    assert call_q(_fmt(), aq=None, asc=None) == 1  # no DQ and no absmax
    assert call_q(_fmt(off=1), off=None) == 1
    assert call_q(_fmt(), w=FAKE + 4) == 4
    assert call_q(_fmt(), off=FAKE + 2) == 4
    # two-pass formats need a workspace: missing, too small, misaligned
    need = L.nf4_quantize_ex_workspace_size(1024, _fmt(bs=128))
    assert need == 256 * ((1024 // 128 * 4 + 255) // 256)
    assert call_q(_fmt(bs=128), ws=None) == 5
    assert call_q(_fmt(bs=128), wsb=need - 1) == 5
    assert call_q(_fmt(bs=128), ws=FAKE + 16) == 4
    assert L.nf4_quantize_ex_workspace_size(1024, _fmt()) == 0
    assert L.nf4_quantize_ex_workspace_size(1024, _fmt(f=2)) == 0
    assert L.nf4_quantize_ex_workspace_size(1024, _fmt(bs=48)) == ctypes.c_size_t(-1).value
    # the mean offset: block scales, then two partial-sum buffers
    # (plus the 256-block group sums when B1 = 64)
    assert L.nf4_quantize_ex_workspace_size(1 << 20, _fmt(off=1)) == 4 * (1 << 14) + 256 + 256 + 256
    assert L.nf4_double_quantize_ex_workspace_size(5000, _fmt(off=1)) == 256 + 256
    assert L.nf4_double_quantize_ex_workspace_size(5000, _fmt(f=1)) == 0

    dq = L.nf4_double_quantize_ex
    assert dq(FAKE, 100, _fmt(dq=5), FAKE, FAKE, None, None, 0, None) == 3
    assert dq(FAKE, -1, _fmt(), FAKE, FAKE, None, None, 0, None) == 2
    assert dq(None, 100, _fmt(), FAKE, FAKE, None, None, 0, None) == 1
    assert dq(FAKE, 100, _fmt(off=1), FAKE, FAKE, None, FAKE, 1024, None) == 1
    assert dq(FAKE, 100, _fmt(off=1), FAKE, FAKE, FAKE, None, 0, None) == 5
    assert dq(FAKE + 2, 100, _fmt(), FAKE, FAKE, None, None, 0, None) == 4

    dz = L.nf4_dequantize_ex
    assert dz(FAKE, 1024, _fmt(bs=32), None, FAKE, FAKE, None, FAKE, 9, None) == 3
    assert dz(FAKE, 1024, _fmt(bs=32, off=1), None, FAKE, FAKE, None, FAKE, 1, None) == 1
    assert dz(FAKE, 1024, _fmt(bs=32), None, None, None, None, FAKE, 1, None) == 1
    assert dz(FAKE + 8, 1024, _fmt(bs=32), FAKE, None, None, None, FAKE, 1, None) == 4
    assert dz(FAKE, 1024, None, FAKE, None, None, None, FAKE, 1, None) == 1
    assert dz(FAKE, 0, _fmt(bs=32), None, None, None, None, None, 1, None) == 0


def test_format_surface():
    f = nq.NF4Format(blocksize=128, dq_format="e5m2", mean_offset=True)
    assert not f.is_default and nq.NF4Format().is_default
    assert f.nblocks(1000) == 8 and f.ngroups(1 << 20) == 32
    with pytest.raises(ValueError):
        nq.NF4Format(dq_format="fp8").struct()
    assert nq.NF4Config(blocksize=128, dq_format="linear8").validate().format() == \
        nq.NF4Format(128, 256, "linear8", False)
    with pytest.raises(ValueError):
        nq.NF4Config(blocksize=96).validate()


def test_merge_lora_validation(L):
    m = L.nf4_merge_lora
    w = _w(n=256, k=512)
    ok = dict(w=ctypes.byref(w), a=FAKE, b=FAKE, r=64, s=2.0, c=FAKE, am=None, aq=FAKE, asc=FAKE,
              ws=FAKE, wsb=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return m(a["w"], a["a"], a["b"], a["r"], a["s"], a["c"], a["am"], a["aq"], a["asc"],
                 a["ws"], a["wsb"], None)

    assert call(w=None) == 1
    assert call(w=ctypes.byref(_w(n=256, k=96))) == 2
    assert call(w=ctypes.byref(_w(n=0, k=512))) == 2
    for r in (0, 4, 12, 264):
        assert call(r=r) == 2
    assert call(w=ctypes.byref(_w(bs=32))) == 3
    assert call(w=ctypes.byref(_w(dq=128))) == 3
    assert call(a=None) == 1 and call(b=None) == 1 and call(c=None) == 1
    assert call(aq=None) == 1
    assert call(aq=None, asc=None) == 1  # no output scales at all
    assert call(a=FAKE + 8) == 4 and call(b=FAKE + 1) == 4 and call(c=FAKE + 4) == 4
    need = L.nf4_merge_lora_workspace_size(256, 512)
    assert need == 256 * 512 // 64 * 4
    assert call(ws=None) == 5 and call(wsb=need - 1) == 5 and call(ws=FAKE + 64) == 4
    assert L.nf4_merge_lora_workspace_size(256, 96) == 0


def test_codebook_levels(L, oracle_mod):
    """The library's codebooks hold the same levels as the oracle's (each
    built by its own code from the same definitions)."""
    for name in ("nf4", "fp4", "int4"):
        got = np.array(nq.nf4_codebook_levels(name), np.float32)
        assert np.array_equal(got.view(np.uint32), oracle_mod.codebook_levels(name).view(np.uint32))
    assert not L.nf4_codebook_levels(3)


def test_storage_bytes_ex_matches_oracle(L, oracle_mod):
    for n in (0, 1, 1000, 1 << 20, 11008 * 4096):
        for bs, dqb, off in ((64, 256, 0), (128, 64, 1), (16, 1, 0), (4096, 4096, 1)):
            for dq in (0, 1):
                got = L.nf4_storage_bytes_ex(n, _fmt(bs, dqb, 0, off), dq)
                assert got == oracle_mod.storage_bytes_ex(n, bs, dqb, bool(dq), bool(off))
    assert L.nf4_storage_bytes_ex(64, _fmt(bs=48), 1) == -1
    assert L.nf4_storage_bytes_ex(-1, _fmt(), 1) == -1


def _entry(w=FAKE, n=16384, codes=FAKE, am=None, aq=FAKE, asc=FAKE):
    return nq.nf4_batch_entry(w, n, codes, am, aq, asc)


def test_batched_validation(L):
    """Every entry is checked before anything is launched: a valid call is
    never made here (it would launch), so each case holds one bad entry, or
    launches nothing at all."""
    def call(fn, entries, count=None, dt=1):
        arr = (nq.nf4_batch_entry * max(1, len(entries)))(*entries)
        return fn(arr, len(entries) if count is None else count, dt, None)

    for fn in (L.nf4_quantize_batched, L.nf4_dequantize_batched):
        good = _entry()
        assert fn(None, 0, 1, None) == 0                         # nothing to do
        assert call(fn, [_entry(n=0, w=None, codes=None)]) == 0  # only empty entries
        assert call(fn, [_entry(n=0)] * 3) == 0
        assert fn(None, 2, 1, None) == 1                         # NULL array, count > 0
        assert call(fn, [good], count=-1) == 2
        assert call(fn, [good], dt=7) == 3
        # the bad entry is last: the good ones before it launch nothing either
        assert call(fn, [good, good, _entry(n=-1)]) == 2
        assert call(fn, [good, _entry(n=(1 << 37) + 1)]) == 2
        assert call(fn, [good, _entry(w=None)]) == 1
        assert call(fn, [good, _entry(codes=None)]) == 1
        assert call(fn, [good, _entry(aq=None)]) == 1            # one of the pair
        assert call(fn, [good, _entry(asc=None)]) == 1
        assert call(fn, [good, _entry(aq=None, asc=None)]) == 1  # no DQ and no absmax
        assert call(fn, [good, _entry(w=FAKE + 8)]) == 4
        assert call(fn, [good, _entry(codes=FAKE + 4)]) == 4
        assert call(fn, [good, _entry(aq=FAKE + 2)]) == 4
        assert call(fn, [good, _entry(asc=FAKE + 1)]) == 4
        assert call(fn, [good, _entry(aq=None, asc=None, am=FAKE + 2)]) == 4


def test_batched_binding_checks():
    """The Python side refuses mismatched lists before calling the library."""
    import torch

    with pytest.raises(ValueError):
        nq._batch([torch.zeros(4)], [], "x")
    with pytest.raises(ValueError):
        nq._batch([torch.zeros(4), torch.zeros(4, dtype=torch.bfloat16)], [None, None], "x")


def test_one_hip_runtime_after_lib():
    """nq.lib() loads torch first, so libnf4.so binds to torch's HIP runtime and
    a process holds one copy (checked in a fresh interpreter, on the CPU)."""
    import subprocess
    import sys

    code = ("import os, nf4_quantize_amd as nq; nq.lib(); import torch; "
            "m = open(f'/proc/{os.getpid()}/maps').read(); "
            "print(len({l.split()[-1] for l in m.splitlines() if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"
