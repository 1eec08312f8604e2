"""The packed storage as a file: codes, 8-bit scale codes, second-level
scales, shape and format are written and read back byte for byte, so the
reloaded weight dequantizes to exactly what was saved. The packed parts are
the oracle's, computed on the CPU from seeded inputs; the file layer is pure
host code (safetensors), so these tests need no GPU.
"""
import numpy as np
import pytest

import nf4_quantize_amd as nq
import oracle
import workloads


def _oracle_packed(seed, n, dq=True):
    import torch

    w = workloads.gaussian_f32(seed, (n,), workloads.SIGMA_W)
    codes, absmax = oracle.quantize(w)
    if not dq:
        return w, nq.NF4Tensor(torch.from_numpy(codes), torch.from_numpy(absmax), None, None,
                               (n,))
    q, sc = oracle.double_quantize(absmax)
    return w, nq.NF4Tensor(torch.from_numpy(codes), None, torch.from_numpy(q),
                           torch.from_numpy(sc), (n,))


def _same_bytes(a, b):
    return a.dtype == b.dtype and a.shape == b.shape and \
        a.numpy().tobytes() == b.numpy().tobytes()


@pytest.mark.parametrize("n,dq", [(1024 * 1024, True), (64 * 300 + 37, True), (1, True),
                                  (64 * 257 + 1, False)])
def test_round_trip_bytes_and_dequant(oracle_mod, tmp_path, n, dq):
    w, t = _oracle_packed(11, n, dq)
    path = str(tmp_path / "w.safetensors")
    nq.save_nf4(path, {"w": t})
    back = nq.load_nf4(path)["w"]
    assert back.shape == t.shape and back.fmt == t.fmt and back.double_quant == dq
    for p in ("codes", "absmax", "absmax_q", "absmax_scale", "absmax_offset"):
        a, b = getattr(t, p), getattr(back, p)
        assert (a is None) == (b is None), p
        if a is not None:
            assert _same_bytes(a, b), p
    kw = dict(q=back.absmax_q.numpy(), scale=back.absmax_scale.numpy()) if dq else \
        dict(absmax=back.absmax.numpy())
    kw0 = dict(q=t.absmax_q.numpy(), scale=t.absmax_scale.numpy()) if dq else \
        dict(absmax=t.absmax.numpy())
    d_back = oracle.dequantize(back.codes.numpy(), n, **kw)
    d_saved = oracle.dequantize(t.codes.numpy(), n, **kw0)
    assert d_back.tobytes() == d_saved.tobytes()
    # and the reload is a usable quantization of the original weight: every
    # value within its block's absmax (the largest level gap is under 1)
    assert np.all(np.abs(d_back - w) <= np.repeat(
        oracle.quantize(w)[1], 64)[:n] * 1.01 + 1e-30)


def test_several_tensors_and_variant_format(oracle_mod, tmp_path):
    import torch

    _, a = _oracle_packed(12, 4096)
    _, b = _oracle_packed(13, 64 * 5, dq=False)
    fmt = nq.NF4Format(128, 64, "e5m2", True, "fp4")
    n = 128 * 70
    c = nq.NF4Tensor(torch.arange((n + 1) // 2, dtype=torch.int64).to(torch.uint8), None,
                     torch.arange(fmt.nblocks(n), dtype=torch.int64).to(torch.uint8),
                     torch.linspace(0.5, 2.0, fmt.ngroups(n), dtype=torch.float32), (70, 128),
                     fmt, torch.tensor([0.25], dtype=torch.float32))
    path = str(tmp_path / "m.safetensors")
    nq.save_nf4(path, {"layer0_q": a, "layer0_k": b, "layer1_v": c})
    back = nq.load_nf4(path)
    assert sorted(back) == ["layer0_k", "layer0_q", "layer1_v"]
    cv = back["layer1_v"]
    assert cv.fmt == fmt and cv.shape == (70, 128)
    for p in ("codes", "absmax_q", "absmax_scale", "absmax_offset"):
        assert _same_bytes(getattr(c, p), getattr(cv, p)), p
    assert back["layer0_k"].absmax_q is None and _same_bytes(b.absmax, back["layer0_k"].absmax)


def test_rejects_inconsistent_files(oracle_mod, tmp_path):
    import torch
    from safetensors.torch import save_file

    _, t = _oracle_packed(14, 64 * 256 * 3)
    with pytest.raises(ValueError):
        nq.save_nf4(str(tmp_path / "x.safetensors"), {})
    with pytest.raises(ValueError):
        nq.save_nf4(str(tmp_path / "x.safetensors"), {"a.b": t})
    good = str(tmp_path / "good.safetensors")
    nq.save_nf4(good, {"w": t})
    from safetensors import safe_open
    with safe_open(good, framework="pt") as fh:
        md = fh.metadata()
        parts = {k: fh.get_tensor(k) for k in fh.keys()}

    def write(name, tensors, metadata):
        p = str(tmp_path / name)
        save_file(tensors, p, metadata=metadata)
        return p

    # not an NF4 file
    with pytest.raises(ValueError):
        nq.load_nf4(write("plain.safetensors", {"x": torch.zeros(4)}, {}))
    # a part missing
    short = {k: v for k, v in parts.items() if k != "w.absmax_scale"}
    with pytest.raises(ValueError):
        nq.load_nf4(write("missing.safetensors", short, md))
    # a part of the wrong length or type
    for k, bad in (("w.codes", parts["w.codes"][:-1].clone()),
                   ("w.absmax_q", parts["w.absmax_q"].to(torch.int8)),
                   ("w.absmax_scale", parts["w.absmax_scale"].double())):
        with pytest.raises(ValueError):
            nq.load_nf4(write("bad.safetensors", {**parts, k: bad}, md))
