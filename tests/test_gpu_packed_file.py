"""GPU round trip of the packed file: quantize on the device, save, load back
onto the device, dequantize. The reloaded parts equal the saved ones byte for
byte and equal the oracle's quantization of the same seeded input; both
dequantizations agree bit for bit.
"""
import numpy as np
import pytest

import nf4_quantize_amd as nq
import oracle
import workloads
from gpu_util import log, to_dev, to_host

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape,keep_absmax", [((1024, 1024), False), ((300, 4096 + 64), True),
                                              ((7, 77), False)])
def test_save_load_dequantize(dev, tmp_path, shape, keep_absmax):
    import torch

    log(f"packed file round trip {shape} keep_absmax={keep_absmax}")
    w = workloads.gaussian_f32(21, shape, workloads.SIGMA_W)
    t = nq.quantize(to_dev(w, dev), keep_absmax=keep_absmax)
    d0 = nq.dequantize(t, out_dtype=torch.float32)
    path = str(tmp_path / "w.safetensors")
    nq.save_nf4(path, {"w": t})
    back = nq.load_nf4(path, device=dev)["w"]
    assert back.codes.device == t.codes.device and back.shape == tuple(shape)
    d1 = nq.dequantize(back, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(d0).view(np.uint32), to_host(d1).view(np.uint32))

    codes, absmax = oracle.quantize(w.ravel())
    q, sc = oracle.double_quantize(absmax)
    assert np.array_equal(to_host(back.codes), codes)
    assert np.array_equal(to_host(back.absmax_q), q)
    assert np.array_equal(to_host(back.absmax_scale).view(np.uint32), sc.view(np.uint32))
    if keep_absmax:
        assert np.array_equal(to_host(back.absmax).view(np.uint32), absmax.view(np.uint32))


@pytest.mark.parametrize("fmt", [("e5m2", True, 64, "nf4"), ("linear8", False, 128, "nf4"),
                                 ("e4m3", False, 64, "fp4")])
def test_save_load_variant_formats(dev, tmp_path, fmt):
    """A storage-format variant survives the file: the format is restored from
    the metadata and the reloaded weight dequantizes bit for bit as before."""
    import torch

    code, off, b1, cb = fmt
    f = nq.NF4Format(b1, 256, code, off, cb)
    log(f"packed file round trip, format {f}")
    w = workloads.gaussian_f32(22, (333, 512), workloads.SIGMA_W)
    t = nq.quantize(to_dev(w, dev), fmt=f)
    d0 = nq.dequantize(t, out_dtype=torch.float32)
    path = str(tmp_path / "v.safetensors")
    nq.save_nf4(path, {"v": t})
    back = nq.load_nf4(path, device=dev)["v"]
    assert back.fmt == f
    d1 = nq.dequantize(back, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(d0).view(np.uint32), to_host(d1).view(np.uint32))
