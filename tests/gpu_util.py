"""Helpers for the GPU parity tests: host <-> device marshalling and the
tolerance metric for the fused matmuls. No quantization arithmetic here."""
import sys

import numpy as np


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, dev):
    """numpy float32 / bf16 bits (uint16) / uint8 -> torch device tensor."""
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def to_host(t):
    import torch

    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def bf16_bits_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_err_metric(y, ref):
    """max_i |y_i - r_i| / max(|r_i|, rms(r)), and the normwise max|y-r|/max|r|.

    The rms floor keeps outputs that cancel to near zero from dominating."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    den = np.maximum(np.abs(ref), rms)
    return float(np.max(np.abs(y - ref) / den)), float(np.max(np.abs(y - ref)) / np.max(np.abs(ref)))


def plain_rel_err(y, ref):
    """max_i |y_i - r_i| / |r_i| over the outputs with r_i != 0, and its
    99.9th percentile: reported beside the gated metric (an output that
    cancels to near zero makes the plain maximum large for any rounding)."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    nz = ref != 0
    e = np.abs(y[nz] - ref[nz]) / np.abs(ref[nz])
    return float(np.max(e)), float(np.quantile(e, 0.999))
