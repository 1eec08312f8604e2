"""GPU parity of quantize / double-quantize / dequantize against the CPU oracle:
bit-exact codes, 8-bit scale codes, second-level scales and dequantized values.

Inputs are seeded synthetic tensors (workloads.py); the oracle sees the same
bytes. No expected value comes from the GPU path.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import nf4_quantize_amd as nq
import oracle
import workloads
from gpu_util import log, to_dev, to_host

pytestmark = pytest.mark.gpu


def gpu_quantize(w, dev, dq=True, keep_absmax=True):
    import torch

    t = nq.quantize(to_dev(w, dev), double_quant=dq, keep_absmax=keep_absmax)
    torch.cuda.synchronize()
    return t


def check_quantize(w, dev, dq=True, keep_absmax=True, label=""):
    log(f"quantize parity: {label} n={w.size} dtype={w.dtype} dq={dq} absmax={keep_absmax}")
    t = gpu_quantize(w, dev, dq, keep_absmax)
    codes, absmax = oracle.quantize(w.ravel())
    assert np.array_equal(to_host(t.codes), codes), "codes differ"
    if t.absmax is not None:
        assert np.array_equal(to_host(t.absmax), absmax), "absmax differs"
    if dq:
        q8, scale = oracle.double_quantize(absmax)
        assert np.array_equal(to_host(t.absmax_q), q8), "E4M3 scale codes differ"
        assert np.array_equal(to_host(t.absmax_scale), scale), "second-level scales differ"
    return t


def test_workload1_fp32_1024(dev):
    w = workloads.weight_1024_f32()
    t = check_quantize(w, dev, dq=True, keep_absmax=False, label="1024x1024 fp32")
    assert t.storage_bytes() == 540_928
    assert t.storage_bytes() / w.size == 0.515869140625
    check_quantize(w, dev, dq=False, label="1024x1024 fp32, no DQ")


SIZES = [1, 2, 63, 64, 65, 127, 16383, 16384, 16385, 3 * 16384 + 7, 5 * 16384 + 64 * 3]


@pytest.mark.parametrize("n", SIZES)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_sizes(dev, n, dtype):
    w = workloads.gaussian_f32(1000 + n, n, 0.02)
    if dtype == "bf16":
        w = workloads.to_bf16_bits(w)
    check_quantize(w, dev, dq=True, keep_absmax=True, label=f"ragged {dtype}")
    check_quantize(w, dev, dq=False, label=f"ragged {dtype} no DQ")


def test_special_blocks(dev):
    blocks = []
    blocks.append(np.zeros(64, np.float32))                 # all zero
    blocks.append(-np.zeros(64, np.float32))                # negative zeros
    one = np.zeros(64, np.float32); one[5] = 0.25; blocks.append(one)
    neg = np.zeros(64, np.float32); neg[63] = -3.0; blocks.append(neg)
    blocks.append(workloads.gaussian_f32(3, 64, 1e-39))     # subnormal scale
    blocks.append(workloads.gaussian_f32(4, 64, 1e-41))
    blocks.append(workloads.gaussian_f32(5, 64, 1e30))      # huge scale
    edge = workloads.gaussian_f32(6, 64, 1.0); edge[0] = np.abs(edge).max(); edge[1] = -edge[0]
    blocks.append(edge)
    w = np.concatenate(blocks * 300)  # spans groups, ends with a partial group
    check_quantize(w, dev, label="special blocks")
    # a group whose c2 is zero next to normal groups
    z = np.concatenate([np.zeros(16384, np.float32), workloads.gaussian_f32(7, 16384, 0.02)])
    check_quantize(z, dev, label="zero group")


def test_ties_and_levels(dev, code_thresholds):
    """Elements whose normalised value is an exact level, an fp32 tie point or
    a switch point of the code function (c1 = 1 is planted as element 0)."""
    q = oracle.codebook()
    ties = np.array([-0.4599952697753906, -0.045525018125772476, 0.03979014977812767,
                     0.2035212516784668, 0.3893125355243683, 0.6427869200706482], np.float32)
    thr = code_thresholds
    vals = np.concatenate([q, ties, thr, np.nextafter(thr, np.float32(-2)),
                           np.nextafter(thr, np.float32(2))]).astype(np.float32)
    vals = np.resize(vals, 63 * 40)
    blocks = vals.reshape(-1, 63)
    w = np.concatenate([np.ones((blocks.shape[0], 1), np.float32), blocks], axis=1).ravel()
    # and the same values scaled by powers of two (the quotient stays exact)
    w = np.concatenate([w, w * np.float32(0.5), w * np.float32(2.0 ** -20), w * np.float32(1024.0)])
    check_quantize(w, dev, label="levels, ties, switch points")


def test_workload2_bf16_outliers(dev):
    w = workloads.weight_mlp_outliers_bf16()
    check_quantize(w.ravel(), dev, dq=True, keep_absmax=True, label="11008x4096 bf16 outliers")


def test_fused_equals_two_step(dev):
    import torch

    w = workloads.to_bf16_bits(workloads.gaussian_f32(8, 16384 * 7 + 640, 0.02))
    fused = gpu_quantize(w, dev, dq=True, keep_absmax=True)
    q8, sc = nq.double_quantize(fused.absmax)
    torch.cuda.synchronize()
    assert torch.equal(q8, fused.absmax_q) and torch.equal(sc, fused.absmax_scale)
    # standalone DQ against the oracle on odd block counts
    for nb in (1, 255, 256, 257, 1000):
        a = np.abs(workloads.gaussian_f32(nb, nb, 0.05))
        a[::7] = 0
        q8, sc = nq.double_quantize(to_dev(a, dev))
        torch.cuda.synchronize()
        oq, osc = oracle.double_quantize(a)
        assert np.array_equal(to_host(q8), oq) and np.array_equal(to_host(sc), osc), nb


def test_double_quantize_signed_and_zero_groups(dev):
    """nf4_double_quantize on block scales of either sign: c2 is the group's
    max |absmax| and a negative ratio gets the E4M3 sign bit, as in the
    oracle. Groups: all zero, all negative, mixed signs with -0, a ragged
    last group."""
    import torch

    rng = np.random.Generator(np.random.PCG64(31))
    nb = 5 * 256 + 77
    a = (rng.standard_normal(nb) * 0.05).astype(np.float32)
    a[:256] = 0.0                                 # group 0: all zero
    a[256:512] = -np.abs(a[256:512])              # group 1: all negative
    a[512:768:3] = -0.0                           # group 2: mixed, with -0
    a[768:1024] *= np.float32(1e-4)               # tiny ratios round to (signed) zero
    a[800] = np.float32(0.5)
    q8, sc = nq.double_quantize(to_dev(a, dev))
    torch.cuda.synchronize()
    oq, osc = oracle.double_quantize(a)
    assert np.array_equal(to_host(q8), oq)
    assert np.array_equal(to_host(sc).view(np.uint32), osc.view(np.uint32))
    assert np.any(oq & 0x80) and np.all(oq[:256] == 0)


@pytest.mark.parametrize("fmt", ["e4m3", "e5m2"])
def test_double_quantize_ex_signed(dev, fmt):
    """nf4_double_quantize_ex (FP8 formats, no mean offset) on signed block
    scales, against the oracle."""
    import torch

    rng = np.random.Generator(np.random.PCG64(32 + len(fmt)))
    for dqb in (1, 64, 256, 4096):
        nb = 2 * max(dqb, 64) + 19
        a = (rng.standard_normal(nb) * 0.05).astype(np.float32)
        a[::5] = -np.abs(a[::5])
        a[1::11] = -0.0
        f = nq.NF4Format(64, dqb, fmt, False)
        q, sc = nq.double_quantize(to_dev(a, dev), fmt=f)
        torch.cuda.synchronize()
        rq, rsc, _ = oracle.double_quantize_ex(a, dqb, fmt, False)
        assert np.array_equal(to_host(q), rq), dqb
        assert np.array_equal(to_host(sc).view(np.uint32), rsc.view(np.uint32)), dqb


def test_code_function_exhaustive_fp32(dev, code_thresholds):
    """Every binary32 n in [-1, 1]: blocks [1.0, n_1 .. n_63] have c1 = 1 and
    normalised values n_j exactly, so the kernel's code must equal the number
    of oracle switch points <= n_j (the step function pinned exhaustively
    against the oracle on the CPU)."""
    import torch

    thr = torch.from_numpy(code_thresholds).to(dev)
    spans = [(0x00000000, 0x3F800001), (0x80000000, 0xBF800001)]
    per = 63 * (1 << 21)  # values per launch
    bad = 0
    total = 0
    for lo, hi in spans:
        for s in range(lo, hi, per):
            e = min(s + per, hi)
            cnt = e - s
            nb = (cnt + 62) // 63
            bits = torch.arange(s, s + nb * 63, dtype=torch.int64, device=dev)
            bits = torch.where(bits < e, bits, torch.full_like(bits, s))  # pad with a real value
            bits = torch.where(bits >= 2 ** 31, bits - 2 ** 32, bits)  # as signed 32-bit patterns
            vals = bits.to(torch.int32).view(torch.float32).view(nb, 63)
            w = torch.cat([torch.ones(nb, 1, device=dev), vals], dim=1).contiguous()
            t = nq.quantize(w, double_quant=False)
            codes = t.codes.view(nb, 32)
            lo_n = codes & 15
            hi_n = codes >> 4
            got = torch.stack([lo_n, hi_n], dim=2).view(nb, 64)[:, 1:]
            want = torch.searchsorted(thr, vals, right=True).to(torch.uint8)
            bad += int((got != want).sum().item())
            total += nb * 63
            del bits, vals, w, t, codes, got, want
    log(f"exhaustive fp32 code function: {total} values, {bad} mismatches")
    assert bad == 0


def test_fp32_reciprocal_near_switch_points(dev, code_thresholds):
    """fp32 input where the reciprocal shortcut can matter: every binary32 c1
    in [1, 2) (2^23 values) with w = fl32(thr_i * c1) and its +-3-ulp
    neighbours for the 15 oracle switch points thr_i, about 8.8e8 (w, c1)
    pairs. Each c1 heads two blocks [c1, w..]. The expected code of w is
    i + (fl32(w / c1) >= thr_i), with the quotient from the host's IEEE
    division (numpy float32): w / c1 lies a few ulps from thr_i and far
    from every other switch point."""
    import torch

    thr = code_thresholds
    offs = np.arange(-3, 4, dtype=np.int32)
    idx = np.repeat(np.arange(15), offs.size)  # switch point of each of the 105 values
    slots = np.r_[1:64, 65:107]                # their places in a c1's two blocks
    per = 1 << 19
    bad = total = 0
    for lo in range(0, 1 << 23, per):
        c1 = (np.uint32(0x3F800000) + np.arange(lo, lo + per, dtype=np.uint32)).view(np.float32)
        base = (c1[:, None] * thr[None, :]).astype(np.float32)
        vals = (base.view(np.int32)[:, :, None] + offs).reshape(per, -1).view(np.float32)
        quot = vals / c1[:, None]
        assert quot.dtype == np.float32 and np.all(np.abs(vals) <= c1[:, None])
        want = (idx + (quot >= thr[idx])).astype(np.uint8)
        w = np.zeros((per, 128), np.float32)
        w[:, 0] = c1
        w[:, 64] = c1
        w[:, slots] = vals
        t = nq.quantize(to_dev(w.ravel(), dev), double_quant=False)
        codes = t.codes.view(per, 64)
        got = torch.stack([codes & 15, codes >> 4], dim=2).view(per, 128)[:, slots]
        bad += int((got != to_dev(want, dev)).sum().item())
        total += want.size
        del t, codes, got
    log(f"fp32 reciprocal sweep: {total} (w, c1) pairs, {bad} mismatches")
    assert bad == 0


def _bf16_pair_blocks(pc_lo, pc_hi):
    """Blocks [c, w_1..w_63] for every positive finite bf16 c with bits in
    [pc_lo, pc_hi) and every bf16 w with |w| <= c (padded with +0)."""
    rows = []
    for pc in range(pc_lo, pc_hi):
        pos = np.arange(0, pc + 1, dtype=np.uint16)
        ws = np.concatenate([pos, pos | np.uint16(0x8000)])
        pad = (-ws.size) % 63
        ws = np.concatenate([ws, np.zeros(pad, np.uint16)]).reshape(-1, 63)
        c = np.full((ws.shape[0], 1), pc, np.uint16)
        rows.append(np.concatenate([c, ws], axis=1))
    return np.concatenate(rows).ravel()


def test_all_bf16_pairs(dev):
    """Every pair of finite bf16 values (w, c) with |w| <= c, c > 0 (about
    1.07e9 pairs): bit-exact codes against the oracle."""
    import torch

    edges = np.sqrt(np.linspace(0, 1, 25)) * 0x7F7F
    edges = np.unique(np.concatenate([[1], edges.astype(np.int64), [0x7F80]]))
    spans = list(zip(edges[:-1], edges[1:]))
    bad = 0
    total = 0

    def oracle_codes(w):
        parts = np.array_split(np.arange(w.size // 64), 16)
        out = [None] * len(parts)

        def run(i):
            p = parts[i]
            if p.size == 0:
                return np.zeros(0, np.uint8)
            seg = w[p[0] * 64:(p[-1] + 1) * 64]
            return oracle.quantize(seg)[0]

        with ThreadPoolExecutor(max_workers=16) as ex:
            out = list(ex.map(run, range(len(parts))))
        return np.concatenate(out)

    bad_exponents = set()
    for lo, hi in spans:
        w = _bf16_pair_blocks(int(lo), int(hi))
        t = nq.quantize(to_dev(w, dev), double_quant=False)
        got = to_host(t.codes)
        want = oracle_codes(w)
        diff = got != want
        bad += int(np.count_nonzero(diff))
        if diff.any():
            blocks = np.unique(np.nonzero(diff)[0] // 32)
            bad_exponents |= set(int(e) for e in np.unique((w[blocks * 64] >> 7) & 0xFF))
        total += w.size
        del t
        torch.cuda.empty_cache()
    log(f"all bf16 pairs: {total} elements, {bad} mismatched code bytes; "
        f"biased exponents of c in mismatching blocks: {sorted(bad_exponents)}")
    assert bad == 0


# ------------------------------------------------------------------ dequant

def check_dequant(codes, n, dev, absmax=None, q8=None, scale=None, label=""):
    import torch

    log(f"dequant parity: {label} n={n}")
    c = to_dev(codes, dev)
    args = {}
    if q8 is not None:
        args = dict(absmax_q=to_dev(q8, dev), absmax_scale=to_dev(scale, dev))
    else:
        args = dict(absmax=to_dev(absmax, dev))
    for odt, dt in ((oracle.F32, torch.float32), (oracle.BF16, torch.bfloat16)):
        out = torch.empty(n, dtype=dt, device=dev)
        nq.nf4_dequantize(c, n, out, **args)
        torch.cuda.synchronize()
        want = oracle.dequantize(codes, n, absmax=absmax, q=q8, scale=scale, out_dtype=odt)
        got = to_host(out)
        if dt == torch.float32:
            assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), f"{label} fp32"
        else:
            assert np.array_equal(got, want), f"{label} bf16"


def oracle_pack(w):
    codes, absmax = oracle.quantize(w)
    q8, scale = oracle.double_quantize(absmax)
    return codes, absmax, q8, scale


def test_dequant_workload1(dev):
    w = workloads.weight_1024_f32().ravel()
    codes, absmax, q8, scale = oracle_pack(w)
    check_dequant(codes, w.size, dev, q8=q8, scale=scale, label="1024x1024 DQ")
    check_dequant(codes, w.size, dev, absmax=absmax, label="1024x1024 no DQ")


def test_dequant_workload2(dev):
    w = workloads.weight_mlp_outliers_bf16().ravel()
    codes, absmax, q8, scale = oracle_pack(w)
    check_dequant(codes, w.size, dev, q8=q8, scale=scale, label="11008x4096 DQ")


@pytest.mark.parametrize("n", SIZES + [2047, 2048, 2049, 4096 + 5])
def test_dequant_ragged(dev, n):
    w = workloads.gaussian_f32(2000 + n, n, 0.02)
    codes, absmax, q8, scale = oracle_pack(w)
    check_dequant(codes, n, dev, q8=q8, scale=scale, label="ragged DQ")
    check_dequant(codes, n, dev, absmax=absmax, label="ragged no DQ")


def test_dequant_all_code_pairs_and_scale_codes(dev):
    """Every code byte (both nibbles) under every E4M3 code 0x00..0x7E and a
    spread of second-level scales, bit-exact."""
    nb = 127 * 16  # blocks: every E4M3 code, spread over 8 groups with different c2
    n = nb * 64
    rng = np.random.Generator(np.random.PCG64(99))
    codes = np.resize(np.arange(256, dtype=np.uint8), n // 2)
    rng.shuffle(codes)
    q8 = np.tile(np.arange(127, dtype=np.uint8), 16)
    ngroups = (nb + 255) // 256
    scale = np.array([0.5, 1.0, 3.0e-3, 7.25, 1e-30, 2.0 ** -126, 123.456, 0.0][:ngroups], np.float32)
    check_dequant(codes, n, dev, q8=q8, scale=scale, label="all code bytes x E4M3 codes")
    absmax = rng.uniform(0, 2, nb).astype(np.float32)
    absmax[::9] = 0
    check_dequant(codes, n, dev, absmax=absmax, label="all code bytes, fp32 scales")


def test_stack_sampled_matrices(dev):
    """The 32-layer stack drawn on the device: sampled matrices quantized and
    dequantized on the GPU, checked bit-exactly against the oracle."""
    import torch

    for layer, mi in ((0, 0), (0, 1), (0, 4), (0, 6), (31, 2), (17, 5)):
        name, shape = workloads.STACK_MATRICES[mi]
        log(f"stack layer {layer} {name} {shape}")
        w = workloads.stack_matrix_bf16(layer, mi, dev)
        t = nq.quantize(w.view(-1), double_quant=True)
        out = nq.dequantize(t, torch.bfloat16)
        torch.cuda.synchronize()
        host = to_host(w.view(-1))
        codes, absmax, q8, scale = oracle_pack(host)
        assert np.array_equal(to_host(t.codes), codes)
        assert np.array_equal(to_host(t.absmax_q), q8)
        assert np.array_equal(to_host(t.absmax_scale), scale)
        want = oracle.dequantize(codes, host.size, q=q8, scale=scale, out_dtype=oracle.BF16)
        assert np.array_equal(to_host(out.view(-1)), want)
        del w, t, out
