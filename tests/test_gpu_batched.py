"""GPU parity of the batched storage path (nf4_quantize_batched,
nf4_dequantize_batched) against the CPU oracle, bit for bit: every entry of a
batch must come out exactly as the oracle's blockwise NF4 + double
quantization and dequantization of that tensor alone.

The batches mix what the launch grouping has to get right: empty, tiny and
ragged tensors (partial last groups, odd lengths), tensors of whole groups,
entries with and without double quantization, more than 32 entries (several
launches of each kind), and the shapes of one layer of the 8B-shaped stack.

Inputs are seeded synthetic tensors; nothing the oracle reads comes from the
GPU.
"""
import numpy as np
import pytest

import nf4_quantize_amd as nq
import oracle
import workloads
from gpu_util import log, to_dev, to_host

pytestmark = pytest.mark.gpu

G = 16384  # weights per DQ group


def weights(seed, n, dtype):
    rng = np.random.Generator(np.random.PCG64(seed))
    w = rng.standard_normal(n, dtype=np.float32) * np.float32(workloads.SIGMA_W)
    if n:
        w[rng.choice(n, size=max(1, n // 1000), replace=False)] *= 10
        w[: min(n, 64)] = 0.0  # an all-zero block
    return workloads.to_bf16_bits(w) if dtype == "bf16" else w


def check_entry(i, w, t, dq, keep_absmax):
    n = w.size
    codes, amax = oracle.quantize(w)
    assert np.array_equal(to_host(t.codes), codes), f"entry {i} (n={n}): codes differ"
    if keep_absmax or not dq:
        assert np.array_equal(to_host(t.absmax), amax), f"entry {i} (n={n}): absmax differs"
    if dq:
        q, sc = oracle.double_quantize(amax)
        assert np.array_equal(to_host(t.absmax_q), q), f"entry {i} (n={n}): scale codes differ"
        assert np.array_equal(to_host(t.absmax_scale).view(np.uint32), sc.view(np.uint32)), \
            f"entry {i} (n={n}): c2 differs"
        return codes, None, q, sc
    return codes, amax, None, None


def run_batch(dev, sizes, dtype, modes, seed0):
    """Quantizes, then dequantizes (bf16 and fp32), every tensor of `sizes` in
    one batched call each; modes[i] = (double quant, keep absmax)."""
    import torch

    log(f"batched {dtype}: {len(sizes)} entries, {sum(sizes)} weights, sizes {sizes[:12]}...")
    ws = [weights(seed0 + i, n, dtype) for i, n in enumerate(sizes)]
    wd = [to_dev(w, dev) for w in ws]
    outs = [nq.empty_nf4((n,), dev, dq, ka) for n, (dq, ka) in zip(sizes, modes)]
    nq.nf4_quantize_batched(wd, outs)
    torch.cuda.synchronize()
    refs = [check_entry(i, w, t, dq, ka) for i, (w, t, (dq, ka)) in enumerate(zip(ws, outs, modes))]
    for odt, oname in ((torch.bfloat16, oracle.BF16), (torch.float32, oracle.F32)):
        ys = [torch.empty(n, dtype=odt, device=dev) for n in sizes]
        nq.nf4_dequantize_batched(outs, ys)
        torch.cuda.synchronize()
        for i, (y, (codes, amax, q, sc)) in enumerate(zip(ys, refs)):
            ref = oracle.dequantize(codes, sizes[i], absmax=amax, q=q, scale=sc, out_dtype=oname)
            got = to_host(y)
            if odt == torch.float32:
                got, ref = got.view(np.uint32), ref.view(np.uint32)
            assert np.array_equal(got, ref), f"entry {i} (n={sizes[i]}): {odt} dequant differs"


SIZES = [0, 1, 2, 63, 64, 65, 4095, G - 1, G, G + 1, 3 * G + 777, 5 * G, 2 * G + 2048, 7]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("mode", ["dq", "dq_absmax", "no_dq"])
def test_batched_mixed_sizes(dev, dtype, mode):
    m = {"dq": (True, False), "dq_absmax": (True, True), "no_dq": (False, True)}[mode]
    run_batch(dev, SIZES, dtype, [m] * len(SIZES), seed0=100)


def test_batched_many_entries_mixed_modes(dev):
    """120 entries, with double quantization on 80 and off on 40, in one call.
    Of the double-quantized ones 37 have full groups and 53 a partial one, so
    both kinds of launch are split over several 32-entry blocks."""
    rng = np.random.Generator(np.random.PCG64(5))
    sizes = [int(x) for x in rng.choice([G, 2 * G, G + 3, 5000, 3 * G + 64, 1, 130, 0], size=120)]
    modes = [((i % 3) != 2, (i % 5) == 0) for i in range(len(sizes))]
    run_batch(dev, sizes, "bf16", modes, seed0=1000)


def test_batched_single_entry(dev):
    run_batch(dev, [4 * G + 100], "bf16", [(True, False)], seed0=7)


def test_batched_stack_layer_matches_single_calls(dev):
    """One layer of the 8B-shaped stack (q, k, v, o, gate, up, down; 218M
    weights drawn on the device): the batched call writes exactly what one
    nf4_quantize / nf4_dequantize call per matrix writes, and k, v (whole
    1024 x 4096 matrices) and the first and last groups of down match the
    oracle."""
    import torch

    ws = [workloads.stack_matrix_bf16(0, mi, dev) for mi in range(len(workloads.STACK_MATRICES))]
    log(f"stack layer 0: {[tuple(w.shape) for w in ws]}")
    batched = nq.quantize_batched(ws)
    single = [nq.quantize(w) for w in ws]
    yb = nq.dequantize_batched(batched)
    ys = [nq.dequantize(t) for t in single]
    torch.cuda.synchronize()
    for name, a, b, y1, y2 in zip([m for m, _ in workloads.STACK_MATRICES], batched, single, yb, ys):
        assert torch.equal(a.codes, b.codes), name
        assert torch.equal(a.absmax_q, b.absmax_q), name
        assert torch.equal(a.absmax_scale, b.absmax_scale), name
        assert torch.equal(y1, y2), name
    for mi in (1, 2):  # k, v
        w = to_host(ws[mi]).ravel()
        codes, amax = oracle.quantize(w)
        q, sc = oracle.double_quantize(amax)
        assert np.array_equal(to_host(batched[mi].codes), codes)
        assert np.array_equal(to_host(batched[mi].absmax_q), q)
        assert np.array_equal(to_host(batched[mi].absmax_scale), sc)
        ref = oracle.dequantize(codes, w.size, q=q, scale=sc, out_dtype=oracle.BF16)
        assert np.array_equal(to_host(yb[mi]).ravel(), ref)
    down = to_host(ws[6]).ravel()
    ng = down.size // G
    for gi in (0, ng - 1):  # whole groups: their own DQ group of the oracle
        w = down[gi * G:(gi + 1) * G]
        codes, amax = oracle.quantize(w)
        q, sc = oracle.double_quantize(amax)
        assert np.array_equal(to_host(batched[6].codes[gi * G // 2:(gi + 1) * G // 2]), codes)
        assert np.array_equal(to_host(batched[6].absmax_q[gi * 256:(gi + 1) * 256]), q)
        assert to_host(batched[6].absmax_scale[gi:gi + 1])[0] == sc[0]
