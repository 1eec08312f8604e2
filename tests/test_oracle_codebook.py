"""Pins of the oracle's codebook and nearest-level rule against the pages and
against mathematics (CPU only).

Sources: "QLoRA: Mathematical Foundations of 4-Bit NormalFloat Quantization,
Double Quantization, and Paged Optimizers", sections "4-Bit NormalFloat (NF4)"
(codebook, construction) and "Block-Wise Quantization Mechanics" (argmin).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
from scipy.stats import norm


def test_codebook_is_the_printed_table(oracle_mod, printed_codebook):
    q = oracle_mod.codebook()
    # Every printed decimal is exactly representable; the oracle holds those values.
    assert np.all(printed_codebook.astype(np.float32).astype(np.float64) == printed_codebook)
    assert np.array_equal(q.astype(np.float64), printed_codebook)


def test_codebook_structure(oracle_mod):
    q = oracle_mod.codebook()
    assert q[0] == -1.0 and q[15] == 1.0  # normalised so that max |q| = 1
    assert q[7] == 0.0 and not np.signbit(q[7])  # exact zero level
    assert np.all(np.diff(q) > 0)  # strictly increasing
    assert int(np.sum(q < 0)) == 7 and int(np.sum(q > 0)) == 8  # 7 negative / 8 positive
    # "balanced range": both ends at magnitude 1, though the halves are not mirrors
    assert q[0] == -q[15]
    assert not np.allclose(q[:7], -q[15:8:-1])


def test_normal_quantile_matches_library(oracle_mod):
    for p in [1e-6, 0.01, 0.2, 0.5, 0.7, 0.9677083, 0.99, 1 - 1e-9]:
        assert abs(oracle_mod.normal_quantile(p) - norm.ppf(p)) < 1e-12 * max(1.0, abs(norm.ppf(p)))


def test_construction_reproduces_printed_table(oracle_mod, printed_codebook):
    # The tail probability delta is not printed; solve it from one printed level
    # (level 14) and check the other 13 non-trivial levels against the table.
    delta = oracle_mod.solve_delta(printed_codebook[14])
    assert 0.9677 < delta < 0.96772
    built = oracle_mod.construct_codebook(delta)
    assert built[7] == 0.0 and built[0] == -1.0 and built[15] == 1.0
    assert np.max(np.abs(built - printed_codebook)) <= 2.5e-7
    # The same construction with the probability grid evaluated by the library quantile.
    pos = norm.ppf(np.linspace(delta, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(delta, 0.5, 8)[:-1])
    ref = np.sort(np.concatenate([pos, [0.0], neg])) / norm.ppf(delta)
    assert np.max(np.abs(built - ref)) < 1e-12


def test_construction_mistakes_are_caught(oracle_mod, printed_codebook):
    # A construction with the halves' step counts swapped cannot match the table.
    delta = oracle_mod.solve_delta(printed_codebook[14])
    pos = norm.ppf(np.linspace(delta, 0.5, 8)[:-1])
    neg = -norm.ppf(np.linspace(delta, 0.5, 9)[:-1])
    wrong = np.sort(np.concatenate([pos, [0.0], neg])) / norm.ppf(delta)
    assert np.max(np.abs(wrong - printed_codebook)) > 1e-2


def test_levels_map_to_themselves(oracle_mod):
    q = oracle_mod.codebook()
    for i, v in enumerate(q):
        assert oracle_mod.nearest_code(v) == i
    assert oracle_mod.nearest_code(-0.0) == 7
    assert oracle_mod.nearest_code(0.0) == 7


def _ord_to_f32(o):
    o = np.asarray(o, dtype=np.int64)
    bits = np.where(o >= 0, o, 0x80000000 | (-o)).astype(np.uint32)
    return bits.view(np.float32)


def test_decision_boundaries_are_the_midpoints(oracle_mod, code_thresholds):
    """A nearest-level quantizer switches from level i to i+1 at their midpoint.
    The oracle's fp32 switch point must bracket the exact real midpoint to one ulp."""
    q = oracle_mod.codebook().astype(np.float64)
    mids = (q[:-1] + q[1:]) / 2.0
    t = code_thresholds.astype(np.float64)
    below = np.nextafter(code_thresholds, np.float32(-2)).astype(np.float64)
    ulp = np.spacing(np.abs(code_thresholds)).astype(np.float64)
    for i in range(15):
        assert below[i] - ulp[i] <= mids[i] <= t[i] + ulp[i], i
        assert oracle_mod.nearest_code(code_thresholds[i]) == i + 1
        assert oracle_mod.nearest_code(np.float32(below[i])) == i


def test_nearest_code_is_exact_nearest_away_from_midpoints(oracle_mod):
    """On random n, the code is the index of the nearest level in exact
    arithmetic, except within 2 ulp of a midpoint (where fp32 rounding decides)."""
    rng = np.random.Generator(np.random.PCG64(11))
    n = rng.uniform(-1, 1, 2_000_000).astype(np.float32)
    q = oracle_mod.codebook().astype(np.float64)
    exact = np.argmin(np.abs(n.astype(np.float64)[:, None] - q[None, :]), axis=1)
    got = oracle_mod.nearest_code_array(n)
    mids = (q[:-1] + q[1:]) / 2.0
    near = np.min(np.abs(n.astype(np.float64)[:, None] - mids[None, :]), axis=1)
    far = near > 2 * np.spacing(np.float32(1.0))
    assert far.mean() > 0.999
    assert np.array_equal(got[far], exact[far])


# fp32 values n at which the fp32 distances to two adjacent levels are equal
# (found by a scan of the fp32 distances); the lowest index must win.
TIES = [
    (-0.4599952697753906, 2),
    (-0.045525018125772476, 6),
    (0.03979014977812767, 7),
    (0.2035212516784668, 9),
    (0.3893125355243683, 11),
    (0.6427869200706482, 13),
]


@pytest.mark.parametrize("n,low", TIES)
def test_ties_go_to_the_lower_index(oracle_mod, n, low):
    q = oracle_mod.codebook()
    n32 = np.float32(n)
    d_lo = np.abs(np.float32(n32 - q[low]))
    d_hi = np.abs(np.float32(n32 - q[low + 1]))
    assert d_lo == d_hi  # a genuine fp32 tie
    assert oracle_mod.nearest_code(n32) == low


def test_brute_force_argmin_small(oracle_mod):
    """Brute force in numpy float32 (first index of the minimum) on 100k values."""
    rng = np.random.Generator(np.random.PCG64(12))
    n = np.concatenate([rng.uniform(-1, 1, 100_000).astype(np.float32),
                        np.array([t for t, _ in TIES], np.float32)])
    q = oracle_mod.codebook()
    d = np.abs(n[:, None] - q[None, :])  # float32 arithmetic
    brute = np.argmin(d, axis=1)
    assert np.array_equal(oracle_mod.nearest_code_array(n), brute)


def test_code_function_exhaustive_is_the_threshold_step_function(oracle_mod, code_thresholds):
    """Every binary32 n in [-1, 1] (about 2.1e9 values): the oracle's code equals
    the number of thresholds <= n, i.e. the code is a monotone step function
    with exactly the 15 switch points of the golden file."""
    lo_neg, hi_neg = 0x80000000, 0xBF800000  # -0.0 .. -1.0
    lo_pos, hi_pos = 0x00000000, 0x3F800000  # +0.0 .. +1.0
    chunk = 1 << 24
    jobs = []
    for lo, hi in ((lo_pos, hi_pos), (lo_neg, hi_neg)):
        for s in range(lo, hi + 1, chunk):
            jobs.append((s, min(s + chunk, hi + 1)))
    thr = code_thresholds

    def run(span):
        s, e = span
        n = np.arange(s, e, dtype=np.uint32).view(np.float32)
        got = oracle_mod.nearest_code_array(n)
        want = np.searchsorted(thr, n, side="right").astype(np.uint8)
        bad = np.nonzero(got != want)[0]
        return (s, int(bad.size))

    with ThreadPoolExecutor(max_workers=8) as ex:
        results = list(ex.map(run, jobs))
    assert all(b == 0 for _, b in results), [r for r in results if r[1]]
