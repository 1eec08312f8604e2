import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle

    oracle.lib()
    return oracle


def read_golden_column(name, col=0, sep="|"):
    """Reads non-comment lines of a golden file, returning column `col` (stripped)."""
    out = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = [p.strip() for p in line.split(sep)] if sep in line else [line]
            out.append(parts if col is None else parts[col])
    return out


@pytest.fixture(scope="session")
def printed_codebook():
    import numpy as np

    vals = [float(v) for v in read_golden_column("nf4_codebook.txt")]
    assert len(vals) == 16
    return np.array(vals, dtype=np.float64)


@pytest.fixture(scope="session")
def code_thresholds():
    import numpy as np

    rows = read_golden_column("nf4_code_thresholds.txt", col=None)
    bits = np.array([int(r[1], 16) for r in rows], dtype=np.uint32)
    assert bits.size == 15
    return bits.view(np.float32)


@pytest.fixture(scope="session")
def dev():
    """The GPU (cuda:0) with the HIP library loaded; skips only without a GPU."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import nf4_quantize_amd as nq

    nq.lib()  # raises NF4LibraryMissing when the library is not built
    return torch.device("cuda:0")
