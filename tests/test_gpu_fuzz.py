"""Seeded shape fuzz of every combine output against the oracle.

The fixed-shape random cases in test_gpu_parity.py draw hidden sizes from a
short list. Here hidden is any multiple of 8 from 8 to about 31,000
(log-uniform, 30% of cases rounded to a multiple of 32 so the MX outputs
run too), which reaches every RMSNorm vector width and masked tail the
launch planner can pick. Each case runs the bf16 combine, residual + RMSNorm
(weight_bias 0 and 1), MXFP8, MXFP4 and RMSNorm + MXFP8, element by element
against the oracle with the same tolerances as the other parity tests.

MOE_FUZZ_CASES sets the number of cases (default 64); MOE_FUZZ_BASE the first
seed index, so longer runs can continue where a previous one ended.
"""
import os

import numpy as np
import pytest

import gen
from tests.test_gpu_parity import check_all_kinds

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("MOE_FUZZ_CASES", "64"))
BASE = int(os.environ.get("MOE_FUZZ_BASE", "0"))


def wide_case(i):
    """Shape and routing of fuzz case i (seeded by i alone)."""
    rng = np.random.default_rng(50000 + i)
    H = int(8 * max(1, round(np.exp(rng.uniform(0, np.log(4096))))))
    if rng.random() < 0.3:
        H = 32 * (H // 32) or 32
    k = int(rng.integers(1, 33)) if rng.random() < 0.3 else int(rng.choice([1, 2, 4, 6, 8]))
    ep = int(rng.choice([1, 2, 3, 4, 8]))
    E = ep * max(-(-k // ep), int(rng.integers(1, 9)))
    T = int(rng.integers(1, 301)) if H <= 8192 else int(rng.integers(1, 40))
    c = dict(T=T, H=H, k=k, ep=ep, E=E, drop_frac=float(rng.choice([0.0, 0.1, 0.5])),
             weights=bool(rng.random() < 0.8), routing="zipf" if rng.random() < 0.3 else "uniform",
             residual_sd=1.0, gamma_sd=0.1)
    if rng.random() < 0.4:
        c["shared_sd"] = 0.5
    return c


@pytest.mark.parametrize("i", range(BASE, BASE + N_CASES))
def test_wide_shape_fuzz(i):
    c = wide_case(i)
    check_all_kinds(gen.make_inputs(c, seed=i), what=f"fuzz case {i}: {c}")
