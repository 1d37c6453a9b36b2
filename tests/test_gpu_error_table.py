"""GPU parity of dc_error_table (the eq. 5 error table of the bit allocation)
against the oracle's error_table, and of the allocation the GPU table leads
to against the oracle's allocation from its own table."""
import numpy as np
import pytest

import synth
import tenant_rank_serving_amd as trs
from oracle import alloc
from gpu_util import error_table_gpu, note, torch

pytestmark = pytest.mark.gpu

WIDTHS = (0, 2, 3, 8)
# products in fp32 over `in` terms, squares summed in fp64: about in * 2^-24
# relative per product, well inside this bar for the shapes below
RTOL = 1e-4


def _gpu_table(sigma, V, X, widths=WIDTHS):
    return error_table_gpu(sigma, V, X, widths)


# (seed, r, in, ncal): ragged row blocks (37, 70 rows x 4 widths), a calibration count that is not a
# multiple of the 64-column chunk, and a 4096-wide row set
CASES = [(0, 37, 384, 50), (1, 70, 256, 64), (2, 16, 4096, 130), (3, 5, 128, 1)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "r%d-in%d-cal%d" % c[1:])
def test_error_table_matches_oracle(case):
    seed, r, inn, ncal = case
    note("error table", case)
    u, s, v = synth.random_singular_pairs(seed, 128, inn, r)
    V = v.copy()
    V[r // 2] = 0.0                       # an all-zero row: every width exact, width 0 too
    if r > 2:
        V[1, :] = 0.25                    # a constant row
    X = np.random.default_rng(seed + 100).standard_normal((inn, ncal)).astype(np.float32)
    got, flag = _gpu_table(s, V, X)
    ref = alloc.error_table(s.astype(np.float64), V, X.astype(np.float64))
    assert flag == 0
    assert got.shape == ref.shape
    zero = ref == 0
    assert np.all(got[zero] == 0)
    rel = np.abs(got[~zero] - ref[~zero]) / ref[~zero]
    print("[parity] error table %s: max rel %.3e (bar %.0e)" % (case, rel.max(), RTOL), flush=True)
    assert rel.max() <= RTOL


def test_allocation_from_the_gpu_table():
    """The allocation computed from the GPU table has the optimum's total
    error under the oracle's table (choices may differ only between widths
    whose errors tie within the table's rounding)."""
    note("allocation from the GPU table")
    r, inn, ncal = 256, 512, 96
    u, s, v = synth.random_singular_pairs(5, 512, inn, r)
    s = (0.05 * np.arange(1, r + 1) ** -0.8).astype(np.float32)
    X = np.random.default_rng(6).standard_normal((inn, ncal)).astype(np.float32)
    got, flag = _gpu_table(s, v, X)
    ref = alloc.error_table(s.astype(np.float64), v, X.astype(np.float64))
    assert flag == 0
    budget = r * 3 // 2
    ref_choice, ref_total = alloc.allocate_exact(ref, list(WIDTHS), budget)
    choice, _ = trs.dc_allocate_bits(got, list(WIDTHS), budget)
    total = float(ref[np.arange(r), choice].sum())
    assert sum(WIDTHS[c] for c in choice) <= budget
    assert abs(total - ref_total) <= 1e-6 * ref_total
    print("[parity] allocation: %d of %d choices equal, total %.6e vs optimum %.6e" %
          (int((choice == ref_choice).sum()), r, total, ref_total), flush=True)


def test_error_table_flags_nonfinite():
    note("error table non-finite")
    V = np.zeros((3, 128), np.float32)
    V[1, 5] = np.nan
    X = np.ones((128, 4), np.float32)
    _, flag = _gpu_table(np.ones(3, np.float32), V, X)
    assert flag == 1
    V[1, 5] = 0.0
    _, flag = _gpu_table(np.ones(3, np.float32), V, X)
    assert flag == 0
