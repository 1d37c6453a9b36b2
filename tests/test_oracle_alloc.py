"""Pins of oracle/alloc.py (bit allocation, [P4] §2.1 eq. 5 and §2.2).

The exact solver is pinned to exhaustive search on small tables, to the
closed-form optima of special cases, and to a feasible point it must beat
(the fixed 8/3/2 rank-group rule); the error model to closed forms.
"""
import numpy as np
import pytest

from oracle import alloc, quant

COST = [0, 2, 3, 8]   # widths 0, 2, 3, 8 bits: cost = width


@pytest.mark.parametrize("seed", range(6))
def test_exact_equals_brute_force(seed):
    rng = np.random.default_rng(seed)
    r = 5
    # decreasing errors in the width, as quantization errors are, with ties and noise
    err = np.sort(rng.random((r, 4)) * rng.choice([1.0, 10.0, 100.0], (r, 1)), axis=1)[:, ::-1].copy()
    if seed % 2:
        err[1] = err[2]                       # equal rows: ties between assignments
    for budget in range(0, 8 * r + 2):
        best, args = alloc.allocate_brute(err, COST, budget)
        choice, total = alloc.allocate_exact(err, COST, budget)
        assert total == best                  # same summation order (row by row): exactly equal
        assert tuple(choice) in args
        assert sum(COST[k] for k in choice) <= budget


def test_exact_arbitrary_errors_and_costs():
    """Not monotone in the width, unequal costs: still the exhaustive optimum."""
    rng = np.random.default_rng(11)
    err = rng.random((6, 3)) * 5.0
    cost = [1, 4, 2]
    for budget in range(6, 25):
        best, args = alloc.allocate_brute(err, cost, budget)
        choice, total = alloc.allocate_exact(err, cost, budget)
        assert total == best and tuple(choice) in args
    with pytest.raises(ValueError):
        alloc.allocate_exact(err, cost, 5)   # six rows of cost >= 1


def test_special_cases():
    rng = np.random.default_rng(3)
    err = np.sort(rng.random((40, 4)), axis=1)[:, ::-1].copy()
    # budget 0: every row dropped
    choice, total = alloc.allocate_exact(err, COST, 0)
    assert np.all(choice == 0) and total == pytest.approx(err[:, 0].sum(), rel=1e-15)
    # budget for every row at 8 bits: each row takes its least error
    choice, total = alloc.allocate_exact(err, COST, 8 * 40)
    assert np.array_equal(choice, np.argmin(err, axis=1))
    # equal difference terms d_b for every row, descending sigma: by the
    # rearrangement inequality the optimum gives wider codes to larger sigma
    sigma = np.sort(rng.random(40))[::-1] + 0.1
    d = np.array([1.0, 0.2, 0.05, 0.0004])
    err = sigma[:, None] ** 2 * d[None, :]
    for budget in (20, 77, 150):
        choice, _ = alloc.allocate_exact(err, COST, budget)
        widths = np.array(COST)[choice]
        assert np.all(np.diff(widths) <= 0), widths


def test_pair_error_closed_forms():
    rng = np.random.default_rng(5)
    v = rng.standard_normal(256) * 0.05
    x = rng.standard_normal((256, 16))
    # dropped: sigma^2 ||v X||^2
    assert alloc.pair_error(2.0, v, x, 0) == pytest.approx(4.0 * float((v @ x) @ (v @ x)), rel=1e-14)
    # sigma = 0: no error at any width
    assert all(alloc.pair_error(0.0, v, x, b) == 0.0 for b in (0, 2, 3, 8))
    # scaling term: quadratic in sigma
    assert alloc.pair_error(3.0, v, x, 3) == pytest.approx(9.0 * alloc.pair_error(1.0, v, x, 3), rel=1e-14)
    # a row already on its 3-bit grid quantizes to itself: no error at 3 bits
    codes, s, z = quant.quantize_vector(v, 3)
    on_grid = quant.dequantize(codes, s, z)
    assert alloc.pair_error(1.0, on_grid, x, 3) == 0.0
    # more bits, less error for this row
    e = [alloc.pair_error(1.0, v, x, b) for b in (0, 2, 3, 8)]
    assert e[0] > e[1] > e[2] > e[3] > 0


def test_allocation_beats_the_fixed_rank_groups():
    """The exact optimum is at most the error of any feasible allocation, in
    particular of the fixed 8/3/2 successive groups at the same budget."""
    rng = np.random.default_rng(7)
    out = inn = 256
    a = np.linalg.qr(rng.standard_normal((out, out)))[0]
    b = np.linalg.qr(rng.standard_normal((inn, inn)))[0]
    s = np.arange(1, 257) ** -1.5
    delta = (a * s) @ b.T
    u, sig, v = quant.svd_pairs(delta)
    x = rng.standard_normal((inn, 32))
    err = alloc.error_table(sig, v, x)
    n8, n3, n2 = quant.rank_groups(out, inn, 16)
    budget = 8 * n8 + 3 * n3 + 2 * n2
    fixed = np.array([3] * n8 + [2] * n3 + [1] * n2 + [0] * (len(sig) - n8 - n3 - n2))
    fixed_err = sum(err[i, k] for i, k in enumerate(fixed))
    choice, total = alloc.allocate_exact(err, COST, budget)
    assert total <= fixed_err
    assert sum(COST[k] for k in choice) <= budget
    (c8, c3, c2), order = alloc.counts_and_order(choice, alloc.WIDTHS, sig)
    assert 8 * c8 + 3 * c3 + 2 * c2 <= budget and len(order) == c8 + c3 + c2
    w = np.array(alloc.WIDTHS)[choice][order]
    assert np.all(np.diff(w) <= 0)            # 8-bit pairs first, then 3, then 2


def test_counts_and_order_hand_example():
    choice = [3, 0, 1, 2, 1, 3]               # widths 8, 0, 2, 3, 2, 8
    sigma = [0.5, 0.9, 0.1, 0.3, 0.2, 0.7]
    (n8, n3, n2), order = alloc.counts_and_order(choice, alloc.WIDTHS, sigma)
    assert (n8, n3, n2) == (2, 1, 2)
    assert order.tolist() == [5, 0, 3, 4, 2]
