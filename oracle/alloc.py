"""Bit allocation of the singular pairs, fp64 reference (test infrastructure only).

[P4] "Enhancing Delta Compression in LLMs via SVD-based Quantization Error
Minimization" (PrinMix explainer):
  §2.1, eq. 5: quantizing row i of V costs about Sigma_ii^2 times
        Delta V_i X X^T Delta V_i^T (a scaling term and a difference term that
        depends on the quantization difference and the calibration samples X);
  §2.2: the widths are chosen by a 0/1 integer linear program: minimize the
        summed error, subject to a bit budget, one width per row (one-hot),
        widths from a candidate set, and a cap on the number of distinct
        widths.

Readings [R] taken here (the pages give no formulas beyond these):
  - Candidate set: this format's widths, 0 (dropped), 2, 3 and 8 bits
    ([P2] "Approach"); with four candidates the cap on distinct widths is
    never binding and is left out.
  - A pair (u_i, v_i) takes one width for both vectors, so a row's storage
    cost is proportional to its width: b_i (out + in) bits; the budget is
    sum_i b_i <= rho out in / (out + in) (the rank-group rule of quant.py).
  - Delta V_i is the fp16 dequantized row minus the row (quant.py's RTN
    quantizer); a dropped row has Delta V_i = -V_i.
  - The program is solved exactly by dynamic programming over the budget
    used (a multiple-choice knapsack), not by a general ILP solver.
"""
from __future__ import annotations

import itertools
from typing import Sequence, Tuple

import numpy as np

from .quant import dequantize, quantize_vector

WIDTHS = (0, 2, 3, 8)


def pair_error(sigma_i: float, v_i, x_cal, bits: int) -> float:
    """[P4] §2.1 eq. 5: Sigma_ii^2 * ||Delta V_i X||^2 for row v_i [in] at
    `bits` bits, X = x_cal [in][n_cal] (calibration activations as columns)."""
    v = np.asarray(v_i, dtype=np.float64)
    if bits == 0:
        dv = -v
    else:
        codes, scale, zero = quantize_vector(v, bits)
        dv = dequantize(codes, scale, zero) - v
    p = dv @ np.asarray(x_cal, dtype=np.float64)
    return float(sigma_i) ** 2 * float(p @ p)


def error_table(sigma, V, x_cal, widths: Sequence[int] = WIDTHS) -> np.ndarray:
    """err[i][k] = pair_error(sigma_i, V_i, X, widths[k]) for every pair."""
    r = len(sigma)
    err = np.empty((r, len(widths)))
    for i in range(r):
        for k, b in enumerate(widths):
            err[i, k] = pair_error(sigma[i], V[i], x_cal, b)
    return err


def allocate_exact(err, cost: Sequence[int], budget: int) -> Tuple[np.ndarray, float]:
    """[P4] §2.2: choose one candidate k_i per row (one-hot) minimizing
    sum_i err[i][k_i] subject to sum_i cost[k_i] <= budget.

    Dynamic programming over the budget used: after row i, best[c] is the
    least error of rows 0..i that use exactly c units.  A row's candidates
    are tried in index order and a later one replaces an earlier one only if
    strictly better; the end state is the least error over c <= budget, the
    smallest c on ties.  Returns (choice [r] int, total error); raises
    ValueError when no choice fits the budget.
    """
    err = np.asarray(err, dtype=np.float64)
    r, nb = err.shape
    cost = [int(c) for c in cost]
    best = np.full(budget + 1, np.inf)
    best[0] = 0.0
    arg = np.zeros((r, budget + 1), np.int32)
    for i in range(r):
        new = np.full(budget + 1, np.inf)
        pick = np.zeros(budget + 1, np.int32)
        for k in range(nb):
            c = cost[k]
            if c > budget:
                continue
            cand = np.full(budget + 1, np.inf)
            cand[c:] = best[:budget + 1 - c] + err[i, k]
            better = cand < new
            new[better] = cand[better]
            pick[better] = k
        best = new
        arg[i] = pick
    if not np.isfinite(best).any():
        raise ValueError("no allocation fits the budget")
    c = int(np.argmin(best))           # first minimum: the smallest budget used
    total = float(best[c])
    choice = np.zeros(r, np.int32)
    for i in range(r - 1, -1, -1):
        k = int(arg[i, c])
        choice[i] = k
        c -= cost[k]
    return choice, total


def allocate_brute(err, cost: Sequence[int], budget: int) -> Tuple[float, list]:
    """Every assignment of candidates to rows (tiny r only): the least total
    error within the budget and all assignments that reach it."""
    err = np.asarray(err, dtype=np.float64)
    r, nb = err.shape
    best, arg = np.inf, []
    for ks in itertools.product(range(nb), repeat=r):
        if sum(cost[k] for k in ks) > budget:
            continue
        e = sum(err[i, k] for i, k in enumerate(ks))
        if e < best:
            best, arg = e, [ks]
        elif e == best:
            arg.append(ks)
    return best, arg


def counts_and_order(choice, widths: Sequence[int], sigma) -> Tuple[Tuple[int, int, int], np.ndarray]:
    """(n8, n3, n2) of an allocation over widths (8, 3, 2, 0) and the pair
    order of the packed format: the 8-bit pairs, then the 3-bit, then the
    2-bit ones, each by descending sigma (stable); dropped pairs are left out."""
    w = np.asarray([widths[k] for k in choice])
    order = []
    for b in (8, 3, 2):
        idx = np.nonzero(w == b)[0]
        idx = idx[np.argsort(-np.asarray(sigma)[idx], kind="stable")]
        order.extend(idx.tolist())
    return (int((w == 8).sum()), int((w == 3).sum()), int((w == 2).sum())), np.asarray(order, np.int64)
