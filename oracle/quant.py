"""Compression side of Delta-CoMe, fp64 reference (test infrastructure only).

Steps, in the pages' order:
  1. the delta of a fine-tuned model against its backbone is decomposed by
     SVD into singular pairs ([P1] technical principles, "low-rank
     decomposition"; [P4] §2.4 step 1);
  2. pairs with larger singular values get more bits: successive groups at
     8, 3 and 2 bits, the rest dropped at 0 bits ([P1] "mixed-precision
     quantization", "long-tail distribution"; [P2] "Approach");
  3. each kept singular vector is quantized to its bit width ([P1];
     [P2] "Builds on: GPTQ"; [P4] §2.1 quantizes V row by row).

The pages give no quantizer formula.  This library's storage format fixes
asymmetric round-to-nearest min/max quantization in groups of 128 elements
with an fp16 scale and an fp16 zero point per group; the details below are
readings [R] of that statement.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

GROUP = 128


class RangeError(ValueError):
    """A group's fp16 scale overflows, or the input is not finite."""


def svd_pairs(delta) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Singular pairs of a delta matrix, largest singular value first.

    delta: [out][in].  Returns U [r][out] (row i is u_i), s [r] descending,
    V [r][in] (row i is v_i), all fp64, with delta = sum_i s_i u_i v_i^T and
    r = min(out, in) ([P4] §2.1 writes W = U Sigma V with V already
    transposed).

    [R] Sign: the pages are silent; a pair (u_i, v_i) and (-u_i, -v_i) give
    the same product but different codes.  Each pair is flipped so that the
    entry of v_i with the largest magnitude is positive (lowest index on
    ties).
    """
    d = np.asarray(delta, dtype=np.float64)
    u, s, vt = np.linalg.svd(d, full_matrices=False)
    u = u.T.copy()
    vt = vt.copy()
    for i in range(s.shape[0]):
        j = int(np.argmax(np.abs(vt[i])))  # first occurrence on ties
        if vt[i, j] < 0:
            u[i] = -u[i]
            vt[i] = -vt[i]
    return u, s, vt


def rank_groups(out: int, inn: int, budget: int) -> Tuple[int, int, int]:
    """(n8, n3, n2) for a matrix at compression 1/budget.

    [P2] "Approach": the compressed delta has the same size as BitDelta's,
    i.e. 1 bit per parameter at 1/16 ([P2] summary: 1/16 compression); the
    1/32 ablation halves it.  A pair at b bits stores b*(out+in) bits, so the
    bit budget is sum_i b_i = rho*out*in/(out+in) with rho = 16/budget.

    [R] The split among the 8/3/2-bit groups is not given for these shapes.
    n8 = 2; n3 = round(budget_bits/64); n2 = the remaining bits at 2 bits
    each, rounded down.  This reproduces every count the workloads print
    (2/32/968 for 4096x4096 at 1/16, 2/16/480 at 1/32).
    """
    rho = 16.0 / budget
    bits = rho * out * inn / (out + inn)
    n8 = 2
    n3 = int(np.floor(bits / 64.0 + 0.5))
    n2 = int(np.floor((bits - 8 * n8 - 3 * n3) / 2.0))
    return n8, n3, n2


def budget_bits(n8: int, n3: int, n2: int, out: int, inn: int) -> int:
    """Bits the kept pairs store, codes only: sum_i b_i (out + in)."""
    return (8 * n8 + 3 * n3 + 2 * n2) * (out + inn)


def fp16_rne(x) -> np.ndarray:
    """fp64 -> fp16, round to nearest even, converted directly (no fp32 step)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16)


def quantize_group(w, bits: int) -> Tuple[np.ndarray, np.float16, np.float16]:
    """Quantize one group (<= 128 values) to `bits` bits.

    [R] Asymmetric min/max round-to-nearest with an integer zero point:
      mn = min(0, min w), mx = max(0, max w), maxq = 2^bits - 1
      s  = (mx - mn) / maxq              in fp64
      s_h = fp16(s), RNE, straight from fp64; s_h = 1 if it rounds to 0;
            an infinite s_h is an error
      z  = clamp(rint(-mn / s_h), 0, maxq)       (stored in fp16, exact)
      q_k = clamp(rint(w_k / s_h) + z, 0, maxq)
    rint is round-half-to-even of the correctly rounded fp64 quotient.
    Returns (codes uint8, s_h, z) with s_h, z as np.float16.
    """
    w = np.asarray(w, dtype=np.float64)
    if not np.all(np.isfinite(w)):
        raise RangeError("non-finite input")
    maxq = (1 << bits) - 1
    mn = min(0.0, float(w.min()))
    mx = max(0.0, float(w.max()))
    s = (mx - mn) / maxq
    sh = fp16_rne(s)
    if sh == 0:
        sh = np.float16(1.0)
    if not np.isfinite(sh):
        raise RangeError("fp16 scale overflow")
    shd = float(sh)
    z = min(max(np.rint(-mn / shd), 0.0), float(maxq))
    q = np.clip(np.rint(w / shd) + z, 0, maxq)
    return q.astype(np.uint8), sh, np.float16(z)


def quantize_vector(w, bits: int):
    """Quantize a singular vector group by group along its length.

    [R] The group axis is the vector's own length, 128 consecutive elements
    per group (groups across ranks are impossible: only 2 pairs sit at 8
    bits).  Returns codes uint8 [n], scale fp16 [n/128], zero fp16 [n/128].
    """
    w = np.asarray(w)
    n = w.shape[0]
    assert n % GROUP == 0
    codes = np.empty(n, np.uint8)
    scale = np.empty(n // GROUP, np.float16)
    zero = np.empty(n // GROUP, np.float16)
    for g in range(n // GROUP):
        c, sh, z = quantize_group(w[g * GROUP:(g + 1) * GROUP], bits)
        codes[g * GROUP:(g + 1) * GROUP] = c
        scale[g] = sh
        zero[g] = z
    return codes, scale, zero


def dequantize(codes, scale, zero) -> np.ndarray:
    """fp16 values of one vector: w_hat_k = fp16(s_h * (q_k - z)).

    codes [n], scale/zero fp16 [n/128].  The product s_h*(q-z) is exact in
    fp64 (11-bit mantissa times a 9-bit integer), so only the final fp16
    rounding (RNE) is taken.
    """
    codes = np.asarray(codes, dtype=np.float64)
    n = codes.shape[-1]
    s = np.repeat(np.asarray(scale, dtype=np.float64), GROUP, axis=-1)[..., :n]
    z = np.repeat(np.asarray(zero, dtype=np.float64), GROUP, axis=-1)[..., :n]
    return fp16_rne(s * (codes - z))


def dequantize_exact(codes, scale, zero) -> np.ndarray:
    """The unrounded grid values s_h * (q_k - z) in fp64 (exact).

    A kernel may multiply by these exact products instead of their fp16
    roundings (e.g. when it folds the zero point out of a dot product:
    sum_k s(q_k - z) x_k = s (sum_k q_k x_k - z sum_k x_k)).  Rounding them
    to fp16 gives `dequantize` bit for bit."""
    codes = np.asarray(codes, dtype=np.float64)
    n = codes.shape[-1]
    s = np.repeat(np.asarray(scale, dtype=np.float64), GROUP, axis=-1)[..., :n]
    z = np.repeat(np.asarray(zero, dtype=np.float64), GROUP, axis=-1)[..., :n]
    return s * (codes - z)


def compress(u, sigma, v, n8: int, n3: int, n2: int):
    """Quantize the first r = n8+n3+n2 pairs: 8-bit, then 3-bit, then 2-bit.

    u [>=r][out], sigma [>=r], v [>=r][in], given in descending-sigma order
    (ties keep the given order).  The rest are dropped (0 bits).  sigma is
    kept unquantized in fp32.
    Returns (codes_u [r][out], codes_v [r][in], sz_u [r][out/128][2],
    sz_v [r][in/128][2], sigma fp32 [r]) where sz holds the fp16 bit patterns
    (scale, zero).
    """
    r = n8 + n3 + n2
    u = np.asarray(u)
    v = np.asarray(v)
    out, inn = u.shape[1], v.shape[1]
    widths = [8] * n8 + [3] * n3 + [2] * n2
    codes_u = np.zeros((r, out), np.uint8)
    codes_v = np.zeros((r, inn), np.uint8)
    sz_u = np.zeros((r, out // GROUP, 2), np.uint16)
    sz_v = np.zeros((r, inn // GROUP, 2), np.uint16)
    for i, b in enumerate(widths):
        cu, su, zu = quantize_vector(u[i], b)
        cv, sv, zv = quantize_vector(v[i], b)
        codes_u[i], codes_v[i] = cu, cv
        sz_u[i, :, 0], sz_u[i, :, 1] = su.view(np.uint16), zu.view(np.uint16)
        sz_v[i, :, 0], sz_v[i, :, 1] = sv.view(np.uint16), zv.view(np.uint16)
    return codes_u, codes_v, sz_u, sz_v, np.asarray(sigma[:r], dtype=np.float32)


def dequant_all(codes, sz, exact: bool = False):
    """fp16 values for all ranks (or the exact fp64 products if `exact`):
    codes [r][n], sz [r][n/128][2] (bit patterns)."""
    codes = np.asarray(codes)
    sz = np.asarray(sz, dtype=np.uint16)
    s = sz[..., 0].view(np.float16)
    z = sz[..., 1].view(np.float16)
    return dequantize_exact(codes, s, z) if exact else dequantize(codes, s, z)
