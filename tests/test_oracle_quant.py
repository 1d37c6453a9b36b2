"""Pins of the oracle's compression side (SVD, rank groups, quantizer).

Each test checks the oracle against something other than itself: a closed
form, a hand-derived value, an exhaustive search, or a construction whose
answer is known.
"""
import numpy as np
import pytest

import synth
from oracle import quant
from conftest import read_golden


# --------------------------------------------------------------------- SVD
def test_svd_reconstructs_small_delta():
    """A full-rank, unquantized SVD rebuilds the c0 delta to 1e-5 relative
    Frobenius norm."""
    c0 = synth.make_c0()
    u, s, v = quant.svd_pairs(c0["delta"])
    rebuilt = (u.T * s) @ v
    d = c0["delta"].astype(np.float64)
    rel = np.linalg.norm(rebuilt - d) / np.linalg.norm(d)
    assert rel <= 1e-5


def test_svd_recovers_construction():
    """c0 is built as U0 diag(i^-1.5) V0^T, so the singular values are
    i^-1.5 (closed form) and the kept vectors match U0/V0 up to sign."""
    c0 = synth.make_c0()
    u, s, v = quant.svd_pairs(c0["delta"])
    i = np.arange(1, 257, dtype=np.float64)
    ref = i ** -1.5
    assert np.all(np.abs(s[:32] - ref[:32]) / ref[:32] < 1e-5)
    assert np.all(np.abs(s - ref) / ref < 1e-4)
    for k in range(32):
        assert abs(abs(u[k] @ c0["u0"][:, k]) - 1.0) < 1e-4
        assert abs(abs(v[k] @ c0["v0"][:, k]) - 1.0) < 1e-4
        # u_k and v_k must carry the same sign flip
        assert (u[k] @ c0["u0"][:, k]) * (v[k] @ c0["v0"][:, k]) > 0


def test_svd_sign_rule():
    """Largest-magnitude entry of each v_i is positive; flipping the input
    sign of a rank-1 delta flips u, not v."""
    rng = np.random.default_rng(5)
    a = rng.standard_normal(64)
    b = rng.standard_normal(48)
    b[np.argmax(np.abs(b))] = -abs(b).max() * 1.5  # dominant entry negative
    for sgn in (1.0, -1.0):
        u, s, v = quant.svd_pairs(sgn * np.outer(a, b))
        j = np.argmax(np.abs(v[0]))
        assert v[0, j] > 0
        assert np.allclose(s[0] * np.outer(u[0], v[0]), sgn * np.outer(a, b), atol=1e-12)
        assert np.sign(u[0] @ a) == -sgn  # v has the sign of -b, so u carries -sgn*a


# -------------------------------------------------------------- rank groups
PRINTED = {  # counts the workloads print
    (4096, 4096, 16): (2, 32, 968),
    (4096, 4096, 32): (2, 16, 480),
}


@pytest.mark.parametrize("key", sorted(PRINTED))
def test_rank_groups_printed_counts(key):
    assert quant.rank_groups(*key) == PRINTED[key]


@pytest.mark.parametrize("key", sorted(synth.RANK_GROUPS))
def test_rank_groups_budget(key):
    """1/16 equals BitDelta's 1 bit per parameter: sum b_i (out+in) <= rho*out*in,
    with less than one 2-bit pair of slack; the generator's table agrees."""
    out, inn, budget = key
    n8, n3, n2 = quant.rank_groups(out, inn, budget)
    assert (n8, n3, n2) == synth.RANK_GROUPS[key]
    cap = out * inn * 16 // budget
    used = quant.budget_bits(n8, n3, n2, out, inn)
    assert used <= cap
    assert cap - used < 2 * (out + inn)
    assert n8 + n3 + n2 <= min(out, inn)


def test_rank_groups_exact_budget_c1():
    # 2*8 + 32*3 + 968*2 = 2048 = 4096*4096/8192, exactly the 1-bit budget
    assert quant.budget_bits(2, 32, 968, 4096, 4096) == 4096 * 4096
    assert quant.budget_bits(2, 16, 480, 4096, 4096) == 4096 * 4096 // 2


# ---------------------------------------------------------------- quantizer
def test_fp16_direct_rounding():
    """fp64 -> fp16 must round once: 1 + 2^-11 + 2^-40 is just above the tie
    between 1 and 1 + 2^-10 and must round up (an fp32 step would round it to
    the tie and then down to 1)."""
    assert float(quant.fp16_rne(1 + 2 ** -11 + 2 ** -40)) == 1 + 2 ** -10
    assert float(quant.fp16_rne(1 + 2 ** -11)) == 1.0            # tie -> even
    assert float(quant.fp16_rne(1 + 3 * 2 ** -11)) == 1 + 2 ** -9  # tie -> even


def test_quantize_ramp_golden():
    g = dict((ln.split()[0], ln.split()[1:]) for ln in read_golden("ramp3.txt"))
    w = (-1.0 + 2.0 * np.arange(128) / 127.0).astype(np.float32)
    q, sh, z = quant.quantize_group(w, 3)
    assert int(np.float16(sh).view(np.uint16)) == int(g["scale_bits"][0], 16)
    assert float(sh) == float(g["scale"][0])
    assert float(z) == float(g["zero"][0])
    hist = np.bincount(q, minlength=8)
    assert hist.tolist() == [int(t) for t in g["histogram"]]
    deq = quant.dequantize(q, [sh], [z])
    assert float(deq[0]) == float(g["deq0"][0])
    assert float(deq[-1]) == float(g["deq7"][0])


def test_dequant_rounds_product_to_fp16():
    """s_h = 1 + 2^-10 and q - z = 3 give 3 + 3*2^-10, a tie between the two
    fp16 neighbours 3 + 2^-9 and 3 + 2^-8; round-half-even picks 3 + 2^-8."""
    sh = np.float16(1 + 2 ** -10)
    v = quant.dequantize(np.array([3] + [0] * 127), [sh], [np.float16(0)])
    assert float(v[0]) == 3 + 2 ** -8


@pytest.mark.parametrize("bits", [8, 3, 2])
@pytest.mark.parametrize("seed", range(6))
def test_quantizer_is_nearest_grid_point(bits, seed):
    """Brute force: each code is the grid point s_h*(c - z), c in [0, maxq],
    nearest to w (ties cannot occur in random data)."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal(128) * rng.uniform(1e-4, 10)).astype(np.float32)
    if seed % 2:
        w = np.abs(w)  # all-positive group: mn = 0 keeps 0 in the range
    q, sh, z = quant.quantize_group(w, bits)
    maxq = (1 << bits) - 1
    grid = float(sh) * (np.arange(maxq + 1) - float(z))
    best = np.argmin(np.abs(w.astype(np.float64)[:, None] - grid[None, :]), axis=1)
    assert np.array_equal(q, best.astype(np.uint8))
    assert 0 <= float(z) <= maxq and float(z) == int(float(z))
    # range covered: min w and max w lie within one step of the grid ends
    assert grid[0] <= min(0.0, w.min()) + float(sh)
    assert grid[-1] >= max(0.0, w.max()) - float(sh)


@pytest.mark.parametrize("bits", [8, 3, 2])
def test_quantizer_exact_grid_roundtrip(bits):
    """Values placed exactly on a grid that uses both code 0 and maxq come
    back with the same scale, zero and codes."""
    rng = np.random.default_rng(bits)
    maxq = (1 << bits) - 1
    for trial in range(20):
        sh = np.float16(rng.uniform(1e-3, 2.0))
        z = int(rng.integers(0, maxq + 1))
        q = rng.integers(0, maxq + 1, size=128)
        q[0], q[1] = 0, maxq
        w = (float(sh) * (q - z)).astype(np.float32)
        assert np.all(w.astype(np.float64) == float(sh) * (q - z))  # exact in fp32
        q2, sh2, z2 = quant.quantize_group(w, bits)
        assert sh2 == sh and int(z2) == z
        assert np.array_equal(q2, q.astype(np.uint8))


def test_quantizer_zero_and_range_cases():
    q, sh, z = quant.quantize_group(np.zeros(128, np.float32), 2)
    assert float(sh) == 1.0 and float(z) == 0 and not q.any()
    with pytest.raises(quant.RangeError):
        quant.quantize_group(np.array([np.nan] + [0.0] * 127), 3)
    with pytest.raises(quant.RangeError):
        quant.quantize_group(np.array([1e6, -1e6] + [0.0] * 126), 2)  # s = 6.7e5 > fp16 max


def test_compress_segments_and_order():
    """compress quantizes the first n8 pairs at 8 bits, next n3 at 3, next n2
    at 2; code ranges tell the widths apart."""
    u, s, v = synth.random_singular_pairs(3, 256, 384, 12)
    cu, cv, su, sv, sg = quant.compress(u, s, v, 2, 4, 5)
    assert cu.shape == (11, 256) and cv.shape == (11, 384)
    assert su.shape == (11, 2, 2) and sv.shape == (11, 3, 2)
    assert cv[:2].max() > 7 and cv[2:6].max() <= 7 and cv[6:].max() <= 3
    assert cv[2:6].max() == 7 and cv[6:].max() == 3
    assert np.array_equal(sg, s[:11])


@pytest.mark.parametrize("bits", [8, 3, 2])
def test_dequantize_exact_rounds_to_dequantize(bits):
    """The exact grid values round to the fp16 dequantized values bit for
    bit, and differ from them by at most half an fp16 ulp."""
    rng = np.random.default_rng(40 + bits)
    w = (rng.standard_normal(128 * 6) * 0.01).astype(np.float32)
    q, s, z = quant.quantize_vector(w, bits)
    ex = quant.dequantize_exact(q, s, z)
    h = quant.dequantize(q, s, z)
    assert np.array_equal(quant.fp16_rne(ex).view(np.uint16), h.view(np.uint16))
    ulp = np.spacing(np.abs(h).astype(np.float16)).astype(np.float64)
    assert np.all(np.abs(ex - h.astype(np.float64)) <= ulp / 2)
    # a hand value: s = 1 + 2^-10, q - z = 3 -> 3 + 3*2^-10 exactly
    assert quant.dequantize_exact(np.array([3] + [0] * 127), [np.float16(1 + 2 ** -10)], [0.0])[0] == 3 + 3 * 2 ** -10
