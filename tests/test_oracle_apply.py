"""Pins of the oracle's apply: brute-force loops, closed forms, special cases
that reduce to a plain matrix product, and routing invariants."""
import numpy as np
import pytest

import synth
from oracle import apply as oap
from oracle import layout, quant


def _tiny(seed=0, out=128, inn=256, spec=(2, 4, 6), tokens=3):
    c = synth.small_case(seed, out, inn, *spec, tokens)
    d = c["delta"]
    u_hat, v_hat = oap.dequant_pairs(d.codes_u, d.codes_v, d.sz_u, d.sz_v)
    return c, d, u_hat, v_hat


def test_brute_force_agrees_with_factored():
    """Triple loop over o, j, i (the definition (W + U diag(s) V) x) against
    the factored W x + U (s * (V x))."""
    c, d, u_hat, v_hat = _tiny()
    y_bf = oap.brute_force(c["w"], c["x"], u_hat, d.sigma, v_hat)
    y = oap.apply_factored(c["w"], c["x"], u_hat, d.sigma, v_hat)
    assert np.max(np.abs(y - y_bf)) <= 1e-12 * np.max(np.abs(y_bf))
    # and the delta alone (W absent), where a dropped term would show
    y_bf = oap.brute_force(None, c["x"], u_hat, d.sigma, v_hat)
    y = oap.apply_factored(None, c["x"], u_hat, d.sigma, v_hat)
    assert np.max(np.abs(y - y_bf)) <= 1e-12 * np.max(np.abs(y_bf))


def test_sigma_zero_gives_backbone_matmul():
    c, d, u_hat, v_hat = _tiny(1)
    y = oap.apply_factored(c["w"], c["x"], u_hat, np.zeros_like(d.sigma), v_hat)
    x = synth.bf16_bits_to_f32(c["x"]).astype(np.float64)
    w = synth.bf16_bits_to_f32(c["w"]).astype(np.float64)
    assert np.allclose(y, np.einsum("tj,oj->to", x, w), rtol=0, atol=1e-13)


def test_single_rank_single_group_closed_form():
    """W = 0, one rank, in = out = 128: y_o = s * u_o * sum_j v_j x_j with the
    dequantized values, summed here element by element."""
    rng = np.random.default_rng(2)
    cu = rng.integers(0, 4, (1, 128)).astype(np.uint8)
    cv = rng.integers(0, 4, (1, 128)).astype(np.uint8)
    su = np.array([[[np.float16(0.01).view(np.uint16), np.float16(2).view(np.uint16)]]], np.uint16)
    sv = np.array([[[np.float16(0.03).view(np.uint16), np.float16(1).view(np.uint16)]]], np.uint16)
    x = synth.activations(rng, 2, 128)
    sig = np.array([0.7], np.float32)
    y = oap.apply_codes(None, x, cu, cv, su, sv, sig)
    uh = np.float16(0.01) * (cu[0].astype(np.float64) - 2)  # fp16 grid values
    vh = np.float16(0.03) * (cv[0].astype(np.float64) - 1)
    uh = uh.astype(np.float16).astype(np.float64)
    vh = vh.astype(np.float16).astype(np.float64)
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    for t in range(2):
        dot = sum(vh[j] * xf[t, j] for j in range(128))
        ref = [float(np.float32(0.7)) * uh[o] * dot for o in range(128)]
        assert np.allclose(y[t], ref, rtol=1e-13, atol=0)


def test_unquantized_pairs_reproduce_dense_delta():
    """All pairs kept and unquantized: the factored apply equals the dense
    delta times x (a plain matrix product)."""
    c0 = synth.make_c0()
    u, s, v = quant.svd_pairs(c0["delta"])
    y = oap.apply_factored(None, c0["x"], u, s, v)
    xf = synth.bf16_bits_to_f32(c0["x"]).astype(np.float64)
    ref = xf @ c0["delta"].astype(np.float64).T
    assert np.max(np.abs(y - ref)) <= 1e-6 * np.max(np.abs(ref))


def test_c0_truncation_error_is_the_dropped_tail():
    """Keeping 32 of 256 unquantized pairs of s_i = i^-1.5 leaves exactly the
    tail's share of the Frobenius norm: sqrt(sum_{i>32} i^-3 / sum_i i^-3),
    about 1.97%.  Quantizing the kept pairs only adds to it."""
    c0 = synth.make_c0()
    u, s, v = quant.svd_pairs(c0["delta"])
    d = c0["delta"].astype(np.float64)
    i = np.arange(1, 257, dtype=np.float64)
    tail = np.sqrt((i[32:] ** -3).sum() / (i ** -3).sum())
    dtrunc = (u[:32].T * s[:32]) @ v[:32]
    rel_t = np.linalg.norm(dtrunc - d) / np.linalg.norm(d)
    assert abs(rel_t - tail) < 1e-4 * tail
    cu, cv, su, sv, sg = quant.compress(u, s, v, *c0["groups"])
    uh, vh = oap.dequant_pairs(cu, cv, su, sv)
    dhat = (uh.astype(np.float64).T * sg.astype(np.float64)) @ vh.astype(np.float64)
    rel = np.linalg.norm(dhat - d) / np.linalg.norm(d)
    assert tail < rel < 0.15


def test_apply_packed_equals_apply_codes():
    spec = (256, 256, 2, 8, 22)
    c = synth.small_case(4, 256, 256, 2, 8, 22, 4)
    d = c["delta"]
    buf = layout.pack(spec, d.codes_u, d.codes_v, d.sz_u, d.sz_v, d.sigma)
    y1 = oap.apply_packed(spec, buf, c["w"], c["x"])
    y2 = oap.apply_codes(c["w"], c["x"], d.codes_u, d.codes_v, d.sz_u, d.sz_v, d.sigma)
    assert np.array_equal(y1, y2)


def _tenants(n, seed=7, out=128, inn=128):
    ts = []
    for k in range(n):
        d = synth.small_delta(seed + k, out, inn, 1, 3, 5)
        uh, vh = oap.dequant_pairs(d.codes_u, d.codes_v, d.sz_u, d.sz_v)
        ts.append((uh, d.sigma, vh))
    return ts


def test_multitenant_routes_each_token():
    rng = np.random.default_rng(3)
    ts = _tenants(4)
    w = synth.base_weight(rng, 128, 128)
    x = synth.activations(rng, 10, 128)
    ids = np.array([0, 3, -1, 1, 1, 2, 7, 0, 3, -1], np.int32)
    y = oap.apply_multitenant(w, x, ids, ts)
    for t, k in enumerate(ids):
        if 0 <= k < 4:
            ref = oap.apply_factored(w, x[t:t + 1], *ts[k])[0]
        else:
            ref = oap.apply_factored(w, x[t:t + 1], ts[0][0], np.zeros(9), ts[0][2])[0]
        assert np.allclose(y[t], ref, rtol=1e-14, atol=1e-14)
    perm = rng.permutation(10)
    yp = oap.apply_multitenant(w, x[perm], ids[perm], ts)
    assert np.allclose(yp, y[perm], rtol=1e-14, atol=1e-14)


def test_prefill_segments():
    rng = np.random.default_rng(4)
    ts = _tenants(3)
    w = synth.base_weight(rng, 128, 128)
    x = synth.activations(rng, 9, 128)
    seg = np.array([0, 2, 2, 9])
    y = oap.apply_prefill(w, x, seg, ts)
    ids = np.array([0, 0, 2, 2, 2, 2, 2, 2, 2])
    assert np.array_equal(y, oap.apply_multitenant(w, x, ids, ts))


def test_rel_l2_per_token():
    a = np.array([[3.0, 4.0], [1.0, 0.0]])
    b = np.array([[3.0, 4.5], [1.0, 0.0]])
    assert np.allclose(oap.rel_l2_per_token(b, a), [0.1, 0.0])
