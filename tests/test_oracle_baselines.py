"""Pins of the oracle's baselines (oracle/baselines.py): the low-rank and
BitDelta deltas at the Delta-CoMe budget, checked against closed forms,
hand-derived words and brute force."""
import numpy as np
import pytest

from oracle import apply as oap
from oracle import baselines as bl
from oracle import quant
import synth


def test_lowrank_rank_fills_the_budget():
    # 1/16: 16 r (out + in) <= out in bits; 4096^2 gives exactly 128 pairs (16*128*8192 = 4096^2)
    assert bl.lowrank_rank(4096, 4096) == 128
    assert 16 * 128 * 8192 == 4096 * 4096
    for out, inn, budget in ((11008, 4096, 16), (4096, 11008, 16), (5120, 5120, 16), (13824, 5120, 16),
                             (1024, 4096, 32), (14336, 4096, 32), (256, 384, 16)):
        r = bl.lowrank_rank(out, inn, budget)
        bits = 16 * out * inn // budget
        assert 16 * r * (out + inn) <= bits < 16 * (r + 1) * (out + inn)
    assert bl.lowrank_rank(11008, 4096) == 186


def test_lowrank_fp16_rounding_and_exact_reconstruction():
    # fp16 of 1/3 is 0x3555 (0.333251953125), round to nearest
    U, sg, V = bl.lowrank_compress(np.array([[1 / 3, 0.5]]), np.array([2.0]), np.array([[-1 / 3, 1.0]]), 1)
    assert U.view(np.uint16)[0, 0] == 0x3555 and V.view(np.uint16)[0, 0] == 0xB555 and sg[0] == 2.0
    # a delta of exact rank r with fp16-representable vectors is reproduced exactly by the factored apply
    rng = np.random.default_rng(3)
    r, out, inn = 5, 256, 384
    u = quant.fp16_rne(rng.standard_normal((r, out))).astype(np.float64)
    v = quant.fp16_rne(rng.standard_normal((r, inn))).astype(np.float64)
    s = np.array([4.0, 2.0, 1.0, 0.5, 0.25])
    U16, s32, V16 = bl.lowrank_compress(u, s, v, r)
    assert np.array_equal(U16.astype(np.float64), u) and np.array_equal(V16.astype(np.float64), v)
    x = synth.activations(rng, 3, inn)
    dense = synth.bf16_bits_to_f32(x).astype(np.float64) @ ((u.T * s) @ v).T
    np.testing.assert_allclose(oap.apply_factored(None, x, U16, s32, V16), dense, rtol=1e-12, atol=1e-12)


def test_lowrank_layout_golden_and_round_trip():
    reg, total = bl.lowrank_regions(256, 384, 5)
    # hand-derived: sigma 20 B at 0; V 16 rank rows * 384 * 2 = 12288 B at 256;
    # U 256 rows * 32 ranks * 2 = 16384 B at 256 + 12288 = 12544
    assert reg == {"SIGMA": (0, 20), "V": (256, 12288), "U": (12544, 16384)} and total == 28928
    U = np.zeros((5, 256), np.float16)
    V = np.zeros((5, 384), np.float16)
    V[3, 77] = 1.0      # tile 0, step 2, slot 3 + 16 * ((77 % 32) / 8) = 3 + 16, element 5
    U[4, 33] = 2.0      # tile 2, step 0, slot 1 + 16 * (4 / 8) = 1, element 4
    buf = bl.lowrank_pack(U, np.arange(5, dtype=np.float32), V)
    v = buf[256:256 + 12288].view(np.float16)
    u = buf[12544:12544 + 16384].view(np.float16)
    assert np.nonzero(v)[0].tolist() == [((0 * 12 + 2) * 64 + 19) * 8 + 5]
    assert np.nonzero(u)[0].tolist() == [((2 * 1 + 0) * 64 + 1) * 8 + 4] and u[(2 * 64 + 1) * 8 + 4] == 2.0
    assert buf[:20].view(np.float32).tolist() == [0.0, 1.0, 2.0, 3.0, 4.0]
    rng = np.random.default_rng(4)
    for r in (5, 16, 37):
        U = rng.standard_normal((r, 256)).astype(np.float16)
        V = rng.standard_normal((r, 384)).astype(np.float16)
        sg = rng.random(r).astype(np.float32)
        U2, sg2, V2 = bl.lowrank_unpack(bl.lowrank_pack(U, sg, V), 256, 384, r)
        assert np.array_equal(U2.view(np.uint16), U.view(np.uint16)) and np.array_equal(V2, V)
        assert np.array_equal(sg2, sg)


def test_bitdelta_signs_and_scale_by_hand():
    d = np.array([[0.5, -0.25], [0.0, -1.0]])
    bits, a = bl.bitdelta_compress(d)
    assert bits.tolist() == [[1, 0], [1, 0]]           # an entry of 0 counts as +1
    assert a == np.float32(0.4375)                       # (0.5 + 0.25 + 0 + 1) / 4


def test_bitdelta_scale_is_l2_optimal():
    rng = np.random.default_rng(5)
    d = rng.standard_normal((64, 48)) * 0.01
    bits, a = bl.bitdelta_compress(d)
    s = bl.signs(bits)
    err = lambda c: float(((d - c * s) ** 2).sum())
    # ||D - c S||^2 = ||D - a* S||^2 + N (c - a*)^2 with a* = mean |D| (exact in fp64)
    astar = float(np.mean(np.abs(d)))
    for c in (0.0, astar * 0.5, astar, astar * 1.7):
        assert err(c) == pytest.approx(err(astar) + d.size * (c - astar) ** 2, rel=1e-10)
    assert abs(float(a) - astar) <= astar * 2.0 ** -24


def test_bitdelta_nibble_positions_golden():
    pos = [bl.nibble_position(k) for k in range(32)]
    assert sorted(pos) == list(range(32))
    # hand-derived: k=0 -> entry 0 -> bit 0; k=1 -> entry 16 -> bit 2; k=2 -> entry 1 -> bit 4;
    # k=16 -> entry 8 -> bit 1; k=17 -> entry 24 -> bit 3; k=31 -> entry 31 -> bit 31
    assert (pos[0], pos[1], pos[2], pos[16], pos[17], pos[31]) == (0, 2, 4, 1, 3, 31)
    # word >> s & 0x11111111 holds entries 8s .. 8s+7 one per nibble, in B-operand element order:
    # element e of that order is code 2e (e < 16) or 2(e - 16) + 1
    for e in range(32):
        k = 2 * e if e < 16 else 2 * (e - 16) + 1
        assert pos[k] == 4 * (e % 8) + e // 8


def test_bitdelta_pack_golden_and_round_trip():
    bits = np.zeros((16, 128), np.uint8)
    bits[0, 1] = 1                 # row 0, chunk 0: only entry 1 is +1 -> bit 2 -> word 0x4
    bits[1, :32] = 1               # row 1, chunk 0: all +1 -> 0xFFFFFFFF
    bits[2, 32 + 16] = 1           # row 2, chunk 1: entry 16 -> bit 1 -> 0x2
    buf = bl.bitdelta_pack(bits, np.float32(0.125))
    assert buf.size == 256 + 16 * 128 // 8
    assert buf[:4].view(np.float32)[0] == 0.125
    w = buf[256:].view(np.uint32).reshape(1, 1, 4, 16)          # [T][g][c][row]
    assert w[0, 0, 0, 0] == 0x4 and w[0, 0, 0, 1] == 0xFFFFFFFF and w[0, 0, 1, 2] == 0x2
    assert int(w.sum()) == 0x4 + 0xFFFFFFFF + 0x2
    rng = np.random.default_rng(6)
    b2 = rng.integers(0, 2, (48, 384)).astype(np.uint8)
    back, a = bl.bitdelta_unpack(bl.bitdelta_pack(b2, np.float32(3.5)), 48, 384)
    assert np.array_equal(back, b2) and a == np.float32(3.5)


def test_bitdelta_apply_brute_force():
    rng = np.random.default_rng(7)
    out, inn, T = 5, 7, 3
    d = rng.standard_normal((out, inn))
    bits, a = bl.bitdelta_compress(d)
    w = synth.base_weight(rng, out, inn)
    x = synth.activations(rng, T, inn)
    xf = oap.bf16_to_f64(x)
    wf = oap.bf16_to_f64(w)
    ref = [[sum((wf[o][j] + float(a) * (1.0 if bits[o][j] else -1.0)) * xf[t][j] for j in range(inn))
            for o in range(out)] for t in range(T)]
    np.testing.assert_allclose(bl.bitdelta_apply(w, x, bits, a), np.array(ref), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(bl.bitdelta_apply(None, x, bits, a),
                               np.array(ref) - xf @ wf.T, rtol=1e-12, atol=1e-12)
    ids = np.array([1, -1, 0])
    ten = [bl.bitdelta_compress(rng.standard_normal((out, inn))), (bits, a)]
    y = bl.bitdelta_apply_multitenant(w, x, ids, ten)
    np.testing.assert_allclose(y[0], bl.bitdelta_apply(w, x[:1], bits, a)[0], rtol=1e-12)
    np.testing.assert_allclose(y[1], xf[1] @ wf.T, rtol=1e-12)


def test_lowrank_multitenant_brute_force():
    rng = np.random.default_rng(8)
    out, inn, T = 6, 5, 4
    ten = []
    for r in (2, 0, 3):
        ten.append((rng.standard_normal((r, out)).astype(np.float16), rng.random(r).astype(np.float32),
                    rng.standard_normal((r, inn)).astype(np.float16)))
    w = synth.base_weight(rng, out, inn)
    x = synth.activations(rng, T, inn)
    ids = np.array([2, -1, 0, 1])
    y = bl.lowrank_apply_multitenant(w, x, ids, ten)
    xf, wf = oap.bf16_to_f64(x), oap.bf16_to_f64(w)
    for t in range(T):
        for o in range(out):
            ref = sum(wf[o][j] * xf[t][j] for j in range(inn))
            if ids[t] >= 0:
                U, sg, V = ten[ids[t]]
                for i in range(len(sg)):
                    ref += float(U[i][o]) * float(sg[i]) * sum(float(V[i][j]) * xf[t][j] for j in range(inn))
            assert abs(y[t][o] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_lowrank_rank_table_matches_the_budget_rule():
    for (out, inn, budget), r in synth.LOWRANK_R.items():
        assert bl.lowrank_rank(out, inn, budget) == r


def test_baseline_generators_are_seeded():
    u, s, v = synth.make_c1_lowrank(4)
    assert u.shape == (186, 11008) and v.shape == (186, 4096) and s.shape == (186,)
    u2, _, _ = synth.make_c1_lowrank(4)
    assert np.array_equal(u.view(np.uint16), u2.view(np.uint16))
    b, a = synth.make_c1_bitdelta(0)
    assert b.shape == (4096, 4096) and set(np.unique(b)) == {0, 1} and 1e-4 < a < 1e-2
