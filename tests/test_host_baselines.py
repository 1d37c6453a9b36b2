"""Host side of the two baselines (fp16 low-rank, BitDelta) against the
oracle, on the CPU: sizes, bit-exact packers, workspace sizes and argument
checks.  Device entry points are called only with arguments the host checks
reject (or T = 0), so no kernel is launched."""
import ctypes

import numpy as np
import pytest

import synth
import tenant_rank_serving_amd as trs
from oracle import baselines as bl

LR, BD = trs.DC_KIND_LOWRANK, trs.DC_KIND_BITDELTA
# Fake device addresses: the host checks reject these calls before any launch.
X, Y, WB, WS, IDS = 0x10000, 0x900000, 0x4000000, 0x8000000, 0xA000000


@pytest.fixture(scope="module")
def L():
    return trs.lib()


@pytest.mark.parametrize("out,inn,r", [(256, 384, 5), (128, 128, 0), (128, 128, 16), (384, 256, 37),
                                        (4096, 4096, 128), (11008, 4096, 186), (1024, 4096, 25)])
def test_lowrank_sizes_match_oracle(out, inn, r):
    _, total = bl.lowrank_regions(out, inn, r)
    assert trs.dc_baseline_bytes(LR, out, inn, r) == total
    assert trs.dc_baseline_algorithmic_bytes(LR, out, inn, r) == 2 * r * (out + inn) + 4 * r


@pytest.mark.parametrize("out,inn", [(128, 128), (256, 384), (4096, 11008)])
def test_bitdelta_sizes_match_oracle(out, inn):
    assert trs.dc_baseline_bytes(BD, out, inn) == bl.bitdelta_bytes(out, inn)
    assert trs.dc_baseline_algorithmic_bytes(BD, out, inn) == out * inn // 8 + 4


def test_sizes_reject_bad_shapes():
    assert trs.dc_baseline_bytes(LR, 200, 128, 4) == 0
    assert trs.dc_baseline_bytes(LR, 128, 128, 129) == 0
    assert trs.dc_baseline_bytes(LR, 128, 128, -1) == 0
    assert trs.dc_baseline_bytes(BD, 128, 100) == 0
    assert trs.dc_baseline_bytes(BD, 128, 128, 1) == 0
    assert trs.dc_baseline_bytes(3, 128, 128, 0) == 0


@pytest.mark.parametrize("seed,out,inn,r", [(0, 256, 384, 5), (1, 384, 256, 37), (2, 128, 128, 128),
                                             (3, 11008, 4096, 186)])
def test_pack_lowrank_bit_exact(seed, out, inn, r):
    U, s, V = synth.random_lowrank(np.random.default_rng(seed), out, inn, r)
    assert np.array_equal(trs.dc_pack_lowrank(U, s, V), bl.lowrank_pack(U, s, V))


@pytest.mark.parametrize("seed,out,inn", [(0, 128, 128), (1, 256, 384), (2, 4096, 4096)])
def test_pack_bitdelta_bit_exact(seed, out, inn):
    bits, a = synth.random_bitdelta(np.random.default_rng(seed), out, inn)
    got = trs.dc_pack_bitdelta(bits, a)
    assert np.array_equal(got, bl.bitdelta_pack(bits, a))
    back, a2 = bl.bitdelta_unpack(got, out, inn)
    assert np.array_equal(back, bits) and a2 == a


def test_pack_errors(L):
    buf = np.zeros(1 << 16, np.uint8)
    U = np.zeros((4, 128), np.uint16)
    V = np.zeros((4, 128), np.uint16)
    s = np.zeros(4, np.float32)
    p = lambda a: a.ctypes.data
    assert L.dc_pack_lowrank(128, 128, 4, None, p(s), p(V), p(buf), buf.size) == trs.DC_ERR_INVALID_ARG
    assert L.dc_pack_lowrank(128, 120, 4, p(U), p(s), p(V), p(buf), buf.size) == trs.DC_ERR_SHAPE
    assert L.dc_pack_lowrank(128, 128, 4, p(U), p(s), p(V), p(buf), 100) == trs.DC_ERR_BUFFER
    assert L.dc_pack_lowrank(128, 128, 0, None, None, None, p(buf), 0) == trs.DC_OK
    bits = np.zeros((128, 128), np.uint8)
    assert L.dc_pack_bitdelta(128, 128, None, ctypes.c_float(1.0), p(buf), buf.size) == trs.DC_ERR_INVALID_ARG
    assert L.dc_pack_bitdelta(128, 128, p(bits), ctypes.c_float(np.inf), p(buf), buf.size) == trs.DC_ERR_RANGE
    assert L.dc_pack_bitdelta(128, 128, p(bits), ctypes.c_float(1.0), p(buf), 100) == trs.DC_ERR_BUFFER


def _bv(kind, out, inn, r, base=0x200000):
    return trs._lib.dc_baseline_view(kind, out, inn, r, ctypes.c_void_p(base))


def _arr(*vs):
    return (trs._lib.dc_baseline_view * len(vs))(*vs)


def test_workspace_bytes_rules(L):
    for kind, r in ((LR, 37), (BD, 0)):
        v = _arr(_bv(kind, 512, 384, r), _bv(kind, 512, 384, r))
        one = L.dc_baseline_workspace_bytes(v, 1, 2, 40)
        assert one > 0 and one % 256 == 0
        assert L.dc_baseline_workspace_bytes(v, 1, 2, 41) >= one
        assert L.dc_baseline_workspace_bytes(v, 1, 2, -1) == 0
        assert L.dc_baseline_workspace_bytes(v, 0, 2, 8) == 0
        assert L.dc_baseline_workspace_bytes(v, 2, 1, 8) > 0   # two matrices of one tenant
    mixed = _arr(_bv(LR, 512, 384, 37), _bv(BD, 512, 384, 0))
    assert L.dc_baseline_workspace_bytes(mixed, 1, 2, 8) == 0
    shapes = _arr(_bv(BD, 512, 384, 0), _bv(BD, 256, 384, 0))
    assert L.dc_baseline_workspace_bytes(shapes, 1, 2, 8) == 0
    assert L.dc_baseline_workspace_bytes(shapes, 2, 1, 8) > 0   # a group: outs may differ
    ins = _arr(_bv(BD, 512, 384, 0), _bv(BD, 512, 256, 0))
    assert L.dc_baseline_workspace_bytes(ins, 2, 1, 8) == 0
    # a wider tenant needs at least as much
    small = L.dc_baseline_workspace_bytes(_arr(_bv(LR, 512, 384, 16)), 1, 1, 64)
    big = L.dc_baseline_workspace_bytes(_arr(_bv(LR, 512, 384, 300)), 1, 1, 64)
    assert big > small


def test_apply_argument_checks(L):
    views = _arr(_bv(LR, 256, 256, 20), _bv(LR, 256, 256, 0, 0))
    T = 8
    need = L.dc_baseline_workspace_bytes(views, 1, 2, T)
    ap = L.dc_apply_baseline_multitenant
    assert ap(views, 2, WB, X, None, Y, T, WS, need, None) == trs.DC_ERR_INVALID_ARG    # no ids
    assert ap(views, 2, WB, None, IDS, Y, T, WS, need, None) == trs.DC_ERR_INVALID_ARG
    assert ap(views, 2, WB, X + 2, IDS, Y, T, WS, need, None) == trs.DC_ERR_ALIGN
    assert ap(views, 2, WB, X, IDS, Y, T, WS + 16, need, None) == trs.DC_ERR_ALIGN
    assert ap(views, 2, WB, X, IDS, Y, T, WS, need - 1, None) == trs.DC_ERR_BUFFER
    assert ap(views, 2, WB, X, IDS, X + 64, T, WS, need, None) == trs.DC_ERR_INVALID_ARG   # overlap
    assert ap(views, 0, WB, X, IDS, Y, T, WS, need, None) == trs.DC_ERR_INVALID_ARG
    assert ap(views, 129, WB, X, IDS, Y, T, WS, need, None) == trs.DC_ERR_UNSUPPORTED
    assert ap(views, 2, WB, X, IDS, Y, 0, WS, need, None) == trs.DC_OK     # T = 0, r = 0 with a NULL base
    nobase = _arr(_bv(LR, 256, 256, 20, 0))
    assert ap(nobase, 1, WB, X, IDS, Y, T, WS, need, None) == trs.DC_ERR_INVALID_ARG
    odd = _arr(_bv(LR, 256, 256, 20, 0x200008))
    assert ap(odd, 1, WB, X, IDS, Y, T, WS, need, None) == trs.DC_ERR_ALIGN
    bd0 = _arr(_bv(BD, 256, 256, 0, 0))
    assert ap(bd0, 1, WB, X, IDS, Y, T, WS, need, None) == trs.DC_ERR_INVALID_ARG    # BitDelta always reads
    assert ap(_arr(_bv(BD, 256, 256, 3)), 1, WB, X, IDS, Y, T, WS, need, None) == trs.DC_ERR_SHAPE
    assert ap(_arr(_bv(LR, 256, 256, 20), _bv(BD, 256, 256, 0)), 2, WB, X, IDS, Y, T, WS, need,
              None) == trs.DC_ERR_SHAPE
    assert ap(_arr(_bv(7, 256, 256, 0)), 1, WB, X, IDS, Y, T, WS, need, None) == trs.DC_ERR_SHAPE


def test_group_argument_checks(L):
    P = ctypes.c_void_p
    v = _arr(_bv(BD, 512, 384, 0), _bv(BD, 512, 384, 0), _bv(BD, 128, 384, 0), _bv(BD, 128, 384, 0))
    need = L.dc_baseline_workspace_bytes(v, 2, 2, 8)
    grp = L.dc_apply_baseline_multitenant_group
    W2 = (P * 2)(WB, None)
    assert grp(v, 2, 2, W2, X, IDS, (P * 2)(Y, Y + 0x100000), 8, WS, need - 1, None) == trs.DC_ERR_BUFFER
    assert grp(v, 2, 2, W2, X, IDS, (P * 2)(Y, Y + 64), 8, WS, need, None) == trs.DC_ERR_INVALID_ARG
    assert grp(v, 5, 2, W2, X, IDS, (P * 2)(Y, Y + 0x100000), 8, WS, need, None) == trs.DC_ERR_UNSUPPORTED
    assert grp(v, 2, 2, W2, X, IDS, (P * 2)(Y, Y + 0x100000), 0, WS, need, None) == trs.DC_OK
