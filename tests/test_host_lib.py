"""Host side of libdeltacome.so against the oracle, on the CPU: exported
symbols, the packed format, bit-exact quantize+pack, and argument checks.

Device entry points are called here only with arguments the host checks
reject (or T = 0), so no kernel is ever launched."""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import synth
import tenant_rank_serving_amd as trs
from oracle import layout, quant

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    return trs.lib()


def test_exports_every_declared_symbol(L):
    hdr = open(os.path.join(ROOT, "include", "deltacome.h")).read()
    declared = set(re.findall(r"^\S.*?\b(dc_\w+)\(", hdr, flags=re.M))
    assert declared == set(trs.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


SPECS = [(128, 128, 1, 1, 1), (256, 256, 2, 8, 22), (384, 128, 3, 0, 17), (128, 384, 0, 33, 0),
         (512, 256, 5, 31, 65), (128, 128, 0, 0, 0), (4096, 4096, 2, 32, 968),
         (11008, 4096, 2, 47, 1414), (1024, 4096, 2, 6, 187)]


@pytest.mark.parametrize("spec", SPECS)
def test_regions_match_oracle(spec):
    assert trs.dc_packed_bytes(spec) == layout.packed_bytes(spec)
    assert trs.dc_algorithmic_bytes(spec) == layout.algorithmic_bytes(spec)
    reg = layout.regions(spec)
    for name in trs.REGIONS:
        assert trs.dc_region(spec, name) == reg[name], name


@pytest.mark.parametrize("spec", SPECS[:6])
def test_pack_codes_bit_exact(spec):
    d = synth.small_delta(21, *spec)
    a = trs.dc_pack_codes(spec, d.codes_u, d.codes_v, d.sz_u, d.sz_v, d.sigma)
    b = layout.pack(spec, d.codes_u, d.codes_v, d.sz_u, d.sz_v, d.sigma)
    assert np.array_equal(a, b)
    back = trs.dc_unpack(spec, a)
    for x, y in zip(back, (d.codes_u, d.codes_v, d.sz_u, d.sz_v, d.sigma)):
        assert np.array_equal(np.asarray(x).view(np.uint8), np.asarray(y).view(np.uint8))


@settings(max_examples=20, deadline=None)
@given(go=st.integers(1, 3), gi=st.integers(1, 3), n8=st.integers(0, 4), n3=st.integers(0, 70),
       n2=st.integers(0, 90), seed=st.integers(0, 2 ** 31))
def test_pack_codes_bit_exact_hypothesis(go, gi, n8, n3, n2, seed):
    spec = (128 * go, 128 * gi, n8, n3, n2)
    if n8 + n3 + n2 > min(spec[0], spec[1]):
        return
    d = synth.small_delta(seed, *spec)
    a = trs.dc_pack_codes(spec, d.codes_u, d.codes_v, d.sz_u, d.sz_v, d.sigma)
    assert np.array_equal(a, layout.pack(spec, d.codes_u, d.codes_v, d.sz_u, d.sz_v, d.sigma))


def _oracle_pack(spec, u, s, v):
    cu, cv, su, sv, sg = quant.compress(u, s, v, *spec[2:])
    return layout.pack(spec, cu, cv, su, sv, sg)


def test_pack_c0_bit_exact():
    """The tiny end-to-end case: SVD on the host, then quantize+pack on both
    sides from the same fp32 singular vectors."""
    c0 = synth.make_c0()
    u, s, v = quant.svd_pairs(c0["delta"])
    u32, s32, v32 = u.astype(np.float32), s.astype(np.float32), v.astype(np.float32)
    spec = (256, 256) + tuple(c0["groups"])
    a = trs.dc_pack(spec, u32[:32], s32[:32], v32[:32])
    assert np.array_equal(a, _oracle_pack(spec, u32, s32, v32))


@pytest.mark.parametrize("seed", range(4))
def test_pack_random_pairs_bit_exact(seed):
    spec = (384, 256, 3, 9, 20)
    u, s, v = synth.random_singular_pairs(seed, 384, 256, 32, scale=10.0 ** (seed - 2))
    assert np.array_equal(trs.dc_pack(spec, u, s, v), _oracle_pack(spec, u, s, v))


@pytest.mark.parametrize("bits,spec", [(8, (128, 128, 1, 0, 0)), (3, (128, 128, 0, 1, 0)),
                                       (2, (128, 128, 0, 0, 1))])
def test_pack_ties_round_half_even(bits, spec):
    """Values exactly halfway between grid points: both sides must round to
    even.  The grid ends (codes 0 and maxq) pin the scale and zero."""
    rng = np.random.default_rng(bits)
    maxq = (1 << bits) - 1
    sh = np.float16(0.0625 * 3)
    z = maxq // 2
    q = rng.integers(0, maxq, size=128)
    w = (float(sh) * (q - z + 0.5)).astype(np.float32)
    w[0], w[1] = float(sh) * (0 - z), float(sh) * (maxq - z)
    assert np.all(w.astype(np.float64)[2:] == float(sh) * (q[2:] - z + 0.5))
    u = w[None, :]
    sig = np.ones(1, np.float32)
    a = trs.dc_pack(spec, u, sig, u)
    b = _oracle_pack(spec, u, sig, u)
    assert np.array_equal(a, b)
    cu = trs.dc_unpack(spec, a)[0][0].astype(np.int64)
    # each code is rint(q - z + 0.5) + z with ties to even
    assert np.array_equal(cu[2:], np.rint(q[2:] - z + 0.5).astype(np.int64) + z)


def test_pack_subnormal_and_tiny_scales():
    spec = (128, 128, 0, 1, 1)
    rng = np.random.default_rng(9)
    u = (rng.standard_normal((2, 128)) * 1e-6).astype(np.float32)  # scales land in fp16 subnormals
    v = (rng.standard_normal((2, 128)) * 3e-8).astype(np.float32)
    s = np.ones(2, np.float32)
    assert np.array_equal(trs.dc_pack(spec, u, s, v), _oracle_pack(spec, u, s, v))


def test_pack_errors():
    spec = (128, 128, 0, 0, 1)
    ok = np.ones((1, 128), np.float32)
    with pytest.raises(trs.DcError) as e:
        trs.dc_pack(spec, np.full((1, 128), np.nan, np.float32), np.ones(1), ok)
    assert e.value.status == trs.DC_ERR_RANGE
    big = np.zeros((1, 128), np.float32)
    big[0, 0], big[0, 1] = 1e5, -1e5   # (mx - mn)/3 overflows fp16
    with pytest.raises(trs.DcError) as e:
        trs.dc_pack(spec, big, np.ones(1), ok)
    assert e.value.status == trs.DC_ERR_RANGE
    with pytest.raises(trs.DcError) as e:
        trs.dc_pack((100, 128, 0, 0, 1), ok, np.ones(1), ok)
    assert e.value.status == trs.DC_ERR_SHAPE
    bad = np.full((1, 128), 4, np.uint8)   # 4 does not fit 2 bits
    z = np.zeros((1, 1, 2), np.uint16)
    with pytest.raises(trs.DcError) as e:
        trs.dc_pack_codes(spec, bad, np.zeros((1, 128), np.uint8), z, z, np.ones(1, np.float32))
    assert e.value.status == trs.DC_ERR_RANGE


def test_shape_checks(L):
    for spec in [(0, 128, 0, 0, 0), (128, 130, 0, 0, 0), (128, 128, -1, 0, 0),
                 (128, 256, 100, 20, 9)]:
        assert trs.dc_check_spec(spec) == trs.DC_ERR_SHAPE
        assert trs.dc_packed_bytes(spec) == 0
    assert trs.dc_check_spec((128, 256, 100, 20, 8)) == trs.DC_OK
    assert L.dc_check_spec(None) == trs.DC_ERR_INVALID_ARG
    buf = np.zeros(16, np.uint8)
    s = trs.make_spec((128, 128, 0, 0, 1))
    out = np.zeros(8, np.uint8)
    assert L.dc_unpack(ctypes.byref(s), buf.ctypes.data, buf.size, out.ctypes.data, out.ctypes.data,
                       out.ctypes.data, out.ctypes.data, out.ctypes.data) == trs.DC_ERR_BUFFER
    assert L.dc_pack_codes(ctypes.byref(s), None, None, None, None, None, buf.ctypes.data,
                           buf.size) == trs.DC_ERR_INVALID_ARG


def test_workspace_bytes_rules():
    sp = [(256, 256, 2, 8, 22)]
    assert trs.dc_workspace_bytes(trs.DC_OP_DECODE, sp, 4) > 0
    assert trs.dc_workspace_bytes(trs.DC_OP_DECODE, sp * 2, 4) == 0
    assert trs.dc_workspace_bytes(trs.DC_OP_MULTITENANT, sp + [(256, 128, 1, 1, 1)], 4) == 0
    assert trs.dc_workspace_bytes(7, sp, 4) == 0
    assert trs.dc_workspace_bytes(trs.DC_OP_MULTITENANT, sp * 3, 64) >= \
        trs.dc_workspace_bytes(trs.DC_OP_MULTITENANT, sp * 3, 4)



def test_prefill_workspace_holds_dense_operands():
    """A prefill workspace of 256 tokens or more adds the dense form's
    buffers to the multi-tenant one: fp32 t [T][rp], an fp32 rescale and a
    uint32 max per token, rp = max over tenants of the rank groups each
    rounded up to 32, summed and rounded up to 128 (at least 128), each region
    256-byte aligned; none below 256 tokens."""
    def pad(v, m):
        return -(-v // m) * m

    def dense(specs, T):
        rp = max(max(128, pad(sum(pad(n, 32) for n in sp[2:]), 128)) for sp in specs)
        return pad(4 * T * rp, 256) + 2 * pad(4 * T, 256)
    for specs, T in (([(256, 384, 2, 9, 40)] * 3, 300), ([(256, 384, 2, 9, 40), (256, 384, 0, 0, 0)] * 6, 1000),
                     ([(1024, 512, 2, 20, 150), (1024, 512, 1, 1, 1)], 513), ([(256, 256, 0, 0, 0)], 256),
                     ([(512, 512, 33, 1, 100)], 256)):
        mt = trs.dc_workspace_bytes(trs.DC_OP_MULTITENANT, specs, T)
        pf = trs.dc_workspace_bytes(trs.DC_OP_PREFILL, specs, T)
        assert pf - mt == dense(specs, T)
    sp = [(256, 384, 2, 9, 40)] * 3
    # fewer than 256 tokens can never take the dense form: no dense operands
    for T in (0, 1, 100, 255):
        assert trs.dc_workspace_bytes(trs.DC_OP_PREFILL, sp, T) == trs.dc_workspace_bytes(trs.DC_OP_MULTITENANT, sp, T)


def test_prefill_workspace_without_the_dense_operands(L):
    """A prefill workspace of the multi-tenant size is enough (the call then
    takes the decode kernels); one byte less is rejected before any launch."""
    spec = (256, 256, 2, 8, 22)
    arr = (trs._lib.dc_delta_view * 2)(_view(spec), _view(spec))
    T = 512
    seg = np.array([0, 256, 512], np.int32)
    need = trs.dc_workspace_bytes(trs.DC_OP_PREFILL, [spec] * 2, T)
    mt = trs.dc_workspace_bytes(trs.DC_OP_MULTITENANT, [spec] * 2, T)
    assert mt < need
    pf = L.dc_apply_prefill
    assert pf(arr, 2, WB, X, seg.ctypes.data, 0x40000000, WS, mt - 1, None) == trs.DC_ERR_BUFFER


# Fake device addresses: the host checks reject these calls before any launch.
X, Y, WB, WS, IDS = 0x10000, 0x900000, 0x4000000, 0x8000000, 0xA000000


def _view(spec, base=0x200000):
    return trs._lib.dc_delta_view(trs.make_spec(spec), ctypes.c_void_p(base))


def test_apply_argument_checks(L):
    spec = (256, 256, 2, 8, 22)
    v = _view(spec)
    T = 4
    need = trs.dc_workspace_bytes(trs.DC_OP_DECODE, [spec], T)
    dec = L.dc_apply_decode
    assert dec(None, WB, X, Y, T, WS, need, None) == trs.DC_ERR_INVALID_ARG
    assert dec(ctypes.byref(v), WB, None, Y, T, WS, need, None) == trs.DC_ERR_INVALID_ARG
    assert dec(ctypes.byref(v), WB, X + 2, Y, T, WS, need, None) == trs.DC_ERR_ALIGN
    assert dec(ctypes.byref(v), WB, X, Y, T, WS + 16, need, None) == trs.DC_ERR_ALIGN
    assert dec(ctypes.byref(v), WB, X, Y, T, WS, need - 1, None) == trs.DC_ERR_BUFFER
    assert dec(ctypes.byref(v), WB, X, X + 64, T, WS, need, None) == trs.DC_ERR_INVALID_ARG  # overlap
    assert dec(ctypes.byref(v), WB, X, Y, -1, WS, need, None) == trs.DC_ERR_INVALID_ARG
    assert dec(ctypes.byref(v), WB, X, Y, 0, WS, need, None) == trs.DC_OK     # T = 0: no-op
    vb = _view(spec, 0x200008)
    assert dec(ctypes.byref(vb), WB, X, Y, T, WS, need, None) == trs.DC_ERR_ALIGN
    vs = _view((256, 200, 2, 8, 22))
    assert dec(ctypes.byref(vs), WB, X, Y, T, WS, need, None) == trs.DC_ERR_SHAPE
    vn = trs._lib.dc_delta_view(trs.make_spec(spec), None)
    assert dec(ctypes.byref(vn), WB, X, Y, T, WS, need, None) == trs.DC_ERR_INVALID_ARG


def test_multitenant_argument_checks(L):
    spec = (256, 256, 2, 8, 22)
    arr = (trs._lib.dc_delta_view * 3)(_view(spec), _view(spec), _view((256, 256, 1, 4, 9)))
    need = trs.dc_workspace_bytes(trs.DC_OP_MULTITENANT, [spec, spec, (256, 256, 1, 4, 9)], 8)
    mt = L.dc_apply_multitenant
    assert mt(arr, 3, WB, X, None, Y, 8, WS, need, None) == trs.DC_ERR_INVALID_ARG   # no ids
    assert mt(arr, 3, WB, X, IDS + 2, Y, 8, WS, need, None) == trs.DC_ERR_ALIGN
    assert mt(arr, 0, WB, X, IDS, Y, 8, WS, need, None) == trs.DC_ERR_INVALID_ARG
    assert mt(arr, 129, WB, X, IDS, Y, 8, WS, need, None) == trs.DC_ERR_UNSUPPORTED
    assert mt(arr, 3, WB, X, IDS, Y, 8, WS, need - 256, None) == trs.DC_ERR_BUFFER
    assert mt(arr, 3, WB, X, IDS, Y, 0, WS, need, None) == trs.DC_OK
    mixed = (trs._lib.dc_delta_view * 2)(_view(spec), _view((128, 256, 1, 1, 1)))
    assert mt(mixed, 2, WB, X, IDS, Y, 8, WS, need, None) == trs.DC_ERR_SHAPE
    pf = L.dc_apply_prefill
    seg = np.array([0, 3, 2, 8], np.int32)
    assert pf(arr, 3, WB, X, seg.ctypes.data, Y, WS, need, None) == trs.DC_ERR_INVALID_ARG
    seg = np.array([1, 3, 5, 8], np.int32)
    assert pf(arr, 3, WB, X, seg.ctypes.data, Y, WS, need, None) == trs.DC_ERR_INVALID_ARG
    seg = np.array([0, 0, 0, 0], np.int32)
    assert pf(arr, 3, WB, X, seg.ctypes.data, Y, WS, need, None) == trs.DC_OK     # T = 0


def test_dequant_argument_checks(L):
    v = _view((256, 256, 2, 8, 22))
    assert L.dc_dequant(ctypes.byref(v), None, X, None) == trs.DC_ERR_INVALID_ARG
    assert L.dc_dequant(ctypes.byref(v), X + 4, Y, None) == trs.DC_ERR_ALIGN
    e = _view((256, 256, 0, 0, 0))
    assert L.dc_dequant(ctypes.byref(e), None, None, None) == trs.DC_OK


def test_status_strings():
    assert trs.dc_status_string(trs.DC_ERR_RANGE) == "DC_ERR_RANGE"
    assert trs.dc_status_string(12345) == "DC_ERR_UNKNOWN"


def test_pack_device_argument_checks(L):
    """Every error of dc_pack_device is found on the host before anything is
    enqueued (fake device addresses, never dereferenced)."""
    spec = (256, 256, 2, 8, 22)
    s = trs.make_spec(spec)
    nb = trs.dc_packed_bytes(spec)
    U, G, V, OUT, FLAG = 0x300000, 0x310000, 0x320000, 0x400000, 0x500000
    pk = L.dc_pack_device
    assert pk(None, U, G, V, OUT, nb, FLAG, None) == trs.DC_ERR_INVALID_ARG
    assert pk(ctypes.byref(s), U, G, V, OUT, nb, None, None) == trs.DC_ERR_INVALID_ARG     # no flag
    assert pk(ctypes.byref(s), None, G, V, OUT, nb, FLAG, None) == trs.DC_ERR_INVALID_ARG
    assert pk(ctypes.byref(s), U, G, V, None, nb, FLAG, None) == trs.DC_ERR_INVALID_ARG
    assert pk(ctypes.byref(s), U + 4, G, V, OUT, nb, FLAG, None) == trs.DC_ERR_ALIGN       # U needs 8 B
    assert pk(ctypes.byref(s), U, G, V, OUT + 8, nb, FLAG, None) == trs.DC_ERR_ALIGN       # out needs 16 B
    assert pk(ctypes.byref(s), U, G, V, OUT, nb, FLAG + 2, None) == trs.DC_ERR_ALIGN
    assert pk(ctypes.byref(s), U, G, V, OUT, nb - 1, FLAG, None) == trs.DC_ERR_BUFFER
    bad = trs.make_spec((256, 200, 2, 8, 22))
    assert pk(ctypes.byref(bad), U, G, V, OUT, nb, FLAG, None) == trs.DC_ERR_SHAPE
    big = trs.make_spec((256, 256, 2, 8, 300))                                               # r > min(out, in)
    assert pk(ctypes.byref(big), U, G, V, OUT, nb, FLAG, None) == trs.DC_ERR_SHAPE


# ----------------------------------------------------------- bit allocation
def test_allocate_bits_matches_oracle():
    """dc_allocate_bits against the oracle's dynamic program: the same choice
    for every pair and the same total, bit for bit (same tie rules, same
    summation order), on random tables and on a 4096-pair table at the 1/16
    budget of a 4096 x 4096 matrix."""
    from oracle import alloc
    rng = np.random.default_rng(21)
    cost = [0, 2, 3, 8]
    for r, budget in ((1, 0), (7, 10), (50, 60), (200, 333)):
        err = np.sort(rng.random((r, 4)) * rng.choice([1.0, 1e3, 1e-3], (r, 1)), axis=1)[:, ::-1].copy()
        err[r // 2] = err[0]                       # tied rows
        ref_choice, ref_total = alloc.allocate_exact(err, cost, budget)
        choice, total = trs.dc_allocate_bits(err, cost, budget)
        assert np.array_equal(choice, ref_choice) and total == ref_total
    sigma = np.sort(rng.random(4096))[::-1] ** 4
    err = sigma[:, None] ** 2 * np.array([1.0, 0.1, 0.02, 1e-4])[None, :] * (1 + 0.1 * rng.random((4096, 4)))
    budget = 4096 * 4096 // 8192
    ref_choice, ref_total = alloc.allocate_exact(err, cost, budget)
    choice, total = trs.dc_allocate_bits(err, cost, budget)
    assert np.array_equal(choice, ref_choice) and total == ref_total


def test_allocate_bits_argument_checks(L):
    f = L.dc_allocate_bits
    err = np.ones((3, 2))
    cost = np.array([1, 2], np.int32)
    ch = np.zeros(3, np.int32)
    P = lambda a: a.ctypes.data
    assert f(3, 2, P(cost), P(err), 6, P(ch), None) == trs.DC_OK
    assert f(3, 2, None, P(err), 6, P(ch), None) == trs.DC_ERR_INVALID_ARG
    assert f(3, 0, P(cost), P(err), 6, P(ch), None) == trs.DC_ERR_INVALID_ARG
    assert f(-1, 2, P(cost), P(err), 6, P(ch), None) == trs.DC_ERR_INVALID_ARG
    assert f(3, 2, P(cost), P(err), -1, P(ch), None) == trs.DC_ERR_INVALID_ARG
    neg = np.array([1, -2], np.int32)
    assert f(3, 2, P(neg), P(err), 6, P(ch), None) == trs.DC_ERR_INVALID_ARG
    bad = err.copy()
    bad[1, 1] = np.nan
    assert f(3, 2, P(cost), P(bad), 6, P(ch), None) == trs.DC_ERR_INVALID_ARG
    assert f(3, 2, P(cost), P(err), 2, P(ch), None) == trs.DC_ERR_RANGE        # three rows of cost >= 1
    assert f(3000, 2, P(cost), P(np.ones((3000, 2))), 1 << 20, P(np.zeros(3000, np.int32)), None) == \
        trs.DC_ERR_UNSUPPORTED                                                  # 3000 x 2^20 choice bytes
    assert f(0, 2, P(cost), None, 0, None, None) == trs.DC_OK                  # no pairs


def test_group_workspace_and_argument_checks(L):
    """dc_group_workspace_bytes of one matrix is the multi-tenant size; a
    group holds each matrix's part once and the shared routing and staged x
    once; the group call rejects bad groups before any launch."""
    sq, sk = (512, 384, 2, 8, 22), (128, 384, 1, 3, 9)
    for T in (1, 40, 300):
        one = trs.dc_group_workspace_bytes([[sq] * 3], 1, T)
        assert one == trs.dc_workspace_bytes(trs.DC_OP_MULTITENANT, [sq] * 3, T)
        two = trs.dc_group_workspace_bytes([[sq] * 3, [sk] * 3], 2, T)
        k_alone = trs.dc_workspace_bytes(trs.DC_OP_MULTITENANT, [sk] * 3, T)
        assert max(one, k_alone) < two < one + k_alone
    assert trs.dc_group_workspace_bytes([[sq] * 3, [(128, 256, 1, 3, 9)] * 3], 2, 8) == 0   # different in
    flat = (trs._lib.dc_spec * 10)(*[trs.make_spec(sq)] * 10)
    assert L.dc_group_workspace_bytes(flat, 0, 2, 8) == 0
    assert L.dc_group_workspace_bytes(flat, 5, 2, 8) == 0
    need = trs.dc_group_workspace_bytes([[sq] * 2, [sk] * 2], 2, 8)
    arr = (trs._lib.dc_delta_view * 4)(_view(sq), _view(sq), _view(sk), _view(sk))
    P = ctypes.c_void_p
    W2 = (P * 2)(WB, None)
    grp = L.dc_apply_multitenant_group
    assert grp(arr, 2, 2, W2, X, IDS, (P * 2)(Y, Y + 0x100000), 8, WS, need - 1, None) == trs.DC_ERR_BUFFER
    assert grp(arr, 2, 2, W2, X, IDS, (P * 2)(Y, Y + 64), 8, WS, need, None) == trs.DC_ERR_INVALID_ARG  # y overlap
    assert grp(arr, 2, 2, W2, X, IDS, (P * 2)(Y, None), 8, WS, need, None) == trs.DC_ERR_INVALID_ARG
    assert grp(arr, 5, 2, W2, X, IDS, (P * 2)(Y, Y + 0x100000), 8, WS, need, None) == trs.DC_ERR_UNSUPPORTED
    assert grp(arr, 2, 2, W2, X, IDS, (P * 2)(Y, Y + 0x100000), 0, WS, need, None) == trs.DC_OK    # T = 0
    bad = (trs._lib.dc_delta_view * 4)(_view(sq), _view(sq), _view((128, 256, 1, 3, 9)), _view((128, 256, 1, 3, 9)))
    assert grp(bad, 2, 2, W2, X, IDS, (P * 2)(Y, Y + 0x100000), 8, WS, need, None) == trs.DC_ERR_SHAPE


def test_error_table_argument_checks(L):
    """dc_error_table rejects bad arguments on the host before any launch."""
    w = np.array([0, 2, 3, 8], np.int32)
    r, inn, ncal = 16, 256, 8
    need = trs.dc_error_table_workspace_bytes(r, inn, 4)
    assert need >= 4 * r * 4 * inn
    assert trs.dc_error_table_workspace_bytes(r, 200, 4) == 0
    assert trs.dc_error_table_workspace_bytes(r, inn, 9) == 0
    et = L.dc_error_table
    S, V, Xc, E, F = 0x100000, 0x200000, 0x300000, 0x400000, 0x500000
    wp = w.ctypes.data
    assert et(r, inn, ncal, S, V, Xc, wp, 4, E, F, WS, need - 1, None) == trs.DC_ERR_BUFFER
    assert et(r, 200, ncal, S, V, Xc, wp, 4, E, F, WS, need, None) == trs.DC_ERR_SHAPE
    assert et(r, inn, 0, S, V, Xc, wp, 4, E, F, WS, need, None) == trs.DC_ERR_INVALID_ARG
    assert et(r, inn, ncal, S, V, Xc, wp, 0, E, F, WS, need, None) == trs.DC_ERR_INVALID_ARG
    assert et(r, inn, ncal, S, V, Xc, wp, 9, E, F, WS, need, None) == trs.DC_ERR_INVALID_ARG
    bad = np.array([0, 9], np.int32)
    assert et(r, inn, ncal, S, V, Xc, bad.ctypes.data, 2, E, F, WS, need, None) == trs.DC_ERR_INVALID_ARG
    assert et(r, inn, ncal, None, V, Xc, wp, 4, E, F, WS, need, None) == trs.DC_ERR_INVALID_ARG
    assert et(r, inn, ncal, S, V, Xc, wp, 4, E, None, WS, need, None) == trs.DC_ERR_INVALID_ARG
    assert et(r, inn, ncal, S, V + 4, Xc, wp, 4, E, F, WS, need, None) == trs.DC_ERR_ALIGN
    assert et(r, inn, ncal, S, V, Xc, wp, 4, E + 4, F, WS, need, None) == trs.DC_ERR_ALIGN
    assert et(-1, inn, ncal, S, V, Xc, wp, 4, E, F, WS, need, None) == trs.DC_ERR_INVALID_ARG


def test_svd_argument_checks(L):
    """dc_svd rejects bad arguments on the host before any launch."""
    out, inn, r = 320, 200, 64
    need = trs.dc_svd_workspace_bytes(out, inn)
    mp = 256   # min(out, in) = 200 padded to a multiple of 64
    assert need >= 2 * mp * mp * 8
    assert trs.dc_svd_workspace_bytes(0, inn) == 0
    assert trs.dc_svd_workspace_bytes(20000, 20000) == 0
    sv = L.dc_svd
    D, U, S, V = 0x100000, 0x200000, 0x300000, 0x400000
    assert sv(out, inn, r, D, U, S, V, WS, need - 1, None, None) == trs.DC_ERR_BUFFER
    assert sv(0, inn, r, D, U, S, V, WS, need, None, None) == trs.DC_ERR_SHAPE
    assert sv(out, -1, r, D, U, S, V, WS, need, None, None) == trs.DC_ERR_SHAPE
    assert sv(out, inn, -1, D, U, S, V, WS, need, None, None) == trs.DC_ERR_INVALID_ARG
    assert sv(out, inn, inn + 1, D, U, S, V, WS, need, None, None) == trs.DC_ERR_INVALID_ARG
    assert sv(out, inn, r, None, U, S, V, WS, need, None, None) == trs.DC_ERR_INVALID_ARG
    assert sv(out, inn, r, D, None, S, V, WS, need, None, None) == trs.DC_ERR_INVALID_ARG
    assert sv(out, inn, r, D, U, S, V, None, need, None, None) == trs.DC_ERR_INVALID_ARG
    assert sv(out, inn, r, D + 2, U, S, V, WS, need, None, None) == trs.DC_ERR_ALIGN
    assert sv(out, inn, r, D, U, S, V, WS + 16, need, None, None) == trs.DC_ERR_ALIGN
    assert sv(20000, 20000, r, D, U, S, V, WS, need, None, None) == trs.DC_ERR_UNSUPPORTED
    # r = 0 writes nothing and launches nothing
    assert sv(out, inn, 0, D, None, None, None, WS, need, None, None) == trs.DC_OK
