"""Pins of the oracle's packed format: golden words, hand-derived region
offsets and single-code placements, and pack/unpack round trips."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import synth
from oracle import layout
from conftest import read_golden


def _golden_words():
    for ln in read_golden("pack_words.txt"):
        bits, n, rule, words = [t.strip() for t in ln.split("|")]
        yield int(bits), int(n), rule, [int(w, 16) for w in words.split()]


@pytest.mark.parametrize("case", list(_golden_words()), ids=lambda c: "%db-%s" % (c[0], c[2]))
def test_bitstream_golden_words(case):
    bits, n, rule, words = case
    codes = np.array([eval(rule, {"k": k}) for k in range(n)], np.uint8)  # rules are tiny literals
    got = layout.bitstream(codes, bits)
    assert got.tolist() == words
    assert layout.unbitstream(got, bits, n).tolist() == codes.tolist()


def test_group_byte_sizes():
    # a 128-code group is 128, 48 and 32 bytes at 8, 3 and 2 bits
    for b, size in ((8, 128), (3, 48), (2, 32)):
        assert layout.bitstream(np.zeros(128, np.uint8), b).nbytes == size


GOLDEN_SPECS = {"layout_tiny.txt": (128, 128, 1, 1, 1), "layout_kblocks.txt": (128, 128, 0, 0, 40)}


@pytest.mark.parametrize("fixture", sorted(GOLDEN_SPECS))
def test_regions_golden(fixture):
    spec = GOLDEN_SPECS[fixture]
    reg = layout.regions(spec)
    for ln in read_golden(fixture):
        f = ln.split()
        if f[0] == "place":
            continue
        assert reg[f[0]] == (int(f[1]), int(f[2])), f[0]
    assert layout.packed_bytes(spec) == reg["END"][0]


@pytest.mark.parametrize("fixture", sorted(GOLDEN_SPECS))
def test_single_code_placements_golden(fixture):
    spec = GOLDEN_SPECS[fixture]
    out, inn, n8, n3, n2 = spec
    r = n8 + n3 + n2
    first = {8: 0, 3: n8, 2: n8 + n3}
    for ln in read_golden(fixture):
        f = ln.split()
        if f[0] != "place":
            continue
        side, b, pos, li, code = f[1], int(f[2]), int(f[3]), int(f[4]), int(f[5])
        off, word = int(f[6]), int(f[7], 16)
        cu = np.zeros((r, out), np.uint8)
        cv = np.zeros((r, inn), np.uint8)
        (cu if side == "U" else cv)[first[b] + li, pos] = code
        zu = np.zeros((r, out // 128, 2), np.uint16)
        zv = np.zeros((r, inn // 128, 2), np.uint16)
        buf = layout.pack(spec, cu, cv, zu, zv, np.zeros(r, np.float32))
        assert buf[off:off + 4].copy().view("<u4")[0] == word
        nz = np.nonzero(buf)[0]
        assert nz.min() >= off and nz.max() < off + 4   # nothing else was written


def test_algorithmic_bytes_c1():
    # codes 2*8+32*3+968*2 bits per (out+in) element pair; scale/zero 4 B per
    # group; sigma 4 B per rank
    assert layout.algorithmic_bytes((4096, 4096, 2, 32, 968)) == 2357672
    assert layout.algorithmic_bytes((11008, 4096, 2, 47, 1414)) == 6332068
    assert layout.algorithmic_bytes((4096, 4096, 2, 16, 480)) == 1178056


def _roundtrip(spec, seed):
    out, inn, n8, n3, n2 = spec
    d = synth.small_delta(seed, out, inn, n8, n3, n2)
    buf = layout.pack(spec, d.codes_u, d.codes_v, d.sz_u, d.sz_v, d.sigma)
    assert buf.size == layout.packed_bytes(spec)
    cu, cv, su, sv, sg = layout.unpack(spec, buf)
    assert np.array_equal(cu, d.codes_u) and np.array_equal(cv, d.codes_v)
    assert np.array_equal(su, d.sz_u) and np.array_equal(sv, d.sz_v)
    assert np.array_equal(sg.view(np.uint32), d.sigma.view(np.uint32))
    return buf


@pytest.mark.parametrize("spec", [(256, 256, 2, 8, 22), (128, 384, 0, 33, 0),
                                  (384, 128, 3, 0, 17), (128, 128, 0, 0, 0),
                                  (512, 256, 5, 31, 65)])
def test_pack_roundtrip(spec):
    _roundtrip(spec, 11)


@settings(max_examples=25, deadline=None)
@given(go=st.integers(1, 4), gi=st.integers(1, 4), n8=st.integers(0, 5),
       n3=st.integers(0, 40), n2=st.integers(0, 70), seed=st.integers(0, 2 ** 31))
def test_pack_roundtrip_hypothesis(go, gi, n8, n3, n2, seed):
    out, inn = 128 * go, 128 * gi
    if n8 + n3 + n2 > min(out, inn):
        return
    _roundtrip((out, inn, n8, n3, n2), seed)


def test_pad_codes_are_zero():
    """U ranks past n inside the last K-block and pad s/z entries are zero."""
    spec = (256, 128, 3, 5, 7)
    d = synth.small_delta(1, *spec)
    d.codes_u[:] = np.where(d.bits()[:, None] == 8, 255, np.where(d.bits()[:, None] == 3, 7, 3))
    buf = layout.pack(spec, d.codes_u, d.codes_v, d.sz_u, d.sz_v, d.sigma)
    reg = layout.regions(spec)
    off, size = reg["UC2"]
    words = buf[off:off + size].view("<u4").reshape(256 // 16, 16)   # one 1-word K-block per row
    assert np.all(words == (1 << 14) - 1)        # 7 codes of value 3: low 14 bits
    off, size = reg["UC3"]
    words = buf[off:off + size].view("<u4").reshape(256 // 16, 16)   # 5 ranks * 3 bits -> 1 word
    assert np.all(words == (1 << 15) - 1)
    off, size = reg["US3"]
    us = buf[off:off + size].view("<u4").reshape(2, 8)
    assert np.all(us[:, 5:] == 0) and np.all(us[:, :5] != 0)
    off, size = reg["UC8"]
    assert np.all(buf[off:off + size] == 255) and size == 256 * 3


def test_u_row_words():
    # full K-blocks take b words; the last keeps ceil(m*b/32)
    assert layout.u_row_words(968, 2) == 30 * 2 + 1
    assert layout.u_row_words(47, 3) == 3 + 2
    assert layout.u_row_words(32, 3) == 3
    assert layout.u_row_words(16, 3) == 2
    assert layout.u_row_words(1414, 2) == 44 * 2 + 1
    assert layout.u_row_words(0, 2) == 0
