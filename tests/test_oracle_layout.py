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


def test_regions_tiny_golden():
    spec = (128, 128, 1, 1, 1)
    reg = layout.regions(spec)
    for ln in read_golden("layout_tiny.txt"):
        f = ln.split()
        if f[0] == "place":
            continue
        assert reg[f[0]] == (int(f[1]), int(f[2])), f[0]
    assert layout.packed_bytes(spec) == 5632


def test_single_code_placements_golden():
    spec = (128, 128, 1, 1, 1)
    seg_rank = {8: 0, 3: 1, 2: 2}
    for ln in read_golden("layout_tiny.txt"):
        f = ln.split()
        if f[0] != "place":
            continue
        side, b, pos, code, off, word = f[1], int(f[2]), int(f[3]), int(f[4]), int(f[5]), int(f[6], 16)
        cu = np.zeros((3, 128), np.uint8)
        cv = np.zeros((3, 128), np.uint8)
        (cu if side == "U" else cv)[seg_rank[b], pos] = code
        z = np.zeros((3, 1, 2), np.uint16)
        buf = layout.pack(spec, cu, cv, z, z, np.zeros(3, np.float32))
        assert buf[off:off + 4].view("<u4")[0] == word
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
    """U ranks past n inside the last K-block, pad s/z entries and pad bytes
    are zero."""
    spec = (256, 128, 3, 5, 7)
    d = synth.small_delta(1, *spec)
    d.codes_u[:] = np.where(d.bits()[:, None] == 8, 255, np.where(d.bits()[:, None] == 3, 7, 3))
    buf = layout.pack(spec, d.codes_u, d.codes_v, d.sz_u, d.sz_v, d.sigma)
    reg = layout.regions(spec)
    off, size = reg["UC2"]
    words = buf[off:off + size].view("<u4").reshape(256 // 16, 1, 16, 2)
    # 7 codes of value 3 -> low 14 bits set in word 0 of each row's K-block
    assert np.all(words[..., 0] == (1 << 14) - 1) and np.all(words[..., 1] == 0)
    off, size = reg["US3"]
    us = buf[off:off + size].view("<u4").reshape(2, 32)
    assert np.all(us[:, 5:] == 0)
    off, size = reg["UC8"]
    uc = buf[off:off + size].reshape(256, 4)
    assert np.all(uc[:, :3] == 255) and np.all(uc[:, 3] == 0)
