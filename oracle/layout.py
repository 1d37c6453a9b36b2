"""The packed delta format, reference pack/unpack (test infrastructure only).

The pages fix no storage layout ([P1] technical principles and [P2]
"Approach" only say that singular vectors are stored at 8, 3 or 2 bits).
This library's format fixes: b-bit codes packed little-endian into uint32
words, 3-bit codes 32 per 3 words, and an fp16 scale and zero per group of
128 elements.  The rest of the layout below is this library's choice, the
same definition that include/deltacome.h states.

One packed buffer holds one tenant's delta for one matrix, spec
(out, in, n8, n3, n2), r = n8+n3+n2, Gi = in/128, Go = out/128.  Ranks are
numbered globally 0..r-1 (8-bit segment, then 3-bit, then 2-bit); "local
rank" i is the index inside a segment of n = n_b ranks.

Bitstream rule: a run of codes c_0, c_1, ... at b bits occupies bits
[b*k, b*k+b) of a little-endian stream of uint32 words (bit t of the stream
is bit t%32 of word t//32).

Regions, in this order, each starting at a multiple of 256 bytes:
  SIGMA  fp32 [r]
  VC_8   V codes at 8 bits: for local rank i, for group g < Gi, the group's
         128 codes as one bitstream of 32 words.  [n][Gi][32] words.
  VC_b   (b = 3, 2)  V codes in 16-rank tiles: the group's 128 codes cut into
         4 chunks of 32 codes, each chunk one bitstream of b words; words
         [ceil(n/16)][Gi][4][16][b]: tile T, group g, chunk q, rank 16T+c of
         the tile (ranks past n are 0).
  VS_b   V scale/zero: uint32 [Gi][pad4(n)], entry (g, i) = fp16 scale bits
         | fp16 zero bits << 16 of v_i's group g; pad entries are 0.
  UC_8   U codes, 8-bit: bytes [out][n8], byte (o, i) = code of u_i at row o.
  UC_b   (b = 3, 2)  U codes packed along the rank axis: ranks cut into
         K-blocks of 32 (KB = ceil(n/32)); the K-block kb of row o is the
         bitstream of the codes of u_{32kb}..u_{32kb+31} at row o (codes past
         n are 0), b words long, except the last K-block, which keeps only
         wl = ceil(m*b/32) words for its m = n - 32(KB-1) ranks.  Rows go in
         16-row tiles; inside a tile, K-block by K-block, the 16 rows' words
         of one K-block are contiguous: a tile is [KB-1][16][b] words followed
         by [16][wl] words.
  US_b   U scale/zero: uint32 [Go][pad4(n)], entry (g, i) for u_i's group g
         (rows 128g..128g+127); pad entries 0.
Total size rounded up to 256 bytes.  Empty segments give empty regions.
"""
from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

GROUP = 128
ALIGN = 256
SEGS = (8, 3, 2)


def pad(n: int, m: int) -> int:
    return -(-n // m) * m


def _counts(spec) -> Dict[int, int]:
    _, _, n8, n3, n2 = spec
    return {8: n8, 3: n3, 2: n2}


def regions(spec) -> Dict[str, Tuple[int, int]]:
    """name -> (byte offset, byte size) for every region, in storage order."""
    out, inn, n8, n3, n2 = spec
    assert out % GROUP == 0 and inn % GROUP == 0
    cnt = _counts(spec)
    r = n8 + n3 + n2
    gi, go = inn // GROUP, out // GROUP
    sizes = [("SIGMA", 4 * r)]
    sizes += [("VC%d" % b, (cnt[b] if b == 8 else pad(cnt[b], 16)) * gi * 16 * b) for b in SEGS]
    sizes += [("VS%d" % b, gi * pad(cnt[b], 4) * 4) for b in SEGS]
    sizes += [("UC8", out * cnt[8])]
    sizes += [("UC%d" % b, (out // 16) * 16 * 4 * u_row_words(cnt[b], b)) for b in (3, 2)]
    sizes += [("US%d" % b, go * pad(cnt[b], 4) * 4) for b in SEGS]
    res = {}
    off = 0
    for name, size in sizes:
        off = pad(off, ALIGN)
        res[name] = (off, size)
        off += size
    res["END"] = (pad(off, ALIGN), 0)
    return res


def u_row_words(n: int, b: int) -> int:
    """Words one row of a 3- or 2-bit U segment of n ranks takes."""
    if n == 0:
        return 0
    kb = -(-n // 32)
    m = n - 32 * (kb - 1)
    return (kb - 1) * b + (-(-(m * b) // 32))


def packed_bytes(spec) -> int:
    return regions(spec)["END"][0]


def algorithmic_bytes(spec) -> int:
    """Bytes the kept pairs need with no padding: codes, fp16 scale+zero, fp32 sigma."""
    out, inn, n8, n3, n2 = spec
    r = n8 + n3 + n2
    codes = (8 * n8 + 3 * n3 + 2 * n2) * (out + inn) // 8
    return codes + r * (inn // GROUP + out // GROUP) * 4 + 4 * r


def bitstream(codes, b: int) -> np.ndarray:
    """Pack the last axis of `codes` (length a multiple of 32) at b bits."""
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.shape[-1]
    assert (n * b) % 32 == 0
    assert np.all(codes < (1 << b))
    bits = (codes[..., None] >> np.arange(b, dtype=np.uint8)) & 1      # [..., n, b]
    stream = bits.reshape(codes.shape[:-1] + (n * b,)).astype(np.uint8)
    by = np.packbits(stream, axis=-1, bitorder="little")             # [..., n*b/8]
    return np.ascontiguousarray(by).view("<u4")


def unbitstream(words, b: int, n: int) -> np.ndarray:
    """Inverse of bitstream: words [..., n*b/32] -> codes [..., n]."""
    w = np.ascontiguousarray(np.asarray(words, dtype="<u4"))
    by = w.view(np.uint8)
    stream = np.unpackbits(by, axis=-1, bitorder="little")[..., :n * b]
    bits = stream.reshape(w.shape[:-1] + (n, b)).astype(np.uint8)
    return (bits << np.arange(b, dtype=np.uint8)).sum(axis=-1).astype(np.uint8)


def _seg_ranges(spec):
    _, _, n8, n3, n2 = spec
    return {8: (0, n8), 3: (n8, n8 + n3), 2: (n8 + n3, n8 + n3 + n2)}


def _sz_words(sz) -> np.ndarray:
    sz = np.asarray(sz, dtype=np.uint32)
    return sz[..., 0] | (sz[..., 1] << 16)


def pack(spec, codes_u, codes_v, sz_u, sz_v, sigma) -> np.ndarray:
    """Build the packed buffer (uint8 array of packed_bytes(spec))."""
    out, inn, n8, n3, n2 = spec
    r = n8 + n3 + n2
    gi = inn // GROUP
    reg = regions(spec)
    buf = np.zeros(packed_bytes(spec), np.uint8)

    def put(name, arr):
        off, size = reg[name]
        raw = np.ascontiguousarray(arr).view(np.uint8).reshape(-1)
        assert raw.size == size, (name, raw.size, size)
        buf[off:off + size] = raw

    put("SIGMA", np.asarray(sigma, dtype="<f4")[:r])
    for b, (lo, hi) in _seg_ranges(spec).items():
        n = hi - lo
        cv = np.asarray(codes_v[lo:hi]).reshape(n, gi, GROUP)
        if b == 8:
            put("VC8", bitstream(cv, 8))
        else:
            nt = pad(n, 16) // 16
            cvp = np.zeros((nt * 16, gi, 4, 32), np.uint8)
            cvp[:n] = cv.reshape(n, gi, 4, 32)
            words = bitstream(cvp, b)                                  # [16T][Gi][4][b]
            words = words.reshape(nt, 16, gi, 4, b).transpose(0, 2, 3, 1, 4)   # [T][Gi][4][16][b]
            put("VC%d" % b, np.ascontiguousarray(words))
        vs = np.zeros((gi, pad(n, 4)), "<u4")
        vs[:, :n] = _sz_words(sz_v[lo:hi]).T
        put("VS%d" % b, vs)
        cu = np.asarray(codes_u[lo:hi]).T                     # [out][n]
        if b == 8:
            put("UC8", np.ascontiguousarray(cu))
        elif n:
            kb = -(-n // 32)
            wl = u_row_words(n, b) - (kb - 1) * b
            uc = np.zeros((out, kb * 32), np.uint8)
            uc[:, :n] = cu
            words = bitstream(uc.reshape(out // 16, 16, kb, 32), b)   # [T][16][KB][b]
            words = words.transpose(0, 2, 1, 3)                       # [T][KB][16][b]
            assert not words[:, kb - 1, :, wl:].any()                 # dropped words hold only pad zeros
            full = words[:, :kb - 1].reshape(out // 16, -1)
            last = np.ascontiguousarray(words[:, kb - 1, :, :wl]).reshape(out // 16, -1)
            put("UC%d" % b, np.concatenate([full, last], axis=1))
        us = np.zeros((out // GROUP, pad(n, 4)), "<u4")
        us[:, :n] = _sz_words(sz_u[lo:hi]).T
        put("US%d" % b, us)
    return buf


def unpack(spec, buf):
    """Inverse of pack: (codes_u, codes_v, sz_u, sz_v, sigma)."""
    out, inn, n8, n3, n2 = spec
    r = n8 + n3 + n2
    gi, go = inn // GROUP, out // GROUP
    reg = regions(spec)
    buf = np.asarray(buf, dtype=np.uint8)

    def get(name, dtype):
        off, size = reg[name]
        return buf[off:off + size].copy().view(dtype)

    sigma = get("SIGMA", "<f4")
    codes_u = np.zeros((r, out), np.uint8)
    codes_v = np.zeros((r, inn), np.uint8)
    sz_u = np.zeros((r, go, 2), np.uint16)
    sz_v = np.zeros((r, gi, 2), np.uint16)
    for b, (lo, hi) in _seg_ranges(spec).items():
        n = hi - lo
        if n == 0:
            continue
        if b == 8:
            words = get("VC8", "<u4").reshape(n, gi, 32)
            codes_v[lo:hi] = unbitstream(words, 8, GROUP).reshape(n, inn)
        else:
            nt = pad(n, 16) // 16
            words = get("VC%d" % b, "<u4").reshape(nt, gi, 4, 16, b).transpose(0, 3, 1, 2, 4)   # [T][16][Gi][4][b]
            codes = unbitstream(words.reshape(nt * 16, gi, 4, b), b, 32)                       # [16T][Gi][4][32]
            codes_v[lo:hi] = codes.reshape(nt * 16, inn)[:n]
        vs = get("VS%d" % b, "<u4").reshape(gi, pad(n, 4))[:, :n].T
        sz_v[lo:hi, :, 0] = vs & 0xFFFF
        sz_v[lo:hi, :, 1] = vs >> 16
        if b == 8:
            uc = get("UC8", np.uint8).reshape(out, n)
        else:
            kb = -(-n // 32)
            wl = u_row_words(n, b) - (kb - 1) * b
            tiles = get("UC%d" % b, "<u4").reshape(out // 16, -1)
            words = np.zeros((out // 16, kb, 16, b), "<u4")
            words[:, :kb - 1] = tiles[:, :(kb - 1) * 16 * b].reshape(out // 16, kb - 1, 16, b)
            words[:, kb - 1, :, :wl] = tiles[:, (kb - 1) * 16 * b:].reshape(out // 16, 16, wl)
            uc = unbitstream(words.transpose(0, 2, 1, 3), b, 32).reshape(out, kb * 32)[:, :n]
        codes_u[lo:hi] = uc.T
        us = get("US%d" % b, "<u4").reshape(go, pad(n, 4))[:, :n].T
        sz_u[lo:hi, :, 0] = us & 0xFFFF
        sz_u[lo:hi, :, 1] = us >> 16
    return codes_u, codes_v, sz_u, sz_v, sigma
