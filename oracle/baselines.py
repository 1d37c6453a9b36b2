"""The two delta-compression baselines the pages compare Delta-CoMe with, at
the same storage budget (test infrastructure only).

[P2] "Key results" and "Experimental setup" ("Baselines: Low-Rank SVD
compression, BitDelta"): at 1/16 compression Delta-CoMe is compared with a
low-rank delta and with BitDelta's 1-bit delta.  [P2] "Approach": Delta-CoMe
has the same size as BitDelta, i.e. 1 bit per delta parameter at 1/16.
[P3] "Delta-CoMe: 大型语言模型的无需训练的混合精度增量压缩" (its list of related
papers, the BitDelta entry): the delta of a fine-tuned model over its
pretrained weights is quantized to 1 bit.

Neither baseline's arithmetic is printed on the pages; the readings [R]:

  Low-rank: the top r singular pairs of the delta, vectors stored as fp16
    (the delta's original precision) and sigma as fp32, with r the largest
    count whose fp16 vectors fit the budget: 16 r (out + in) <= out in / rho
    bits, rho = 1 at 1/16 and 1/2 at 1/32 (the same accounting as the 8/3/2
    groups, which count code bits only).  Apply: y = W x + U (sigma * (V x))
    with the fp16 values.
  BitDelta: one bit per delta entry, its sign (an entry of 0 counts as +1),
    and one fp32 scale per matrix.  For fixed signs s the scale minimizing
    ||Delta - a s||_F is a = mean |Delta| (d/da of sum (|D| - a)^2 = 0), the
    training-free value; the page's method then calibrates it, which needs
    data and is out of scope.  Apply: y = W x + a S x, S the sign matrix
    (+1 / -1).

Storage layouts (this library's, restated by include/deltacome.h):
  Low-rank buffer: SIGMA fp32 [r], then V and U as fp16 in 16-row tiles of
    32-element steps, each region at a multiple of 256 bytes:
      V [ceil(r/16)][in/32][64][8]: v_i[k] sits in tile i/16, step k/32,
        slot (i % 16) + 16 ((k % 32) / 8), element k % 8;
      U [out/16][ceil(r/32)][64][8]: u_i[o] sits in tile o/16, step i/32,
        slot (o % 16) + 16 ((i % 32) / 8), element i % 8;
    ranks from r up to the tile edge hold zeros.
  BitDelta buffer: SCALE fp32 (one word, region padded to 256 bytes), then
    the sign bits in 16-row tiles, [out/16][in/128][4][16] words: word
    (T, g, c, i) holds the 32 entries of row 16T + i, columns
    128 g + 32 c + k, k < 32, bit b(k) = 1 meaning +1.  Inside the word the
    bits are interleaved by nibble so that word >> s & 0x11111111 holds 8
    entries one per nibble: entry k sits at bit 4 (k' % 8) + k' / 8 where
    k' = k / 2 for even k and 16 + k / 2 for odd k.
"""
from __future__ import annotations

import numpy as np

from . import quant

GROUP = 128
ALIGN = 256


def _pad(n: int, m: int) -> int:
    return -(-n // m) * m


# ------------------------------------------------------------------ low-rank
def lowrank_rank(out: int, inn: int, budget: int = 16) -> int:
    """Pairs of fp16 vectors within 1/budget of the fp16 delta: the largest r
    with 16 r (out + in) <= 16 out in / budget bits."""
    return (out * inn) // (budget * (out + inn))


def lowrank_compress(u, sigma, v, r: int):
    """The top r pairs (given in descending-sigma order) as fp16 vectors
    (round to nearest even from their values) and fp32 sigma.
    Returns (U fp16 [r][out], sigma fp32 [r], V fp16 [r][in])."""
    u = np.asarray(u)[:r]
    v = np.asarray(v)[:r]
    return (quant.fp16_rne(np.asarray(u, np.float64)), np.asarray(sigma[:r], np.float32),
            quant.fp16_rne(np.asarray(v, np.float64)))


def lowrank_regions(out: int, inn: int, r: int):
    """name -> (byte offset, byte size), and the total size."""
    res, off = {}, 0
    for name, size in (("SIGMA", 4 * r), ("V", 2 * _pad(r, 16) * inn), ("U", 2 * out * _pad(r, 32))):
        off = _pad(off, ALIGN)
        res[name] = (off, size)
        off += size
    return res, _pad(off, ALIGN)


def _tile(m, rows_pad: int, cols: int):
    """[rows][cols] -> [rows/16][cols/32][64][8] with slot (row % 16) + 16 ((col % 32) / 8)."""
    a = np.zeros((rows_pad, cols), m.dtype)
    a[:m.shape[0]] = m
    return a.reshape(rows_pad // 16, 16, cols // 32, 4, 8).transpose(0, 2, 3, 1, 4)


def _untile(t, rows: int, cols: int):
    return t.transpose(0, 3, 1, 2, 4).reshape(-1, cols)[:rows]


def lowrank_pack(U16, sigma, V16) -> np.ndarray:
    """U16 fp16 [r][out] (row i = u_i), sigma [r], V16 fp16 [r][in] (row i = v_i)."""
    U16, V16 = np.asarray(U16, np.float16), np.asarray(V16, np.float16)
    r, out = U16.shape
    inn = V16.shape[1]
    reg, total = lowrank_regions(out, inn, r)
    buf = np.zeros(total, np.uint8)
    ut = np.zeros((out, _pad(r, 32)), np.float16)
    ut[:, :r] = U16.T
    for name, arr in (("SIGMA", np.asarray(sigma, np.float32)), ("V", _tile(V16, _pad(r, 16), inn)),
                      ("U", _tile(ut, out, _pad(r, 32)))):
        o, n = reg[name]
        buf[o:o + n] = np.ascontiguousarray(arr).view(np.uint8).ravel()
    return buf


def lowrank_unpack(buf, out: int, inn: int, r: int):
    reg, _ = lowrank_regions(out, inn, r)
    b = np.asarray(buf, np.uint8)
    o, n = reg["SIGMA"]
    sg = b[o:o + n].view(np.float32).copy()
    o, n = reg["V"]
    V = _untile(b[o:o + n].view(np.float16).reshape(_pad(r, 16) // 16, inn // 32, 4, 16, 8), r, inn).copy()
    o, n = reg["U"]
    ut = _untile(b[o:o + n].view(np.float16).reshape(out // 16, _pad(r, 32) // 32, 4, 16, 8), out, _pad(r, 32))
    return np.ascontiguousarray(ut[:, :r].T), sg, V


# ------------------------------------------------------------------ BitDelta
def bitdelta_compress(delta):
    """Signs (1 for +1, 0 for -1; an entry of 0 counts as +1) and the
    L2-optimal scale for them, mean |delta| in fp64 rounded once to fp32."""
    d = np.asarray(delta, np.float64)
    bits = (d >= 0).astype(np.uint8)
    alpha = np.float32(np.mean(np.abs(d)))
    return bits, alpha


def signs(bits) -> np.ndarray:
    """The +1 / -1 matrix of sign bits."""
    return 2.0 * np.asarray(bits, np.float64) - 1.0


def nibble_position(k: int) -> int:
    """Bit of a BitDelta word that holds entry k (0..31) of its 32."""
    kp = k // 2 if k % 2 == 0 else 16 + k // 2
    return 4 * (kp % 8) + kp // 8


def bitdelta_bytes(out: int, inn: int) -> int:
    return ALIGN + out * inn // 8


def bitdelta_pack(bits, alpha) -> np.ndarray:
    bits = np.asarray(bits, np.uint8)
    out, inn = bits.shape
    assert out % 16 == 0 and inn % GROUP == 0
    words = np.zeros((out // 16, inn // GROUP, 4, 16), np.uint32)
    for k in range(32):
        col = bits.reshape(out // 16, 16, inn // GROUP, 4, 32)[..., k]   # [T][i][g][c]
        words |= np.transpose(col, (0, 2, 3, 1)).astype(np.uint32) << np.uint32(nibble_position(k))
    buf = np.zeros(bitdelta_bytes(out, inn), np.uint8)
    buf[:4] = np.array([alpha], np.float32).view(np.uint8)
    buf[ALIGN:] = words.view(np.uint8).ravel()
    return buf


def bitdelta_unpack(buf, out: int, inn: int):
    b = np.asarray(buf, np.uint8)
    alpha = b[:4].view(np.float32)[0]
    words = b[ALIGN:ALIGN + out * inn // 8].view(np.uint32).reshape(out // 16, inn // GROUP, 4, 16)
    bits = np.zeros((out // 16, 16, inn // GROUP, 4, 32), np.uint8)
    for k in range(32):
        bits[..., k] = np.transpose((words >> np.uint32(nibble_position(k))) & 1, (0, 3, 1, 2))
    return bits.reshape(out, inn), np.float32(alpha)


def bitdelta_apply(w_bits, x_bits, bits, alpha) -> np.ndarray:
    """y[t] = W x_t + alpha S x_t in fp64 (W None: delta only)."""
    from .apply import bf16_to_f64
    x = bf16_to_f64(x_bits)
    y = x @ (alpha * signs(bits)).T
    if w_bits is not None:
        y += x @ bf16_to_f64(w_bits).T
    return y


def bitdelta_apply_multitenant(w_bits, x_bits, ids, tenants) -> np.ndarray:
    """tenants: list of (bits, alpha); ids outside [0, n): backbone only."""
    from .apply import bf16_to_f64
    ids = np.asarray(ids)
    x = bf16_to_f64(x_bits)
    out = np.asarray(tenants[0][0]).shape[0]
    y = np.zeros((x.shape[0], out)) if w_bits is None else x @ bf16_to_f64(w_bits).T
    for k, (bits, alpha) in enumerate(tenants):
        sel = np.nonzero(ids == k)[0]
        if sel.size:
            y[sel] += x[sel] @ (float(alpha) * signs(bits)).T
    return y


def lowrank_apply_multitenant(w_bits, x_bits, ids, tenants) -> np.ndarray:
    """tenants: list of (U16 [r][out], sigma [r], V16 [r][in]); ids outside
    [0, n): backbone only.  Each token: y = W x + U (sigma * (V x)) in fp64."""
    from .apply import apply_factored, bf16_to_f64
    ids = np.asarray(ids)
    x = bf16_to_f64(x_bits)
    out = np.asarray(tenants[0][0]).shape[1]
    y = np.zeros((x.shape[0], out)) if w_bits is None else x @ bf16_to_f64(w_bits).T
    for k, (U16, sg, V16) in enumerate(tenants):
        sel = np.nonzero(ids == k)[0]
        if sel.size:
            y[sel] += apply_factored(None, np.asarray(x_bits)[sel], U16, sg, V16)
    return y
