"""Seeded synthetic inputs for the Delta-CoMe delta-apply path.

This module only draws random numbers and rounds them to the storage dtypes
the path consumes (bf16 activations and backbone weights, fp16 scale/zero,
fp32 singular values, uint8 codes).  It holds none of the method's
arithmetic: no quantizer, no packing, no apply.  Both the CPU oracle and the
HIP path take their inputs from here, so neither has to trust the other's
inputs.

Workloads (shapes after the pages' 7B/13B Llama and Mistral models; the pages
name the backbones in "Delta-CoMe - what it is / technical principles" of the
paooo.com article and the experimental-setup list of the scime.ai summary):

  c0  one 256x256 fp32 delta built as U0.diag(s).V0^T (U0, V0 orthonormal by
      QR of Gaussians, s_i = i^-1.5); rank groups 2/8/22; bf16 base N(0,0.02);
      4 tokens x ~ N(0,1).
  c1  Llama-2-7B decoder layer (q,k,v,o 4096x4096; gate,up 11008x4096;
      down 4096x11008) at the 1/16 budget, one tenant, decode.
  c2  32 layers of c1 shapes x 50 tenant deltas, 64 tokens routed by
      Zipf(1.1) over the tenants.
  c3  13B layer (5120 hidden, 13824 MLP) at 1/16, 8 tenants x 2048 tokens.
  c4  Mistral-7B GQA layer at the 1/32 budget, 16 tenants, 128 tokens,
      uniform routing.

Codes are uniform over [0, 2^b-1]; scales are fp16 of a log-normal(-6, 0.5)
draw; zero points are uniform integers over [0, 2^b-1] stored in fp16;
singular values are s_i = 0.05 * i^-0.8.  Random streams: numpy
``default_rng`` seeded from ``SeedSequence(seed).spawn``; within one delta the
draw order is codes (V then U, segment by segment), V scales, U scales, V
zeros, U zeros.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Sequence, Tuple

import numpy as np

GROUP = 128

# ---------------------------------------------------------------------------
# Shapes.  (name, out, in) in nn.Linear orientation: W is [out][in].
# ---------------------------------------------------------------------------
LLAMA2_7B = (("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096),
             ("o", 4096, 4096), ("gate", 11008, 4096), ("up", 11008, 4096),
             ("down", 4096, 11008))
LLAMA2_13B = (("q", 5120, 5120), ("k", 5120, 5120), ("v", 5120, 5120),
              ("o", 5120, 5120), ("gate", 13824, 5120), ("up", 13824, 5120),
              ("down", 5120, 13824))
MISTRAL_7B = (("q", 4096, 4096), ("k", 1024, 4096), ("v", 1024, 4096),
              ("o", 4096, 4096), ("gate", 14336, 4096), ("up", 14336, 4096),
              ("down", 4096, 14336))

# Rank-group counts (n8, n3, n2) for each (out, in, budget).  These are data
# for the generator, not a rule: the tests check every entry against the
# oracle's budget rule.  budget 16 means 1/16 of the fp16 size (1 bit per
# parameter), 32 means 1/32.
RANK_GROUPS: Dict[Tuple[int, int, int], Tuple[int, int, int]] = {
    (4096, 4096, 16): (2, 32, 968),
    (11008, 4096, 16): (2, 47, 1414),
    (4096, 11008, 16): (2, 47, 1414),
    (5120, 5120, 16): (2, 40, 1212),
    (13824, 5120, 16): (2, 58, 1773),
    (5120, 13824, 16): (2, 58, 1773),
    (4096, 4096, 32): (2, 16, 480),
    (1024, 4096, 32): (2, 6, 187),
    (14336, 4096, 32): (2, 25, 750),
    (4096, 14336, 32): (2, 25, 750),
}
C0_GROUPS = (2, 8, 22)

# Pairs kept by the fp16 low-rank baseline at the same budgets (data for the
# generator; the tests check every entry against the oracle's budget rule).
LOWRANK_R: Dict[Tuple[int, int, int], int] = {
    (4096, 4096, 16): 128,
    (11008, 4096, 16): 186,
    (4096, 11008, 16): 186,
    (5120, 5120, 16): 160,
    (13824, 5120, 16): 233,
    (5120, 13824, 16): 233,
    (4096, 4096, 32): 64,
    (1024, 4096, 32): 25,
    (14336, 4096, 32): 99,
    (4096, 14336, 32): 99,
}


# ---------------------------------------------------------------------------
# dtype rounding of inputs (round-to-nearest-even), bit patterns as uint16
# ---------------------------------------------------------------------------
def to_bf16_bits(a) -> np.ndarray:
    """fp32 round-to-nearest-even to bfloat16; returns the uint16 bit patterns."""
    f = np.ascontiguousarray(np.asarray(a, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32)


def to_f16_bits(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float16)).view(np.uint16)


# ---------------------------------------------------------------------------
# Containers
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class DeltaCodes:
    """One tenant's compressed delta for one matrix, unpacked.

    codes_v  uint8 [r][in]    code of v_i at position j
    codes_u  uint8 [r][out]   code of u_i at position o
    sz_v     uint16 [r][in/128][2]   (fp16 scale bits, fp16 zero bits)
    sz_u     uint16 [r][out/128][2]
    sigma    float32 [r]
    ranks are ordered 8-bit segment, 3-bit segment, 2-bit segment.
    """
    out: int
    inn: int
    n8: int
    n3: int
    n2: int
    codes_v: np.ndarray
    codes_u: np.ndarray
    sz_v: np.ndarray
    sz_u: np.ndarray
    sigma: np.ndarray

    @property
    def r(self) -> int:
        return self.n8 + self.n3 + self.n2

    @property
    def spec(self) -> Tuple[int, int, int, int, int]:
        return (self.out, self.inn, self.n8, self.n3, self.n2)

    def bits(self) -> np.ndarray:
        return np.array([8] * self.n8 + [3] * self.n3 + [2] * self.n2, dtype=np.int64)

    def subset(self, lo: int, hi: int, spec) -> "DeltaCodes":
        """Ranks [lo, hi) re-labelled under another (n8, n3, n2) split."""
        n8, n3, n2 = spec
        assert n8 + n3 + n2 == hi - lo
        return DeltaCodes(self.out, self.inn, n8, n3, n2,
                          self.codes_v[lo:hi].copy(), self.codes_u[lo:hi].copy(),
                          self.sz_v[lo:hi].copy(), self.sz_u[lo:hi].copy(),
                          self.sigma[lo:hi].copy())


def sigma_profile(r: int) -> np.ndarray:
    i = np.arange(1, r + 1, dtype=np.float64)
    return (0.05 * i ** -0.8).astype(np.float32)


def spectral_delta(seed: int, out: int, inn: int) -> np.ndarray:
    """fp32 delta [out][in] = U0 diag(sigma) V0^T with orthonormal U0, V0
    (QR of Gaussian matrices) and sigma_i = 0.05 i^-0.8 over min(out, in)
    pairs: a few large singular values and a long tail, the spectrum shape the
    pages describe for fine-tuning deltas.  Draw order: U0, V0."""
    rng = np.random.default_rng(seed)
    m = min(out, inn)
    u0, _ = np.linalg.qr(rng.standard_normal((out, m)))
    v0, _ = np.linalg.qr(rng.standard_normal((inn, m)))
    s = sigma_profile(m).astype(np.float64)
    return ((u0 * s) @ v0.T).astype(np.float32)


def random_delta_codes(rng: np.random.Generator, out: int, inn: int,
                       n8: int, n3: int, n2: int) -> DeltaCodes:
    """Uniform codes, log-normal fp16 scales, uniform integer zeros."""
    assert out % GROUP == 0 and inn % GROUP == 0
    r = n8 + n3 + n2
    widths = [8] * n8 + [3] * n3 + [2] * n2
    codes_v = np.zeros((r, inn), np.uint8)
    codes_u = np.zeros((r, out), np.uint8)
    lo = 0
    for b, n in ((8, n8), (3, n3), (2, n2)):
        codes_v[lo:lo + n] = rng.integers(0, 1 << b, size=(n, inn), dtype=np.uint8)
        lo += n
    lo = 0
    for b, n in ((8, n8), (3, n3), (2, n2)):
        codes_u[lo:lo + n] = rng.integers(0, 1 << b, size=(n, out), dtype=np.uint8)
        lo += n
    gv, gu = inn // GROUP, out // GROUP
    sv = np.abs(rng.lognormal(-6.0, 0.5, size=(r, gv))).astype(np.float16)
    su = np.abs(rng.lognormal(-6.0, 0.5, size=(r, gu))).astype(np.float16)
    maxq = np.array([(1 << b) - 1 for b in widths], dtype=np.int64)
    zv = rng.integers(0, maxq[:, None] + 1, size=(r, gv)).astype(np.float16) if r else np.zeros((0, gv), np.float16)
    zu = rng.integers(0, maxq[:, None] + 1, size=(r, gu)).astype(np.float16) if r else np.zeros((0, gu), np.float16)
    sz_v = np.stack([sv.view(np.uint16), zv.view(np.uint16)], axis=-1)
    sz_u = np.stack([su.view(np.uint16), zu.view(np.uint16)], axis=-1)
    return DeltaCodes(out, inn, n8, n3, n2, codes_v, codes_u,
                      np.ascontiguousarray(sz_v), np.ascontiguousarray(sz_u),
                      sigma_profile(r))


def base_weight(rng: np.random.Generator, out: int, inn: int) -> np.ndarray:
    """bf16 bits of N(0, 0.02) [out][in]."""
    return to_bf16_bits(rng.normal(0.0, 0.02, size=(out, inn)).astype(np.float32))


def activations(rng: np.random.Generator, t: int, inn: int) -> np.ndarray:
    """bf16 bits of N(0, 1) [t][in]."""
    return to_bf16_bits(rng.standard_normal((t, inn)).astype(np.float32))


def zipf_ids(rng: np.random.Generator, n_tenants: int, t: int, s: float = 1.1) -> np.ndarray:
    p = np.arange(1, n_tenants + 1, dtype=np.float64) ** -s
    p /= p.sum()
    return rng.choice(n_tenants, size=t, p=p).astype(np.int32)


def _child(seed: int, *path: int) -> np.random.Generator:
    """Deterministic sub-stream for (seed, path...)."""
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=tuple(path)))


# ---------------------------------------------------------------------------
# c0: tiny end-to-end case
# ---------------------------------------------------------------------------
def make_c0(seed: int = 0) -> dict:
    rng = np.random.default_rng(seed)
    n = 256
    u0, _ = np.linalg.qr(rng.standard_normal((n, n)))
    v0, _ = np.linalg.qr(rng.standard_normal((n, n)))
    s = np.arange(1, n + 1, dtype=np.float64) ** -1.5
    delta = ((u0 * s) @ v0.T).astype(np.float32)
    w = base_weight(rng, n, n)
    x = activations(rng, 4, n)
    return dict(delta=delta, u0=u0, v0=v0, sigma=s, w=w, x=x,
                groups=C0_GROUPS, out=n, inn=n)


# ---------------------------------------------------------------------------
# c1..c4
# ---------------------------------------------------------------------------
def groups_for(out: int, inn: int, budget: int) -> Tuple[int, int, int]:
    return RANK_GROUPS[(out, inn, budget)]


def make_c1_matrix(mi: int, seed: int = 1, tokens: int = 64) -> dict:
    """Matrix mi (0..6 over LLAMA2_7B) of the c1 layer."""
    name, out, inn = LLAMA2_7B[mi]
    rng = _child(seed, mi)
    w = base_weight(rng, out, inn)
    d = random_delta_codes(rng, out, inn, *groups_for(out, inn, 16))
    x = activations(rng, tokens, inn)
    return dict(name=name, out=out, inn=inn, w=w, delta=d, x=x)


C2_LAYERS, C2_TENANTS, C2_TOKENS = 32, 50, 64


def c2_ids(seed: int = 2) -> np.ndarray:
    return zipf_ids(_child(seed, 0), C2_TENANTS, C2_TOKENS, 1.1)


def make_c2_base(layer: int, mi: int, seed: int = 2) -> np.ndarray:
    _, out, inn = LLAMA2_7B[mi]
    return base_weight(_child(seed, 1, layer, mi), out, inn)


def make_c2_delta(layer: int, mi: int, tenant: int, seed: int = 2) -> DeltaCodes:
    _, out, inn = LLAMA2_7B[mi]
    return random_delta_codes(_child(seed, 2, layer, mi, tenant), out, inn,
                              *groups_for(out, inn, 16))


def make_c2_x(layer: int, mi: int, seed: int = 2) -> np.ndarray:
    _, out, inn = LLAMA2_7B[mi]
    return activations(_child(seed, 3, layer, mi), C2_TOKENS, inn)


C3_TENANTS, C3_TOKENS_PER = 8, 2048


def make_c3_matrix(mi: int, seed: int = 3, tokens_per: int = C3_TOKENS_PER,
                   tenants: int = C3_TENANTS) -> dict:
    name, out, inn = LLAMA2_13B[mi]
    w = base_weight(_child(seed, 1, mi), out, inn)
    deltas = [random_delta_codes(_child(seed, 2, mi, k), out, inn, *groups_for(out, inn, 16))
              for k in range(tenants)]
    x = activations(_child(seed, 3, mi), tenants * tokens_per, inn)
    seg = np.arange(tenants + 1, dtype=np.int64) * tokens_per
    return dict(name=name, out=out, inn=inn, w=w, deltas=deltas, x=x, seg=seg)


C4_TENANTS, C4_TOKENS = 16, 128


def c4_ids(seed: int = 4) -> np.ndarray:
    return _child(seed, 0).integers(0, C4_TENANTS, size=C4_TOKENS).astype(np.int32)


def make_c4_matrix(mi: int, seed: int = 4, tenants: int = C4_TENANTS) -> dict:
    name, out, inn = MISTRAL_7B[mi]
    w = base_weight(_child(seed, 1, mi), out, inn)
    deltas = [random_delta_codes(_child(seed, 2, mi, k), out, inn, *groups_for(out, inn, 32))
              for k in range(tenants)]
    x = activations(_child(seed, 3, mi), C4_TOKENS, inn)
    return dict(name=name, out=out, inn=inn, w=w, deltas=deltas, x=x, ids=c4_ids(seed))


def small_delta(seed: int, out: int, inn: int, n8: int, n3: int, n2: int) -> DeltaCodes:
    """A random delta at any shape, for parity cases that span tiles and tails."""
    return random_delta_codes(np.random.default_rng(seed), out, inn, n8, n3, n2)


def small_case(seed: int, out: int, inn: int, n8: int, n3: int, n2: int,
               tokens: int) -> dict:
    rng = np.random.default_rng(seed)
    w = base_weight(rng, out, inn)
    d = random_delta_codes(rng, out, inn, n8, n3, n2)
    x = activations(rng, tokens, inn)
    return dict(out=out, inn=inn, w=w, delta=d, x=x)


def random_singular_pairs(seed: int, out: int, inn: int, r: int,
                          scale: float = 1.0) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """fp32 U [r][out], sigma [r] (descending), V [r][in] for quantizer tests."""
    rng = np.random.default_rng(seed)
    u = (rng.standard_normal((r, out)) * scale / np.sqrt(out)).astype(np.float32)
    v = (rng.standard_normal((r, inn)) * scale / np.sqrt(inn)).astype(np.float32)
    s = np.sort(np.abs(rng.standard_normal(r)))[::-1].astype(np.float32)
    return u, s, v


# ---------------------------------------------------------------------------
# the two baselines the pages compare with: fp16 low-rank pairs and 1-bit
# sign deltas with one scale per matrix
# ---------------------------------------------------------------------------
def random_lowrank(rng: np.random.Generator, out: int, inn: int, r: int):
    """fp16 U [r][out] and V [r][in] with N(0, 1/dim) entries (vectors of
    about unit norm), fp32 sigma_i = 0.05 i^-0.8.  Draw order: U, V."""
    u = (rng.standard_normal((r, out)) / np.sqrt(out)).astype(np.float16)
    v = (rng.standard_normal((r, inn)) / np.sqrt(inn)).astype(np.float16)
    return u, sigma_profile(r), v


def random_bitdelta(rng: np.random.Generator, out: int, inn: int):
    """Uniform sign bits uint8 [out][in] (1 = +1) and an fp32 scale drawn as
    |log-normal(-7, 0.5)| (about 1e-3, the size of a fine-tuning delta entry).
    Draw order: bits, scale."""
    bits = rng.integers(0, 2, size=(out, inn), dtype=np.uint8)
    alpha = np.float32(abs(rng.lognormal(-7.0, 0.5)))
    return bits, alpha


def lowrank_r(out: int, inn: int, budget: int) -> int:
    return LOWRANK_R[(out, inn, budget)]


def make_c1_lowrank(mi: int, seed: int = 1):
    _, out, inn = LLAMA2_7B[mi]
    return random_lowrank(_child(seed, mi, 7), out, inn, lowrank_r(out, inn, 16))


def make_c1_bitdelta(mi: int, seed: int = 1):
    _, out, inn = LLAMA2_7B[mi]
    return random_bitdelta(_child(seed, mi, 8), out, inn)
