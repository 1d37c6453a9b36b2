"""Serving side of Delta-CoMe in fp64 (test infrastructure only).

Many fine-tuned models share one backbone; each is served as the backbone
plus its own compressed delta ([P1] application scenarios, multi-tenant
serving; [P2] "Key results", 50 models on one GPU; [P2] "Problem").  For a
token x routed to tenant k the output is the plain definition

    y = (W_base + U_k diag(sigma_k) V_k) x

with U_k, V_k the dequantized fp16 singular vectors.  The factored form
W x + U (sigma * (V x)) reaches the same value (associativity) and is what
the oracle evaluates; `brute_force` evaluates the definition term by term.
"""
from __future__ import annotations

import numpy as np

from . import layout, quant


def bf16_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64, exact."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f16_to_f64(h) -> np.ndarray:
    return np.asarray(h, dtype=np.float16).astype(np.float64)


def apply_factored(w_bits, x_bits, u_hat, sigma, v_hat) -> np.ndarray:
    """y[t] = W x_t + sum_i u_i sigma_i (v_i . x_t), fp64.

    w_bits bf16 [out][in] or None (delta only); x_bits bf16 [T][in];
    u_hat [r][out], v_hat [r][in] (fp16 or any float); sigma [r].
    Returns fp64 [T][out].
    """
    x = bf16_to_f64(x_bits)
    u = np.asarray(u_hat, dtype=np.float64)
    v = np.asarray(v_hat, dtype=np.float64)
    s = np.asarray(sigma, dtype=np.float64)
    out = u.shape[1]
    y = np.zeros((x.shape[0], out))
    if w_bits is not None:
        y += x @ bf16_to_f64(w_bits).T
    if s.shape[0]:
        t = (x @ v.T) * s            # [T][r]
        y += t @ u
    return y


def brute_force(w_bits, x_bits, u_hat, sigma, v_hat) -> np.ndarray:
    """The definition y_o = sum_j (W_oj + sum_i u_i[o] sigma_i v_i[j]) x_j, in
    pure-Python loops over o, j and i.  For tiny shapes only."""
    x = bf16_to_f64(x_bits).tolist()
    u = np.asarray(u_hat, dtype=np.float64).tolist()
    v = np.asarray(v_hat, dtype=np.float64).tolist()
    s = np.asarray(sigma, dtype=np.float64).tolist()
    w = None if w_bits is None else bf16_to_f64(w_bits).tolist()
    r = len(s)
    out = len(u[0]) if r else len(w)
    inn = len(x[0])
    y = []
    for xt in x:
        row = []
        for o in range(out):
            acc = 0.0
            for j in range(inn):
                m = w[o][j] if w is not None else 0.0
                for i in range(r):
                    m += u[i][o] * s[i] * v[i][j]
                acc += m * xt[j]
            row.append(acc)
        y.append(row)
    return np.array(y)


def dequant_pairs(codes_u, codes_v, sz_u, sz_v, exact: bool = False):
    """fp16 singular vectors from codes and (scale, zero) bit patterns (or
    the exact fp64 grid values s*(q-z) if `exact`)."""
    return quant.dequant_all(codes_u, sz_u, exact), quant.dequant_all(codes_v, sz_v, exact)


def apply_codes(w_bits, x_bits, codes_u, codes_v, sz_u, sz_v, sigma) -> np.ndarray:
    u_hat, v_hat = dequant_pairs(codes_u, codes_v, sz_u, sz_v)
    return apply_factored(w_bits, x_bits, u_hat, sigma, v_hat)


def apply_packed(spec, buf, w_bits, x_bits) -> np.ndarray:
    """Unpack, dequantize to the fp16 values, then the fp64 factored apply."""
    cu, cv, su, sv, sg = layout.unpack(spec, buf)
    return apply_codes(w_bits, x_bits, cu, cv, su, sv, sg)


def apply_multitenant(w_bits, x_bits, ids, tenants) -> np.ndarray:
    """Decode batch over many tenants sharing one backbone.

    tenants: list of (u_hat, sigma, v_hat) per tenant id 0..n-1.  Token t is
    served by tenant ids[t]; an id outside [0, n) means backbone only (the
    delta is skipped).  Token by token, in plain loops over tenants.
    """
    ids = np.asarray(ids)
    x = np.asarray(x_bits)
    out = bf16_to_f64(w_bits).shape[0] if w_bits is not None else np.asarray(tenants[0][0]).shape[1]
    y = np.zeros((x.shape[0], out))
    if w_bits is not None:
        y += bf16_to_f64(x) @ bf16_to_f64(w_bits).T
    for k, (u_hat, sigma, v_hat) in enumerate(tenants):
        sel = np.nonzero(ids == k)[0]
        if sel.size:
            y[sel] += apply_factored(None, x[sel], u_hat, sigma, v_hat)
    return y


def apply_prefill(w_bits, x_bits, seg, tenants) -> np.ndarray:
    """Tokens seg[k]..seg[k+1]-1 belong to tenant k (contiguous segments)."""
    seg = np.asarray(seg)
    ids = np.full(np.asarray(x_bits).shape[0], -1, np.int64)
    for k in range(len(tenants)):
        ids[seg[k]:seg[k + 1]] = k
    return apply_multitenant(w_bits, x_bits, ids, tenants)


def rel_l2_per_token(y, y_ref) -> np.ndarray:
    """||y_t - ref_t||_2 / ||ref_t||_2 for each token t."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    num = np.sqrt(((y - y_ref) ** 2).sum(axis=-1))
    den = np.sqrt((y_ref ** 2).sum(axis=-1))
    return num / np.where(den == 0, 1.0, den)
