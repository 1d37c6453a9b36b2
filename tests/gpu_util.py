"""Helpers for the GPU tests: upload packed deltas, run the C-ABI entry
points, compare with the oracle.  Inputs come from synth; expected values
from oracle/ only."""
import sys

import numpy as np

import synth
import tenant_rank_serving_amd as trs
from oracle import apply as oap

TOL = 2e-3   # per-token relative L2 of bf16 outputs against the fp64 oracle


def torch():
    import torch as _t
    return _t


def note(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev_u16(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def dev_i32(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def upload(spec, d: synth.DeltaCodes):
    buf = trs.dc_pack_codes(spec, d.codes_u, d.codes_v, d.sz_u, d.sz_v, d.sigma)
    t = torch()
    g = t.from_numpy(buf.copy()).cuda() if buf.size else t.zeros(256, dtype=t.uint8, device="cuda")
    return trs.DeltaView(spec, g)


def workspace(op, specs, T):
    t = torch()
    n = trs.dc_workspace_bytes(op, specs, T)
    assert n > 0
    return t.empty(n, dtype=t.uint8, device="cuda")


def y_to_f64(y):
    return synth.bf16_bits_to_f32(y.cpu().numpy().view(np.uint16)).astype(np.float64)


def oracle_tenant(d: synth.DeltaCodes, exact: bool = False):
    """(U, sigma, V) for the oracle: the fp16 dequantized values, or with
    `exact` the values the kernels multiply by: fp16 for 8-bit pairs, the
    exact grid values s*(q-z) for 3- and 2-bit pairs."""
    uh, vh = oap.dequant_pairs(d.codes_u, d.codes_v, d.sz_u, d.sz_v)
    if exact:
        ue, ve = oap.dequant_pairs(d.codes_u, d.codes_v, d.sz_u, d.sz_v, True)
        low = (d.bits() < 8)[:, None]
        uh = np.where(low, ue, uh.astype(np.float64))
        vh = np.where(low, ve, vh.astype(np.float64))
    return uh, d.sigma, vh


def run_decode(d, w, x, with_base=True):
    """Decode through dc_apply_decode; returns bf16 output as fp64 [T][out]."""
    t = torch()
    spec = d.spec
    view = upload(spec, d)
    T = x.shape[0]
    ws = workspace(trs.DC_OP_DECODE, [spec], T)
    xd = dev_u16(x)
    wd = dev_u16(w) if with_base else None
    y = t.empty((T, d.out), dtype=t.int16, device="cuda")
    trs.dc_apply_decode(view, wd, xd, y, ws)
    t.cuda.synchronize()
    return y_to_f64(y), y.cpu().numpy()


FMT_FLOOR = 1.5e-3   # bf16 rounding of the reference alone above this: a degenerate output
OWN_TOL = 1e-3       # then the kernel must sit this close to the rounded exact-product reference


def _round_bf16(a):
    return synth.bf16_bits_to_f32(synth.to_bf16_bits(np.asarray(a, np.float32))).astype(np.float64)


def check_close(y, ref, tol=TOL, what="", ref_exact=None):
    """Per token: relative L2 against the unrounded fp64 oracle <= tol.

    Exception, for outputs so degenerate that the bf16 format itself cannot
    meet the bar (e.g. one rank on 128 rows, where rounding errors repeat with
    the codes): if rounding the reference to bf16 already costs more than
    FMT_FLOOR, the token passes when it lies within OWN_TOL of the correctly
    rounded `ref_exact`, the oracle evaluated with the exact grid values
    s*(q-z) that the kernels multiply by (their fp16 roundings differ by up
    to 2^-11 relative per weight, which a rank-1 output does not average)."""
    rel = oap.rel_l2_per_token(y, ref)
    fmt = oap.rel_l2_per_token(_round_bf16(ref), ref)
    rx = ref if ref_exact is None else ref_exact
    own = oap.rel_l2_per_token(y, _round_bf16(rx))
    ok = (rel <= tol) | ((fmt > FMT_FLOOR) & (own <= OWN_TOL))
    bad = np.nonzero(~ok)[0]
    assert bad.size == 0, "%s: token %d rel L2 %.3g (bf16 floor %.3g, vs rounded ref %.3g) > %.3g" % (
        what, bad[0], rel[bad[0]], fmt[bad[0]], own[bad[0]], tol)
    return rel.max()
