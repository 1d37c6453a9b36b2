"""GPU parity of dc_svd (the on-device SVD of a delta, the first step of
compressing it) against the oracle's svd_pairs: singular values, both
vectors of every pair after the same sign rule, and the invariants the
factorization must keep (orthonormal rows, reconstruction)."""
import numpy as np
import pytest

import synth
import tenant_rank_serving_amd as trs
from oracle import quant
from gpu_util import note, torch

pytestmark = pytest.mark.gpu

# Tolerances.  The outputs are fp32 (about 6e-8 relative per entry).  The
# method's own error is far below that for these spectra: sigma_i is off by
# about 1e-16 sigma_1^2 / sigma_i^2 relative (the Gram matrix squares the
# condition; sigma_1 / sigma_m is at most 1024^0.8 = 256 here, so about 7e-12),
# a vector by that over its relative gap to the neighbouring values (0.8 / i
# for this profile, so at most about 1e-8 for i <= 1024).
SIG_RTOL = 1e-6
VEC_ATOL = 1e-5


def svd_gpu(delta, r):
    t = torch()
    out, inn = delta.shape
    d = t.from_numpy(np.ascontiguousarray(delta)).cuda()
    U = t.empty((r, out), dtype=t.float32, device="cuda")
    s = t.empty((r,), dtype=t.float32, device="cuda")
    V = t.empty((r, inn), dtype=t.float32, device="cuda")
    ws = t.empty(trs.dc_svd_workspace_bytes(out, inn), dtype=t.uint8, device="cuda")
    sweeps = trs.dc_svd(d, r, U, s, V, ws)
    return U.cpu().numpy(), s.cpu().numpy(), V.cpu().numpy(), sweeps


def check(delta, r, what, rows=None):
    U, s, V, sweeps = svd_gpu(delta, r)
    u0, s0, v0 = quant.svd_pairs(delta.astype(np.float64))
    rows = np.arange(r) if rows is None else rows
    srel = np.abs(s.astype(np.float64) - s0[:r]) / s0[:r]
    du = np.abs(U[rows].astype(np.float64) - u0[rows]).max()
    dv = np.abs(V[rows].astype(np.float64) - v0[rows]).max()
    print("[parity] svd %s: %d sweeps, sigma max rel %.2e, |du| %.2e, |dv| %.2e" % (what, sweeps, srel.max(), du, dv),
          flush=True)
    assert srel.max() <= SIG_RTOL
    assert du <= VEC_ATOL and dv <= VEC_ATOL
    assert np.all(np.diff(s) <= 0)
    return U, s, V


# (seed, out, in, r): out > in and out < in (the other Gram matrix), sizes
# that are not multiples of the 64-index padding, r below and at min(out, in)
CASES = [(0, 256, 192, 192), (1, 160, 384, 100), (2, 320, 200, 200), (3, 64, 64, 17), (4, 1024, 1024, 300),
         (5, 2048, 2048, 1002), (6, 1024, 2560, 512)]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%dx%d-r%d" % c[1:])
def test_svd_matches_oracle(case):
    seed, out, inn, r = case
    note("svd", case)
    delta = synth.spectral_delta(seed, out, inn)
    U, s, V = check(delta, r, "%dx%d r=%d" % (out, inn, r))
    # invariants of the GPU factors themselves
    assert np.abs(U @ U.T - np.eye(r)).max() <= 1e-5
    assert np.abs(V @ V.T - np.eye(r)).max() <= 1e-5
    if r == min(out, inn):
        rec = (U.T.astype(np.float64) * s) @ V.astype(np.float64)
        assert np.abs(rec - delta).max() <= 1e-5 * np.abs(delta).max()


def test_svd_rank_deficient():
    """A delta of rank 40 in 128 x 96: the 40 pairs match; the rest have sigma
    at the rounding level and (out >= in) a zero derived vector u when sigma
    is exactly 0, else unit vectors."""
    note("svd rank deficient")
    rng = np.random.default_rng(11)
    a = (rng.standard_normal((128, 40)) @ rng.standard_normal((40, 96))).astype(np.float32)
    U, s, V, _ = svd_gpu(a, 96)
    u0, s0, v0 = quant.svd_pairs(a.astype(np.float64))
    assert np.all(np.abs(s[:40] - s0[:40]) <= SIG_RTOL * s0[:40])
    assert np.abs(U[:40] - u0[:40]).max() <= VEC_ATOL and np.abs(V[:40] - v0[:40]).max() <= VEC_ATOL
    assert s[40:].max() <= 1e-5 * s[0]


def test_svd_rejects_nonfinite():
    note("svd non-finite")
    a = synth.spectral_delta(12, 96, 64)
    a[5, 7] = np.nan
    with pytest.raises(trs.DcError) as ei:
        svd_gpu(a, 8)
    assert ei.value.status == trs.DC_ERR_RANGE


def test_svd_feeds_the_device_packer():
    """dc_svd then dc_pack_device on the GPU, against the oracle's SVD then its
    quantizer and layout: the codes may differ where a value sits on a
    rounding boundary (the two SVDs differ in the last bits), so at least 99%
    of the packed bytes must equal the oracle's."""
    note("svd -> pack")
    t = torch()
    spec = (256, 256, 2, 8, 22)
    delta = synth.spectral_delta(13, 256, 256)
    r = sum(spec[2:])
    U, s, V, _ = svd_gpu(delta, r)
    buf = t.empty(trs.dc_packed_bytes(spec), dtype=t.uint8, device="cuda")
    flag = t.zeros(1, dtype=t.int32, device="cuda")
    trs.dc_pack_device(spec, t.from_numpy(U).cuda(), t.from_numpy(s).cuda(), t.from_numpy(V).cuda(), buf, flag)
    t.cuda.synchronize()
    assert int(flag.item()) == 0
    from oracle import layout
    u0, s0, v0 = quant.svd_pairs(delta.astype(np.float64))
    f32 = lambda a: a[:r].astype(np.float32)
    ref = layout.pack(spec, *quant.compress(f32(u0), f32(s0), f32(v0), *spec[2:]))
    got = buf.cpu().numpy()
    same = float(np.mean(got == ref))
    print("[parity] svd -> pack: %.4f of the packed bytes equal the oracle-SVD packing" % same, flush=True)
    assert same >= 0.99
