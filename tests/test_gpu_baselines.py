"""GPU parity of the two baselines (fp16 low-rank, BitDelta) through the C
ABI against the oracle (oracle/baselines.py), on seeded synthetic inputs:
tiles, ragged input slices and rank tails, the backbone-only bucket, ids
out of range, the split and tiled backbone products, grouped calls and
repeatability."""
import numpy as np
import pytest

import synth
import tenant_rank_serving_amd as trs
from oracle import baselines as bl
from gpu_util import check_close, dev_i32, dev_u16, note, torch, y_to_f64

pytestmark = pytest.mark.gpu

LR, BD = trs.DC_KIND_LOWRANK, trs.DC_KIND_BITDELTA


def _dev_bytes(buf):
    t = torch()
    return t.from_numpy(buf.copy()).cuda() if buf.size else None


def _ws(views, m, T):
    t = torch()
    n = trs.dc_baseline_workspace_bytes(views, m, T)
    assert n > 0
    return t.empty(n, dtype=t.uint8, device="cuda")


def _ids(rng, n, T, extra=()):
    ids = rng.integers(-1, n, size=T).astype(np.int32)
    for i, v in extra:
        ids[i] = v
    return ids


def _run(views, w, x, ids, out, ws=None):
    t = torch()
    T = x.shape[0]
    ws = _ws(views, 1, T) if ws is None else ws
    y = t.empty((T, out), dtype=t.int16, device="cuda")
    trs.dc_apply_baseline_multitenant(views, dev_u16(w) if w is not None else None, dev_u16(x), dev_i32(ids), y, ws)
    t.cuda.synchronize()
    return y, ws


def _bd_case(seed, out, inn, n):
    rng = np.random.default_rng(seed)
    ts = [synth.random_bitdelta(rng, out, inn) for _ in range(n)]
    views = [trs.BaselineView(BD, out, inn, 0, _dev_bytes(trs.dc_pack_bitdelta(b, a))) for b, a in ts]
    return rng, ts, views


def _lr_case(seed, out, inn, rs):
    rng = np.random.default_rng(seed)
    ts = [synth.random_lowrank(rng, out, inn, r) for r in rs]
    views = [trs.BaselineView(LR, out, inn, r, _dev_bytes(trs.dc_pack_lowrank(*t_))) for r, t_ in zip(rs, ts)]
    return rng, ts, views


# (seed, out, in, tenants, T): slices of 16 input groups (2304: 16 + 2; 4224: 16 + 16 + 1),
# 128-row blocks, T = 1, a full C1/C2 shape, and T > 256 (tiled backbone product)
BD_CASES = [(0, 384, 2304, 3, 21), (1, 256, 256, 1, 1), (2, 128, 4224, 2, 40), (3, 4096, 4096, 4, 64),
            (4, 256, 384, 3, 300)]


@pytest.mark.parametrize("case", BD_CASES, ids=lambda c: "x".join(map(str, c[1:])))
def test_bitdelta_multitenant(case):
    seed, out, inn, n, T = case
    note("bitdelta", case)
    rng, ts, views = _bd_case(seed, out, inn, n)
    w = synth.base_weight(rng, out, inn)
    x = synth.activations(rng, T, inn)
    ids = _ids(rng, n, T, extra=[(0, 0)])
    for with_w in (True, False):
        y, _ = _run(views, w if with_w else None, x, ids, out)
        ref = bl.bitdelta_apply_multitenant(w if with_w else None, x, ids, ts)
        check_close(y_to_f64(y), ref, what="bitdelta %s %s" % ("fused" if with_w else "delta", case))


# (seed, out, in, ranks per tenant, T): V slices of 512 inputs (1152: 512 + 512 + 128, three partials
# added in order; 256 and 1024: one and two, atomics), rank tails (5, 37, 70), a tenant with r = 0,
# more than 256 ranks (two U windows), the C2 shapes 4096^2 (r 128) and 11008 x 4096 (r 186), and
# 4096 x 11008 (22 slices: more than one batch of 8 in the fixed-order sum)
LR_CASES = [(0, 384, 1152, (5, 37, 0), 21), (1, 256, 256, (70,), 9), (2, 128, 1024, (128, 16), 40),
            (3, 4096, 4096, (128, 128, 128, 128), 64), (4, 11008, 4096, (186, 186), 16),
            (5, 4096, 11008, (186,), 8), (6, 384, 512, (300,), 12), (7, 256, 384, (20, 33), 300)]


@pytest.mark.parametrize("case", LR_CASES, ids=lambda c: "%dx%d-r%s-T%d" % (c[1], c[2], "_".join(map(str, c[3])), c[4]))
def test_lowrank_multitenant(case):
    seed, out, inn, rs, T = case
    note("lowrank", case)
    rng, ts, views = _lr_case(seed, out, inn, rs)
    w = synth.base_weight(rng, out, inn)
    x = synth.activations(rng, T, inn)
    ids = _ids(rng, len(rs), T, extra=[(0, 0)])
    for with_w in (True, False):
        y, _ = _run(views, w if with_w else None, x, ids, out)
        ref = bl.lowrank_apply_multitenant(w if with_w else None, x, ids, ts)
        check_close(y_to_f64(y), ref, what="lowrank %s %s" % ("fused" if with_w else "delta", case))


def test_ids_out_of_range_are_flagged():
    note("baseline ids out of range")
    t = torch()
    for kind in (BD, LR):
        if kind == BD:
            rng, ts, views = _bd_case(10, 256, 384, 2)
            oracle = bl.bitdelta_apply_multitenant
        else:
            rng, ts, views = _lr_case(10, 256, 384, (24, 9))
            oracle = bl.lowrank_apply_multitenant
        w = synth.base_weight(rng, 256, 384)
        x = synth.activations(rng, 10, 384)
        ids = np.array([0, 1, 5, -1, 1, -7, 0, 2, 1, 0], np.int32)
        y, ws = _run(views, w, x, ids, 256)
        assert int(ws[:4].view(t.int32).item()) == 1
        served = np.where((ids >= 0) & (ids < 2), ids, -1)
        check_close(y_to_f64(y), oracle(w, x, served, ts), what="kind %d ids out of range" % kind)
        ok = np.array([0, 1, -1, 0], np.int32)
        _run(views, w, x[:4], ok, 256, ws)
        assert int(ws[:4].view(t.int32).item()) == 0


@pytest.mark.parametrize("kind", [BD, LR])
def test_repeatable_bits(kind):
    """Every sum is in a fixed order: repeated calls on a dirtied workspace
    give the same bits."""
    note("baseline repeatable", kind)
    t = torch()
    if kind == BD:
        rng, ts, views = _bd_case(11, 384, 4224, 3)
        inn = 4224
    else:
        rng, ts, views = _lr_case(11, 384, 2560, (130, 64, 7))
        inn = 2560
    w = synth.base_weight(rng, 384, inn)
    x = synth.activations(rng, 48, inn)
    ids = _ids(rng, 3, 48)
    y0, ws = _run(views, w, x, ids, 384)
    a = y0.clone()
    for _ in range(3):
        ws.random_(0, 255)
        y1, _ = _run(views, w, x, ids, 384, ws)
        assert t.equal(a, y1)


@pytest.mark.parametrize("kind", [BD, LR])
def test_group_matches_single_calls(kind):
    """A grouped call (q + k + v shape: outs 512, 128, 128) equals each
    matrix's single call bit for bit, with one matrix delta only."""
    note("baseline group", kind)
    t = torch()
    inn, T, n = 1152, 40, 3
    outs = (512, 128, 128)
    rng = np.random.default_rng(12)
    views, tss = [], []
    for j, out in enumerate(outs):
        if kind == BD:
            _, ts, vs = _bd_case(100 + j, out, inn, n)
        else:
            _, ts, vs = _lr_case(100 + j, out, inn, (40 + j, 17, 100))
        views.append(vs)
        tss.append(ts)
    ws_ = [synth.base_weight(rng, out, inn) for out in outs]
    x = synth.activations(rng, T, inn)
    ids = _ids(rng, n, T)
    Wd = [dev_u16(ws_[0]), None, dev_u16(ws_[2])]
    ys = [t.empty((T, out), dtype=t.int16, device="cuda") for out in outs]
    ws = _ws(views, len(outs), T)
    trs.dc_apply_baseline_multitenant_group(views, Wd, dev_u16(x), dev_i32(ids), ys, ws)
    t.cuda.synchronize()
    oracle = bl.bitdelta_apply_multitenant if kind == BD else bl.lowrank_apply_multitenant
    for j, out in enumerate(outs):
        y1, _ = _run(views[j], ws_[j] if Wd[j] is not None else None, x, ids, out)
        assert t.equal(ys[j], y1), "matrix %d" % j
        check_close(y_to_f64(ys[j]), oracle(ws_[j] if Wd[j] is not None else None, x, ids, tss[j]),
                    what="kind %d group matrix %d" % (kind, j))
