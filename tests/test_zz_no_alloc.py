"""dc_apply_multitenant_noalloc (the library's own scratch array as the
workspace) against dc_apply_multitenant with a workspace of its own, through
the C ABI: two calls in a row, the second with a smaller input, each
bit-identical to the workspace call (the same kernels in the same order) and
within the oracle's bar; a call whose workspace would exceed the array is
rejected before anything is enqueued."""
import ctypes

import numpy as np
import pytest

import synth
import tenant_rank_serving_amd as trs
from gpu_util import check_multitenant, dev_i32, dev_u16, note, torch, upload, workspace, y_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    t = torch()
    if not t.cuda.is_available():
        pytest.skip("no GPU")
    trs.lib()


def _case(seed, out, inn, shapes, T):
    rng = np.random.default_rng(seed)
    specs = [(out, inn) + sh for sh in shapes]
    ds = [synth.small_delta(seed + 10 + k, *sp) for k, sp in enumerate(specs)]
    views = [upload(sp, d) for sp, d in zip(specs, ds)]
    w = synth.base_weight(rng, out, inn)
    x = synth.activations(rng, T, inn)
    ids = rng.integers(-1, len(specs), size=T).astype(np.int32)
    return specs, ds, views, w, x, ids


def test_noalloc_matches_workspace_call():
    t = torch()
    cases = [(_case(900, 512, 512, [(2, 8, 22), (1, 40, 100), (0, 0, 60)], 40), "first, 3 tenants 512x512 T=40"),
             (_case(950, 256, 384, [(2, 9, 40), (3, 0, 0)], 9), "second, 2 tenants 256x384 T=9")]
    for (specs, ds, views, w, x, ids), what in cases:
        note("noalloc", what)
        T = x.shape[0]
        for wb in (w, None):
            xd, idd = dev_u16(x), dev_i32(ids)
            wd = dev_u16(wb) if wb is not None else None
            y_ws = t.empty((T, specs[0][0]), dtype=t.int16, device="cuda")
            y_na = t.full((T, specs[0][0]), 0x7FC0, dtype=t.int16, device="cuda")   # NaN pattern: must be overwritten
            trs.dc_apply_multitenant(views, wd, xd, idd, y_ws, workspace(trs.DC_OP_MULTITENANT, specs, T))
            trs.dc_apply_multitenant_noalloc(views, wd, xd, idd, y_na)
            t.cuda.synchronize()
            assert t.equal(y_na, y_ws), what
            check_multitenant(y_to_f64(y_na), wb, x, ids, ds, specs[0][0],
                              "noalloc %s %s" % (what, "fused" if wb is not None else "delta"))


def test_noalloc_rejects_a_call_beyond_the_array():
    note("noalloc limit")
    spec = (4096, 4096, 2, 32, 968)
    T = 4096
    assert trs.dc_workspace_bytes(trs.DC_OP_MULTITENANT, [spec], T) > trs.DC_SCRATCH_BYTES
    v = trs._lib.dc_delta_view(trs.make_spec(spec), ctypes.c_void_p(0x200000))
    arr = (trs._lib.dc_delta_view * 1)(v)
    # fake device addresses: the host check rejects the call before any launch
    st = trs.lib().dc_apply_multitenant_noalloc(arr, 1, 0x4000000, 0x10000, 0xA000000, 0x40000000, T, None)
    assert st == trs.DC_ERR_UNSUPPORTED
