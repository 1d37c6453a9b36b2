"""ctypes binding of libdeltacome.so.  Argument marshalling only: every step
of the apply runs in the library's HIP kernels.  Device buffers are torch
tensors (memory and streams only); host buffers are numpy arrays.

There is no fallback: if the library is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence, Tuple

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdeltacome.so")

DC_OK = 0
DC_ERR_INVALID_ARG = -1
DC_ERR_SHAPE = -2
DC_ERR_ALIGN = -3
DC_ERR_BUFFER = -4
DC_ERR_RANGE = -5
DC_ERR_HIP = -6
DC_ERR_UNSUPPORTED = -7
DC_MAX_TENANTS = 128
DC_SCRATCH_BYTES = 32 << 20
DC_MAX_GROUP = 4
DC_OP_DECODE, DC_OP_MULTITENANT, DC_OP_PREFILL = 0, 1, 2
REGIONS = ("SIGMA", "VC8", "VC3", "VC2", "VS8", "VS3", "VS2",
           "UC8", "UC3", "UC2", "US8", "US3", "US2")
EXPORTS = ("dc_status_string", "dc_check_spec", "dc_packed_bytes", "dc_algorithmic_bytes",
           "dc_region", "dc_pack", "dc_pack_codes", "dc_unpack", "dc_workspace_bytes",
           "dc_apply_decode", "dc_apply_multitenant", "dc_apply_multitenant_timed",
           "dc_apply_prefill", "dc_dequant", "dc_pack_device", "dc_allocate_bits",
           "dc_apply_multitenant_noalloc", "dc_apply_multitenant_group", "dc_group_workspace_bytes",
           "dc_apply_multitenant_group_timed", "dc_baseline_bytes", "dc_baseline_algorithmic_bytes",
           "dc_pack_lowrank", "dc_pack_bitdelta", "dc_baseline_workspace_bytes",
           "dc_apply_baseline_multitenant", "dc_apply_baseline_multitenant_group",
           "dc_error_table_workspace_bytes", "dc_error_table", "dc_svd_workspace_bytes", "dc_svd")
DC_ERR_MAX_WIDTHS = 8
DC_KIND_LOWRANK, DC_KIND_BITDELTA = 1, 2
_SIZE_FNS = ("dc_status_string", "dc_packed_bytes", "dc_algorithmic_bytes", "dc_workspace_bytes",
             "dc_group_workspace_bytes", "dc_baseline_bytes", "dc_baseline_algorithmic_bytes",
             "dc_baseline_workspace_bytes", "dc_error_table_workspace_bytes", "dc_svd_workspace_bytes")
STAGES = ("route", "xprep", "base", "vside", "uside")


class DcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (%d)" % (where, _status_name(status), status))


class dc_spec(ctypes.Structure):
    _fields_ = [("out", ctypes.c_int32), ("in_", ctypes.c_int32), ("n8", ctypes.c_int32),
                ("n3", ctypes.c_int32), ("n2", ctypes.c_int32)]


class dc_delta_view(ctypes.Structure):
    _fields_ = [("spec", dc_spec), ("base", ctypes.c_void_p)]


class dc_baseline_view(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("out", ctypes.c_int32), ("in_", ctypes.c_int32),
                ("r", ctypes.c_int32), ("base", ctypes.c_void_p)]


_P = ctypes.c_void_p
_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libdeltacome.so is not built (python -m tenant_rank_serving_amd.build)")
        # torch first: its HIP runtime (libamdhip64.so.7, bundled with torch)
        # is then the one the library binds to.  Loaded the other way round,
        # the process holds two HIP runtimes and the library's finds no
        # device ("no ROCm-capable device is detected").
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        sp = ctypes.POINTER(dc_spec)
        vp = ctypes.POINTER(dc_delta_view)
        L.dc_status_string.restype = ctypes.c_char_p
        L.dc_status_string.argtypes = [ctypes.c_int32]
        L.dc_check_spec.argtypes = [sp]
        L.dc_packed_bytes.restype = ctypes.c_size_t
        L.dc_packed_bytes.argtypes = [sp]
        L.dc_algorithmic_bytes.restype = ctypes.c_size_t
        L.dc_algorithmic_bytes.argtypes = [sp]
        L.dc_region.argtypes = [sp, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t),
                                ctypes.POINTER(ctypes.c_size_t)]
        L.dc_pack.argtypes = [sp, _P, _P, _P, _P, ctypes.c_size_t]
        L.dc_pack_codes.argtypes = [sp, _P, _P, _P, _P, _P, _P, ctypes.c_size_t]
        L.dc_unpack.argtypes = [sp, _P, ctypes.c_size_t, _P, _P, _P, _P, _P]
        L.dc_workspace_bytes.restype = ctypes.c_size_t
        L.dc_workspace_bytes.argtypes = [ctypes.c_int32, sp, ctypes.c_int32, ctypes.c_int32]
        L.dc_apply_decode.argtypes = [vp, _P, _P, _P, ctypes.c_int32, _P, ctypes.c_size_t, _P]
        L.dc_apply_multitenant.argtypes = [vp, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32, _P,
                                           ctypes.c_size_t, _P]
        L.dc_apply_multitenant_timed.argtypes = [vp, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32,
                                                 _P, ctypes.c_size_t, _P, ctypes.POINTER(_P)]
        L.dc_apply_prefill.argtypes = [vp, ctypes.c_int32, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
        L.dc_apply_multitenant_noalloc.argtypes = [vp, ctypes.c_int32, _P, _P, _P, _P, ctypes.c_int32, _P]
        L.dc_apply_multitenant_group.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P,
                                                 ctypes.c_int32, _P, ctypes.c_size_t, _P]
        L.dc_apply_multitenant_group_timed.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, _P, _P, _P, _P,
                                                       ctypes.c_int32, _P, ctypes.c_size_t, _P, ctypes.POINTER(_P)]
        L.dc_group_workspace_bytes.restype = ctypes.c_size_t
        L.dc_group_workspace_bytes.argtypes = [sp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        L.dc_dequant.argtypes = [vp, _P, _P, _P]
        L.dc_pack_device.argtypes = [sp, _P, _P, _P, _P, ctypes.c_size_t, _P, _P]
        L.dc_allocate_bits.argtypes = [ctypes.c_int32, ctypes.c_int32, _P, _P, ctypes.c_int64, _P, _P]
        bp = ctypes.POINTER(dc_baseline_view)
        i32 = ctypes.c_int32
        L.dc_baseline_bytes.restype = ctypes.c_size_t
        L.dc_baseline_bytes.argtypes = [i32, i32, i32, i32]
        L.dc_baseline_algorithmic_bytes.restype = ctypes.c_size_t
        L.dc_baseline_algorithmic_bytes.argtypes = [i32, i32, i32, i32]
        L.dc_pack_lowrank.argtypes = [i32, i32, i32, _P, _P, _P, _P, ctypes.c_size_t]
        L.dc_pack_bitdelta.argtypes = [i32, i32, _P, ctypes.c_float, _P, ctypes.c_size_t]
        L.dc_baseline_workspace_bytes.restype = ctypes.c_size_t
        L.dc_baseline_workspace_bytes.argtypes = [bp, i32, i32, i32]
        L.dc_apply_baseline_multitenant.argtypes = [bp, i32, _P, _P, _P, _P, i32, _P, ctypes.c_size_t, _P]
        L.dc_apply_baseline_multitenant_group.argtypes = [bp, i32, i32, _P, _P, _P, _P, i32, _P,
                                                          ctypes.c_size_t, _P]
        L.dc_error_table_workspace_bytes.restype = ctypes.c_size_t
        L.dc_error_table_workspace_bytes.argtypes = [i32, i32, i32]
        L.dc_error_table.argtypes = [i32, i32, i32, _P, _P, _P, _P, i32, _P, _P, _P, ctypes.c_size_t, _P]
        L.dc_svd_workspace_bytes.restype = ctypes.c_size_t
        L.dc_svd_workspace_bytes.argtypes = [i32, i32]
        L.dc_svd.argtypes = [i32, i32, i32, _P, _P, _P, _P, _P, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int32), _P]
        for name in EXPORTS:
            if name not in _SIZE_FNS:
                getattr(L, name).restype = ctypes.c_int32
        _lib = L
    return _lib


def _status_name(s: int) -> str:
    try:
        return lib().dc_status_string(int(s)).decode()
    except ImportError:
        return str(s)


def _check(status: int, where: str) -> None:
    if status != DC_OK:
        raise DcError(status, where)


def make_spec(spec) -> dc_spec:
    if isinstance(spec, dc_spec):
        return spec
    out, inn, n8, n3, n2 = (int(v) for v in spec)
    return dc_spec(out, inn, n8, n3, n2)


def _np_ptr(a, dtype) -> Tuple[np.ndarray, int]:
    arr = np.ascontiguousarray(a, dtype=dtype)
    return arr, arr.ctypes.data


# ------------------------------------------------------------------- host
def dc_status_string(status: int) -> str:
    return lib().dc_status_string(int(status)).decode()


def dc_check_spec(spec) -> int:
    return int(lib().dc_check_spec(ctypes.byref(make_spec(spec))))


def dc_packed_bytes(spec) -> int:
    return int(lib().dc_packed_bytes(ctypes.byref(make_spec(spec))))


def dc_algorithmic_bytes(spec) -> int:
    return int(lib().dc_algorithmic_bytes(ctypes.byref(make_spec(spec))))


def dc_region(spec, region) -> Tuple[int, int]:
    rid = REGIONS.index(region) if isinstance(region, str) else int(region)
    off, size = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().dc_region(ctypes.byref(make_spec(spec)), rid, ctypes.byref(off), ctypes.byref(size)),
           "dc_region")
    return off.value, size.value


def dc_pack(spec, U, sigma, V) -> np.ndarray:
    s = make_spec(spec)
    _check(lib().dc_check_spec(ctypes.byref(s)), "dc_pack")
    nbytes = dc_packed_bytes(s)
    out = np.zeros(max(nbytes, 1), np.uint8)
    u, pu = _np_ptr(U, np.float32)
    g, pg = _np_ptr(sigma, np.float32)
    v, pv = _np_ptr(V, np.float32)
    _check(lib().dc_pack(ctypes.byref(s), pu, pg, pv, out.ctypes.data, out.size), "dc_pack")
    return out[:nbytes]


def dc_pack_codes(spec, codes_u, codes_v, sz_u, sz_v, sigma) -> np.ndarray:
    s = make_spec(spec)
    _check(lib().dc_check_spec(ctypes.byref(s)), "dc_pack_codes")
    nbytes = dc_packed_bytes(s)
    out = np.zeros(max(nbytes, 1), np.uint8)
    cu, p1 = _np_ptr(codes_u, np.uint8)
    cv, p2 = _np_ptr(codes_v, np.uint8)
    su, p3 = _np_ptr(sz_u, np.uint16)
    sv, p4 = _np_ptr(sz_v, np.uint16)
    g, p5 = _np_ptr(sigma, np.float32)
    _check(lib().dc_pack_codes(ctypes.byref(s), p1, p2, p3, p4, p5, out.ctypes.data, out.size),
           "dc_pack_codes")
    return out[:nbytes]


def dc_unpack(spec, buf):
    s = make_spec(spec)
    r = s.n8 + s.n3 + s.n2
    b, pb = _np_ptr(buf, np.uint8)
    cu = np.zeros((r, s.out), np.uint8)
    cv = np.zeros((r, s.in_), np.uint8)
    su = np.zeros((r, s.out // 128, 2), np.uint16)
    sv = np.zeros((r, s.in_ // 128, 2), np.uint16)
    sg = np.zeros(r, np.float32)
    _check(lib().dc_unpack(ctypes.byref(s), pb, b.size, cu.ctypes.data, cv.ctypes.data,
                           su.ctypes.data, sv.ctypes.data, sg.ctypes.data), "dc_unpack")
    return cu, cv, su, sv, sg


def dc_workspace_bytes(op: int, specs, T: int) -> int:
    arr = (dc_spec * len(specs))(*[make_spec(s) for s in specs])
    return int(lib().dc_workspace_bytes(int(op), arr, len(specs), int(T)))


def dc_group_workspace_bytes(specs, m: int, T: int) -> int:
    """specs: [m][n] (a list of m lists of n specs, or m*n specs in order)."""
    flat = [s for row in specs for s in row] if specs and isinstance(specs[0], (list, tuple)) and \
        not isinstance(specs[0][0], int) else list(specs)
    arr = (dc_spec * len(flat))(*[make_spec(s) for s in flat])
    return int(lib().dc_group_workspace_bytes(arr, int(m), len(flat) // int(m), int(T)))


# ----------------------------------------------------------------- device
class DeltaView:
    """A packed delta resident in device memory (keeps its tensor alive)."""

    def __init__(self, spec, buf):
        self.spec = make_spec(spec)
        self.buf = buf
        self.c = dc_delta_view(self.spec, ctypes.c_void_p(int(buf.data_ptr())))


def _dptr(t, what: str) -> int:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % what)
    return int(t.data_ptr())


def _stream(stream) -> int:
    if stream is not None:
        return int(stream)
    import torch
    return int(torch.cuda.current_stream().cuda_stream)


def _views(views: Sequence[DeltaView]):
    return (dc_delta_view * len(views))(*[v.c for v in views])


def dc_apply_decode(view: DeltaView, W_base, x, y, ws, T: int = None, stream=None) -> None:
    T = x.shape[0] if T is None else T
    _check(lib().dc_apply_decode(ctypes.byref(view.c), _dptr(W_base, "W_base"), _dptr(x, "x"),
                                 _dptr(y, "y"), int(T), _dptr(ws, "ws"), ws.numel() * ws.element_size(),
                                 _stream(stream)), "dc_apply_decode")


def dc_apply_multitenant(views: Sequence[DeltaView], W_base, x, tenant_ids, y, ws, T: int = None,
                         stream=None) -> None:
    T = x.shape[0] if T is None else T
    _check(lib().dc_apply_multitenant(_views(views), len(views), _dptr(W_base, "W_base"), _dptr(x, "x"),
                                      _dptr(tenant_ids, "tenant_ids"), _dptr(y, "y"), int(T),
                                      _dptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "dc_apply_multitenant")


def dc_apply_multitenant_noalloc(views: Sequence[DeltaView], W_base, x, tenant_ids, y, T: int = None,
                                 stream=None) -> None:
    """dc_apply_multitenant on the library's own scratch array (no workspace
    argument, nothing allocated by the call)."""
    T = x.shape[0] if T is None else T
    _check(lib().dc_apply_multitenant_noalloc(_views(views), len(views), _dptr(W_base, "W_base"), _dptr(x, "x"),
                                              _dptr(tenant_ids, "tenant_ids"), _dptr(y, "y"), int(T),
                                              _stream(stream)), "dc_apply_multitenant_noalloc")


def _ptr_array(ts, what):
    return (_P * len(ts))(*[_dptr(t, what) for t in ts])


class GroupCall:
    """dc_apply_multitenant_group with its arguments marshalled once.
    views: [m][n] DeltaViews; W_base: list of m tensors (None entries: delta
    only) or None; y: list of m output tensors."""

    def __init__(self, views, W_base, x, tenant_ids, y, ws, T: int = None, stream=None):
        m, n = len(views), len(views[0])
        T = x.shape[0] if T is None else T
        flat = [v for row in views for v in row]
        self._keep = (flat, W_base, x, tenant_ids, y, ws)
        self._arr = _views(flat)
        self._w = _ptr_array(W_base, "W_base") if W_base is not None else None
        self._y = _ptr_array(y, "y")
        self.args = (self._arr, m, n, self._w, _dptr(x, "x"), _dptr(tenant_ids, "tenant_ids"), self._y, int(T),
                     _dptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream))
        self._fn = lib().dc_apply_multitenant_group
        self._fn_t = lib().dc_apply_multitenant_group_timed

    def __call__(self) -> None:
        st = self._fn(*self.args)
        if st != DC_OK:
            raise DcError(st, "dc_apply_multitenant_group")

    def timed_array(self, ev) -> None:
        """ev: MultitenantCall.event_array(...) (stage events of the whole group)."""
        st = self._fn_t(*self.args, ev)
        if st != DC_OK:
            raise DcError(st, "dc_apply_multitenant_group_timed")


def dc_apply_multitenant_group(views, W_base, x, tenant_ids, y, ws, T: int = None, stream=None) -> None:
    GroupCall(views, W_base, x, tenant_ids, y, ws, T, stream)()


def dc_apply_multitenant_timed(views: Sequence[DeltaView], W_base, x, tenant_ids, y, ws, events,
                               T: int = None, stream=None) -> None:
    """events: len(STAGES)+1 raw hipEvent_t handles (ints) or None entries."""
    T = x.shape[0] if T is None else T
    ev = (_P * (len(STAGES) + 1))(*[None if e is None else int(e) for e in events])
    _check(lib().dc_apply_multitenant_timed(_views(views), len(views), _dptr(W_base, "W_base"),
                                            _dptr(x, "x"), _dptr(tenant_ids, "tenant_ids"), _dptr(y, "y"),
                                            int(T), _dptr(ws, "ws"), ws.numel() * ws.element_size(),
                                            _stream(stream), ev), "dc_apply_multitenant_timed")


def dc_apply_prefill(views: Sequence[DeltaView], W_base, x, seg_offsets, y, ws, stream=None) -> None:
    seg = np.ascontiguousarray(seg_offsets, dtype=np.int32)
    _check(lib().dc_apply_prefill(_views(views), len(views), _dptr(W_base, "W_base"), _dptr(x, "x"),
                                  seg.ctypes.data, _dptr(y, "y"), _dptr(ws, "ws"),
                                  ws.numel() * ws.element_size(), _stream(stream)), "dc_apply_prefill")


def dc_dequant(view: DeltaView, u_fp16, v_fp16, stream=None) -> None:
    _check(lib().dc_dequant(ctypes.byref(view.c), _dptr(u_fp16, "u_fp16"), _dptr(v_fp16, "v_fp16"),
                            _stream(stream)), "dc_dequant")


def dc_pack_device(spec, U, sigma, V, out, flag, stream=None) -> None:
    """Quantize and pack on the GPU (asynchronous): U [r][out], sigma [r] and
    V [r][in] device float32 tensors; out a device uint8 tensor of at least
    dc_packed_bytes(spec) bytes; flag a device int32/uint32 tensor of one
    element, 1 after the stream completes if an input was non-finite or a
    scale overflowed fp16."""
    s = make_spec(spec)
    _check(lib().dc_pack_device(ctypes.byref(s), _dptr(U, "U"), _dptr(sigma, "sigma"), _dptr(V, "V"),
                                _dptr(out, "out"), out.numel() * out.element_size(), _dptr(flag, "flag"),
                                _stream(stream)), "dc_pack_device")


class MultitenantCall:
    """dc_apply_multitenant with its arguments marshalled once, for callers
    that issue the same call many times (a serving loop, a benchmark)."""

    def __init__(self, views: Sequence[DeltaView], W_base, x, tenant_ids, y, ws, T: int = None,
                 stream=None):
        self._keep = (list(views), W_base, x, tenant_ids, y, ws)
        T = x.shape[0] if T is None else T
        self._arr = _views(views)
        self.args = (self._arr, len(views), _dptr(W_base, "W_base"), _dptr(x, "x"),
                     _dptr(tenant_ids, "tenant_ids"), _dptr(y, "y"), int(T), _dptr(ws, "ws"),
                     ws.numel() * ws.element_size(), _stream(stream))
        self._fn = lib().dc_apply_multitenant
        self._fn_t = lib().dc_apply_multitenant_timed

    def __call__(self) -> None:
        st = self._fn(*self.args)
        if st != DC_OK:
            raise DcError(st, "dc_apply_multitenant")

    def timed(self, events) -> None:
        self.timed_array(self.event_array(events))

    @staticmethod
    def event_array(events):
        """The events argument of dc_apply_multitenant_timed, marshalled once."""
        return (_P * (len(STAGES) + 1))(*[None if e is None else int(e) for e in events])

    def timed_array(self, ev) -> None:
        st = self._fn_t(*self.args, ev)
        if st != DC_OK:
            raise DcError(st, "dc_apply_multitenant_timed")


def dc_allocate_bits(err, cost, budget: int):
    """One candidate per pair minimizing the summed error within the budget
    (host): err [r][nb] float64, cost [nb] int.  Returns (choice int32 [r],
    total error)."""
    e = np.ascontiguousarray(err, dtype=np.float64)
    if e.ndim != 2:
        raise ValueError("err must be [r][nb]")
    c = np.ascontiguousarray(cost, dtype=np.int32)
    r, nb = e.shape
    choice = np.zeros(r, np.int32)
    total = ctypes.c_double(0.0)
    _check(lib().dc_allocate_bits(r, nb, c.ctypes.data, e.ctypes.data, int(budget), choice.ctypes.data,
                                  ctypes.addressof(total)), "dc_allocate_bits")
    return choice, total.value


# -------------------------------------------------------------- baselines
def dc_baseline_bytes(kind: int, out: int, inn: int, r: int = 0) -> int:
    return int(lib().dc_baseline_bytes(int(kind), int(out), int(inn), int(r)))


def dc_baseline_algorithmic_bytes(kind: int, out: int, inn: int, r: int = 0) -> int:
    return int(lib().dc_baseline_algorithmic_bytes(int(kind), int(out), int(inn), int(r)))


def dc_pack_lowrank(U16, sigma, V16) -> np.ndarray:
    """U16 fp16 [r][out], sigma fp32 [r], V16 fp16 [r][in] -> packed bytes."""
    U16 = np.ascontiguousarray(np.asarray(U16, np.float16))
    V16 = np.ascontiguousarray(np.asarray(V16, np.float16))
    r, out = U16.shape
    inn = V16.shape[1]
    sg, sp = _np_ptr(sigma, np.float32)
    n = dc_baseline_bytes(DC_KIND_LOWRANK, out, inn, r)
    buf = np.zeros(max(n, 1), np.uint8)
    _check(lib().dc_pack_lowrank(out, inn, r, U16.ctypes.data, sp, V16.ctypes.data, buf.ctypes.data, n),
           "dc_pack_lowrank")
    return buf[:n]


def dc_pack_bitdelta(signs, alpha) -> np.ndarray:
    """signs uint8 [out][in] (nonzero = +1), alpha float -> packed bytes."""
    sg, sp = _np_ptr(signs, np.uint8)
    out, inn = sg.shape
    n = dc_baseline_bytes(DC_KIND_BITDELTA, out, inn, 0)
    buf = np.zeros(max(n, 1), np.uint8)
    _check(lib().dc_pack_bitdelta(out, inn, sp, ctypes.c_float(float(alpha)), buf.ctypes.data, n),
           "dc_pack_bitdelta")
    return buf[:n]


class BaselineView:
    """A packed baseline delta in device memory (keeps its tensor alive)."""

    def __init__(self, kind: int, out: int, inn: int, r: int, buf):
        self.kind, self.out, self.inn, self.r = int(kind), int(out), int(inn), int(r)
        self.buf = buf
        self.c = dc_baseline_view(self.kind, self.out, self.inn, self.r,
                                  ctypes.c_void_p(int(buf.data_ptr()) if buf is not None else 0))


def _bviews(views):
    return (dc_baseline_view * len(views))(*[v.c for v in views])


def dc_baseline_workspace_bytes(views, m: int, T: int) -> int:
    """views: [m][n] BaselineViews (a list of m lists, or m*n in order)."""
    flat = [v for row in views for v in row] if isinstance(views[0], (list, tuple)) else list(views)
    return int(lib().dc_baseline_workspace_bytes(_bviews(flat), int(m), len(flat) // int(m), int(T)))


def dc_apply_baseline_multitenant(views, W_base, x, tenant_ids, y, ws, T: int = None, stream=None) -> None:
    T = x.shape[0] if T is None else T
    _check(lib().dc_apply_baseline_multitenant(_bviews(views), len(views), _dptr(W_base, "W_base"), _dptr(x, "x"),
                                               _dptr(tenant_ids, "tenant_ids"), _dptr(y, "y"), int(T),
                                               _dptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
           "dc_apply_baseline_multitenant")


class BaselineGroupCall:
    """dc_apply_baseline_multitenant_group with its arguments marshalled once
    (views [m][n] BaselineViews; W_base list of m tensors or None; y list of m)."""

    def __init__(self, views, W_base, x, tenant_ids, y, ws, T: int = None, stream=None):
        m, n = len(views), len(views[0])
        T = x.shape[0] if T is None else T
        flat = [v for row in views for v in row]
        self._keep = (flat, W_base, x, tenant_ids, y, ws)
        self._arr = _bviews(flat)
        self._w = _ptr_array(W_base, "W_base") if W_base is not None else None
        self._y = _ptr_array(y, "y")
        self.args = (self._arr, m, n, self._w, _dptr(x, "x"), _dptr(tenant_ids, "tenant_ids"), self._y, int(T),
                     _dptr(ws, "ws"), ws.numel() * ws.element_size(), _stream(stream))
        self._fn = lib().dc_apply_baseline_multitenant_group

    def __call__(self) -> None:
        st = self._fn(*self.args)
        if st != DC_OK:
            raise DcError(st, "dc_apply_baseline_multitenant_group")


def dc_apply_baseline_multitenant_group(views, W_base, x, tenant_ids, y, ws, T: int = None, stream=None) -> None:
    BaselineGroupCall(views, W_base, x, tenant_ids, y, ws, T, stream)()


# ------------------------------------------------------------ error table
def dc_error_table_workspace_bytes(r: int, inn: int, nw: int) -> int:
    return int(lib().dc_error_table_workspace_bytes(int(r), int(inn), int(nw)))


def dc_error_table(sigma, V, X, widths, err, flag, ws, stream=None) -> None:
    """sigma fp32 [r], V fp32 [r][in], X fp32 [in][ncal] (device tensors);
    err fp64 [r][len(widths)] and flag uint32/int32 [1] (device) are written."""
    w = np.ascontiguousarray(widths, dtype=np.int32)
    r, inn = V.shape
    ncal = X.shape[1]
    _check(lib().dc_error_table(int(r), int(inn), int(ncal), _dptr(sigma, "sigma"), _dptr(V, "V"), _dptr(X, "X"),
                                w.ctypes.data, int(w.size), _dptr(err, "err"), _dptr(flag, "flag"), _dptr(ws, "ws"),
                                ws.numel() * ws.element_size(), _stream(stream)), "dc_error_table")


def dc_svd_workspace_bytes(out: int, inn: int) -> int:
    return int(lib().dc_svd_workspace_bytes(int(out), int(inn)))


def dc_svd(delta, r: int, U, sigma, V, ws, stream=None) -> int:
    """delta fp32 [out][in] (device tensor); U fp32 [r][out], sigma fp32 [r],
    V fp32 [r][in] (device) are written; returns the Jacobi sweeps run.
    Synchronous."""
    out, inn = delta.shape
    sw = ctypes.c_int32(0)
    _check(lib().dc_svd(int(out), int(inn), int(r), _dptr(delta, "delta"), _dptr(U, "U"), _dptr(sigma, "sigma"),
                        _dptr(V, "V"), _dptr(ws, "ws"), ws.numel() * ws.element_size(), ctypes.byref(sw),
                        _stream(stream)), "dc_svd")
    return int(sw.value)
