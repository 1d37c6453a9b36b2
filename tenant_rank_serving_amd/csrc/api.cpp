// Device entry points of libdeltacome.so: argument checks on the host, then
// kernel launches on the caller's stream.  No allocation, no synchronization.
#include <cstdint>
#include <cstring>

#include "dc_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x0 = reinterpret_cast<uintptr_t>(a), y0 = reinterpret_cast<uintptr_t>(b);
  return x0 < y0 + nb && y0 < x0 + na;
}

// Checks the tenant specs of one matrix of a call; fills its shape and the
// work-split maxima.
struct Dims {
  int32_t out, in, rmax, tw, vb, prp;   // prp: padded rank rows of the dense prefill form
};

dc_status check_specs(const dc_spec* specs, int32_t n, Dims* d) {
  if (!specs || n < 1) return DC_ERR_INVALID_ARG;
  if (n > DC_MAX_TENANTS) return DC_ERR_UNSUPPORTED;
  d->out = specs[0].out;
  d->in = specs[0].in;
  d->rmax = d->tw = d->vb = d->prp = 0;
  for (int k = 0; k < n; ++k) {
    if (dc_check_spec(&specs[k]) != DC_OK) return DC_ERR_SHAPE;
    if (specs[k].out != d->out || specs[k].in != d->in) return DC_ERR_SHAPE;
    const int32_t r = specs[k].n8 + specs[k].n3 + specs[k].n2;
    if (r > d->rmax) d->rmax = r;
    const int32_t vb = dc::v_blocks(specs[k].n8, specs[k].n3, specs[k].n2);
    if (vb > d->vb) d->vb = vb;
    const int32_t tw = dc::t_width(specs[k].n8, specs[k].n3, specs[k].n2);
    if (tw > d->tw) d->tw = tw;
    const int32_t prp = dc::pf_rank_pad(specs[k].n8, specs[k].n3, specs[k].n2);
    if (prp > d->prp) d->prp = prp;
  }
  return DC_OK;
}

// The specs of a group: specs [m][n]; every matrix with the same in.
dc_status check_group(const dc_spec* specs, int32_t m, int32_t n, Dims* d) {
  if (!specs || m < 1 || n < 1) return DC_ERR_INVALID_ARG;
  if (m > DC_MAX_GROUP || n > DC_MAX_TENANTS) return DC_ERR_UNSUPPORTED;
  for (int j = 0; j < m; ++j) {
    const dc_status st = check_specs(specs + (size_t)j * n, n, &d[j]);
    if (st != DC_OK) return st;
    if (d[j].in != d[0].in) return DC_ERR_SHAPE;
  }
  return DC_OK;
}

bool layout_of_group(const Dims* d, int32_t m, int32_t n, int32_t T, int32_t drp, dc::WsLayout* wl) {
  int32_t out[DC_MAX_GROUP], rs[DC_MAX_GROUP], vb[DC_MAX_GROUP];
  for (int j = 0; j < m; ++j) {
    out[j] = d[j].out;
    rs[j] = d[j].tw;
    vb[j] = d[j].vb;
  }
  return dc::ws_layout(T, d[0].in, n, m, out, rs, vb, drp, wl);
}

// Checks baseline views [m][n]: one kind, one out/in per matrix, one in for
// the group; fills each matrix's shape and largest rank.
struct BDims {
  int32_t out, in, rmax;
};

dc_status check_baseline(const dc_baseline_view* v, int32_t m, int32_t n, int32_t* kind, BDims* d) {
  if (!v || m < 1 || n < 1) return DC_ERR_INVALID_ARG;
  if (m > DC_MAX_GROUP || n > DC_MAX_TENANTS) return DC_ERR_UNSUPPORTED;
  *kind = v[0].kind;
  if (*kind != DC_KIND_LOWRANK && *kind != DC_KIND_BITDELTA) return DC_ERR_SHAPE;
  for (int j = 0; j < m; ++j) {
    d[j].out = v[(size_t)j * n].out;
    d[j].in = v[(size_t)j * n].in;
    d[j].rmax = 0;
    for (int k = 0; k < n; ++k) {
      const dc_baseline_view& e = v[(size_t)j * n + k];
      if (e.kind != *kind || e.out != d[j].out || e.in != d[j].in) return DC_ERR_SHAPE;
      if (!dc::baseline_valid(e.kind, e.out, e.in, e.r)) return DC_ERR_SHAPE;
      if (e.r > d[j].rmax) d[j].rmax = e.r;
    }
    if (d[j].in != d[0].in) return DC_ERR_SHAPE;
  }
  return DC_OK;
}

bool baseline_layout(int32_t kind, const BDims* d, int32_t m, int32_t n, int32_t T, dc::WsLayout* wl) {
  int32_t out[DC_MAX_GROUP], rs[DC_MAX_GROUP], vb[DC_MAX_GROUP];
  for (int j = 0; j < m; ++j) {
    out[j] = d[j].out;
    if (kind == DC_KIND_LOWRANK) {
      rs[j] = (int32_t)dc::round_up((size_t)(d[j].rmax > 0 ? d[j].rmax : 1), 16);
      vb[j] = dc::lr_vblocks(d[j].rmax);
    } else {
      rs[j] = 8;
      vb[j] = d[j].out / dc::kBdRows;
    }
  }
  return dc::ws_layout(T, d[0].in, n, m, out, rs, vb, 0, wl, kind);
}

}  // namespace

namespace dc {
dc_status run_apply(const dc_delta_view* views, int32_t m, int32_t n, const uint16_t* const* W, const uint16_t* x,
                    const int32_t* ids, const int32_t* seg, int32_t mode, uint16_t* const* y, int32_t T, void* ws,
                    size_t ws_bytes, void* stream, void* const* events, size_t ws_limit) {
  if (!views || n < 1 || m < 1 || !y) return DC_ERR_INVALID_ARG;
  if (n > DC_MAX_TENANTS || m > DC_MAX_GROUP) return DC_ERR_UNSUPPORTED;
  if (T < 0) return DC_ERR_INVALID_ARG;
  dc_spec specs[DC_MAX_GROUP * DC_MAX_TENANTS];
  for (int i = 0; i < m * n; ++i) specs[i] = views[i].spec;
  Dims dm[DC_MAX_GROUP];
  dc_status st = check_group(specs, m, n, dm);
  if (st != DC_OK) return st;
  const int32_t in = dm[0].in;
  dc::TenantTable tables[DC_MAX_GROUP];
  for (int j = 0; j < m; ++j) {
    std::memset(&tables[j], 0, sizeof(tables[j]));
    for (int k = 0; k < n; ++k) {
      const dc_delta_view& v = views[(size_t)j * n + k];
      const int32_t r = v.spec.n8 + v.spec.n3 + v.spec.n2;
      if (r > 0 && !v.base) return DC_ERR_INVALID_ARG;
      if (!aligned(v.base, 16)) return DC_ERR_ALIGN;
      tables[j].t[k].base = static_cast<const uint8_t*>(v.base);
      tables[j].t[k].n8 = v.spec.n8;
      tables[j].t[k].n3 = v.spec.n3;
      tables[j].t[k].n2 = v.spec.n2;
    }
  }
  if (!x || (!ws && ws_limit == 0)) return DC_ERR_INVALID_ARG;
  if (mode == 1 && !ids) return DC_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(ws, 256) || (ids && !aligned(ids, 4))) return DC_ERR_ALIGN;
  for (int j = 0; j < m; ++j) {
    if (!y[j]) return DC_ERR_INVALID_ARG;
    if (!aligned(y[j], 16) || (W && W[j] && !aligned(W[j], 16))) return DC_ERR_ALIGN;
    if (overlap(x, (size_t)T * in * 2, y[j], (size_t)T * dm[j].out * 2)) return DC_ERR_INVALID_ARG;
    for (int i = 0; i < j; ++i)
      if (overlap(y[i], (size_t)T * dm[i].out * 2, y[j], (size_t)T * dm[j].out * 2)) return DC_ERR_INVALID_ARG;
  }
  dc::WsLayout wl{};
  if (!layout_of_group(dm, m, n, T, 0, &wl)) return DC_ERR_INVALID_ARG;
  if (ws_limit > 0) {   // the library's own scratch array: its size is the limit, its address comes later
    if (wl.total > ws_limit) return DC_ERR_UNSUPPORTED;
    ws_bytes = ws_limit;
  } else if (ws_bytes < wl.total) {
    return DC_ERR_BUFFER;
  }
  if (mode == 2 && m == 1 && T >= dc::kDenseMin) {
    // the dense prefill operands, when the workspace holds them; without them
    // the call takes the decode kernels
    dc::WsLayout wd{};
    layout_of_group(dm, 1, n, T, dm[0].prp, &wd);
    if (ws_bytes >= wd.total) wl = wd;
  }
  // the kernels address t, the backbone product and each packed buffer with 32-bit byte offsets
  const size_t lim = (size_t)INT32_MAX;
  for (int j = 0; j < m; ++j)
    if ((size_t)T * wl.mat[j].rs * 4 > lim || (size_t)T * dm[j].out * 4 > lim) return DC_ERR_UNSUPPORTED;
  for (int i = 0; i < m * n; ++i)
    if (dc_packed_bytes(&specs[i]) > lim) return DC_ERR_UNSUPPORTED;
  if (T == 0) return DC_OK;
  if (ws_limit > 0) {
    ws = scratch_ptr();
    if (!ws) return DC_ERR_HIP;
  }
  dc::ApplyArgs a{};
  a.m = m;
  for (int j = 0; j < m; ++j) {
    a.mat[j].tenants = &tables[j];
    a.mat[j].out = dm[j].out;
    a.mat[j].rmax = dm[j].rmax;
    a.mat[j].W = W ? W[j] : nullptr;
    a.mat[j].y = y[j];
  }
  a.n = n;
  a.in = in;
  a.T = T;
  a.x = x;
  a.ids = ids;
  a.seg = seg;
  a.mode = mode;
  a.ws = static_cast<uint8_t*>(ws);
  a.wl = wl;
  a.stream = stream;
  a.events = events;
  return dc::launch_apply(a) == 0 ? DC_OK : DC_ERR_HIP;
}

dc_status run_baseline(const dc_baseline_view* views, int32_t m, int32_t n, const uint16_t* const* W,
                       const uint16_t* x, const int32_t* ids, uint16_t* const* y, int32_t T, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!views || n < 1 || m < 1 || !y || T < 0) return DC_ERR_INVALID_ARG;
  int32_t kind = 0;
  BDims dm[DC_MAX_GROUP];
  dc_status st = check_baseline(views, m, n, &kind, dm);
  if (st != DC_OK) return st;
  const int32_t in = dm[0].in;
  dc::TenantTable tables[DC_MAX_GROUP];
  for (int j = 0; j < m; ++j) {
    std::memset(&tables[j], 0, sizeof(tables[j]));
    for (int k = 0; k < n; ++k) {
      const dc_baseline_view& v = views[(size_t)j * n + k];
      const bool reads = kind == DC_KIND_BITDELTA || v.r > 0;
      if (reads && !v.base) return DC_ERR_INVALID_ARG;
      if (!aligned(v.base, 16)) return DC_ERR_ALIGN;
      tables[j].t[k].base = static_cast<const uint8_t*>(v.base);
      tables[j].t[k].n8 = kind == DC_KIND_LOWRANK ? v.r : 0;
    }
  }
  if (!x || !ws || !ids) return DC_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(ws, 256) || !aligned(ids, 4)) return DC_ERR_ALIGN;
  for (int j = 0; j < m; ++j) {
    if (!y[j]) return DC_ERR_INVALID_ARG;
    if (!aligned(y[j], 16) || (W && W[j] && !aligned(W[j], 16))) return DC_ERR_ALIGN;
    if (overlap(x, (size_t)T * in * 2, y[j], (size_t)T * dm[j].out * 2)) return DC_ERR_INVALID_ARG;
    for (int i = 0; i < j; ++i)
      if (overlap(y[i], (size_t)T * dm[i].out * 2, y[j], (size_t)T * dm[j].out * 2)) return DC_ERR_INVALID_ARG;
  }
  dc::WsLayout wl{};
  if (!baseline_layout(kind, dm, m, n, T, &wl)) return DC_ERR_INVALID_ARG;
  if (ws_bytes < wl.total) return DC_ERR_BUFFER;
  // the kernels address t, the backbone product and each buffer with 32-bit byte offsets
  const size_t lim = (size_t)INT32_MAX;
  for (int j = 0; j < m; ++j)
    if ((size_t)T * wl.mat[j].rs * 4 > lim || (size_t)T * dm[j].out * 4 > lim ||
        dc_baseline_bytes(kind, dm[j].out, in, dm[j].rmax) > lim)
      return DC_ERR_UNSUPPORTED;
  if (T == 0) return DC_OK;
  dc::ApplyArgs a{};
  a.kind = kind;
  a.m = m;
  for (int j = 0; j < m; ++j) {
    a.mat[j].tenants = &tables[j];
    a.mat[j].out = dm[j].out;
    a.mat[j].rmax = dm[j].rmax;
    a.mat[j].W = W ? W[j] : nullptr;
    a.mat[j].y = y[j];
  }
  a.n = n;
  a.in = in;
  a.T = T;
  a.x = x;
  a.ids = ids;
  a.seg = nullptr;
  a.mode = 1;
  a.ws = static_cast<uint8_t*>(ws);
  a.wl = wl;
  a.stream = stream;
  a.events = nullptr;
  return dc::launch_apply(a) == 0 ? DC_OK : DC_ERR_HIP;
}
}  // namespace dc

namespace {
dc_status run(const dc_delta_view* views, int32_t n, const uint16_t* W, const uint16_t* x, const int32_t* ids,
              const int32_t* seg, int32_t mode, uint16_t* y, int32_t T, void* ws, size_t ws_bytes, void* stream,
              void* const* events = nullptr) {
  return dc::run_apply(views, 1, n, &W, x, ids, seg, mode, &y, T, ws, ws_bytes, stream, events, 0);
}
}  // namespace

extern "C" {

size_t dc_workspace_bytes(int32_t op, const dc_spec* specs, int32_t n, int32_t T) {
  if (op < DC_OP_DECODE || op > DC_OP_PREFILL || T < 0) return 0;
  if (op == DC_OP_DECODE && n != 1) return 0;
  Dims dm;
  if (check_specs(specs, n, &dm) != DC_OK) return 0;
  dc::WsLayout wl{};
  if (!layout_of_group(&dm, 1, n, T, op == DC_OP_PREFILL && T >= dc::kDenseMin ? dm.prp : 0,
                       &wl))
    return 0;
  return wl.total;
}

size_t dc_group_workspace_bytes(const dc_spec* specs, int32_t m, int32_t n, int32_t T) {
  if (T < 0) return 0;
  Dims dm[DC_MAX_GROUP];
  if (check_group(specs, m, n, dm) != DC_OK) return 0;
  dc::WsLayout wl{};
  if (!layout_of_group(dm, m, n, T, 0, &wl)) return 0;
  return wl.total;
}

dc_status dc_apply_decode(const dc_delta_view* d, const uint16_t* W_base, const uint16_t* x,
                          uint16_t* y, int32_t T, void* ws, size_t ws_bytes, void* stream) {
  if (!d) return DC_ERR_INVALID_ARG;
  return run(d, 1, W_base, x, nullptr, nullptr, 0, y, T, ws, ws_bytes, stream);
}

dc_status dc_apply_multitenant(const dc_delta_view* views, int32_t n, const uint16_t* W_base,
                               const uint16_t* x, const int32_t* tenant_ids, uint16_t* y,
                               int32_t T, void* ws, size_t ws_bytes, void* stream) {
  return run(views, n, W_base, x, tenant_ids, nullptr, 1, y, T, ws, ws_bytes, stream);
}

dc_status dc_apply_multitenant_group(const dc_delta_view* views, int32_t m, int32_t n, const uint16_t* const* W_base,
                                     const uint16_t* x, const int32_t* tenant_ids, uint16_t* const* y, int32_t T,
                                     void* ws, size_t ws_bytes, void* stream) {
  return dc::run_apply(views, m, n, W_base, x, tenant_ids, nullptr, 1, y, T, ws, ws_bytes, stream, nullptr, 0);
}

dc_status dc_apply_multitenant_group_timed(const dc_delta_view* views, int32_t m, int32_t n,
                                           const uint16_t* const* W_base, const uint16_t* x,
                                           const int32_t* tenant_ids, uint16_t* const* y, int32_t T, void* ws,
                                           size_t ws_bytes, void* stream, void* const* events) {
  return dc::run_apply(views, m, n, W_base, x, tenant_ids, nullptr, 1, y, T, ws, ws_bytes, stream, events, 0);
}

dc_status dc_apply_multitenant_timed(const dc_delta_view* views, int32_t n, const uint16_t* W_base,
                                     const uint16_t* x, const int32_t* tenant_ids, uint16_t* y,
                                     int32_t T, void* ws, size_t ws_bytes, void* stream,
                                     void* const* events) {
  return run(views, n, W_base, x, tenant_ids, nullptr, 1, y, T, ws, ws_bytes, stream, events);
}

dc_status dc_apply_prefill(const dc_delta_view* views, int32_t n, const uint16_t* W_base,
                           const uint16_t* x, const int32_t* seg_offsets, uint16_t* y, void* ws,
                           size_t ws_bytes, void* stream) {
  if (!seg_offsets || n < 1) return DC_ERR_INVALID_ARG;
  if (n > DC_MAX_TENANTS) return DC_ERR_UNSUPPORTED;
  if (seg_offsets[0] != 0) return DC_ERR_INVALID_ARG;
  for (int k = 0; k < n; ++k)
    if (seg_offsets[k + 1] < seg_offsets[k]) return DC_ERR_INVALID_ARG;
  return run(views, n, W_base, x, nullptr, seg_offsets, 2, y, seg_offsets[n], ws, ws_bytes, stream);
}

size_t dc_baseline_workspace_bytes(const dc_baseline_view* views, int32_t m, int32_t n, int32_t T) {
  if (T < 0) return 0;
  int32_t kind = 0;
  BDims dm[DC_MAX_GROUP];
  if (check_baseline(views, m, n, &kind, dm) != DC_OK) return 0;
  dc::WsLayout wl{};
  if (!baseline_layout(kind, dm, m, n, T, &wl)) return 0;
  return wl.total;
}

dc_status dc_apply_baseline_multitenant(const dc_baseline_view* views, int32_t n, const uint16_t* W_base,
                                        const uint16_t* x, const int32_t* tenant_ids, uint16_t* y, int32_t T,
                                        void* ws, size_t ws_bytes, void* stream) {
  return dc::run_baseline(views, 1, n, &W_base, x, tenant_ids, &y, T, ws, ws_bytes, stream);
}

dc_status dc_apply_baseline_multitenant_group(const dc_baseline_view* views, int32_t m, int32_t n,
                                              const uint16_t* const* W_base, const uint16_t* x,
                                              const int32_t* tenant_ids, uint16_t* const* y, int32_t T,
                                              void* ws, size_t ws_bytes, void* stream) {
  return dc::run_baseline(views, m, n, W_base, x, tenant_ids, y, T, ws, ws_bytes, stream);
}

dc_status dc_pack_device(const dc_spec* spec, const float* U, const float* sigma, const float* V, void* out,
                         size_t out_bytes, uint32_t* flag, void* stream) {
  if (!spec || !out || !flag) return DC_ERR_INVALID_ARG;
  if (dc_check_spec(spec) != DC_OK) return DC_ERR_SHAPE;
  const int32_t r = spec->n8 + spec->n3 + spec->n2;
  if (r > 0 && (!U || !V || !sigma)) return DC_ERR_INVALID_ARG;
  if (!aligned(out, 16) || !aligned(flag, 4) || (U && !aligned(U, 8)) || (V && !aligned(V, 8)) ||
      (sigma && !aligned(sigma, 4)))
    return DC_ERR_ALIGN;
  const size_t need = dc_packed_bytes(spec);
  if (out_bytes < need) return DC_ERR_BUFFER;
  if (need > (size_t)INT32_MAX) return DC_ERR_UNSUPPORTED;
  return dc::launch_pack(spec->out, spec->in, spec->n8, spec->n3, spec->n2, U, sigma, V,
                         static_cast<uint8_t*>(out), flag, stream) == 0 ? DC_OK : DC_ERR_HIP;
}

size_t dc_error_table_workspace_bytes(int32_t r, int32_t in, int32_t nw) {
  if (r < 0 || in <= 0 || in % dc::kGroup || nw < 1 || nw > DC_ERR_MAX_WIDTHS) return 0;
  return dc::round_up(4 * (size_t)r * nw * in, 256) + 256;
}

dc_status dc_error_table(int32_t r, int32_t in, int32_t ncal, const float* sigma, const float* V, const float* X,
                         const int32_t* widths, int32_t nw, double* err, uint32_t* flag, void* ws, size_t ws_bytes,
                         void* stream) {
  if (r < 0 || ncal < 1 || !widths || nw < 1 || nw > DC_ERR_MAX_WIDTHS || !flag) return DC_ERR_INVALID_ARG;
  for (int k = 0; k < nw; ++k)
    if (widths[k] < 0 || widths[k] > 8) return DC_ERR_INVALID_ARG;
  if (in <= 0 || in % dc::kGroup) return DC_ERR_SHAPE;
  if (r > 0 && (!sigma || !V || !X || !err || !ws)) return DC_ERR_INVALID_ARG;
  if (!aligned(flag, 4) || (V && !aligned(V, 8)) || (X && !aligned(X, 4)) || (sigma && !aligned(sigma, 4)) ||
      (err && !aligned(err, 8)) || (ws && !aligned(ws, 256)))
    return DC_ERR_ALIGN;
  const size_t lim = (size_t)INT32_MAX;
  if ((size_t)r * in > lim || (size_t)in * ncal > lim || (size_t)r * nw * in > lim) return DC_ERR_UNSUPPORTED;
  if (ws_bytes < dc_error_table_workspace_bytes(r, in, nw)) return DC_ERR_BUFFER;
  return dc::launch_error_table(r, in, ncal, sigma, V, X, widths, nw, err, flag, static_cast<float*>(ws), stream) == 0
             ? DC_OK
             : DC_ERR_HIP;
}

dc_status dc_dequant(const dc_delta_view* d, uint16_t* u_fp16, uint16_t* v_fp16, void* stream) {
  if (!d) return DC_ERR_INVALID_ARG;
  if (dc_check_spec(&d->spec) != DC_OK) return DC_ERR_SHAPE;
  const int32_t r = d->spec.n8 + d->spec.n3 + d->spec.n2;
  if (r == 0) return DC_OK;
  if (!d->base || !u_fp16 || !v_fp16) return DC_ERR_INVALID_ARG;
  if (!aligned(d->base, 16) || !aligned(u_fp16, 16) || !aligned(v_fp16, 16)) return DC_ERR_ALIGN;
  dc::Tenant t;
  t.base = static_cast<const uint8_t*>(d->base);
  t.n8 = d->spec.n8;
  t.n3 = d->spec.n3;
  t.n2 = d->spec.n2;
  t.pad_ = 0;
  return dc::launch_dequant(t, d->spec.out, d->spec.in, u_fp16, v_fp16, stream) == 0 ? DC_OK : DC_ERR_HIP;
}

size_t dc_svd_workspace_bytes(int32_t out, int32_t in) {
  if (out < 1 || in < 1 || (out < in ? out : in) > 16384) return 0;
  return dc::svd_layout(out, in, 0).total;
}

dc_status dc_svd(int32_t out, int32_t in, int32_t r, const float* delta, float* U, float* sigma, float* V, void* ws,
                 size_t ws_bytes, int32_t* sweeps, void* stream) {
  if (sweeps) *sweeps = 0;
  if (out < 1 || in < 1) return DC_ERR_SHAPE;
  const int32_t m = out < in ? out : in;
  if (r < 0 || r > m || !delta || !ws || (r > 0 && (!U || !sigma || !V))) return DC_ERR_INVALID_ARG;
  if (m > 16384 || (size_t)out * in >= ((size_t)1 << 31)) return DC_ERR_UNSUPPORTED;
  if (!aligned(delta, 4) || !aligned(ws, 256) || (U && !aligned(U, 4)) || (V && !aligned(V, 4)) ||
      (sigma && !aligned(sigma, 4)))
    return DC_ERR_ALIGN;
  if (ws_bytes < dc_svd_workspace_bytes(out, in)) return DC_ERR_BUFFER;
  if (r == 0) return DC_OK;   // nothing to write
  const int st = dc::launch_svd(out, in, r, delta, U, sigma, V, static_cast<uint8_t*>(ws), sweeps, stream);
  return st == 0 ? DC_OK : (st > 0 ? DC_ERR_RANGE : DC_ERR_HIP);
}

}  // extern "C"
