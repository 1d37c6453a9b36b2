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

// Checks the tenant specs of one call; fills the shape and the work-split maxima.
struct Dims {
  int32_t out, in, rmax, tw, vb;
};

dc_status check_specs(const dc_spec* specs, int32_t n, Dims* d) {
  if (!specs || n < 1) return DC_ERR_INVALID_ARG;
  if (n > DC_MAX_TENANTS) return DC_ERR_UNSUPPORTED;
  d->out = specs[0].out;
  d->in = specs[0].in;
  d->rmax = d->tw = d->vb = 0;
  for (int k = 0; k < n; ++k) {
    if (dc_check_spec(&specs[k]) != DC_OK) return DC_ERR_SHAPE;
    if (specs[k].out != d->out || specs[k].in != d->in) return DC_ERR_SHAPE;
    const int32_t r = specs[k].n8 + specs[k].n3 + specs[k].n2;
    if (r > d->rmax) d->rmax = r;
    const int32_t vb = dc::v_blocks(specs[k].n8, specs[k].n3, specs[k].n2);
    if (vb > d->vb) d->vb = vb;
    const int32_t tw = dc::t_width(specs[k].n8, specs[k].n3, specs[k].n2);
    if (tw > d->tw) d->tw = tw;
  }
  return DC_OK;
}

}  // namespace

namespace dc {
dc_status run_apply(const dc_delta_view* views, int32_t n, const uint16_t* W, const uint16_t* x,
                    const int32_t* ids, const int32_t* seg, int32_t mode, uint16_t* y, int32_t T, void* ws,
                    size_t ws_bytes, void* stream, void* const* events, size_t ws_limit) {
  if (!views || n < 1) return DC_ERR_INVALID_ARG;
  if (n > DC_MAX_TENANTS) return DC_ERR_UNSUPPORTED;
  if (T < 0) return DC_ERR_INVALID_ARG;
  dc_spec specs[DC_MAX_TENANTS] = {};
  for (int k = 0; k < n; ++k) specs[k] = views[k].spec;
  Dims dm;
  dc_status st = check_specs(specs, n, &dm);
  if (st != DC_OK) return st;
  const int32_t out = dm.out, in = dm.in, rmax = dm.rmax;
  dc::TenantTable table;
  std::memset(&table, 0, sizeof(table));
  for (int k = 0; k < n; ++k) {
    const int32_t r = specs[k].n8 + specs[k].n3 + specs[k].n2;
    if (r > 0 && !views[k].base) return DC_ERR_INVALID_ARG;
    if (!aligned(views[k].base, 16)) return DC_ERR_ALIGN;
    table.t[k].base = static_cast<const uint8_t*>(views[k].base);
    table.t[k].n8 = specs[k].n8;
    table.t[k].n3 = specs[k].n3;
    table.t[k].n2 = specs[k].n2;
  }
  if (!x || !y || (!ws && ws_limit == 0)) return DC_ERR_INVALID_ARG;
  if (mode == 1 && !ids) return DC_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(y, 16) || (W && !aligned(W, 16)) || !aligned(ws, 256) ||
      (ids && !aligned(ids, 4)))
    return DC_ERR_ALIGN;
  if (overlap(x, (size_t)T * in * 2, y, (size_t)T * out * 2)) return DC_ERR_INVALID_ARG;
  dc::WsLayout wl{};
  dc::ws_layout(T, in, out, dm.tw, n, true, dm.vb, 0, &wl);
  if (ws_limit > 0) {   // the library's own scratch array: its size is the limit, its address comes later
    if (wl.total > ws_limit) return DC_ERR_UNSUPPORTED;
    ws_bytes = ws_limit;
  } else if (ws_bytes < wl.total) {
    return DC_ERR_BUFFER;
  }
  if (mode == 2 && T >= dc::kDenseMin) {
    // the dense prefill operands, when the workspace holds them; without them
    // the call takes the decode kernels
    dc::WsLayout wd{};
    dc::ws_layout(T, in, out, dm.tw, n, true, dm.vb, dc::dense_rank_pad(rmax), &wd);
    if (ws_bytes >= wd.total) wl = wd;
  }
  // the kernels address t, the backbone partials and each packed buffer with 32-bit byte offsets
  const size_t lim = (size_t)INT32_MAX;
  if ((size_t)T * wl.rs * 4 > lim || (size_t)T * out * 4 > lim) return DC_ERR_UNSUPPORTED;
  for (int k = 0; k < n; ++k)
    if (dc_packed_bytes(&specs[k]) > lim) return DC_ERR_UNSUPPORTED;
  if (T == 0) return DC_OK;
  if (ws_limit > 0) {
    ws = scratch_ptr();
    if (!ws) return DC_ERR_HIP;
  }
  dc::ApplyArgs a;
  a.tenants = &table;
  a.n = n;
  a.out = out;
  a.in = in;
  a.rmax = rmax;
  a.T = T;
  a.W = W;
  a.x = x;
  a.ids = ids;
  a.seg = seg;
  a.mode = mode;
  a.y = y;
  a.ws = static_cast<uint8_t*>(ws);
  a.wl = wl;
  a.stream = stream;
  a.events = events;
  return dc::launch_apply(a) == 0 ? DC_OK : DC_ERR_HIP;
}
}  // namespace dc

namespace {
dc_status run(const dc_delta_view* views, int32_t n, const uint16_t* W, const uint16_t* x, const int32_t* ids,
              const int32_t* seg, int32_t mode, uint16_t* y, int32_t T, void* ws, size_t ws_bytes, void* stream,
              void* const* events = nullptr) {
  return dc::run_apply(views, n, W, x, ids, seg, mode, y, T, ws, ws_bytes, stream, events, 0);
}
}  // namespace

extern "C" {

size_t dc_workspace_bytes(int32_t op, const dc_spec* specs, int32_t n, int32_t T) {
  if (op < DC_OP_DECODE || op > DC_OP_PREFILL || T < 0) return 0;
  if (op == DC_OP_DECODE && n != 1) return 0;
  Dims dm;
  if (check_specs(specs, n, &dm) != DC_OK) return 0;
  dc::WsLayout wl{};
  dc::ws_layout(T, dm.in, dm.out, dm.tw, n, true, dm.vb,
                 op == DC_OP_PREFILL && T >= dc::kDenseMin ? dc::dense_rank_pad(dm.rmax) : 0, &wl);
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

}  // extern "C"
