// The library's own device workspace, for callers that cannot allocate
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): dc_apply_multitenant_noalloc runs dc_apply_multitenant with
// this array as its workspace.
//
// The array is a file-scope __device__ variable, so every GPU the library
// runs on holds its own copy from the time the code object is loaded until
// the process ends.  In host code its name is only a host-side stand-in:
// the device address is looked up once per device with hipGetSymbolAddress
// (with that device current) and kept in a table; kernels receive that
// address, never the name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dc_internal.h"

namespace dc {
namespace {

constexpr size_t kScratchBytes = (size_t)DC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[dev] = p;
  }
  return g_ptr[dev];
}

}  // namespace dc

extern "C" dc_status dc_apply_multitenant_noalloc(const dc_delta_view* views, int32_t n, const uint16_t* W_base,
                                                  const uint16_t* x, const int32_t* tenant_ids, uint16_t* y,
                                                  int32_t T, void* stream) {
  return dc::run_apply(views, 1, n, &W_base, x, tenant_ids, nullptr, 1, &y, T, nullptr, 0, stream, nullptr,
                       dc::kScratchBytes);
}
