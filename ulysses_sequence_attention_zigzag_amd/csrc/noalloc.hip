// usp_ring_fwd_noalloc: usp_ring_fwd with its workspace in a file-scope
// device array instead of caller memory, for callers that cannot allocate.
//
// The array is allocated with the library's code object on each GPU it runs
// on and stays there until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in symbol): the
// first call on a device looks up that device's copy with
// hipGetSymbolAddress, with the device current, and keeps the address per
// device; every later use goes through that address.

#include <hip/hip_runtime.h>

#include <mutex>

#include "usp_internal.h"

namespace usp {
namespace {

// Workspace bytes the allocation-free ring call can use (the small and
// window workloads need a few MiB at most: staged q / k / v of a natural-order
// non-basic layout, an f32 accumulator for a bf16 or reordered output, and
// the tile plans).
constexpr size_t kScratchBytes = size_t(64) << 20;

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's copy of `scratch` (looked up once per device).
usp_status scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error("hipGetDevice failed: %s", hipGetErrorString(e));
    return USP_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device ordinal %d beyond the %d devices the scratch table holds", dev, kMaxDevices);
    return USP_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_error("hipGetSymbolAddress of the scratch array failed: %s", hipGetErrorString(e));
      return USP_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return USP_OK;
}

}  // namespace
}  // namespace usp

using namespace usp;

extern "C" {

usp_status usp_ring_fwd_noalloc(const usp_ring_args* a, void* stream) {
  const size_t need = usp_ring_fwd_workspace_size(a);
  if (need == 0) {
    // invalid arguments: usp_ring_fwd reports which, before touching anything
    return usp_ring_fwd(a, nullptr, 0, stream);
  }
  if (need > kScratchBytes) {
    set_error("usp_ring_fwd_noalloc: these arguments need %zu bytes of workspace, more than its %zu-byte "
              "scratch; use usp_ring_fwd with a caller workspace", need, kScratchBytes);
    return USP_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  const usp_status st = scratch_of_current_device(&ws);
  if (st != USP_OK) return st;
  // the ring rewrites everything it reads from its workspace (tile plans,
  // staged rows, accumulators), so nothing needs clearing between calls
  return usp_ring_fwd(a, ws, kScratchBytes, stream);
}

}  // extern "C"
