// gmlp_group_quantize_noalloc: gmlp_group_quantize with its workspace in a fixed device array of
// this library, for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The workspace of a group quantize holds the per-call split tables (prefix sums of m_splits)
// and, for NVFP4, the per-group amax slots of the Hadamard-amax pass.  Here it is the array
// `scratch` below: one copy per GPU, held until the process ends.  Every call rewrites the split
// tables and clears the amax slots in its first kernel (the split scan), so no state carries over
// from the previous call; calls that overlap on one GPU (different streams, no ordering) share
// the array and race.
#include "gmlp.h"
#include "planner.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

constexpr int kStaticMaxGroups = 1024;
constexpr size_t kStaticWsBytes = 288 * 1024;   // >= the workspace of 1024 groups (checked per call)

// The device array.  Host code never uses its name as an address (on the host it is only a
// stand-in for the symbol): the device address of each GPU's copy comes from
// hipGetSymbolAddress, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[kStaticWsBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices];

gmlp_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return gmlp::set_error(GMLP_HIP_ERROR, "system: hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return gmlp::set_error(GMLP_UNSUPPORTED, "system: device %d is beyond the %d devices supported", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return gmlp::set_error(GMLP_HIP_ERROR, "system: hipGetSymbolAddress of the static workspace failed: %s",
                             hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GMLP_OK;
}

}  // namespace

extern "C" gmlp_status gmlp_group_quantize_noalloc(const void* x, int64_t M, int64_t K, const int32_t* m_splits,
                                                   int32_t G, gmlp_recipe recipe, int32_t want_row,
                                                   int32_t want_col, const gmlp_grouped_q* out,
                                                   hipStream_t stream) {
  if (G < 1 || G > kStaticMaxGroups)
    return gmlp::set_error(GMLP_UNSUPPORTED,
                           "dims: the allocation-free group quantize takes 1 to %d groups, got %d (use "
                           "gmlp_group_quantize with a caller workspace)", kStaticMaxGroups, G);
  const size_t need = gmlp::group_quantize_ws_need(G);
  if (need > kStaticWsBytes)
    return gmlp::set_error(GMLP_WORKSPACE, "workspace: %zu bytes needed, the static workspace holds %zu", need,
                           kStaticWsBytes);
  void* ws = nullptr;
  const gmlp_status st = scratch_address(&ws);
  if (st != GMLP_OK) return st;
  return gmlp::group_quantize_on(x, M, K, m_splits, G, recipe, want_row, want_col, out, ws, kStaticWsBytes, stream);
}
