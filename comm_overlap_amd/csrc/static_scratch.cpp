// Allocation-free MLP forward: tpslice_mlp_fwd with its workspace (the activations H and the
// split-k partial products of the up-projection) in a fixed device array of this library instead
// of a caller buffer, for callers that cannot allocate device memory (code under stream capture,
// tight serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ variable: every GPU the library runs on holds its own copy,
// at its own address, until the process ends. In host code its name only stands for the symbol,
// so its device address is looked up once per device (with that device current) and kept; kernels
// receive that address, never the name. Calls on one GPU share its copy: two calls that overlap in
// time on the same GPU race on it. Nothing in it needs to start at zero (the up-projection writes
// every element of H and of the partial products before the down-projection reads them).
#include <hip/hip_runtime.h>

#include <cstddef>
#include <mutex>

#include "plan.hpp"

namespace {

constexpr size_t kScratchBytes = TPSLICE_STATIC_SCRATCH_BYTES;  // the largest workspace it takes
constexpr int kMaxDevices = 64;

__device__ __align__(256) char scratch[kScratchBytes];

void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The device address of the current device's copy of `scratch`, looked up on the first call on
// that device.
tpslice_status_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return tps::fail(TPSLICE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return tps::fail(TPSLICE_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                     kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return tps::fail(TPSLICE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TPSLICE_OK;
}

}  // namespace

extern "C" tpslice_status_t tpslice_mlp_fwd_static(tpslice_plan_t p, const void* X, const void* W1, const void* b1,
                                                   const void* W2, void* Z, void* U_save, void* Z_handoff,
                                                   const tpslice_streams_t* streams) {
  tps::clear_error();
  if (!tps::plan_ok(p)) return tps::fail(TPSLICE_ERR_INVALID, "invalid plan handle");
  const size_t need = tps::mlp_fwd_ws(p).total;
  if (need > kScratchBytes)
    return tps::fail(TPSLICE_ERR_WORKSPACE,
                     "the MLP forward of this plan needs %zu bytes of workspace; the static scratch holds %zu",
                     need, kScratchBytes);
  void* ws = nullptr;
  const tpslice_status_t st = scratch_address(&ws);
  if (st != TPSLICE_OK) return st;
  return tpslice_mlp_fwd(p, X, W1, b1, W2, Z, U_save, Z_handoff, ws, kScratchBytes, streams);
}
