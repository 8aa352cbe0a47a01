// sscan_noalloc.hip -- sscan_fwd_noalloc: sscan_fwd with its workspace taken from a
// fixed device array of this library instead of caller memory, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).
//
// The array lives in this file's code object: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  Host code never
// passes the array's name to a kernel (in host code that name is only a stand-in
// for the symbol): the device address of the copy on each device is looked up
// once, with that device current, and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sscan.h"

namespace {

// The most workspace a no-alloc call may need (sscan_workspace_bytes of the call).
constexpr size_t kScratchBytes = size_t(64) << 20;
static_assert(SSCAN_NOALLOC_SCRATCH_BYTES == kScratchBytes, "scratch size mismatch");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lookup;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` per device, once looked up

// The current device's copy of the array (the device the caller's stream belongs
// to).  The first call on a device looks its address up with that device current.
int current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SSCAN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_lookup);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSCAN_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SSCAN_OK;
}

}  // namespace

extern "C" {

SSCAN_API int sscan_fwd_noalloc(const void* u, const void* delta, const float* delta_bias, int softplus,
                                const float* A, const void* B, const void* C, const float* D, const void* z, void* y,
                                int64_t batch, int64_t dim, int64_t len, int64_t dstate, int reverse, void* stream,
                                int io_dtype, int bc_dtype) {
  // 0 for invalid sizes too: sscan_fwd then reports them before any HIP call
  const size_t need = sscan_workspace_bytes(batch, dim, len, dstate, 0);
  if (need > kScratchBytes) return SSCAN_ERR_TOO_LARGE;
  void* ws = nullptr;
  if (need > 0) {
    // every argument first, so that an invalid call touches no device: without a
    // workspace the checks end at the workspace, the last one
    const int st = sscan_validate_fwd(u, delta, delta_bias, softplus, A, B, C, D, z, y, batch, dim, len, dstate,
                                      reverse, io_dtype, bc_dtype, nullptr, 0);
    if (st != SSCAN_ERR_WORKSPACE) return st == SSCAN_OK ? SSCAN_ERR_WORKSPACE : st;
    const int sc = current_scratch(&ws);
    if (sc != SSCAN_OK) return sc;
  }
  return sscan_fwd(u, delta, delta_bias, softplus, A, B, C, D, z, y, batch, dim, len, dstate, reverse, stream,
                   io_dtype, bc_dtype, ws, need > 0 ? kScratchBytes : 0);
}

}  // extern "C"
