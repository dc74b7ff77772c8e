// An end-to-end denoise entry point that allocates nothing: for callers that
// cannot allocate device memory (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  Its workspace is a file-scope
// device array of a fixed size, one copy per GPU the library runs on, held
// until the process ends.
//
// Host code never uses the array's name as an address: the name is a
// host-side stand-in.  The first call on a device, with that device current,
// asks the runtime for the array's device address (hipGetSymbolAddress) and
// keeps it per device; every later use -- the workspace handed to the
// kernels -- is that address.
#include <cstdio>
#include <mutex>

#include "internal.h"

namespace oidn {
namespace {

constexpr size_t kScratchBytes = size_t(OIDN_NOALLOC_SCRATCH_MB) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` per device, once looked up

// The array's address on the current device, looked up on the first call
// for that device.  Returns OIDN_OK or an error status (message set).
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(OIDN_E_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return set_error(OIDN_E_UNSUPPORTED, "device index out of range");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(OIDN_E_HIP, "hipGetSymbolAddress of the no-alloc scratch failed");
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return OIDN_OK;
}

}  // namespace
}  // namespace oidn

using namespace oidn;

extern "C" int oidn_unet_forward_noalloc(const void* d_weights, int in_channels,
                                         const float* color, const float* albedo,
                                         const float* normal, int w, int h, int hdr, int transfer,
                                         float input_scale, int max_tile, int overlap,
                                         float* out_rgba, int dtype, hipStream_t stream) {
  // size check first, on the host: one tile's workspace must fit
  size_t per_tile = 0;
  int rc = tile_workspace_bytes(in_channels, w, h, max_tile, overlap, dtype, &per_tile);
  if (rc) return rc;
  if (per_tile > kScratchBytes) {
    char msg[256];
    snprintf(msg, sizeof(msg),
             "a tile of this plan needs %zu bytes of workspace, more than the %zu-byte no-alloc "
             "scratch holds: use a smaller max_tile, or oidn_unet_forward", per_tile, kScratchBytes);
    return set_error(OIDN_E_WORKSPACE, msg);
  }
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  return denoise_fit(d_weights, in_channels, color, albedo, normal, w, h, hdr, transfer,
                     input_scale, max_tile, overlap, ws, kScratchBytes, out_rgba, dtype, stream);
}

extern "C" int oidn_unet_noalloc_scratch_bytes(size_t* bytes) {
  if (!bytes) return set_error(OIDN_E_INVALID, "null bytes pointer");
  *bytes = kScratchBytes;
  return clear_error();
}
