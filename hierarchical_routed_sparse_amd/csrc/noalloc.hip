// The backward without a caller workspace: hga_attend_bwd_noalloc.
//
// For callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): the
// backward's scratch (row statistics, group-mask map, dK/dV work orders; the
// layout hga_attend_bwd_workspace describes) lives in a file-scope device
// array of kScratchBytes instead of a workspace argument.  Each GPU the
// library runs on holds its own copy of the array until the process ends.
//
// In host code `scratch` names a host-side stand-in, not a device address;
// its device address is taken once per device with hipGetSymbolAddress (on
// that device's first call) and only that address is ever passed on.
#include <hip/hip_runtime.h>

#include <mutex>

#include "hga.h"

namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;   // HGA_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == HGA_NOALLOC_SCRATCH_BYTES, "header and array agree");
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

// The device address of this device's copy of `scratch`, looked up on the
// device's first call; nullptr when HIP cannot resolve it.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" hga_status hga_attend_bwd_noalloc(const hga_shape* shape, const void* Q,
                                             const void* K, const void* V, const void* O,
                                             const float* lse, const void* dO,
                                             const int32_t* group_idx, void* dQ, void* dK,
                                             void* dV, void* stream) {
  size_t need = 0;
  hga_status st = hga_attend_bwd_workspace(shape, &need);
  if (st != HGA_OK) return st;
  if (need > kScratchBytes) return HGA_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (!ws) return HGA_ERR_HIP;
  // every part of the scratch is written before it is read (delta and the
  // group-mask map by the dQ kernel, the work orders by their ordering pass),
  // so nothing needs clearing between calls
  return hga_attend_bwd(shape, Q, K, V, O, lse, dO, group_idx, dQ, dK, dV, ws, kScratchBytes,
                        stream);
}
