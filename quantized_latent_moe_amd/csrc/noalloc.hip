// The expert stage without a caller workspace, for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).
//
// The workspace the kernels need (routing tables, H in sorted order, the
// weighted slot rows, the split activation rows) lives in `scratch`, a
// file-scope device array of LAT_MOE_NOALLOC_SCRATCH_BYTES that every GPU the
// library runs on holds until the process ends.  In host code the array's
// name is only a host-side stand-in: its device address on the current GPU
// comes from hipGetSymbolAddress, taken once per device and kept, and that
// address is what the kernels receive.  The kernels need no initialised
// workspace (every word they read is written earlier in the same call), so
// nothing is cleared between calls.  Calls on one GPU share its array: calls
// that overlap in time on one GPU (two streams, two threads) race.
#include <mutex>

#include "lat_moe_internal.h"

namespace {

constexpr size_t kScratchBytes = LAT_MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kScratchBytes];

// This GPU's copy of scratch: hipGetSymbolAddress once per device, with that
// device current, the address kept for later calls.
int scratch_address(void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LAT_MOE_EDEVICE;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return LAT_MOE_ELAUNCH;
    addr[dev] = p;
  }
  *out = addr[dev];
  return LAT_MOE_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" int lat_moe_expert_forward_noalloc(const void* x_q8_1, const int32_t* router_idx, const float* router_w,
                                              const void* gateup_q3k, const void* down_iq4nl,
                                              const lat_moe_shapes* shapes, float* y, void* stream) {
  // argument checks first, with no HIP call (as every entry point)
  const size_t need = lat_moe_workspace_size(shapes);
  if (need == 0) return LAT_MOE_EINVAL;
  if (need > kScratchBytes) return LAT_MOE_ESCRATCH;
  if (shapes->T == 0) return LAT_MOE_OK;
  const void* ptrs[] = {x_q8_1, router_idx, router_w, gateup_q3k, down_iq4nl, y};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return LAT_MOE_EINVAL;
  int rc = latmoe::device_check(nullptr);
  if (rc != LAT_MOE_OK) return rc;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != LAT_MOE_OK) return rc;
  return latmoe::stage_forward(x_q8_1, router_idx, router_w, gateup_q3k, down_iq4nl, shapes, y, ws, kScratchBytes,
                               stream);
}
