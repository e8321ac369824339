// zs_noalloc.hip -- zero_shard_reduce_noalloc: the one-shot shard reduce
// with its norm slots in a static device array of this library instead of a
// caller's workspace, for callers that cannot allocate device memory.
//
// `scratch` below is a __device__ array: each GPU the library runs on holds
// its own copy (64 KiB) until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in symbol); the
// first call on a device, with that device current, asks the runtime for
// that device's address of the array and keeps it, and every launch uses
// that address.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "zero_step.h"
#include "zs_internal.h"

namespace {

constexpr int kSlots = ZERO_REDUCE_WORKSPACE_BYTES / static_cast<int>(sizeof(zero_norm_acc));
static_assert(kSlots * sizeof(zero_norm_acc) == ZERO_REDUCE_WORKSPACE_BYTES, "slot layout");

static __device__ __align__(256) zero_norm_acc scratch[kSlots];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

constexpr size_t kMaxNormElems = size_t(1) << 37;

// This device's address of `scratch`, looked up once per device.
hipError_t scratch_for_current_device(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_scratch_err[dev] != hipSuccess) return g_scratch_err[dev];
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int zero_shard_reduce_noalloc(const void* const* replicas, int P, int dtype,
                                         size_t n, float inv_scale, float* g_out,
                                         zero_norm_acc* acc, void* stream) {
  try {
    if (replicas == nullptr || P < 1 || P > ZERO_MAX_REPLICAS) return ZERO_EINVAL;
    if (dtype != ZERO_F32 && dtype != ZERO_BF16) return ZERO_EINVAL;
    for (int k = 0; k < P; ++k) {
      if (replicas[k] == nullptr) return ZERO_EINVAL;
      if (!aligned16(replicas[k])) return ZERO_EALIGN;
    }
    if (g_out == nullptr && acc == nullptr) return ZERO_EINVAL;
    if ((g_out && !aligned16(g_out)) || (acc && !aligned16(acc))) return ZERO_EALIGN;
    if (acc != nullptr && n > kMaxNormElems) return ZERO_ESIZE;
    if (n == 0) return ZERO_OK;
    void* slots = nullptr;
    if (scratch_for_current_device(&slots) != hipSuccess) return ZERO_EHIP;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // The slots keep whatever the last call on this device left: clear them
    // (a fill kernel, so the call can also be recorded in a graph), then the
    // one-shot reduce, whose fold launch clears them again.
    if (zs::launch_acc_clear(static_cast<zero_norm_acc*>(slots), kSlots, st) != hipSuccess)
      return ZERO_EHIP;
    return zs::launch_reduce(replicas, P, dtype, n, inv_scale, g_out, acc, st, nullptr, slots) ==
                   hipSuccess
               ? ZERO_OK
               : ZERO_EHIP;
  } catch (...) {
    return ZERO_EHIP;
  }
}
