// Static exchange-record storage for mk_decode_step_noalloc (include/mk.h): the decode step for
// callers that cannot allocate device memory.  The persistent decode kernel's scratch -- the
// epoch-tagged exchange records every phase publishes and polls, and the per-workgroup argmax
// records -- lives here in one file-scope device array instead of the caller's workspace.
//
// In host code `scratch` names a host-side stand-in, not device memory.  Its device address is
// looked up once per device, with that device current, when a context is created on it
// (mk_noalloc_scratch, called from mk_create), and only that address is ever handed to kernels.
// Every context on a device shares the one array, and it keeps the last call's records: the
// entry point clears the part a call uses before launching, and calls that overlap on one device
// race.

#include <hip/hip_runtime.h>

#include <mutex>

#include "mk_internal.h"

static __device__ __align__(256) unsigned char scratch[MK_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;

std::mutex g_mu;
bool g_done[kMaxDevices];
hipError_t g_rc[kMaxDevices];
void* g_ptr[kMaxDevices];

}  // namespace

// Device address of `scratch` on `device` (which the caller has made current), looked up on the
// first call for that device and kept for the process.  Returns 0, or -1 with *err set when the
// lookup failed (the failure is kept too: the array is not usable on that device).
extern "C" int mk_noalloc_scratch(int device, void** out, const char** err) {
  if (device < 0 || device >= kMaxDevices) {
    *err = "device index beyond the static scratch table";
    return -1;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_done[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_rc[device] = e;
    g_ptr[device] = e == hipSuccess ? p : nullptr;
    g_done[device] = true;
  }
  if (g_rc[device] != hipSuccess) {
    *err = hipGetErrorString(g_rc[device]);
    return -1;
  }
  *out = g_ptr[device];
  return 0;
}
