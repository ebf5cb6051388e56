// psattn_noalloc.hip -- device-resident scratch of the allocation-free forward
// entry point (psattn_fwd_noalloc).
//
// The paged forward's split pass writes one partial (O, LSE) per split and
// the merge reads them back; psattn_fwd takes that scratch from the caller.
// For callers that cannot allocate at call time, this file holds a fixed
// array in device memory instead.  Each GPU the library runs on holds its own
// copy of the array from module load until the process ends.  Its device
// address is looked up once per device (the device of the call's stream,
// made current for the lookup) and kept;
// host code never passes the array's own name to a kernel, since on the host
// that name is only a stand-in for the device symbol.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/psattn.h"
#include "launch.h"

namespace psattn {
namespace {

static __device__ __attribute__((aligned(256))) char scratch[PSATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // per-device address of `scratch`, once looked up

}  // namespace

int noalloc_scratch(void* stream, void** ptr) {
  // the array of the device the kernels will run on: the stream's
  int dev = 0;
  hipError_t e = hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // the symbol's address on that device, looked up with it current
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return (int)e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return (int)e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

}  // namespace psattn
