// Device scratch memory for the entry point that allocates nothing
// (hga_decode_step_noalloc): callers that cannot allocate -- code under HIP
// graph capture, tight serving loops, harnesses that forbid allocation -- get the
// generation step's workspace from a file-scope device array instead of a
// caller-provided buffer.
//
// Each GPU the library runs on holds its own copy of the array (kScratchBytes)
// until the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory, so the array's device address is looked up once per device with
// hipGetSymbolAddress and only that address is used afterwards.  Every call on a
// GPU shares that GPU's array and leaves its contents behind: the arrival counters
// at its start are zero before the first call (static storage, and cleared once at
// set-up) and every call returns them to zero; the rest is written before it is
// read within a call.  Calls that overlap on one GPU (two streams, two threads)
// race on the array.
#include <mutex>

#include "hga_internal.h"

// The array itself.  Host code never uses this name as memory: it only passes it to
// hipGetSymbolAddress below.
static __device__ __align__(256) unsigned char scratch[hga::kNoallocScratchBytes];

namespace hga {
namespace {

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
DeviceScratch g_devices[kMaxDevices];

__global__ void clear_words(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t noalloc_scratch(void** ptr, hipStream_t s) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  DeviceScratch& g = g_devices[dev];
  bool first = false;
  std::call_once(g.once, [&] {
    void* p = nullptr;
    g.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g.ptr = g.err == hipSuccess ? p : nullptr;
    first = true;
  });
  if (g.err != hipSuccess) return g.err;
  if (first) {
    // The counter arrays must start at zero: cleared once, on the first call's stream
    // and ahead of its kernels (static storage is zero already; this makes it explicit).
    const int64_t words = (int64_t)(decode_counter_bytes(kNoallocCounterSlots) / 4);
    e = launch_kernel(clear_words, dim3((unsigned)((words + 255) / 256)), dim3(256), s, (uint32_t*)g.ptr, words);
    if (e != hipSuccess) return e;
  }
  *ptr = g.ptr;
  return hipSuccess;
}

}  // namespace hga
