// GEMM workspace held in the library itself, for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid hipMalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds its own copy
// until the process ends.  Host code never passes the array's name to a kernel (on the host
// it is only a stand-in for the symbol); it asks the runtime for the array's device address
// once per device, with that device current, and passes that address as the workspace.
#include <mutex>

#include "w12_kernels.h"

namespace w12 {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_workspace(void** ws, hipStream_t stream) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    // the arrival counters must be zero on entry to every GEMM; each GEMM leaves them zero
    e = init_gemm_workspace(p, kCounterBytes, stream);
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *ws = g_ptr[dev];
  return hipSuccess;
}

}  // namespace w12
