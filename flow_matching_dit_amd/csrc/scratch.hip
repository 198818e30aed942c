// A fixed device scratch area for entry points that must not allocate: a file-scope
// __device__ array that every GPU the library runs on holds from the library's load until
// the process ends. Host code never passes the array's name to a kernel or a copy (on the
// host it names a stand-in, not device memory): it asks for the device address once per
// device with hipGetSymbolAddress and uses that.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace gr00t {
namespace {
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

size_t static_scratch_bytes() { return kStaticScratchBytes; }

// The device address of `scratch` on `device`, which must be the current device. Looked up on
// the first request for that device, then kept.
hipError_t static_scratch_address(int device, void** ptr) {
  *ptr = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  int cur = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != device) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[device]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[device] = p;
  }
  *ptr = g_addr[device];
  return hipSuccess;
}

}  // namespace gr00t
