// The library's static device scratch: a file-scope device array that backs
// ccl_execute_static, the entry point for callers that cannot allocate device memory.
// Every GPU the library runs on holds one copy of it until the process ends. In host
// code the array's name is only a stand-in for the symbol: its device address on a
// device comes from hipGetSymbolAddress, looked up once per device (with that device
// current) and kept here; host code uses that address, never the name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ccl_internal.h"

static __device__ __align__(256) unsigned char scratch[ccl::kStaticScratchBytes];

namespace ccl {

int static_scratch_base(int device, unsigned char** base, std::string* err) {
  static std::mutex mu;
  static unsigned char* ptr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) {
    *err = "device id out of range";
    return CCL_ERR_INVALID_ARGUMENT;
  }
  std::lock_guard<std::mutex> lk(mu);
  if (!ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess || cur != device) {
      *err = "the static scratch is looked up with its device current";
      return CCL_ERR_INVALID_ARGUMENT;
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
      return CCL_ERR_HIP;
    }
    ptr[device] = static_cast<unsigned char*>(p);
  }
  *base = ptr[device];
  return CCL_OK;
}

}  // namespace ccl
