// The library's one static device buffer: scratch for w4a8_gemm_noalloc,
// the entry point for callers that cannot allocate.  It holds the tiled
// GEMM's int32 partial sums when K is split over workgroups, the memory
// w4a8_gemm takes from the caller's workspace.
//
// Each GPU the library runs on holds its own copy of the array for the life
// of the process.  In host code the array's name is only a stand-in for its
// device address, so the address is looked up once per device, with that
// device current, by hipGetSymbolAddress, and that pointer is what kernels
// and copies receive.

#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace w4a8 {
namespace {

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace w4a8
