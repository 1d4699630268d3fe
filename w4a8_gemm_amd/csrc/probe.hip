// Read-only stream probe for gfx950: the practical HBM read ceiling that the
// weight-streaming GEMMs are compared against.  It is not part of the layer.
//
// Every thread of a grid of `workgroups` x 512 threads walks the buffer with
// a grid stride, four non-temporal 16-byte loads in flight per iteration,
// and folds what it reads into one register.  A store happens only when
// that register equals a fixed value, so the loads cannot be optimised away
// while the kernel writes (almost) nothing.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace w4a8 {
namespace {

constexpr int kProbeThreads = 512;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4* __restrict__ src,
                                                                   size_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const size_t stride = size_t(gridDim.x) * kProbeThreads;
  size_t i = size_t(blockIdx.x) * kProbeThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    const u32x4 b = __builtin_nontemporal_load(src + i + stride);
    const u32x4 c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4 d = __builtin_nontemporal_load(src + i + 3 * stride);
    x ^= (a.x ^ a.y ^ a.z ^ a.w) + (b.x ^ b.y ^ b.z ^ b.w) + (c.x ^ c.y ^ c.z ^ c.w) +
         (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(src + i);
    x ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (x == 0x9E3779B9u) sink[blockIdx.x] = x;
}

}  // namespace

hipError_t launch_read_probe(const void* src, size_t bytes, int workgroups, uint32_t* sink,
                             hipStream_t stream) {
  const u32x4* s = static_cast<const u32x4*>(src);
  size_t n16 = bytes / 16;
  void* args[] = {&s, &n16, &sink};
  return hipLaunchKernel(reinterpret_cast<const void*>(&read_probe_kernel), dim3(workgroups),
                         dim3(kProbeThreads), args, 0, stream);
}

}  // namespace w4a8
