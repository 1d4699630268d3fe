// Per-token int8 activation quantizer for gfx950.
//
// One workgroup (4 waves) per token row.  Pass 1 finds the row's absolute
// maximum by comparing fp16 bit patterns with the sign cleared (monotone for
// finite values); pass 2 re-reads the row, which the first pass left in
// cache, and writes int8.  The row is at most 48 KiB for the supported
// layer widths, so the re-read costs L2 bandwidth, not HBM.
//
// Per-token dynamic scaling is the activation scheme the PrefixQuant page
// ("Key Findings") treats as the usual practice; the 8-bit activation side of
// W4A8 is from the QServe/QoQ abstract.  Reading used here:
//   s_a = fp16(fp32(absmax / 127)),  A8 = clamp(rint(A * fp32(1 / s_a)), +-127)
// Both divisions are IEEE-correct fp32 divisions (HIP's default for '/'),
// conversions to fp16 and rint round half to even.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace w4a8 {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float h2f(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 va = __builtin_bit_cast(u16x2, a), vb = __builtin_bit_cast(u16x2, b);
  u16x2 r = va > vb ? va : vb;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ int quant1(uint16_t h, float r) {
  float v = __builtin_rintf(h2f(h) * r);
  v = fminf(fmaxf(v, -127.0f), 127.0f);
  return static_cast<int>(v);
}

__device__ __forceinline__ uint32_t quant4(uint32_t h01, uint32_t h23, float r) {
  uint32_t b0 = uint32_t(quant1(uint16_t(h01 & 0xFFFFu), r)) & 0xFFu;
  uint32_t b1 = uint32_t(quant1(uint16_t(h01 >> 16), r)) & 0xFFu;
  uint32_t b2 = uint32_t(quant1(uint16_t(h23 & 0xFFFFu), r)) & 0xFFu;
  uint32_t b3 = uint32_t(quant1(uint16_t(h23 >> 16), r)) & 0xFFu;
  return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// VEC: rows are 16-byte aligned and k % 8 == 0 (8 halves per load).
template <bool VEC>
__global__ __launch_bounds__(kThreads) void quant_act_kernel(const uint16_t* __restrict__ a,
                                                             int k, int lda,
                                                             int8_t* __restrict__ a8, int lda8,
                                                             uint16_t* __restrict__ s_a) {
  const int row = blockIdx.x;
  const uint16_t* src = a + size_t(row) * size_t(lda);
  int8_t* dst = a8 + size_t(row) * size_t(lda8);
  const int tid = threadIdx.x;

  uint32_t mx = 0;  // two running maxima of |h| bit patterns
  if (VEC) {
    for (int i = tid * 8; i < k; i += kThreads * 8) {
      uint4 v = *reinterpret_cast<const uint4*>(src + i);
      mx = pk_max_u16(mx, v.x & 0x7FFF7FFFu);
      mx = pk_max_u16(mx, v.y & 0x7FFF7FFFu);
      mx = pk_max_u16(mx, v.z & 0x7FFF7FFFu);
      mx = pk_max_u16(mx, v.w & 0x7FFF7FFFu);
    }
  } else {
    for (int i = tid; i < k; i += kThreads) mx = pk_max_u16(mx, uint32_t(src[i]) & 0x7FFFu);
  }
  uint32_t m16 = max(mx & 0xFFFFu, mx >> 16);
  // wave reduction, then across the four waves through LDS
  for (int off = 32; off > 0; off >>= 1) m16 = max(m16, uint32_t(__shfl_xor(int(m16), off)));
  __shared__ uint32_t wave_max[kThreads / 64];
  if ((tid & 63) == 0) wave_max[tid >> 6] = m16;
  __syncthreads();
  uint32_t amax_bits = max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));

  const float amax = h2f(uint16_t(amax_bits));
  const _Float16 scale_h = static_cast<_Float16>(amax / 127.0f);
  const float scale = static_cast<float>(scale_h);
  const float r = scale != 0.0f ? 1.0f / scale : 0.0f;
  if (tid == 0) s_a[row] = __builtin_bit_cast(uint16_t, scale_h);

  if (VEC) {
    for (int i = tid * 8; i < k; i += kThreads * 8) {
      uint4 v = *reinterpret_cast<const uint4*>(src + i);
      uint2 o;
      o.x = quant4(v.x, v.y, r);
      o.y = quant4(v.z, v.w, r);
      *reinterpret_cast<uint2*>(dst + i) = o;
    }
  } else {
    for (int i = tid; i < k; i += kThreads) dst[i] = int8_t(quant1(src[i], r));
  }
}

}  // namespace

hipError_t launch_quant_act(const uint16_t* a, int m, int k, int lda, int8_t* a8, int lda8,
                            uint16_t* s_a, hipStream_t stream) {
  const bool vec = (k % 8 == 0) && (lda % 8 == 0) && (lda8 % 8 == 0) &&
                   (reinterpret_cast<uintptr_t>(a) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(a8) % 8 == 0);
  dim3 grid(m), block(kThreads);
  void* args[] = {&a, &k, &lda, &a8, &lda8, &s_a};
  // hipLaunchKernel reports this launch's own status (the runtime's
  // last-error slot may hold an unrelated earlier error of the caller)
  const void* fn = vec ? reinterpret_cast<const void*>(&quant_act_kernel<true>)
                       : reinterpret_cast<const void*>(&quant_act_kernel<false>);
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace w4a8
