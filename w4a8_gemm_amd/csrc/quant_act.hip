// Per-token int8 activation quantizer for gfx950.
//
// One workgroup (4 waves) per token row.  The row's absolute maximum comes
// from comparing fp16 bit patterns with the sign cleared (monotone for finite
// values).  Rows of up to 32768 halves are loaded once into registers (up to
// 16 chunks of 8 halves per thread), all loads in flight together, and
// quantized from there; longer rows are read twice (the second pass hits the
// cache).
//
// The arithmetic (scale, reciprocal, rounding, clamp) is in quant_common.h,
// shared with the fused small-M GEMM.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"
#include "quant_common.h"

namespace w4a8 {
namespace {

using namespace dev;

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t row_absmax_bits(uint32_t mx, int tid) {
  // wave reduction, then across the four waves through LDS
  const uint32_t m16 = wave_max_u32(absmax_bits(mx));
  __shared__ uint32_t wave_max[kThreads / 64];
  if ((tid & 63) == 0) wave_max[tid >> 6] = m16;
  __syncthreads();
  return max(max(wave_max[0], wave_max[1]), max(wave_max[2], wave_max[3]));
}

// writes s_a (thread 0) and returns the multiplier fp32(1 / s_a)
__device__ __forceinline__ float row_scale(uint32_t amax_bits, uint16_t* s_a_out, bool write) {
  const uint16_t sb = act_scale_bits(amax_bits);
  if (write) *s_a_out = sb;
  return act_recip(sb);
}

// VEC: rows are 16-byte aligned and k % 8 == 0 (8 halves per load).
// CH > 0: k <= CH * 8 * kThreads, the row is held in CH registers chunks.
template <bool VEC, int CH>
__global__ __launch_bounds__(kThreads) void quant_act_kernel(const uint16_t* __restrict__ a,
                                                             int k, int lda,
                                                             int8_t* __restrict__ a8, int lda8,
                                                             uint16_t* __restrict__ s_a) {
  const int row = blockIdx.x;
  const uint16_t* src = a + size_t(row) * size_t(lda);
  int8_t* dst = a8 + size_t(row) * size_t(lda8);
  const int tid = threadIdx.x;

  uint32_t mx = 0;  // two running maxima of |h| bit patterns
  if (VEC && CH > 0) {
    uint4 v[CH > 0 ? CH : 1];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int i = (c * kThreads + tid) * 8;
      v[c] = i < k ? *reinterpret_cast<const uint4*>(src + i) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int c = 0; c < CH; ++c) mx = absmax8(mx, v[c]);
    const float r = row_scale(row_absmax_bits(mx, tid), s_a + row, tid == 0);
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int i = (c * kThreads + tid) * 8;
      if (i < k) *reinterpret_cast<uint2*>(dst + i) = quant8(v[c], r);
    }
    return;
  }
  if (VEC) {
    for (int i = tid * 8; i < k; i += kThreads * 8) {
      mx = absmax8(mx, *reinterpret_cast<const uint4*>(src + i));
    }
  } else {
    for (int i = tid; i < k; i += kThreads) mx = pk_max_u16(mx, uint32_t(src[i]) & 0x7FFFu);
  }
  const float r = row_scale(row_absmax_bits(mx, tid), s_a + row, tid == 0);

  if (VEC) {
    for (int i = tid * 8; i < k; i += kThreads * 8) {
      *reinterpret_cast<uint2*>(dst + i) = quant8(*reinterpret_cast<const uint4*>(src + i), r);
    }
  } else {
    for (int i = tid; i < k; i += kThreads) dst[i] = int8_t(quant1(src[i], r));
  }
}

// Static per-tensor scale: no reduction, each thread quantizes 8 halves (or
// one when rows are not 16-byte aligned) with the multiplier fp32(1 / s)
// and row 0's threads also write s_a[m] = s for the GEMM epilogue.
template <bool VEC>
__global__ __launch_bounds__(kThreads) void quant_act_static_kernel(
    const uint16_t* __restrict__ a, int m, int k, int lda, uint16_t scale_bits,
    int8_t* __restrict__ a8, int lda8, uint16_t* __restrict__ s_a) {
  const float r = act_recip(scale_bits);
  const int per = VEC ? 8 : 1;
  const int row_items = (k + per - 1) / per;
  const long idx = long(blockIdx.x) * kThreads + threadIdx.x;
  if (idx < m) s_a[idx] = scale_bits;
  if (idx >= long(m) * row_items) return;
  const int row = int(idx / row_items);
  const int i = int(idx - long(row) * row_items) * per;
  const uint16_t* src = a + size_t(row) * size_t(lda) + i;
  int8_t* dst = a8 + size_t(row) * size_t(lda8) + i;
  if (VEC)
    *reinterpret_cast<uint2*>(dst) = quant8(*reinterpret_cast<const uint4*>(src), r);
  else
    *dst = int8_t(quant1(*src, r));
}

}  // namespace

hipError_t launch_quant_act_static(const uint16_t* a, int m, int k, int lda, uint16_t scale_bits,
                                   int8_t* a8, int lda8, uint16_t* s_a, hipStream_t stream) {
  const bool vec = (k % 8 == 0) && (lda % 8 == 0) && (lda8 % 8 == 0) &&
                   (reinterpret_cast<uintptr_t>(a) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(a8) % 8 == 0);
  const long items = long(m) * (vec ? k / 8 : k);
  const long threads = items > m ? items : m;
  dim3 grid(unsigned((threads + kThreads - 1) / kThreads)), block(kThreads);
  void* args[] = {&a, &m, &k, &lda, &scale_bits, &a8, &lda8, &s_a};
  const void* fn = vec ? reinterpret_cast<const void*>(&quant_act_static_kernel<true>)
                       : reinterpret_cast<const void*>(&quant_act_static_kernel<false>);
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

hipError_t launch_quant_act(const uint16_t* a, int m, int k, int lda, int8_t* a8, int lda8,
                            uint16_t* s_a, hipStream_t stream) {
  const bool vec = (k % 8 == 0) && (lda % 8 == 0) && (lda8 % 8 == 0) &&
                   (reinterpret_cast<uintptr_t>(a) % 16 == 0) &&
                   (reinterpret_cast<uintptr_t>(a8) % 8 == 0);
  dim3 grid(m), block(kThreads);
  void* args[] = {&a, &k, &lda, &a8, &lda8, &s_a};
  // hipLaunchKernel reports this launch's own status (the runtime's
  // last-error slot may hold an unrelated earlier error of the caller)
  const void* fn = reinterpret_cast<const void*>(&quant_act_kernel<false, 0>);
  if (vec) {
    const int chunks = (k + 8 * kThreads - 1) / (8 * kThreads);
    if (chunks <= 2) fn = reinterpret_cast<const void*>(&quant_act_kernel<true, 2>);
    else if (chunks <= 4) fn = reinterpret_cast<const void*>(&quant_act_kernel<true, 4>);
    else if (chunks <= 8) fn = reinterpret_cast<const void*>(&quant_act_kernel<true, 8>);
    else if (chunks <= 16) fn = reinterpret_cast<const void*>(&quant_act_kernel<true, 16>);
    else fn = reinterpret_cast<const void*>(&quant_act_kernel<true, 0>);
  }
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace w4a8
