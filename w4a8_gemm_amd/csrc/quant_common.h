// Per-token activation quantization arithmetic shared by the standalone
// quantizer and the fused small-M GEMM, so that both produce identical bits.
//
// Reading (8-bit per-token activations of the QServe/QoQ abstract; per-token
// dynamic scaling as the PrefixQuant page's "Key Findings" describe it):
//   s_a = fp16(fp32(absmax / 127)),  A8 = clamp(rint(A * fp32(1 / s_a)), +-127)
// Both divisions are IEEE-correct fp32 divisions (HIP's default for '/'),
// conversions to fp16 and rint round half to even.  A zero row gives s_a = 0
// and A8 = 0.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {
namespace dev {

__device__ __forceinline__ float h2f(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ uint16_t f2h_bits(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

// lane-wise maximum of two pairs of 16-bit values
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
  u16x2_t va = __builtin_bit_cast(u16x2_t, a), vb = __builtin_bit_cast(u16x2_t, b);
  u16x2_t r = va > vb ? va : vb;
  return __builtin_bit_cast(uint32_t, r);
}

// running maximum of |h| over 8 halves (fp16 bit patterns with the sign
// cleared compare like the magnitudes for finite values)
__device__ __forceinline__ uint32_t absmax8(uint32_t mx, uint4 v) {
  mx = pk_max_u16(mx, v.x & 0x7FFF7FFFu);
  mx = pk_max_u16(mx, v.y & 0x7FFF7FFFu);
  mx = pk_max_u16(mx, v.z & 0x7FFF7FFFu);
  return pk_max_u16(mx, v.w & 0x7FFF7FFFu);
}

__device__ __forceinline__ uint32_t absmax_bits(uint32_t mx) { return max(mx & 0xFFFFu, mx >> 16); }

// s_a (fp16 bits) for a row whose largest |A| has fp16 bits amax_bits
__device__ __forceinline__ uint16_t act_scale_bits(uint32_t amax_bits) {
  const float amax = h2f(uint16_t(amax_bits));
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(amax / 127.0f));
}

// the multiplier fp32(1 / s_a), 0 for a zero row
__device__ __forceinline__ float act_recip(uint16_t scale_bits) {
  const float scale = h2f(scale_bits);
  return scale != 0.0f ? 1.0f / scale : 0.0f;
}

__device__ __forceinline__ int quant1(uint16_t h, float r) {
  float v = __builtin_rintf(h2f(h) * r);
  v = fminf(fmaxf(v, -127.0f), 127.0f);
  return static_cast<int>(v);
}

// four halves (two dwords) to four int8 in one dword
__device__ __forceinline__ uint32_t quant4(uint32_t h01, uint32_t h23, float r) {
  uint32_t b0 = uint32_t(quant1(uint16_t(h01 & 0xFFFFu), r)) & 0xFFu;
  uint32_t b1 = uint32_t(quant1(uint16_t(h01 >> 16), r)) & 0xFFu;
  uint32_t b2 = uint32_t(quant1(uint16_t(h23 & 0xFFFFu), r)) & 0xFFu;
  uint32_t b3 = uint32_t(quant1(uint16_t(h23 >> 16), r)) & 0xFFu;
  return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// eight halves to eight int8
__device__ __forceinline__ uint2 quant8(uint4 v, float r) {
  uint2 o;
  o.x = quant4(v.x, v.y, r);
  o.y = quant4(v.z, v.w, r);
  return o;
}

}  // namespace dev
}  // namespace w4a8
