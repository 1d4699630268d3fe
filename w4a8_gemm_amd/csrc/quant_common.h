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

// Maximum of x over the 64 lanes of a wave, in every lane, on the VALU's
// cross-lane paths (no LDS round trip): lane bits 5 and 4 by the permlane32 /
// permlane16 swaps (each leaves a lane and its partner's value in the two
// results), bits 3 .. 0 by DPP (row rotate by 8, half-row mirror, two quad
// permutes: partners that differ in that bit).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  const auto s32 = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  x = max(uint32_t(s32[0]), uint32_t(s32[1]));
  const auto s16 = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max(uint32_t(s16[0]), uint32_t(s16[1]));
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0u, x, 0x128, 0xF, 0xF, false)));
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0u, x, 0x141, 0xF, 0xF, false)));
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0u, x, 0x4E, 0xF, 0xF, false)));
  x = max(x, uint32_t(__builtin_amdgcn_update_dpp(0u, x, 0xB1, 0xF, 0xF, false)));
  return x;
}

// the multiplier fp32(1 / s_a), 0 for a zero row
__device__ __forceinline__ float act_recip(uint16_t scale_bits) {
  const float scale = h2f(scale_bits);
  return scale != 0.0f ? 1.0f / scale : 0.0f;
}

// int8 code of one half h under the multiplier r, as the low byte of the
// returned word: v = fp32(h * r) is clamped to +-127 (a median of three;
// clamping before rounding gives the same integer because the bounds are
// integers), then rounded half to even by adding 1.5 * 2^23.  The addition
// rounds its exact sum once, and fp32 values in [2^23, 2^24) are spaced 1
// apart, so the sum is 1.5 * 2^23 + rint(v) exactly and its low byte is
// rint(v) in two's complement.  The product is written as fma(h, r, +0):
// one rounding of the exact product, as a multiply, and the hardware folds
// the fp16 conversion into it (v_fma_mix_f32); a -0 product becomes +0,
// which gives the same code.  The rounding add stays a separate instruction
// (the library is built without contraction).
__device__ __forceinline__ uint32_t quant_byte(uint16_t h, float r) {
  const float v = __builtin_amdgcn_fmed3f(__builtin_fmaf(h2f(h), r, 0.0f), -127.0f, 127.0f);
  return __builtin_bit_cast(uint32_t, v + 12582912.0f);
}

__device__ __forceinline__ int quant1(uint16_t h, float r) {
  return int(int8_t(uint8_t(quant_byte(h, r) & 0xFFu)));
}

// four halves (two dwords) to four int8 in one dword: two byte permutes
// gather the low bytes of the four codes, a third merges the pairs
__device__ __forceinline__ uint32_t quant4(uint32_t h01, uint32_t h23, float r) {
  const uint32_t b0 = quant_byte(uint16_t(h01 & 0xFFFFu), r);
  const uint32_t b1 = quant_byte(uint16_t(h01 >> 16), r);
  const uint32_t b2 = quant_byte(uint16_t(h23 & 0xFFFFu), r);
  const uint32_t b3 = quant_byte(uint16_t(h23 >> 16), r);
  const uint32_t p01 = __builtin_amdgcn_perm(b1, b0, 0x0c0c0400u);   // b0.0, b1.0, 0, 0
  const uint32_t p23 = __builtin_amdgcn_perm(b3, b2, 0x04000c0cu);   // 0, 0, b2.0, b3.0
  return __builtin_amdgcn_perm(p23, p01, 0x07060100u);
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
