// Device-side pieces shared by the W4A8 GEMM kernels (gfx950): the
// in-register decode of 4-bit codes to int8 MFMA operands, fp16 helpers and
// the scale epilogue.
//
// The decode of 4-bit codes to the int8 MFMA operand happens in registers
// with integer operations only (the progressive-quantization point of the
// QServe/QoQ abstract; the LiquidGEMM digest, section "Метод", sets the bar
// of a couple of arithmetic operations per four weights).  Per 32-bit word of
// packed codes (eight weights):
//     lo = w & 0x0F0F0F0F,  hi = (w >> 4) & 0x0F0F0F0F        (4 codes each)
//     b  = pk_mad_u16(x, s2|s2<<16, c*0x01010101) ^ 0x80808080
// with c = 128 - z*s2.  Each byte of pk_mad is q*s2 + 128 - z*s2 =
// (q - z)*s2 + 128, which lies in [0, 255] because the packer guarantees the
// decoded weight is inside int8, so no carry crosses a byte and the xor turns
// the biased byte into the two's-complement int8 (q - z)*s2.  That is 7 VALU
// operations per 8 weights, plus 7 per lane and group for the constants.
//
// int8 MFMA v_mfma_i32_16x16x64_i8 accumulates exactly in int32 over all of K
// (no per-group rescale of partial sums, because s2 and z are folded into the
// int8 operand).  Operand mapping (lane l of a wave):
//   A (activations): row l % 16, k = kbase + 16*(l/16) + [0..15]
//   B (weights):     column l % 16, same k; both operands use the same k order
//   D:               lane l, register r holds row 4*(l/16) + r, column l % 16
//
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codebook.h"
#include "kernels.h"
#include "quant_common.h"

namespace w4a8 {
namespace dev {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// v_mul_i32_i24: the product of the low 24 bits of a and b, read as signed
// integers (the LLVM intrinsic, reached through its symbol name).  Exact when
// both factors lie in [-2^23, 2^23); a full-rate instruction, where a 32-bit
// multiply takes four issue cycles.
extern "C" __device__ int w4a8_mul_i24(int a, int b) __asm("llvm.amdgcn.mul.i24");

__device__ __forceinline__ uint32_t pk_mad_u16(uint32_t a, uint32_t b, uint32_t c) {
  u16x2 va = __builtin_bit_cast(u16x2, a);
  u16x2 vb = __builtin_bit_cast(u16x2, b);
  u16x2 vc = __builtin_bit_cast(u16x2, c);
  return __builtin_bit_cast(uint32_t, (u16x2)(va * vb + vc));
}

struct GroupConst {
  uint32_t s2s2;  // s2 in both 16-bit halves
  uint32_t cccc;  // (128 - z*s2) in all four bytes
};

// The constants of the group whose meta byte starts at bit `sh` of the
// dword m (low nibble z, high nibble s2 - 1): two bit-field extracts, two
// 24-bit multiply-adds (s2 = (s2 - 1) + 1 folded into both), a subtract
// and a byte splat.
__device__ __forceinline__ GroupConst group_const_at(uint32_t m, uint32_t sh) {
  const uint32_t s2m1 = __builtin_amdgcn_ubfe(m, sh + 4u, 4u);
  const uint32_t z = __builtin_amdgcn_ubfe(m, sh, 4u);
  GroupConst g;
  g.s2s2 = __umul24(s2m1, 0x10001u) + 0x10001u;            // s2 | s2 << 16
  const uint32_t zs2 = __umul24(z, s2m1) + z;               // z * s2
  g.cccc = __builtin_amdgcn_perm(0u, 128u - zs2, 0u);       // replicate byte 0
  return g;
}


__device__ __forceinline__ uint32_t dec4(uint32_t nibbles, GroupConst g) {
  return pk_mad_u16(nibbles, g.s2s2, g.cccc) ^ 0x80808080u;
}

// Two packed words (16 codes) -> one B operand (16 int8, k order j = 0..15).
__device__ __forceinline__ v4i decode16(uint32_t w0, uint32_t w1, GroupConst g) {
  v4i b;
  b[0] = int(dec4(w0 & 0x0F0F0F0Fu, g));
  b[1] = int(dec4((w0 >> 4) & 0x0F0F0F0Fu, g));
  b[2] = int(dec4(w1 & 0x0F0F0F0Fu, g));
  b[3] = int(dec4((w1 >> 4) & 0x0F0F0F0Fu, g));
  return b;
}

// Groups that cover whole MFMA steps (a 128-k block, a 64-k half, or the
// row) can be factored out of the inner product: the MFMA multiplies the raw
// codes q, and the group enters as s2 * (sum a * q - z * sum a), an integer
// identity with sum a * (q - z) * s2, so the int32 sums are the same.  The
// row sums of A come from an MFMA against a B operand of ones.

// Two packed words (16 codes) -> the raw codes as one B operand, in the k
// order of decode16.
__device__ __forceinline__ v4i codes16(uint32_t w0, uint32_t w1) {
  return v4i{int(w0 & 0x0F0F0F0Fu), int((w0 >> 4) & 0x0F0F0F0Fu), int(w1 & 0x0F0F0F0Fu),
             int((w1 >> 4) & 0x0F0F0F0Fu)};
}

// acc[0 .. NV) += s2 * (g - z * s) for the group of meta byte mb, in 24-bit
// products: valid while |s|, |g - z * s| < 2^23, i.e. for groups of up to
// 2048 k (|a|, q, z <= 127, 15, 15).
template <int NV>
__device__ __forceinline__ void add_group(v4i& acc, const v4i& g, const v4i& s, uint32_t mb) {
  const int s2 = int(mb >> 4) + 1, z = int(mb & 15u);
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] += w4a8_mul_i24(s2, g[i] - w4a8_mul_i24(z, s[i]));
}

// Epilogue scales of one lane, fetched at kernel start so that the final
// stores do not wait on a dependent global load.
template <int MR, int NC>
struct EpiScales {
  float s1[NC];      // column (tile0 + c) * 16 + lane % 16
  float sa[MR][4];   // rows (row_tile0 + i) * 16 + 4 * (lane / 16) + r
};

template <int MR, int NC>
__device__ __forceinline__ EpiScales<MR, NC> load_scales(const GemmParams& p, int row_tile0,
                                                         int tile0, int lane) {
  EpiScales<MR, NC> e;
#pragma unroll
  for (int c = 0; c < NC; ++c) e.s1[c] = h2f(p.s1[min((tile0 + c) * 16 + (lane & 15), p.n - 1)]);
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      e.sa[i][r] = h2f(p.s_a[min((row_tile0 + i) * 16 + 4 * (lane >> 4) + r, p.m - 1)]);
  return e;
}

// Store one 16x16 accumulator fragment (4 values per lane) with the epilogue
// Y = fp16((acc * s_a) * s1) in fp32.
__device__ __forceinline__ void store_frag(const GemmParams& p, int row0, int col0, int lane,
                                           const int32_t v[4], float s1, const float sa[4]) {
  const int col = col0 + (lane & 15);
  if (col >= p.n) return;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = row0 + 4 * (lane >> 4) + r;
    if (row < p.m) {
      const float y = (static_cast<float>(v[r]) * sa[r]) * s1;
      p.y[size_t(row) * p.ldy + col] = f2h_bits(y);
      if (p.acc) p.acc[size_t(row) * p.ldacc + col] = v[r];
    }
  }
}

// Codebook mode: four codes (one per byte, low 4 bits selected by `sel`,
// bit 3 by `pick`) to their int8 levels with three byte permutes: the low
// and high halves of the 16-entry table each give a candidate byte, and the
// code's bit 3 chooses between them.
//   sel  = code & 7 in every byte
//   pick = byte index i, plus 4 where the code's bit 3 is set
__device__ __forceinline__ uint32_t lut4(uint32_t sel, uint32_t pick) {
  const uint32_t lo = __builtin_amdgcn_perm(nf_dword(1), nf_dword(0), sel);   // levels 0..7
  const uint32_t hi = __builtin_amdgcn_perm(nf_dword(3), nf_dword(2), sel);   // levels 8..15
  return __builtin_amdgcn_perm(hi, lo, pick);
}

// Two packed words (16 codes) -> one B operand, codebook mode.
__device__ __forceinline__ v4i decode16_lut(uint32_t w0, uint32_t w1) {
  v4i b;
  b[0] = int(lut4(w0 & 0x07070707u, ((w0 >> 1) & 0x04040404u) | 0x03020100u));
  b[1] = int(lut4((w0 >> 4) & 0x07070707u, ((w0 >> 5) & 0x04040404u) | 0x03020100u));
  b[2] = int(lut4(w1 & 0x07070707u, ((w1 >> 1) & 0x04040404u) | 0x03020100u));
  b[3] = int(lut4((w1 >> 4) & 0x07070707u, ((w1 >> 5) & 0x04040404u) | 0x03020100u));
  return b;
}

}  // namespace dev
}  // namespace w4a8
