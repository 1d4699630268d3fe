// W4A8 GEMM kernels for gfx950 (CDNA4).
//
// Y[m,n] = fp16(s_a[m] * s1[n] * sum_k A8[m,k] * W8^[n,k]),  W8^ = (q - z) * s2.
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
// Variants
//   skinny: for small M (<= 64).  One workgroup owns a few 16-column tiles
//     over all of K, and its waves split K between them (split-K inside the
//     workgroup); partial int32 tiles are summed exactly through LDS, so no
//     workspace, atomics or second launch are needed.  Every wave issues its
//     128-bit weight loads early, which is what the memory-bound regime
//     needs (the FLUTE abstract: at small batch the cost is moving weights
//     from global memory to registers).
//   tiled: for larger M.  Waves of a workgroup own disjoint column slices
//     and all rows of the tile, so no weight is decoded twice in a
//     workgroup.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace w4a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

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

__device__ __forceinline__ GroupConst group_const(uint32_t mb) {
  GroupConst g;
  uint32_t s2 = (mb >> 4) + 1u;
  uint32_t z = mb & 15u;
  g.s2s2 = s2 | (s2 << 16);
  uint32_t c = 128u - __umul24(z, s2);
  g.cccc = __builtin_amdgcn_perm(0u, c, 0u);  // replicate byte 0
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

__device__ __forceinline__ uint16_t f2h_bits(float v) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(v));
}

__device__ __forceinline__ float h2f(uint16_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, h));
}

// Group index of the 16-k chunk starting at kchunk (a multiple of 16).
__device__ __forceinline__ int group_of(int kchunk, int gpb_shift) {
  // g in {128, 64, 32}: 1, 2 or 4 groups per 128-k block; per channel: 0
  return gpb_shift < 0 ? 0 : ((kchunk >> 7) << gpb_shift) + ((kchunk & 127) >> (7 - gpb_shift));
}

// Store one 16x16 accumulator fragment (4 values per lane) with the epilogue.
__device__ __forceinline__ void store_frag(const GemmParams& p, int row0, int col0, int lane,
                                           const int32_t v[4]) {
  const int col = col0 + (lane & 15);
  if (col >= p.n) return;
  const float s1 = h2f(p.s1[col]);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = row0 + 4 * (lane >> 4) + r;
    if (row < p.m) {
      const float sa = h2f(p.s_a[row]);
      const float y = (static_cast<float>(v[r]) * sa) * s1;
      p.y[size_t(row) * p.ldy + col] = f2h_bits(y);
      if (p.acc) p.acc[size_t(row) * p.ldacc + col] = v[r];
    }
  }
}

// One kernel template for both variants.  Workgroup = NW x KW waves:
//   wave (wn, wk) owns column tiles [(bx*NW + wn)*NC, +NC) and row tiles
//   [by*MR, +MR) and the wk-th share of the 128-k blocks.
template <int MR, int NC, int NW, int KW>
__global__ __launch_bounds__(64 * NW * KW) void gemm_kernel(GemmParams p) {
  extern __shared__ int32_t red[];  // KW > 1: [KW][NW][MR*NC][4][64]
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wn = wave % NW;
  const int wk = wave / NW;
  const int quarter = lane >> 4;
  const int r16 = lane & 15;

  const int ntiles = p.n >> 4;
  const int kblocks = p.k >> 7;
  const int tile0 = (blockIdx.x * NW + wn) * NC;
  const int row_tile0 = blockIdx.y * MR;

  // k-block range of this wave
  const int kb0 = (kblocks * wk) / KW;
  const int kb1 = (kblocks * (wk + 1)) / KW;

  // per-column-tile base pointers (tiles past the end are clamped for loads)
  const uint8_t* qptr[NC];
  const uint8_t* mptr[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    int t = min(tile0 + c, ntiles - 1);
    qptr[c] = p.q + (size_t(t) * kblocks * 64 + lane) * 16;
    mptr[c] = p.meta + size_t(t) * p.groups * 16 + r16;
  }
  const int8_t* aptr[MR];
  bool arow_ok[MR];
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    int row = (row_tile0 + i) * 16 + r16;
    arow_ok[i] = row < p.m;
    aptr[i] = p.a8 + size_t(arow_ok[i] ? row : 0) * p.lda8 + 16 * quarter;
  }

  v4i acc[MR][NC];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[i][c] = v4i{0, 0, 0, 0};

  uint4 qcur[NC];
  v4i acur[MR][2];
  if (kb0 < kb1) {
#pragma unroll
    for (int c = 0; c < NC; ++c) qcur[c] = *reinterpret_cast<const uint4*>(qptr[c] + size_t(kb0) * 1024);
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        acur[i][h] = arow_ok[i] ? *reinterpret_cast<const v4i*>(aptr[i] + kb0 * 128 + 64 * h)
                                : v4i{0, 0, 0, 0};
  }

  for (int kb = kb0; kb < kb1; ++kb) {
    // prefetch the next block while this one is decoded and multiplied
    uint4 qnext[NC];
    v4i anext[MR][2];
    const bool more = kb + 1 < kb1;
    if (more) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        qnext[c] = *reinterpret_cast<const uint4*>(qptr[c] + size_t(kb + 1) * 1024);
#pragma unroll
      for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          anext[i][h] = arow_ok[i]
                            ? *reinterpret_cast<const v4i*>(aptr[i] + (kb + 1) * 128 + 64 * h)
                            : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int grp = group_of(kb * 128 + 64 * h + 16 * quarter, p.gpb_shift);
      v4i b[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const GroupConst gc = group_const(mptr[c][grp * 16]);
        const uint32_t w0 = h ? qcur[c].z : qcur[c].x;
        const uint32_t w1 = h ? qcur[c].w : qcur[c].y;
        b[c] = decode16(w0, w1, gc);
      }
#pragma unroll
      for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          acc[i][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(acur[i][h], b[c], acc[i][c], 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int c = 0; c < NC; ++c) qcur[c] = qnext[c];
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        acur[i][0] = anext[i][0];
        acur[i][1] = anext[i][1];
      }
    }
  }

  if (KW == 1) {
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (tile0 + c >= ntiles) continue;
        int32_t v[4] = {acc[i][c][0], acc[i][c][1], acc[i][c][2], acc[i][c][3]};
        store_frag(p, (row_tile0 + i) * 16, (tile0 + c) * 16, lane, v);
      }
    return;
  }

  // split-K inside the workgroup: exact int32 sum of the KW partial tiles
  constexpr int F = MR * NC;
  int32_t* mine = red + ((wk * NW + wn) * F) * 256;
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) mine[(f * 4 + r) * 64 + lane] = acc[f / NC][f % NC][r];
  __syncthreads();
  for (int f = wk; f < F; f += KW) {
    const int i = f / NC, c = f % NC;
    if (tile0 + c >= ntiles) continue;
    int32_t v[4] = {0, 0, 0, 0};
    for (int w = 0; w < KW; ++w) {
      const int32_t* part = red + ((w * NW + wn) * F + f) * 256;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] += part[r * 64 + lane];
    }
    store_frag(p, (row_tile0 + i) * 16, (tile0 + c) * 16, lane, v);
  }
}

template <int MR, int NC, int NW, int KW>
hipError_t launch(const GemmParams& p, hipStream_t stream) {
  const int ntiles = p.n / 16;
  dim3 grid((ntiles + NW * NC - 1) / (NW * NC), (p.m + 16 * MR - 1) / (16 * MR));
  dim3 block(64 * NW * KW);
  size_t lds = KW > 1 ? size_t(KW) * NW * MR * NC * 256 * sizeof(int32_t) : 0;
  GemmParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&gemm_kernel<MR, NC, NW, KW>), grid, block,
                         args, lds, stream);
}

}  // namespace

#define W4A8_SKINNY_CASE(MR, NC, KW)                          \
  if constexpr (KW * MR * NC <= 64) {                         \
    if (c.mr == MR && c.nc == NC && c.kw == KW) return launch<MR, NC, 1, KW>(p, stream); \
  }

#define W4A8_SKINNY_KW(MR, NC) \
  W4A8_SKINNY_CASE(MR, NC, 1)  \
  W4A8_SKINNY_CASE(MR, NC, 2)  \
  W4A8_SKINNY_CASE(MR, NC, 4)  \
  W4A8_SKINNY_CASE(MR, NC, 8)  \
  W4A8_SKINNY_CASE(MR, NC, 16)

hipError_t launch_gemm_skinny(const GemmParams& p, const SkinnyConfig& c, hipStream_t stream) {
  W4A8_SKINNY_KW(1, 1)
  W4A8_SKINNY_KW(1, 2)
  W4A8_SKINNY_KW(1, 4)
  W4A8_SKINNY_KW(2, 1)
  W4A8_SKINNY_KW(2, 2)
  W4A8_SKINNY_KW(4, 1)
  W4A8_SKINNY_KW(4, 2)
  return hipErrorInvalidValue;
}

bool skinny_config_supported(const SkinnyConfig& c) {
  const bool kw_ok = c.kw == 1 || c.kw == 2 || c.kw == 4 || c.kw == 8 || c.kw == 16;
  const bool shape_ok = (c.mr == 1 && (c.nc == 1 || c.nc == 2 || c.nc == 4)) ||
                        (c.mr == 2 && (c.nc == 1 || c.nc == 2)) ||
                        (c.mr == 4 && (c.nc == 1 || c.nc == 2));
  // partial tiles of all waves must fit in 64 KiB of LDS
  const bool lds_ok = c.kw * c.mr * c.nc <= 64;
  return kw_ok && shape_ok && lds_ok;
}

hipError_t launch_gemm_tiled(const GemmParams& p, const TiledConfig& c, hipStream_t stream) {
  if (c.mr == 4 && c.nc == 4 && c.nw == 4) return launch<4, 4, 4, 1>(p, stream);
  if (c.mr == 4 && c.nc == 2 && c.nw == 4) return launch<4, 2, 4, 1>(p, stream);
  return hipErrorInvalidValue;
}

bool tiled_config_supported(const TiledConfig& c) {
  return c.mr == 4 && (c.nc == 4 || c.nc == 2) && c.nw == 4;
}

}  // namespace w4a8
