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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

// Meta byte of group `grp` for a lane whose row pointer is mrow.
__device__ __forceinline__ uint32_t meta_byte(const uint8_t* mrow, int grp) {
  return mrow[grp];
}

// ---------------------------------------------------------------- skinny
// Small M (<= 64).  Workgroup = KW waves (KW = blockDim.x / 64) over NC
// column tiles and MR row tiles; wave wk owns the 128-k blocks
// [wk * kbw, (wk + 1) * kbw).  Each wave streams its blocks through a
// register ring of D slots: the loads of block b + D (weight codes, one meta
// dword, activations) are issued right after block b has been decoded and
// multiplied, so D blocks are always in flight and decode overlaps the
// memory stream.  Partial int32 tiles of the KW waves are summed exactly
// through LDS (split-K inside the workgroup: no workspace, no atomics).
//
// GPB = groups per 128-k block (1, 2, 4 for g = 128, 64, 32; 0 per channel).
// The meta dword loaded for block kb holds every group the block uses.
template <int MR, int NC, int GPB, int D>
__global__ __launch_bounds__(512) void skinny_kernel(GemmParams p) {
  extern __shared__ int32_t red[];  // [KW][MR*NC][4][64]
  const int lane = threadIdx.x & 63;
  // the wave index is uniform across the wave: keep it (and all the loop
  // control derived from it) in scalar registers
  const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = blockDim.x >> 6;
  const int quarter = lane >> 4;
  const int r16 = lane & 15;

  const int ntiles = p.n >> 4;
  const int kblocks = p.k >> 7;
  const int tile0 = blockIdx.x * NC;
  const int row_tile0 = blockIdx.y * MR;
  const int kb_begin = min(kblocks, wk * p.kb_per_wave);
  const int kb_end = min(kblocks, kb_begin + p.kb_per_wave);
  const int kb_last = max(kb_begin, kb_end - 1);   // loads past the end re-read this block

  const uint8_t* qptr[NC];
  const uint32_t* mrow[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int t = min(tile0 + c, ntiles - 1);
    qptr[c] = p.q + (size_t(t) * kblocks * 64 + lane) * 16;
    mrow[c] = reinterpret_cast<const uint32_t*>(p.meta + size_t(t * 16 + r16) * p.meta_row_bytes);
  }
  // lanes of rows past M skip their activation loads; the MFMA rows they
  // feed are never stored
  const int8_t* aptr[MR];
  bool arow_ok[MR];
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    const int row = (row_tile0 + i) * 16 + r16;
    arow_ok[i] = row < p.m;
    aptr[i] = p.a8 + size_t(min(row, p.m - 1)) * p.lda8 + 16 * quarter;
  }

  const EpiScales<MR, NC> es = load_scales<MR, NC>(p, row_tile0, tile0, lane);

  v4i acc[MR][NC];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[i][c] = v4i{0, 0, 0, 0};

  // Ring slot j holds block kb0 + j.  kbw is a multiple of D = 4, so slot 0
  // always starts a meta dword; a dword covers 4 / GPB blocks, and only the
  // slots that start one load it (g = 128: one meta load per 4 blocks).
  constexpr int MSTEP = GPB == 0 ? D : 4 / GPB;   // slots per meta dword
  u32x4 q[D][NC];
  uint32_t md[D][NC];
  v4i a[D][MR][2];
  auto issue = [&](int j, int slot_kb) {
    const int kb = min(slot_kb, kb_last);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      q[j][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qptr[c] + size_t(kb) * 1024));
    if (j % MSTEP == 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c) md[j][c] = mrow[c][GPB == 0 ? 0 : (kb * GPB) >> 2];
    }
    // only lanes that hold a real token row fetch activations
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      if (arow_ok[i]) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          a[j][i][h] = *reinterpret_cast<const v4i*>(aptr[i] + kb * 128 + 64 * h);
      }
    }
  };

  // decode block kb from ring slot j and multiply it into acc
  auto compute = [&](int j, int kb) {
    const u32x4 (&qs)[NC] = q[j];
    const uint32_t (&ms)[NC] = md[j - j % MSTEP];
    const v4i (&as)[MR][2] = a[j];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // byte of this lane's group inside the block's meta dword
      int byte = 0;
      if (GPB == 1) byte = kb & 3;
      if (GPB == 2) byte = 2 * (kb & 1) + h;
      if (GPB == 4) byte = 2 * h + (quarter >> 1);
      v4i bf[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const GroupConst gc = group_const((ms[c] >> (8 * byte)) & 0xFFu);
        const uint32_t w0 = h ? qs[c].z : qs[c].x;
        const uint32_t w1 = h ? qs[c].w : qs[c].y;
        bf[c] = decode16(w0, w1, gc);
      }
#pragma unroll
      for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          acc[i][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(as[i][h], bf[c], acc[i][c], 0, 0, 0);
    }
  };

  // rows past M never load: give their operand registers a defined value
#pragma unroll
  for (int j = 0; j < D; ++j)
#pragma unroll
    for (int i = 0; i < MR; ++i) a[j][i][0] = a[j][i][1] = v4i{0, 0, 0, 0};

  if (kb_begin < kb_end) {
#pragma unroll
    for (int j = 0; j < D; ++j) issue(j, kb_begin + j);
    int kb0 = kb_begin;
    // steady state: D blocks in flight; every load is unconditional (clamped)
    for (; kb0 + D < kb_end; kb0 += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        compute(j, kb0 + j);
        issue(j, kb0 + D + j);
      }
    }
    // last group: no further loads
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (kb0 + j < kb_end) compute(j, kb0 + j);
  }

  constexpr int F = MR * NC;
  if (kw == 1) {
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int i = f / NC, c = f % NC;
      if (tile0 + c >= ntiles) continue;
      int32_t v[4] = {acc[i][c][0], acc[i][c][1], acc[i][c][2], acc[i][c][3]};
      store_frag(p, (row_tile0 + i) * 16, (tile0 + c) * 16, lane, v, es.s1[c], es.sa[i]);
    }
    return;
  }
  // split-K inside the workgroup: exact int32 sum of the kw partial tiles
  int32_t* mine = red + wk * F * 256;
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) mine[(f * 4 + r) * 64 + lane] = acc[f / NC][f % NC][r];
  __syncthreads();
  for (int f = wk; f < F; f += kw) {
    const int i = f / NC, c = f % NC;
    if (tile0 + c >= ntiles) continue;
    int32_t v[4] = {0, 0, 0, 0};
    for (int w = 0; w < kw; ++w) {
      const int32_t* part = red + (w * F + f) * 256;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] += part[r * 64 + lane];
    }
    // f is wave-uniform but not a compile-time index: pick the scales out
    float s1 = es.s1[0];
    float sa[4] = {es.sa[0][0], es.sa[0][1], es.sa[0][2], es.sa[0][3]};
#pragma unroll
    for (int cc = 1; cc < NC; ++cc)
      if (cc == c) s1 = es.s1[cc];
#pragma unroll
    for (int ii = 1; ii < MR; ++ii)
      if (ii == i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) sa[r] = es.sa[ii][r];
      }
    store_frag(p, (row_tile0 + i) * 16, (tile0 + c) * 16, lane, v, s1, sa);
  }
}

// ---------------------------------------------------------------- tiled
// Larger M.  Workgroup = NW waves along N; wave wn owns column tiles
// [(bx*NW + wn)*NC, +NC) and row tiles [by*MR, +MR) over all of K, so no
// weight is decoded twice in a workgroup.
template <int MR, int NC, int NW, int GPB>
__global__ __launch_bounds__(64 * NW) void tiled_kernel(GemmParams p) {
  const int lane = threadIdx.x & 63;
  const int wn = threadIdx.x >> 6;
  const int quarter = lane >> 4;
  const int r16 = lane & 15;

  const int ntiles = p.n >> 4;
  const int kblocks = p.k >> 7;
  const int tile0 = (blockIdx.x * NW + wn) * NC;
  const int row_tile0 = blockIdx.y * MR;

  const uint8_t* qptr[NC];
  const uint8_t* mrow[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int t = min(tile0 + c, ntiles - 1);
    qptr[c] = p.q + (size_t(t) * kblocks * 64 + lane) * 16;
    mrow[c] = p.meta + size_t(t * 16 + r16) * p.meta_row_bytes;
  }
  const int8_t* aptr[MR];
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    const int row = min((row_tile0 + i) * 16 + r16, p.m - 1);
    aptr[i] = p.a8 + size_t(row) * p.lda8 + 16 * quarter;
  }

  const EpiScales<MR, NC> es = load_scales<MR, NC>(p, row_tile0, tile0, lane);

  v4i acc[MR][NC];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[i][c] = v4i{0, 0, 0, 0};

  uint4 qcur[NC];
  uint32_t mcur[2][NC];
  v4i acur[MR][2];
  auto load_block = [&](int kb, uint4 (&qv)[NC], uint32_t (&mv)[2][NC], v4i (&av)[MR][2]) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qv[c] = *reinterpret_cast<const uint4*>(qptr[c] + size_t(kb) * 1024);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kc = 64 * h + 16 * quarter;
        const int grp = GPB == 0 ? 0 : kb * GPB + ((kc * GPB) >> 7);
        mv[h][c] = meta_byte(mrow[c], grp);
      }
    }
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) av[i][h] = *reinterpret_cast<const v4i*>(aptr[i] + kb * 128 + 64 * h);
  };
  load_block(0, qcur, mcur, acur);
  for (int kb = 0; kb < kblocks; ++kb) {
    uint4 qnext[NC];
    uint32_t mnext[2][NC];
    v4i anext[MR][2];
    const bool more = kb + 1 < kblocks;
    if (more) load_block(kb + 1, qnext, mnext, anext);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4i bf[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint32_t w0 = h ? qcur[c].z : qcur[c].x;
        const uint32_t w1 = h ? qcur[c].w : qcur[c].y;
        bf[c] = decode16(w0, w1, group_const(mcur[h][c]));
      }
#pragma unroll
      for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          acc[i][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(acur[i][h], bf[c], acc[i][c], 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        qcur[c] = qnext[c];
        mcur[0][c] = mnext[0][c];
        mcur[1][c] = mnext[1][c];
      }
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        acur[i][0] = anext[i][0];
        acur[i][1] = anext[i][1];
      }
    }
  }
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (tile0 + c >= ntiles) continue;
      int32_t v[4] = {acc[i][c][0], acc[i][c][1], acc[i][c][2], acc[i][c][3]};
      store_frag(p, (row_tile0 + i) * 16, (tile0 + c) * 16, lane, v, es.s1[c], es.sa[i]);
    }
}

template <int MR, int NC, int GPB>
hipError_t launch_skinny(const GemmParams& p, const SkinnyConfig& c, hipStream_t stream) {
  constexpr int D = 4;
  const int ntiles = p.n / 16;
  dim3 grid((ntiles + NC - 1) / NC, (p.m + 16 * MR - 1) / (16 * MR));
  dim3 block(64 * c.kw);
  const size_t lds = c.kw > 1 ? size_t(c.kw) * MR * NC * 256 * sizeof(int32_t) : 0;
  GemmParams arg = p;
  arg.kb_per_wave = c.kbw;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&skinny_kernel<MR, NC, GPB, D>), grid,
                         block, args, lds, stream);
}

template <int MR, int NC, int GPB>
hipError_t launch_tiled_t(const GemmParams& p, hipStream_t stream) {
  constexpr int NW = 4;
  const int ntiles = p.n / 16;
  dim3 grid((ntiles + NW * NC - 1) / (NW * NC), (p.m + 16 * MR - 1) / (16 * MR));
  dim3 block(64 * NW);
  GemmParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&tiled_kernel<MR, NC, NW, GPB>), grid,
                         block, args, 0, stream);
}

template <int MR, int NC>
hipError_t skinny_by_gpb(const GemmParams& p, int gpb, const SkinnyConfig& c, hipStream_t s) {
  switch (gpb) {
    case 0: return launch_skinny<MR, NC, 0>(p, c, s);
    case 1: return launch_skinny<MR, NC, 1>(p, c, s);
    case 2: return launch_skinny<MR, NC, 2>(p, c, s);
    case 4: return launch_skinny<MR, NC, 4>(p, c, s);
  }
  return hipErrorInvalidValue;
}

template <int MR, int NC>
hipError_t tiled_by_gpb(const GemmParams& p, int gpb, hipStream_t s) {
  switch (gpb) {
    case 0: return launch_tiled_t<MR, NC, 0>(p, s);
    case 1: return launch_tiled_t<MR, NC, 1>(p, s);
    case 2: return launch_tiled_t<MR, NC, 2>(p, s);
    case 4: return launch_tiled_t<MR, NC, 4>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool skinny_config_supported(const SkinnyConfig& c, int k, int gpb) {
  const bool shape_ok = (c.mr == 1 && (c.nc == 1 || c.nc == 2 || c.nc == 4)) ||
                        ((c.mr == 2 || c.mr == 4) && (c.nc == 1 || c.nc == 2));
  if (!shape_ok) return false;
  (void)gpb;
  if (c.kw < 1 || c.kw > 8 || c.kbw < 1 || c.kbw % 4) return false;   // ring groups of 4
  return c.kw * c.kbw * 128 >= k;                    // the waves cover all of K
}

hipError_t launch_gemm_skinny(const GemmParams& p, int gpb, const SkinnyConfig& c,
                              hipStream_t stream) {
  if (c.mr == 1 && c.nc == 1) return skinny_by_gpb<1, 1>(p, gpb, c, stream);
  if (c.mr == 1 && c.nc == 2) return skinny_by_gpb<1, 2>(p, gpb, c, stream);
  if (c.mr == 1 && c.nc == 4) return skinny_by_gpb<1, 4>(p, gpb, c, stream);
  if (c.mr == 2 && c.nc == 1) return skinny_by_gpb<2, 1>(p, gpb, c, stream);
  if (c.mr == 2 && c.nc == 2) return skinny_by_gpb<2, 2>(p, gpb, c, stream);
  if (c.mr == 4 && c.nc == 1) return skinny_by_gpb<4, 1>(p, gpb, c, stream);
  if (c.mr == 4 && c.nc == 2) return skinny_by_gpb<4, 2>(p, gpb, c, stream);
  return hipErrorInvalidValue;
}

bool tiled_config_supported(const TiledConfig& c) {
  return c.mr == 4 && (c.nc == 4 || c.nc == 2) && c.nw == 4;
}

hipError_t launch_gemm_tiled(const GemmParams& p, int gpb, const TiledConfig& c,
                             hipStream_t stream) {
  if (c.mr == 4 && c.nc == 4 && c.nw == 4) return tiled_by_gpb<4, 4>(p, gpb, stream);
  if (c.mr == 4 && c.nc == 2 && c.nw == 4) return tiled_by_gpb<4, 2>(p, gpb, stream);
  return hipErrorInvalidValue;
}

}  // namespace w4a8
