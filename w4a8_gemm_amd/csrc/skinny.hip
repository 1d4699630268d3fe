// W4A8 GEMM for gfx950 (CDNA4): the small-M (skinny) kernel.
//
// Y[m,n] = fp16(s_a[m] * s1[n] * sum_k A8[m,k] * W8^[n,k]),  W8^ = (q - z) * s2.
//
// For M <= 64 the layer is bound by streaming the packed weights from HBM
// (the FLUTE abstract: at small batch the cost is moving weights from global
// memory to registers).  One workgroup owns a few 16-column tiles over all
// of K, and its waves split K between them (split-K inside the workgroup);
// partial int32 tiles are summed exactly through LDS, so no workspace,
// atomics or second launch are needed.  Each wave streams its blocks through
// a register ring so that its 128-bit weight loads are always in flight.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"
#include "kernels.h"

namespace w4a8 {
namespace {

using namespace dev;

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
// GPB = groups per 128-k block (1, 2, 4 for g = 128, 64, 32; 0 per channel;
// -1 codebook mode: no meta, codes decode through the level table).
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

  // Epilogue scales: the column scales now; the row scales too, except for
  // 64-row tiles, whose 16 row scales per lane would stay live through the
  // whole K loop beside the ring: those load before the last ring group.
  EpiScales<MR, NC> es;
#pragma unroll
  for (int c = 0; c < NC; ++c) es.s1[c] = h2f(p.s1[min((tile0 + c) * 16 + (lane & 15), p.n - 1)]);
  auto load_row_scales = [&]() {
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        es.sa[i][r] = h2f(p.s_a[min((row_tile0 + i) * 16 + 4 * (lane >> 4) + r, p.m - 1)]);
  };
  constexpr bool kLateRowScales = MR > 2;
  if constexpr (!kLateRowScales) load_row_scales();

  v4i acc[MR][NC];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[i][c] = v4i{0, 0, 0, 0};

  // Ring slot j holds block kb0 + j.  kbw is a multiple of D = 4, so slot 0
  // always starts a meta dword; a dword covers MSTEP = 4 / GPB blocks, and
  // only the slots that start one load it (g = 128: one meta load per 4
  // blocks).  Meta loads land in mdn (next group) and become md (current
  // group) once the current group has been decoded, because the slots of a
  // group that share a dword are decoded after slot 0 has been refilled.
  constexpr int MSTEP = GPB <= 0 ? D : 4 / GPB;   // slots per meta dword
  u32x4 q[D][NC];
  uint32_t md[D][NC], mdn[D][NC];
  v4i a[D][MR][2];
  auto issue = [&](int j, int slot_kb) {
    const int kb = min(slot_kb, kb_last);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      q[j][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qptr[c] + size_t(kb) * 1024));
    if (GPB >= 0 && j % MSTEP == 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c) mdn[j][c] = mrow[c][GPB == 0 ? 0 : (kb * GPB) >> 2];
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
  auto next_group_meta = [&]() {
    if (GPB < 0) return;
#pragma unroll
    for (int j = 0; j < D; j += MSTEP)
#pragma unroll
      for (int c = 0; c < NC; ++c) md[j][c] = mdn[j][c];
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
        const uint32_t w0 = h ? qs[c].z : qs[c].x;
        const uint32_t w1 = h ? qs[c].w : qs[c].y;
        if constexpr (GPB < 0) {
          bf[c] = decode16_lut(w0, w1);
        } else {
          const GroupConst gc = group_const_at(ms[c], 8u * byte);
          bf[c] = decode16(w0, w1, gc);
        }
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
    next_group_meta();
    int kb0 = kb_begin;
    // steady state: D blocks in flight; every load is unconditional (clamped)
    for (; kb0 + D < kb_end; kb0 += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        compute(j, kb0 + j);
        issue(j, kb0 + D + j);
      }
      next_group_meta();
    }
    if constexpr (kLateRowScales) load_row_scales();
    // last group: no further loads
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (kb0 + j < kb_end) compute(j, kb0 + j);
  } else if constexpr (kLateRowScales) {
    load_row_scales();
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

template <int MR, int NC>
hipError_t skinny_by_gpb(const GemmParams& p, int gpb, const SkinnyConfig& c, hipStream_t s) {
  switch (gpb) {
    case -1: return launch_skinny<MR, NC, -1>(p, c, s);
    case 0: return launch_skinny<MR, NC, 0>(p, c, s);
    case 1: return launch_skinny<MR, NC, 1>(p, c, s);
    case 2: return launch_skinny<MR, NC, 2>(p, c, s);
    case 4: return launch_skinny<MR, NC, 4>(p, c, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

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

}  // namespace w4a8
