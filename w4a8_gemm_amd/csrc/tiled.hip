// W4A8 GEMM for gfx950 (CDNA4): the tiled kernel for larger M.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"
#include "kernels.h"

namespace w4a8 {
namespace {

using namespace dev;

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
