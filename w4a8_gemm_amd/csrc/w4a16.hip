// W4A16 comparison GEMM for gfx950 (small M): the same packed 4-bit weights
// as the W4A8 path, decoded to fp16 and multiplied with fp16 activations on
// the fp16 MFMA, accumulating in fp32.
//
// This is the weight-only baseline the pages measure W4A8 against (the
// QServe/QoQ abstract's AWQ-style W4A16, the mixed-precision GEMMs of the
// QUICK abstract and the FLUTE page).  Reading used here, on the W4A8 blob:
//     W16^[n,k] = fp16(s1[n] * W8^[n,k]),   Y = fp16(sum_k A[m,k] * W16^[n,k])
// Decode: the integer step of the W4A8 decode yields the biased byte
// b = W8^ + 128 in [0, 255]; v_perm places it under the fp16 exponent of
// 1024 (0x64bb is 1024 + b), one packed fp16 add of -1152 leaves W8^ exactly,
// and one packed fp16 multiply by s1 rounds the product once.
//
// Work split as in the skinny W4A8 kernel: a workgroup owns NC column tiles
// over all of K, its waves split K and add their fp32 tiles through LDS in
// a fixed order; each wave streams its k-blocks through a 4-slot register
// ring.  MFMA: v_mfma_f32_16x16x32_f16; lane l holds row (A) or column (B)
// l % 16 and the 8 k values 64h + 16(l/16) + 8s + [0, 8) for half h and
// step s, the same k order on both operands.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"
#include "kernels.h"
#include "tile_common.h"

namespace w4a8 {
namespace {

using namespace dev;

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

// four biased bytes (b = W8^ + 128) -> four fp16 values fp16(s1 * W8^), as
// two packed halves (elements 0,1 and 2,3)
__device__ __forceinline__ void biased_to_f16(uint32_t b, v2h s1s1, uint32_t& lo, uint32_t& hi) {
  const v2h bias = {static_cast<_Float16>(-1152.0f), static_cast<_Float16>(-1152.0f)};
  v2h x = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, b, 0x04010400u));
  v2h y = __builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, b, 0x04030402u));
  x = (x + bias) * s1s1;
  y = (y + bias) * s1s1;
  lo = __builtin_bit_cast(uint32_t, x);
  hi = __builtin_bit_cast(uint32_t, y);
}

// one packed word (8 codes, k order j = 0..7 as laid out in the blob) ->
// the 8-element fp16 B operand
__device__ __forceinline__ v8h decode8_f16(uint32_t w, GroupConst g, v2h s1s1) {
  const uint32_t blo = pk_mad_u16(w & 0x0F0F0F0Fu, g.s2s2, g.cccc);          // j = 0..3
  const uint32_t bhi = pk_mad_u16((w >> 4) & 0x0F0F0F0Fu, g.s2s2, g.cccc);   // j = 4..7
  uint32_t r0, r1, r2, r3;
  biased_to_f16(blo, s1s1, r0, r1);
  biased_to_f16(bhi, s1s1, r2, r3);
  return __builtin_bit_cast(v8h, u32x4{r0, r1, r2, r3});
}

template <int MR, int NC, int GPB, int D>
__global__ __launch_bounds__(512) void w4a16_skinny_kernel(Gemm16Params p) {
  extern __shared__ float red16[];   // [KW][MR*NC][4][64]
  const int lane = threadIdx.x & 63;
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
  const int kb_last = max(kb_begin, kb_end - 1);

  const uint8_t* qptr[NC];
  const uint32_t* mrow[NC];
  v2h s1s1[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const int t = min(tile0 + c, ntiles - 1);
    qptr[c] = p.q + (size_t(t) * kblocks * 64 + lane) * 16;
    mrow[c] = reinterpret_cast<const uint32_t*>(p.meta + size_t(t * 16 + r16) * p.meta_row_bytes);
    const uint16_t s1 = p.s1[t * 16 + r16];
    s1s1[c] = __builtin_bit_cast(v2h, uint32_t(s1) | (uint32_t(s1) << 16));
  }
  const uint16_t* aptr[MR];
  bool arow_ok[MR];
#pragma unroll
  for (int i = 0; i < MR; ++i) {
    const int row = (row_tile0 + i) * 16 + r16;
    arow_ok[i] = row < p.m;
    aptr[i] = p.a + size_t(min(row, p.m - 1)) * p.lda + 16 * quarter;
  }

  v4f acc[MR][NC];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[i][c] = v4f{0.f, 0.f, 0.f, 0.f};

  constexpr int MSTEP = GPB == 0 ? D : 4 / GPB;
  u32x4 q[D][NC];
  uint32_t md[D][NC], mdn[D][NC];
  v8h a[D][MR][2][2];   // [slot][row tile][half h][step s]
  auto issue = [&](int j, int slot_kb) {
    const int kb = min(slot_kb, kb_last);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      q[j][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(qptr[c] + size_t(kb) * 1024));
    if (j % MSTEP == 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c) mdn[j][c] = mrow[c][GPB == 0 ? 0 : (kb * GPB) >> 2];
    }
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      if (arow_ok[i]) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int s = 0; s < 2; ++s)
            a[j][i][h][s] = *reinterpret_cast<const v8h*>(aptr[i] + kb * 128 + 64 * h + 8 * s);
      }
    }
  };
  auto next_group_meta = [&]() {
#pragma unroll
    for (int j = 0; j < D; j += MSTEP)
#pragma unroll
      for (int c = 0; c < NC; ++c) md[j][c] = mdn[j][c];
  };
  auto compute = [&](int j, int kb) {
    const u32x4 (&qs)[NC] = q[j];
    const uint32_t (&ms)[NC] = md[j - j % MSTEP];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int byte = 0;
      if (GPB == 1) byte = kb & 3;
      if (GPB == 2) byte = 2 * (kb & 1) + h;
      if (GPB == 4) byte = 2 * h + (quarter >> 1);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const GroupConst gc = group_const_at(ms[c], 8u * byte);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint32_t w = s ? (h ? qs[c].w : qs[c].y) : (h ? qs[c].z : qs[c].x);
          const v8h bf = decode8_f16(w, gc, s1s1[c]);
#pragma unroll
          for (int i = 0; i < MR; ++i)
            acc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j][i][h][s], bf, acc[i][c], 0, 0, 0);
        }
      }
    }
  };

  // rows past M never load: give their operand registers a defined value
#pragma unroll
  for (int j = 0; j < D; ++j)
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) a[j][i][h][0] = a[j][i][h][1] = v8h{};

  if (kb_begin < kb_end) {
#pragma unroll
    for (int j = 0; j < D; ++j) issue(j, kb_begin + j);
    next_group_meta();
    int kb0 = kb_begin;
    for (; kb0 + D < kb_end; kb0 += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        compute(j, kb0 + j);
        issue(j, kb0 + D + j);
      }
      next_group_meta();
    }
#pragma unroll
    for (int j = 0; j < D; ++j)
      if (kb0 + j < kb_end) compute(j, kb0 + j);
  }

  // fp32 partial tiles of the kw waves, added in wave order through LDS
  constexpr int F = MR * NC;
  auto store = [&](int i, int c, const float v[4]) {
    const int col = (tile0 + c) * 16 + r16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = (row_tile0 + i) * 16 + 4 * quarter + r;
      if (row < p.m) p.y[size_t(row) * p.ldy + col] = f2h_bits(v[r]);
    }
  };
  if (kw == 1) {
#pragma unroll
    for (int f = 0; f < F; ++f) {
      const int i = f / NC, c = f % NC;
      if (tile0 + c >= ntiles) continue;
      const float v[4] = {acc[i][c][0], acc[i][c][1], acc[i][c][2], acc[i][c][3]};
      store(i, c, v);
    }
    return;
  }
  float* mine = red16 + wk * F * 256;
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int r = 0; r < 4; ++r) mine[(f * 4 + r) * 64 + lane] = acc[f / NC][f % NC][r];
  __syncthreads();
  for (int f = wk; f < F; f += kw) {
    const int i = f / NC, c = f % NC;
    if (tile0 + c >= ntiles) continue;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    for (int w = 0; w < kw; ++w) {
      const float* part = red16 + (w * F + f) * 256;
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] += part[r * 64 + lane];
    }
    store(i, c, v);
  }
}

// ------------------------------------------------------------------ tiled
// Larger M: the fp16 MFMA becomes the bound, as in the W4A8 tiled kernel.
// A workgroup of 2 x 4 waves computes a 256 x 128 tile; wave (rg, cg) owns
// the 8 row tiles of row group rg and the 2 column tiles of column group cg.
// Each 128-k block's fp16 activation tile (256 rows x 256 bytes), weight
// codes and group meta go from HBM to LDS with direct-to-LDS buffer loads,
// two stages deep, one barrier per k-block.  The activation tile's 16-byte
// chunks are XOR-swizzled by row (16 chunks per row) so that the 16 rows a
// ds_read_b128 of a quarter-wave covers fall on distinct banks.
constexpr int kW16Rows = 256, kW16Cols = 128;

template <int GPB>
__global__ __launch_bounds__(512, 1) void w4a16_tiled_kernel(Gemm16Params p) {
  using namespace tile;
  constexpr int MR = 8, NC = 2, NW = 4, S = 2;
  constexpr int A_BYTES = kW16Rows * 256;            // 128 k of fp16 per row
  constexpr int W_BYTES = NW * NC * 1024;
  constexpr int M_BYTES = NW * NC * 256;
  constexpr int STAGE = A_BYTES + W_BYTES + M_BYTES;
  constexpr int CPW = A_BYTES / (16 * 512);          // activation chunks per lane
  constexpr int LOADS = CPW + 2;
  static_assert(S * STAGE <= 160 * 1024, "LDS");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cg = wave % NW;
  const int rg = wave / NW;
  const int quarter = lane >> 4;
  const int r16 = lane & 15;

  const int ntiles = p.n >> 4;
  const int kblocks = p.k >> 7;
  const int nbm = (p.m + kW16Rows - 1) / kW16Rows;
  const int nbn = (ntiles + NW * NC - 1) / (NW * NC);
  int bm, bn;
  tile_of(blockIdx.x, nbm, nbn, &bm, &bn);
  const int row0 = bm * kW16Rows;
  const int wtile0 = bn * NW * NC;                   // first column tile of the workgroup
  const int tile0 = wtile0 + cg * NC;                // first column tile of this wave

  // each wave loads the codes and meta of one of the workgroup's 8 tiles
  const int my_tile = min(wtile0 + wave, ntiles - 1);
  const __amdgpu_buffer_rsrc_t q_rsrc =
      make_rsrc(p.q + size_t(my_tile) * kblocks * 1024, uint32_t(kblocks) * 1024u);
  const __amdgpu_buffer_rsrc_t m_rsrc =
      make_rsrc(p.meta + size_t(my_tile) * 16 * p.meta_row_bytes, 16u * uint32_t(p.meta_row_bytes));
  const uint32_t q_lane = uint32_t(lane) * 16;
  const uint32_t m_lane = uint32_t(r16) * uint32_t(p.meta_row_bytes);
  const __amdgpu_buffer_rsrc_t a_rsrc =
      make_rsrc(p.a + size_t(row0) * p.lda, uint32_t(kW16Rows) * uint32_t(p.lda) * 2u);
  uint32_t a_lane[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int s = (wave * CPW + j) * 64 + lane;      // 16-byte slot of the LDS tile
    const int row = s >> 4;
    const int chunk = (s & 15) ^ (row & 15);
    a_lane[j] = (uint32_t(min(row0 + row, p.m - 1) - row0) * uint32_t(p.lda) + uint32_t(chunk * 8)) * 2u;
  }

  v4f acc[MR][NC];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[i][c] = v4f{0.f, 0.f, 0.f, 0.f};
  v2h s1s1[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const uint16_t s1 = p.s1[min((tile0 + c) * 16 + r16, p.n - 1)];
    s1s1[c] = __builtin_bit_cast(v2h, uint32_t(s1) | (uint32_t(s1) << 16));
  }

  auto issue = [&](int kb, int stage) {
    uint8_t* st = smem + stage * STAGE;
#pragma unroll
    for (int j = 0; j < CPW; ++j)
      buffer_to_lds16(a_rsrc, st + (wave * CPW + j) * 1024, a_lane[j], uint32_t(kb) * 256u);
    buffer_to_lds16(q_rsrc, st + A_BYTES + wave * 1024, q_lane, uint32_t(kb) * 1024u);
    buffer_to_lds4(m_rsrc, st + A_BYTES + W_BYTES + wave * 256, m_lane,
                   GPB == 0 ? 0u : uint32_t((kb * GPB) >> 2) * 4u);
  };
  auto compute = [&](int kb, const uint8_t* st) {
    u32x4 qv[NC];
    uint32_t mv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qv[c] = *reinterpret_cast<const u32x4*>(st + A_BYTES + (cg * NC + c) * 1024 + lane * 16);
      mv[c] = *reinterpret_cast<const uint32_t*>(st + A_BYTES + W_BYTES + (cg * NC + c) * 256 + lane * 4);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int byte = 0;
      if (GPB == 1) byte = kb & 3;
      if (GPB == 2) byte = 2 * (kb & 1) + h;
      if (GPB == 4) byte = 2 * h + (quarter >> 1);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        v8h af[MR];
        const int chunk = (8 * h + 2 * quarter + s) ^ r16;   // rows rg*128 + 16i + r16
#pragma unroll
        for (int i = 0; i < MR; ++i)
          af[i] = *reinterpret_cast<const v8h*>(st + (rg * 128 + i * 16 + r16) * 256 + chunk * 16);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const uint32_t w = s ? (h ? qv[c].w : qv[c].y) : (h ? qv[c].z : qv[c].x);
          const v8h bf = decode8_f16(w, group_const_at(mv[c], 8u * byte), s1s1[c]);
#pragma unroll
          for (int i = 0; i < MR; ++i)
            acc[i][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[i], bf, acc[i][c], 0, 0, 0);
        }
      }
    }
  };

  // stage k % 2 holds k-block k; the loads of k-block k + 1 go to the other
  // stage after the barrier that follows every wave's last read of it
  issue(0, 0);
  for (int k = 0; k < kblocks; ++k) {
    wait_vm<0>();                  // this wave's loads of k-block k have landed
    __builtin_amdgcn_s_barrier();
    if (k + 1 < kblocks) issue(k + 1, (k + 1) & 1);
    compute(k, smem + (k & 1) * STAGE);
  }

#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int col = (tile0 + c) * 16 + r16;
      if (tile0 + c >= ntiles) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + rg * 128 + i * 16 + 4 * quarter + r;
        if (row < p.m) p.y[size_t(row) * p.ldy + col] = f2h_bits(acc[i][c][r]);
      }
    }
}

template <int GPB>
hipError_t launch_w4a16_tiled_t(const Gemm16Params& p, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&w4a16_tiled_kernel<GPB>);
  const size_t lds = size_t(2) * (kW16Rows * 256 + 4 * 2 * (1024 + 256));
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  const int nbm = (p.m + kW16Rows - 1) / kW16Rows;
  const int nbn = (p.n / 16 + kW16Cols / 16 - 1) / (kW16Cols / 16);
  Gemm16Params arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, dim3(nbm * nbn), dim3(512), args, lds, stream);
}

template <int MR, int NC, int GPB>
hipError_t launch_w4a16_t(const Gemm16Params& p, const SkinnyConfig& c, hipStream_t stream) {
  constexpr int D = 4;
  const int ntiles = p.n / 16;
  dim3 grid((ntiles + NC - 1) / NC, (p.m + 16 * MR - 1) / (16 * MR));
  dim3 block(64 * c.kw);
  const size_t lds = c.kw > 1 ? size_t(c.kw) * MR * NC * 256 * sizeof(float) : 0;
  Gemm16Params arg = p;
  arg.kb_per_wave = c.kbw;
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(&w4a16_skinny_kernel<MR, NC, GPB, D>),
                         grid, block, args, lds, stream);
}

template <int MR, int NC>
hipError_t w4a16_by_gpb(const Gemm16Params& p, int gpb, const SkinnyConfig& c, hipStream_t s) {
  switch (gpb) {
    case 0: return launch_w4a16_t<MR, NC, 0>(p, c, s);
    case 1: return launch_w4a16_t<MR, NC, 1>(p, c, s);
    case 2: return launch_w4a16_t<MR, NC, 2>(p, c, s);
    case 4: return launch_w4a16_t<MR, NC, 4>(p, c, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_w4a16_tiled(const Gemm16Params& p, int gpb, hipStream_t stream) {
  switch (gpb) {
    case 0: return launch_w4a16_tiled_t<0>(p, stream);
    case 1: return launch_w4a16_tiled_t<1>(p, stream);
    case 2: return launch_w4a16_tiled_t<2>(p, stream);
    case 4: return launch_w4a16_tiled_t<4>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_w4a16_skinny(const Gemm16Params& p, int gpb, const SkinnyConfig& c,
                               hipStream_t stream) {
  if (c.mr != 1) return hipErrorInvalidValue;
  if (c.nc == 1) return w4a16_by_gpb<1, 1>(p, gpb, c, stream);
  if (c.nc == 2) return w4a16_by_gpb<1, 2>(p, gpb, c, stream);
  if (c.nc == 4) return w4a16_by_gpb<1, 4>(p, gpb, c, stream);
  return hipErrorInvalidValue;
}

}  // namespace w4a8
