// W4A8 GEMM for gfx950 (CDNA4): the tiled kernel for larger M.
//
// Y[m,n] = fp16(s_a[m] * s1[n] * sum_k A8[m,k] * W8^[n,k]),  W8^ = (q - z) * s2.
//
// Once M reaches a few hundred tokens the layer is bound by the int8 MFMA
// rate, and the cost that progressive quantization targets (the QServe/QoQ
// abstract: dequantization on the slow general-purpose cores) is the decode
// of the 4-bit codes.  The tiling keeps that decode cheap:
//
//  * A workgroup of RW x 4 waves computes a BM x BN tile, BM = RW * 16 * MR
//    rows and BN = 4 * NC * 16 columns.  Wave (rg, cg) owns the MR row tiles
//    of row group rg and the NC column tiles of column group cg, so each
//    weight code is decoded RW times per workgroup and each decoded operand
//    feeds MR MFMAs.  RW = 2 (eight waves, 256 x 256 tiles, one workgroup per
//    compute unit) moves 28 % fewer bytes per MFMA through the vector memory
//    path than two RW = 1 workgroups of 128 x 256; it runs as the ping-pong
//    kernel tiled_pp_kernel, its two row groups taking turns at the MFMAs.
//  * Everything a k-block needs (the activation tile, the weight codes and
//    their group meta) goes from HBM to LDS with direct-to-LDS 128-bit buffer
//    loads, S stages deep, with one barrier per k-block.  The weight codes
//    already sit in the MFMA B-operand order (the offline interleaving of the
//    QUICK abstract), so a wave reads its codes with one ds_read_b128 per
//    column tile.  The activation tile's 16-byte chunks are XOR-swizzled by
//    row so that the ds_read_b128 operand reads of 16 consecutive rows do not
//    collide on LDS banks.
//  * Workgroups are mapped to tiles XCD by XCD, and within an XCD in groups
//    of kGroupM row tiles, so that the workgroups resident on one XCD at the
//    same time share weight columns and activation rows in that XCD's L2.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.h"
#include "kernels.h"
#include "tile_common.h"

namespace w4a8 {
namespace {

using namespace dev;
using namespace tile;

constexpr int kColGroups = kTiledColGroups;   // waves along N per workgroup
constexpr int kTiledMaxLds = 160 * 1024;   // LDS of one gfx950 compute unit

// One LDS stage: for each of the KG k-groups, the activation tile, weight
// codes and meta of one k-block.
template <int MR, int NC, int RW, int KG>
constexpr int tiled_stage_bytes() {
  return KG * (RW * 16 * MR * 128 + kColGroups * NC * (1024 + 256));
}

// RW row groups x KG k-groups x 4 column groups of waves.  With KG = 2 the
// two k-groups take alternate k-blocks of the same tile (an exact split of
// K inside the workgroup) and add their int32 tiles through LDS at the end.
template <int MR, int NC, int RW, int KG, int GPB, int S>
__global__ __launch_bounds__(64 * kColGroups * RW * KG, 2 / (RW * KG)) void tiled_kernel(
    GemmParams p) {
  static_assert(RW * KG <= 2, "at most eight waves (two per SIMD)");
  constexpr int NW = kColGroups;
  constexpr int KWAVES = NW * RW;                // waves of one k-group
  constexpr int BM = RW * 16 * MR;
  constexpr int A_BYTES = BM * 128;              // activation tile of one k-block
  constexpr int W_BYTES = NW * NC * 1024;        // weight codes of one k-block
  constexpr int M_BYTES = NW * NC * 256;         // meta dwords of one k-block
  constexpr int SUB = A_BYTES + W_BYTES + M_BYTES;
  constexpr int STAGE = KG * SUB;
  static_assert(STAGE == tiled_stage_bytes<MR, NC, RW, KG>(), "stage layout");
  constexpr int CPW = BM * 8 / (64 * KWAVES);    // activation chunks per lane
  constexpr int NCL = NC / RW;                   // column tiles whose codes this wave loads
  // vector-memory ops per lane per stage (codebook mode, GPB < 0: no meta)
  constexpr int LOADS = CPW + (GPB < 0 ? 1 : 2) * NCL;
  static_assert(CPW >= 1 && BM * 8 % (64 * KWAVES) == 0, "tile must split evenly over lanes");
  static_assert(NCL >= 1 && NC % RW == 0, "code loads split evenly over row groups");
  static_assert(S >= 2 && (S - 2) * LOADS < 64, "vmcnt range");
  static_assert(KG == 1 || S * STAGE >= KWAVES * MR * NC * 1024, "LDS holds the k-group sum");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];   // S stages

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cg = wave % NW;                      // column group
  const int rg = (wave / NW) % RW;               // row group
  const int kg = wave / KWAVES;                  // k-group
  const int wk = wave % KWAVES;                  // wave inside its k-group
  const int quarter = lane >> 4;
  const int r16 = lane & 15;

  const int ntiles = p.n >> 4;
  const int kblocks = p.k >> 7;
  const int nbm = (p.m + BM - 1) / BM;
  const int nbn = (ntiles + NW * NC - 1) / (NW * NC);
  // K slice of this workgroup: k-blocks [kb0, kb1)
  const int slice = blockIdx.x / (nbm * nbn);
  const int kb0 = slice * p.kb_per_slice;
  const int kb1 = min(kblocks, kb0 + p.kb_per_slice);
  int bm, bn;
  tile_of(blockIdx.x - slice * (nbm * nbn), nbm, nbn, &bm, &bn);
  const int row0 = bm * BM;
  const int tile0 = (bn * NW + cg) * NC;

  // Loads go through buffer resources: the base is wave-uniform (scalar
  // registers), each lane adds one fixed 32-bit offset and each k-block one
  // scalar offset, so issuing a load costs no vector arithmetic.  Offsets
  // past a resource's size would read 0; every offset below is in range.
  const int tlo = min(tile0, ntiles - 1);
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(
      p.q + size_t(tlo) * kblocks * 1024, uint32_t(NC) * uint32_t(kblocks) * 1024u);
  const __amdgpu_buffer_rsrc_t m_rsrc = make_rsrc(
      p.meta + size_t(tlo) * 16 * p.meta_row_bytes, uint32_t(NC) * 16u * uint32_t(p.meta_row_bytes));
  const uint32_t q_lane = uint32_t(lane) * 16;
  const uint32_t m_lane = uint32_t(r16) * uint32_t(p.meta_row_bytes);
  // this wave loads the codes and meta of column tiles rg * NCL + [0, NCL)
  // of its column group (clamped); the other row groups load the rest
  uint32_t q_tile[NCL], m_tile[NCL];
#pragma unroll
  for (int c = 0; c < NCL; ++c) {
    const int t = min(tile0 + rg * NCL + c, ntiles - 1) - tlo;
    q_tile[c] = uint32_t(t) * uint32_t(kblocks) * 1024u;
    m_tile[c] = uint32_t(t) * 16u * uint32_t(p.meta_row_bytes);
  }
  // Activation tile: instruction j of this wave fills 16-byte slots
  // [(wk * CPW + j) * 64, +64); slot s holds row s / 8, physical chunk
  // s % 8, i.e. logical chunk (s % 8) ^ (row % 8).  Offsets are relative to
  // row0 (rows past M read row M - 1, whose results are never stored).
  const __amdgpu_buffer_rsrc_t a_rsrc =
      make_rsrc(p.a8 + size_t(row0) * p.lda8, uint32_t(BM) * uint32_t(p.lda8));
  uint32_t a_lane[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int s = (wk * CPW + j) * 64 + lane;
    const int row = s >> 3;
    const int lchunk = (s & 7) ^ (row & 7);
    a_lane[j] = uint32_t(min(row0 + row, p.m - 1) - row0) * uint32_t(p.lda8) + uint32_t(lchunk * 16);
  }
  // operand reads: row (rg * MR + i) * 16 + r16, logical chunk 4h + quarter
  int a_off[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    a_off[h] = kg * SUB + rg * (16 * MR * 128) + r16 * 128 +
               (((4 * h + quarter) ^ (r16 & 7)) * 16);
  // the weight codes and meta of this wave's column group inside a stage
  // (lane-linear, as loaded)
  const int w_off = kg * SUB + A_BYTES + cg * NC * 1024 + lane * 16;
  const int m_off = kg * SUB + A_BYTES + W_BYTES + cg * NC * 256 + lane * 4;

  v4i acc[MR][NC];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[i][c] = v4i{0, 0, 0, 0};

  // every load of k-block kb goes straight to this k-group's part of LDS
  // stage `stage`
  auto issue = [&](int kb, int stage) {
    uint8_t* st = smem + stage * STAGE + kg * SUB;
#pragma unroll
    for (int j = 0; j < CPW; ++j)
      buffer_to_lds16(a_rsrc, st + (wk * CPW + j) * 1024, a_lane[j], uint32_t(kb) * 128u);
#pragma unroll
    for (int c = 0; c < NCL; ++c)
      buffer_to_lds16(q_rsrc, st + A_BYTES + (cg * NC + rg * NCL + c) * 1024, q_lane,
                      q_tile[c] + uint32_t(kb) * 1024u);
    if (GPB >= 0) {
#pragma unroll
      for (int c = 0; c < NCL; ++c)
        buffer_to_lds4(m_rsrc, st + A_BYTES + W_BYTES + (cg * NC + rg * NCL + c) * 256, m_lane,
                       m_tile[c] + (GPB == 0 ? 0u : uint32_t((kb * GPB) >> 2) * 4u));
    }
  };

  auto compute = [&](int kb, const uint8_t* st) {
    u32x4 qv[NC];
    uint32_t mv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qv[c] = *reinterpret_cast<const u32x4*>(st + w_off + c * 1024);
      mv[c] = GPB >= 0 ? *reinterpret_cast<const uint32_t*>(st + m_off + c * 256) : 0u;
    }
    // g >= 128 or per channel: both halves of the block share one group
    GroupConst gblk[NC];
    if (GPB >= 0 && GPB <= 1) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        gblk[c] = group_const_at(mv[c], GPB == 1 ? 8u * (kb & 3) : 0u);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int byte = 0;
      if (GPB == 2) byte = 2 * (kb & 1) + h;
      if (GPB == 4) byte = 2 * h + (quarter >> 1);
      v4i bf[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint32_t w0 = h ? qv[c].z : qv[c].x;
        const uint32_t w1 = h ? qv[c].w : qv[c].y;
        if constexpr (GPB < 0) {
          bf[c] = decode16_lut(w0, w1);
        } else {
          const GroupConst gc =
              GPB <= 1 ? gblk[c] : group_const_at(mv[c], 8u * byte);
          bf[c] = decode16(w0, w1, gc);
        }
      }
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        const v4i af = *reinterpret_cast<const v4i*>(st + i * 16 * 128 + a_off[h]);
#pragma unroll
        for (int c = 0; c < NC; ++c)
          acc[i][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[c], acc[i][c], 0, 0, 0);
      }
    }
  };

  // Pipeline of depth S - 1 over super-blocks of KG k-blocks (k-group kg
  // takes k-block kb0 + sb * KG + kg): at iteration sb the loads of super-blocks
  // sb + 1 .. sb + S - 2 are in flight; super-block sb + S - 1 is issued
  // into the stage that iteration sb - 1 consumed, after the barrier that
  // proves every wave is done with it.  Loads past the end re-read the last
  // k-block into a part of a stage whose results are never used, so the
  // loop has no branch around the loads.
  const int nsb = (kb1 - kb0 + KG - 1) / KG;
#pragma unroll
  for (int j = 0; j < S - 1; ++j) issue(min(kb0 + j * KG + kg, kb1 - 1), j);
  for (int sb = 0; sb < nsb; ++sb) {
    wait_vm<(S - 2) * LOADS>();    // this wave's loads of super-block sb have landed
    __builtin_amdgcn_s_barrier();  // ... and every other wave's share of the tile
    issue(min(kb0 + (sb + S - 1) * KG + kg, kb1 - 1), (sb + S - 1) % S);
    const int kb = kb0 + sb * KG + kg;
    if (KG == 1 || kb < kb1) compute(kb, smem + (sb % S) * STAGE);
  }
  wait_vm<0>();                    // no LDS write still in flight at exit

  if (KG == 2) {
    // k-group 1 hands its int32 tile to k-group 0 through LDS (exact sum)
    __syncthreads();               // every wave is done reading the stages
    v4i* red = reinterpret_cast<v4i*>(smem) + wk * (MR * NC * 64) + lane;
    if (kg == 1) {
#pragma unroll
      for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int c = 0; c < NC; ++c) red[(i * NC + c) * 64] = acc[i][c];
    }
    __syncthreads();
    if (kg == 1) return;
  }

  // scales are fetched only now: this kernel runs long enough that one
  // more round trip at the end does not matter, and keeping them live
  // through the K loop would cost registers
  const int rt0 = row0 / 16 + rg * MR;           // first row tile of this wave
  if (p.part) {
    // K split over workgroups: raw partial sums, added by split_reduce_kernel
    int32_t* part = p.part + size_t(slice) * size_t(p.m) * size_t(p.n);
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int col = (tile0 + c) * 16 + r16;
        if (tile0 + c >= ntiles) continue;
        v4i t = acc[i][c];
        if (KG == 2)
          t += reinterpret_cast<const v4i*>(smem)[wk * (MR * NC * 64) + (i * NC + c) * 64 + lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = (rt0 + i) * 16 + 4 * quarter + r;
          if (row < p.m) part[size_t(row) * p.n + col] = t[r];
        }
      }
    return;
  }
  const EpiScales<MR, NC> es = load_scales<MR, NC>(p, rt0, tile0, lane);
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (tile0 + c >= ntiles) continue;
      v4i t = acc[i][c];
      if (KG == 2)   // plus k-group 1's share, left in LDS above
        t += reinterpret_cast<const v4i*>(smem)[wk * (MR * NC * 64) + (i * NC + c) * 64 + lane];
      int32_t v[4] = {t[0], t[1], t[2], t[3]};
      store_frag(p, (rt0 + i) * 16, (tile0 + c) * 16, lane, v, es.s1[c], es.sa[i]);
    }
}

// The 256 x 256 tile (eight waves: two row groups of 128 x 64 waves) as a
// ping-pong.  Each compute unit's SIMD holds one wave of each row group, and
// with both running the same mix of decode and MFMAs the older wave takes
// the issue slots first: it finishes its k-block long before the younger
// one and idles at the barrier while the SIMD runs a single wave.  Here the
// two row groups take turns instead.  A wave's k-block is two phases: D
// (issue the loads of a later k-block, read its codes, meta and activation
// fragments from LDS and decode the codes into MFMA operands, all held in
// registers) and M (its 64 MFMAs, at raised priority, reading no memory).
// Row group 1 runs one phase behind row group 0, so in every phase one wave
// of each SIMD multiplies while the other decodes; all eight waves meet at a
// barrier after each phase.  Stage k of the S = 3 LDS ring is read by the D
// phases of k-block k (phases 2k and 2k + 1) and refilled by the D phases of
// k-block k + 1 onward, after both of those phases, so every refill comes
// after a barrier that follows the last read of its stage; and every wave
// waits for its own loads of a stage before the barrier that precedes the
// first D phase reading it.  Measured against the single-barrier loop of
// tiled_kernel with the same tile: 2-4 % faster on the Qwen1.5-72B shapes.
// (Shader-clock stamps per phase show the M phase still near 28 cycles per
// MFMA against 16.5 for the same MFMAs beside a decode-only wave: while the
// partner wave's D phase runs, the MFMA wave issues little.)
template <int GPB>
__global__ __launch_bounds__(512, 1) void tiled_pp_kernel(GemmParams p) {
  constexpr int MR = 8, NC = 4, RW = 2, NW = kColGroups, S = 3;
  constexpr int KWAVES = NW * RW;
  constexpr int BM = RW * 16 * MR;
  constexpr int A_BYTES = BM * 128;
  constexpr int W_BYTES = NW * NC * 1024;
  constexpr int M_BYTES = NW * NC * 256;
  constexpr int STAGE = A_BYTES + W_BYTES + M_BYTES;
  static_assert(STAGE == tiled_stage_bytes<MR, NC, RW, 1>(), "stage layout");
  constexpr int CPW = BM * 8 / (64 * KWAVES);
  constexpr int NCL = NC / RW;
  constexpr int LOADS = CPW + (GPB < 0 ? 1 : 2) * NCL;
  static_assert(LOADS < 64, "vmcnt range");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int cg = wave % NW;
  const int rg = wave / NW;
  const int quarter = lane >> 4;
  const int r16 = lane & 15;

  const int ntiles = p.n >> 4;
  const int kblocks = p.k >> 7;
  const int nbm = (p.m + BM - 1) / BM;
  const int nbn = (ntiles + NW * NC - 1) / (NW * NC);
  const int slice = blockIdx.x / (nbm * nbn);
  const int kb0 = slice * p.kb_per_slice;
  const int kb1 = min(kblocks, kb0 + p.kb_per_slice);
  int bm, bn;
  tile_of(blockIdx.x - slice * (nbm * nbn), nbm, nbn, &bm, &bn);
  const int row0 = bm * BM;
  const int tile0 = (bn * NW + cg) * NC;

  const int tlo = min(tile0, ntiles - 1);
  const __amdgpu_buffer_rsrc_t q_rsrc = make_rsrc(
      p.q + size_t(tlo) * kblocks * 1024, uint32_t(NC) * uint32_t(kblocks) * 1024u);
  const __amdgpu_buffer_rsrc_t m_rsrc = make_rsrc(
      p.meta + size_t(tlo) * 16 * p.meta_row_bytes, uint32_t(NC) * 16u * uint32_t(p.meta_row_bytes));
  const uint32_t q_lane = uint32_t(lane) * 16;
  const uint32_t m_lane = uint32_t(r16) * uint32_t(p.meta_row_bytes);
  uint32_t q_tile[NCL], m_tile[NCL];
#pragma unroll
  for (int c = 0; c < NCL; ++c) {
    const int t = min(tile0 + rg * NCL + c, ntiles - 1) - tlo;
    q_tile[c] = uint32_t(t) * uint32_t(kblocks) * 1024u;
    m_tile[c] = uint32_t(t) * 16u * uint32_t(p.meta_row_bytes);
  }
  const __amdgpu_buffer_rsrc_t a_rsrc =
      make_rsrc(p.a8 + size_t(row0) * p.lda8, uint32_t(BM) * uint32_t(p.lda8));
  uint32_t a_lane[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int s = (wave * CPW + j) * 64 + lane;
    const int row = s >> 3;
    const int lchunk = (s & 7) ^ (row & 7);
    a_lane[j] = uint32_t(min(row0 + row, p.m - 1) - row0) * uint32_t(p.lda8) + uint32_t(lchunk * 16);
  }
  int a_off[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
    a_off[h] = rg * (16 * MR * 128) + r16 * 128 + (((4 * h + quarter) ^ (r16 & 7)) * 16);
  const int w_off = A_BYTES + cg * NC * 1024 + lane * 16;
  const int m_off = A_BYTES + W_BYTES + cg * NC * 256 + lane * 4;

  v4i acc[MR][NC];
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[i][c] = v4i{0, 0, 0, 0};

  auto issue = [&](int kb, int stage) {
    uint8_t* st = smem + stage * STAGE;
#pragma unroll
    for (int j = 0; j < CPW; ++j)
      buffer_to_lds16(a_rsrc, st + (wave * CPW + j) * 1024, a_lane[j], uint32_t(kb) * 128u);
#pragma unroll
    for (int c = 0; c < NCL; ++c)
      buffer_to_lds16(q_rsrc, st + A_BYTES + (cg * NC + rg * NCL + c) * 1024, q_lane,
                      q_tile[c] + uint32_t(kb) * 1024u);
    if (GPB >= 0) {
#pragma unroll
      for (int c = 0; c < NCL; ++c)
        buffer_to_lds4(m_rsrc, st + A_BYTES + W_BYTES + (cg * NC + rg * NCL + c) * 256, m_lane,
                       m_tile[c] + (GPB == 0 ? 0u : uint32_t((kb * GPB) >> 2) * 4u));
    }
  };

  // operands of one k-block, carried from its D phase to its M phase
  v4i afr[2][MR];
  v4i bf[2][NC];
  auto dphase = [&](int kb, const uint8_t* st) {
    u32x4 qv[NC];
    uint32_t mv[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      qv[c] = *reinterpret_cast<const u32x4*>(st + w_off + c * 1024);
      mv[c] = GPB >= 0 ? *reinterpret_cast<const uint32_t*>(st + m_off + c * 256) : 0u;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < MR; ++i)
        afr[h][i] = *reinterpret_cast<const v4i*>(st + i * 16 * 128 + a_off[h]);
    GroupConst gblk[NC];
    if (GPB >= 0 && GPB <= 1) {
#pragma unroll
      for (int c = 0; c < NC; ++c)
        gblk[c] = group_const_at(mv[c], GPB == 1 ? 8u * (kb & 3) : 0u);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int byte = 0;
      if (GPB == 2) byte = 2 * (kb & 1) + h;
      if (GPB == 4) byte = 2 * h + (quarter >> 1);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint32_t w0 = h ? qv[c].z : qv[c].x;
        const uint32_t w1 = h ? qv[c].w : qv[c].y;
        if constexpr (GPB < 0) {
          bf[h][c] = decode16_lut(w0, w1);
        } else {
          const GroupConst gc =
              GPB <= 1 ? gblk[c] : group_const_at(mv[c], 8u * byte);
          bf[h][c] = decode16(w0, w1, gc);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): every operand in registers
  };
  auto mphase = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int c = 0; c < NC; ++c)
          acc[i][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(afr[h][i], bf[h][c], acc[i][c], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };

  // Phases: row group 0 runs D(0) M(0) D(1) M(1) ... then idles one phase;
  // row group 1 idles one phase, then D(0) M(0) ...  Before the barrier that
  // ends every odd phase (row group 0's M, row group 1's D) each wave waits
  // for its share of the stage row group 0 reads next (issued two D phases
  // earlier).
  const int nsb = kb1 - kb0;
#pragma unroll
  for (int j = 0; j < S - 1; ++j) issue(min(kb0 + j, kb1 - 1), j);
  wait_vm<LOADS>();                // this wave's share of stage 0 has landed
  __builtin_amdgcn_s_barrier();
  auto phase_end = [&](bool odd) {
    if (odd) wait_vm<LOADS>();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  if (rg == 0) {
    for (int k = 0; k < nsb; ++k) {
      issue(min(kb0 + k + S - 1, kb1 - 1), (k + S - 1) % S);
      dphase(kb0 + k, smem + (k % S) * STAGE);
      phase_end(false);
      mphase();
      phase_end(true);
    }
    phase_end(false);
  } else {
    phase_end(false);
    for (int k = 0; k < nsb; ++k) {
      issue(min(kb0 + k + S - 1, kb1 - 1), (k + S - 1) % S);
      dphase(kb0 + k, smem + (k % S) * STAGE);
      phase_end(true);
      mphase();
      phase_end(false);
    }
  }
  wait_vm<0>();                    // no LDS write still in flight at exit

  const int rt0 = row0 / 16 + rg * MR;
  if (p.part) {
    int32_t* part = p.part + size_t(slice) * size_t(p.m) * size_t(p.n);
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int col = (tile0 + c) * 16 + r16;
        if (tile0 + c >= ntiles) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = (rt0 + i) * 16 + 4 * quarter + r;
          if (row < p.m) part[size_t(row) * p.n + col] = acc[i][c][r];
        }
      }
    return;
  }
  const EpiScales<MR, NC> es = load_scales<MR, NC>(p, rt0, tile0, lane);
#pragma unroll
  for (int i = 0; i < MR; ++i)
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (tile0 + c >= ntiles) continue;
      int32_t v[4] = {acc[i][c][0], acc[i][c][1], acc[i][c][2], acc[i][c][3]};
      store_frag(p, (rt0 + i) * 16, (tile0 + c) * 16, lane, v, es.s1[c], es.sa[i]);
    }
}

template <int GPB>
hipError_t launch_pp_t(const GemmParams& p, int slices, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&tiled_pp_kernel<GPB>);
  const size_t lds = size_t(3) * tiled_stage_bytes<8, 4, 2, 1>();
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (e != hipSuccess) return e;
  const int ntiles = p.n / 16;
  const int nbm = (p.m + 255) / 256;
  const int nbn = (ntiles + 15) / 16;
  dim3 grid(nbm * nbn * slices);
  GemmParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, grid, dim3(512), args, lds, stream);
}

hipError_t pp_by_gpb(const GemmParams& p, int gpb, int sl, hipStream_t s) {
  switch (gpb) {
    case -1: return launch_pp_t<-1>(p, sl, s);
    case 0: return launch_pp_t<0>(p, sl, s);
    case 1: return launch_pp_t<1>(p, sl, s);
    case 2: return launch_pp_t<2>(p, sl, s);
    case 4: return launch_pp_t<4>(p, sl, s);
  }
  return hipErrorInvalidValue;
}

// Sum of the K slices' int32 partial tiles (exact) and the epilogue
// Y = fp16((acc * s_a) * s1).  One thread per 4 consecutive outputs, so the
// partial rows are read with coalesced 16-byte loads, the 4 column scales
// with one 8-byte load (the s1 section is 256-byte aligned and col % 4 == 0)
// and, when Y's rows allow it, the 4 outputs are written with one 8-byte
// store.
__global__ __launch_bounds__(256) void split_reduce_kernel(GemmParams p, int slices, int y_vec) {
  const int n4 = p.n >> 2;
  const long idx = long(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= long(p.m) * n4) return;
  const int row = int(idx / n4);
  const int col = int(idx - long(row) * n4) * 4;
  const size_t plane = size_t(p.m) * size_t(p.n);
  const v4i* src = reinterpret_cast<const v4i*>(p.part + size_t(row) * p.n + col);
  v4i t = src[0];
  for (int sl = 1; sl < slices; ++sl) t += src[sl * (plane >> 2)];
  const float sa = h2f(p.s_a[row]);
  const uint2 s1x4 = *reinterpret_cast<const uint2*>(p.s1 + col);
  const uint16_t s1v[4] = {uint16_t(s1x4.x), uint16_t(s1x4.x >> 16), uint16_t(s1x4.y),
                           uint16_t(s1x4.y >> 16)};
  uint16_t yv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) yv[j] = f2h_bits((static_cast<float>(t[j]) * sa) * h2f(s1v[j]));
  uint16_t* dst = p.y + size_t(row) * p.ldy + col;
  if (y_vec) {
    *reinterpret_cast<uint2*>(dst) =
        uint2{uint32_t(yv[0]) | (uint32_t(yv[1]) << 16), uint32_t(yv[2]) | (uint32_t(yv[3]) << 16)};
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = yv[j];
  }
  if (p.acc) {
#pragma unroll
    for (int j = 0; j < 4; ++j) p.acc[size_t(row) * p.ldacc + col + j] = t[j];
  }
}

template <int MR, int NC, int RW, int KG, int GPB, int S>
hipError_t launch_tiled_t(const GemmParams& p, int slices, hipStream_t stream) {
  const void* fn = reinterpret_cast<const void*>(&tiled_kernel<MR, NC, RW, KG, GPB, S>);
  const size_t lds = size_t(S) * tiled_stage_bytes<MR, NC, RW, KG>();
  if (lds > 65536) {
    // above the default dynamic-LDS limit: opt in (the attribute is per
    // kernel and process-wide, setting it again is harmless)
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  const int ntiles = p.n / 16;
  const int nbm = (p.m + RW * 16 * MR - 1) / (RW * 16 * MR);
  const int nbn = (ntiles + kColGroups * NC - 1) / (kColGroups * NC);
  dim3 grid(nbm * nbn * slices);
  dim3 block(64 * kColGroups * RW * KG);
  GemmParams arg = p;
  void* args[] = {&arg};
  return hipLaunchKernel(fn, grid, block, args, lds, stream);
}

template <int MR, int NC, int RW, int KG, int S>
hipError_t tiled_by_gpb(const GemmParams& p, int gpb, int sl, hipStream_t s) {
  switch (gpb) {
    case -1: return launch_tiled_t<MR, NC, RW, KG, -1, S>(p, sl, s);
    case 0: return launch_tiled_t<MR, NC, RW, KG, 0, S>(p, sl, s);
    case 1: return launch_tiled_t<MR, NC, RW, KG, 1, S>(p, sl, s);
    case 2: return launch_tiled_t<MR, NC, RW, KG, 2, S>(p, sl, s);
    case 4: return launch_tiled_t<MR, NC, RW, KG, 4, S>(p, sl, s);
  }
  return hipErrorInvalidValue;
}

template <int MR, int NC>
hipError_t four_wave_by_stages(const GemmParams& p, int gpb, int stages, int sl, hipStream_t s) {
  switch (stages) {
    case 2: return tiled_by_gpb<MR, NC, 1, 1, 2>(p, gpb, sl, s);
    case 3: return tiled_by_gpb<MR, NC, 1, 1, 3>(p, gpb, sl, s);
    case 4: return tiled_by_gpb<MR, NC, 1, 1, 4>(p, gpb, sl, s);
    case 5:
      if constexpr (5 * tiled_stage_bytes<MR, NC, 1, 1>() <= kTiledMaxLds)
        return tiled_by_gpb<MR, NC, 1, 1, 5>(p, gpb, sl, s);
      break;
    case 6:
      if constexpr (6 * tiled_stage_bytes<MR, NC, 1, 1>() <= kTiledMaxLds)
        return tiled_by_gpb<MR, NC, 1, 1, 6>(p, gpb, sl, s);
      break;
    case 8:
      if constexpr (8 * tiled_stage_bytes<MR, NC, 1, 1>() <= kTiledMaxLds)
        return tiled_by_gpb<MR, NC, 1, 1, 8>(p, gpb, sl, s);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_tiled(const GemmParams& p, int gpb, const TiledConfig& c, int sl,
                             hipStream_t stream) {
  if (!tiled_config_supported(c) || sl < 1 || sl > kMaxSlices) return hipErrorInvalidValue;
  if (sl > 1 && (p.part == nullptr || p.kb_per_slice * (sl - 1) >= p.k / 128))
    return hipErrorInvalidValue;
  if (c.rw == 2) return pp_by_gpb(p, gpb, sl, stream);
  if (c.kg == 2) {
    if (c.mr == 8 && c.nc == 4) return tiled_by_gpb<8, 4, 1, 2, 2>(p, gpb, sl, stream);
    if (c.mr == 4 && c.nc == 4) return tiled_by_gpb<4, 4, 1, 2, 2>(p, gpb, sl, stream);
    if (c.mr == 8 && c.nc == 2) {
      if (c.stages == 2) return tiled_by_gpb<8, 2, 1, 2, 2>(p, gpb, sl, stream);
      return tiled_by_gpb<8, 2, 1, 2, 3>(p, gpb, sl, stream);
    }
    if (c.mr == 4 && c.nc == 2) {
      if (c.stages == 2) return tiled_by_gpb<4, 2, 1, 2, 2>(p, gpb, sl, stream);
      if (c.stages == 3) return tiled_by_gpb<4, 2, 1, 2, 3>(p, gpb, sl, stream);
      return tiled_by_gpb<4, 2, 1, 2, 4>(p, gpb, sl, stream);
    }
    return hipErrorInvalidValue;
  }
  if (c.mr == 8 && c.nc == 4) return four_wave_by_stages<8, 4>(p, gpb, c.stages, sl, stream);
  if (c.mr == 4 && c.nc == 4) return four_wave_by_stages<4, 4>(p, gpb, c.stages, sl, stream);
  if (c.mr == 8 && c.nc == 2) return four_wave_by_stages<8, 2>(p, gpb, c.stages, sl, stream);
  if (c.mr == 4 && c.nc == 2) return four_wave_by_stages<4, 2>(p, gpb, c.stages, sl, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_split_reduce(const GemmParams& p, int slices, hipStream_t stream) {
  if (p.part == nullptr || p.n % 4 || slices < 1) return hipErrorInvalidValue;
  const long threads = long(p.m) * (p.n / 4);
  GemmParams arg = p;
  int sl = slices;
  int y_vec = (reinterpret_cast<uintptr_t>(p.y) % 8 == 0) && (p.ldy % 4 == 0);
  void* args[] = {&arg, &sl, &y_vec};
  return hipLaunchKernel(reinterpret_cast<const void*>(&split_reduce_kernel),
                         dim3(unsigned((threads + 255) / 256)), dim3(256), args, 0, stream);
}

}  // namespace w4a8
