// W4A8 linear layer for gfx950 with the per-token activation quantization
// fused into the small-M GEMM: one launch instead of quantizer + GEMM.
//
// The quantization needs each token's largest |A| over all of K before any
// int8 operand exists, and every workgroup multiplies all of K, so every
// workgroup quantizes all M x K activations itself (the standalone quantizer
// does it once for the whole GPU).  That costs vector-ALU time per
// workgroup, so the grid is persistent: about one workgroup per compute unit,
// each walking column-tile groups blockIdx.x, blockIdx.x + gridDim.x, ...,
// quantizes A once and reuses the int8 rows for all its tiles.
//
// Workgroup = kw waves splitting K (wave wk owns the 128-k blocks
// [wk * KBW, (wk + 1) * KBW)), one 16-row tile (M <= 16), NC 16-column tiles
// per group.  Partial int32 tiles of the waves are summed exactly through LDS.
//
// Prologue: each wave loads its K range of rows 0 .. M-1 (fp16, 16-byte
// chunks spread over all 64 lanes) into registers; after a barrier that puts
// every wave's activation loads ahead of any weight load, the weight ring of
// the first tile group is issued, so the weight stream starts at once.  The
// waves' partial row maxima meet in LDS (a transposed butterfly on the
// VALU's cross-lane paths leaves each lane with one row); every lane derives the
// s_a and fp32(1 / s_a) of one row as the standalone quantizer does (the same
// device functions, so the same bits), so all rows take their divisions at
// once, and each wave writes its int8 rows to its own LDS slab, from which
// its K loop reads the MFMA A operands: no workgroup barrier between the
// quantization and the K loop.  The epilogue takes s_a from the lanes that
// derived it.  Workgroup 0 also stores A8 and s_a.
//
// All loops over the kw waves (the row maxima, the split-K sum) read LDS at
// clamped indices without branches, so their reads are issued together.
//
// K loop: groups of whole MFMA steps (g = 128, g = 64, per row) are factored
// out of the inner product (raw codes into the MFMA, one correction per
// group and output value); g = 32 and codebook weights are decoded to int8
// operands first.
//
// Weight ring of D slots (4, or 8 for ranges of 8 or 16 blocks): slot
// j = v % D holds block v of the wave's range; once block v has been
// multiplied the slot is refilled with block v + D, which past the end of
// the range is block v + D - KBW of the next tile group, so the stream does
// not drain between groups.  The first 4 slots are issued before the
// prologue, the rest after its row-maxima barrier: a wave cannot issue many
// more loads at once and would stall at the issue, delaying its own
// prologue (a 16-slot ring did).  Blocks past the wave's real range
// (the last wave, when K does not fill kw * KBW blocks) are loaded clamped to
// its last real block (a cache hit) and not multiplied.
//
// LDS: [kw][16] uint32 row maxima, [2][kw][NC][256] int32 partial tiles
// when kw > 1 (the halves alternate between tile groups, so one
// barrier per group suffices), then [kw][M][slab] int8 rows with
// slab = KBW * 128 + 16 bytes (the pad staggers rows over the banks).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "gemm_common.h"
#include "kernels.h"

namespace w4a8 {
namespace {

using namespace dev;

template <int NC, int GPB, int D, int MF, int KBW>
__global__ __launch_bounds__(512) void fused_kernel(GemmParams p, const uint16_t* a, int lda) {
  static_assert(KBW % D == 0, "ring groups must tile the wave's range");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int CPL = KBW / 4;   // 16-byte fp16 chunks per lane and row
  const int lane = threadIdx.x & 63;
  const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kw = blockDim.x >> 6;
  const int quarter = lane >> 4;
  const int r16 = lane & 15;

  const int ntiles = p.n >> 4;
  const int ngroups = (ntiles + NC - 1) / NC;
  const int kblocks = p.k >> 7;
  const int kb_begin = min(kblocks, wk * KBW);
  const int nreal = min(kblocks - kb_begin, KBW);            // may be 0
  const int kb_last = min(kblocks - 1, kb_begin + max(nreal, 1) - 1);
  constexpr int slab = KBW * 128 + 16;

  uint32_t* amax_lds = reinterpret_cast<uint32_t*>(lds);
  int32_t* red = reinterpret_cast<int32_t*>(lds + kw * 64);
  const int red_bytes = kw > 1 ? 2 * kw * NC * 1024 : 0;
  int8_t* my_slab = reinterpret_cast<int8_t*>(lds + kw * 64 + red_bytes) + wk * p.m * slab;

  constexpr int MSTEP = GPB <= 0 ? D : 4 / GPB;   // ring slots per meta dword
  u32x4 q[D][NC];
  uint32_t md[D][NC], mdn[D][NC];
  // load block vv of the wave's range, column-tile group tg, into slot j
  auto issue = [&](int j, int tg, int vv) {
    const int kb = min(kb_begin + vv, kb_last);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      const int t = min(tg * NC + c, ntiles - 1);
      q[j][c] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(p.q + ((size_t(t) * kblocks + kb) * 64 + lane) * 16));
    }
    if (GPB >= 0 && j % MSTEP == 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int t = min(tg * NC + c, ntiles - 1);
        const uint32_t* mrow =
            reinterpret_cast<const uint32_t*>(p.meta + size_t(t * 16 + r16) * p.meta_row_bytes);
        mdn[j][c] = mrow[GPB == 0 ? 0 : (kb * GPB) >> 2];
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

  // ---- quantization prologue.  The activation loads go out first and the
  // weight ring right behind them: vector-memory counters complete in order,
  // so waiting for the activations does not wait for the weights.
  const int k0 = kb_begin * 128;
  const int cpr = nreal * 16;   // chunks per row in the wave's range
  uint4 chunk[MF][CPL];
#pragma unroll
  for (int r = 0; r < MF; ++r) {
    const uint16_t* src = a + size_t(min(r, p.m - 1)) * lda + k0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = j * 64 + lane;
      chunk[r][j] = (r < p.m && c < cpr) ? *reinterpret_cast<const uint4*>(src + c * 8)
                                         : uint4{0, 0, 0, 0};
    }
  }
  // s1 of a group is loaded one group ahead (raw bits, converted where the
  // epilogue uses them), so its latency never reaches the epilogue
  const int tg0 = blockIdx.x;
  uint16_t s1_next[NC];
  auto load_s1 = [&](int tg) {
#pragma unroll
    for (int c = 0; c < NC; ++c) s1_next[c] = p.s1[min((tg * NC + c) * 16 + r16, p.n - 1)];
  };
  load_s1(tg0);
  // every wave's activation loads enter the memory pipeline ahead of any
  // weight load (else a late wave's rows queue behind the others' weights
  // and the workgroup waits for them at the row-maxima barrier)
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  constexpr int D0 = D < 4 ? D : 4;   // slots issued before the prologue
#pragma unroll
  for (int j = 0; j < D0; ++j) issue(j, tg0, j);
  __builtin_amdgcn_sched_barrier(0);
  // Row maxima, all rows at once: each lane starts with its partial maximum
  // of every row; a transposed butterfly halves the rows a lane holds at each
  // of the first log2(MF) exchange steps (the lanes with the step's lane bit
  // set keep the upper half), so afterwards lane l holds row l / (64 / MF),
  // and the remaining steps reduce over the lanes that share a row.  The
  // steps run on the cross-lane paths of the VALU: lane bits 5 and 4 by
  // the permlane32/permlane16 swaps, bits 3 .. 0 by DPP (row rotate by 8,
  // half-row mirror, two quad permutes: partners that differ in that bit).
  uint32_t pm[MF];
#pragma unroll
  for (int r = 0; r < MF; ++r) {
    uint32_t mx = 0;
#pragma unroll
    for (int j = 0; j < CPL; ++j) mx = absmax8(mx, chunk[r][j]);
    pm[r] = absmax_bits(mx);
  }
  // (the step count and row counts are closed forms of the unrolled step
  // index, so every pm index is a compile-time constant)
#pragma unroll
  for (int step = 0; step < 6; ++step) {
    const int off = 32 >> step;
    const int half = (MF >> step) / 2;   // rows handed over at this step (0: none)
    const int n = half > 0 ? half : 1;
#pragma unroll
    for (int i = 0; i < n; ++i) {
      const uint32_t x = pm[i], y = half > 0 ? pm[i + half] : pm[i];
      if (off >= 16) {
        // the swap leaves lanes without the bit holding (x, partner's x)
        // and lanes with it (partner's y, y)
        const auto sw = off == 32 ? __builtin_amdgcn_permlane32_swap(x, y, false, false)
                                  : __builtin_amdgcn_permlane16_swap(x, y, false, false);
        pm[i] = max(uint32_t(sw[0]), uint32_t(sw[1]));
      } else {
        // lanes with the bit keep y and send x: a bitwise blend under a lane
        // mask (a select of two elements would be folded into a runtime
        // index into pm, which costs a compare chain per element)
        const uint32_t upper = (lane & off) ? 0xFFFFFFFFu : 0u;
        const uint32_t diff = x ^ y;
        const uint32_t keep = x ^ (diff & upper);
        const uint32_t send = keep ^ diff;
        constexpr int kDpp[4] = {0xB1, 0x4E, 0x141, 0x128};   // xor 1, xor 2, xor 7, xor 8
        const int ctrl = kDpp[5 - step];
        uint32_t got;
        switch (ctrl) {
          case 0xB1: got = __builtin_amdgcn_update_dpp(0u, send, 0xB1, 0xF, 0xF, false); break;
          case 0x4E: got = __builtin_amdgcn_update_dpp(0u, send, 0x4E, 0xF, 0xF, false); break;
          case 0x141: got = __builtin_amdgcn_update_dpp(0u, send, 0x141, 0xF, 0xF, false); break;
          default: got = __builtin_amdgcn_update_dpp(0u, send, 0x128, 0xF, 0xF, false); break;
        }
        pm[i] = max(keep, got);
      }
    }
  }
  constexpr int LPR = 64 / MF;   // lanes per row after the butterfly
  if (lane % LPR == 0) amax_lds[wk * 16 + lane / LPR] = pm[0];
  __syncthreads();
#pragma unroll
  for (int j = D0; j < D; ++j) issue(j, tg0, j);
  // lane l derives the scale of row l % 16 (rows past M have maximum 0);
  // the reads repeat the last wave's entry past kw (a maximum is idempotent)
  const bool store_a8 = blockIdx.x == 0;
  uint32_t am = 0;
#pragma unroll
  for (int w = 0; w < 8; ++w) am = max(am, amax_lds[min(w, kw - 1) * 16 + r16]);
  if (r16 >= MF) am = 0;
  const uint16_t sb = act_scale_bits(am);
  const float rc = act_recip(sb);
  if (store_a8 && wk == 0 && quarter == 0 && r16 < p.m) p.s_a_out[r16] = sb;
#pragma unroll
  for (int r = 0; r < MF; ++r) {
    if (r >= p.m) continue;   // (not break: the loop must stay unrolled)
    const float rcr = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, rc), r));
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = j * 64 + lane;
      if (c < cpr) {
        const uint2 o = quant8(chunk[r][j], rcr);
        *reinterpret_cast<uint2*>(my_slab + r * slab + c * 8) = o;
        if (store_a8) *reinterpret_cast<uint2*>(p.a8_out + size_t(r) * p.lda8 + k0 + c * 8) = o;
      }
    }
  }
  // s_a of the rows this lane stores in the epilogue, from lanes 0 .. 15
  const float saf = h2f(sb);
  float sa[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) sa[r] = __shfl(saf, min(4 * quarter + r, p.m - 1));

  // A operand of lane (row r16, k quarter) for block v, half h; rows past M
  // read row M - 1 (their products are never stored)
  const int8_t* arow = my_slab + min(r16, p.m - 1) * slab + 16 * quarter;
  v4i acc[NC];
  v4i sacc;   // per-row groups: row sums of A8 over the wave's range

  // Groups that cover whole MFMA steps (a 128-k block, a 64-k half, or the
  // row; a wave's range spans at most 2048 k) are factored out of the inner
  // product: raw codes into the MFMA, s2 * (sum a * q - z * sum a) per group,
  // the row sums from one more MFMA against ones, shared by the NC tiles.
  // The codes need 3 vector instructions per 8 weights instead of 7, plus 3
  // per output value and group.  Only the values that can hold a row below
  // MF are corrected: with MF <= 4 the valid rows are values 0 .. MF-1 of
  // lanes 0 .. 15, and the rest are never stored.
  constexpr bool FACTORED = GPB == 0 || GPB == 1 || GPB == 2;
  // add_group's 24-bit products are exact while a factored group spans at
  // most 2048 k: |sum a| <= 127 * 2048 and |sum a * q|, |z * sum a| <=
  // 127 * 15 * 2048, so every factor and difference stays below 2^23
  static_assert(!FACTORED || KBW * 128 <= 2048, "factored groups need wave ranges of <= 2048 k");
  constexpr int NV = MF < 4 ? MF : 4;
  const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
  auto codes = [&](const u32x4& qc, int h) { return h ? codes16(qc.z, qc.w) : codes16(qc.x, qc.y); };

  // decode block v from ring slot j = v % D and multiply it into acc
  auto compute = [&](int j, int v) {
    const u32x4 (&qs)[NC] = q[j];
    const uint32_t (&ms)[NC] = md[j - j % MSTEP];
    if constexpr (FACTORED) {
      v4i af[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) af[h] = *reinterpret_cast<const v4i*>(arow + v * 128 + 64 * h);
      if constexpr (GPB == 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          sacc = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[h], ones, sacc, 0, 0, 0);
#pragma unroll
          for (int c = 0; c < NC; ++c)
            acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[h], codes(qs[c], h), acc[c], 0, 0, 0);
        }
      } else if constexpr (GPB == 1) {
        v4i sm = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[0], ones, v4i{0, 0, 0, 0}, 0, 0, 0);
        sm = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[1], ones, sm, 0, 0, 0);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          v4i g = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[0], codes(qs[c], 0), v4i{0, 0, 0, 0}, 0, 0, 0);
          g = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[1], codes(qs[c], 1), g, 0, 0, 0);
          add_group<NV>(acc[c], g, sm, (ms[c] >> (8 * (v & 3))) & 0xFFu);
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const v4i sm = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[h], ones, v4i{0, 0, 0, 0}, 0, 0, 0);
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const v4i g =
                __builtin_amdgcn_mfma_i32_16x16x64_i8(af[h], codes(qs[c], h), v4i{0, 0, 0, 0}, 0, 0, 0);
            add_group<NV>(acc[c], g, sm, (ms[c] >> (8 * (2 * (v & 1) + h))) & 0xFFu);
          }
        }
      }
      return;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4i af = *reinterpret_cast<const v4i*>(arow + v * 128 + 64 * h);
      // byte of this lane's group in the meta dword (kb_begin % 4 == 0)
      int byte = 0;
      if (GPB == 1) byte = v & 3;
      if (GPB == 2) byte = 2 * (v & 1) + h;
      if (GPB == 4) byte = 2 * h + (quarter >> 1);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint32_t w0 = h ? qs[c].z : qs[c].x;
        const uint32_t w1 = h ? qs[c].w : qs[c].y;
        v4i bf;
        if constexpr (GPB < 0) {
          bf = decode16_lut(w0, w1);
        } else {
          bf = decode16(w0, w1, group_const_at(ms[c], 8u * byte));
        }
        acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf, acc[c], 0, 0, 0);
      }
    }
  };

  // One column-tile group: K loop, then the split-K sum and the epilogue.
  // With HAS_NEXT the ring slots freed by the last D blocks are refilled
  // from the next group; the workgroup's last group issues no such loads.
  // The two copies keep every load unconditional inside the unrolled loop.
  auto run_group = [&](int tg, int tg_next, int it, auto has_next) {
    constexpr bool HAS_NEXT = decltype(has_next)::value;
    uint16_t s1_bits[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) s1_bits[c] = s1_next[c];
    if (HAS_NEXT) load_s1(tg_next);
#pragma unroll
    for (int c = 0; c < NC; ++c) acc[c] = v4i{0, 0, 0, 0};
    sacc = v4i{0, 0, 0, 0};
    uint32_t row_meta[NC];   // per-row groups: this group's meta, before the ring moves on
#pragma unroll
    for (int c = 0; c < NC; ++c) row_meta[c] = md[0][c];
#pragma unroll
    for (int v = 0; v < KBW; ++v) {
      const int j = v % D;
      if (v < nreal) compute(j, v);
      if (v + D < KBW) issue(j, tg, v + D);
      else if (HAS_NEXT) issue(j, tg_next, v + D - KBW);
      if (j == D - 1) next_group_meta();
    }

    if constexpr (GPB == 0) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const v4i raw = acc[c];
        acc[c] = v4i{0, 0, 0, 0};
        add_group<NV>(acc[c], raw, sacc, row_meta[c] & 0xFFu);
      }
    }
    if (kw == 1) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        if (tg * NC + c >= ntiles) continue;
        int32_t v[4] = {acc[c][0], acc[c][1], acc[c][2], acc[c][3]};
        store_frag(p, 0, (tg * NC + c) * 16, lane, v, h2f(s1_bits[c]), sa);
      }
      return;
    }
    int32_t* part = red + (it & 1) * kw * NC * 256;
    int32_t* mine = part + wk * NC * 256;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) mine[(c * 4 + r) * 64 + lane] = acc[c][r];
    __syncthreads();
    for (int c = wk; c < NC; c += kw) {
      if (tg * NC + c >= ntiles || 4 * quarter >= p.m) continue;
      int32_t v[4] = {0, 0, 0, 0};
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int32_t* pp = part + (min(w, kw - 1) * NC + c) * 256;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int32_t x = pp[r * 64 + lane];
          v[r] += w < kw ? x : 0;
        }
      }
      uint16_t s1c = s1_bits[0];
#pragma unroll
      for (int cc = 1; cc < NC; ++cc)
        if (cc == c) s1c = s1_bits[cc];
      store_frag(p, 0, (tg * NC + c) * 16, lane, v, h2f(s1c), sa);
    }
  };

  next_group_meta();
  const int stride = gridDim.x;
  int tg = tg0, it = 0;
  for (; tg + stride < ngroups; tg += stride, ++it)
    run_group(tg, tg + stride, it, std::true_type{});
  run_group(tg, tg, it, std::false_type{});   // tg0 < ngroups: every workgroup has a last group
}

template <int NC, int GPB, int MF, int KBW>
hipError_t launch_fused_t(const GemmParams& p, const uint16_t* a, int lda, const SkinnyConfig& c,
                          hipStream_t stream) {
  constexpr int D = KBW >= 8 ? 8 : 4;
  const void* fn = reinterpret_cast<const void*>(&fused_kernel<NC, GPB, D, MF, KBW>);
  const size_t lds = fused_lds_bytes(c.kw, NC, p.m, KBW);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
  }
  const int ngroups = (p.n / 16 + NC - 1) / NC;
  const int grid = c.wgs > 0 ? std::min(c.wgs, ngroups) : ngroups;
  GemmParams arg = p;
  arg.kb_per_wave = KBW;
  const uint16_t* a_arg = a;
  int lda_arg = lda;
  void* args[] = {&arg, &a_arg, &lda_arg};
  return hipLaunchKernel(fn, dim3(grid), dim3(64 * c.kw), args, lds, stream);
}

template <int NC, int MF, int KBW>
hipError_t fused_by_gpb(const GemmParams& p, const uint16_t* a, int lda, int gpb,
                        const SkinnyConfig& c, hipStream_t s) {
  switch (gpb) {
    case -1: return launch_fused_t<NC, -1, MF, KBW>(p, a, lda, c, s);
    case 0: return launch_fused_t<NC, 0, MF, KBW>(p, a, lda, c, s);
    case 1: return launch_fused_t<NC, 1, MF, KBW>(p, a, lda, c, s);
    case 2: return launch_fused_t<NC, 2, MF, KBW>(p, a, lda, c, s);
    case 4: return launch_fused_t<NC, 4, MF, KBW>(p, a, lda, c, s);
  }
  return hipErrorInvalidValue;
}

template <int MF, int KBW>
hipError_t fused_by_nc(const GemmParams& p, const uint16_t* a, int lda, int gpb,
                       const SkinnyConfig& c, hipStream_t s) {
  switch (c.nc) {
    case 1: return fused_by_gpb<1, MF, KBW>(p, a, lda, gpb, c, s);
    case 2: return fused_by_gpb<2, MF, KBW>(p, a, lda, gpb, c, s);
  }
  return hipErrorInvalidValue;
}

template <int MF>
hipError_t fused_by_kbw(const GemmParams& p, const uint16_t* a, int lda, int gpb,
                        const SkinnyConfig& c, hipStream_t s) {
  switch (c.kbw) {
    case 4: return fused_by_nc<MF, 4>(p, a, lda, gpb, c, s);
    case 8:
      if constexpr (MF * 8 <= kFusedMaxHold) return fused_by_nc<MF, 8>(p, a, lda, gpb, c, s);
      break;
    case 16:
      if constexpr (MF * 16 <= kFusedMaxHold) return fused_by_nc<MF, 16>(p, a, lda, gpb, c, s);
      break;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_fused(const GemmParams& p, const uint16_t* a, int lda, int gpb,
                             const SkinnyConfig& c, hipStream_t stream) {
  if (!fused_config_supported(c, p.m, p.k)) return hipErrorInvalidValue;
  switch (fused_rows(p.m)) {
    case 1: return fused_by_kbw<1>(p, a, lda, gpb, c, stream);
    case 2: return fused_by_kbw<2>(p, a, lda, gpb, c, stream);
    case 4: return fused_by_kbw<4>(p, a, lda, gpb, c, stream);
    case 8: return fused_by_kbw<8>(p, a, lda, gpb, c, stream);
    case 16: return fused_by_kbw<16>(p, a, lda, gpb, c, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace w4a8
