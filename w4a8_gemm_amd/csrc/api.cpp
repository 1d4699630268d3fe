// C ABI entry points for the GPU side: argument validation (host only, before
// any HIP call) and kernel selection.  The packer entry points live in
// pack.cpp.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstdint>

#include "../../include/w4a8.h"
#include "kernels.h"
#include "layout.h"

namespace {

using namespace w4a8;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

thread_local hipError_t t_last_hip_error = hipSuccess;

w4a8_status device_status(hipError_t e) {
  if (e == hipSuccess) return W4A8_OK;
  t_last_hip_error = e;
  return W4A8_ERR_DEVICE;
}

bool gemm_shape_supported(int n, int k, int g) {
  if (n % kColTile || k % kKBlock || k > W4A8_K_MAX || n > W4A8_N_MAX) return false;
  if (g == W4A8_GROUP_PER_CHANNEL || g == k || g == W4A8_CODEBOOK_NF) return true;
  return (g == 32 || g == 64 || g == 128) && k % g == 0;
}

// K blocks per wave for a given split: a multiple of the kernel's ring
// depth (4), so that every wave starts on a meta dword.
int blocks_per_wave(int kblocks, int kw) { return ((kblocks + kw - 1) / kw + 3) / 4 * 4; }

// Automatic choice for the skinny kernel (M <= 64), from rocprofv3 sweeps on
// MI355X over the Llama-3-8B decode shapes.  Narrow layers (<= 256 column
// tiles) need every wave they can get, so K is split over 8 waves and each
// wave keeps one column tile; wider layers give each wave 2 (or, for
// 5..16 tokens, 4) column tiles so that the activation fragments loaded per
// block serve more weights.
SkinnyConfig choose_skinny(int m, int n, int k) {
  SkinnyConfig c;
  c.mr = m <= 16 ? 1 : (m <= 32 ? 2 : 4);
  const int ntiles = n / kColTile;
  const int kblocks = k / kKBlock;
  int kw = 8;
  if (ntiles <= 256) {
    c.nc = 1;
  } else if (ntiles <= 1024 || c.mr > 1 || m <= 4) {
    c.nc = 2;
  } else {
    c.nc = 4;
    kw = 4;
  }
  kw = std::min(kw, std::max(1, kblocks / 4));
  c.kbw = blocks_per_wave(kblocks, kw);
  // keep all kw waves even when rounding the range up to a multiple of 4
  // blocks leaves the last one idle: two waves on every SIMD beat an uneven
  // split (K = 14336: 8 waves with one idle are 5 % faster than 7)
  c.kw = kw;
  return c;
}

}  // namespace

extern "C" const char* w4a8_status_string(w4a8_status s) {
  switch (s) {
    case W4A8_OK: return "ok";
    case W4A8_ERR_INVALID_ARGUMENT: return "invalid argument";
    case W4A8_ERR_UNSUPPORTED: return "unsupported shape or group size";
    case W4A8_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case W4A8_ERR_NONFINITE: return "non-finite weight";
    case W4A8_ERR_RANGE: return "scale overflows fp16";
    case W4A8_ERR_LAYOUT: return "blob layout mismatch";
    case W4A8_ERR_DEVICE: return "HIP error";
  }
  return "unknown status";
}

extern "C" w4a8_status w4a8_quant_act(const uint16_t* a_dev, int m, int k, int lda,
                                      int8_t* a8_dev, int lda8, uint16_t* s_a_dev,
                                      void* stream) {
  if (m < 0 || m > W4A8_M_MAX || k <= 0 || k > W4A8_ACT_K_MAX || lda < k || lda8 < k)
    return W4A8_ERR_INVALID_ARGUMENT;
  if (m == 0) return W4A8_OK;
  if (!a_dev || !a8_dev || !s_a_dev) return W4A8_ERR_INVALID_ARGUMENT;
  return device_status(launch_quant_act(a_dev, m, k, lda, a8_dev, lda8, s_a_dev,
                                        static_cast<hipStream_t>(stream)));
}

extern "C" w4a8_status w4a8_quant_act_static(const uint16_t* a_dev, int m, int k, int lda,
                                             uint16_t scale_f16, int8_t* a8_dev, int lda8,
                                             uint16_t* s_a_dev, void* stream) {
  if (m < 0 || m > W4A8_M_MAX || k <= 0 || k > W4A8_ACT_K_MAX || lda < k || lda8 < k)
    return W4A8_ERR_INVALID_ARGUMENT;
  // the scale must be a finite, non-negative fp16 value (sign bit clear,
  // exponent field not all ones)
  if ((scale_f16 & 0x8000u) || (scale_f16 & 0x7C00u) == 0x7C00u) return W4A8_ERR_INVALID_ARGUMENT;
  if (m == 0) return W4A8_OK;
  if (!a_dev || !a8_dev || !s_a_dev) return W4A8_ERR_INVALID_ARGUMENT;
  return device_status(launch_quant_act_static(a_dev, m, k, lda, scale_f16, a8_dev, lda8, s_a_dev,
                                               static_cast<hipStream_t>(stream)));
}

namespace {

// Everything the automatic choice (or a forced one) decides for one call.
struct Plan {
  w4a8_status status = W4A8_OK;
  int variant = 0;          // 1 skinny, 2 tiled
  SkinnyConfig skinny{};
  TiledConfig tiled{};
  int slices = 1;           // tiled: workgroups splitting K (partials in the workspace)
  int kb_per_slice = 0;
  size_t workspace = 0;     // bytes
};

// Workgroup tiles of rows x cols over the output.
long tiled_tiles(int m, int n, int rows, int cols = 256) {
  return ((long(m) + rows - 1) / rows) * ((long(n) + cols - 1) / cols);
}

// Forced options outside the ranges any kernel takes (and negative values)
// are rejected before they enter any size arithmetic.
bool opts_in_range(const w4a8_gemm_opts* o) {
  if (!o) return true;
  return o->variant >= 0 && o->variant <= 3 && o->k_split >= 0 && o->k_split <= 8 &&
         o->n_tiles >= 0 && o->n_tiles <= 4 && o->m_tiles >= 0 && o->m_tiles <= 16 &&
         o->stages >= 0 && o->stages <= 8 && o->row_groups >= 0 && o->row_groups <= 2 &&
         o->slices >= 0 && o->slices <= kMaxSlices && o->workgroups >= 0;
}

Plan plan_gemm(int m, int n, int k, const w4a8_gemm_opts* opts) {
  Plan pl;
  if (!opts_in_range(opts)) { pl.status = W4A8_ERR_INVALID_ARGUMENT; return pl; }
  pl.variant = opts ? opts->variant : 0;
  if (pl.variant < 0 || pl.variant > 2) { pl.status = W4A8_ERR_INVALID_ARGUMENT; return pl; }
  const int kblocks = k / kKBlock;
  // the skinny kernel up to 16 tokens, and up to 64 unless the layer is
  // wide enough to give the tiled kernel's 64 x 128 tiles most of the GPU
  // (its activation fragments, re-read by every workgroup, grow with M), or
  // K is long enough that those re-reads (M * K bytes per workgroup) cost
  // more than splitting K over workgroups
  const long t64 = tiled_tiles(m, n, 64, 128);
  // ... or, from 40 tokens and K >= 4096, the layer has 80-191 such tiles
  // (over ~10k columns): there 64 x 128 tiles with K split in two beat the
  // skinny kernel by 15-37 % at K = 4096-5120 (11008, 13824 and 16384
  // columns), while up to 64 tiles the skinny kernel stays ahead at every
  // M <= 48
  const bool split_small = m > 16 && m <= 64 &&
                           ((kblocks >= 64 && long(m) * k >= kSplitSmallElems) ||
                            (m >= 40 && kblocks >= 32 && t64 >= 80 && t64 < 192));
  if (pl.variant == 0)
    pl.variant = (m <= 16 || (m <= 64 && t64 < 192 && !split_small)) ? 1 : 2;
  if (pl.variant == 1) {
    if (m > 64) { pl.status = W4A8_ERR_UNSUPPORTED; return pl; }
    SkinnyConfig& c = pl.skinny;
    c = choose_skinny(m, n, k);
    if (opts && opts->n_tiles > 0) c.nc = opts->n_tiles;
    if (opts && opts->k_split > 0) {
      c.kw = opts->k_split;
      c.kbw = blocks_per_wave(kblocks, c.kw);
    }
    return pl;
  }
  // Tiled (choices from graph-replay timing sweeps on the Llama-3-8B layer
  // shapes, M = 32 .. 1024): the kernel needs about one workgroup of eight
  // waves, or two of four, per compute unit, so the tile shrinks with the
  // grid it yields:
  //   >= 192 tiles of 256 x 256 whose rounds beat 128 x 128 ones (below)
  //                                      -> 256 x 256, eight waves, 3 stages
  //   M <= 64 (or <= 128 with K <= 16384), K >= 8192, < 192 tiles of 64 x 128
  //                                      -> 64 x 128 with K split over 2..16
  //                                         workgroups (~256 in all)
  //   129 <= M <= 192, 8192 <= K <= 16384, < 192 tiles of 64 x 128
  //                                      -> 64 x 128 with K split (~384)
  //   M >= 1024, K >= 12288, < 384 of 128 x 128 (and not the above)
  //                                      -> 256 x 256 (ping-pong) with K split
  //                                         so that ~256 workgroups run, each
  //                                         slice >= 16 k-blocks (the 1024 x
  //                                         4096 x 14336 down projection: 81
  //                                         against 90 us for 128 x 256 split
  //                                         three ways)
  //   K >= 8192 and < 192 of 128 x 256   -> 128 x 256 with K split over
  //                                         2..8 workgroups (~384 in all)
  //   > 256 tiles of 128 x 128, M > 64  -> 128 x 128, four waves, 3 stages
  //   > 256 tiles of 64 x 128, M > 64   -> 128 x 128, two k-groups, 2 stages
  //   otherwise                          -> 64 x 128, two k-groups, 3 stages
  // (the eight-wave kernels run one workgroup per compute unit, so each
  // keeps its tiles to one round of 256 workgroups: 512 x 5120 x 5120 takes
  // 34 us on 160 tiles of 128 x 128 against 41 on 320 of 64 x 128, and the
  // 1024 x 4096 x 4096 layer 29 against 31 us with four waves per tile;
  // at M <= 64 a 128-row tile is half empty: 64 x 128 tiles, same count)
  // Forced options select among the four-wave kernels (or the eight-wave
  // ones they name) with the rest from the 128 x 256 defaults.
  TiledConfig& c = pl.tiled;
  c.nw = 4;
  const long t256 = tiled_tiles(m, n, 256);
  const long t128x256 = tiled_tiles(m, n, 128);
  const long t128x128 = tiled_tiles(m, n, 128, 128);
  const bool forced = opts && (opts->m_tiles > 0 || opts->stages > 0 || opts->k_split > 0 ||
                               opts->row_groups > 0 || opts->n_tiles > 0 || opts->slices > 0);
  // 256 x 256 tiles run one workgroup per compute unit, 128 x 128 four-wave
  // tiles two: whole rounds of 256 and 512 workgroups, a round of 128 x 128
  // tiles costing about 0.6 of a 256 x 256 one (sweeps at K = 4096-8192:
  // 0.58-0.65).  So the ping-pong kernel is taken when its rounds win, which
  // keeps a 258- or 324-tile grid off a nearly empty second round
  // (1536 x 11008 x 4096: 105 against 124 us).
  const bool pp_rounds_win =
      t256 >= 192 && 5 * ((t256 + 255) / 256) < 3 * ((t128x128 + 511) / 512);
  int slices = 1;
  if (forced) {
    c.nc = 4;
    c.rw = 1;
    c.kg = 1;
    if (opts->row_groups > 0) c.rw = opts->row_groups;
    if (opts->k_split > 0) c.kg = opts->k_split;
    c.mr = (c.rw == 2 || t128x256 >= 192) ? 8 : 4;
    if (opts->m_tiles > 0) c.mr = opts->m_tiles;
    c.stages = (c.rw == 2 || (c.mr == 4 && c.kg == 1)) ? 3 : 2;
    if (opts->stages > 0) c.stages = opts->stages;
    if (opts->n_tiles > 0) c.nc = opts->n_tiles;

  } else if (pp_rounds_win) {
    c = TiledConfig{8, 4, 4, 2, 1, 3};
  } else if ((split_small || ((m <= 64 || (m <= 128 && kblocks <= 128)) && kblocks >= 64)) &&
             t64 < 192) {
    // 17..128 tokens, long K (up to 16384 above 64 tokens), or 40..64 tokens
    // on wide layers: 64 x 128 tiles, K split so that ~256 workgroups run
    // (each slice re-reads only its part of A8); at 96-128 tokens 20-25 %
    // faster than 128 x 256 tiles on the 4096 x 14336 and 8192 x 8192
    // layers, slower at K = 24576
    c = TiledConfig{4, 2, 4, 1, 1, 3};
    slices = int(std::max(2L, std::min<long>(256 / t64, kMaxSlices)));
  } else if (m > 128 && m <= 192 && kblocks >= 64 && kblocks <= 128 && t64 < 192) {
    // 129..192 tokens: three 64-row tiles waste less than two 128-row ones,
    // and with K split so that ~384 workgroups run (two per compute unit
    // fit) 11-50 % faster than 128 x 256 tiles split over 8 (M = 129, 160
    // and 192 on 4096 x 11008, 5120 x 13824 and 2048 x 8192; within 2 % on
    // 4096 x 14336)
    c = TiledConfig{4, 2, 4, 1, 1, 3};
    slices = int(std::max(2L, std::min<long>((384 + t64 - 1) / t64, kblocks / 16)));
  } else if (m >= 1024 && kblocks >= 96 && t256 >= 32 && t128x128 < 384) {
    c = TiledConfig{8, 4, 4, 2, 1, 3};
    slices = int(std::max(2L, std::min<long>({256 / t256, 8L, long(kblocks / 16)})));
  } else if (kblocks >= 64 && t128x256 < 192) {
    c = TiledConfig{8, 4, 4, 1, 1, 2};
    const long want = (384 + t128x256 - 1) / t128x256;
    slices = int(std::max(2L, std::min<long>(want, 8)));
  } else if (m > 64 && t128x128 > 256) {
    c = TiledConfig{8, 2, 4, 1, 1, 3};
  } else if (m > 64 && t64 > 256) {
    c = TiledConfig{8, 2, 4, 1, 2, 2};
  } else {
    c = TiledConfig{4, 2, 4, 1, 2, 3};
  }
  if (opts && opts->slices > 0) slices = opts->slices;
  if (slices > kMaxSlices) { pl.status = W4A8_ERR_INVALID_ARGUMENT; return pl; }
  if (!tiled_config_supported(c)) { pl.status = W4A8_ERR_INVALID_ARGUMENT; return pl; }
  // one launch holds every (tile, slice) workgroup
  if (tiled_tiles(m, n, c.rw * 16 * c.mr, c.nw * c.nc * 16) * slices > kMaxWorkgroups) {
    pl.status = W4A8_ERR_UNSUPPORTED;
    return pl;
  }
  slices = std::min(slices, kblocks);
  pl.kb_per_slice = (kblocks + slices - 1) / slices;
  pl.slices = (kblocks + pl.kb_per_slice - 1) / pl.kb_per_slice;   // none empty
  if (pl.slices > 1) pl.workspace = size_t(pl.slices) * size_t(m) * size_t(n) * 4u;
  return pl;
}

}  // namespace

extern "C" size_t w4a8_gemm_workspace_size(int m, int n, int k, int g,
                                           const w4a8_gemm_opts* opts) {
  if (m <= 0 || m > W4A8_M_MAX || n <= 0 || k <= 0 || !gemm_shape_supported(n, k, g)) return 0;
  const Plan pl = plan_gemm(m, n, k, opts);
  return pl.status == W4A8_OK ? pl.workspace : 0;
}

namespace {

// Every host-side check of a w4a8_gemm call, with no HIP call: shape, the
// plan (automatic or forced) and the workspace.  w4a8_linear runs it before
// it launches the quantizer, so a call the GEMM would reject leaves no
// kernel behind.  m > 0; a8/s_a may be checked by the caller instead (the
// fused layer writes them).
w4a8_status check_plan(const Plan& pl, int k, int g) {
  if (pl.status != W4A8_OK) return pl.status;
  const int gpb = groups_per_block(k, g);
  if (pl.variant == 1 && !skinny_config_supported(pl.skinny, k, gpb))
    return W4A8_ERR_INVALID_ARGUMENT;
  if (pl.variant == 2 && !tiled_config_supported(pl.tiled)) return W4A8_ERR_INVALID_ARGUMENT;
  return W4A8_OK;
}

w4a8_status check_gemm(const Plan& pl, int k, int g, void* workspace_dev, size_t workspace_bytes) {
  const w4a8_status st = check_plan(pl, k, g);
  if (st != W4A8_OK) return st;
  if (pl.workspace) {
    if (!workspace_dev || workspace_bytes < pl.workspace) return W4A8_ERR_BUFFER_TOO_SMALL;
    if (!aligned16(workspace_dev)) return W4A8_ERR_INVALID_ARGUMENT;
  }
  return W4A8_OK;
}

// The pointer and size checks shared by w4a8_gemm and w4a8_gemm_noalloc
// (m > 0).
bool gemm_args_ok(const int8_t* a8_dev, int lda8, const uint16_t* s_a_dev, const void* blob_dev,
                  int n, int k, const uint16_t* y_dev, int ldy, const int32_t* acc_dev,
                  int ldacc) {
  if (!a8_dev || !s_a_dev || !blob_dev || !y_dev) return false;
  if (lda8 < k || lda8 % 16 || lda8 > W4A8_LD_MAX || ldy < n || (acc_dev && ldacc < n)) return false;
  return aligned16(a8_dev) && aligned16(blob_dev);
}

// Enqueue a checked plan; `part` is the K-split partial-sum buffer (the
// workspace, or the static scratch) when the plan splits K.
w4a8_status run_gemm(const Plan& pl, const int8_t* a8_dev, int lda8, const uint16_t* s_a_dev,
                     int m, const void* blob_dev, int n, int k, int g, uint16_t* y_dev, int ldy,
                     int32_t* acc_dev, int ldacc, void* part, hipStream_t s) {
  const int gpb = groups_per_block(k, g);
  Sections sec = sections(n, k, g);
  const uint8_t* base = static_cast<const uint8_t*>(blob_dev);
  GemmParams p;
  p.a8 = a8_dev;
  p.lda8 = lda8;
  p.s_a = s_a_dev;
  p.m = m;
  p.q = base + sec.q_off;
  p.meta = base + sec.meta_off;
  p.s1 = reinterpret_cast<const uint16_t*>(base + sec.s1_off);
  p.n = n;
  p.k = k;
  p.meta_row_bytes = sec.meta_row_bytes;
  p.kb_per_wave = 0;
  p.y = y_dev;
  p.ldy = ldy;
  p.acc = acc_dev;
  p.ldacc = acc_dev ? ldacc : 0;
  p.part = nullptr;
  p.kb_per_slice = k / kKBlock;
  p.a8_out = nullptr;
  p.s_a_out = nullptr;

  hipError_t e;
  if (pl.variant == 1) {
    e = launch_gemm_skinny(p, gpb, pl.skinny, s);
  } else {
    if (pl.slices > 1) {
      p.part = static_cast<int32_t*>(part);
      p.kb_per_slice = pl.kb_per_slice;
    }
    e = launch_gemm_tiled(p, gpb, pl.tiled, pl.slices, s);
    if (e == hipSuccess && pl.slices > 1) e = launch_split_reduce(p, pl.slices, s);
  }
  return device_status(e);
}

}  // namespace

extern "C" w4a8_status w4a8_gemm(const int8_t* a8_dev, int lda8, const uint16_t* s_a_dev, int m,
                                 const void* blob_dev, int n, int k, int g, uint16_t* y_dev,
                                 int ldy, int32_t* acc_dev, int ldacc, void* workspace_dev,
                                 size_t workspace_bytes, const w4a8_gemm_opts* opts,
                                 void* stream) {
  if (m < 0 || m > W4A8_M_MAX || n <= 0 || k <= 0 || g < 0) return W4A8_ERR_INVALID_ARGUMENT;
  if (!gemm_shape_supported(n, k, g)) return W4A8_ERR_UNSUPPORTED;
  if (m == 0) return W4A8_OK;
  if (!gemm_args_ok(a8_dev, lda8, s_a_dev, blob_dev, n, k, y_dev, ldy, acc_dev, ldacc))
    return W4A8_ERR_INVALID_ARGUMENT;
  const Plan pl = plan_gemm(m, n, k, opts);
  const w4a8_status st = check_gemm(pl, k, g, workspace_dev, workspace_bytes);
  if (st != W4A8_OK) return st;
  return run_gemm(pl, a8_dev, lda8, s_a_dev, m, blob_dev, n, k, g, y_dev, ldy, acc_dev, ldacc,
                  workspace_dev, static_cast<hipStream_t>(stream));
}

namespace {

// The automatic plan with its K split narrowed until the partial sums fit
// the static scratch (every split gives the same int32 sums); a forced
// split that does not fit is left as it is and rejected by the caller.
Plan plan_gemm_in_scratch(int m, int n, int k, const w4a8_gemm_opts* opts) {
  Plan pl = plan_gemm(m, n, k, opts);
  if (pl.status != W4A8_OK || pl.workspace <= kScratchBytes || (opts && opts->slices > 0))
    return pl;
  const int kblocks = k / kKBlock;
  const size_t plane = size_t(m) * size_t(n) * 4u;
  int slices = int(kScratchBytes / plane);        // the most that fit (0 or 1: none)
  if (slices <= 1) {
    pl.slices = 1;
    pl.kb_per_slice = kblocks;
    pl.workspace = 0;
    return pl;
  }
  slices = std::min(slices, pl.slices);
  pl.kb_per_slice = (kblocks + slices - 1) / slices;
  pl.slices = (kblocks + pl.kb_per_slice - 1) / pl.kb_per_slice;   // none empty
  pl.workspace = pl.slices > 1 ? size_t(pl.slices) * plane : 0;
  return pl;
}

}  // namespace

extern "C" w4a8_status w4a8_gemm_noalloc(const int8_t* a8_dev, int lda8, const uint16_t* s_a_dev,
                                         int m, const void* blob_dev, int n, int k, int g,
                                         uint16_t* y_dev, int ldy, int32_t* acc_dev, int ldacc,
                                         const w4a8_gemm_opts* opts, void* stream) {
  if (m < 0 || m > W4A8_M_MAX || n <= 0 || k <= 0 || g < 0) return W4A8_ERR_INVALID_ARGUMENT;
  if (!gemm_shape_supported(n, k, g)) return W4A8_ERR_UNSUPPORTED;
  if (m == 0) return W4A8_OK;
  if (!gemm_args_ok(a8_dev, lda8, s_a_dev, blob_dev, n, k, y_dev, ldy, acc_dev, ldacc))
    return W4A8_ERR_INVALID_ARGUMENT;
  const Plan pl = plan_gemm_in_scratch(m, n, k, opts);
  const w4a8_status st = check_plan(pl, k, g);
  if (st != W4A8_OK) return st;
  if (pl.workspace > kScratchBytes) return W4A8_ERR_BUFFER_TOO_SMALL;   // a forced split
  void* part = nullptr;
  if (pl.workspace) {
    hipError_t e = scratch_address(&part);
    if (e != hipSuccess) return device_status(e);
  }
  return run_gemm(pl, a8_dev, lda8, s_a_dev, m, blob_dev, n, k, g, y_dev, ldy, acc_dev, ldacc,
                  part, static_cast<hipStream_t>(stream));
}

namespace {

// Configuration of the fused kernel: one row tile; one column tile per
// group for narrow layers (<= 256 tiles), else two; K split over up to 8
// waves with 4, 8 or 16 blocks each (every wave kept, as for the skinny
// kernel); a persistent grid of kFusedAutoWgs workgroups unless forced.
SkinnyConfig fused_plan(int m, int n, int k, const w4a8_gemm_opts* opts) {
  SkinnyConfig c{};
  c.mr = 1;
  const int kblocks = k / kKBlock;
  c.nc = n / kColTile > kFusedPairTiles && m > 2 ? 2 : 1;
  c.kw = std::min(8, std::max(1, kblocks / 4));
  if (opts && opts->k_split > 0) c.kw = opts->k_split;
  const int per = (kblocks + c.kw - 1) / c.kw;
  c.kbw = per <= 4 ? 4 : (per <= 8 ? 8 : (per <= 16 ? 16 : 0));
  if (opts && opts->n_tiles > 0) c.nc = opts->n_tiles;
  const int groups = (n / kColTile + c.nc - 1) / c.nc;
  const int rounds = (groups + kFusedAutoWgs - 1) / kFusedAutoWgs;
  c.wgs = (groups + rounds - 1) / rounds;
  if (opts && opts->workgroups != 0) c.wgs = opts->workgroups;
  return c;
}

// The automatic choice runs the fused kernel wherever it applies for up to
// kFusedAutoElems activations, kFusedWideElems on wide layers.
bool fused_by_default(int m, int n, int k) {
  const long elems = long(m) * k;
  return elems <= kFusedAutoElems || (elems <= kFusedWideElems && n / kColTile >= kFusedWideTiles);
}

}  // namespace

extern "C" w4a8_status w4a8_linear(const uint16_t* a_dev, int lda, int m, int k,
                                   const void* blob_dev, int n, int g, uint16_t* y_dev, int ldy,
                                   int8_t* a8_dev, int lda8, uint16_t* s_a_dev, int32_t* acc_dev,
                                   int ldacc, void* workspace_dev, size_t workspace_bytes,
                                   const w4a8_gemm_opts* opts, void* stream) {
  if (m < 0 || m > W4A8_M_MAX || n <= 0 || k <= 0 || g < 0) return W4A8_ERR_INVALID_ARGUMENT;
  if (!gemm_shape_supported(n, k, g)) return W4A8_ERR_UNSUPPORTED;
  if (m == 0) return W4A8_OK;
  if (!a_dev || !blob_dev || !y_dev || !a8_dev || !s_a_dev) return W4A8_ERR_INVALID_ARGUMENT;
  if (lda < k || lda % 8 || lda > W4A8_LD_MAX || lda8 < k || lda8 % 16 || lda8 > W4A8_LD_MAX ||
      ldy < n || (acc_dev && ldacc < n))
    return W4A8_ERR_INVALID_ARGUMENT;
  if (!aligned16(a_dev) || !aligned16(a8_dev) || !aligned16(blob_dev))
    return W4A8_ERR_INVALID_ARGUMENT;
  const int variant = opts ? opts->variant : 0;
  if (variant < 0 || variant > 3 || !opts_in_range(opts)) return W4A8_ERR_INVALID_ARGUMENT;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const SkinnyConfig fc = fused_plan(m, n, k, opts);
  const bool fused_ok = fused_config_supported(fc, m, k);
  if (variant == 3 && !fused_ok) return W4A8_ERR_UNSUPPORTED;
  if (variant == 3 || (variant == 0 && fused_ok && fused_by_default(m, n, k))) {
    Sections sec = sections(n, k, g);
    const uint8_t* base = static_cast<const uint8_t*>(blob_dev);
    GemmParams p{};
    p.a8 = a8_dev;
    p.lda8 = lda8;
    p.s_a = s_a_dev;
    p.m = m;
    p.q = base + sec.q_off;
    p.meta = base + sec.meta_off;
    p.s1 = reinterpret_cast<const uint16_t*>(base + sec.s1_off);
    p.n = n;
    p.k = k;
    p.meta_row_bytes = sec.meta_row_bytes;
    p.y = y_dev;
    p.ldy = ldy;
    p.acc = acc_dev;
    p.ldacc = acc_dev ? ldacc : 0;
    p.part = nullptr;
    p.kb_per_slice = k / kKBlock;
    p.a8_out = a8_dev;
    p.s_a_out = s_a_dev;
    return device_status(launch_gemm_fused(p, a_dev, lda, groups_per_block(k, g), fc, s));
  }
  // two launches: the quantizer, then the GEMM on its output; the GEMM's
  // checks run first, so that a call it would reject enqueues nothing
  w4a8_status st = check_gemm(plan_gemm(m, n, k, opts), k, g, workspace_dev, workspace_bytes);
  if (st != W4A8_OK) return st;
  st = w4a8_quant_act(a_dev, m, k, lda, a8_dev, lda8, s_a_dev, stream);
  if (st != W4A8_OK) return st;
  return w4a8_gemm(a8_dev, lda8, s_a_dev, m, blob_dev, n, k, g, y_dev, ldy, acc_dev, ldacc,
                   workspace_dev, workspace_bytes, opts, stream);
}

extern "C" w4a8_status w4a16_gemm(const uint16_t* a_dev, int lda, int m, int k,
                                  const void* blob_dev, int n, int g, uint16_t* y_dev, int ldy,
                                  const w4a8_gemm_opts* opts, void* stream) {
  if (m < 0 || m > W4A8_M_MAX || n <= 0 || k <= 0 || g < 0) return W4A8_ERR_INVALID_ARGUMENT;
  if (!gemm_shape_supported(n, k, g)) return W4A8_ERR_UNSUPPORTED;
  if (m == 0) return W4A8_OK;
  if (!a_dev || !blob_dev || !y_dev) return W4A8_ERR_INVALID_ARGUMENT;
  if (lda < k || lda % 8 || lda > W4A8_LD_MAX || ldy < n) return W4A8_ERR_INVALID_ARGUMENT;
  if (!aligned16(a_dev) || !aligned16(blob_dev)) return W4A8_ERR_INVALID_ARGUMENT;
  if (opts && (opts->variant > 2 || opts->variant < 0 || !opts_in_range(opts)))
    return W4A8_ERR_INVALID_ARGUMENT;
  if (g == W4A8_CODEBOOK_NF) return W4A8_ERR_UNSUPPORTED;
  // automatic choice: the skinny kernel (one 16-row tile per workgroup, the
  // weights streamed once per row tile) up to 64 tokens, and up to 128 when
  // the tiled kernel's grid would hold fewer than 128 workgroups of 256 x 128
  // (it has no K split, so such a grid leaves most compute units idle)
  const long w16_tiles = ((long(m) + 255) / 256) * ((long(n) / 16 + 7) / 8);
  const int variant = opts && opts->variant ? opts->variant
                                            : (m <= 64 || (m <= 128 && w16_tiles < 128) ? 1 : 2);
  if (variant == 1 && m > 128) return W4A8_ERR_UNSUPPORTED;
  const int gpb = groups_per_block(k, g);
  Sections sec = sections(n, k, g);
  const uint8_t* base = static_cast<const uint8_t*>(blob_dev);
  Gemm16Params p{};
  p.a = a_dev;
  p.lda = lda;
  p.m = m;
  p.q = base + sec.q_off;
  p.meta = base + sec.meta_off;
  p.s1 = reinterpret_cast<const uint16_t*>(base + sec.s1_off);
  p.n = n;
  p.k = k;
  p.meta_row_bytes = sec.meta_row_bytes;
  p.y = y_dev;
  p.ldy = ldy;
  if (variant == 2) {
    if (w16_tiles > kMaxWorkgroups) return W4A8_ERR_UNSUPPORTED;
    return device_status(launch_w4a16_tiled(p, gpb, static_cast<hipStream_t>(stream)));
  }
  // one row tile per workgroup (more row tiles go to grid.y): fp16 operands
  // take twice the registers of int8 ones, and a deeper row tile would spill
  SkinnyConfig c = choose_skinny(std::min(m, 16), n, k);
  c.mr = 1;
  if (opts && opts->n_tiles > 0) c.nc = opts->n_tiles;
  if (opts && opts->k_split > 0) {
    c.kw = opts->k_split;
    c.kbw = blocks_per_wave(k / kKBlock, c.kw);
  }
  if (!skinny_config_supported(c, k, gpb)) return W4A8_ERR_INVALID_ARGUMENT;
  return device_status(launch_w4a16_skinny(p, gpb, c, static_cast<hipStream_t>(stream)));
}

extern "C" int w4a8_linear_launches(int m, int n, int k, int g, const w4a8_gemm_opts* opts) {
  if (m <= 0 || m > W4A8_M_MAX || n <= 0 || k <= 0 || !gemm_shape_supported(n, k, g)) return 0;
  const int variant = opts ? opts->variant : 0;
  if (variant < 0 || variant > 3 || !opts_in_range(opts)) return 0;
  const bool fused_ok = fused_config_supported(fused_plan(m, n, k, opts), m, k);
  if (variant == 3) return fused_ok ? 1 : 0;
  if (variant == 0 && fused_ok && fused_by_default(m, n, k)) return 1;
  return plan_gemm(m, n, k, opts).slices > 1 ? 3 : 2;
}

extern "C" w4a8_status w4a8_read_probe(const void* src_dev, size_t bytes, int workgroups,
                                       uint32_t* sink_dev, void* stream) {
  if (bytes == 0) return W4A8_OK;
  if (!src_dev || !sink_dev || bytes % 16 || !aligned16(src_dev) || workgroups < 1 ||
      workgroups > 65536)
    return W4A8_ERR_INVALID_ARGUMENT;
  return device_status(
      launch_read_probe(src_dev, bytes, workgroups, sink_dev, static_cast<hipStream_t>(stream)));
}

extern "C" const char* w4a8_last_device_error(void) {
  return t_last_hip_error == hipSuccess ? "no error" : hipGetErrorString(t_last_hip_error);
}
