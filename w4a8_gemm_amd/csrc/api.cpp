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
  if (n % kColTile || k % kKBlock || k > W4A8_K_MAX) return false;
  if (g == W4A8_GROUP_PER_CHANNEL || g == k) return true;
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
  c.kw = (kblocks + c.kbw - 1) / c.kbw;
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
  if (m < 0 || k <= 0 || lda < k || lda8 < k) return W4A8_ERR_INVALID_ARGUMENT;
  if (m == 0) return W4A8_OK;
  if (!a_dev || !a8_dev || !s_a_dev) return W4A8_ERR_INVALID_ARGUMENT;
  return device_status(launch_quant_act(a_dev, m, k, lda, a8_dev, lda8, s_a_dev,
                                        static_cast<hipStream_t>(stream)));
}

extern "C" size_t w4a8_gemm_workspace_size(int m, int n, int k, int g) {
  (void)m;
  (void)n;
  (void)k;
  (void)g;
  return 0;  // both variants reduce split-K partials on chip
}

extern "C" w4a8_status w4a8_gemm(const int8_t* a8_dev, int lda8, const uint16_t* s_a_dev, int m,
                                 const void* blob_dev, int n, int k, int g, uint16_t* y_dev,
                                 int ldy, int32_t* acc_dev, int ldacc, void* workspace_dev,
                                 size_t workspace_bytes, const w4a8_gemm_opts* opts,
                                 void* stream) {
  (void)workspace_dev;
  if (m < 0 || n <= 0 || k <= 0 || g < 0) return W4A8_ERR_INVALID_ARGUMENT;
  if (!gemm_shape_supported(n, k, g)) return W4A8_ERR_UNSUPPORTED;
  if (m == 0) return W4A8_OK;
  if (!a8_dev || !s_a_dev || !blob_dev || !y_dev) return W4A8_ERR_INVALID_ARGUMENT;
  if (lda8 < k || lda8 % 16 || ldy < n || (acc_dev && ldacc < n)) return W4A8_ERR_INVALID_ARGUMENT;
  if (!aligned16(a8_dev) || !aligned16(blob_dev)) return W4A8_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < w4a8_gemm_workspace_size(m, n, k, g)) return W4A8_ERR_BUFFER_TOO_SMALL;

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
  const int gpb = groups_per_block(k, g);
  p.y = y_dev;
  p.ldy = ldy;
  p.acc = acc_dev;
  p.ldacc = acc_dev ? ldacc : 0;

  int variant = opts ? opts->variant : 0;
  if (variant < 0 || variant > 2) return W4A8_ERR_INVALID_ARGUMENT;
  if (variant == 0) variant = m <= 64 ? 1 : 2;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (variant == 1) {
    if (m > 64) return W4A8_ERR_UNSUPPORTED;
    SkinnyConfig c = choose_skinny(m, n, k);
    if (opts && opts->n_tiles > 0) c.nc = opts->n_tiles;
    if (opts && opts->k_split > 0) {
      c.kw = opts->k_split;
      c.kbw = blocks_per_wave(k / kKBlock, c.kw);
    }
    if (!skinny_config_supported(c, k, gpb)) return W4A8_ERR_INVALID_ARGUMENT;
    e = launch_gemm_skinny(p, gpb, c, s);
  } else {
    // Tiled (choices from timing sweeps on the layer shapes): 256 x 256
    // tiles of eight waves with 3 stages when they fill every compute unit
    // at least once; else 128 x 256 tiles of four waves with 2 stages (two
    // workgroups per compute unit) when there are enough of them; else
    // 64 x 256 tiles with 3 stages.
    TiledConfig c;
    c.nw = 4;
    c.nc = 4;
    const long col256 = long((n / kColTile + 15) / 16);
    const long tiles256 = long((m + 255) / 256) * col256;
    const long tiles128 = long((m + 127) / 128) * col256;
    c.rw = tiles256 >= 256 ? 2 : 1;
    // a forced row-tile count or stage count without a forced row-group
    // count selects among the four-wave kernels
    if (opts && (opts->m_tiles > 0 || opts->stages > 0)) c.rw = 1;
    if (opts && opts->row_groups > 0) c.rw = opts->row_groups;
    c.mr = (c.rw == 2 || tiles128 >= 192) ? 8 : 4;
    if (opts && opts->m_tiles > 0) c.mr = opts->m_tiles;
    c.stages = (c.rw == 2 || c.mr == 4) ? 3 : 2;
    if (opts && opts->stages > 0) c.stages = opts->stages;
    if (opts && opts->n_tiles > 0) c.nc = opts->n_tiles;
    if (!tiled_config_supported(c)) return W4A8_ERR_INVALID_ARGUMENT;
    e = launch_gemm_tiled(p, gpb, c, s);
  }
  return device_status(e);
}

extern "C" const char* w4a8_last_device_error(void) {
  return t_last_hip_error == hipSuccess ? "no error" : hipGetErrorString(t_last_hip_error);
}
