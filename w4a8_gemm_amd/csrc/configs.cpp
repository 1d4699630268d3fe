// Host-side checks of kernel configurations: which tile shapes, pipeline
// depths and fused-kernel plans have a compiled kernel and fit a compute
// unit's LDS.  Plain C++ with no device code, so that the C ABI's argument
// validation can also be built for the host alone.
#include <stddef.h>

#include "kernels.h"

namespace w4a8 {
namespace {

// Four-wave tiles (RW = KG = 1) and their pipeline depths.  Deeper
// pipelines keep more k-blocks in flight per workgroup, which is what a
// grid of about one workgroup per compute unit needs to cover the memory
// latency; each depth fits the 160 KB of LDS and the vmcnt range.
bool four_wave_stages_ok(int mr, int nc, int s) {
  if (mr == 8 && nc == 4) return s >= 2 && s <= 4;
  if (mr == 4 && nc == 4) return s >= 2 && s <= 5;
  if (mr == 8 && nc == 2) return s >= 2 && s <= 6;
  if (mr == 4 && nc == 2) return s == 2 || s == 3 || s == 4 || s == 6 || s == 8;
  return false;
}

// Two k-groups of four waves (eight waves, KG = 2): the 256-column tiles
// with 2 stages, the 128-column tiles deeper.
bool two_group_stages_ok(int mr, int nc, int s) {
  if (nc == 4) return (mr == 8 || mr == 4) && s == 2;
  if (mr == 8 && nc == 2) return s == 2 || s == 3;
  if (mr == 4 && nc == 2) return s >= 2 && s <= 4;
  return false;
}

}  // namespace

bool tiled_config_supported(const TiledConfig& c) {
  if (c.nw != kTiledColGroups) return false;
  if (c.rw == 2) return c.kg == 1 && c.mr == 8 && c.nc == 4 && c.stages == 3;
  if (c.kg == 2) return c.rw == 1 && two_group_stages_ok(c.mr, c.nc, c.stages);
  return c.rw == 1 && c.kg == 1 && four_wave_stages_ok(c.mr, c.nc, c.stages);
}

bool skinny_config_supported(const SkinnyConfig& c, int k, int gpb) {
  const bool shape_ok = (c.mr == 1 && (c.nc == 1 || c.nc == 2 || c.nc == 4)) ||
                        ((c.mr == 2 || c.mr == 4) && (c.nc == 1 || c.nc == 2));
  if (!shape_ok) return false;
  (void)gpb;
  if (c.kw < 1 || c.kw > 8 || c.kbw < 1 || c.kbw % 4) return false;   // ring groups of 4
  return c.kw * c.kbw * 128 >= k;                    // the waves cover all of K
}

size_t fused_lds_bytes(int kw, int nc, int m, int kbw) {
  const size_t red = kw > 1 ? 2 * size_t(kw) * nc * 1024 : 0;
  return size_t(kw) * 64 + red + size_t(kw) * m * (size_t(kbw) * 128 + 16);
}

int fused_rows(int m) { return m <= 1 ? 1 : (m <= 2 ? 2 : (m <= 4 ? 4 : (m <= 8 ? 8 : 16))); }

bool fused_config_supported(const SkinnyConfig& c, int m, int k) {
  if (m < 1 || m > kFusedMaxRows || c.mr != 1) return false;
  if (c.nc != 1 && c.nc != 2) return false;
  if (c.kw < 1 || c.kw > 8 || !(c.kbw == 4 || c.kbw == 8 || c.kbw == 16)) return false;
  if (c.kw * c.kbw * 128 < k) return false;
  if (fused_rows(m) * c.kbw > kFusedMaxHold) return false;
  if (c.wgs < 0) return false;
  return fused_lds_bytes(c.kw, c.nc, m, c.kbw) <= kFusedMaxLds;
}

}  // namespace w4a8
