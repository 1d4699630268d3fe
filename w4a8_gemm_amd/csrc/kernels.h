// Launch interface between the C ABI layer (api.cpp) and the HIP kernels.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace w4a8 {

struct GemmParams {
  const int8_t* a8;
  int lda8;
  const uint16_t* s_a;
  int m;
  const uint8_t* q;      // q section of the device blob
  const uint8_t* meta;   // meta section
  const uint16_t* s1;    // s1 section
  int n, k;
  int groups;            // groups per row (K / g, or 1 per channel)
  int gpb_shift;         // log2(groups per 128-k block) for g in {128,64,32}; -1 per channel
  uint16_t* y;
  int ldy;
  int32_t* acc;          // optional raw accumulators
  int ldacc;
};

struct SkinnyConfig {
  int mr;   // 16-row tiles per workgroup (1, 2 or 4)
  int nc;   // 16-column tiles per wave (1, 2 or 4)
  int kw;   // waves splitting K inside one workgroup (1..16)
};

struct TiledConfig {
  int mr;   // 16-row tiles per wave
  int nc;   // 16-column tiles per wave
  int nw;   // waves along N per workgroup
};

hipError_t launch_quant_act(const uint16_t* a, int m, int k, int lda, int8_t* a8, int lda8,
                            uint16_t* s_a, hipStream_t stream);
hipError_t launch_gemm_skinny(const GemmParams& p, const SkinnyConfig& c, hipStream_t stream);
hipError_t launch_gemm_tiled(const GemmParams& p, const TiledConfig& c, hipStream_t stream);
bool skinny_config_supported(const SkinnyConfig& c);
bool tiled_config_supported(const TiledConfig& c);

}  // namespace w4a8
