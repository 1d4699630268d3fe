// The 16 levels of the non-uniform (NormalFloat-style) 4-bit weight code,
// used by the packer and decoded by the GEMM kernels (the LUT-quantized
// weights of the FLUTE page, section 方法详解, with the table held in
// registers rather than shared memory).
//
// Reading (the page prints no levels): the standard-normal quantiles at the
// probabilities (i + 1/2) / 16, i = 0..15, scaled so that the largest is 119
// (the level-1 int8 range, so every decoded weight is an int8 MFMA operand)
// and rounded half-to-even.  Code i decodes to kNfLevels[i]; the packer picks
// the level nearest to the level-1 int8 value, ties to the lower code.
#pragma once
#include <stdint.h>

namespace w4a8 {

constexpr int kCodebookG = 1;   // the group-size value that selects this code
constexpr int8_t kNfLevels[16] = {-119, -84, -65, -50, -37, -26, -15, -5,
                                  5,    15,  26,  37,  50,  65,  84,  119};

// the levels as four little-endian dwords (levels 4i .. 4i+3 in dword i)
constexpr uint32_t nf_dword(int i) {
  return uint32_t(uint8_t(kNfLevels[4 * i])) | (uint32_t(uint8_t(kNfLevels[4 * i + 1])) << 8) |
         (uint32_t(uint8_t(kNfLevels[4 * i + 2])) << 16) |
         (uint32_t(uint8_t(kNfLevels[4 * i + 3])) << 24);
}

}  // namespace w4a8
