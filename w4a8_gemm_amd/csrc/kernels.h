// Launch interface between the C ABI layer (api.cpp) and the HIP kernels.
#pragma once
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "../../include/w4a8.h"

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
  int meta_row_bytes;    // meta bytes per output row (groups rounded up to 4)
  uint16_t* y;
  int ldy;
  int32_t* acc;          // optional raw accumulators
  int ldacc;
  int kb_per_wave;       // skinny: 128-k blocks per wave (a multiple of 4 / groups-per-block)
  int32_t* part;         // tiled, K split over workgroups: slices x m x n int32 partial sums
  int kb_per_slice;      // tiled: 128-k blocks per K slice (all of K when not split)
  int8_t* a8_out;        // fused: A8 written by workgroup 0 (row stride lda8)
  uint16_t* s_a_out;     // fused: s_a written by workgroup 0
};

constexpr int kMaxSlices = 16;   // workgroups splitting K of one tile
constexpr long kMaxWorkgroups = (1L << 31) - 1;   // workgroups of one launch
// 17..64 tokens with K >= 8192: from this many activations (M * K) on, 64 x
// 128 tiles with K split over workgroups beat the skinny kernel, whose every
// workgroup re-reads all of A8 (graph replays on MI355X: down projection
// 4096 x 14336 at M = 64 22.5 against 35.1 us, M = 32 20.6 against 21.7;
// 8192 x 8192 at M = 48 20.7 against 21.9, M = 32 20.0 against 16.8)
constexpr long kSplitSmallElems = 393216;

// W4A16 comparison GEMM on the same blob: fp16 activations, fp16 output.
struct Gemm16Params {
  const uint16_t* a;     // m x k fp16, row stride lda elements
  int lda;
  int m;
  const uint8_t* q;
  const uint8_t* meta;
  const uint16_t* s1;
  int n, k;
  int meta_row_bytes;
  uint16_t* y;
  int ldy;
  int kb_per_wave;
};

// Groups per 128-k block: 1, 2 or 4 for g = 128, 64, 32; 0 in per-channel
// mode; -1 in the codebook mode (g == 1: no groups, no meta).
inline int groups_per_block(int k, int g) {
  if (g == 1) return -1;
  if (g == 0 || g == k) return 0;
  return 128 / g;
}

struct SkinnyConfig {
  int mr;    // 16-row tiles per workgroup (1, 2 or 4)
  int nc;    // 16-column tiles per wave (1 or 2)
  int kw;    // waves splitting K inside one workgroup (1..8)
  int kbw;   // 128-k blocks per wave
  int wgs = 0;   // fused kernel: workgroups of the persistent grid (0: one per column-tile group)
};

// Waves along N in every tiled workgroup.
constexpr int kTiledColGroups = 4;

struct TiledConfig {
  int mr;       // 16-row tiles per wave
  int nc;       // 16-column tiles per wave
  int nw;       // waves along N per workgroup (4)
  int rw;       // waves along M per workgroup (1, or 2 for 256 x 256 tiles)
  int kg;       // wave groups splitting the k-blocks inside a workgroup (1 or 2)
  int stages;   // LDS pipeline stages (2 or 3)
};

hipError_t launch_quant_act(const uint16_t* a, int m, int k, int lda, int8_t* a8, int lda8,
                            uint16_t* s_a, hipStream_t stream);
hipError_t launch_quant_act_static(const uint16_t* a, int m, int k, int lda, uint16_t scale_bits,
                                   int8_t* a8, int lda8, uint16_t* s_a, hipStream_t stream);
hipError_t launch_gemm_skinny(const GemmParams& p, int gpb, const SkinnyConfig& c,
                              hipStream_t stream);
// slices > 1: workgroup (tile, slice) covers k-blocks [slice * kb_per_slice,
// +kb_per_slice) and writes its raw int32 tile to p.part; launch_split_reduce
// then adds the slices and applies the epilogue.
hipError_t launch_gemm_tiled(const GemmParams& p, int gpb, const TiledConfig& c, int slices,
                             hipStream_t stream);
hipError_t launch_split_reduce(const GemmParams& p, int slices, hipStream_t stream);
bool skinny_config_supported(const SkinnyConfig& c, int k, int gpb);

hipError_t launch_w4a16_skinny(const Gemm16Params& p, int gpb, const SkinnyConfig& c,
                               hipStream_t stream);
// W4A16 tiled kernel (w4a16.hip): 256 x 128 tiles for larger M, any m >= 1.
hipError_t launch_w4a16_tiled(const Gemm16Params& p, int gpb, hipStream_t stream);

// Fused quantization + skinny GEMM (fused.hip): M <= kFusedMaxRows, one
// row tile, 1 or 2 column tiles per group, 4, 8 or 16 k-blocks per wave with
// rows x blocks per wave <= kFusedMaxHold (the fp16 chunks each lane holds
// while the row maxima are reduced: kFusedMaxHold VGPRs), LDS within
// kFusedMaxLds.
constexpr int kFusedMaxRows = 16;
// Automatic choice (graph-replay timings on MI355X over the Llama-3-8B
// decode layers): every workgroup quantizes all M x K activations, about
// four vector instructions per element, which costs more than the launch it
// saves beyond 57344 elements (M = 14 at K = 4096, M = 4 at K = 14336; up
// to there the fused layer is 0.1-3 us faster), or beyond 65536 elements on
// layers of at least kFusedWideTiles column tiles, whose workgroups walk
// several tile groups and so quantize once for more weights (gate+up at
// M = 16: 16.6 against 18.0 us).  The persistent grid holds at most one
// workgroup per compute unit (256 on MI355X), and fewer where that evens out
// the groups each one walks without adding a round: 224 workgroups of 4
// groups beat 256 of 3 or 4 (gate+up above 2 tokens, 896 groups: 13.4
// against 13.8 us at M = 4).  Groups hold one column tile, except on
// layers of more than kFusedPairTiles tiles above 2 tokens, where two tiles
// per group halve the per-group split-K sums and barriers.
constexpr long kFusedAutoElems = 57344;
constexpr long kFusedWideElems = 65536;
constexpr int kFusedWideTiles = 1024;
constexpr int kFusedPairTiles = 512;
constexpr int kFusedAutoWgs = 256;
constexpr int kFusedMaxHold = 64;
constexpr size_t kFusedMaxLds = 128 * 1024;
size_t fused_lds_bytes(int kw, int nc, int m, int kbw);
// Rows of the fused kernel's tile: m rounded up to a power of two (1..16).
int fused_rows(int m);
bool fused_config_supported(const SkinnyConfig& c, int m, int k);
hipError_t launch_gemm_fused(const GemmParams& p, const uint16_t* a, int lda, int gpb,
                             const SkinnyConfig& c, hipStream_t stream);
bool tiled_config_supported(const TiledConfig& c);

// The static scratch buffer of w4a8_gemm_noalloc (scratch.hip): bytes per
// device, and its device address for the current device (looked up once
// per device by hipGetSymbolAddress).
constexpr size_t kScratchBytes = W4A8_SCRATCH_BYTES;
hipError_t scratch_address(void** ptr);

// Read-only stream over `bytes` (a multiple of 16) with `workgroups` x 512
// threads (probe.hip); a measurement aid, not part of the layer.
hipError_t launch_read_probe(const void* src, size_t bytes, int workgroups, uint32_t* sink,
                             hipStream_t stream);

}  // namespace w4a8
