// Packed-blob layout v1, shared by the host packer and the GPU launchers.
//
// The weight codes are stored in the order the gfx950 int8 MFMA
// (v_mfma_i32_16x16x64_i8) consumes its B operand, so that one 128-bit load
// per lane brings the codes for two consecutive 64-deep k-steps of one
// column and decode happens in registers, with no LDS round trip for the
// weights (the offline interleaving idea of the QUICK abstract and the
// offline restructuring of the FLUTE abstract, re-derived for the 64-wide
// wavefront).
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "codebook.h"

namespace w4a8 {

constexpr int kKBlock = 128;     // k covered by one 16-byte lane chunk (2 MFMA k-steps)
constexpr int kColTile = 16;     // output columns per MFMA tile
constexpr int kHeaderBytes = 256;
constexpr uint32_t kLayoutVersion = 1;
constexpr char kMagic[8] = {'W', '4', 'A', '8', 'B', 'L', 'O', 'B'};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Group length actually used: g for grouped mode, K for per-channel mode.
inline int effective_group(int k, int g) { return (g == 0 || g == k) ? k : g; }

struct Sections {
  size_t q_off, q_bytes;
  size_t meta_off, meta_bytes;
  size_t s1_off, s1_bytes;
  size_t total;
  int groups;         // groups per row
  int meta_row_bytes; // groups per row rounded up to a multiple of 4
};

// In the codebook mode (g == kCodebookG) there are no groups and no meta
// section: a code decodes through the fixed level table alone.
inline Sections sections(int n, int k, int g) {
  Sections s;
  if (g == kCodebookG) {
    s.groups = 0;
    s.meta_row_bytes = 0;
  } else {
    int ge = effective_group(k, g);
    s.groups = k / ge;
    s.meta_row_bytes = (s.groups + 3) & ~3;
  }
  s.q_off = kHeaderBytes;
  s.q_bytes = size_t(n) * size_t(k) / 2;
  s.meta_off = s.q_off + align256(s.q_bytes);
  s.meta_bytes = size_t(n) * size_t(s.meta_row_bytes);
  s.s1_off = s.meta_off + align256(s.meta_bytes);
  s.s1_bytes = size_t(n) * 2;
  s.total = s.s1_off + align256(s.s1_bytes);
  return s;
}

// Byte offset (inside the q section) and nibble (0 low, 1 high) of code (n, k).
inline void q_position(int n, int k, int kblocks, size_t* byte, int* nibble) {
  int t = n / kColTile, r = n % kColTile;
  int b = k / kKBlock, kk = k % kKBlock;
  int h = kk / 64, quarter = (kk % 64) / 16, j = kk % 16;
  int lane = quarter * 16 + r;
  int dword = 2 * h + j / 8;
  int jj = j % 8;
  *byte = ((size_t(t) * kblocks + b) * 64 + lane) * 16 + dword * 4 + (jj % 4);
  *nibble = jj / 4;
}

// Byte offset (inside the meta section) of group `grp` of row n: one row of
// meta bytes per output row, padded to whole dwords so that a lane can fetch
// four consecutive groups of its row with one 32-bit load.
inline size_t meta_position(int n, int grp, int meta_row_bytes) {
  return size_t(n) * size_t(meta_row_bytes) + size_t(grp);
}

}  // namespace w4a8
