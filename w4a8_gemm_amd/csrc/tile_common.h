// Device helpers shared by the LDS-tiled GEMM kernels (gfx950): buffer
// resources, direct-to-LDS buffer loads, the vector-memory wait, and the
// XCD-aware mapping of workgroups to output tiles.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {
namespace tile {

static constexpr int kNumXcd = 8;     // MI355X: 8 accelerator complex dies, round-robin dispatch
// row tiles per raster group: the 32 workgroups an XCD runs at once then
// cover 4 row tiles x 8 column tiles, which minimises the distinct
// activation (2 bytes per tile row and k) plus weight (1 per column and k)
// slices per k-block among the shapes of 32 tiles; 4 measured ~1 % faster
// than 8 or 2, and 16 2 % slower, on the Qwen1.5-72B and batched Llama-3-8B
// shapes
static constexpr int kGroupM = 4;

// Raw buffer resource over [base, base + bytes) (gfx9 descriptor, 32-bit
// data format; out-of-range reads return 0).
static __device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_ptr;

// Buffer loads that write straight to LDS: lane i's `size` bytes from
// base + voffset + soffset land at dst + i * size.
static __device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voffset,
                                                uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 16, voffset, soffset, 0, 0);
}
static __device__ __forceinline__ void buffer_to_lds4(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t voffset,
                                               uint32_t soffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)dst, 4, voffset, soffset, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] | expcnt << 4 | lgkmcnt << 8 | vmcnt[5:4] << 14).
template <int N>
static __device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Map the linear workgroup id to (row tile, column tile): XCD-major, then
// grouped raster inside the XCD's share.
static __device__ __forceinline__ void tile_of(int bid, int nbm, int nbn, int* bm, int* bn) {
  const int total = nbm * nbn;
  int logical = bid;
  if (total % kNumXcd == 0) {
    const int per = total / kNumXcd;
    logical = (bid % kNumXcd) * per + bid / kNumXcd;
  }
  const int group_size = kGroupM * nbn;
  const int group = logical / group_size;
  const int first_m = group * kGroupM;
  const int gm = min(nbm - first_m, kGroupM);
  const int in_group = logical % group_size;
  *bm = first_m + in_group % gm;
  *bn = in_group / gm;
}

}  // namespace tile
}  // namespace w4a8
