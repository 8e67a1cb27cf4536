// Row-major token tiles in LDS for the gfx950 attention kernels: DMA
// staging (global_load_lds_dwordx4), the chunk swizzle, and the types of the
// transposing operand reads (ds_read_b64_tr_b16) that the kernels build on.
//
// A tile row holds one token's 128 bf16 (256 bytes); 16-byte chunk c of row
// r sits at c ^ rsw(r), rsw(r) = 2 (r & 7) + ((r >> 3) & 1).  16 consecutive
// rows reading one chunk each (an MFMA row operand, ds_read_b128) hit 16
// distinct positions, and a transposing read (4 aligned rows x 2 adjacent
// chunks per 16 lanes) hits 8 distinct positions: neither has bank conflicts.
#pragma once

#include "common.h"

namespace pst {

constexpr int kTileRowB = 256;  // tile row: 128 bf16

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

__device__ __forceinline__ int rsw(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

// DMA staging, issued through inline assembly (M0 = LDS base), so the
// compiler does not track it as an LDS store: it then inserts no
// conservative vmcnt(0) before reads of other buffers, and the caller owns
// every wait (vmcnt) and the barrier (whose "memory" clobber orders the LDS
// reads after it).  Each copy takes a wave-uniform base address (an SGPR
// pair) plus a 32-bit lane offset that stays fixed for the whole kernel, so
// a step's staging costs no per-lane 64-bit address arithmetic.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) uint8_t*)(p)));
}
// 16 bytes per lane: base + voff -> LDS lds_base + 16 * lane
__device__ __forceinline__ void dma16_s(const void* base, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_base), "v"(voff), "s"(base)
               : "memory", "m0");
}
// 4 bytes per lane: base + voff -> LDS lds_base + 4 * lane
__device__ __forceinline__ void dma4_s(const void* base, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds_base), "v"(voff), "s"(base)
               : "memory", "m0");
}

// NROWS token rows of 256 bytes (row stride `stride` bytes in memory) ->
// swizzled LDS tile; the NW waves of a workgroup issue NROWS / (4 NW) DMA
// instructions each, instruction n covering rows 4n .. 4n+3.  tile_offsets
// gives the lane's byte offsets within the rows (computed once), dma_tile_s
// issues the copies from a tile's first row `base`.
template <int NROWS, int NW = 4>
struct TileOff {
  static_assert(NROWS % (4 * NW) == 0, "whole instructions per wave");
  static constexpr int kOps = NROWS / (4 * NW);
  uint32_t v[kOps];
};
template <int NROWS, int NW = 4>
__device__ __forceinline__ TileOff<NROWS, NW> tile_offsets(uint32_t stride, int wave, int lane) {
  TileOff<NROWS, NW> o;
#pragma unroll
  for (int i = 0; i < TileOff<NROWS, NW>::kOps; ++i) {
    const int n = TileOff<NROWS, NW>::kOps * wave + i;
    const int r = 4 * n + (lane >> 4);
    o.v[i] = static_cast<uint32_t>(r) * stride + (static_cast<uint32_t>((lane & 15) ^ rsw(r)) << 4);
  }
  return o;
}
template <int NROWS, int NW = 4>
__device__ __forceinline__ void dma_tile_s(const char* base, const TileOff<NROWS, NW>& o, uint32_t dst,
                                           int wave) {
#pragma unroll
  for (int i = 0; i < TileOff<NROWS, NW>::kOps; ++i) {
    const int n = TileOff<NROWS, NW>::kOps * wave + i;
    dma16_s(base, o.v[i], __builtin_amdgcn_readfirstlane(dst + n * 1024));
  }
}

}  // namespace pst
