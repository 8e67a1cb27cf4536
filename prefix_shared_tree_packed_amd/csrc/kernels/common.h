// Shared device-side definitions for the gfx950 (CDNA4) kernels of libpst:
// element types, MFMA fragment types, the per-tree metadata view, and small
// wave-level helpers.  Wave size is 64 everywhere.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pst {

typedef uint16_t bf16_t;  // bf16 storage (the upper half of an fp32)

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kTile = 128;  // BLOCK_SIZE: queries and keys per tile
// Persistent dK/dV workgroups: key-block lists for 1, 2, 4, ..., kMaxLanes
// lanes per key/value group
constexpr int kLaneLevels = 9;
constexpr int kMaxLanes = 1 << (kLaneLevels - 1);

// Device view of one packed tree's metadata (one device allocation; see
// tree_meta in capi.cpp for the layout).
struct TreeDev {
  const int32_t* se;           // [Np] subtree end of every key
  const int32_t* q_ptr;        // [nb+1] tiles of each query block
  const int32_t* q_tile;       // [n_tiles] (key block << 1) | full
  const int32_t* kb_qhi;       // [nb] last query block seeing each key block
  const int32_t* fwd_order;    // [nb] query blocks by first key block, heaviest first
  const int32_t* bwd_order;    // [nb] key blocks by range end, longest range first
  const int32_t* row_out_ptr;  // [Np+1] outputs of each row (none for pad rows)
  const int32_t* out_pos;      // [n_out] output slot
  const int32_t* out_tgt;      // [n_out] next-token id, -1 for a last token
  const int32_t* blk32;        // [Np/32][2] min and max subtree end of each 32-key block
  const int32_t* q_cls;        // [n_tiles] 2-bit class of each 32x32 sub-block (query
                               // sub-block qs, key sub-block ks at bit 2*(4*qs+ks)):
                               // 0 no visible pair, 1 some, 2 all
  const int32_t* pos;          // [Np] depth of every row (position id), 0 for pad rows
  const int32_t* step_ptr;     // [nb+1] steps of each query block
  const int32_t* steps;        // [n_steps] non-empty 32-key columns of the block's tiles:
                               // (32-key block << 8) | class of 32-query sub-block qs
                               // at bits 2 qs (0 no visible pair, 1 some, 2 all)
  const int32_t* unit_ptr;     // [Np/32+1] blocks of each 32-query unit
  const int32_t* unit_steps;   // [n_blk32] non-empty 32x32 blocks of a unit:
                               // (32-key block << 2) | class (1 some, 2 all)
  const int32_t* unit_order;   // [Np/32] units, grouped by first key block
  const int32_t* bwd_lanes;    // for P = 2^i lanes (i < kLaneLevels), in turn: [P+1]
                               // lane offsets, then [nb] key blocks, lane by lane
  int32_t N;
  int32_t Np;
  int32_t nb;
  int32_t n_tiles;
};

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Two fp32 -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of lane (lane ^ 32): swaps the two halves of the wave.
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

// Both halves' values at every lane: {x[l % 32], x[32 + l % 32]} for lane l,
// by one v_permlane32_swap (a VALU op; a shuffle through ds_bpermute costs an
// LDS round trip).
__device__ __forceinline__ void half_pair(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_halves(float x) {
  float a, b;
  half_pair(x, a, b);
  return a + b;
}

// Linear workgroup id -> logical work id such that consecutive logical ids
// land on the same XCD.  Workgroups are dispatched round-robin over the 8
// XCDs, so XCD x receives linear ids x, x+8, x+16, ...; those become the
// logical range [x*per, (x+1)*per).  Identity when the grid is not a
// multiple of 8.
__device__ __forceinline__ int xcd_remap(int b, int total) {
  constexpr int kXcd = 8;
  if (total % kXcd) return b;
  return (b % kXcd) * (total / kXcd) + b / kXcd;
}

}  // namespace pst
