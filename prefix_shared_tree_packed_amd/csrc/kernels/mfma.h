// MFMA fragment helpers for the attention kernels (gfx950).
//
// Both element types use a 32x32 output tile per wave (16 fp32 accumulators
// per lane):
//   bf16: v_mfma_f32_32x32x16_bf16, 16-deep contraction, 8 bf16 per lane;
//   fp32: v_mfma_f32_32x32x2_f32,    2-deep contraction, 1 fp32 per lane.
// Operand layout (lane l, half = l / 32): the A operand holds row l % 32 and
// contraction slots [half*E, half*E + E); the B operand holds column l % 32
// and the same slots; accumulator r = 4*i + j holds row 8*i + 4*half + j,
// column l % 32.
//
// The attention kernels compute S^T = K.Q^T so that a lane owns one query
// (column) and its scores run down the registers.  Feeding those registers
// back as the B operand of O^T += V^T.P^T needs the contraction slots of a
// step to be mapped to keys in accumulator order: slot m of half `half` in
// step t is accumulator register E*t + m, i.e. key 8*i + 4*half + j of the
// 32-key block with i = (E*t+m)/4, j = (E*t+m)%4.  The A operand (V^T, read
// from LDS) is gathered with the same slot->key map, so the product is exact.
#pragma once

#include "common.h"

namespace pst {

template <typename T>
struct Mfma;

template <>
struct Mfma<bf16_t> {
  static constexpr int KS = 16;  // contraction depth per instruction
  static constexpr int E = 8;    // operand elements per lane
  typedef bf16x8_t Frag;
  static __device__ __forceinline__ f32x16_t mma(Frag a, Frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // E contiguous elements starting at p (16-byte aligned).
  static __device__ __forceinline__ Frag load(const bf16_t* p) {
    return __builtin_bit_cast(Frag, *reinterpret_cast<const uint4*>(p));
  }
  // Slots of step t from an fp32 accumulator: registers 8t..8t+7.
  static __device__ __forceinline__ Frag from_acc(const f32x16_t& acc, int t) {
    typedef float f32x8_t __attribute__((ext_vector_type(8)));
    f32x8_t x = {acc[8 * t + 0], acc[8 * t + 1], acc[8 * t + 2], acc[8 * t + 3],
                 acc[8 * t + 4], acc[8 * t + 5], acc[8 * t + 6], acc[8 * t + 7]};
    return __builtin_convertvector(x, bf16x8_t);
  }
  // Slots of step t gathered from a key-contiguous LDS row (row[key]):
  // keys 16t + 4*half + 0..3 and 16t + 8 + 4*half + 0..3 of the 32-key block.
  static __device__ __forceinline__ Frag gather_keys(const bf16_t* row, int t, int half) {
    const uint2 lo = *reinterpret_cast<const uint2*>(row + 16 * t + 4 * half);
    const uint2 hi = *reinterpret_cast<const uint2*>(row + 16 * t + 8 + 4 * half);
    const uint4 v = {lo.x, lo.y, hi.x, hi.y};
    return __builtin_bit_cast(Frag, v);
  }
};

template <>
struct Mfma<float> {
  static constexpr int KS = 2;
  static constexpr int E = 1;
  typedef float Frag;
  static __device__ __forceinline__ f32x16_t mma(Frag a, Frag b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Frag load(const float* p) { return *p; }
  static __device__ __forceinline__ Frag from_acc(const f32x16_t& acc, int t) { return acc[t]; }
  // Slot of step t: accumulator register t -> key 8*(t/4) + 4*half + t%4.
  static __device__ __forceinline__ Frag gather_keys(const float* row, int t, int half) {
    return row[8 * (t / 4) + 4 * half + (t % 4)];
  }
};

// Key (0..31 within a 32-key block) held by accumulator register r of a lane
// in wave half `half`.
__device__ __forceinline__ int acc_key(int r, int half) { return 8 * (r / 4) + 4 * half + (r % 4); }

// Writes four key rows of one 16-byte chunk (rows[j] = 16 bytes of key
// key0+j, elements d0..d0+EPC-1) into a d-major LDS array dst[d][key].
template <typename T>
__device__ __forceinline__ void store_transposed(T* dst, int stride, int d0, int key0,
                                                 const uint4 (&rows)[4]);

template <>
__device__ __forceinline__ void store_transposed<bf16_t>(bf16_t* dst, int stride, int d0,
                                                         int key0, const uint4 (&rows)[4]) {
  const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&rows[0]);
  const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&rows[1]);
  const uint32_t* r2 = reinterpret_cast<const uint32_t*>(&rows[2]);
  const uint32_t* r3 = reinterpret_cast<const uint32_t*>(&rows[3]);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    // element 2p: low halves; element 2p+1: high halves
    const uint2 even = {(r0[p] & 0xffffu) | (r1[p] << 16), (r2[p] & 0xffffu) | (r3[p] << 16)};
    const uint2 odd = {(r0[p] >> 16) | (r1[p] & 0xffff0000u), (r2[p] >> 16) | (r3[p] & 0xffff0000u)};
    *reinterpret_cast<uint2*>(dst + (d0 + 2 * p) * stride + key0) = even;
    *reinterpret_cast<uint2*>(dst + (d0 + 2 * p + 1) * stride + key0) = odd;
  }
}

template <>
__device__ __forceinline__ void store_transposed<float>(float* dst, int stride, int d0, int key0,
                                                        const uint4 (&rows)[4]) {
  const uint4 c0 = {rows[0].x, rows[1].x, rows[2].x, rows[3].x};
  const uint4 c1 = {rows[0].y, rows[1].y, rows[2].y, rows[3].y};
  const uint4 c2 = {rows[0].z, rows[1].z, rows[2].z, rows[3].z};
  const uint4 c3 = {rows[0].w, rows[1].w, rows[2].w, rows[3].w};
  *reinterpret_cast<uint4*>(dst + (d0 + 0) * stride + key0) = c0;
  *reinterpret_cast<uint4*>(dst + (d0 + 1) * stride + key0) = c1;
  *reinterpret_cast<uint4*>(dst + (d0 + 2) * stride + key0) = c2;
  *reinterpret_cast<uint4*>(dst + (d0 + 3) * stride + key0) = c3;
}

// Four fp32 values -> four elements of T at p (8-byte aligned for bf16,
// 16-byte for fp32).
template <typename T>
__device__ __forceinline__ void store4(T* p, float a, float b, float c, float d);

template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, float a, float b, float c, float d) {
  const uint2 v = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
  *reinterpret_cast<uint2*>(p) = v;
}

template <>
__device__ __forceinline__ void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}

}  // namespace pst
