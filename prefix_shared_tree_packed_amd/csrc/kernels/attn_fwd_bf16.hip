// Tree attention forward pass, bf16 with head_dim 128: the performance path
// on gfx950.  Same mathematics as attn_fwd.hip.  A workgroup is four waves of
// 32 query rows: for the largest multiple of four of each key/value group's
// query heads, the four waves are four heads of the group on the same 32
// queries (a "unit": every wave has work in every step, and each staged K/V
// tile serves four heads); for the remaining heads they are the four 32-row
// slices of one 128-query block of one head.  How every step is fed:
//
//  * All products use v_mfma_f32_16x16x32_bf16.  A wave's 32 queries x 32
//    keys of scores are four 16x16 blocks, accumulated as four independent
//    chains over the four 32-deep slices of the head dimension (a dependent
//    MFMA waits for its predecessor's result, so one chain alone would run
//    at a fraction of the matrix core's rate), and O^T is sixteen
//    independent 16x16 blocks.  S^T = K.Q^T puts one query in each lane
//    column: a lane holds four keys of each block, so a query's row
//    reductions span the four 16-lane groups (three permlane swaps serve
//    both 16-query halves at once).
//  * The unit's non-empty 32x32 blocks (or the block's non-empty 32-key
//    columns, dropping columns no wave sees), listed by the host, are walked
//    through a three-stage LDS ring: while the waves compute one step, the K and V rows
//    and subtree ends of the step after next stream global -> LDS directly
//    (global_load_lds_dwordx4: no VGPRs, no VALU) into row-major tiles
//    (swizzle of lds_tiles.h); one barrier per step, two steps in flight.
//    Each copy takes the step's base address in SGPRs and a lane offset
//    fixed for the whole kernel, so staging costs no per-lane address
//    arithmetic (the per-lane 64-bit form cost ~10 % of the kernel's time,
//    VALU issue and registers); in units they are spread over the S^T
//    MFMAs.  48 KB of LDS and at most 168 VGPRs let three workgroups share
//    a CU.
//  * LDS operand reads run ahead of the MFMAs that use them: K one
//    fragment, V^T two d blocks (held in place by a scheduling barrier,
//    since the compiler otherwise sinks loads back to their use).
//  * K rows are the A operand of S^T = K.Q^T as they stand (one 16-byte read
//    per operand, shared by the two 16-query halves); the V^T operands of
//    O^T += V^T.P^T come from the same row-major V tile through two
//    ds_read_b64_tr_b16 transposing reads, whose key order is the order in
//    which the score registers feed P^T.
//  * The mask is evaluated per (wave, 32-key block): a block whose keys no
//    query of the wave sees is skipped (no MFMA, no exp), a block every query
//    sees runs unmasked, and only the rest pay a per-element test under one
//    branch: i <= se[j] alone off the diagonal (one compare), plus j <= i as
//    a second pass on the diagonal block.
//  * Scores stay unscaled; the softmax scale is folded into the exponent's
//    FMA, and the running max is refreshed lazily: O and the row sums are
//    rescaled only when a row's max grows by more than 2^8, so exponentials
//    stay below 256 and most steps skip the rescale.  Row sums stay per lane
//    (each lane's own keys) until the end, and are taken on the bf16
//    probabilities that O accumulates, two per v_dot2 against (1, 1).
#include "launch.h"
#include "lds_tiles.h"
#include "mfma.h"

#include <cmath>

namespace pst {
namespace {

constexpr int D = 128;
constexpr int kStep = 32;              // keys per pipeline step
constexpr int kKRow = D * 2;              // K row: 256 B
constexpr int kBufBytes = kStep * kKRow;  // 8 KB for K, 8 KB for V
constexpr int kHalfTile = 16 * kKRow;     // byte offset of keys 16..31 of a step tile
constexpr float kRescale = 8.0f;          // lazy-rescale threshold (log2 units)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
constexpr bf16x2_t kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};

typedef const __attribute__((address_space(4))) int32_t cint32;  // read-only: scalar loads

__device__ __forceinline__ cint32* cst(const int32_t* p) { return (cint32*)(p); }

__device__ __forceinline__ f32x4_t mma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t lds_frag(const uint8_t* base, int byte_off) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(base + byte_off));
}

// max without NaN quieting: the scores are finite or -inf, and permlane
// results would otherwise be canonicalised first (two extra VALU ops each)
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Row maxima of both query halves at once: on entry x (y) holds each lane's
// partial max of query half 0 (1); on return every lane holds, in x and y,
// the max over the four lanes l % 16 + 16 g (g = 0..3) of its query.  Three
// swaps serve both halves: after the first, rows 0, 2 carry x and rows 1, 3
// carry y; the 32-lane swap folds rows 0 + 2 and 1 + 3; the last 16-lane
// swap spreads x and y back over all four rows.
__device__ __forceinline__ void quad_max2(float& x, float& y) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  const float m1 = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m1), __float_as_uint(m1), false, false);
  const float m2 = vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(m2), __float_as_uint(m2), false, false);
  x = __uint_as_float(c[0]);
  y = __uint_as_float(c[1]);
}
// Sum over the four lanes l % 16 + 16 g (g = 0..3) that hold one query.
__device__ __forceinline__ float quad_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  return sum_halves(y);
}

// V^T operand of one 16-row d block from a row-major V step tile: lane
// (group g, index i) gets d = 16 db + i of keys 4g .. 4g+3 (slots 0..3) and
// 16 + 4g .. 16 + 4g + 3 (slots 4..7), the key order of the score registers.
// `trv` is the lane's byte offset for db = 0 (d blocks differ in bits 5..7).
__device__ __forceinline__ bf16x8_t lds_vt_frag(const uint8_t* tile, int trv, int db) {
  const int off = trv ^ (db << 5);
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + off));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + kHalfTile + off));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, w);
}

// A unit workgroup is one 32-query unit of NW heads of one key/value group
// (one wave per head, same queries) and walks the unit's non-empty 32x32
// blocks: every wave has work in every step, and the staged K/V tile serves
// NW heads.  A block workgroup is one 128-query block of one head (four
// waves of 32 queries) and walks the block's non-empty 32-key columns.
// MODE 0: 128-query blocks only; 1: units only (heads per group a multiple
// of four); 2: mixed, for a group size G = 4 m + r: the first workgroups
// are units of the group's first 4 m heads, the rest 128-query blocks of
// its last r heads.
template <int MODE, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 ? 3 : 2) void tree_attn_fwd_bf16_d128(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    bf16_t* __restrict__ o, float* __restrict__ lse, TreeDev tr, int hq, int hkv, float c) {
  // two separately named buffers (not one array indexed by the step parity)
  // so the compiler can tell the in-flight DMA target from the buffer being
  // read and does not drain the prefetch before every LDS read
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds2[kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds0[kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds1[kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t v_lds2[kBufBytes];
  __shared__ __attribute__((aligned(16))) int32_t se_lds0[kStep];
  __shared__ __attribute__((aligned(16))) int32_t se_lds1[kStep];
  __shared__ __attribute__((aligned(16))) int32_t se_lds2[kStep];

  const int G = hq / hkv;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int tid = threadIdx.x;
  // wave index as a scalar, so the per-wave block classes branch on SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int li = lane % 16;  // query column of the 16x16 blocks
  const int lg = lane / 16;  // 16-lane group: keys 4 lg .. 4 lg + 3 of each block
  // logical work ids run group by group (so each XCD keeps one group's K/V
  // in its L2): first the group's units, then its 128-query blocks
  const int G4 = MODE == 0 ? 0 : G / NW * NW;  // heads of each group served by units
  const int GR = G - G4;                       // heads served by 128-query blocks
  const int per_unit = MODE == 0 ? 1 : G4 / NW;  // unit workgroups per unit and group
  const int u_g = MODE == 0 ? 0 : per_unit * (tr.Np / 32);  // unit workgroups per group
  const int per_g = u_g + GR * tr.nb;
  const int g = logical / per_g;
  const int rem = logical - g * per_g;
  const bool UNIT = rem < u_g;
  int h, qlo, n_steps;
  cint32* steps;
  if (UNIT) {
    const int rank = rem / per_unit;
    h = g * G + (rem - rank * per_unit) * NW + wave;
    const int u = cst(tr.unit_order)[rank];
    qlo = u * 32;
    steps = cst(tr.unit_steps) + cst(tr.unit_ptr)[u];
    n_steps = cst(tr.unit_ptr)[u + 1] - cst(tr.unit_ptr)[u];
  } else {
    const int rb = rem - u_g;
    const int rank = rb / GR;
    h = g * G + G4 + (rb - rank * GR);
    const int qb = cst(tr.fwd_order)[rank];
    qlo = qb * kTile + wave * 32;  // first query row of this wave
    // the query block's non-empty 32-key columns (scalar metadata reads)
    steps = cst(tr.steps) + cst(tr.step_ptr)[qb];
    n_steps = cst(tr.step_ptr)[qb + 1] - cst(tr.step_ptr)[qb];
  }

  bf16x8_t qf[2][4];  // B operands of S^T = K.Q^T, loaded below
  // A operands: key row li (+16 for the second key half), chunk 4 s + lg
  int koff[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) koff[s] = li * kKRow + (((4 * s + lg) ^ rsw(li)) << 4);
  // V^T reads: lane i of group lg addresses key 4 lg + i / 4 at d = 4 (i % 4) .. +3
  int trv;
  {
    const int t = 4 * lg + li / 4;
    const int a = li % 4;
    trv = t * kKRow + ((((a >> 1) ^ rsw(t))) << 4) + ((a & 1) << 3);
  }

  // Global loads: a wave-uniform base pointer plus a 32-bit lane offset.
  const uint32_t kv_bytes = static_cast<uint32_t>(hkv) * D * 2;  // one token's K (or V) rows
  const char* kgb = reinterpret_cast<const char*>(k + static_cast<size_t>(g) * D);
  const char* vgb = reinterpret_cast<const char*>(v + static_cast<size_t>(g) * D);

  f32x4_t oacc[8][2];  // O^T block (d block db, query half qh)
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db][0] = oacc[db][1] = f32x4_t{};
  float m_used[2] = {-INFINITY, -INFINITY};
  float negm[2] = {0.f, 0.f};    // -m_used, 0 while m_used is -inf
  float l_part[2] = {0.f, 0.f};  // this lane's share of each row sum

  const int step_shift = UNIT ? 2 : 8;
  auto step_key0 = [&](int st) { return (steps[st] >> step_shift) * kStep; };

  // Staging of one step: the subtree ends of its keys (eight lanes of wave
  // 0) and its K and V rows, all global -> LDS.  Every wave issues kDmaOps
  // DMA instructions per step (wave 0 one more, first), so a wait for
  // vmcnt(kDmaOps) lands every step but the newest.
  constexpr int kDmaOps = 2 * ((8 + NW - 1) / NW);
  // per-lane byte offsets of this wave's rows within a step's K (or V)
  // slice: eight 1 KB instructions of 4 rows each, over NW waves (with NW
  // not dividing 8 the last waves repeat an instruction of the first ones:
  // same data, same place, so every wave issues the same count)
  constexpr int kRowOps = (8 + NW - 1) / NW;
  uint32_t roff[kRowOps];
  int rslot[kRowOps];
#pragma unroll
  for (int i = 0; i < kRowOps; ++i) {
    int n = wave + NW * i;
    if (n >= 8) n -= 8;
    const int r = 4 * n + (lane >> 4);
    roff[i] = static_cast<uint32_t>(r) * kv_bytes + ((((lane & 15) ^ rsw(r))) << 4);
    rslot[i] = n * 1024;
  }
  auto issue_loads = [&](int st, uint8_t* kdst, uint8_t* vdst, int32_t* sdst) {
    const int k0 = step_key0(st);
    if (wave == 0 && lane < kStep / 4)
      dma16_s(tr.se + k0, 16u * lane, lds_addr(sdst));
    const char* kb = kgb + static_cast<size_t>(k0) * kv_bytes;
    const char* vb = vgb + static_cast<size_t>(k0) * kv_bytes;
#pragma unroll
    for (int i = 0; i < kRowOps; ++i) dma16_s(kb, roff[i], lds_addr(kdst) + rslot[i]);
#pragma unroll
    for (int i = 0; i < kRowOps; ++i) dma16_s(vb, roff[i], lds_addr(vdst) + rslot[i]);
  };

  auto step = [&](int st, const uint8_t* kcur, const uint8_t* vcur, const int32_t* scur,
                  uint8_t* kfill, uint8_t* vfill, int32_t* sfill) {
    const int k0 = step_key0(st);
    // step st staged by every wave (each waits for its own DMA), step st-1's
    // LDS reads returned; a plain s_barrier, since a workgroup fence would
    // also drain the newer prefetch
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kDmaOps) : "memory");
    // prefetch two steps ahead into the buffer step st-1 used; past the end
    // the last step again (in bounds, never read), so the code stays
    // branch-free and the count of outstanding DMA stays fixed
    const int k0p = step_key0(st + 2 < n_steps ? st + 2 : n_steps - 1);
    if (wave == 0 && lane < kStep / 4) dma16_s(tr.se + k0p, 16u * lane, lds_addr(sfill));
    const char* kbp = kgb + static_cast<size_t>(k0p) * kv_bytes;
    const char* vbp = vgb + static_cast<size_t>(k0p) * kv_bytes;
    // copy j of this wave's 2 kRowOps for the step (K rows, then V rows)
    auto dma_op = [&](int j) {
      if (j < kRowOps) dma16_s(kbp, roff[j], lds_addr(kfill) + rslot[j]);
      else dma16_s(vbp, roff[j - kRowOps], lds_addr(vfill) + rslot[j - kRowOps]);
    };
    // Units (MODE 1) never hold an empty step: their copies are spread over
    // the S^T MFMAs below, one per 32-deep slice, instead of leaving the
    // barrier as one burst from every wave (measured 2 % faster).  Blocks
    // issue them here, since a wave may skip the step.
    static_assert(MODE != 1 || 2 * kRowOps == 4, "one copy per d slice");
    if (MODE != 1) {
#pragma unroll
      for (int j = 0; j < 2 * kRowOps; ++j) dma_op(j);
    }

    // class of this wave's 32x32 block: 0 empty, 1 partial, 2 full
    const uint32_t cls = UNIT ? static_cast<uint32_t>(steps[st]) & 3
                              : (static_cast<uint32_t>(steps[st]) >> (2 * wave)) & 3;
    if (MODE == 1 || cls) {
      // S^T blocks (key half kh, query half qh): four independent chains
      f32x4_t sacc[2][2];
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) sacc[kh][0] = sacc[kh][1] = f32x4_t{};
      bf16x8_t kf = lds_frag(kcur, koff[0]);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          if (MODE == 1 && kh == 1) dma_op(s);
          bf16x8_t kn = kf;
          if (kh == 0) kn = lds_frag(kcur, kHalfTile + koff[s]);
          else if (s < 3) kn = lds_frag(kcur, koff[s + 1]);
          sacc[kh][0] = mma16(kf, qf[0][s], sacc[kh][0]);
          sacc[kh][1] = mma16(kf, qf[1][s], sacc[kh][1]);
          kf = kn;
        }

      // Mask a partial block: register i of block (kh, qh) is key
      // j = kb + 16 kh + i (kb = k0 + 4 lg) of query q = qlo + 16 qh + li,
      // and j sees q iff j <= q <= se[j].  With A = q - kb and S = se[j] - kb
      // the second condition is A <= S (one compare per element, S formed
      // once per key); the first holds for every pair off the diagonal
      // block, and on it is a second pass, 16 kh + i <= A.
      if (cls == 1) {
        const int kb = k0 + 4 * lg;
        const int4 s0 = *reinterpret_cast<const int4*>(scur + 4 * lg);
        const int4 s1 = *reinterpret_cast<const int4*>(scur + 16 + 4 * lg);
        const int S[2][4] = {{s0.x - kb, s0.y - kb, s0.z - kb, s0.w - kb},
                             {s1.x - kb, s1.y - kb, s1.z - kb, s1.w - kb}};
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
          const int A = qlo + 16 * qh + li - kb;
#pragma unroll
          for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int i = 0; i < 4; ++i) sacc[kh][qh][i] = A <= S[kh][i] ? sacc[kh][qh][i] : -INFINITY;
        }
        if (k0 + kStep > qlo) {
#pragma unroll
          for (int qh = 0; qh < 2; ++qh) {
            const int A = qlo + 16 * qh + li - kb;
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
              for (int i = 0; i < 4; ++i) sacc[kh][qh][i] = 16 * kh + i <= A ? sacc[kh][qh][i] : -INFINITY;
          }
        }
      }
      // row max of the raw scores
      float mx[2];
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        float m = vmax(sacc[0][qh][0], sacc[0][qh][1]);
        m = vmax(vmax(m, sacc[0][qh][2]), sacc[0][qh][3]);
        m = vmax(vmax(m, sacc[1][qh][0]), sacc[1][qh][1]);
        m = vmax(vmax(m, sacc[1][qh][2]), sacc[1][qh][3]);
        mx[qh] = m;
      }
      quad_max2(mx[0], mx[1]);
      mx[0] *= c;
      mx[1] *= c;
      if (__any(mx[0] > m_used[0] + kRescale || mx[1] > m_used[1] + kRescale)) {
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
          const float m_new = vmax(m_used[qh], mx[qh]);
          const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_used[qh] - m_new);
          l_part[qh] *= alpha;
#pragma unroll
          for (int db = 0; db < 8; ++db) oacc[db][qh] *= alpha;
          m_used[qh] = m_new;
          negm[qh] = m_new == -INFINITY ? 0.f : -m_new;
        }
      }
      bf16x8_t pf[2];
#pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        float e[8];
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
          for (int i = 0; i < 4; ++i) e[4 * kh + i] = fast_exp2(fmaf(sacc[kh][qh][i], c, negm[qh]));
        typedef float f32x8_t __attribute__((ext_vector_type(8)));
        const f32x8_t ev = {e[0], e[1], e[2], e[3], e[4], e[5], e[6], e[7]};
        pf[qh] = __builtin_convertvector(ev, bf16x8_t);
        // row sum of the bf16 probabilities that O accumulates, two per
        // v_dot2 against (1, 1).  (Written out with literal lane indices:
        // taking the pairs as bit casts of a uint32 vector's elements was
        // compiled into four reads of the first pair.)
        const bf16x8_t& p8 = pf[qh];
        float sum = l_part[qh];
        sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 0, 1), kOnes2, sum, false);
        sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 2, 3), kOnes2, sum, false);
        sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 4, 5), kOnes2, sum, false);
        sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 6, 7), kOnes2, sum, false);
        l_part[qh] = sum;
      }

      // O^T += V^T.P^T: sixteen independent blocks
      // V^T reads two d blocks ahead of their MFMAs; the scheduling barrier
      // keeps the compiler from sinking them back next to their use
      bf16x8_t vb[3];
      vb[0] = lds_vt_frag(vcur, trv, 0);
      vb[1] = lds_vt_frag(vcur, trv, 1);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        if (db + 2 < 8) vb[(db + 2) % 3] = lds_vt_frag(vcur, trv, db + 2);
        __builtin_amdgcn_sched_barrier(0);
        oacc[db][0] = mma16(vb[db % 3], pf[0], oacc[db][0]);
        oacc[db][1] = mma16(vb[db % 3], pf[1], oacc[db][1]);
      }
    }
  };

  if (n_steps > 0) {
    issue_loads(0, k_lds0, v_lds0, se_lds0);
    issue_loads(n_steps > 1 ? 1 : 0, k_lds1, v_lds1, se_lds1);
  }
  // query qlo + 16 qh + li, d = 32 s + 8 lg .. +7; loaded while the first
  // two steps stream in, and completed here (empty asm uses pin them before
  // the loop): the compiler does not count the assembly DMA, so its own
  // waits for these loads, left inside the loop, would drain the prefetch
#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const bf16_t* qp = q + (static_cast<size_t>(qlo + 16 * qh + li) * hq + h) * D + 8 * lg;
#pragma unroll
    for (int s = 0; s < 4; ++s) qf[qh][s] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(qp + 32 * s));
  }
#pragma unroll
  for (int qh = 0; qh < 2; ++qh)
#pragma unroll
    for (int s = 0; s < 4; ++s) asm volatile("" ::"v"(qf[qh][s]));
  for (int st = 0; st < n_steps; st += 3) {  // three-stage ring: step st uses buffer st % 3
    step(st, k_lds0, v_lds0, se_lds0, k_lds2, v_lds2, se_lds2);
    if (st + 1 < n_steps) step(st + 1, k_lds1, v_lds1, se_lds1, k_lds0, v_lds0, se_lds0);
    if (st + 2 < n_steps) step(st + 2, k_lds2, v_lds2, se_lds2, k_lds1, v_lds1, se_lds1);
  }
  // the last steps' prefetch must land before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const float l = quad_sum(l_part[qh]);
    const float inv = 1.f / l;
    const int qrow = qlo + 16 * qh + li;
    bf16_t* op = o + (static_cast<size_t>(qrow) * hq + h) * D + 4 * lg;
#pragma unroll
    for (int db = 0; db < 8; ++db)
      store4<bf16_t>(op + 16 * db, oacc[db][qh][0] * inv, oacc[db][qh][1] * inv,
                     oacc[db][qh][2] * inv, oacc[db][qh][3] * inv);
    if (lg == 0)
      lse[static_cast<size_t>(h) * tr.Np + qrow] = (m_used[qh] + fast_log2(l)) * 0.69314718055994531f;
  }
}

}  // namespace

hipError_t launch_attn_fwd_bf16_d128(const void* q, const void* k, const void* v, void* o,
                                     float* lse, const TreeDev& tr, int hq, int hkv, float scale,
                                     hipStream_t stream) {
  const float c = scale * 1.4426950408889634f;  // scores in the exp2 domain
  const int G = hq / hkv;
  const auto* qp = static_cast<const bf16_t*>(q);
  const auto* kp = static_cast<const bf16_t*>(k);
  const auto* vp = static_cast<const bf16_t*>(v);
  auto* op = static_cast<bf16_t*>(o);
  // 32-query units of four heads for as many heads of each group as a
  // multiple of four covers (measured 11 % faster than 128-query blocks at
  // four heads per group, 2 % at eight); 128-query blocks of one head for
  // the rest
  const unsigned units = static_cast<unsigned>(tr.Np / 32);
  const unsigned nb = static_cast<unsigned>(tr.nb);
  const unsigned G4 = G / 4 * 4, GR = G - G4;
  const dim3 grid(hkv * ((G4 / 4) * units + GR * nb));
  if (GR == 0)
    hipLaunchKernelGGL((tree_attn_fwd_bf16_d128<1, 4>), grid, dim3(256), 0, stream, qp, kp, vp, op,
                       lse, tr, hq, hkv, c);
  else if (G4 > 0)
    hipLaunchKernelGGL((tree_attn_fwd_bf16_d128<2, 4>), grid, dim3(256), 0, stream, qp, kp, vp, op,
                       lse, tr, hq, hkv, c);
  else
    hipLaunchKernelGGL((tree_attn_fwd_bf16_d128<0, 4>), grid, dim3(256), 0, stream, qp, kp, vp, op,
                       lse, tr, hq, hkv, c);
  return hipGetLastError();
}

}  // namespace pst
