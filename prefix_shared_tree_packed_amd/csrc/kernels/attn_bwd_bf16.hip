// Tree attention backward pass, bf16 with head_dim 128: the performance path
// on gfx950.  Same mathematics and deterministic result as attn_bwd.hip, in
// two launches: first dQ per query block (or 32-query unit) over the
// forward's step lists, which also forms D = rowsum(dO*O) for its rows;
// then dK/dV per key block walking its contiguous range of visible query
// blocks, in persistent workgroups.  Both are fed the way the forward
// kernel of attn_fwd_bf16.hip is fed:
//
//  * Every tile reaches LDS row-major (token rows of 256 bytes) by
//    global_load_lds_dwordx4 (no VGPRs, no VALU) through three-stage rings,
//    issued from inline assembly with the step's base address in SGPRs and
//    lane offsets fixed for the kernel, so that only the kernels' own waits
//    gate the prefetch: Q and dO in 64-query steps for dK/dV (one workgroup
//    per CU), K and V in 32-key steps for dQ (two workgroups per CU; in
//    32-query units of four heads for the largest multiple of four of each
//    head group, in 128-query blocks for the rest, as the forward).
//  * Both passes use 16x16x32 MFMAs throughout, so every wave has eight
//    independent S / dP chains and sixteen independent dK / dV (or dQ)
//    blocks in flight.  LDS operand reads run two fragments ahead of their
//    MFMAs, held there by scheduling barriers.  The dP accumulators start
//    at -D, so the MFMAs leave dP - D.
//  * Products that contract over tokens need the tile transposed (dV^T +=
//    dO^T.P, dK^T += Q^T.dS, dQ^T += K^T.dS^T).  Their A operands come from
//    the same row-major tile through ds_read_b64_tr_b16: two transposing
//    reads per MFMA operand, at nearly the rate of ordinary 16-byte reads,
//    so no transposed copy exists anywhere.
//  * 16-byte chunk c of tile row r sits at c ^ rsw(r), rsw(r) = 2 (r & 7) +
//    ((r >> 3) & 1): 16 consecutive rows reading one chunk each hit 16
//    distinct positions, and a transposing read (4 aligned rows x 2 adjacent
//    chunks per 16 lanes) hits 8 distinct positions: no bank conflicts.
//  * Work per (wave, 32x32 sub-block) is skipped when no pair is visible; a
//    partially visible one first sets its invisible scores to -inf in one
//    pass under one branch (dK/dV: (unsigned)(i - j) <= se[j] - j; dQ, as
//    the forward: i <= se[j] alone off the diagonal, j <= i as a second pass
//    on it), so fully visible sub-blocks pay no mask.
//  * P is rounded to bf16 before the dV product and dS before the dK and dQ
//    products; accumulation is fp32.
#include "launch.h"
#include "lds_tiles.h"
#include "mfma.h"

#include <cmath>
#include <type_traits>

namespace pst {
namespace {

constexpr int D = 128;
constexpr int kRowB = kTileRowB;
constexpr float kLog2e = 1.4426950408889634f;

typedef const __attribute__((address_space(4))) int32_t cint32;  // read-only: scalar loads

__device__ __forceinline__ cint32* cst(const int32_t* p) { return (cint32*)(p); }

__device__ __forceinline__ bf16x8_t lds_frag(const uint8_t* base, int byte_off) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(base + byte_off));
}

// Sum over the four lanes l % 16 + 16 g (g = 0..3), which hold one row's
// four 32-wide slices of the head dimension in the 16x16 operand layouts.
__device__ __forceinline__ float quad_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return sum_halves(__uint_as_float(a[0]) + __uint_as_float(a[1]));
}

// --------------------------------------------------------------------- dK, dV
// A pair of waves owns 32 keys (two 16-key halves kh) of one key/value head
// and walks every visible query block of the G query heads in 64-query
// steps (three stages of LDS, one workgroup per CU).  All products are
// 16x16x32 MFMAs: per 32-query slice, S = Q.K^T and dP = dO.V^T are eight
// independent 16x16 chains, and dV^T += dO^T.P, dK^T += Q^T.dS sixteen
// independent blocks each.
constexpr int kKvStep = 64;                 // queries per step
constexpr int kKvBuf = kKvStep * kRowB;     // 16 KB
constexpr int kHalf16 = 16 * kRowB;         // byte offset of rows 16..31 of a 32-row slice
// stage layout: Q tile | dO tile | LSE [64] | D [64]
constexpr int kStDo = kKvBuf, kStLs = 2 * kKvBuf, kStDd = 2 * kKvBuf + 4 * kKvStep;
constexpr int kStageB = 2 * kKvBuf + 8 * kKvStep;

__device__ __forceinline__ f32x4_t mma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Transposed operand of one 16-row d block from a row-major 32-token slice:
// lane (group g, index i) gets d = 16 db + i of tokens 4g .. 4g+3 (slots
// 0..3) and 16 + 4g .. 16 + 4g + 3 (slots 4..7), the token order in which
// 16x16 accumulators feed a B operand.
__device__ __forceinline__ bf16x8_t lds_t16_frag(const uint8_t* slice, int trv, int db) {
  const int off = trv ^ (db << 5);
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(slice + off));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(slice + kHalf16 + off));
  typedef short i16x8_t __attribute__((ext_vector_type(8)));
  const i16x8_t w = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8_t, w);
}
__device__ __forceinline__ bf16x8_t pack8(const f32x4_t& lo, const f32x4_t& hi) {
  typedef float f32x8_t __attribute__((ext_vector_type(8)));
  const f32x8_t x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_convertvector(x, bf16x8_t);
}

// Eight waves: four pairs, pair p owning keys kbase .. kbase + 31 (kbase =
// 128 kb + 32 p).  Wave p (role A) computes S = Q.K^T, masks it, forms
// P = exp(S c - LSE) and accumulates dV^T += dO^T.P; it hands P (bf16, in
// its accumulator layout) to wave p + 4 (role B) through LDS.  B computes
// dP = dO.V^T (accumulators starting at -D) and, one 64-query step behind
// A, dS = P (dP - D) and dK^T += Q^T.dS.  Each wave holds one accumulator
// set and one of K, V, so two waves share a SIMD.  A software-pipelines the
// two 32-query sub-blocks of a step: the first sub-block's exponentials
// issue between the MFMAs of the second's S, the second's between those of
// the first's dV, so its VALU work runs beside the matrix core (measured
// 3 % faster than sub-blocks in turn; the same for B's dS cost 1.5 %).
// Every wave passes one barrier per step (which also waits for the step's
// tiles) and one after the loop for B's last step.  Three tile stages:
// while a step computes, B reads the previous step's Q and the next step
// streams in.
constexpr int kKvStages = 3;
constexpr int kPexB = 2 * 1024;  // one pair's P of one sub-block: 2 chunks x 64 lanes x 16 B
constexpr int kPexSlots = 4;     // two steps of two 32-query sub-blocks

__global__ __launch_bounds__(512, 1) void bwd_dkdv_bf16(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dsum,
    bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, TreeDev tr, int hq, int hkv, float c,
    float scale, int lanes, int lanes_log2) {
  // one named array per stage, so the compiler tells the in-flight DMA
  // target from the stage being read
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[kStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t stage2[kStageB];
  // P handed from A to B: [pair][slot: step parity x half][chunk kh][lane] x 16 B
  __shared__ __attribute__((aligned(1024))) uint8_t pex[4 * kPexSlots * kPexB];

  const int G = hq / hkv;
  // persistent: `lanes` workgroups per key/value group, each walking the
  // key blocks the host's list scheduling dealt to its lane
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int g = logical / lanes;
  const int lane_id = logical - g * lanes;
  cint32* lane_ptr = cst(tr.bwd_lanes) + (lanes - 1) + lanes_log2 + lanes_log2 * tr.nb;
  const int it0 = lane_ptr[lane_id], it1 = lane_ptr[lane_id + 1];
  cint32* lane_items = lane_ptr + lanes + 1;
  // the current key block and its per-block state (set for each block below)
  int kb = 0, kbase = 0, smin = 0, smax = 0, qhi = 0, n_steps = 0;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int pair = wave & 3;
  const bool roleA = wave < 4;  // wave-uniform
  const int li = lane % 16;     // key column of the 16x16 blocks
  const int lg = lane / 16;     // 16-lane group: queries 4 lg .. 4 lg + 3 of each block
  int span_k[2];  // se - key of this lane's key in each half (A); loaded below
  cint32* blk32 = cst(tr.blk32);
  // B operands: K^T (A) or V^T (B), key kbase + 16 kh + li, d = 32 s + 8 lg
  // .. +7; loaded below, once the first tiles are on their way
  bf16x8_t kvf[2][4];
  // A operands Q / dO: query row li of a 16-row block, chunk 4 s + lg
  int roff[4];
  #pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) roff[s4] = li * kRowB + (((4 * s4 + lg) ^ rsw(li)) << 4);
  // transposed reads: lane i of group lg addresses token 4 lg + i / 4 at d = 4 (i % 4) .. +3
  int trv;
  {
    const int t = 4 * lg + li / 4;
    const int a = li % 4;
    trv = t * kRowB + ((((a >> 1) ^ rsw(t))) << 4) + ((a & 1) << 3);
  }

  f32x4_t acc[8][2];  // (d block db, key half kh): dV^T (A) or dK^T (B)
  f32x4_t dpacc[2][2][2];  // B: dP - D of the step it finishes next (32-query half, q16, kh)

  const uint32_t q_bytes = static_cast<uint32_t>(hq) * D * 2;  // one token's Q (or dO) rows
  // step -> (query block, head of the group, half): steps walk halves, then
  // heads, then blocks from qhi down to kb (the key blocks sharing qhi run
  // side by side and read the same query rows at about the same time);
  // cursors advance one step at a time
  struct Cursor {
    int qb, r, half;
  };
  auto cursor_at = [&](int st) {
    const int rest = st >> 1;
    return Cursor{qhi - rest / G, rest % G, st & 1};
  };
  auto advance = [&](Cursor& cu) {
    cu.half ^= 1;
    if (cu.half == 0 && ++cu.r == G) {
      cu.r = 0;
      --cu.qb;
    }
  };
  auto decode = [&](const Cursor& cu, int& h, int& q0) {
    h = g * G + cu.r;
    q0 = cu.qb * kTile + kKvStep * cu.half;
  };
  // all eight waves share each step's tile DMA
  constexpr int kNw = 8;
  const TileOff<kKvStep, kNw> qoff = tile_offsets<kKvStep, kNw>(q_bytes, wave, lane);
  auto issue_loads = [&](const Cursor& cu, uint8_t* stg) {
    int h, q0;
    decode(cu, h, q0);
    const size_t r0 = static_cast<size_t>(h) * tr.Np + q0;
    const uint32_t base = lds_addr(stg);
    if (wave == 0)
      dma4_s(lse + r0, 4u * lane, base + kStLs);
    else if (wave == 1)
      dma4_s(dsum + r0, 4u * lane, base + kStDd);
    const size_t row0 = static_cast<size_t>(q0) * q_bytes + static_cast<size_t>(h) * D * 2;
    dma_tile_s<kKvStep, kNw>(reinterpret_cast<const char*>(q) + row0, qoff, base, wave);
    dma_tile_s<kKvStep, kNw>(reinterpret_cast<const char*>(dout) + row0, qoff, base + kStDo, wave);
  };
  auto empty_at = [&](int qlo) { return kbase > qlo + 31 || smax < qlo; };
  uint8_t* const pex_pair = pex + pair * (kPexSlots * kPexB);
  // A operand reads of fragment f (d slice f / 2, query half f % 2) of a slice
  auto qoffs = [&](int f) { return ((f & 1) ? kHalf16 : 0) + roff[f >> 1]; };

  // A's pieces for one 32-query sub-block (half qs of a stage, first query
  // qlo).  S = Q.K^T: eight independent 16x16 chains.
  auto a_scores = [&](const uint8_t* stg, int qs, f32x4_t (&sacc)[2][2]) {
    const uint8_t* qsl = stg + 32 * qs * kRowB;
    #pragma unroll
    for (int a = 0; a < 2; ++a) sacc[a][0] = sacc[a][1] = f32x4_t{};
    bf16x8_t qbuf[3];
    qbuf[0] = lds_frag(qsl, qoffs(0));
    qbuf[1] = lds_frag(qsl, qoffs(1));
    #pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f + 2 < 8) qbuf[(f + 2) % 3] = lds_frag(qsl, qoffs(f + 2));
      __builtin_amdgcn_sched_barrier(0);
      const int s4 = f >> 1, q16 = f & 1;
      #pragma unroll
      for (int kh = 0; kh < 2; ++kh) sacc[q16][kh] = mma16(qbuf[f % 3], kvf[kh][s4], sacc[q16][kh]);
    }
  };
  // register i of block (q16, kh) is query qlo + 16 q16 + 4 lg + i, key
  // kbase + 16 kh + li; key j sees query q iff (unsigned)(q - j) <= se[j] - j.
  // A sub-block every pair of which is visible skips the test.
  auto a_mask = [&](f32x4_t (&sacc)[2][2], int qlo) {
    if (kbase + 31 <= qlo && smin >= qlo + 31) return;
    const int A = qlo + 4 * lg - kbase - li;
    #pragma unroll
    for (int q16 = 0; q16 < 2; ++q16)
      #pragma unroll
      for (int kh = 0; kh < 2; ++kh)
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t dlt = static_cast<uint32_t>(A + 16 * q16 + i - 16 * kh);
          sacc[q16][kh][i] = dlt <= static_cast<uint32_t>(span_k[kh]) ? sacc[q16][kh][i] : -INFINITY;
        }
  };
  // the rows' LSE in the exp2 domain: lv[q16][i] for query 16 q16 + 4 lg + i
  auto a_lse = [&](const uint8_t* stg, int qs, float (&lv)[2][4]) {
    const float* lsl = reinterpret_cast<const float*>(stg + kStLs);
    #pragma unroll
    for (int q16 = 0; q16 < 2; ++q16) {
      const float4 l4 = *reinterpret_cast<const float4*>(lsl + 32 * qs + 16 * q16 + 4 * lg);
      lv[q16][0] = l4.x * kLog2e;
      lv[q16][1] = l4.y * kLog2e;
      lv[q16][2] = l4.z * kLog2e;
      lv[q16][3] = l4.w * kLog2e;
    }
  };
  // P = exp2(S c - LSE) of element e (q16 = e / 8, kh = e / 4 % 2, i = e % 4)
  auto a_exp = [&](f32x4_t (&sacc)[2][2], const float (&lv)[2][4], int e) {
    const int q16 = e >> 3, kh = (e >> 2) & 1, i = e & 3;
    sacc[q16][kh][i] = fast_exp2(fmaf(sacc[q16][kh][i], c, -lv[q16][i]));
  };
  // P to bf16 (B operands of dV^T += dO^T.P), and to pex slot `slot` for B
  auto a_pack = [&](const f32x4_t (&sacc)[2][2], int slot, bf16x8_t (&pf)[2]) {
    #pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      pf[kh] = pack8(sacc[0][kh], sacc[1][kh]);
      *reinterpret_cast<bf16x8_t*>(pex_pair + slot * kPexB + kh * 1024 + lane * 16) = pf[kh];
    }
  };
  // dV^T += dO^T.P of half qs, transposed reads two d blocks ahead; with
  // kNext, the exponentials of the next sub-block's scores `nxt` issue
  // between the MFMAs, two per d block
  auto a_dv = [&](auto next, const uint8_t* stg, int qs, const bf16x8_t (&pf)[2],
                  f32x4_t (&nxt)[2][2], const float (&nlv)[2][4]) {
    constexpr bool kNext = decltype(next)::value;
    const uint8_t* dosl = stg + kStDo + 32 * qs * kRowB;
    bf16x8_t obuf[3];
    obuf[0] = lds_t16_frag(dosl, trv, 0);
    obuf[1] = lds_t16_frag(dosl, trv, 1);
    #pragma unroll
    for (int db = 0; db < 8; ++db) {
      if (db + 2 < 8) obuf[(db + 2) % 3] = lds_t16_frag(dosl, trv, db + 2);
      __builtin_amdgcn_sched_barrier(0);
      acc[db][0] = mma16(obuf[db % 3], pf[0], acc[db][0]);
      if constexpr (kNext) a_exp(nxt, nlv, 2 * db);
      acc[db][1] = mma16(obuf[db % 3], pf[1], acc[db][1]);
      if constexpr (kNext) a_exp(nxt, nlv, 2 * db + 1);
    }
  };
  // A on one sub-block: S, mask, P, dV
  auto run_a = [&](const uint8_t* stg, int qs, int qlo, int slot) {
    f32x4_t sacc[2][2];
    a_scores(stg, qs, sacc);
    a_mask(sacc, qlo);
    float lv[2][4];
    a_lse(stg, qs, lv);
    #pragma unroll
    for (int e = 0; e < 16; ++e) a_exp(sacc, lv, e);
    bf16x8_t pf[2];
    a_pack(sacc, slot, pf);
    a_dv(std::false_type{}, stg, qs, pf, sacc, lv);
  };
  // A on both sub-blocks of a step, software-pipelined: the first
  // sub-block's exponentials issue between the second's S MFMAs, the
  // second's between the first's dV MFMAs, so the VALU work runs beside
  // the matrix core rather than between this wave's MFMA phases
  auto run_a2 = [&](const uint8_t* stg, int q0, int par) {
    f32x4_t s0[2][2], s1[2][2];
    float lv0[2][4], lv1[2][4];
    a_scores(stg, 0, s0);
    a_mask(s0, q0);
    a_lse(stg, 0, lv0);
    {  // S of the second sub-block with P of the first
      const uint8_t* qsl = stg + 32 * kRowB;
      #pragma unroll
      for (int a = 0; a < 2; ++a) s1[a][0] = s1[a][1] = f32x4_t{};
      bf16x8_t qbuf[3];
      qbuf[0] = lds_frag(qsl, qoffs(0));
      qbuf[1] = lds_frag(qsl, qoffs(1));
      #pragma unroll
      for (int f = 0; f < 8; ++f) {
        if (f + 2 < 8) qbuf[(f + 2) % 3] = lds_frag(qsl, qoffs(f + 2));
        __builtin_amdgcn_sched_barrier(0);
        const int s4 = f >> 1, q16 = f & 1;
        s1[q16][0] = mma16(qbuf[f % 3], kvf[0][s4], s1[q16][0]);
        a_exp(s0, lv0, 2 * f);
        s1[q16][1] = mma16(qbuf[f % 3], kvf[1][s4], s1[q16][1]);
        a_exp(s0, lv0, 2 * f + 1);
      }
    }
    bf16x8_t pf0[2], pf1[2];
    a_pack(s0, 2 * par, pf0);
    a_mask(s1, q0 + 32);
    a_lse(stg, 1, lv1);
    a_dv(std::true_type{}, stg, 0, pf0, s1, lv1);
    a_pack(s1, 2 * par + 1, pf1);
    a_dv(std::false_type{}, stg, 1, pf1, s1, lv1);
  };
  // B, first half of its work on a sub-block: dP - D into dpacc[qs]
  auto run_b_dp = [&](const uint8_t* stg, int qs) {
    const uint8_t* dosl = stg + kStDo + 32 * qs * kRowB;
    const float* ddl = reinterpret_cast<const float*>(stg + kStDd);
    #pragma unroll
    for (int a = 0; a < 2; ++a) {
      const float4 d4 = *reinterpret_cast<const float4*>(ddl + 32 * qs + 16 * a + 4 * lg);
      const f32x4_t negd = {-d4.x, -d4.y, -d4.z, -d4.w};
      dpacc[qs][a][0] = dpacc[qs][a][1] = negd;
    }
    bf16x8_t dbuf[3];
    dbuf[0] = lds_frag(dosl, qoffs(0));
    dbuf[1] = lds_frag(dosl, qoffs(1));
    #pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f + 2 < 8) dbuf[(f + 2) % 3] = lds_frag(dosl, qoffs(f + 2));
      __builtin_amdgcn_sched_barrier(0);
      const int s4 = f >> 1, q16 = f & 1;
      #pragma unroll
      for (int kh = 0; kh < 2; ++kh) dpacc[qs][q16][kh] = mma16(dbuf[f % 3], kvf[kh][s4], dpacc[qs][q16][kh]);
    }
  };
  // B, second half: dS = P (dP - D) with A's P from pex slot `slot`, dK^T += Q^T.dS
  auto run_b_dk = [&](const uint8_t* stg, int qs, int slot) {
    const uint8_t* qsl = stg + 32 * qs * kRowB;
    bf16x8_t sf[2];
    #pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const uint4 pw = *reinterpret_cast<const uint4*>(pex_pair + slot * kPexB + kh * 1024 + lane * 16);
      const uint32_t w[4] = {pw.x, pw.y, pw.z, pw.w};
      f32x4_t lo, hi;  // dS of query halves 0 and 1 (P in slots 0..3, 4..7)
      #pragma unroll
      for (int i = 0; i < 2; ++i) {
        lo[2 * i] = __uint_as_float(w[i] << 16) * dpacc[qs][0][kh][2 * i];
        lo[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u) * dpacc[qs][0][kh][2 * i + 1];
        hi[2 * i] = __uint_as_float(w[2 + i] << 16) * dpacc[qs][1][kh][2 * i];
        hi[2 * i + 1] = __uint_as_float(w[2 + i] & 0xffff0000u) * dpacc[qs][1][kh][2 * i + 1];
      }
      sf[kh] = pack8(lo, hi);
    }
    bf16x8_t tbuf[3];
    tbuf[0] = lds_t16_frag(qsl, trv, 0);
    tbuf[1] = lds_t16_frag(qsl, trv, 1);
    #pragma unroll
    for (int db = 0; db < 8; ++db) {
      if (db + 2 < 8) tbuf[(db + 2) % 3] = lds_t16_frag(qsl, trv, db + 2);
      __builtin_amdgcn_sched_barrier(0);
      #pragma unroll
      for (int kh = 0; kh < 2; ++kh) acc[db][kh] = mma16(tbuf[db % 3], sf[kh], acc[db][kh]);
    }
  };

  for (int it = it0; it < it1; ++it) {
    kb = lane_items[it];
    kbase = kb * kTile + 32 * pair;  // first key of this pair
    smin = blk32[2 * (kbase >> 5)];
    smax = blk32[2 * (kbase >> 5) + 1];
    qhi = cst(tr.kb_qhi)[kb];
    n_steps = (qhi - kb + 1) * G * 2;
    #pragma unroll
    for (int db = 0; db < 8; ++db) acc[db][0] = acc[db][1] = f32x4_t{};
    // the previous block's LDS reads are done before its stages refill
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // the first step's tiles start streaming, then the K/V rows and subtree
    // ends load beside them and complete here (empty asm uses pin them before
    // the loop: the compiler does not count the assembly DMA, so its own
    // waits for these loads, left inside the loop, would drain the prefetch)
    issue_loads(cursor_at(0), stage0);
    {
      const bf16_t* src = roleA ? k : v;
      #pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        span_k[kh] = tr.se[kbase + 16 * kh + li] - (kbase + 16 * kh + li);
        const size_t off = (static_cast<size_t>(kbase + 16 * kh + li) * hkv + g) * D + 8 * lg;
        #pragma unroll
        for (int s4 = 0; s4 < 4; ++s4)
          kvf[kh][s4] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(src + off + 32 * s4));
      }
    }
    #pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      asm volatile("" ::"v"(span_k[kh]));
      #pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) asm volatile("" ::"v"(kvf[kh][s4]));
    }

    // The step loop, instantiated once per role so that neither role's
    // registers flow through the other's branches; both pass the same
    // barriers in the same order (s_barrier counts arrivals, wherever they
    // come from).
    auto loop = [&](auto role) {
      constexpr bool kA = decltype(role)::value;
      Cursor cur = cursor_at(0), pf = cursor_at(1);  // n_steps >= 2
      // B's pending step: its stage, and which of its halves have any pair
      const uint8_t* pend_stg = stage0;
      int pend_par = 0;
      bool pend_live[2] = {false, false};
      auto step = [&](int st, const uint8_t* stg, uint8_t* fill) {
        int h, q0;
        decode(cur, h, q0);
        advance(cur);
        // step st staged, the previous step's P written and LDS reads done;
        // then step st + 1 streams into the stage step st - 2 used (B finished
        // with it during step st - 1)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (st + 1 < n_steps) {
          issue_loads(pf, fill);
          advance(pf);
        }
        const int par = st & 1;
        bool live[2];
        #pragma unroll
        for (int qs = 0; qs < 2; ++qs) live[qs] = !empty_at(q0 + 32 * qs);
        if constexpr (kA) {
          if (live[0] && live[1]) {
            run_a2(stg, q0, par);
          } else {
            #pragma unroll
            for (int qs = 0; qs < 2; ++qs)
              if (live[qs]) run_a(stg, qs, q0 + 32 * qs, 2 * par + qs);
          }
        } else {
          #pragma unroll
          for (int qs = 0; qs < 2; ++qs)
            if (pend_live[qs]) run_b_dk(pend_stg, qs, 2 * pend_par + qs);
          #pragma unroll
          for (int qs = 0; qs < 2; ++qs)
            if (live[qs]) run_b_dp(stg, qs);
          pend_stg = stg;
          pend_par = par;
          pend_live[0] = live[0];
          pend_live[1] = live[1];
        }
      };
      for (int st = 0; st < n_steps; st += kKvStages) {  // three-stage ring: step st uses stage st % 3
        step(st, stage0, stage1);
        if (st + 1 < n_steps) step(st + 1, stage1, stage2);
        if (st + 2 < n_steps) step(st + 2, stage2, stage0);
      }
      // B's last step
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      if constexpr (!kA) {
        #pragma unroll
        for (int qs = 0; qs < 2; ++qs)
          if (pend_live[qs]) run_b_dk(pend_stg, qs, 2 * pend_par + qs);
      }
    };
    if (roleA)
      loop(std::true_type{});
    else
      loop(std::false_type{});
    // the last steps' prefetch lands before the stages refill or are released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    bf16_t* const out = roleA ? dv : dk;
    const float osc = roleA ? 1.f : scale;
    #pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      const size_t off = (static_cast<size_t>(kbase + 16 * kh + li) * hkv + g) * D + 4 * lg;
      #pragma unroll
      for (int db = 0; db < 8; ++db)
        store4<bf16_t>(out + off + 16 * db, acc[db][kh][0] * osc, acc[db][kh][1] * osc,
                       acc[db][kh][2] * osc, acc[db][kh][3] * osc);
    }
  }
}

// --------------------------------------------------------------------- dQ
// A wave owns 32 query rows (two 16-row halves qh) of one head and walks the
// query block's non-empty 32-key columns through a three-stage LDS ring (K, V
// and subtree ends; two workgroups per CU).  S^T = K.Q^T and dP^T = V.dO^T are
// eight independent 16x16 chains; dQ^T += K^T.dS^T sixteen blocks.
constexpr int kQStep = 32;
constexpr int kQBuf = kQStep * kRowB;  // 8 KB
// stage layout: K tile | V tile | subtree ends [32]
constexpr int kQStV = kQBuf, kQStSe = 2 * kQBuf;
constexpr int kQStageB = 2 * kQBuf + 4 * kQStep;

// A unit workgroup is one 32-query unit of four heads of one key/value group
// (one wave per head), walking the unit's non-empty 32x32 blocks; a block
// workgroup is one 128-query block of one head.  MODE 0: blocks only; 1:
// units only (heads per group a multiple of four); 2: mixed, for a group
// size G = 4 m + r: units for the group's first 4 m heads, blocks for its
// last r (as the forward).
template <int MODE>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ o, const bf16_t* __restrict__ dout, const float* __restrict__ lse,
    float* __restrict__ dsum, bf16_t* __restrict__ dq, TreeDev tr, int hq, int hkv, float c,
    float scale) {
  __shared__ __attribute__((aligned(1024))) uint8_t stage0[kQStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t stage1[kQStageB];
  __shared__ __attribute__((aligned(1024))) uint8_t stage2[kQStageB];

  const int G = hq / hkv;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int li = lane % 16;  // query column of the 16x16 blocks
  const int lg = lane / 16;  // 16-lane group: keys 4 lg .. 4 lg + 3 of each block
  // work ids run group by group (each XCD keeps one group's K/V in its L2):
  // first the group's units, then its 128-query blocks
  const int G4 = MODE == 0 ? 0 : G / 4 * 4;  // heads of each group served by units
  const int GR = G - G4;                     // heads served by 128-query blocks
  const int per_unit = G4 / 4;               // unit workgroups per unit and group
  const int u_g = per_unit * (tr.Np / 32);
  const int per_g = u_g + GR * tr.nb;
  const int g = logical / per_g;
  const int rem = logical - g * per_g;
  const bool UNIT = MODE == 1 || (MODE == 2 && rem < u_g);
  int h, qlo, n_steps;
  cint32* steps;
  if (UNIT) {
    const int rank = rem / per_unit;
    h = g * G + (rem - rank * per_unit) * 4 + wave;
    const int u = cst(tr.unit_order)[rank];
    qlo = u * 32;
    steps = cst(tr.unit_steps) + cst(tr.unit_ptr)[u];
    n_steps = cst(tr.unit_ptr)[u + 1] - cst(tr.unit_ptr)[u];
  } else {
    const int rb = rem - u_g;
    const int rank = rb / GR;
    h = g * G + G4 + (rb - rank * GR);
    const int qb = cst(tr.fwd_order)[rank];
    qlo = qb * kTile + wave * 32;
    // the query block's non-empty 32-key columns (scalar metadata reads)
    steps = cst(tr.steps) + cst(tr.step_ptr)[qb];
    n_steps = cst(tr.step_ptr)[qb + 1] - cst(tr.step_ptr)[qb];
  }

  // B operands Q^T / dO^T (query qlo + 16 qh + li, d = 32 s + 8 lg .. +7),
  // the rows' LSE and D; loaded below, once the first tiles are on their way
  bf16x8_t qf[2][4], df[2][4];
  float lse2[2], dsq[2];
  // A operands K / V: key row li (+16 for the second key half), chunk 4 s + lg
  int roff[4];
  #pragma unroll
  for (int s4 = 0; s4 < 4; ++s4) roff[s4] = li * kRowB + (((4 * s4 + lg) ^ rsw(li)) << 4);
  int trv;  // transposed K reads: lane i of group lg addresses key 4 lg + i / 4, d = 4 (i % 4) ..
  {
    const int t = 4 * lg + li / 4;
    const int a = li % 4;
    trv = t * kRowB + ((((a >> 1) ^ rsw(t))) << 4) + ((a & 1) << 3);
  }

  f32x4_t dqacc[8][2];  // (d block db, query half qh)
  #pragma unroll
  for (int db = 0; db < 8; ++db) dqacc[db][0] = dqacc[db][1] = f32x4_t{};

  const uint32_t kv_bytes = static_cast<uint32_t>(hkv) * D * 2;
  const char* kgb = reinterpret_cast<const char*>(k + static_cast<size_t>(g) * D);
  const char* vgb = reinterpret_cast<const char*>(v + static_cast<size_t>(g) * D);
  auto step_key0 = [&](int st) { return (steps[st] >> (UNIT ? 2 : 8)) * kQStep; };

  // Every wave issues kDmaOps tile DMA instructions per step; wave 0 also the
  // subtree ends, first, so a wait for vmcnt(kDmaOps) lands every step but
  // the newest.
  constexpr int kDmaOps = 2 * (kQStep / 16);
  const TileOff<kQStep> koffs = tile_offsets<kQStep>(kv_bytes, wave, lane);
  auto issue_loads = [&](int st, uint8_t* stg) {
    const int k0 = step_key0(st);
    const uint32_t base = lds_addr(stg);
    if (wave == 0 && lane < kQStep / 4) dma16_s(tr.se + k0, 16u * lane, base + kQStSe);
    dma_tile_s<kQStep>(kgb + static_cast<size_t>(k0) * kv_bytes, koffs, base, wave);
    dma_tile_s<kQStep>(vgb + static_cast<size_t>(k0) * kv_bytes, koffs, base + kQStV, wave);
  };

  auto step = [&](int st, const uint8_t* stg, uint8_t* fill) {
    const int k0 = step_key0(st);
    const uint8_t* kl = stg;
    const uint8_t* vl = stg + kQStV;
    const int32_t* sel = reinterpret_cast<const int32_t*>(stg + kQStSe);
    // step st staged by every wave, step st-1's LDS reads returned; a plain
    // s_barrier, since a workgroup fence would also drain the newer prefetch
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kDmaOps) : "memory");
    issue_loads(st + 2 < n_steps ? st + 2 : n_steps - 1, fill);

    const uint32_t cls = UNIT ? static_cast<uint32_t>(steps[st]) & 3
                              : (static_cast<uint32_t>(steps[st]) >> (2 * wave)) & 3;
    if (cls == 0) return;
    // S^T and dP^T blocks (key half kh, query half qh): eight chains
    f32x4_t sacc[2][2], dpacc[2][2];
    #pragma unroll
    for (int kh = 0; kh < 2; ++kh) {
      // dP^T accumulators start at -D of their query (all four registers of
      // a lane belong to query qlo + 16 qh + li): the MFMAs leave dP - D
      sacc[kh][0] = sacc[kh][1] = f32x4_t{};
      dpacc[kh][0] = f32x4_t{-dsq[0], -dsq[0], -dsq[0], -dsq[0]};
      dpacc[kh][1] = f32x4_t{-dsq[1], -dsq[1], -dsq[1], -dsq[1]};
    }
    // operand reads run two (s4, kh) pairs ahead of their MFMAs, held in
    // place by scheduling barriers
    auto koffs_f = [&](int f) { return ((f & 1) ? kHalf16 : 0) + roff[f >> 1]; };
    bf16x8_t kbuf[3], vbuf[3];
    #pragma unroll
    for (int f = 0; f < 2; ++f) {
      kbuf[f] = lds_frag(kl, koffs_f(f));
      vbuf[f] = lds_frag(vl, koffs_f(f));
    }
    #pragma unroll
    for (int f = 0; f < 8; ++f) {
      if (f + 2 < 8) {
        kbuf[(f + 2) % 3] = lds_frag(kl, koffs_f(f + 2));
        vbuf[(f + 2) % 3] = lds_frag(vl, koffs_f(f + 2));
      }
      __builtin_amdgcn_sched_barrier(0);
      const int s4 = f >> 1, kh = f & 1;
      #pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        sacc[kh][qh] = mma16(kbuf[f % 3], qf[qh][s4], sacc[kh][qh]);
        dpacc[kh][qh] = mma16(vbuf[f % 3], df[qh][s4], dpacc[kh][qh]);
      }
    }
    // Register i of block (kh, qh) is key j = kb + 16 kh + i (kb = k0 + 4 lg)
    // of query q = qlo + 16 qh + li, and j sees q iff j <= q <= se[j].  A
    // partial block first sets its invisible scores to -inf (one branch per
    // step): with A = q - kb and S = se[j] - kb the second condition is
    // A <= S; the first holds off the diagonal block and is a second pass
    // on it, 16 kh + i <= A.
    if (cls == 1) {
      const int kb = k0 + 4 * lg;
      const int4 s0 = *reinterpret_cast<const int4*>(sel + 4 * lg);
      const int4 s1 = *reinterpret_cast<const int4*>(sel + 16 + 4 * lg);
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
      if (k0 + kQStep > qlo) {
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
    // P = exp(S c - LSE), 0 where masked; dS = P (dP - D)
    #pragma unroll
    for (int kh = 0; kh < 2; ++kh)
      #pragma unroll
      for (int qh = 0; qh < 2; ++qh)
        #pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = fast_exp2(fmaf(sacc[kh][qh][i], c, -lse2[qh]));
          dpacc[kh][qh][i] = e * dpacc[kh][qh][i];
        }
    // dQ^T += K^T.dS^T
    bf16x8_t sf[2];
    #pragma unroll
    for (int qh = 0; qh < 2; ++qh) sf[qh] = pack8(dpacc[0][qh], dpacc[1][qh]);
    // transposed K reads two d blocks ahead, held in place the same way
    bf16x8_t kt[3];
    kt[0] = lds_t16_frag(kl, trv, 0);
    kt[1] = lds_t16_frag(kl, trv, 1);
    #pragma unroll
    for (int db = 0; db < 8; ++db) {
      if (db + 2 < 8) kt[(db + 2) % 3] = lds_t16_frag(kl, trv, db + 2);
      __builtin_amdgcn_sched_barrier(0);
      dqacc[db][0] = mma16(kt[db % 3], sf[0], dqacc[db][0]);
      dqacc[db][1] = mma16(kt[db % 3], sf[1], dqacc[db][1]);
    }
  };

  // the first two steps' tiles start streaming, then the row operands load
  // beside them and complete here (empty asm uses pin them before the
  // loop), so no compiler wait inside the loop drains the prefetch
  if (n_steps > 0) {
    issue_loads(0, stage0);
    issue_loads(n_steps > 1 ? 1 : 0, stage1);
  }
  // B operands Q^T / dO^T: query qlo + 16 qh + li, d = 32 s + 8 lg .. +7.
  // D = rowsum(dO * O) of these rows is formed here (each (row, head) pair
  // belongs to exactly one wave of one workgroup) and written with dQ at
  // the end, for the dK/dV pass, which runs after this one (a store here
  // would hold the in-order vmcnt waits of the loop's first steps).
  #pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    const int row = qlo + 16 * qh + li;
    const size_t off = (static_cast<size_t>(row) * hq + h) * D + 8 * lg;
    float part = 0.f;
    #pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      qf[qh][s4] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(q + off + 32 * s4));
      df[qh][s4] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(dout + off + 32 * s4));
      const bf16x8_t of = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(o + off + 32 * s4));
      const bf16x8_t& dd = df[qh][s4];
      part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(of, of, 0, 1),
                                             __builtin_shufflevector(dd, dd, 0, 1), part, false);
      part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(of, of, 2, 3),
                                             __builtin_shufflevector(dd, dd, 2, 3), part, false);
      part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(of, of, 4, 5),
                                             __builtin_shufflevector(dd, dd, 4, 5), part, false);
      part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(of, of, 6, 7),
                                             __builtin_shufflevector(dd, dd, 6, 7), part, false);
    }
    dsq[qh] = quad_sum(part);  // the four lanes of this row hold its 128 d
    lse2[qh] = lse[static_cast<size_t>(h) * tr.Np + row] * kLog2e;
  }
  #pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    asm volatile("" ::"v"(lse2[qh]), "v"(dsq[qh]));
    #pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) asm volatile("" ::"v"(qf[qh][s4]), "v"(df[qh][s4]));
  }
  for (int st = 0; st < n_steps; st += 3) {  // three-stage ring: step st uses stage st % 3
    step(st, stage0, stage2);
    if (st + 1 < n_steps) step(st + 1, stage1, stage0);
    if (st + 2 < n_steps) step(st + 2, stage2, stage1);
  }
  // the last steps' prefetch must land before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  #pragma unroll
  for (int qh = 0; qh < 2; ++qh) {
    if (lg == 0) dsum[static_cast<size_t>(h) * tr.Np + qlo + 16 * qh + li] = dsq[qh];
    bf16_t* op = dq + (static_cast<size_t>(qlo + 16 * qh + li) * hq + h) * D + 4 * lg;
    #pragma unroll
    for (int db = 0; db < 8; ++db)
      store4<bf16_t>(op + 16 * db, dqacc[db][qh][0] * scale, dqacc[db][qh][1] * scale,
                     dqacc[db][qh][2] * scale, dqacc[db][qh][3] * scale);
  }
}

}  // namespace

size_t attn_bwd_bf16_d128_workspace(int Np, int hq, int hkv) {
  (void)hkv;
  return static_cast<size_t>(Np) * hq * sizeof(float);
}

hipError_t launch_attn_bwd_bf16_d128(const void* q, const void* k, const void* v, const void* o,
                                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                     void* ws, const TreeDev& tr, int hq, int hkv, float scale,
                                     hipStream_t stream) {
  const float c = scale * kLog2e;
  float* dsum = static_cast<float*>(ws);
  // dQ first: it also forms D = rowsum(dO * O) for its rows into the
  // workspace, which the dK/dV pass reads.  dQ runs in 32-query units of
  // four heads for as many heads of each group as a multiple of four
  // covers, 128-query blocks of one head for the rest, as the forward.
  const unsigned G = static_cast<unsigned>(hq / hkv), G4 = G / 4 * 4, GR = G - G4;
  const dim3 grid(static_cast<unsigned>(hkv) *
                  ((G4 / 4) * static_cast<unsigned>(tr.Np / 32) + GR * static_cast<unsigned>(tr.nb)));
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, static_cast<const bf16_t*>(q),
                       static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
                       static_cast<const bf16_t*>(o), static_cast<const bf16_t*>(dout), lse, dsum,
                       static_cast<bf16_t*>(dq), tr, hq, hkv, c, scale);
  };
  if (GR == 0)
    launch(bwd_dq_bf16<1>);
  else if (G4 > 0)
    launch(bwd_dq_bf16<2>);
  else
    launch(bwd_dq_bf16<0>);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dK/dV: persistent workgroups (one per CU at a time: their LDS allows no
  // second), each walking its lane's list of key blocks.  Lanes per
  // key/value group: the power of two P whose hkv * P workgroups, run in
  // rounds of 256, finish soonest if every lane carries the same work
  // (rounds / P smallest; the fewest workgroups on ties): 32 at eight
  // key/value heads (one workgroup per CU), 256 at five (five rounds
  // rather than 160 of the 256 CUs busy).  More rounds than needed cost
  // about 3 % (dispatch between workgroups).
  int lanes_log2 = 0;
  for (int i = 1; i < kLaneLevels; ++i) {
    const int64_t rounds_i = (static_cast<int64_t>(hkv) * (1 << i) + 255) / 256;
    const int64_t rounds_b = (static_cast<int64_t>(hkv) * (1 << lanes_log2) + 255) / 256;
    if (rounds_i * (1 << lanes_log2) < rounds_b * (1 << i)) lanes_log2 = i;
  }
  const int lanes = 1 << lanes_log2;
  hipLaunchKernelGGL(bwd_dkdv_bf16, dim3(static_cast<unsigned>(hkv) * lanes), dim3(512), 0, stream,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), static_cast<const bf16_t*>(dout), lse, dsum,
                     static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv), tr, hq, hkv, c, scale,
                     lanes, lanes_log2);
  return hipGetLastError();
}

}  // namespace pst
