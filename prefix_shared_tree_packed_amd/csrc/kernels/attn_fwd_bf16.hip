// Tree attention forward pass, bf16 with head_dim 128: the performance path
// on gfx950.  Same mathematics and work decomposition as attn_fwd.hip (one
// workgroup per 128-row query block and query head, four waves of 32 rows,
// S^T = K.Q^T with the query in the lane, O^T += V^T.P^T fed from the score
// accumulators); what changes is how every step is fed:
//
//  * Each non-empty 128x128 tile is walked in four 32-key steps through a
//    double-buffered LDS pipeline: while the waves compute one step, the next
//    step's K and V rows stream global -> LDS directly (global_load_lds_dwordx4:
//    no VGPRs, no VALU) into row-major tiles (swizzle of lds_tiles.h).  One
//    barrier per step.  33 KB of LDS and 168 VGPRs let three workgroups share
//    a CU (three waves per SIMD), which measured faster than 64-key steps at
//    two workgroups per CU: the kernel is bound by latency, not by LDS or
//    HBM bandwidth.
//  * K rows are the A operand of S^T = K.Q^T as they stand (one 16-byte read
//    per MFMA operand); the V^T operands of O^T += V^T.P^T come from the same
//    row-major V tile through two ds_read_b64_tr_b16 transposing reads, whose
//    slot order is the order in which the score accumulators feed P^T.
//  * The mask is evaluated per (wave, 32-key block): a block whose keys no
//    query of the wave sees is skipped (no MFMA, no exp), a block every query
//    sees runs unmasked, and only the rest pay the per-element test
//    (unsigned)(i - j) <= se[j] - j, three VALU ops.
//  * Scores stay unscaled; the softmax scale is folded into the exponent's
//    FMA, and the running max is refreshed lazily: O and the row sum are
//    rescaled only when a row's max grows by more than 2^8, so exponentials
//    stay below 256 and most steps skip the rescale.
#include "launch.h"
#include "lds_tiles.h"
#include "mfma.h"

#include <cmath>

namespace pst {
namespace {

constexpr int D = 128;
constexpr int kStep = 32;              // keys per pipeline step
constexpr int kSpt = kTile / kStep;    // steps per tile
constexpr int kNkb = kStep / 32;       // 32-key blocks per step
constexpr int kKRow = D * 2;              // K row: 256 B
constexpr int kBufBytes = kStep * kKRow;  // 8 KB for K, 8 KB for V
constexpr float kRescale = 8.0f;          // lazy-rescale threshold (log2 units)

typedef const __attribute__((address_space(4))) int32_t cint32;  // read-only: scalar loads

__device__ __forceinline__ cint32* cst(const int32_t* p) { return (cint32*)(p); }

__device__ __forceinline__ bf16x8_t lds_frag(const uint8_t* base, int byte_off) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(base + byte_off));
}

__global__ __launch_bounds__(256, 3) void tree_attn_fwd_bf16_d128(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    bf16_t* __restrict__ o, float* __restrict__ lse, TreeDev tr, int hq, int hkv, float c) {
  using M = Mfma<bf16_t>;
  // two separately named buffers (not one array indexed by the step parity)
  // so the compiler can tell the in-flight DMA target from the buffer being
  // read and does not drain the prefetch before every LDS read
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds0[kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t k_lds1[kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t vt_lds0[kBufBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t vt_lds1[kBufBytes];
  __shared__ __attribute__((aligned(16))) int32_t span_lds0[kStep];
  __shared__ __attribute__((aligned(16))) int32_t span_lds1[kStep];

  const int G = hq / hkv;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int per_g = G * tr.nb;
  const int g = logical / per_g;
  const int rem = logical - g * per_g;
  const int rank = rem / G;
  const int h = g * G + (rem - rank * G);
  const int qb = cst(tr.fwd_order)[rank];

  const int tid = threadIdx.x;
  // wave index as a scalar, so the per-wave block classes branch on SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int lq = lane % 32;
  const int half = lane / 32;
  const int qlo = qb * kTile + wave * 32;  // first query row of this wave
  const int qrow = qlo + lq;

  bf16x8_t qf[8];
  {
    const bf16_t* qp = q + (static_cast<size_t>(qrow) * hq + h) * D + half * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = M::load(qp + 16 * s);
  }
  // LDS byte offsets of this lane's 16-byte K chunk for contraction step s
  // (row lq of a 32-key block); V^T operands come through transposing reads
  int koff_rd[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) koff_rd[s] = lq * kKRow + (((2 * s + half) ^ rsw(lq)) << 4);
  const TrOff tro = tr_offsets(lane);

  // Global loads: a wave-uniform base pointer plus a 32-bit lane offset.
  const uint32_t kv_bytes = static_cast<uint32_t>(hkv) * D * 2;  // one token's K (or V) rows
  const char* kgb = reinterpret_cast<const char*>(k + static_cast<size_t>(g) * D);
  const char* vgb = reinterpret_cast<const char*>(v + static_cast<size_t>(g) * D);

  f32x16_t oacc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) oacc[b] = f32x16_t{};
  float m_used = -INFINITY, l = 0.f;

  cint32* q_ptr = cst(tr.q_ptr);
  cint32* q_tile = cst(tr.q_tile);
  cint32* q_cls = cst(tr.q_cls);
  const int t_begin = q_ptr[qb];
  const int n_steps = kSpt * (q_ptr[qb + 1] - t_begin);
  // tile index of a step, pinned to an SGPR so metadata reads stay scalar
  auto tile_of = [&](int st) { return __builtin_amdgcn_readfirstlane(t_begin + st / kSpt); };
  auto step_key0 = [&](int st) { return (q_tile[tile_of(st)] >> 1) * kTile + kStep * (st % kSpt); };

  int4 se4 = make_int4(0, 0, 0, 0);
  auto issue_loads = [&](int st, uint8_t* kdst, uint8_t* vdst) {
    const int k0 = step_key0(st);
    // every lane loads (lanes past 16 repeat a quad; only 16 are stored), so
    // no load sits in a divergent branch; first, so that its wait leaves the
    // DMA in flight
    se4 = *reinterpret_cast<const int4*>(tr.se + k0 + 4 * (tid & 15));
    dma_tile<kStep>(kgb + static_cast<size_t>(k0) * kv_bytes, kv_bytes, kdst, wave, lane);
    dma_tile<kStep>(vgb + static_cast<size_t>(k0) * kv_bytes, kv_bytes, vdst, wave, lane);
  };
  auto store_span = [&](int st, int32_t* sdst) {
    if (tid < kStep / 4) {
      const int key = step_key0(st) + 4 * tid;
      const int4 span = make_int4(se4.x - key, se4.y - key - 1, se4.z - key - 2, se4.w - key - 3);
      *reinterpret_cast<int4*>(sdst + 4 * tid) = span;
    }
  };

  auto step = [&](int st, const uint8_t* kcur, const uint8_t* vcur, const int32_t* scur,
                  uint8_t* knext, uint8_t* vnext, int32_t* snext) {
    const int k0 = step_key0(st);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // step st staged by every wave; step st-1 consumed
    // prefetch the next step; after the last step this reloads the last step
    // into the idle buffer (in bounds, never read) so the code stays
    // branch-free and the compiler keeps the DMA and the reads apart
    const int st_next = st + 1 < n_steps ? st + 1 : st;
    issue_loads(st_next, knext, vnext);

    // class of this wave's two 32x32 sub-blocks: 0 empty, 1 partial, 2 full
    const uint32_t bits = static_cast<uint32_t>(q_cls[tile_of(st)]);
    int cls[kNkb];
#pragma unroll
    for (int kb = 0; kb < kNkb; ++kb) cls[kb] = (bits >> (2 * (4 * wave + kNkb * (st % kSpt) + kb))) & 3;

    bool any_cls = false;
#pragma unroll
    for (int kb = 0; kb < kNkb; ++kb) any_cls |= cls[kb] != 0;
    if (any_cls) {
      // S^T = K.Q^T for the non-empty 32-key blocks
      f32x16_t sacc[kNkb];
#pragma unroll
      for (int kb = 0; kb < kNkb; ++kb) {
        sacc[kb] = f32x16_t{};
        if (cls[kb]) {
#pragma unroll
          for (int s = 0; s < 8; ++s)
            sacc[kb] = M::mma(lds_frag(kcur, kb * 32 * kKRow + koff_rd[s]), qf[s], sacc[kb]);
        }
      }

      // mask partial blocks; row max of the raw scores
      float mx = -INFINITY;
      const int A = qrow - k0 - 4 * half;
#pragma unroll
      for (int kb = 0; kb < kNkb; ++kb) {
        if (cls[kb] == 1) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int4 sp = *reinterpret_cast<const int4*>(scur + 32 * kb + 8 * i + 4 * half);
            const int spv[4] = {sp.x, sp.y, sp.z, sp.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t dlt = static_cast<uint32_t>(A - (32 * kb + 8 * i + j));
              const float x = dlt <= static_cast<uint32_t>(spv[j]) ? sacc[kb][4 * i + j] : -INFINITY;
              sacc[kb][4 * i + j] = x;
              mx = fmaxf(mx, x);
            }
          }
        } else if (cls[kb] == 2) {
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
        }
      }
      mx = max_halves(mx);
      const float mxc = mx * c;
      if (__any(mxc > m_used + kRescale)) {
        const float m_new = fmaxf(m_used, mxc);
        const float alpha = m_new == -INFINITY ? 1.f : fast_exp2(m_used - m_new);
        l *= alpha;
#pragma unroll
        for (int b = 0; b < 4; ++b) oacc[b] *= alpha;
        m_used = m_new;
      }
      const float negm = m_used == -INFINITY ? 0.f : -m_used;
      float sum = 0.f;
#pragma unroll
      for (int kb = 0; kb < kNkb; ++kb) {
        if (cls[kb]) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(sacc[kb][r], c, negm));
            sacc[kb][r] = p;
            sum += p;
          }
        }
      }
      sum = sum_halves(sum);
      l += sum;

      // O^T += V^T.P^T
#pragma unroll
      for (int kb = 0; kb < kNkb; ++kb) {
        if (cls[kb]) {
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const bf16x8_t pf = M::from_acc(sacc[kb], s2);
#pragma unroll
            for (int b = 0; b < 4; ++b)
              oacc[b] = M::mma(lds_tr_frag(vcur, tro, 32 * kb + 16 * s2, 32 * b), pf, oacc[b]);
          }
        }
      }
    }

    store_span(st_next, snext);
  };

  if (n_steps > 0) {
    issue_loads(0, k_lds0, vt_lds0);
    store_span(0, span_lds0);
  }
  for (int st = 0; st < n_steps; st += 2) {  // n_steps is a multiple of kSpt, so even
    step(st, k_lds0, vt_lds0, span_lds0, k_lds1, vt_lds1, span_lds1);
    step(st + 1, k_lds1, vt_lds1, span_lds1, k_lds0, vt_lds0, span_lds0);
  }

  const float inv = 1.f / l;
  bf16_t* op = o + (static_cast<size_t>(qrow) * hq + h) * D;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = b * 32 + 8 * i + 4 * half;
      store4<bf16_t>(op + d, oacc[b][4 * i] * inv, oacc[b][4 * i + 1] * inv,
                     oacc[b][4 * i + 2] * inv, oacc[b][4 * i + 3] * inv);
    }
  if (half == 0)
    lse[static_cast<size_t>(h) * tr.Np + qrow] = (m_used + fast_log2(l)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_attn_fwd_bf16_d128(const void* q, const void* k, const void* v, void* o,
                                     float* lse, const TreeDev& tr, int hq, int hkv, float scale,
                                     hipStream_t stream) {
  const float c = scale * 1.4426950408889634f;  // scores in the exp2 domain
  const dim3 grid(static_cast<unsigned>(tr.nb) * hq);
  hipLaunchKernelGGL(tree_attn_fwd_bf16_d128, grid, dim3(256), 0, stream,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), static_cast<bf16_t*>(o), lse, tr, hq, hkv, c);
  return hipGetLastError();
}

}  // namespace pst
