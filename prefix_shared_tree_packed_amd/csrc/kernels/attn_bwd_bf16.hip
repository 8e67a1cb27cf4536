// Tree attention backward pass, bf16 with head_dim 128: the performance path
// on gfx950.  Same mathematics and deterministic three-pass structure as
// attn_bwd.hip (D = rowsum(dO*O); dK/dV per key block walking its contiguous
// range of visible query blocks; dQ per query block over the forward tile
// list), fed the way the forward kernel of attn_fwd_bf16.hip is fed:
//
//  * Every tile reaches LDS row-major (token rows of 256 bytes) by
//    global_load_lds_dwordx4 (no VGPRs, no VALU), double-buffered through
//    two named buffers: Q and dO in 64-query steps for dK/dV (one workgroup
//    per CU), K and V in 32-key steps for dQ (two workgroups per CU).
//  * Products that contract over tokens need the tile transposed (dV^T +=
//    dO^T.P, dK^T += Q^T.dS, dQ^T += K^T.dS^T).  Their A operands come from
//    the same row-major tile through ds_read_b64_tr_b16: two transposing
//    reads per MFMA operand, at nearly the rate of ordinary 16-byte reads,
//    so no transposed copy exists anywhere and the prep pass only computes D.
//  * 16-byte chunk c of tile row r sits at c ^ rsw(r), rsw(r) = 2 (r & 7) +
//    ((r >> 3) & 1): 16 consecutive rows reading one chunk each hit 16
//    distinct positions, and a transposing read (4 aligned rows x 2 adjacent
//    chunks per 16 lanes) hits 8 distinct positions: no bank conflicts.
//  * Work per (wave, 32x32 sub-block) is skipped when no pair is visible and
//    masked element by element only when some are: (unsigned)(i - j) <=
//    se[j] - j.
//  * P is rounded to bf16 before the dV product and dS before the dK and dQ
//    products; accumulation is fp32.
#include "launch.h"
#include "lds_tiles.h"
#include "mfma.h"

#include <cmath>

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

// --------------------------------------------------------------------- D
// D[h][row] = dO[row][h] . O[row][h]: 16 lanes per (row, head), 16 bytes each.
__global__ __launch_bounds__(256) void bwd_dsum_bf16(const bf16_t* __restrict__ o,
                                                     const bf16_t* __restrict__ dout,
                                                     float* __restrict__ dsum, int Np, int hq) {
  const int pair = blockIdx.x * 16 + (threadIdx.x >> 4);  // row * hq + h
  const int part = threadIdx.x & 15;
  float acc = 0.f;
  if (pair < Np * hq) {
    const size_t off = static_cast<size_t>(pair) * D + part * 8;
    const uint4 ov = *reinterpret_cast<const uint4*>(o + off);
    const uint4 dov = *reinterpret_cast<const uint4*>(dout + off);
    const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w};
    const uint32_t dw[4] = {dov.x, dov.y, dov.z, dov.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc = fmaf(__uint_as_float(ow[e] << 16), __uint_as_float(dw[e] << 16), acc);
      acc = fmaf(__uint_as_float(ow[e] & 0xffff0000u), __uint_as_float(dw[e] & 0xffff0000u), acc);
    }
  }
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (part == 0 && pair < Np * hq) {
    const int row = pair / hq, h = pair - row * hq;
    dsum[static_cast<size_t>(h) * Np + row] = acc;
  }
}

// --------------------------------------------------------------------- dK, dV
constexpr int kKvStep = 64;                 // queries per step
constexpr int kKvBuf = kKvStep * kRowB;     // 16 KB

__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dsum,
    bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, TreeDev tr, int hq, int hkv, float c,
    float scale) {
  using M = Mfma<bf16_t>;
  __shared__ __attribute__((aligned(1024))) uint8_t q_l0[kKvBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t q_l1[kKvBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t do_l0[kKvBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t do_l1[kKvBuf];
  __shared__ __attribute__((aligned(16))) float ls_l0[kKvStep];
  __shared__ __attribute__((aligned(16))) float ls_l1[kKvStep];
  __shared__ __attribute__((aligned(16))) float dd_l0[kKvStep];
  __shared__ __attribute__((aligned(16))) float dd_l1[kKvStep];

  const int G = hq / hkv;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int g = logical / tr.nb;
  const int kb = cst(tr.bwd_order)[logical - g * tr.nb];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int lq = lane % 32;
  const int half = lane / 32;
  const int kbase = kb * kTile + 32 * wave;  // first key of this wave
  const int key = kbase + lq;
  const int span_k = tr.se[key] - key;
  cint32* blk32 = cst(tr.blk32);
  const int smin = blk32[2 * (kbase >> 5)], smax = blk32[2 * (kbase >> 5) + 1];

  bf16x8_t kf[8], vf[8];
  {
    const size_t off = (static_cast<size_t>(key) * hkv + g) * D + half * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kf[s] = M::load(k + off + 16 * s);
      vf[s] = M::load(v + off + 16 * s);
    }
  }
  int roff[8];  // row operand: row lq of a 32-row block, contraction step s
#pragma unroll
  for (int s = 0; s < 8; ++s) roff[s] = lq * kRowB + (((2 * s + half) ^ rsw(lq)) << 4);
  const TrOff tro = tr_offsets(lane);

  f32x16_t dkacc[4], dvacc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    dkacc[b] = f32x16_t{};
    dvacc[b] = f32x16_t{};
  }

  const uint32_t q_bytes = static_cast<uint32_t>(hq) * D * 2;  // one token's Q (or dO) rows
  const int qhi = cst(tr.kb_qhi)[kb];
  const int n_steps = (qhi - kb + 1) * G * 2;
  // step -> (query block, head, half); steps walk halves, then heads, then blocks
  auto decode = [&](int st, int& qb, int& h, int& q0) {
    const int rest = st >> 1;
    const int r = rest % G;
    qb = kb + rest / G;
    h = g * G + r;
    q0 = qb * kTile + kKvStep * (st & 1);
  };
  auto issue_loads = [&](int st, uint8_t* ql, uint8_t* dol, float* lsl, float* ddl) {
    int qb, h, q0;
    decode(st, qb, h, q0);
    const size_t row0 = static_cast<size_t>(q0) * q_bytes + static_cast<size_t>(h) * D * 2;
    dma_tile<kKvStep>(reinterpret_cast<const char*>(q) + row0, q_bytes, ql, wave, lane);
    dma_tile<kKvStep>(reinterpret_cast<const char*>(dout) + row0, q_bytes, dol, wave, lane);
    const size_t r0 = static_cast<size_t>(h) * tr.Np + q0;
    if (wave == 0)
      __builtin_amdgcn_global_load_lds(lse + r0 + lane, (lds_void*)lsl, 4, 0, 0);
    else if (wave == 1)
      __builtin_amdgcn_global_load_lds(dsum + r0 + lane, (lds_void*)ddl, 4, 0, 0);
  };

  auto step = [&](int st, const uint8_t* ql, const uint8_t* dol, const float* lsl, const float* ddl,
                  uint8_t* nql, uint8_t* ndol, float* nlsl, float* nddl) {
    int qb, h, q0;
    decode(st, qb, h, q0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // step st staged; step st-1 consumed
    const int st_next = st + 1 < n_steps ? st + 1 : st;
    issue_loads(st_next, nql, ndol, nlsl, nddl);

    const int A = q0 + 4 * half - key;  // (query - key) of register 0 of sub-block 0
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int qlo = q0 + 32 * qs;
      const bool empty = kbase > qlo + 31 || smax < qlo;
      if (empty) continue;
      const bool full = kbase + 31 <= qlo && smin >= qlo + 31;

      // S = Q.K^T: rows are queries, this lane's column is its key
      f32x16_t p = f32x16_t{};
#pragma unroll
      for (int s = 0; s < 8; ++s) p = M::mma(lds_frag(ql, qs * 32 * kRowB + roff[s]), kf[s], p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 l4 = *reinterpret_cast<const float4*>(lsl + 32 * qs + 8 * i + 4 * half);
        const float lv[4] = {l4.x * kLog2e, l4.y * kLog2e, l4.z * kLog2e, l4.w * kLog2e};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float e = fast_exp2(fmaf(p[4 * i + j], c, -lv[j]));
          if (full) {
            p[4 * i + j] = e;
          } else {
            const uint32_t dlt = static_cast<uint32_t>(A + 32 * qs + 8 * i + j);
            p[4 * i + j] = dlt <= static_cast<uint32_t>(span_k) ? e : 0.f;
          }
        }
      }
      // dV^T += dO^T.P
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8_t pf = M::from_acc(p, s2);
#pragma unroll
        for (int b = 0; b < 4; ++b)
          dvacc[b] = M::mma(lds_tr_frag(dol, tro, 32 * qs + 16 * s2, 32 * b), pf, dvacc[b]);
      }
      // dP = dO.V^T, dS = P (dP - D)
      f32x16_t dp = f32x16_t{};
#pragma unroll
      for (int s = 0; s < 8; ++s) dp = M::mma(lds_frag(dol, qs * 32 * kRowB + roff[s]), vf[s], dp);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 d4 = *reinterpret_cast<const float4*>(ddl + 32 * qs + 8 * i + 4 * half);
        const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) p[4 * i + j] *= dp[4 * i + j] - dv4[j];
      }
      // dK^T += Q^T.dS
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8_t sf = M::from_acc(p, s2);
#pragma unroll
        for (int b = 0; b < 4; ++b)
          dkacc[b] = M::mma(lds_tr_frag(ql, tro, 32 * qs + 16 * s2, 32 * b), sf, dkacc[b]);
      }
    }
  };

  if (n_steps > 0) issue_loads(0, q_l0, do_l0, ls_l0, dd_l0);
  for (int st = 0; st < n_steps; st += 2) {  // n_steps is even
    step(st, q_l0, do_l0, ls_l0, dd_l0, q_l1, do_l1, ls_l1, dd_l1);
    step(st + 1, q_l1, do_l1, ls_l1, dd_l1, q_l0, do_l0, ls_l0, dd_l0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const size_t off = (static_cast<size_t>(key) * hkv + g) * D;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = b * 32 + 8 * i + 4 * half;
      store4<bf16_t>(dk + off + d, dkacc[b][4 * i] * scale, dkacc[b][4 * i + 1] * scale,
                     dkacc[b][4 * i + 2] * scale, dkacc[b][4 * i + 3] * scale);
      store4<bf16_t>(dv + off + d, dvacc[b][4 * i], dvacc[b][4 * i + 1], dvacc[b][4 * i + 2],
                     dvacc[b][4 * i + 3]);
    }
}

// --------------------------------------------------------------------- dQ
// 32-key steps (two 8 KB tiles per stage, 33 KB of LDS): two workgroups per
// CU, two waves per SIMD.
constexpr int kQStep = 32;
constexpr int kQBuf = kQStep * kRowB;  // 8 KB

__global__ __launch_bounds__(256, 2) void bwd_dq_bf16(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dsum,
    bf16_t* __restrict__ dq, TreeDev tr, int hq, int hkv, float c, float scale) {
  using M = Mfma<bf16_t>;
  __shared__ __attribute__((aligned(1024))) uint8_t k_l0[kQBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t k_l1[kQBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t v_l0[kQBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t v_l1[kQBuf];
  __shared__ __attribute__((aligned(16))) int32_t sp_l0[kQStep];
  __shared__ __attribute__((aligned(16))) int32_t sp_l1[kQStep];

  const int G = hq / hkv;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int per_g = G * tr.nb;
  const int g = logical / per_g;
  const int rem = logical - g * per_g;
  const int rank = rem / G;
  const int h = g * G + (rem - rank * G);
  const int qb = cst(tr.fwd_order)[rank];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int lane = tid % kWave;
  const int lq = lane % 32;
  const int half = lane / 32;
  const int qrow = qb * kTile + wave * 32 + lq;

  bf16x8_t qf[8], df[8];
  {
    const size_t off = (static_cast<size_t>(qrow) * hq + h) * D + half * 8;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qf[s] = M::load(q + off + 16 * s);
      df[s] = M::load(dout + off + 16 * s);
    }
  }
  const float lse2 = lse[static_cast<size_t>(h) * tr.Np + qrow] * kLog2e;
  const float dsum_q = dsum[static_cast<size_t>(h) * tr.Np + qrow];
  int roff[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) roff[s] = lq * kRowB + (((2 * s + half) ^ rsw(lq)) << 4);
  const TrOff tro = tr_offsets(lane);

  f32x16_t dqacc[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) dqacc[b] = f32x16_t{};

  const uint32_t kv_bytes = static_cast<uint32_t>(hkv) * D * 2;
  const char* kgb = reinterpret_cast<const char*>(k + static_cast<size_t>(g) * D);
  const char* vgb = reinterpret_cast<const char*>(v + static_cast<size_t>(g) * D);
  cint32* q_ptr = cst(tr.q_ptr);
  cint32* q_tile = cst(tr.q_tile);
  cint32* q_cls = cst(tr.q_cls);
  const int t_begin = q_ptr[qb];
  const int n_steps = 4 * (q_ptr[qb + 1] - t_begin);  // four 32-key steps per tile
  auto tile_of = [&](int st) { return __builtin_amdgcn_readfirstlane(t_begin + (st >> 2)); };
  auto step_kb = [&](int st) { return q_tile[tile_of(st)] >> 1; };

  int se1 = 0;
  auto issue_loads = [&](int st, uint8_t* kl, uint8_t* vl) {
    const int k0 = step_kb(st) * kTile + kQStep * (st & 3);
    // the subtree end first: its wait then leaves the DMA in flight
    se1 = tr.se[k0 + (tid & 31)];
    dma_tile<kQStep>(kgb + static_cast<size_t>(k0) * kv_bytes, kv_bytes, kl, wave, lane);
    dma_tile<kQStep>(vgb + static_cast<size_t>(k0) * kv_bytes, kv_bytes, vl, wave, lane);
  };
  auto store_span = [&](int st, int32_t* spl) {
    if (tid < kQStep) spl[tid] = se1 - (step_kb(st) * kTile + kQStep * (st & 3) + tid);
  };

  auto step = [&](int st, const uint8_t* kl, const uint8_t* vl, const int32_t* spl, uint8_t* nkl,
                  uint8_t* nvl, int32_t* nspl) {
    const int k0 = step_kb(st) * kTile + kQStep * (st & 3);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int st_next = st + 1 < n_steps ? st + 1 : st;
    issue_loads(st_next, nkl, nvl);

    const uint32_t bits = static_cast<uint32_t>(q_cls[tile_of(st)]);
    const int cls = (bits >> (2 * (4 * wave + (st & 3)))) & 3;
    if (cls != 0) {
      const int A = qrow - k0 - 4 * half;
      // P^T (rows are keys, this lane's column is its query), dP^T = V.dO^T
      f32x16_t p = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        p = M::mma(lds_frag(kl, roff[s]), qf[s], p);
        dp = M::mma(lds_frag(vl, roff[s]), df[s], dp);
      }
      if (cls == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int4 sp = *reinterpret_cast<const int4*>(spl + 8 * i + 4 * half);
          const int spv[4] = {sp.x, sp.y, sp.z, sp.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t dlt = static_cast<uint32_t>(A - (8 * i + j));
            const float e = fast_exp2(fmaf(p[4 * i + j], c, -lse2));
            p[4 * i + j] = dlt <= static_cast<uint32_t>(spv[j]) ? e : 0.f;
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = fast_exp2(fmaf(p[r], c, -lse2));
      }
      // dS^T = P^T (dP^T - D), dQ^T += K^T.dS^T
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] *= dp[r] - dsum_q;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8_t sf = M::from_acc(p, s2);
#pragma unroll
        for (int b = 0; b < 4; ++b)
          dqacc[b] = M::mma(lds_tr_frag(kl, tro, 16 * s2, 32 * b), sf, dqacc[b]);
      }
    }
    store_span(st_next, nspl);
  };

  if (n_steps > 0) {
    issue_loads(0, k_l0, v_l0);
    store_span(0, sp_l0);
  }
  for (int st = 0; st < n_steps; st += 2) {  // n_steps is a multiple of 4
    step(st, k_l0, v_l0, sp_l0, k_l1, v_l1, sp_l1);
    step(st + 1, k_l1, v_l1, sp_l1, k_l0, v_l0, sp_l0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  bf16_t* op = dq + (static_cast<size_t>(qrow) * hq + h) * D;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = b * 32 + 8 * i + 4 * half;
      store4<bf16_t>(op + d, dqacc[b][4 * i] * scale, dqacc[b][4 * i + 1] * scale,
                     dqacc[b][4 * i + 2] * scale, dqacc[b][4 * i + 3] * scale);
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
  const unsigned pairs = static_cast<unsigned>(tr.Np) * hq;
  hipLaunchKernelGGL(bwd_dsum_bf16, dim3((pairs + 15) / 16), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(o), static_cast<const bf16_t*>(dout), dsum, tr.Np, hq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkdv_bf16, dim3(static_cast<unsigned>(tr.nb) * hkv), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), static_cast<const bf16_t*>(dout), lse, dsum,
                     static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv), tr, hq, hkv, c, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dq_bf16, dim3(static_cast<unsigned>(tr.nb) * hq), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), static_cast<const bf16_t*>(dout), lse, dsum,
                     static_cast<bf16_t*>(dq), tr, hq, hkv, c, scale);
  return hipGetLastError();
}

}  // namespace pst
