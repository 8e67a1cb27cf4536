// Tree attention backward pass, bf16 with head_dim 128: the performance path
// on gfx950.  Same mathematics and deterministic three-pass structure as
// attn_bwd.hip (D = rowsum(dO*O); dK/dV per key block walking its contiguous
// range of visible query blocks; dQ per query block over the forward tile
// list), fed the way the forward kernel of attn_fwd_bf16.hip is fed:
//
//  * prep writes, next to D, transposed copies of Q and dO (per query head)
//    and of K (per key/value head) into the caller's workspace: 128x128
//    tiles, d-major, whose token positions are permuted inside each group of
//    16 (token 16t+8a+4h+j sits at 16t+8h+4a+j).  A contraction over tokens
//    then reads each MFMA operand as ONE 16-byte LDS load, and every tile --
//    row-major or transposed -- reaches LDS by global_load_lds_dwordx4 (no
//    VGPRs, no VALU) through two named buffers: 64 queries per step in the
//    dK/dV kernel (one workgroup per CU, 129 KB), 32 keys per step in the dQ
//    kernel (49 KB, two workgroups per CU, which measured 1.5x faster than
//    one; the dK/dV kernel at 32 does not fit two waves per SIMD without
//    spilling and measured slower).
//  * Row-major LDS tiles store 16-byte chunk c of row r at c ^ (r & 15);
//    transposed half-tiles (128-byte rows) store it at c ^ ((d >> 1) & 7),
//    transposed 32-token slices (64-byte rows) at c ^ ((d >> 2) & 3).
//  * Work per (wave, 32x32 sub-block) is skipped when no pair is visible and
//    masked element by element only when some are: (unsigned)(i - j) <=
//    se[j] - j.
//  * P is rounded to bf16 before the dV product and dS before the dK and dQ
//    products; accumulation is fp32.
#include "launch.h"
#include "mfma.h"

#include <cmath>

namespace pst {
namespace {

constexpr int D = 128;
constexpr int kHalf = 64;           // tokens per pipeline step
constexpr int kRowB = 256;          // row-major tile row: 128 bf16
constexpr int kTRowB = 128;         // transposed half-tile row: 64 bf16
constexpr int kBuf = kHalf * kRowB; // 16 KB per half-tile (either layout)
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(4))) int32_t cint32;  // read-only: scalar loads

__device__ __forceinline__ cint32* cst(const int32_t* p) { return (cint32*)(p); }

__device__ __forceinline__ bf16x8_t lds_frag(const uint8_t* base, int byte_off) {
  return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(base + byte_off));
}

// token of the 128-block held at permuted position p
__device__ __forceinline__ int perm_token(int p) {
  return 16 * (p >> 4) + 8 * ((p >> 2) & 1) + 4 * ((p >> 3) & 1) + (p & 3);
}

// Row-major half-tile: 64 rows of 256 bytes starting at `src` (row stride
// `stride` bytes) -> LDS, by the four waves with 4 DMA instructions each.
__device__ __forceinline__ void dma_rows(const char* src, uint32_t stride, uint8_t* dst, int wave,
                                         int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * (4 * wave + i) + (lane >> 4);
    const int cch = (lane & 15) ^ (r & 15);
    __builtin_amdgcn_global_load_lds(src + static_cast<size_t>(r) * stride + (cch << 4),
                                     (lds_void*)(dst + (4 * wave + i) * 1024), 16, 0, 0);
  }
}

// Transposed half-tile: 128 rows (d) of 128 bytes (64 permuted positions)
// starting at `src` (row stride 256 bytes in the workspace tile) -> LDS.
__device__ __forceinline__ void dma_trows(const char* src, uint8_t* dst, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = 8 * (4 * wave + i) + (lane >> 3);
    const int cch = (lane & 7) ^ ((d >> 1) & 7);
    __builtin_amdgcn_global_load_lds(src + static_cast<size_t>(d) * kRowB + (cch << 4),
                                     (lds_void*)(dst + (4 * wave + i) * 1024), 16, 0, 0);
  }
}

// --------------------------------------------------------------------- prep
// One workgroup per (128-block, head): items with x < hq transpose Q and dO
// of query head x and compute D; items x >= hq transpose K of kv head x-hq.
constexpr int kPrepStride = D + 2;  // LDS row stride (elements): column reads conflict-free

__global__ __launch_bounds__(256) void bwd_prep_bf16(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ o,
    const bf16_t* __restrict__ dout, float* __restrict__ dsum, bf16_t* __restrict__ qt,
    bf16_t* __restrict__ dot, bf16_t* __restrict__ kt, int Np, int nb, int hq, int hkv) {
  __shared__ __attribute__((aligned(16))) bf16_t ta[kTile * kPrepStride];
  __shared__ __attribute__((aligned(16))) bf16_t tb[kTile * kPrepStride];
  const int blk = blockIdx.x % nb;
  const int x = blockIdx.x / nb;
  const bool qitem = x < hq;
  const int heads = qitem ? hq : hkv;
  const int hx = qitem ? x : x - hq;
  const int tid = threadIdx.x;
  const size_t stride = static_cast<size_t>(heads) * D;
  const bf16_t* a_src = (qitem ? q : k) + static_cast<size_t>(blk) * kTile * stride + hx * D;
  const bf16_t* b_src = dout + static_cast<size_t>(blk) * kTile * stride + hx * D;

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int cidx = tid + 256 * i;
    const int r = cidx >> 4, cc = cidx & 15;
    const uint4 va = *reinterpret_cast<const uint4*>(a_src + r * stride + cc * 8);
    uint32_t* da = reinterpret_cast<uint32_t*>(ta + r * kPrepStride + cc * 8);
    da[0] = va.x; da[1] = va.y; da[2] = va.z; da[3] = va.w;
    if (qitem) {
      const uint4 vb = *reinterpret_cast<const uint4*>(b_src + r * stride + cc * 8);
      uint32_t* db = reinterpret_cast<uint32_t*>(tb + r * kPrepStride + cc * 8);
      db[0] = vb.x; db[1] = vb.y; db[2] = vb.z; db[3] = vb.w;
    }
  }
  __syncthreads();

  if (qitem) {
    // D for the 128 rows: two threads per row, 64 dims each
    const int r = tid >> 1, hh = tid & 1;
    const bf16_t* orow = o + (static_cast<size_t>(blk) * kTile + r) * stride + hx * D + 64 * hh;
    float acc = 0.f;
#pragma unroll
    for (int c8 = 0; c8 < 8; ++c8) {
      const uint4 ov = *reinterpret_cast<const uint4*>(orow + 8 * c8);
      const uint32_t ow[4] = {ov.x, ov.y, ov.z, ov.w};
      const uint32_t* dw = reinterpret_cast<const uint32_t*>(tb + r * kPrepStride + 64 * hh + 8 * c8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t dv = dw[e];
        acc = fmaf(__uint_as_float(ow[e] << 16), __uint_as_float(dv << 16), acc);
        acc = fmaf(__uint_as_float(ow[e] & 0xffff0000u), __uint_as_float(dv & 0xffff0000u), acc);
      }
    }
    acc += __shfl_xor(acc, 1);
    if (hh == 0) dsum[static_cast<size_t>(hx) * Np + blk * kTile + r] = acc;
  }

  // transposed tiles: chunk (d, c) holds positions 8c..8c+7 of row d
  bf16_t* a_dst = (qitem ? qt : kt) + (static_cast<size_t>(hx) * nb + blk) * kTile * kTile;
  bf16_t* b_dst = dot + (static_cast<size_t>(hx) * nb + blk) * kTile * kTile;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = tid + 256 * i;
    const int c = idx >> 7, d = idx & 127;
    uint32_t wa[4], wb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r0 = perm_token(8 * c + 2 * e), r1 = perm_token(8 * c + 2 * e + 1);
      wa[e] = static_cast<uint32_t>(ta[r0 * kPrepStride + d]) |
              (static_cast<uint32_t>(ta[r1 * kPrepStride + d]) << 16);
      if (qitem)
        wb[e] = static_cast<uint32_t>(tb[r0 * kPrepStride + d]) |
                (static_cast<uint32_t>(tb[r1 * kPrepStride + d]) << 16);
    }
    *reinterpret_cast<uint4*>(a_dst + d * kTile + 8 * c) = make_uint4(wa[0], wa[1], wa[2], wa[3]);
    if (qitem)
      *reinterpret_cast<uint4*>(b_dst + d * kTile + 8 * c) = make_uint4(wb[0], wb[1], wb[2], wb[3]);
  }
}

// The dQ kernel streams 32 keys per pipeline step (8 KB per tile), so that
// two workgroups share a CU and two waves share each SIMD.
constexpr int kQStep = 32;
constexpr int kQBuf = kQStep * kRowB;  // 8 KB
constexpr int kQTRowB = kQStep * 2;    // transposed slice row: 64 bytes

// Transposed slice: 128 rows (d) of 64 bytes (32 permuted positions) at `src`
// (row stride 256 bytes in the workspace tile) -> LDS, chunk c of row d at
// c ^ ((d >> 2) & 3); two DMA instructions per wave.
__device__ __forceinline__ void dma_trows32(const char* src, uint8_t* dst, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int d = 16 * (2 * wave + i) + (lane >> 2);
    const int cch = (lane & 3) ^ ((d >> 2) & 3);
    __builtin_amdgcn_global_load_lds(src + static_cast<size_t>(d) * kRowB + (cch << 4),
                                     (lds_void*)(dst + (2 * wave + i) * 1024), 16, 0, 0);
  }
}

// Row-major slice: 32 rows of 256 bytes (row stride `stride`) -> LDS, chunk
// c of row r at c ^ (r & 15); two DMA instructions per wave.
__device__ __forceinline__ void dma_rows32(const char* src, uint32_t stride, uint8_t* dst, int wave,
                                           int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 4 * (2 * wave + i) + (lane >> 4);
    const int cch = (lane & 15) ^ (r & 15);
    __builtin_amdgcn_global_load_lds(src + static_cast<size_t>(r) * stride + (cch << 4),
                                     (lds_void*)(dst + (2 * wave + i) * 1024), 16, 0, 0);
  }
}

// --------------------------------------------------------------------- dK, dV
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dsum,
    const bf16_t* __restrict__ qt, const bf16_t* __restrict__ dot, bf16_t* __restrict__ dk,
    bf16_t* __restrict__ dv, TreeDev tr, int hq, int hkv, float c, float scale) {
  using M = Mfma<bf16_t>;
  __shared__ __attribute__((aligned(1024))) uint8_t q_l0[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t q_l1[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t qt_l0[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t qt_l1[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t do_l0[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t do_l1[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t dt_l0[kBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t dt_l1[kBuf];
  __shared__ __attribute__((aligned(16))) float ls_l0[kHalf];
  __shared__ __attribute__((aligned(16))) float ls_l1[kHalf];
  __shared__ __attribute__((aligned(16))) float dd_l0[kHalf];
  __shared__ __attribute__((aligned(16))) float dd_l1[kHalf];

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
  int roff[8];  // row-major operand chunk (row lq of a 32-row block, step s)
#pragma unroll
  for (int s = 0; s < 8; ++s) roff[s] = lq * kRowB + (((2 * s + half) ^ (lq & 15)) << 4);
  int toff[4];  // transposed operand chunk (row lq of a 32-row block, token step s)
#pragma unroll
  for (int s = 0; s < 4; ++s) toff[s] = lq * kTRowB + (((2 * s + half) ^ ((lq >> 1) & 7)) << 4);

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
    q0 = qb * kTile + kHalf * (st & 1);
  };
  auto issue_loads = [&](int st, uint8_t* ql, uint8_t* qtl, uint8_t* dol, uint8_t* dtl, float* lsl,
                         float* ddl) {
    int qb, h, q0;
    decode(st, qb, h, q0);
    const size_t row0 = static_cast<size_t>(q0) * q_bytes + static_cast<size_t>(h) * D * 2;
    dma_rows(reinterpret_cast<const char*>(q) + row0, q_bytes, ql, wave, lane);
    dma_rows(reinterpret_cast<const char*>(dout) + row0, q_bytes, dol, wave, lane);
    const size_t toff0 = ((static_cast<size_t>(h) * tr.nb + qb) * kTile * kTile + kHalf * (st & 1)) * 2;
    dma_trows(reinterpret_cast<const char*>(qt) + toff0, qtl, wave, lane);
    dma_trows(reinterpret_cast<const char*>(dot) + toff0, dtl, wave, lane);
    const size_t r0 = static_cast<size_t>(h) * tr.Np + q0;
    if (wave == 0)
      __builtin_amdgcn_global_load_lds(lse + r0 + lane, (lds_void*)lsl, 4, 0, 0);
    else if (wave == 1)
      __builtin_amdgcn_global_load_lds(dsum + r0 + lane, (lds_void*)ddl, 4, 0, 0);
  };

  auto step = [&](int st, const uint8_t* ql, const uint8_t* qtl, const uint8_t* dol,
                  const uint8_t* dtl, const float* lsl, const float* ddl, uint8_t* nql,
                  uint8_t* nqtl, uint8_t* ndol, uint8_t* ndtl, float* nlsl, float* nddl) {
    int qb, h, q0;
    decode(st, qb, h, q0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // step st staged; step st-1 consumed
    const int st_next = st + 1 < n_steps ? st + 1 : st;
    issue_loads(st_next, nql, nqtl, ndol, ndtl, nlsl, nddl);

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
          dvacc[b] = M::mma(lds_frag(dtl, b * 32 * kTRowB + toff[2 * qs + s2]), pf, dvacc[b]);
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
          dkacc[b] = M::mma(lds_frag(qtl, b * 32 * kTRowB + toff[2 * qs + s2]), sf, dkacc[b]);
      }
    }
  };

  if (n_steps > 0) issue_loads(0, q_l0, qt_l0, do_l0, dt_l0, ls_l0, dd_l0);
  for (int st = 0; st < n_steps; st += 2) {  // n_steps is even
    step(st, q_l0, qt_l0, do_l0, dt_l0, ls_l0, dd_l0, q_l1, qt_l1, do_l1, dt_l1, ls_l1, dd_l1);
    step(st + 1, q_l1, qt_l1, do_l1, dt_l1, ls_l1, dd_l1, q_l0, qt_l0, do_l0, dt_l0, ls_l0, dd_l0);
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
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const bf16_t* __restrict__ v,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dsum,
    const bf16_t* __restrict__ kt, bf16_t* __restrict__ dq, TreeDev tr, int hq, int hkv, float c,
    float scale) {
  using M = Mfma<bf16_t>;
  __shared__ __attribute__((aligned(1024))) uint8_t k_l0[kQBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t k_l1[kQBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t v_l0[kQBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t v_l1[kQBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t kt_l0[kQBuf];
  __shared__ __attribute__((aligned(1024))) uint8_t kt_l1[kQBuf];
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
  for (int s = 0; s < 8; ++s) roff[s] = lq * kRowB + (((2 * s + half) ^ (lq & 15)) << 4);
  int toff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) toff[s] = lq * kQTRowB + (((2 * s + half) ^ ((lq >> 2) & 3)) << 4);

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
  auto issue_loads = [&](int st, uint8_t* kl, uint8_t* vl, uint8_t* ktl) {
    const int kbk = step_kb(st);
    const int k0 = kbk * kTile + kQStep * (st & 3);
    // the subtree end first: its wait then leaves the DMA in flight
    se1 = tr.se[k0 + (tid & 31)];
    dma_rows32(kgb + static_cast<size_t>(k0) * kv_bytes, kv_bytes, kl, wave, lane);
    dma_rows32(vgb + static_cast<size_t>(k0) * kv_bytes, kv_bytes, vl, wave, lane);
    const size_t toff0 = ((static_cast<size_t>(g) * tr.nb + kbk) * kTile * kTile + kQStep * (st & 3)) * 2;
    dma_trows32(reinterpret_cast<const char*>(kt) + toff0, ktl, wave, lane);
  };
  auto store_span = [&](int st, int32_t* spl) {
    if (tid < kQStep) spl[tid] = se1 - (step_kb(st) * kTile + kQStep * (st & 3) + tid);
  };

  auto step = [&](int st, const uint8_t* kl, const uint8_t* vl, const uint8_t* ktl,
                  const int32_t* spl, uint8_t* nkl, uint8_t* nvl, uint8_t* nktl, int32_t* nspl) {
    const int k0 = step_kb(st) * kTile + kQStep * (st & 3);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const int st_next = st + 1 < n_steps ? st + 1 : st;
    issue_loads(st_next, nkl, nvl, nktl);

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
          dqacc[b] = M::mma(lds_frag(ktl, b * 32 * kQTRowB + toff[s2]), sf, dqacc[b]);
      }
    }
    store_span(st_next, nspl);
  };

  if (n_steps > 0) {
    issue_loads(0, k_l0, v_l0, kt_l0);
    store_span(0, sp_l0);
  }
  for (int st = 0; st < n_steps; st += 2) {  // n_steps is a multiple of 4
    step(st, k_l0, v_l0, kt_l0, sp_l0, k_l1, v_l1, kt_l1, sp_l1);
    step(st + 1, k_l1, v_l1, kt_l1, sp_l1, k_l0, v_l0, kt_l0, sp_l0);
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
  return static_cast<size_t>(Np) * hq * sizeof(float) +
         (2 * static_cast<size_t>(hq) + hkv) * Np * D * sizeof(bf16_t);
}

hipError_t launch_attn_bwd_bf16_d128(const void* q, const void* k, const void* v, const void* o,
                                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                     void* ws, const TreeDev& tr, int hq, int hkv, float scale,
                                     hipStream_t stream) {
  const float c = scale * kLog2e;
  const size_t Np = tr.Np;
  float* dsum = static_cast<float*>(ws);
  bf16_t* qt = reinterpret_cast<bf16_t*>(dsum + Np * hq);
  bf16_t* dot = qt + Np * hq * D;
  bf16_t* kt = dot + Np * hq * D;
  hipLaunchKernelGGL(bwd_prep_bf16, dim3(static_cast<unsigned>(tr.nb) * (hq + hkv)), dim3(256), 0,
                     stream, static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(o), static_cast<const bf16_t*>(dout), dsum, qt, dot, kt,
                     tr.Np, tr.nb, hq, hkv);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkdv_bf16, dim3(static_cast<unsigned>(tr.nb) * hkv), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), static_cast<const bf16_t*>(dout), lse, dsum, qt, dot,
                     static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv), tr, hq, hkv, c, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dq_bf16, dim3(static_cast<unsigned>(tr.nb) * hq), dim3(256), 0, stream,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                     static_cast<const bf16_t*>(v), static_cast<const bf16_t*>(dout), lse, dsum, kt,
                     static_cast<bf16_t*>(dq), tr, hq, hkv, c, scale);
  return hipGetLastError();
}

}  // namespace pst
