// Tree attention backward pass for gfx950.
//
// Gradients of sum(dO * O) for the tree-masked softmax attention of
// attn_fwd.hip (a packed token attends only to itself and its ancestors,
// AReaL tree-training page, section "树构建过程"), with P recomputed from the
// forward LSE:
//     D_i  = sum_d dO_i . O_i
//     P_ij = exp(scale * q_i.k_j - LSE_i)          (0 where j is not visible)
//     dV_j = sum_i P_ij dO_i
//     dS_ij = P_ij (dO_i . v_j - D_i)
//     dQ_i = scale * sum_j dS_ij k_j,   dK_j = scale * sum_i dS_ij q_i
// Three kernels, no atomics (bitwise deterministic):
//   pre   D for every (head, row);
//   dkdv  one workgroup per (key block, K/V head).  Key j is visible only to
//         queries j..se[j], so the query blocks that see key block kb form the
//         contiguous range kb..kb_qhi[kb]; the workgroup walks it for each
//         query head of its group (GQA sums inside the workgroup).  Each wave
//         owns 32 keys: K and V rows sit in registers, Q and dO tiles are
//         staged in LDS both row-major and transposed;
//   dq    one workgroup per (query block, query head) over the same tile list
//         as the forward pass; Q and dO rows in registers, K (row-major and
//         transposed) and V (row-major) tiles in LDS.
// MFMA operand/accumulator conventions are those of mfma.h: an accumulator
// tile is reused directly as the B operand of the next product, its
// registers mapped to contraction slots in accumulator order.
#include "launch.h"
#include "mfma.h"

#include <cmath>

namespace pst {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <typename T, int D>
struct BwdCfg {
  static constexpr int kThreads = 256;
  static constexpr int RSTR = D + 16 / static_cast<int>(sizeof(T));  // row-major stride
  static constexpr int TSTR = kTile + 4;                             // transposed stride
  static constexpr int NDB = D / 32;
  static constexpr int NKS = D / Mfma<T>::KS;
  static constexpr int EPC = 16 / static_cast<int>(sizeof(T));
  static constexpr int CPR = D / EPC;
  static constexpr int PSTEPS = 16 / Mfma<T>::E;
};

// Stages 128 rows (row stride `stride` elements, starting at src) into a
// row-major LDS tile and, if `tdst` is given, also a transposed one.
template <typename T, int D, bool kTransposed>
__device__ __forceinline__ void stage_tile(const T* __restrict__ src, size_t stride, T* rdst,
                                           T* tdst, int tid) {
  using C = BwdCfg<T, D>;
#pragma unroll
  for (int it = tid; it < (kTile / 4) * C::CPR; it += C::kThreads) {
    const int quad = it / C::CPR, cc = it % C::CPR;
    uint4 rows[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      rows[j] = *reinterpret_cast<const uint4*>(src + (4 * quad + j) * stride + cc * C::EPC);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint4*>(rdst + (4 * quad + j) * C::RSTR + cc * C::EPC) = rows[j];
    if constexpr (kTransposed) store_transposed<T>(tdst, C::TSTR, cc * C::EPC, 4 * quad, rows);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ o,
                                                      const T* __restrict__ dout,
                                                      float* __restrict__ dsum, int Np, int hq) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int CPR = D / EPC;  // lanes per row (8, 16 or 32)
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int row = gid / CPR;  // row = i * hq + h
  const int cc = gid % CPR;
  float acc = 0.f;
  if (row < Np * hq) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + static_cast<size_t>(row) * D + cc * EPC);
    const uint4 b = *reinterpret_cast<const uint4*>(dout + static_cast<size_t>(row) * D + cc * EPC);
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w};
    const uint32_t wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (sizeof(T) == 2) {
        acc = fmaf(__uint_as_float(wa[i] << 16), __uint_as_float(wb[i] << 16), acc);
        acc = fmaf(__uint_as_float(wa[i] & 0xffff0000u), __uint_as_float(wb[i] & 0xffff0000u), acc);
      } else {
        acc = fmaf(__uint_as_float(wa[i]), __uint_as_float(wb[i]), acc);
      }
    }
  }
#pragma unroll
  for (int off = CPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < Np * hq && cc == 0) {
    const int i = row / hq, h = row % hq;
    dsum[static_cast<size_t>(h) * Np + i] = acc;
  }
}

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dsum,
    T* __restrict__ dk, T* __restrict__ dv, TreeDev tr, int hq, int hkv, float c, float scale) {
  using M = Mfma<T>;
  using C = BwdCfg<T, D>;
  __shared__ __attribute__((aligned(16))) T q_lds[kTile * C::RSTR];
  __shared__ __attribute__((aligned(16))) T qt_lds[D * C::TSTR];
  __shared__ __attribute__((aligned(16))) T do_lds[kTile * C::RSTR];
  __shared__ __attribute__((aligned(16))) T dot_lds[D * C::TSTR];
  __shared__ __attribute__((aligned(16))) float lse_lds[kTile];
  __shared__ __attribute__((aligned(16))) float d_lds[kTile];

  const int G = hq / hkv;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int g = logical / tr.nb;
  const int kb = tr.bwd_order[logical - g * tr.nb];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int lq = lane % 32;
  const int half = lane / 32;
  const int key = kb * kTile + wave * 32 + lq;
  const int sek = tr.se[key];

  typename M::Frag kf[C::NKS], vf[C::NKS];
  {
    const size_t off = (static_cast<size_t>(key) * hkv + g) * D + half * M::E;
#pragma unroll
    for (int s = 0; s < C::NKS; ++s) {
      kf[s] = M::load(k + off + s * M::KS);
      vf[s] = M::load(v + off + s * M::KS);
    }
  }
  f32x16_t dkacc[C::NDB], dvacc[C::NDB];
#pragma unroll
  for (int b = 0; b < C::NDB; ++b) {
    dkacc[b] = f32x16_t{};
    dvacc[b] = f32x16_t{};
  }

  const size_t qstride = static_cast<size_t>(hq) * D;
  const int qhi = tr.kb_qhi[kb];
  for (int qb = kb; qb <= qhi; ++qb) {
    const int q0 = qb * kTile;
    for (int r = 0; r < G; ++r) {
      const int h = g * G + r;
      __syncthreads();
      stage_tile<T, D, true>(q + static_cast<size_t>(q0) * qstride + h * D, qstride, q_lds, qt_lds, tid);
      stage_tile<T, D, true>(dout + static_cast<size_t>(q0) * qstride + h * D, qstride, do_lds, dot_lds, tid);
      if (tid < kTile) {
        lse_lds[tid] = lse[static_cast<size_t>(h) * tr.Np + q0 + tid] * kLog2e;
        d_lds[tid] = dsum[static_cast<size_t>(h) * tr.Np + q0 + tid];
      }
      __syncthreads();

      // S = Q.K^T: accumulator rows are queries, this lane's column is its key
      f32x16_t pacc[4];
#pragma unroll
      for (int qk = 0; qk < 4; ++qk) {
        pacc[qk] = f32x16_t{};
        const T* qp = q_lds + (qk * 32 + lq) * C::RSTR + half * M::E;
#pragma unroll
        for (int s = 0; s < C::NKS; ++s) pacc[qk] = M::mma(M::load(qp + s * M::KS), kf[s], pacc[qk]);
      }
#pragma unroll
      for (int qk = 0; qk < 4; ++qk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ql = qk * 32 + 8 * i + 4 * half;
          const float4 l4 = *reinterpret_cast<const float4*>(lse_lds + ql);
          const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int qg = q0 + ql + j;
            const bool vis = qg >= key && qg <= sek;
            const float p = fast_exp2(fmaf(pacc[qk][4 * i + j], c, -lv[j]));
            pacc[qk][4 * i + j] = vis ? p : 0.f;
          }
        }
      // dV^T += dO^T . P
#pragma unroll
      for (int qk = 0; qk < 4; ++qk)
#pragma unroll
        for (int st = 0; st < C::PSTEPS; ++st) {
          const typename M::Frag pf = M::from_acc(pacc[qk], st);
#pragma unroll
          for (int b = 0; b < C::NDB; ++b)
            dvacc[b] = M::mma(M::gather_keys(dot_lds + (b * 32 + lq) * C::TSTR + qk * 32, st, half), pf, dvacc[b]);
        }
      // dP = dO.V^T, then dS = P (dP - D) in place
#pragma unroll
      for (int qk = 0; qk < 4; ++qk) {
        f32x16_t dp = f32x16_t{};
        const T* dp_row = do_lds + (qk * 32 + lq) * C::RSTR + half * M::E;
#pragma unroll
        for (int s = 0; s < C::NKS; ++s) dp = M::mma(M::load(dp_row + s * M::KS), vf[s], dp);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 d4 = *reinterpret_cast<const float4*>(d_lds + qk * 32 + 8 * i + 4 * half);
          const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) pacc[qk][4 * i + j] *= dp[4 * i + j] - dv4[j];
        }
      }
      // dK^T += Q^T . dS
#pragma unroll
      for (int qk = 0; qk < 4; ++qk)
#pragma unroll
        for (int st = 0; st < C::PSTEPS; ++st) {
          const typename M::Frag sf = M::from_acc(pacc[qk], st);
#pragma unroll
          for (int b = 0; b < C::NDB; ++b)
            dkacc[b] = M::mma(M::gather_keys(qt_lds + (b * 32 + lq) * C::TSTR + qk * 32, st, half), sf, dkacc[b]);
        }
    }
  }

  const size_t off = (static_cast<size_t>(key) * hkv + g) * D;
#pragma unroll
  for (int b = 0; b < C::NDB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = b * 32 + 8 * i + 4 * half;
      store4<T>(dk + off + d, dkacc[b][4 * i] * scale, dkacc[b][4 * i + 1] * scale,
                dkacc[b][4 * i + 2] * scale, dkacc[b][4 * i + 3] * scale);
      store4<T>(dv + off + d, dvacc[b][4 * i], dvacc[b][4 * i + 1], dvacc[b][4 * i + 2], dvacc[b][4 * i + 3]);
    }
}

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void bwd_dq_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dsum,
    T* __restrict__ dq, TreeDev tr, int hq, int hkv, float c, float scale) {
  using M = Mfma<T>;
  using C = BwdCfg<T, D>;
  __shared__ __attribute__((aligned(16))) T k_lds[kTile * C::RSTR];
  __shared__ __attribute__((aligned(16))) T kt_lds[D * C::TSTR];
  __shared__ __attribute__((aligned(16))) T v_lds[kTile * C::RSTR];
  __shared__ __attribute__((aligned(16))) int32_t se_lds[kTile];

  const int G = hq / hkv;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int per_g = G * tr.nb;
  const int g = logical / per_g;
  const int rem = logical - g * per_g;
  const int rank = rem / G;
  const int h = g * G + (rem - rank * G);
  const int qb = tr.fwd_order[rank];

  const int tid = threadIdx.x;
  const int wave = tid / kWave;
  const int lane = tid % kWave;
  const int lq = lane % 32;
  const int half = lane / 32;
  const int qrow = qb * kTile + wave * 32 + lq;

  typename M::Frag qf[C::NKS], df[C::NKS];
  {
    const size_t off = (static_cast<size_t>(qrow) * hq + h) * D + half * M::E;
#pragma unroll
    for (int s = 0; s < C::NKS; ++s) {
      qf[s] = M::load(q + off + s * M::KS);
      df[s] = M::load(dout + off + s * M::KS);
    }
  }
  const float lse2 = lse[static_cast<size_t>(h) * tr.Np + qrow] * kLog2e;
  const float dsum_q = dsum[static_cast<size_t>(h) * tr.Np + qrow];
  f32x16_t dqacc[C::NDB];
#pragma unroll
  for (int b = 0; b < C::NDB; ++b) dqacc[b] = f32x16_t{};

  const size_t kv_stride = static_cast<size_t>(hkv) * D;
  const int t_end = tr.q_ptr[qb + 1];
  for (int t = tr.q_ptr[qb]; t < t_end; ++t) {
    const int tile = tr.q_tile[t];
    const int k0 = (tile >> 1) * kTile;
    const bool full = tile & 1;
    __syncthreads();
    stage_tile<T, D, true>(k + static_cast<size_t>(k0) * kv_stride + g * D, kv_stride, k_lds, kt_lds, tid);
    stage_tile<T, D, false>(v + static_cast<size_t>(k0) * kv_stride + g * D, kv_stride, v_lds, nullptr, tid);
    if (tid < kTile / 4)
      *reinterpret_cast<int4*>(se_lds + 4 * tid) = *reinterpret_cast<const int4*>(tr.se + k0 + 4 * tid);
    __syncthreads();

    // P^T = exp(S^T - LSE): accumulator rows are keys, this lane's column its query
    f32x16_t sacc[4];
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      sacc[kq] = f32x16_t{};
      const T* kp = k_lds + (kq * 32 + lq) * C::RSTR + half * M::E;
#pragma unroll
      for (int s = 0; s < C::NKS; ++s) sacc[kq] = M::mma(M::load(kp + s * M::KS), qf[s], sacc[kq]);
    }
#pragma unroll
    for (int kq = 0; kq < 4; ++kq)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kl = kq * 32 + 8 * i + 4 * half;
        const int4 se4 = *reinterpret_cast<const int4*>(se_lds + kl);
        const int sev[4] = {se4.x, se4.y, se4.z, se4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kg = k0 + kl + j;
          const bool vis = full || (kg <= qrow && qrow <= sev[j]);
          const float p = fast_exp2(fmaf(sacc[kq][4 * i + j], c, -lse2));
          sacc[kq][4 * i + j] = vis ? p : 0.f;
        }
      }
    // dP^T = V.dO^T, dS^T = P^T (dP^T - D)
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      f32x16_t dp = f32x16_t{};
      const T* vp = v_lds + (kq * 32 + lq) * C::RSTR + half * M::E;
#pragma unroll
      for (int s = 0; s < C::NKS; ++s) dp = M::mma(M::load(vp + s * M::KS), df[s], dp);
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kq][r] *= dp[r] - dsum_q;
    }
    // dQ^T += K^T . dS^T
#pragma unroll
    for (int kq = 0; kq < 4; ++kq)
#pragma unroll
      for (int st = 0; st < C::PSTEPS; ++st) {
        const typename M::Frag sf = M::from_acc(sacc[kq], st);
#pragma unroll
        for (int b = 0; b < C::NDB; ++b)
          dqacc[b] = M::mma(M::gather_keys(kt_lds + (b * 32 + lq) * C::TSTR + kq * 32, st, half), sf, dqacc[b]);
      }
  }

  T* op = dq + (static_cast<size_t>(qrow) * hq + h) * D;
#pragma unroll
  for (int b = 0; b < C::NDB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = b * 32 + 8 * i + 4 * half;
      store4<T>(op + d, dqacc[b][4 * i] * scale, dqacc[b][4 * i + 1] * scale,
                dqacc[b][4 * i + 2] * scale, dqacc[b][4 * i + 3] * scale);
    }
}

template <typename T, int D>
hipError_t launch(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  const void* dout, void* dq, void* dk, void* dv, float* ws, const TreeDev& tr,
                  int hq, int hkv, float scale, hipStream_t stream) {
  constexpr int CPR = D / (16 / static_cast<int>(sizeof(T)));
  const float c = scale * kLog2e;
  const int rows = tr.Np * hq;
  const dim3 pre_grid(static_cast<unsigned>((static_cast<int64_t>(rows) * CPR + 255) / 256));
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), pre_grid, dim3(256), 0, stream,
                     static_cast<const T*>(o), static_cast<const T*>(dout), ws, tr.Np, hq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D>), dim3(static_cast<unsigned>(tr.nb) * hkv), dim3(256), 0,
                     stream, static_cast<const T*>(q), static_cast<const T*>(k),
                     static_cast<const T*>(v), static_cast<const T*>(dout), lse, ws,
                     static_cast<T*>(dk), static_cast<T*>(dv), tr, hq, hkv, c, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D>), dim3(static_cast<unsigned>(tr.nb) * hq), dim3(256), 0,
                     stream, static_cast<const T*>(q), static_cast<const T*>(k),
                     static_cast<const T*>(v), static_cast<const T*>(dout), lse, ws,
                     static_cast<T*>(dq), tr, hq, hkv, c, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(int dtype, int head_dim, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout, void* dq, void* dk,
                           void* dv, void* workspace, const TreeDev& tr, int hq, int hkv,
                           float scale, hipStream_t stream) {
  float* ws = static_cast<float*>(workspace);
  if (dtype == kDtypeBf16) {
    if (head_dim == 128)
      return launch_attn_bwd_bf16_d128(q, k, v, o, lse, dout, dq, dk, dv, workspace, tr, hq, hkv,
                                       scale, stream);
    if (head_dim == 64)
      return launch<bf16_t, 64>(q, k, v, o, lse, dout, dq, dk, dv, ws, tr, hq, hkv, scale, stream);
  } else {
    // fp32 is built for head_dim 64 only (its LDS tiles at 128 would exceed 160 KB)
    if (head_dim == 64)
      return launch<float, 64>(q, k, v, o, lse, dout, dq, dk, dv, ws, tr, hq, hkv, scale, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pst
