// Tree attention forward pass for gfx950.
//
// A packed token attends only to itself and its ancestors (AReaL
// tree-training page, section "树构建过程", attention-mask column).  In
// preorder the queries that see key j are exactly the tokens of j's subtree,
// the contiguous range [j, se[j]], so the mask of a (query, key) pair is
//     j <= i <= se[j]
// and needs no dense mask: each 128x128 tile is either skipped (empty), run
// without a mask (full), or masked element by element from the 128 se values
// of its key block (partial).  The host encoder lists the non-empty tiles of
// every query block (q_ptr / q_tile), diagonal tile first.
//
// One workgroup = one 128-row query block x one query head; 4 waves, each
// owning 32 query rows.  Per tile, the K tile (row-major) and the V tile
// (transposed, d-major) are staged in LDS; each wave computes S^T = K.Q^T
// with Q held in registers, so a lane owns one query and reduces its row
// max/sum in registers plus one exchange with the other wave half; then
// O^T += V^T.P^T with P taken straight from the score registers (see mfma.h
// for the slot->key map).  Online softmax in the exp2 domain, fp32
// accumulation; with bf16 inputs P is rounded to bf16 before the P.V product.
//
// This file holds the generic instance (fp32, and bf16 with head_dim 64);
// bf16 with head_dim 128 runs the specialised kernel of attn_fwd_bf16.hip.
//
// Workgroups are ordered heaviest query block first (longest-processing-time
// order from the encoder) and grouped by key/value head per XCD, so the
// query heads sharing a K/V head run on one XCD and share its L2.
#include "launch.h"
#include "mfma.h"

#include <cmath>

namespace pst {
namespace {

template <typename T, int D>
struct FwdCfg {
  static constexpr int kThreads = 256;
  static constexpr int KSTR = D + 16 / static_cast<int>(sizeof(T));  // K row stride (elements)
  static constexpr int VSTR = kTile + 4;                             // V^T row stride (keys)
  static constexpr int NDB = D / 32;                                 // 32-wide d blocks
  static constexpr int NKS = D / Mfma<T>::KS;                        // contraction steps over d
  static constexpr int EPC = 16 / static_cast<int>(sizeof(T));       // elements per 16 bytes
  static constexpr int CPR = D / EPC;                                // 16-byte chunks per row
  static constexpr int PSTEPS = 16 / Mfma<T>::E;                     // P.V steps per 32 keys
};

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void tree_attn_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    T* __restrict__ o, float* __restrict__ lse, TreeDev tr, int hq, int hkv, float c) {
  using M = Mfma<T>;
  using C = FwdCfg<T, D>;
  __shared__ __attribute__((aligned(16))) T k_lds[kTile * C::KSTR];
  __shared__ __attribute__((aligned(16))) T vt_lds[D * C::VSTR];
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

  typename M::Frag qf[C::NKS];
  {
    const T* qp = q + (static_cast<size_t>(qrow) * hq + h) * D + half * M::E;
#pragma unroll
    for (int s = 0; s < C::NKS; ++s) qf[s] = M::load(qp + s * M::KS);
  }

  f32x16_t oacc[C::NDB];
#pragma unroll
  for (int b = 0; b < C::NDB; ++b) oacc[b] = f32x16_t{};
  float m = -INFINITY, l = 0.f;

  const size_t kv_stride = static_cast<size_t>(hkv) * D;
  const T* kg = k + static_cast<size_t>(g) * D;
  const T* vg = v + static_cast<size_t>(g) * D;

  const int t_end = tr.q_ptr[qb + 1];
  for (int t = tr.q_ptr[qb]; t < t_end; ++t) {
    const int tile = tr.q_tile[t];
    const int k0 = (tile >> 1) * kTile;
    const bool full = tile & 1;

    __syncthreads();  // the previous tile is consumed
#pragma unroll
    for (int ch = tid; ch < kTile * C::CPR; ch += C::kThreads) {
      const int r = ch / C::CPR, cc = ch % C::CPR;
      const uint4 val = *reinterpret_cast<const uint4*>(kg + (k0 + r) * kv_stride + cc * C::EPC);
      *reinterpret_cast<uint4*>(k_lds + r * C::KSTR + cc * C::EPC) = val;
    }
#pragma unroll
    for (int it = tid; it < (kTile / 4) * C::CPR; it += C::kThreads) {
      const int quad = it / C::CPR, cc = it % C::CPR;
      uint4 rows[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        rows[j] = *reinterpret_cast<const uint4*>(vg + (k0 + 4 * quad + j) * kv_stride + cc * C::EPC);
      store_transposed<T>(vt_lds, C::VSTR, cc * C::EPC, 4 * quad, rows);
    }
    if (tid < kTile / 4)
      *reinterpret_cast<int4*>(se_lds + 4 * tid) = *reinterpret_cast<const int4*>(tr.se + k0 + 4 * tid);
    __syncthreads();

    // S^T = K . Q^T over four 32-key blocks
    f32x16_t sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = f32x16_t{};
      const T* kp = k_lds + (kb * 32 + lq) * C::KSTR + half * M::E;
#pragma unroll
      for (int s = 0; s < C::NKS; ++s) sacc[kb] = M::mma(M::load(kp + s * M::KS), qf[s], sacc[kb]);
    }

    float mx = -INFINITY;
    if (full) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          sacc[kb][r] *= c;
          mx = fmaxf(mx, sacc[kb][r]);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kl = kb * 32 + 8 * i + 4 * half;  // first of 4 consecutive keys
          const int4 se4 = *reinterpret_cast<const int4*>(se_lds + kl);
          const int sev[4] = {se4.x, se4.y, se4.z, se4.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = k0 + kl + j;
            const bool vis = key <= qrow && qrow <= sev[j];
            const float x = vis ? sacc[kb][4 * i + j] * c : -INFINITY;
            sacc[kb][4 * i + j] = x;
            mx = fmaxf(mx, x);
          }
        }
    }
    mx = fmaxf(mx, swap_halves(mx));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m - m_use);
    float sum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(sacc[kb][r] - m_use);
        sacc[kb][r] = p;
        sum += p;
      }
    sum += swap_halves(sum);
    l = l * alpha + sum;
    m = m_new;
#pragma unroll
    for (int b = 0; b < C::NDB; ++b) oacc[b] *= alpha;

    // O^T += V^T . P^T
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int st = 0; st < C::PSTEPS; ++st) {
        const typename M::Frag pf = M::from_acc(sacc[kb], st);
#pragma unroll
        for (int b = 0; b < C::NDB; ++b) {
          const T* vrow = vt_lds + (b * 32 + lq) * C::VSTR + kb * 32;
          oacc[b] = M::mma(M::gather_keys(vrow, st, half), pf, oacc[b]);
        }
      }
  }

  const float inv = 1.f / l;
  T* op = o + (static_cast<size_t>(qrow) * hq + h) * D;
#pragma unroll
  for (int b = 0; b < C::NDB; ++b)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = b * 32 + 8 * i + 4 * half;
      store4<T>(op + d, oacc[b][4 * i] * inv, oacc[b][4 * i + 1] * inv, oacc[b][4 * i + 2] * inv,
                oacc[b][4 * i + 3] * inv);
    }
  if (half == 0) lse[static_cast<size_t>(h) * tr.Np + qrow] = (m + fast_log2(l)) * 0.69314718055994531f;
}

template <typename T, int D>
hipError_t launch(const void* q, const void* k, const void* v, void* o, float* lse,
                  const TreeDev& tr, int hq, int hkv, float scale, hipStream_t stream) {
  const float c = scale * 1.4426950408889634f;  // scores in the exp2 domain
  const dim3 grid(static_cast<unsigned>(tr.nb) * hq);
  hipLaunchKernelGGL((tree_attn_fwd_kernel<T, D>), grid, dim3(256), 0, stream,
                     static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     static_cast<T*>(o), lse, tr, hq, hkv, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(int dtype, int head_dim, const void* q, const void* k, const void* v,
                           void* o, float* lse, const TreeDev& tr, int hq, int hkv, float scale,
                           hipStream_t stream) {
  if (dtype == kDtypeBf16) {
    if (head_dim == 128) return launch_attn_fwd_bf16_d128(q, k, v, o, lse, tr, hq, hkv, scale, stream);
    if (head_dim == 64) return launch<bf16_t, 64>(q, k, v, o, lse, tr, hq, hkv, scale, stream);
  } else {
    // fp32 is built for head_dim 64 only, like the backward pass
    if (head_dim == 64) return launch<float, 64>(q, k, v, o, lse, tr, hq, hkv, scale, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pst
