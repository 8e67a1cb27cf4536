// Log-probability / entropy gather over packed-tree logits for gfx950.
//
// The AReaL tree-training page (section "对数概率计算") computes per-sequence
// log-probabilities from a packed tree: labels cannot come from rolling the
// input ids because positions are shared, each sequence recovers its own
// token order, and results are cached per node so shared prefixes are not
// recomputed.  Here that cache is structural: every real packed row is read
// from HBM exactly once, its log-sum-exp and entropy are formed in one
// streaming pass, and the row then serves every (sequence, position) that
// passes through it -- including a branch row, whose sequences continue with
// different next tokens.  The host's row_out_ptr / out_pos / out_tgt map
// lists those outputs per row.
//
// One 256-thread workgroup per row; pad rows (no outputs) return at once.
// Each thread streams 16-byte chunks (eight in flight, the last batch
// masked) and keeps an online (max, sum e^(x-max), sum e^(x-max)*x)
// triple; triples merge across the wave with butterfly shuffles and across
// the four waves through LDS.  Pad rows are never read.  The kernel is
// HBM-bound: N*V*sizeof(logit) bytes in, 8 bytes per output out.
#include "launch.h"

#include <cmath>

namespace pst {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

struct Acc {
  float m;  // running max (natural units)
  float s;  // sum of exp(x - m)
  float t;  // sum of exp(x - m) * x
};

__device__ __forceinline__ Acc merge(Acc a, Acc b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -INFINITY) return a;
  const float fa = fast_exp2((a.m - m) * kLog2e);
  const float fb = fast_exp2((b.m - m) * kLog2e);
  return Acc{m, a.s * fa + b.s * fb, a.t * fa + b.t * fb};
}

template <int N>
__device__ __forceinline__ void absorb(Acc& a, const float (&x)[N]) {
  float cm = x[0];
#pragma unroll
  for (int i = 1; i < N; ++i) cm = fmaxf(cm, x[i]);
  if (cm > a.m) {
    const float f = fast_exp2((a.m - cm) * kLog2e);
    a.s *= f;
    a.t *= f;
    a.m = cm;
  }
  if (a.m == -INFINITY) return;  // nothing but -inf so far
  const float mb = a.m * kLog2e;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float e = fast_exp2(fmaf(x[i], kLog2e, -mb));
    a.s += e;
    // p log-term of a zero probability is 0 (also for x = -inf, where e * x
    // would be NaN)
    a.t = fmaf(e, e > 0.f ? x[i] : 0.f, a.t);
  }
}

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t x) { return bf16_to_f32(x); }
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }

template <typename T>
__device__ __forceinline__ void unpack(const uint4& u, float (&x)[16 / sizeof(T)]);
template <>
__device__ __forceinline__ void unpack<bf16_t>(const uint4& u, float (&x)[8]) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
template <>
__device__ __forceinline__ void unpack<float>(const uint4& u, float (&x)[4]) {
  x[0] = __uint_as_float(u.x);
  x[1] = __uint_as_float(u.y);
  x[2] = __uint_as_float(u.z);
  x[3] = __uint_as_float(u.w);
}

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte chunks in flight per thread

template <typename T>
__global__ __launch_bounds__(kThreads) void gather_kernel(const T* __restrict__ logits, int64_t V,
                                                          TreeDev tr, float* __restrict__ logprobs,
                                                          float* __restrict__ entropy,
                                                          float* __restrict__ stats_out) {
  constexpr int EPC = 16 / sizeof(T);
  __shared__ Acc part[kThreads / kWave];
  __shared__ float row_stats[2];

  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int o_begin = tr.row_out_ptr[row];
  const int o_end = tr.row_out_ptr[row + 1];
  if (o_begin == o_end) return;  // a pad row: nothing reads it
  const T* x = logits + static_cast<size_t>(row) * V;

  // aligned body in 16-byte chunks, unaligned head/tail element by element
  const uintptr_t addr = reinterpret_cast<uintptr_t>(x);
  int64_t head = static_cast<int64_t>(((16 - (addr & 15)) & 15) / sizeof(T));
  if (head > V) head = V;
  const int64_t nch = (V - head) / EPC;
  const int64_t tail0 = head + nch * EPC;
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t* body = reinterpret_cast<const u32x4_t*>(x + head);

  // every batch keeps kUnroll loads in flight per thread; chunks past the
  // end read as -inf (no contribution)
  const uint32_t ninf = sizeof(T) == 2 ? 0xff80ff80u : 0xff800000u;
  const u32x4_t pad = {ninf, ninf, ninf, ninf};
  Acc a{-INFINITY, 0.f, 0.f};
  for (int64_t base = 0; base < nch; base += kUnroll * kThreads) {
    u32x4_t u[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t c = base + tid + j * kThreads;
      u[j] = c < nch ? __builtin_nontemporal_load(body + c) : pad;
    }
    // one max and one rescale per batch, then the exponentials
    float f[kUnroll * EPC];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      float g[EPC];
      unpack<T>(uint4{u[j].x, u[j].y, u[j].z, u[j].w}, g);
#pragma unroll
      for (int e = 0; e < EPC; ++e) f[j * EPC + e] = g[e];
    }
    absorb(a, f);
  }
  for (int64_t e = tid; e < head; e += kThreads) {
    float f[1] = {to_f32<T>(x[e])};
    absorb(a, f);
  }
  for (int64_t e = tail0 + tid; e < V; e += kThreads) {
    float f[1] = {to_f32<T>(x[e])};
    absorb(a, f);
  }

#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const Acc b{__shfl_xor(a.m, off), __shfl_xor(a.s, off), __shfl_xor(a.t, off)};
    a = merge(a, b);
  }
  if (tid % kWave == 0) part[tid / kWave] = a;
  __syncthreads();
  if (tid == 0) {
    Acc r = part[0];
#pragma unroll
    for (int w = 1; w < kThreads / kWave; ++w) r = merge(r, part[w]);
    const float lse = r.m + fast_log2(r.s) * kLn2;
    row_stats[0] = lse;
    row_stats[1] = lse - r.t / r.s;
    if (stats_out)  // (lse, entropy) of the row, for the backward
      *reinterpret_cast<float2*>(stats_out + 2 * static_cast<size_t>(row)) =
          make_float2(row_stats[0], row_stats[1]);
  }
  __syncthreads();
  const float lse = row_stats[0];
  const float ent = row_stats[1];
  for (int k = o_begin + tid; k < o_end; k += kThreads) {
    const int slot = tr.out_pos[k];
    const int tgt = tr.out_tgt[k];
    entropy[slot] = ent;
    logprobs[slot] = tgt < 0 ? 0.f : to_f32<T>(x[tgt]) - lse;
  }
}

// ------------------------------------------------------------------ backward
// d logits of sum(dlogprob * logprob + dentropy * entropy), one workgroup per
// row.  With log p = x - lse and H = lse - sum p x, a row serving outputs k
// (next token t_k, or none at a sequence's last position) gets
//   dx_v = -p_v (A + B (log p_v + H)) + sum_{k: t_k = v} dlogprob_k,
//   A = sum_{k with a next token} dlogprob_k,  B = sum_k dentropy_k.
// Pass 1 streams the row for (lse, H) exactly as the forward does (or, with
// STATS, takes them as the forward saved them and only sums A and B); pass 2
// streams it (again) and writes -p_v (A + B (log p_v + H));
// then each distinct target of the row is rewritten once with its one-hot
// terms added, so every element is rounded to the output type once.  Rows no
// output reads (pad rows) are zero-filled.

template <typename T>
__device__ __forceinline__ uint4 pack_out(const float (&g)[16 / sizeof(T)]);
template <>
__device__ __forceinline__ uint4 pack_out<bf16_t>(const float (&g)[8]) {
  return make_uint4(pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3]), pack_bf16x2(g[4], g[5]),
                    pack_bf16x2(g[6], g[7]));
}
template <>
__device__ __forceinline__ uint4 pack_out<float>(const float (&g)[4]) {
  return make_uint4(__float_as_uint(g[0]), __float_as_uint(g[1]), __float_as_uint(g[2]),
                    __float_as_uint(g[3]));
}
template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  return static_cast<bf16_t>(pack_bf16x2(x, 0.f) & 0xffffu);
}
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }

// -p (A + B (log p + H)) for logit x; a zero probability gives 0
__device__ __forceinline__ float grad_base(float x, float lse, float H, float A, float B) {
  const float logp = x - lse;
  const float p = fast_exp2(logp * kLog2e);
  return p > 0.f ? -p * fmaf(B, logp + H, A) : 0.f;
}

template <typename T, int TPB, bool STATS>
__global__ __launch_bounds__(TPB) void gather_bwd_kernel(
    const T* __restrict__ logits, int64_t V, TreeDev tr, const float* __restrict__ dlogprobs,
    const float* __restrict__ dentropy, const float* __restrict__ stats_in,
    T* __restrict__ dlogits) {
  constexpr int EPC = 16 / sizeof(T);
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  __shared__ Acc part[TPB / kWave];
  __shared__ float sums[2][TPB / kWave];
  __shared__ float row_stats[4];

  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int o_begin = tr.row_out_ptr[row];
  const int o_end = tr.row_out_ptr[row + 1];
  const T* x = logits + static_cast<size_t>(row) * V;
  T* gx = dlogits + static_cast<size_t>(row) * V;

  // aligned body in 16-byte chunks, unaligned head/tail element by element
  // (logits and dlogits share their alignment modulo 16)
  const uintptr_t addr = reinterpret_cast<uintptr_t>(x);
  int64_t head = static_cast<int64_t>(((16 - (addr & 15)) & 15) / sizeof(T));
  if (head > V) head = V;
  const int64_t nch = (V - head) / EPC;
  const int64_t tail0 = head + nch * EPC;
  const u32x4_t* body = reinterpret_cast<const u32x4_t*>(x + head);
  u32x4_t* gbody = reinterpret_cast<u32x4_t*>(gx + head);

  if (o_begin == o_end) {  // a pad row: nothing reads it, its gradient is 0
    const u32x4_t z = {0u, 0u, 0u, 0u};
    for (int64_t c = tid; c < nch; c += TPB) __builtin_nontemporal_store(z, gbody + c);
    for (int64_t e = tid; e < head; e += TPB) gx[e] = from_f32<T>(0.f);
    for (int64_t e = tail0 + tid; e < V; e += TPB) gx[e] = from_f32<T>(0.f);
    return;
  }

  // ---- pass 1: (max, sum e, sum e x) of the row; A and B of its outputs
  const uint32_t ninf = sizeof(T) == 2 ? 0xff80ff80u : 0xff800000u;
  const u32x4_t pad = {ninf, ninf, ninf, ninf};
  Acc a{-INFINITY, 0.f, 0.f};
  for (int64_t base = 0; base < (STATS ? 0 : nch); base += kUnroll * TPB) {
    u32x4_t u[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t c = base + tid + j * TPB;
      u[j] = c < nch ? body[c] : pad;
    }
    float f[kUnroll * EPC];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      float g[EPC];
      unpack<T>(uint4{u[j].x, u[j].y, u[j].z, u[j].w}, g);
#pragma unroll
      for (int e = 0; e < EPC; ++e) f[j * EPC + e] = g[e];
    }
    absorb(a, f);
  }
  for (int64_t e = tid; e < (STATS ? 0 : head); e += TPB) {
    float f[1] = {to_f32<T>(x[e])};
    absorb(a, f);
  }
  for (int64_t e = tail0 + tid; e < (STATS ? 0 : V); e += TPB) {
    float f[1] = {to_f32<T>(x[e])};
    absorb(a, f);
  }
  float sa = 0.f, sb = 0.f;
  for (int k = o_begin + tid; k < o_end; k += TPB) {
    const int slot = tr.out_pos[k];
    if (tr.out_tgt[k] >= 0) sa += dlogprobs[slot];
    sb += dentropy[slot];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const Acc b{__shfl_xor(a.m, off), __shfl_xor(a.s, off), __shfl_xor(a.t, off)};
    a = merge(a, b);
    sa += __shfl_xor(sa, off);
    sb += __shfl_xor(sb, off);
  }
  if (tid % kWave == 0) {
    part[tid / kWave] = a;
    sums[0][tid / kWave] = sa;
    sums[1][tid / kWave] = sb;
  }
  __syncthreads();
  if (tid == 0) {
    Acc r = part[0];
    float A = sums[0][0], B = sums[1][0];
    for (int w = 1; w < TPB / kWave; ++w) {
      r = merge(r, part[w]);
      A += sums[0][w];
      B += sums[1][w];
    }
    if (STATS) {
      const float2 st = *reinterpret_cast<const float2*>(stats_in + 2 * static_cast<size_t>(row));
      row_stats[0] = st.x;
      row_stats[1] = st.y;
    } else {
      const float lse = r.m + fast_log2(r.s) * kLn2;
      row_stats[0] = lse;
      row_stats[1] = lse - r.t / r.s;
    }
    row_stats[2] = A;
    row_stats[3] = B;
  }
  __syncthreads();
  const float lse = row_stats[0], H = row_stats[1], A = row_stats[2], B = row_stats[3];

  // ---- pass 2: -p (A + B (log p + H)) for every entry; each batch's
  // kUnroll loads are issued before any of its stores (logits and d logits
  // never overlap, but the compiler cannot move a load above a store to
  // another pointer of the same type on its own), so kUnroll 16-byte reads
  // per thread are in flight at once
  for (int64_t base = 0; base < nch; base += kUnroll * TPB) {
    u32x4_t u[kUnroll];
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t c = base + tid + j * TPB;
      u[j] = c < nch ? __builtin_nontemporal_load(body + c) : pad;
    }
#pragma unroll
    for (int j = 0; j < kUnroll; ++j) {
      const int64_t c = base + tid + j * TPB;
      if (c < nch) {
        float f[EPC], g[EPC];
        unpack<T>(uint4{u[j].x, u[j].y, u[j].z, u[j].w}, f);
#pragma unroll
        for (int e = 0; e < EPC; ++e) g[e] = grad_base(f[e], lse, H, A, B);
        const uint4 o = pack_out<T>(g);
        __builtin_nontemporal_store(u32x4_t{o.x, o.y, o.z, o.w}, gbody + c);
      }
    }
  }
  for (int64_t e = tid; e < head; e += TPB)
    gx[e] = from_f32<T>(grad_base(to_f32<T>(x[e]), lse, H, A, B));
  for (int64_t e = tail0 + tid; e < V; e += TPB)
    gx[e] = from_f32<T>(grad_base(to_f32<T>(x[e]), lse, H, A, B));
  __syncthreads();  // pass-2 stores done before the targets are rewritten

  // ---- one-hot terms: each distinct target once, its dlogprobs in order
  for (int k = o_begin + tid; k < o_end; k += TPB) {
    const int t = tr.out_tgt[k];
    if (t < 0) continue;
    bool first = true;
    for (int j = o_begin; j < k; ++j) first &= tr.out_tgt[j] != t;
    if (!first) continue;
    float add = 0.f;
    for (int j = k; j < o_end; ++j)
      if (tr.out_tgt[j] == t) add += dlogprobs[tr.out_pos[j]];
    gx[t] = from_f32<T>(grad_base(to_f32<T>(x[t]), lse, H, A, B) + add);
  }
}

// Register-resident variant: the workgroup holds its whole row (up to TPB x
// CPT 16-byte chunks, as many threads as the row needs) in registers between
// the two passes, so the row is read from HBM once.  Rows must be 16-byte
// aligned (no head/tail elements).
template <typename T, int TPB, int CPT>
__global__ __launch_bounds__(TPB) void gather_bwd_resident_kernel(
    const T* __restrict__ logits, int64_t V, TreeDev tr, const float* __restrict__ dlogprobs,
    const float* __restrict__ dentropy, T* __restrict__ dlogits) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int NW = TPB / kWave;
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  __shared__ Acc part[NW];
  __shared__ float sums[2][NW];
  __shared__ float row_stats[4];

  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int o_begin = tr.row_out_ptr[row];
  const int o_end = tr.row_out_ptr[row + 1];
  const T* x = logits + static_cast<size_t>(row) * V;
  T* gx = dlogits + static_cast<size_t>(row) * V;
  const int nch = static_cast<int>(V / EPC);
  const u32x4_t* body = reinterpret_cast<const u32x4_t*>(x);
  u32x4_t* gbody = reinterpret_cast<u32x4_t*>(gx);

  if (o_begin == o_end) {  // a pad row: its gradient is 0
    const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = tid + j * TPB;
      if (c < nch) __builtin_nontemporal_store(z, gbody + c);
    }
    return;
  }

  const uint32_t ninf = sizeof(T) == 2 ? 0xff80ff80u : 0xff800000u;
  const u32x4_t pad = {ninf, ninf, ninf, ninf};
  u32x4_t u[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = tid + j * TPB;
    u[j] = c < nch ? __builtin_nontemporal_load(body + c) : pad;
  }
  // statistics in batches of CB chunks
  constexpr int CB = 4;
  Acc a{-INFINITY, 0.f, 0.f};
#pragma unroll
  for (int j0 = 0; j0 < CPT; j0 += CB) {
    float f[CB * EPC];
#pragma unroll
    for (int j = 0; j < CB; ++j) {
      float g[EPC];
      const u32x4_t w = j0 + j < CPT ? u[j0 + j] : pad;
      unpack<T>(uint4{w.x, w.y, w.z, w.w}, g);
#pragma unroll
      for (int e = 0; e < EPC; ++e) f[j * EPC + e] = g[e];
    }
    absorb(a, f);
  }
  float sa = 0.f, sb = 0.f;
  for (int k = o_begin + tid; k < o_end; k += TPB) {
    const int slot = tr.out_pos[k];
    if (tr.out_tgt[k] >= 0) sa += dlogprobs[slot];
    sb += dentropy[slot];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const Acc b{__shfl_xor(a.m, off), __shfl_xor(a.s, off), __shfl_xor(a.t, off)};
    a = merge(a, b);
    sa += __shfl_xor(sa, off);
    sb += __shfl_xor(sb, off);
  }
  if (tid % kWave == 0) {
    part[tid / kWave] = a;
    sums[0][tid / kWave] = sa;
    sums[1][tid / kWave] = sb;
  }
  __syncthreads();
  if (tid == 0) {
    Acc r = part[0];
    float A = sums[0][0], B = sums[1][0];
    for (int w = 1; w < NW; ++w) {
      r = merge(r, part[w]);
      A += sums[0][w];
      B += sums[1][w];
    }
    const float lse = r.m + fast_log2(r.s) * kLn2;
    row_stats[0] = lse;
    row_stats[1] = lse - r.t / r.s;
    row_stats[2] = A;
    row_stats[3] = B;
  }
  __syncthreads();
  const float lse = row_stats[0], H = row_stats[1], A = row_stats[2], B = row_stats[3];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = tid + j * TPB;
    if (c < nch) {
      float f[EPC], g[EPC];
      unpack<T>(uint4{u[j].x, u[j].y, u[j].z, u[j].w}, f);
#pragma unroll
      for (int e = 0; e < EPC; ++e) g[e] = grad_base(f[e], lse, H, A, B);
      const uint4 o = pack_out<T>(g);
      __builtin_nontemporal_store(u32x4_t{o.x, o.y, o.z, o.w}, gbody + c);
    }
  }
  __syncthreads();  // pass-2 stores done before the targets are rewritten
  for (int k = o_begin + tid; k < o_end; k += TPB) {
    const int t = tr.out_tgt[k];
    if (t < 0) continue;
    bool first = true;
    for (int j = o_begin; j < k; ++j) first &= tr.out_tgt[j] != t;
    if (!first) continue;
    float add = 0.f;
    for (int j = k; j < o_end; ++j)
      if (tr.out_tgt[j] == t) add += dlogprobs[tr.out_pos[j]];
    gx[t] = from_f32<T>(grad_base(to_f32<T>(x[t]), lse, H, A, B) + add);
  }
}

}  // namespace

hipError_t launch_gather(int dtype, const void* logits, int64_t vocab, const TreeDev& tr,
                         float* logprobs, float* entropy, float* row_stats, hipStream_t stream) {
  if (tr.Np == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(tr.Np));  // pad rows exit at once
  if (dtype == kDtypeBf16)
    hipLaunchKernelGGL(gather_kernel<bf16_t>, grid, dim3(kThreads), 0, stream,
                       static_cast<const bf16_t*>(logits), vocab, tr, logprobs, entropy, row_stats);
  else
    hipLaunchKernelGGL(gather_kernel<float>, grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(logits), vocab, tr, logprobs, entropy, row_stats);
  return hipGetLastError();
}

}  // namespace pst

namespace pst {

hipError_t launch_gather_bwd(int dtype, const void* logits, int64_t vocab, const TreeDev& tr,
                             const float* dlogprobs, const float* dentropy, const float* row_stats,
                             void* dlogits, hipStream_t stream) {
  if (tr.Np == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(tr.Np));
  const size_t esz = dtype == kDtypeBf16 ? 2 : 4;
  // rows that are whole 16-byte chunks and fit a workgroup's registers (up
  // to 4096 chunks: 32768 bf16 or 16384 fp32 entries) are read once; larger
  // rows are read once too when the forward's row statistics are given, and
  // otherwise take the two-pass kernel with 1024 threads per row, which
  // keeps few enough rows in flight for their second read to hit the
  // fabric-side cache
  const bool aligned = reinterpret_cast<uintptr_t>(logits) % 16 == 0 && (vocab * esz) % 16 == 0;
  const int64_t nch = static_cast<int64_t>(vocab * esz / 16);
  auto launch = [&](auto kern, int tpb, auto tag) {
    using T = decltype(tag);
    hipLaunchKernelGGL(kern, grid, dim3(tpb), 0, stream, static_cast<const T*>(logits), vocab, tr,
                       dlogprobs, dentropy, static_cast<T*>(dlogits));
  };
  auto launch2 = [&](auto kern, int tpb, auto tag) {
    using T = decltype(tag);
    hipLaunchKernelGGL(kern, grid, dim3(tpb), 0, stream, static_cast<const T*>(logits), vocab, tr,
                       dlogprobs, dentropy, row_stats, static_cast<T*>(dlogits));
  };
  if (dtype == kDtypeBf16) {
    if (aligned && nch <= 256 * 16)
      launch(gather_bwd_resident_kernel<bf16_t, 256, 16>, 256, bf16_t{});
    else if (row_stats)
      launch2(gather_bwd_kernel<bf16_t, 512, true>, 512, bf16_t{});
    else
      launch2(gather_bwd_kernel<bf16_t, 1024, false>, 1024, bf16_t{});
  } else {
    if (aligned && nch <= 256 * 16)
      launch(gather_bwd_resident_kernel<float, 256, 16>, 256, float{});
    else if (row_stats)
      launch2(gather_bwd_kernel<float, 512, true>, 512, float{});
    else
      launch2(gather_bwd_kernel<float, 1024, false>, 1024, float{});
  }
  return hipGetLastError();
}

}  // namespace pst
