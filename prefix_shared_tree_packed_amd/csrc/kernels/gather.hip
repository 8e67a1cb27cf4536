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
                                                          float* __restrict__ entropy) {
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

}  // namespace

hipError_t launch_gather(int dtype, const void* logits, int64_t vocab, const TreeDev& tr,
                         float* logprobs, float* entropy, hipStream_t stream) {
  if (tr.Np == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(tr.Np));  // pad rows exit at once
  if (dtype == kDtypeBf16)
    hipLaunchKernelGGL(gather_kernel<bf16_t>, grid, dim3(kThreads), 0, stream,
                       static_cast<const bf16_t*>(logits), vocab, tr, logprobs, entropy);
  else
    hipLaunchKernelGGL(gather_kernel<float>, grid, dim3(kThreads), 0, stream,
                       static_cast<const float*>(logits), vocab, tr, logprobs, entropy);
  return hipGetLastError();
}

}  // namespace pst
