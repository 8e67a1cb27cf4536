// Dense attention mask of packed trees for gfx950 (for consumers that need
// the mask as a tensor, e.g. to save it for gradient checkpointing).
//
// M[i][j] is visible iff key j is query i or one of its ancestors, which in
// preorder is the subtree range j <= i <= se(j); pad rows see only
// themselves (their se is their own index).  Formats: uint8 (1 visible,
// 0 hidden) or an additive float32 / bf16 mask (0 visible, -inf hidden).
//
// Each thread owns one 16-byte chunk of columns and keeps their subtree
// ends in registers; a workgroup walks kRowsPerWg (4) rows, writing every chunk
// once with a non-temporal store.  Rows where no lane of a wave sees any of
// its keys (above the diagonal, or past every subtree of its chunk) take the
// constant hidden pattern without per-element tests.  Write-bound:
// Np * Np * element bytes.
#include "launch.h"

namespace pst {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWg = 4;  // small workgroups: enough waves in flight to saturate writes

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// E columns per 16-byte chunk; element e of the chunk is visible or not
template <int FMT>
struct MaskFmt;
template <>
struct MaskFmt<kMaskU8> {
  static constexpr int E = 16;
  static __device__ __forceinline__ u32x4_t pack(const bool (&vis)[16]) {
    u32x4_t w;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t x = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) x |= (vis[4 * q + b] ? 1u : 0u) << (8 * b);
      w[q] = x;
    }
    return w;
  }
};
template <>
struct MaskFmt<kMaskAddF32> {
  static constexpr int E = 4;
  static __device__ __forceinline__ u32x4_t pack(const bool (&vis)[4]) {
    u32x4_t w;
#pragma unroll
    for (int q = 0; q < 4; ++q) w[q] = vis[q] ? 0u : 0xff800000u;  // -inf
    return w;
  }
};
template <>
struct MaskFmt<kMaskAddBf16> {
  static constexpr int E = 8;
  static __device__ __forceinline__ u32x4_t pack(const bool (&vis)[8]) {
    u32x4_t w;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = (vis[2 * q] ? 0u : 0xff80u) | ((vis[2 * q + 1] ? 0u : 0xff80u) << 16);  // -inf
    return w;
  }
};

template <int FMT>
__global__ __launch_bounds__(kThreads) void dense_mask_kernel(TreeDev tr, void* __restrict__ out,
                                                              size_t row_bytes) {
  constexpr int E = MaskFmt<FMT>::E;
  const int c0 = (blockIdx.x * kThreads + threadIdx.x) * E;
  if (c0 >= tr.Np) return;  // Np is a multiple of 128, so a chunk is whole
  int se[E];
#pragma unroll
  for (int e = 0; e < E; e += 4) {
    const int4 s = *reinterpret_cast<const int4*>(tr.se + c0 + e);
    se[e] = s.x;
    se[e + 1] = s.y;
    se[e + 2] = s.z;
    se[e + 3] = s.w;
  }
  int se_max = se[0];
#pragma unroll
  for (int e = 1; e < E; ++e) se_max = max(se_max, se[e]);
  char* base = static_cast<char*>(out) + static_cast<size_t>(c0) * (16 / E);
  const bool none[E] = {};
  const u32x4_t hidden = MaskFmt<FMT>::pack(none);
  // row groups y, y + gridDim.y, ... (the grid's y extent is capped; Np is a
  // multiple of 128, so every group is whole)
  for (int r0 = blockIdx.y * kRowsPerWg; r0 < tr.Np; r0 += gridDim.y * kRowsPerWg)
  for (int r = r0; r < r0 + kRowsPerWg; ++r) {
    u32x4_t w;
    // most of the matrix is hidden: above the diagonal (r < c0) or past
    // every subtree of the chunk's keys; a wave whose lanes all see
    // nothing stores the hidden pattern without the per-element tests
    if (__all(r < c0 || r > se_max)) {
      w = hidden;
    } else {
      bool vis[E];
#pragma unroll
      for (int e = 0; e < E; ++e) vis[e] = c0 + e <= r && r <= se[e];
      w = MaskFmt<FMT>::pack(vis);
    }
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4_t*>(base + static_cast<size_t>(r) * row_bytes));
  }
}

template <int FMT>
hipError_t launch_fmt(const TreeDev& tr, void* out, hipStream_t stream) {
  constexpr int E = MaskFmt<FMT>::E;
  const int cols_per_wg = kThreads * E;
  // columns in x (at most Np / 1024 workgroups for float32, well inside the
  // x limit); row groups in y, capped at the y limit and strided over
  const unsigned groups = static_cast<unsigned>(tr.Np / kRowsPerWg);
  const dim3 grid(static_cast<unsigned>((tr.Np + cols_per_wg - 1) / cols_per_wg),
                  groups < 65535u ? groups : 65535u);
  const size_t row_bytes = static_cast<size_t>(tr.Np) * (16 / E);
  hipLaunchKernelGGL(dense_mask_kernel<FMT>, grid, dim3(kThreads), 0, stream, tr, out, row_bytes);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dense_mask(int format, const TreeDev& tr, void* out, hipStream_t stream) {
  if (tr.Np == 0) return hipSuccess;
  switch (format) {
    case kMaskU8:
      return launch_fmt<kMaskU8>(tr, out, stream);
    case kMaskAddF32:
      return launch_fmt<kMaskAddF32>(tr, out, stream);
    default:
      return launch_fmt<kMaskAddBf16>(tr, out, stream);
  }
}

}  // namespace pst
