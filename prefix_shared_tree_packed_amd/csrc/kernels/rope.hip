// Rotary position embedding of packed tree tokens for gfx950, in place.
//
// The position of a packed token is its depth in the trie (the position it
// has in every sequence that contains it), carried in the tree metadata.
// Dims i and i + d/2 of every head form a pair rotated by the angle
// pos * theta^(-2i/d) (the rotate-half pairing); the inverse rotation is the
// backward (gradient of the output with respect to the input, applied to the
// output gradient).
//
// One 256-thread workgroup per row.  The row's d/2 angles are formed once in
// float64 (exact power, reduction modulo 2 pi, sin/cos) and shared through
// LDS by all heads; each thread then rotates 16-byte chunks of one dim-pair
// half and its partner.  Pad rows are skipped (position 0: the identity).
// HBM-bound: the tensor is read and written once.
#include "launch.h"

#include <cmath>

namespace pst {
namespace {

constexpr int kThreads = 256;

template <typename T>
struct Vec;
template <>
struct Vec<bf16_t> {
  static constexpr int E = 8;
  static __device__ __forceinline__ void unpack(const uint4& u, float (&x)[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float (&x)[8]) {
    return make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                      pack_bf16x2(x[6], x[7]));
  }
};
template <>
struct Vec<float> {
  static constexpr int E = 4;
  static __device__ __forceinline__ void unpack(const uint4& u, float (&x)[4]) {
    x[0] = __uint_as_float(u.x);
    x[1] = __uint_as_float(u.y);
    x[2] = __uint_as_float(u.z);
    x[3] = __uint_as_float(u.w);
  }
  static __device__ __forceinline__ uint4 pack(const float (&x)[4]) {
    return make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                      __float_as_uint(x[3]));
  }
};

template <typename T>
__global__ __launch_bounds__(kThreads) void rope_kernel(T* __restrict__ x, TreeDev tr, int heads,
                                                        int d, double theta, float sign) {
  constexpr int E = Vec<T>::E;
  __shared__ float cs[2][kTile];  // cos, sin of the row's d/2 angles (d <= 256)
  const int row = blockIdx.x;
  if (tr.row_out_ptr[row] == tr.row_out_ptr[row + 1]) return;  // a pad row: position 0
  const int half = d / 2;
  const int tid = threadIdx.x;
  if (tid < half) {
    const double a = static_cast<double>(tr.pos[row]) * pow(theta, -2.0 * tid / d);
    const double r = fmod(a, 6.283185307179586476925286766559);
    cs[0][tid] = static_cast<float>(cos(r));
    cs[1][tid] = sign * static_cast<float>(sin(r));
  }
  __syncthreads();
  // chunk c of the row: head c / (half / E), dims (c % (half / E)) * E ..
  const int cph = half / E;  // chunks per pair half of one head
  T* xr = x + static_cast<size_t>(row) * heads * d;
  for (int c = tid; c < heads * cph; c += kThreads) {
    const int h = c / cph;
    const int i0 = (c - h * cph) * E;
    uint4* p1 = reinterpret_cast<uint4*>(xr + h * d + i0);
    uint4* p2 = reinterpret_cast<uint4*>(xr + h * d + half + i0);
    float a[E], b[E], ya[E], yb[E];
    Vec<T>::unpack(*p1, a);
    Vec<T>::unpack(*p2, b);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float co = cs[0][i0 + e], si = cs[1][i0 + e];
      ya[e] = a[e] * co - b[e] * si;
      yb[e] = b[e] * co + a[e] * si;
    }
    *p1 = Vec<T>::pack(ya);
    *p2 = Vec<T>::pack(yb);
  }
}

}  // namespace

hipError_t launch_rope(int dtype, void* x, const TreeDev& tr, int heads, int head_dim,
                       float theta, bool inverse, hipStream_t stream) {
  if (tr.Np == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(tr.Np));
  const float sign = inverse ? -1.f : 1.f;
  if (dtype == kDtypeBf16)
    hipLaunchKernelGGL(rope_kernel<bf16_t>, grid, dim3(kThreads), 0, stream, static_cast<bf16_t*>(x),
                       tr, heads, head_dim, static_cast<double>(theta), sign);
  else
    hipLaunchKernelGGL(rope_kernel<float>, grid, dim3(kThreads), 0, stream, static_cast<float*>(x),
                       tr, heads, head_dim, static_cast<double>(theta), sign);
  return hipGetLastError();
}

}  // namespace pst
