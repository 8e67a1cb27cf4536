// Rotary position embedding of packed tree tokens for gfx950, in place.
//
// The position of a packed token is its depth in the trie (the position it
// has in every sequence that contains it), carried in the tree metadata.
// Dims i and i + d/2 of every head form a pair rotated by the angle
// pos * theta^(-2i/d) (the rotate-half pairing); the inverse rotation is the
// backward (gradient of the output with respect to the input, applied to the
// output gradient).
//
// One 256-thread workgroup per four rows.  Each row's d/2 angles are formed
// once: the powers theta^(-2i/d) in float64 on the host, the product with
// the position and its reduction modulo 2 pi in float64 on the device, then
// float sin/cos of the reduced angle; they are shared through LDS by all
// heads; each thread then rotates 16-byte chunks of one
// dim-pair half and its partner.  Pad rows are skipped (position 0: the
// identity).
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

constexpr int kRows = 4;  // rows per workgroup

// theta^(-2i/d) for i < d/2, formed on the host in double precision
struct InvFreq {
  double f[kTile];
};

template <typename T>
__global__ __launch_bounds__(kThreads) void rope_kernel(T* __restrict__ x, TreeDev tr, int heads,
                                                        int d, InvFreq inv, float sign) {
  constexpr int E = Vec<T>::E;
  __shared__ float cs[kRows][2][kTile];  // cos, sin of each row's d/2 angles (d <= 256)
  const int row0 = blockIdx.x * kRows;
  const int half = d / 2;
  const int tid = threadIdx.x;
  for (int k = tid; k < kRows * half; k += kThreads) {
    const int r = k / half, i = k - r * half;
    const int row = row0 + r;
    // the angle in double, reduced to [0, 2 pi) there; float sin/cos of
    // the reduced angle are then accurate to float rounding
    constexpr double kTwoPi = 6.283185307179586476925286766559;
    const double a = row < tr.Np ? static_cast<double>(tr.pos[row]) * inv.f[i] : 0.0;
    const float red = static_cast<float>(a - kTwoPi * floor(a / kTwoPi));
    float sn, cn;
    sincosf(red, &sn, &cn);
    cs[r][0][i] = cn;
    cs[r][1][i] = sign * sn;
  }
  __syncthreads();
  // chunk c of a row: head c / (half / E), dims (c % (half / E)) * E ..
  // A thread's chunk pairs are disjoint from every other thread's, so each
  // batch of kBatch pairs is loaded before any of them is rotated and
  // stored: the loads are in flight together (in place, the compiler would
  // otherwise keep every load behind the previous pair's stores).
  const int cph = half / E;  // chunks per pair half of one head
  const int per_row = heads * cph;
  constexpr int kBatch = 4;
  for (int c0 = tid; c0 < kRows * per_row; c0 += kBatch * kThreads) {
    uint4 a4[kBatch], b4[kBatch];
    uint4* p1[kBatch];
    uint4* p2[kBatch];
    int rr[kBatch], ii[kBatch];
    bool live[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int c = c0 + j * kThreads;
      const int row = row0 + c / per_row;
      // rows past the end and pad rows (position 0: the identity) are skipped
      live[j] = c < kRows * per_row && row < tr.Np && tr.row_out_ptr[row] != tr.row_out_ptr[row + 1];
      const int cl = live[j] ? c : 0;  // a skipped slot addresses chunk 0 of row0, unused
      const int r = cl / per_row;
      const int cr = cl - r * per_row;
      const int h = cr / cph;
      rr[j] = r;
      ii[j] = (cr - h * cph) * E;
      T* xr = x + static_cast<size_t>(row0 + r) * heads * d;
      p1[j] = reinterpret_cast<uint4*>(xr + h * d + ii[j]);
      p2[j] = reinterpret_cast<uint4*>(xr + h * d + half + ii[j]);
      if (live[j]) {
        a4[j] = *p1[j];
        b4[j] = *p2[j];
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (!live[j]) continue;
      float a[E], b[E], ya[E], yb[E];
      Vec<T>::unpack(a4[j], a);
      Vec<T>::unpack(b4[j], b);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float co = cs[rr[j]][0][ii[j] + e], si = cs[rr[j]][1][ii[j] + e];
        ya[e] = a[e] * co - b[e] * si;
        yb[e] = b[e] * co + a[e] * si;
      }
      *p1[j] = Vec<T>::pack(ya);
      *p2[j] = Vec<T>::pack(yb);
    }
  }
}

}  // namespace

hipError_t launch_rope(int dtype, void* x, const TreeDev& tr, int heads, int head_dim,
                       float theta, bool inverse, hipStream_t stream) {
  if (tr.Np == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((tr.Np + kRows - 1) / kRows));
  const float sign = inverse ? -1.f : 1.f;
  InvFreq inv{};
  for (int i = 0; i < head_dim / 2; ++i)
    inv.f[i] = std::pow(static_cast<double>(theta), -2.0 * i / head_dim);
  if (dtype == kDtypeBf16)
    hipLaunchKernelGGL(rope_kernel<bf16_t>, grid, dim3(kThreads), 0, stream, static_cast<bf16_t*>(x),
                       tr, heads, head_dim, inv, sign);
  else
    hipLaunchKernelGGL(rope_kernel<float>, grid, dim3(kThreads), 0, stream, static_cast<float*>(x),
                       tr, heads, head_dim, inv, sign);
  return hipGetLastError();
}

}  // namespace pst
