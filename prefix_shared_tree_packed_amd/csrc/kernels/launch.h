// Host-side launchers of the gfx950 kernels.  Shapes and pointers are
// validated by the C ABI layer before any of these is called; each launcher
// enqueues its kernels on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "common.h"

namespace pst {

constexpr int kDtypeF32 = 0;
constexpr int kDtypeBf16 = 1;

hipError_t launch_attn_fwd(int dtype, int head_dim, const void* q, const void* k, const void* v,
                           void* o, float* lse, const TreeDev& tr, int hq, int hkv, float scale,
                           hipStream_t stream);

// bf16 / head_dim 128 performance kernel (attn_fwd_bf16.hip), reached through
// launch_attn_fwd.
hipError_t launch_attn_fwd_bf16_d128(const void* q, const void* k, const void* v, void* o,
                                     float* lse, const TreeDev& tr, int hq, int hkv, float scale,
                                     hipStream_t stream);

// workspace: float32 [hq, Np] (the per-row dO.O sums).
hipError_t launch_attn_bwd(int dtype, int head_dim, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout, void* dq, void* dk,
                           void* dv, void* workspace, const TreeDev& tr, int hq, int hkv,
                           float scale, hipStream_t stream);

// bf16 / head_dim 128 performance kernels (attn_bwd_bf16.hip), reached
// through launch_attn_bwd.
size_t attn_bwd_bf16_d128_workspace(int Np, int hq, int hkv);
hipError_t launch_attn_bwd_bf16_d128(const void* q, const void* k, const void* v, const void* o,
                                     const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                     void* workspace, const TreeDev& tr, int hq, int hkv, float scale,
                                     hipStream_t stream);

// row_stats (nullable): float [Np][2], (lse, entropy) of every real row.
hipError_t launch_gather(int dtype, const void* logits, int64_t vocab, const TreeDev& tr,
                         float* logprobs, float* entropy, float* row_stats, hipStream_t stream);

// dlogits [Np, vocab] (dtype) from dlogprobs / dentropy (float32 [n_out]).
hipError_t launch_gather_bwd(int dtype, const void* logits, int64_t vocab, const TreeDev& tr,
                             const float* dlogprobs, const float* dentropy, const float* row_stats,
                             void* dlogits, hipStream_t stream);

// In-place rotary embedding of x [Np, heads, head_dim] with pos = depth
// (inverse: the opposite rotation, the backward).
hipError_t launch_rope(int dtype, void* x, const TreeDev& tr, int heads, int head_dim,
                       float theta, bool inverse, hipStream_t stream);

// Dense [Np, Np] attention mask (row = query, column = key) in one of the
// formats below; out is 16-byte aligned.
enum { kMaskU8 = 0, kMaskAddF32 = 1, kMaskAddBf16 = 2 };
hipError_t launch_dense_mask(int format, const TreeDev& tr, void* out, hipStream_t stream);

}  // namespace pst
