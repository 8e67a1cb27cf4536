// The device entry points of libpst's C ABI (declared in include/pst.h):
// argument checks, the device metadata, and kernel dispatch.  The host-only
// entry points (builder, forest accessors, packing, error status) are in
// capi_host.cpp.
#include "pst.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <numeric>
#include <queue>
#include <vector>
#include <mutex>
#include <new>
#include <string>

#include "capi_internal.h"
#include "kernels/launch.h"

using pst::check_tree;
using pst::fail;
using pst::fill_sizes;
using pst::ok;

// Device scratch of pst_tree_attn_bwd_noalloc: the backward's per-row sums
// D = rowsum(dO * O) (float32 [hq, Np]), which pst_tree_attn_bwd takes in a
// caller workspace.  One copy per GPU the library runs on, held until the
// process ends.  Host code never passes `scratch` itself to a kernel (in
// host code the name is a stand-in, not a device address): it uses the
// device address that hipGetSymbolAddress returns for the current device.
constexpr size_t kNoAllocScratchBytes = size_t{64} << 20;  // 64 MiB
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

// Device layout of one tree's metadata: a single int32 allocation holding
// se [Np] | q_ptr [nb+1] | q_tile [n_tiles] | kb_qhi [nb] | fwd_order [nb] |
// bwd_order [nb] | row_out_ptr [Np+1] | out_pos [n_out] | out_tgt [n_out] |
// blk32 [Np/32][2] (min, max subtree end of each 32-key block) |
// q_cls [n_tiles] (32x32 sub-block classes of each tile) | step_ptr [nb+1] |
// steps [n_steps] (the non-empty 32-key columns of each query block's
// tiles: (32-key block << 8) | the four 32-query sub-blocks' classes) |
// unit_ptr [Np/32+1] | unit_steps [n_blk32] (the non-empty 32x32 blocks of
// each 32-query unit: (32-key block << 2) | class) | unit_order [Np/32] |
// pos [Np] (depth of every row, 0 for pad rows), every section starting on
// a 16-byte boundary.  It is filled in one of two pinned staging buffers and
// uploaded asynchronously; the uploads alternate between the two, and an
// event after each upload says when its staging buffer may be refilled, so
// an update waits only for the upload issued two updates before.
struct pst_tree_meta {
  int device = -1;
  int32_t* dbuf = nullptr;   // device words (capacity dcap)
  size_t dcap = 0;
  int32_t* hbuf[2] = {nullptr, nullptr};  // pinned staging (capacity hcap[i])
  size_t hcap[2] = {0, 0};
  hipEvent_t uploaded[2] = {nullptr, nullptr};  // after the upload from hbuf[i]
  bool pending[2] = {false, false};             // uploaded[i] recorded
  int next = 0;                                 // staging buffer of the next update
  bool valid = false;  // false while an upload is in progress or after one failed
  size_t n_words = 0;
  pst_tree_sizes sizes{};
  pst::TreeDev dev{};
  int32_t min_target = 0;
  int32_t max_target = -1;
};

namespace {

int hip_fail(hipError_t e, const char* what) {
  return fail(PST_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// The metadata lives on the current device and, unless only its device is
// asked about, holds a complete upload.
int check_meta_device(const pst_tree_meta* meta, bool need_valid = true) {
  if (need_valid && !meta->valid)
    return fail(PST_EINVAL, "tree metadata is not usable: its last update failed");
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != meta->device)
    return fail(PST_EINVAL, "tree metadata lives on device " + std::to_string(meta->device) +
                                " but the current device is " + std::to_string(dev));
  return PST_OK;
}

int check_attn_args(const pst_tree_meta* meta, int32_t hq, int32_t hkv, int32_t head_dim,
                    int32_t dtype) {
  if (!meta) return fail(PST_EINVAL, "tree metadata is NULL");
  if (dtype != PST_F32 && dtype != PST_BF16)
    return fail(PST_EDTYPE, "unknown dtype " + std::to_string(dtype));
  if (hq <= 0 || hkv <= 0) return fail(PST_ESHAPE, "head counts must be positive");
  if (hq % hkv)
    return fail(PST_ESHAPE, "hq=" + std::to_string(hq) + " is not a multiple of hkv=" +
                                std::to_string(hkv));
  if (dtype == PST_BF16 && head_dim != 64 && head_dim != 128)
    return fail(PST_ESHAPE, "bf16 head_dim must be 64 or 128, got " + std::to_string(head_dim));
  if (dtype == PST_F32 && head_dim != 64)
    return fail(PST_ESHAPE, "fp32 head_dim must be 64, got " + std::to_string(head_dim));
  if (static_cast<int64_t>(meta->sizes.n_padded) * hq >= (int64_t{1} << 31))
    return fail(PST_ESHAPE, "Np * hq exceeds 2^31");
  return PST_OK;
}

int check_ptrs(std::initializer_list<const void*> ps, const char* names) {
  for (const void* p : ps) {
    if (!p) return fail(PST_EINVAL, std::string("NULL device pointer among ") + names);
    if (!aligned16(p)) return fail(PST_ESHAPE, std::string("device pointer not 16-byte aligned among ") + names);
  }
  return PST_OK;
}

// Device address of `scratch` on the current device, looked up on the
// device's first call and kept.
int scratch_on_current_device(void** out) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* ptrs[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PST_EINVAL, "device " + std::to_string(dev) + " beyond the scratch table");
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(PST_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return PST_OK;
}

float resolve_scale(float s, int32_t head_dim) {
  return s > 0.f ? s : 1.0f / std::sqrt(static_cast<float>(head_dim));
}

// Builds the metadata of `trees`, laid back to back in the given order, and
// uploads it into `m` on `stream`, reusing m's buffers when they are large
// enough: rows of tree t follow the padded rows of the trees before it, its
// outputs follow theirs.  Attention never crosses trees, so the
// concatenation is itself a valid packed layout and one launch serves all of
// them.
int upload_meta(const std::vector<const pst::Tree*>& trees, void* stream, pst_tree_meta* m) {
  int64_t Np = 0, nb = 0, n_tiles = 0, n_out = 0, n_steps = 0, n_blk32 = 0;
  pst_tree_sizes sz{};
  // the four 32-query sub-blocks' classes of column ks of a tile
  auto column_classes = [](int32_t bits, int ks) {
    int32_t c4 = 0;
    for (int qs = 0; qs < 4; ++qs) c4 |= ((bits >> (2 * (4 * qs + ks))) & 3) << (2 * qs);
    return c4;
  };
  for (const pst::Tree* t : trees) {
    pst_tree_sizes ts{};
    fill_sizes(*t, &ts);
    for (int32_t bits : t->q_cls)
      for (int ks = 0; ks < 4; ++ks) {
        n_steps += column_classes(bits, ks) != 0;
        for (int qs = 0; qs < 4; ++qs) n_blk32 += ((bits >> (2 * (4 * qs + ks))) & 3) != 0;
      }
    Np += t->Np;
    nb += t->nb;
    n_tiles += t->n_tiles();
    n_out += t->n_out();
    sz.n_tokens += ts.n_tokens;
    sz.n_nodes += ts.n_nodes;
    sz.n_seqs += ts.n_seqs;
    sz.n_edges += ts.n_edges;
    sz.n_node_seq += ts.n_node_seq;
    sz.n_pairs += ts.n_pairs;
  }
  if (Np >= (int64_t{1} << 30) || n_out >= (int64_t{1} << 31) || n_tiles >= (int64_t{1} << 31))
    return fail(PST_EINVAL, "forest too large for 32-bit row, tile or output indices");
  sz.n_padded = static_cast<int32_t>(Np);
  sz.n_blocks = static_cast<int32_t>(nb);
  sz.n_tiles = static_cast<int32_t>(n_tiles);
  sz.n_out = n_out;

  auto round4 = [](int64_t n) { return static_cast<size_t>((n + 3) / 4 * 4); };
  size_t off = 0;
  const size_t o_se = off;        off += round4(Np);
  const size_t o_qptr = off;      off += round4(nb + 1);
  const size_t o_qtile = off;     off += round4(n_tiles);
  const size_t o_qhi = off;       off += round4(nb);
  const size_t o_ford = off;      off += round4(nb);
  const size_t o_bord = off;      off += round4(nb);
  const size_t o_rptr = off;      off += round4(Np + 1);
  const size_t o_opos = off;      off += round4(n_out);
  const size_t o_otgt = off;      off += round4(n_out);
  const size_t o_blk = off;       off += round4(Np / 16);
  const size_t o_qcls = off;      off += round4(n_tiles);
  const size_t o_sptr = off;      off += round4(nb + 1);
  const size_t o_step = off;      off += round4(n_steps);
  const size_t o_uptr = off;      off += round4(Np / 32 + 1);
  const size_t o_ustep = off;     off += round4(n_blk32);
  const size_t o_uord = off;      off += round4(Np / 32);
  const size_t o_pos = off;       off += round4(Np);
  const size_t o_lanes = off;     off += round4((2 * pst::kMaxLanes - 1) + (pst::kLaneLevels + pst::kLaneLevels * nb));
  const size_t words = off;

  // until this upload completes, device calls refuse the metadata (a failure
  // below may have released the buffers its device view points into)
  m->valid = false;
  const int buf = m->next;
  // the staging buffer's previous upload must have read it before refilling
  if (m->pending[buf]) {
    hipError_t e = hipEventSynchronize(m->uploaded[buf]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    m->pending[buf] = false;
  }
  if (m->hcap[buf] < words) {
    if (m->hbuf[buf]) {
      hipError_t e = hipHostFree(m->hbuf[buf]);
      m->hbuf[buf] = nullptr;
      m->hcap[buf] = 0;
      if (e != hipSuccess) return hip_fail(e, "hipHostFree");
    }
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&m->hbuf[buf]), words * sizeof(int32_t),
                                 hipHostMallocDefault);
    if (e != hipSuccess) {
      m->hbuf[buf] = nullptr;
      return fail(PST_ENOMEM, std::string("hipHostMalloc: ") + hipGetErrorString(e));
    }
    m->hcap[buf] = words;
  }
  if (m->dcap < words) {
    if (m->dbuf) {
      // queued work on any stream may still read the old words
      hipError_t e = hipDeviceSynchronize();
      if (e != hipSuccess) return hip_fail(e, "hipDeviceSynchronize");
      e = hipFree(m->dbuf);
      m->dbuf = nullptr;
      m->dcap = 0;
      if (e != hipSuccess) return hip_fail(e, "hipFree");
    }
    hipError_t e = hipMalloc(reinterpret_cast<void**>(&m->dbuf), words * sizeof(int32_t));
    if (e != hipSuccess) {
      m->dbuf = nullptr;
      return fail(PST_ENOMEM, std::string("hipMalloc: ") + hipGetErrorString(e));
    }
    m->dcap = words;
  }
  m->min_target = 0;
  m->max_target = -1;
  int32_t* h = m->hbuf[buf];
  std::memset(h, 0, words * sizeof(int32_t));
  int32_t row0 = 0, blk0 = 0, tile0 = 0, out0 = 0;
  bool any_target = false;
  for (const pst::Tree* tp : trees) {
    const pst::Tree& t = *tp;
    for (int32_t i = 0; i < t.Np; ++i) h[o_se + row0 + i] = t.se[i] + row0;
    for (int32_t i = 0; i < t.Np; ++i) h[o_pos + row0 + i] = t.pos[i];
    for (int32_t qb = 0; qb < t.nb; ++qb) h[o_qptr + blk0 + qb] = tile0 + t.q_ptr[qb];
    for (int32_t i = 0; i < t.n_tiles(); ++i) {
      h[o_qtile + tile0 + i] = ((t.q_kb[i] + blk0) << 1) | (t.q_full[i] & 1);
      h[o_qcls + tile0 + i] = t.q_cls[i];
    }
    for (int32_t kb = 0; kb < t.nb; ++kb) h[o_qhi + blk0 + kb] = t.kb_qhi[kb] + blk0;
    for (int32_t r = 0; r < t.Np; ++r)
      h[o_rptr + row0 + r] = out0 + (r < t.N ? t.row_out_ptr[r] : static_cast<int32_t>(t.n_out()));
    for (int64_t o = 0; o < t.n_out(); ++o) {
      h[o_opos + out0 + o] = out0 + t.out_pos[o];
      h[o_otgt + out0 + o] = t.out_tgt[o];
    }
    if (t.max_target >= 0) {
      m->min_target = any_target ? std::min(m->min_target, t.min_target) : t.min_target;
      m->max_target = any_target ? std::max(m->max_target, t.max_target) : t.max_target;
      any_target = true;
    }
    row0 += t.Np;
    blk0 += t.nb;
    tile0 += t.n_tiles();
    out0 += static_cast<int32_t>(t.n_out());
  }
  h[o_qptr + nb] = tile0;
  h[o_rptr + Np] = out0;
  {  // compacted step lists: a column every wave of the query block skips is not staged
    int32_t ns = 0;
    for (int64_t qb = 0; qb < nb; ++qb) {
      h[o_sptr + qb] = ns;
      for (int32_t ti = h[o_qptr + qb]; ti < h[o_qptr + qb + 1]; ++ti)
        for (int ks = 0; ks < 4; ++ks) {
          const int32_t c4 = column_classes(h[o_qcls + ti], ks);
          if (c4) h[o_step + ns++] = (((h[o_qtile + ti] >> 1) * 4 + ks) << 8) | c4;
        }
    }
    h[o_sptr + nb] = ns;
    // 32-query units: their non-empty 32x32 blocks, diagonal tile first
    int32_t nu = 0;
    for (int64_t u = 0; u < Np / 32; ++u) {
      h[o_uptr + u] = nu;
      const int64_t qb = u / 4;
      const int qs = static_cast<int>(u % 4);
      for (int32_t ti = h[o_qptr + qb]; ti < h[o_qptr + qb + 1]; ++ti)
        for (int ks = 0; ks < 4; ++ks) {
          const int32_t cls = (h[o_qcls + ti] >> (2 * (4 * qs + ks))) & 3;
          if (cls) h[o_ustep + nu++] = (((h[o_qtile + ti] >> 1) * 4 + ks) << 2) | cls;
        }
    }
    h[o_uptr + Np / 32] = nu;
  }
  for (int64_t b = 0; b < Np / 32; ++b) {
    const int32_t* se = h + o_se + 32 * b;
    h[o_blk + 2 * b] = *std::min_element(se, se + 32);
    h[o_blk + 2 * b + 1] = *std::max_element(se, se + 32);
  }
  // Work orders over every block of every tree.  Query blocks (forward and
  // dQ): grouped by their first key block, so that the blocks resident on an
  // XCD at one time share their prompt's K/V in L2, heaviest first within a
  // group (longest processing time); measured 3-4 % faster than one global
  // heaviest-first order.  Key blocks (dK/dV): grouped by the last query
  // block that sees them (the end of their subtree), the group with the
  // longest range first, first key block first within a group.  The dK/dV
  // pass walks each range downwards from that end, so the workgroups of a
  // group that are resident on an XCD read the same query rows at about the
  // same time and share them in L2 (in a heaviest-first order they belong
  // to unrelated subtrees, and nearly every Q / dO tile came from HBM).
  {
    std::vector<int32_t> ord(nb);
    std::iota(ord.begin(), ord.end(), 0);
    const int32_t* qp = h + o_qptr;
    const int32_t* qt = h + o_qtile;
    auto minkb = [&](int32_t a) { return qt[qp[a + 1] - 1] >> 1; };
    std::stable_sort(ord.begin(), ord.end(), [&](int32_t a, int32_t b) {
      if (minkb(a) != minkb(b)) return minkb(a) < minkb(b);
      return qp[a + 1] - qp[a] > qp[b + 1] - qp[b];
    });
    std::copy(ord.begin(), ord.end(), h + o_ford);
    std::iota(ord.begin(), ord.end(), 0);
    const int32_t* qhi = h + o_qhi;
    std::vector<int32_t> span(nb, 0);  // per range end: the longest range ending there
    for (int32_t b = 0; b < nb; ++b) span[qhi[b]] = std::max(span[qhi[b]], qhi[b] - b + 1);
    std::stable_sort(ord.begin(), ord.end(), [&](int32_t a, int32_t b) {
      if (span[qhi[a]] != span[qhi[b]]) return span[qhi[a]] > span[qhi[b]];
      if (qhi[a] != qhi[b]) return qhi[a] < qhi[b];
      return a < b;
    });
    std::copy(ord.begin(), ord.end(), h + o_bord);
    // Persistent dK/dV workgroups: for every lane count P = 2^i (i < 9),
    // the key blocks of the order above dealt out by greedy list scheduling
    // (each to the lane with the least work so far, work ~ the blocks of
    // its query range), stored as P + 1 lane offsets and nb block ids,
    // lanes in turn.  No lane waits for the hardware to dispatch its next
    // workgroup (one workgroup fills a CU's LDS, so nothing covered that
    // wait), and lanes that run side by side stay at neighbouring key blocks
    // of the order, sharing their query rows in L2.  (Dealing longest first
    // instead balanced the lanes better but lost that sharing: 4-6 % slower.)
    {
      int32_t* lv = h + o_lanes;
      std::vector<int32_t> lane_of(nb), fill;
      for (int i = 0; i < pst::kLaneLevels; ++i) {
        const int P = 1 << i;
        int32_t* lptr = lv;
        int32_t* items = lv + P + 1;
        std::priority_queue<std::pair<int64_t, int32_t>, std::vector<std::pair<int64_t, int32_t>>,
                            std::greater<>> heap;
        for (int32_t l = 0; l < P; ++l) heap.emplace(0, l);
        for (int64_t r = 0; r < nb; ++r) {
          const int32_t b = ord[r];
          auto [w, l] = heap.top();
          heap.pop();
          lane_of[r] = l;
          heap.emplace(w + 4 * (int64_t{qhi[b]} - b + 1) + 1, l);
        }
        std::fill(lptr, lptr + P + 1, 0);
        for (int64_t r = 0; r < nb; ++r) lptr[lane_of[r] + 1]++;
        for (int l = 0; l < P; ++l) lptr[l + 1] += lptr[l];
        fill.assign(lptr, lptr + P);
        for (int64_t r = 0; r < nb; ++r) items[fill[lane_of[r]]++] = ord[r];
        lv += P + 1 + nb;
      }
    }
    // 32-query units: the same grouping by first key block, most blocks first
    std::vector<int32_t> uord(Np / 32);
    std::iota(uord.begin(), uord.end(), 0);
    const int32_t* up = h + o_uptr;
    const int32_t* us = h + o_ustep;
    auto ufirst = [&](int32_t a) {  // smallest 32-key block of the unit
      int32_t m = INT32_MAX;
      for (int32_t i = up[a]; i < up[a + 1]; ++i) m = std::min(m, us[i] >> 2);
      return m;
    };
    std::vector<int32_t> first(uord.size());
    for (size_t a = 0; a < uord.size(); ++a) first[a] = ufirst(static_cast<int32_t>(a));
    std::stable_sort(uord.begin(), uord.end(), [&](int32_t a, int32_t b) {
      if (first[a] / 4 != first[b] / 4) return first[a] / 4 < first[b] / 4;
      return up[a + 1] - up[a] > up[b + 1] - up[b];
    });
    std::copy(uord.begin(), uord.end(), h + o_uord);
  }
  hipError_t e = hipMemcpyAsync(m->dbuf, h, words * sizeof(int32_t), hipMemcpyHostToDevice,
                                static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync");
  e = hipEventRecord(m->uploaded[buf], static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  m->pending[buf] = true;
  m->next = buf ^ 1;
  m->valid = true;
  m->n_words = words;
  m->sizes = sz;
  int32_t* d = m->dbuf;
  m->dev = pst::TreeDev{d + o_se,   d + o_qptr, d + o_qtile, d + o_qhi,  d + o_ford,
                        d + o_bord, d + o_rptr, d + o_opos,  d + o_otgt, d + o_blk, d + o_qcls,
                        d + o_pos,  d + o_sptr, d + o_step, d + o_uptr, d + o_ustep,
                        d + o_uord, d + o_lanes, sz.n_tokens, sz.n_padded, sz.n_blocks, sz.n_tiles};
  return PST_OK;
}

// Frees everything `m` holds (the caller has synchronized its uploads).
int release_meta(pst_tree_meta* m) {
  hipError_t first = hipSuccess;
  auto keep = [&](hipError_t e) {
    if (first == hipSuccess) first = e;
  };
  if (m->dbuf) keep(hipFree(m->dbuf));
  for (int i = 0; i < 2; ++i) {
    if (m->hbuf[i]) keep(hipHostFree(m->hbuf[i]));
    if (m->uploaded[i]) keep(hipEventDestroy(m->uploaded[i]));
  }
  delete m;
  if (first != hipSuccess) return hip_fail(first, "releasing tree metadata");
  return PST_OK;
}

// A new metadata object on the current device holding the upload of `trees`.
int create_meta(const std::vector<const pst::Tree*>& trees, void* stream, pst_tree_meta** out) {
  pst_tree_meta* m = new (std::nothrow) pst_tree_meta;
  if (!m) return fail(PST_ENOMEM, "out of host memory");
  hipError_t e = hipGetDevice(&m->device);
  for (int i = 0; i < 2 && e == hipSuccess; ++i)
    e = hipEventCreateWithFlags(&m->uploaded[i], hipEventDisableTiming);
  if (e != hipSuccess) {
    const int r = hip_fail(e, "creating tree metadata");
    (void)release_meta(m);
    return r;
  }
  if (int r = upload_meta(trees, stream, m)) {
    const std::string msg = pst_last_error();
    (void)release_meta(m);
    return fail(r, msg);
  }
  *out = m;
  return ok();
}

}  // namespace

extern "C" {

int pst_tree_meta_create(const pst_forest* forest, int32_t tree, void* stream,
                         pst_tree_meta** out) {
  if (!out) return fail(PST_EINVAL, "out is NULL");
  *out = nullptr;
  if (int e = check_tree(forest, tree)) return e;
  return create_meta({&forest->f.trees[tree]}, stream, out);
}

int pst_forest_meta_create(const pst_forest* forest, void* stream, pst_tree_meta** out) {
  if (!out) return fail(PST_EINVAL, "out is NULL");
  *out = nullptr;
  if (!forest) return fail(PST_EINVAL, "forest is NULL");
  std::vector<const pst::Tree*> trees;
  for (const pst::Tree& t : forest->f.trees) trees.push_back(&t);
  return create_meta(trees, stream, out);
}

int pst_tree_meta_sizes(const pst_tree_meta* meta, pst_tree_sizes* out) {
  if (!meta || !out) return fail(PST_EINVAL, "NULL argument");
  *out = meta->sizes;
  return ok();
}

int pst_forest_meta_update(const pst_forest* forest, void* stream, pst_tree_meta* meta) {
  if (!forest || !meta) return fail(PST_EINVAL, "NULL argument");
  if (int e = check_meta_device(meta, false)) return e;
  std::vector<const pst::Tree*> trees;
  for (const pst::Tree& t : forest->f.trees) trees.push_back(&t);
  if (int e = upload_meta(trees, stream, meta)) return e;
  return ok();
}

int pst_tree_meta_destroy(pst_tree_meta* meta) {
  if (!meta) return ok();
  if (int e = release_meta(meta)) return e;
  return ok();
}

int pst_tree_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      const pst_tree_meta* meta, int32_t hq, int32_t hkv, int32_t head_dim,
                      int32_t dtype, float softmax_scale, void* stream) {
  if (int e = check_attn_args(meta, hq, hkv, head_dim, dtype)) return e;
  if (int e = check_ptrs({q, k, v, o, lse}, "q, k, v, o, lse")) return e;
  if (int e = check_meta_device(meta)) return e;
  const hipError_t e = pst::launch_attn_fwd(dtype, head_dim, q, k, v, o, lse, meta->dev, hq, hkv,
                                            resolve_scale(softmax_scale, head_dim),
                                            static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tree_attn_fwd launch");
  return ok();
}

static size_t bwd_workspace_bytes(const pst_tree_meta* meta, int hq, int hkv, int head_dim,
                                  int dtype) {
  const int Np = meta->sizes.n_padded;
  if (dtype == PST_BF16 && head_dim == 128) return pst::attn_bwd_bf16_d128_workspace(Np, hq, hkv);
  return static_cast<size_t>(Np) * hq * sizeof(float);
}

int pst_tree_attn_bwd_workspace_bytes(const pst_tree_meta* meta, int32_t hq, int32_t hkv,
                                      int32_t head_dim, int32_t dtype, size_t* bytes) {
  if (!bytes) return fail(PST_EINVAL, "NULL argument");
  if (int e = check_attn_args(meta, hq, hkv, head_dim, dtype)) return e;
  *bytes = bwd_workspace_bytes(meta, hq, hkv, head_dim, dtype);
  return ok();
}

int pst_tree_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, const pst_tree_meta* meta,
                      int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype,
                      float softmax_scale, void* stream) {
  if (int e = check_attn_args(meta, hq, hkv, head_dim, dtype)) return e;
  if (int e = check_ptrs({q, k, v, o, lse, dout, dq, dk, dv, workspace},
                         "q, k, v, o, lse, dout, dq, dk, dv, workspace"))
    return e;
  const size_t need = bwd_workspace_bytes(meta, hq, hkv, head_dim, dtype);
  if (workspace_bytes < need)
    return fail(PST_EINVAL, "workspace of " + std::to_string(workspace_bytes) + " bytes < " +
                                std::to_string(need) + " needed");
  if (int e = check_meta_device(meta)) return e;
  const hipError_t e = pst::launch_attn_bwd(
      dtype, head_dim, q, k, v, o, lse, dout, dq, dk, dv, workspace,
      meta->dev, hq, hkv, resolve_scale(softmax_scale, head_dim), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tree_attn_bwd launch");
  return ok();
}

int pst_tree_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              const pst_tree_meta* meta, int32_t hq, int32_t hkv,
                              int32_t head_dim, int32_t dtype, float softmax_scale,
                              void* stream) {
  if (int e = check_attn_args(meta, hq, hkv, head_dim, dtype)) return e;
  if (int e = check_ptrs({q, k, v, o, lse, dout, dq, dk, dv}, "q, k, v, o, lse, dout, dq, dk, dv"))
    return e;
  const size_t need = bwd_workspace_bytes(meta, hq, hkv, head_dim, dtype);
  if (need > kNoAllocScratchBytes)
    return fail(PST_ESHAPE, "these shapes need " + std::to_string(need) +
                                " bytes of backward scratch, above the " +
                                std::to_string(kNoAllocScratchBytes) +
                                "-byte limit of pst_tree_attn_bwd_noalloc (use pst_tree_attn_bwd "
                                "with a workspace)");
  if (int e = check_meta_device(meta)) return e;
  void* ws = nullptr;
  if (int e = scratch_on_current_device(&ws)) return e;
  const hipError_t e = pst::launch_attn_bwd(
      dtype, head_dim, q, k, v, o, lse, dout, dq, dk, dv, ws, meta->dev, hq, hkv,
      resolve_scale(softmax_scale, head_dim), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "tree_attn_bwd_noalloc launch");
  return ok();
}

int pst_gather_tree_logprobs_entropy(const void* logits, int64_t vocab, int32_t dtype,
                                     const pst_tree_meta* meta, float* logprobs,
                                     float* entropy, float* row_stats, void* stream) {
  if (!meta) return fail(PST_EINVAL, "tree metadata is NULL");
  if (dtype != PST_F32 && dtype != PST_BF16)
    return fail(PST_EDTYPE, "unknown dtype " + std::to_string(dtype));
  if (vocab <= 0) return fail(PST_EINVAL, "vocab must be positive");
  if (meta->max_target >= vocab || meta->min_target < 0)
    return fail(PST_EINVAL, "next-token ids span [" + std::to_string(meta->min_target) + ", " +
                                std::to_string(meta->max_target) + "], outside the vocab of " +
                                std::to_string(vocab));
  if (!logits || !logprobs || !entropy) return fail(PST_EINVAL, "NULL device pointer");
  const size_t esz = dtype == PST_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(logits) % esz)
    return fail(PST_ESHAPE, "logits pointer is not aligned to its element size");
  if (reinterpret_cast<uintptr_t>(row_stats) % 8)
    return fail(PST_ESHAPE, "row_stats pointer is not 8-byte aligned");
  if (int e = check_meta_device(meta)) return e;
  const hipError_t e = pst::launch_gather(dtype, logits, vocab, meta->dev, logprobs, entropy,
                                          row_stats, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return ok();
}

int pst_gather_tree_logprobs_entropy_bwd(const void* logits, int64_t vocab, int32_t dtype,
                                         const pst_tree_meta* meta, const float* dlogprobs,
                                         const float* dentropy, const float* row_stats,
                                         void* dlogits, void* stream) {
  if (!meta) return fail(PST_EINVAL, "tree metadata is NULL");
  if (dtype != PST_F32 && dtype != PST_BF16)
    return fail(PST_EDTYPE, "unknown dtype " + std::to_string(dtype));
  if (vocab <= 0) return fail(PST_EINVAL, "vocab must be positive");
  if (meta->max_target >= vocab || meta->min_target < 0)
    return fail(PST_EINVAL, "next-token ids span [" + std::to_string(meta->min_target) + ", " +
                                std::to_string(meta->max_target) + "], outside the vocab of " +
                                std::to_string(vocab));
  if (!logits || !dlogprobs || !dentropy || !dlogits)
    return fail(PST_EINVAL, "NULL device pointer");
  const size_t esz = dtype == PST_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(logits) % esz || reinterpret_cast<uintptr_t>(dlogits) % esz)
    return fail(PST_ESHAPE, "logits or dlogits pointer is not aligned to its element size");
  if ((reinterpret_cast<uintptr_t>(logits) - reinterpret_cast<uintptr_t>(dlogits)) % 16)
    return fail(PST_ESHAPE, "logits and dlogits must share their alignment modulo 16 bytes");
  if (reinterpret_cast<uintptr_t>(row_stats) % 8)
    return fail(PST_ESHAPE, "row_stats pointer is not 8-byte aligned");
  if (int e = check_meta_device(meta)) return e;
  const hipError_t e = pst::launch_gather_bwd(dtype, logits, vocab, meta->dev, dlogprobs, dentropy,
                                              row_stats, dlogits, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "gather backward launch");
  return ok();
}

int pst_tree_rope(void* x, const pst_tree_meta* meta, int32_t n_heads, int32_t head_dim,
                  int32_t dtype, float theta, int32_t inverse, void* stream) {
  if (!meta) return fail(PST_EINVAL, "tree metadata is NULL");
  if (dtype != PST_F32 && dtype != PST_BF16)
    return fail(PST_EDTYPE, "unknown dtype " + std::to_string(dtype));
  if (n_heads <= 0) return fail(PST_ESHAPE, "n_heads must be positive");
  const int unit = dtype == PST_BF16 ? 16 : 8;  // two 16-byte chunks per dim pair half
  if (head_dim <= 0 || head_dim > 256 || head_dim % unit)
    return fail(PST_ESHAPE, "head_dim must be a multiple of " + std::to_string(unit) +
                                " in (0, 256], got " + std::to_string(head_dim));
  if (int e = check_ptrs({x}, "x")) return e;
  if (int e = check_meta_device(meta)) return e;
  const hipError_t e = pst::launch_rope(dtype, x, meta->dev, n_heads, head_dim,
                                        theta > 0.f ? theta : 10000.f, inverse != 0,
                                        static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rope launch");
  return ok();
}

int pst_tree_dense_mask(const pst_tree_meta* meta, int32_t format, void* out, void* stream) {
  if (!meta) return fail(PST_EINVAL, "tree metadata is NULL");
  if (format != PST_MASK_U8 && format != PST_MASK_ADD_F32 && format != PST_MASK_ADD_BF16)
    return fail(PST_EDTYPE, "unknown mask format " + std::to_string(format));
  if (int e = check_ptrs({out}, "out")) return e;
  if (int e = check_meta_device(meta)) return e;
  static_assert(PST_MASK_U8 == pst::kMaskU8 && PST_MASK_ADD_F32 == pst::kMaskAddF32 &&
                    PST_MASK_ADD_BF16 == pst::kMaskAddBf16,
                "mask format codes");
  const hipError_t e =
      pst::launch_dense_mask(format, meta->dev, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dense mask launch");
  return ok();
}

}  // extern "C"
