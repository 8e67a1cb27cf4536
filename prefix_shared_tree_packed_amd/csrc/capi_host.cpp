// The host-only entry points of libpst's C ABI (include/pst.h): the trie
// builder, the forest accessors, host packing and the error status.  Plain
// C++17 with no HIP dependency, so it is also built for the CPU with the
// address and undefined-behaviour sanitizers.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "capi_internal.h"
#include "host/packing.h"

namespace pst {

namespace {
thread_local std::string g_error;
}  // namespace

int fail(int code, const std::string& msg) {
  g_error = msg;
  return code;
}

int ok() {
  g_error.clear();
  return PST_OK;
}

namespace {
const char* last_error() { return g_error.c_str(); }
}  // namespace

void fill_sizes(const Tree& t, pst_tree_sizes* s) {
  s->n_tokens = t.N;
  s->n_padded = t.Np;
  s->n_blocks = t.nb;
  s->n_nodes = static_cast<int32_t>(t.node_start.size());
  s->n_seqs = static_cast<int32_t>(t.seq_ids.size());
  s->n_edges = static_cast<int32_t>(t.child_idx.size());
  s->n_tiles = t.n_tiles();
  s->n_node_seq = static_cast<int32_t>(t.node_seq_ids.size());
  s->n_out = t.n_out();
  s->n_pairs = t.n_pairs;
}

int check_tree(const pst_forest* forest, int32_t tree) {
  if (!forest) return fail(PST_EINVAL, "forest is NULL");
  if (tree < 0 || tree >= static_cast<int32_t>(forest->f.trees.size()))
    return fail(PST_ERANGE, "tree index " + std::to_string(tree) + " out of range [0, " +
                                std::to_string(forest->f.trees.size()) + ")");
  return PST_OK;
}

namespace {

template <typename A, typename B>
void copy_out(B* dst, const std::vector<A>& src) {
  if (dst && !src.empty()) std::memcpy(dst, src.data(), src.size() * sizeof(A));
}

}  // namespace

}  // namespace pst

using pst::check_tree;
using pst::copy_out;
using pst::fail;
using pst::fill_sizes;
using pst::ok;

extern "C" {

int pst_pack_allocate(const int64_t* values, int32_t n, int64_t capacity, int32_t min_groups,
                      int32_t divisor, int32_t algorithm, int32_t* group_of, int32_t* n_groups,
                      int32_t* fell_back) {
  if (!values || !group_of || !n_groups) return fail(PST_EINVAL, "NULL argument");
  if (algorithm != PST_PACK_FFD && algorithm != PST_PACK_KK)
    return fail(PST_EINVAL, "unknown packing algorithm " + std::to_string(algorithm) +
                                "; valid: PST_PACK_FFD (0), PST_PACK_KK (1)");
  if (n < 1) return fail(PST_EINVAL, "no items");
  if (capacity <= 0) return fail(PST_EINVAL, "capacity must be positive");
  if (min_groups < 1 || divisor < 1) return fail(PST_EINVAL, "min_groups and divisor must be >= 1");
  pst::PackResult r;
  pst::PackStatus st;
  try {
    st = algorithm == PST_PACK_KK ? pst::pack_kk(values, n, capacity, min_groups, divisor, &r)
                                  : pst::pack_ffd(values, n, capacity, min_groups, divisor, &r);
  } catch (const std::bad_alloc&) {
    return fail(PST_ENOMEM, "out of host memory while packing");
  }
  if (st == pst::kPackCapacity) return fail(PST_ECAPACITY, "an item exceeds the capacity");
  if (st != pst::kPackOk) return fail(PST_EINVAL, "negative item or item total beyond int64");
  std::copy(r.group_of.begin(), r.group_of.end(), group_of);
  *n_groups = r.n_groups;
  if (fell_back) *fell_back = r.fell_back ? 1 : 0;
  return ok();
}

int pst_pack_metrics_compute(const int64_t* values, int32_t n, const int32_t* group_of,
                             int32_t n_groups, int64_t capacity, pst_pack_metrics* out) {
  if (!values || !group_of || !out) return fail(PST_EINVAL, "NULL argument");
  if (n < 1 || n_groups < 1 || capacity <= 0)
    return fail(PST_EINVAL, "need n >= 1, n_groups >= 1, capacity > 0");
  std::vector<int64_t> sums(n_groups, 0);
  for (int32_t i = 0; i < n; ++i) {
    if (group_of[i] < 0 || group_of[i] >= n_groups)
      return fail(PST_ERANGE, "group index out of range at item " + std::to_string(i));
    sums[group_of[i]] += values[i];
  }
  int64_t total = 0;
  for (int64_t v : sums) total += v;
  const int64_t mx = *std::max_element(sums.begin(), sums.end());
  const int64_t mn = *std::min_element(sums.begin(), sums.end());
  const double mean = static_cast<double>(total) / n_groups;
  double var = 0;
  for (int64_t v : sums) var += (v - mean) * (v - mean);
  var /= n_groups;
  out->n_groups = n_groups;
  out->total = total;
  out->max_load = mx;
  out->min_load = mn;
  out->spread = mx - mn;
  out->std_dev = std::sqrt(var);
  out->imbalance_ratio = mean > 0 ? mx / mean : 1.0;
  out->cv = mean > 0 ? out->std_dev / mean : 0.0;
  out->utilization = static_cast<double>(total) / (static_cast<double>(n_groups) * capacity);
  out->wasted_tokens = static_cast<int64_t>(n_groups) * capacity - total;
  return ok();
}

const char* pst_last_error(void) { return pst::last_error(); }

// the build script passes the digest of the sources it compiles
#ifndef PST_SOURCES_SHA256
#define PST_SOURCES_SHA256 "unknown"
#endif
const char* pst_build_sources_sha256(void) { return PST_SOURCES_SHA256; }

int pst_build_tree_ex(const int32_t* tokens, const int64_t* seq_offsets, int32_t n_seqs,
                      int32_t max_tokens_per_mb, int32_t flags, pst_forest** out) {
  if (!out) return fail(PST_EINVAL, "out is NULL");
  *out = nullptr;
  if (flags & ~PST_BUILD_PAD_TO_MAXIMUM)
    return fail(PST_EINVAL, "unknown build flags " + std::to_string(flags));
  if (!seq_offsets) return fail(PST_EINVAL, "seq_offsets is NULL");
  if (n_seqs >= 1 && !tokens) return fail(PST_EINVAL, "tokens is NULL");
  pst_forest* f = new (std::nothrow) pst_forest;
  if (!f) return fail(PST_ENOMEM, "out of host memory");
  std::string err;
  int st;
  try {
    st = pst::build_forest(tokens, seq_offsets, n_seqs, max_tokens_per_mb,
                           (flags & PST_BUILD_PAD_TO_MAXIMUM) != 0, f->f, err);
  } catch (const std::bad_alloc&) {
    delete f;
    return fail(PST_ENOMEM, "out of host memory while packing");
  }
  if (st != pst::kBuildOk) {
    delete f;
    const int code = st == pst::kBuildCapacity ? PST_ECAPACITY
                     : st == pst::kBuildBlock  ? PST_EBLOCK
                                               : PST_EINVAL;
    return fail(code, err);
  }
  *out = f;
  return ok();
}

int pst_build_tree(const int32_t* tokens, const int64_t* seq_offsets, int32_t n_seqs,
                   int32_t max_tokens_per_mb, pst_forest** out) {
  return pst_build_tree_ex(tokens, seq_offsets, n_seqs, max_tokens_per_mb, 0, out);
}

int pst_forest_num_trees(const pst_forest* forest, int32_t* n_trees) {
  if (!forest || !n_trees) return fail(PST_EINVAL, "NULL argument");
  *n_trees = static_cast<int32_t>(forest->f.trees.size());
  return ok();
}

int pst_forest_tree_sizes(const pst_forest* forest, int32_t tree, pst_tree_sizes* out) {
  if (int e = check_tree(forest, tree)) return e;
  if (!out) return fail(PST_EINVAL, "out is NULL");
  fill_sizes(forest->f.trees[tree], out);
  return ok();
}

int pst_forest_export_tree(const pst_forest* forest, int32_t tree, const pst_tree_arrays* a) {
  if (int e = check_tree(forest, tree)) return e;
  if (!a) return fail(PST_EINVAL, "arrays is NULL");
  const pst::Tree& t = forest->f.trees[tree];
  copy_out(a->token, t.token);
  copy_out(a->pos, t.pos);
  copy_out(a->parent, t.parent);
  copy_out(a->subtree_end, t.se);
  copy_out(a->node, t.node);
  copy_out(a->node_start, t.node_start);
  copy_out(a->node_end, t.node_end);
  copy_out(a->node_parent, t.node_parent);
  copy_out(a->node_seq_ptr, t.node_seq_ptr);
  copy_out(a->node_seq_ids, t.node_seq_ids);
  copy_out(a->seq_ids, t.seq_ids);
  copy_out(a->seq_out_offsets, t.seq_out_offsets);
  copy_out(a->seq_index, t.seq_index);
  copy_out(a->child_ptr, t.child_ptr);
  copy_out(a->child_idx, t.child_idx);
  copy_out(a->q_ptr, t.q_ptr);
  copy_out(a->q_kb, t.q_kb);
  copy_out(a->q_full, t.q_full);
  copy_out(a->q_cls, t.q_cls);
  copy_out(a->kb_qhi, t.kb_qhi);
  copy_out(a->fwd_order, t.fwd_order);
  copy_out(a->bwd_order, t.bwd_order);
  return ok();
}

int pst_forest_seq_tree(const pst_forest* forest, int32_t* tree_of_seq) {
  if (!forest || !tree_of_seq) return fail(PST_EINVAL, "NULL argument");
  copy_out(tree_of_seq, forest->f.seq_tree);
  return ok();
}

int pst_forest_stats(const pst_forest* forest, pst_stats* out) {
  if (!forest || !out) return fail(PST_EINVAL, "NULL argument");
  const pst::Forest& f = forest->f;
  pst_stats s{};
  s.n_trees = static_cast<int32_t>(f.trees.size());
  s.n_seqs = f.n_seqs;
  s.orig_tokens = f.orig_tokens;
  s.causal_pairs = f.causal_pairs;
  for (const pst::Tree& t : f.trees) {
    s.tree_tokens += t.N;
    s.padded_tokens += t.Np;
    s.n_pairs += t.n_pairs;
    s.n_tiles += t.n_tiles();
  }
  s.tree_token_ratio = static_cast<double>(s.tree_tokens) / static_cast<double>(s.orig_tokens);
  *out = s;
  return ok();
}

void pst_forest_free(pst_forest* forest) { delete forest; }

}  // extern "C"
