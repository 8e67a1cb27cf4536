// First-fit-decreasing trie packing, chain compression, preorder flattening,
// padding and the tile encoder (AReaL tree-training page, section "树构建过程").
#include "forest.h"

#include <algorithm>
#include <atomic>
#include <exception>
#include <numeric>
#include <system_error>
#include <thread>
#include <unordered_map>

namespace pst {
namespace {

// Above this many children a trie node's children are also indexed in a hash
// map; below it a linear scan of the sibling list is cheaper.
constexpr int32_t kWideNode = 16;

struct TrieNode {
  int32_t token;
  int32_t parent;
  int32_t first_child = -1;
  int32_t last_child = -1;
  int32_t next_sibling = -1;
  int32_t n_children = 0;
  int32_t n_ending = 0;  // sequences whose last token is this one
};

struct Trie {
  std::vector<TrieNode> nodes;                  // nodes[0] is the virtual root
  std::unordered_map<uint64_t, int32_t> wide;   // (parent, token) of wide nodes
  int64_t count = 0;                            // real tokens
  std::vector<int32_t> members;                 // sequence ids, insertion order

  Trie() { nodes.push_back(TrieNode{-1, -1}); }

  static uint64_t key(int32_t p, int32_t t) {
    return (static_cast<uint64_t>(static_cast<uint32_t>(p)) << 32) | static_cast<uint32_t>(t);
  }

  int32_t child(int32_t p, int32_t t) const {
    const TrieNode& n = nodes[p];
    if (n.n_children > kWideNode) {
      auto it = wide.find(key(p, t));
      return it == wide.end() ? -1 : it->second;
    }
    for (int32_t c = n.first_child; c != -1; c = nodes[c].next_sibling)
      if (nodes[c].token == t) return c;
    return -1;
  }

  int32_t add_child(int32_t p, int32_t t) {
    const int32_t c = static_cast<int32_t>(nodes.size());
    nodes.push_back(TrieNode{t, p});
    TrieNode& n = nodes[p];
    if (n.last_child == -1) n.first_child = c; else nodes[n.last_child].next_sibling = c;
    n.last_child = c;
    n.n_children++;
    if (n.n_children == kWideNode + 1) {
      for (int32_t x = n.first_child; x != -1; x = nodes[x].next_sibling)
        wide.emplace(key(p, nodes[x].token), x);
    } else if (n.n_children > kWideNode + 1) {
      wide.emplace(key(p, t), c);
    }
    return c;
  }

  // Length of the longest prefix of s already in the trie; *end is the node
  // of its last token (the root for an empty prefix).
  int64_t shared_prefix(const int32_t* s, int64_t len, int32_t* end) const {
    int32_t cur = 0;
    int64_t n = 0;
    for (; n < len; ++n) {
      const int32_t c = child(cur, s[n]);
      if (c < 0) break;
      cur = c;
    }
    *end = cur;
    return n;
  }

  // Inserts the sequence, whose first `shared` tokens are already in the
  // trie ending at node `at`, and records the trie node of each token.
  void insert(const int32_t* s, int64_t len, int64_t shared, int32_t at, int32_t* path) {
    for (int32_t i = static_cast<int32_t>(shared) - 1, c = at; i >= 0; --i) {
      path[i] = c;
      c = nodes[c].parent;
    }
    int32_t cur = at;
    for (int64_t i = shared; i < len; ++i) {
      cur = add_child(cur, s[i]);
      path[i] = cur;
    }
    nodes[cur].n_ending++;
  }
};

void flatten(const Trie& trie, int32_t tid, const int32_t* tokens, const int64_t* offsets,
             const std::vector<int32_t>& path, int32_t pad_to, Tree& t) {
  const int32_t N = static_cast<int32_t>(trie.count);
  const int32_t Np = pad_to > 0 ? pad_to : (N + kBlock - 1) / kBlock * kBlock;
  const int32_t nb = Np / kBlock;
  t.id = tid;
  t.N = N;
  t.Np = Np;
  t.nb = nb;

  // preorder, children in first-insertion order
  std::vector<int32_t> flat(trie.nodes.size(), -1);
  std::vector<int32_t> order;  // trie node of each flat index
  order.reserve(N);
  {
    std::vector<int32_t> stack;
    std::vector<int32_t> kids;
    auto push_children = [&](int32_t p) {
      kids.clear();
      for (int32_t c = trie.nodes[p].first_child; c != -1; c = trie.nodes[c].next_sibling)
        kids.push_back(c);
      for (auto it = kids.rbegin(); it != kids.rend(); ++it) stack.push_back(*it);
    };
    push_children(0);
    while (!stack.empty()) {
      const int32_t x = stack.back();
      stack.pop_back();
      flat[x] = static_cast<int32_t>(order.size());
      order.push_back(x);
      push_children(x);
    }
  }

  t.token.assign(Np, 0);
  t.pos.assign(Np, 0);
  t.parent.assign(Np, -1);
  t.node.assign(Np, -1);
  t.se.resize(Np);
  std::iota(t.se.begin(), t.se.end(), 0);
  for (int32_t i = 0; i < N; ++i) {
    const TrieNode& n = trie.nodes[order[i]];
    t.token[i] = n.token;
    if (n.parent != 0) {
      t.parent[i] = flat[n.parent];
      t.pos[i] = t.pos[t.parent[i]] + 1;
    }
  }
  // subtree end: children come after their parent in preorder, so one reverse
  // sweep pushes every subtree's last index up to its root
  for (int32_t i = N - 1; i >= 0; --i)
    if (t.parent[i] >= 0) t.se[t.parent[i]] = std::max(t.se[t.parent[i]], t.se[i]);

  // chain compression: a node starts at a depth-0 token or after a token that
  // has other than one child or on which a sequence ends
  t.node_start.clear();
  t.node_end.clear();
  t.node_parent.clear();
  for (int32_t i = 0; i < N; ++i) {
    const int32_t p = t.parent[i];
    bool starts = p < 0;
    if (!starts) {
      const TrieNode& pn = trie.nodes[order[p]];
      starts = pn.n_children != 1 || pn.n_ending > 0;
    }
    if (starts) {
      t.node.at(i) = static_cast<int32_t>(t.node_start.size());
      t.node_start.push_back(i);
      t.node_end.push_back(i);
      t.node_parent.push_back(p < 0 ? -1 : t.node[p]);
    } else {
      t.node[i] = t.node[p];
      t.node_end[t.node[i]] = i;
    }
  }
  const int32_t n_nodes = static_cast<int32_t>(t.node_start.size());

  // sequences of the tree, ascending input index
  t.seq_ids = trie.members;
  std::sort(t.seq_ids.begin(), t.seq_ids.end());
  t.seq_out_offsets.assign(1, 0);
  t.seq_index.clear();
  t.orig_tokens = 0;
  for (int32_t s : t.seq_ids) {
    const int64_t len = offsets[s + 1] - offsets[s];
    for (int64_t k = 0; k < len; ++k) t.seq_index.push_back(flat[path[offsets[s] + k]]);
    t.seq_out_offsets.push_back(t.seq_out_offsets.back() + len);
    t.orig_tokens += len;
  }

  // TrieNode.sequence_ids: every node on a sequence's path, walking node
  // parents up from the node of its last token; ascending because sequences
  // are visited in ascending order
  {
    std::vector<std::vector<int32_t>> lists(n_nodes);
    for (size_t k = 0; k < t.seq_ids.size(); ++k) {
      const int32_t last = t.seq_index[t.seq_out_offsets[k + 1] - 1];
      for (int32_t nd = t.node[last]; nd != -1; nd = t.node_parent[nd])
        lists[nd].push_back(t.seq_ids[k]);
    }
    t.node_seq_ptr.assign(1, 0);
    t.node_seq_ids.clear();
    for (auto& l : lists) {
      t.node_seq_ids.insert(t.node_seq_ids.end(), l.begin(), l.end());
      t.node_seq_ptr.push_back(static_cast<int32_t>(t.node_seq_ids.size()));
    }
  }

  // child-target CSR: preorder makes insertion order ascending flat order
  t.child_ptr.assign(1, 0);
  t.child_idx.clear();
  for (int32_t i = 0; i < N; ++i) {
    for (int32_t c = trie.nodes[order[i]].first_child; c != -1; c = trie.nodes[c].next_sibling)
      t.child_idx.push_back(flat[c]);
    t.child_ptr.push_back(static_cast<int32_t>(t.child_idx.size()));
  }

  t.n_pairs = 0;
  for (int32_t i = 0; i < N; ++i) t.n_pairs += t.pos[i] + 1;

  // tile encoder.  Key j is visible to queries j..se[j] of its own subtree,
  // so for a key block kb and a later query block qb the tile is non-empty
  // iff max se over kb reaches qb's first row and full iff min se over kb
  // reaches qb's last row; the diagonal tile is never full (a query never
  // sees a later key) and never empty; tiles above the diagonal are empty.
  std::vector<int32_t> kmin(nb), kmax(nb);
  for (int32_t kb = 0; kb < nb; ++kb) {
    const auto b = t.se.begin() + kb * kBlock;
    kmin[kb] = *std::min_element(b, b + kBlock);
    kmax[kb] = *std::max_element(b, b + kBlock);
  }
  t.q_ptr.assign(1, 0);
  t.q_kb.clear();
  t.q_full.clear();
  t.q_cls.clear();
  // 32-key blocks: min and max subtree end.  Query and key sub-blocks share
  // the 32-alignment, so a key sub-block is entirely before, equal to, or
  // entirely after a query sub-block, and its class follows from the range
  // rule exactly as for whole tiles.
  const int32_t nb32 = Np / 32;
  std::vector<int32_t> smin32(nb32), smax32(nb32);
  for (int32_t b = 0; b < nb32; ++b) {
    const auto s0 = t.se.begin() + 32 * b;
    smin32[b] = *std::min_element(s0, s0 + 32);
    smax32[b] = *std::max_element(s0, s0 + 32);
  }
  auto sub_class = [&](int32_t qlo, int32_t kbase) {
    const int32_t qhi = qlo + 31;
    const int32_t b = kbase / 32;
    if (kbase > qhi || smax32[b] < qlo) return 0;
    if (kbase + 31 <= qlo && smin32[b] >= qhi) return 2;
    return 1;
  };
  std::vector<int32_t> per_q(nb, 0), per_k(nb, 0);
  for (int32_t qb = 0; qb < nb; ++qb) {
    const int32_t first = qb * kBlock, last = first + kBlock - 1;
    for (int32_t kb = qb; kb >= 0; --kb) {
      if (kb < qb && kmax[kb] < first) continue;
      t.q_kb.push_back(kb);
      t.q_full.push_back(kb < qb && kmin[kb] >= last ? 1 : 0);
      uint32_t bits = 0;
      for (int32_t qs = 0; qs < 4; ++qs)
        for (int32_t ks = 0; ks < 4; ++ks)
          bits |= static_cast<uint32_t>(sub_class(first + 32 * qs, kb * kBlock + 32 * ks)) << (2 * (4 * qs + ks));
      t.q_cls.push_back(static_cast<int32_t>(bits));
      per_q[qb]++;
      per_k[kb]++;
    }
    t.q_ptr.push_back(static_cast<int32_t>(t.q_kb.size()));
  }
  t.kb_qhi.resize(nb);
  for (int32_t kb = 0; kb < nb; ++kb) t.kb_qhi[kb] = kmax[kb] / kBlock;
  auto lpt = [&](const std::vector<int32_t>& cnt) {
    std::vector<int32_t> o(nb);
    std::iota(o.begin(), o.end(), 0);
    std::stable_sort(o.begin(), o.end(), [&](int32_t a, int32_t b) { return cnt[a] > cnt[b]; });
    return o;
  };
  t.fwd_order = lpt(per_q);
  t.bwd_order = lpt(per_k);

  // gather map: outputs grouped by the packed row they read, ascending slot
  const int64_t n_out = t.n_out();
  t.row_out_ptr.assign(N + 1, 0);
  for (int64_t o = 0; o < n_out; ++o) t.row_out_ptr[t.seq_index[o] + 1]++;
  for (int32_t i = 0; i < N; ++i) t.row_out_ptr[i + 1] += t.row_out_ptr[i];
  t.out_pos.assign(n_out, 0);
  t.out_tgt.assign(n_out, -1);
  t.min_target = 0;
  t.max_target = -1;
  bool any_target = false;
  {
    std::vector<int32_t> fill(t.row_out_ptr.begin(), t.row_out_ptr.end() - 1);
    for (size_t k = 0; k < t.seq_ids.size(); ++k) {
      const int32_t s = t.seq_ids[k];
      const int64_t base = t.seq_out_offsets[k];
      const int64_t len = t.seq_out_offsets[k + 1] - base;
      for (int64_t p = 0; p < len; ++p) {
        const int32_t row = t.seq_index[base + p];
        const int32_t slot = fill[row]++;
        t.out_pos[slot] = static_cast<int32_t>(base + p);
        if (p + 1 < len) {
          const int32_t tgt = tokens[offsets[s] + p + 1];
          t.out_tgt[slot] = tgt;
          if (!any_target || tgt < t.min_target) t.min_target = tgt;
          if (!any_target || tgt > t.max_target) t.max_target = tgt;
          any_target = true;
        }
      }
    }
  }
}

}  // namespace

int build_forest(const int32_t* tokens, const int64_t* offsets, int32_t n_seqs,
                 int32_t capacity, bool pad_to_maximum, Forest& out, std::string& err) {
  if (capacity <= 0) {
    err = "max_tokens_per_mb must be positive, got " + std::to_string(capacity);
    return kBuildInvalid;
  }
  if (capacity % kBlock) {
    err = "max_tokens_per_mb=" + std::to_string(capacity) + " is not a multiple of 128";
    return kBuildBlock;
  }
  if (n_seqs < 1) {
    err = "no sequences";
    return kBuildInvalid;
  }
  if (offsets[0] < 0) {
    err = "seq_offsets[0] is negative";
    return kBuildInvalid;
  }
  int64_t total = 0;
  for (int32_t s = 0; s < n_seqs; ++s) {
    const int64_t len = offsets[s + 1] - offsets[s];
    if (len <= 0) {
      err = len == 0 ? "sequence " + std::to_string(s) + " is empty"
                     : "seq_offsets decrease at sequence " + std::to_string(s);
      return kBuildInvalid;
    }
    if (len > capacity) {
      err = "sequence " + std::to_string(s) + " has " + std::to_string(len) +
            " tokens > max_tokens_per_mb=" + std::to_string(capacity);
      return kBuildCapacity;
    }
    total += len;
  }
  if (total >= (int64_t{1} << 31)) {
    err = "more than 2^31-1 tokens in total";
    return kBuildInvalid;
  }

  out = Forest{};
  out.n_seqs = n_seqs;
  out.capacity = capacity;
  out.orig_tokens = total;
  out.seq_tree.assign(n_seqs, -1);

  std::vector<int32_t> order(n_seqs);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return offsets[a + 1] - offsets[a] > offsets[b + 1] - offsets[b];
  });

  std::vector<int32_t> path(static_cast<size_t>(offsets[n_seqs]));
  std::vector<Trie> tries;
  // a trie never holds more than min(capacity, all tokens) nodes
  const size_t trie_cap = static_cast<size_t>(std::min<int64_t>(capacity, total)) + 1;
  for (int32_t s : order) {
    const int32_t* seq = tokens + offsets[s];
    const int64_t len = offsets[s + 1] - offsets[s];
    int32_t chosen = -1, at = 0;
    int64_t shared = 0;
    for (size_t t = 0; t < tries.size(); ++t) {
      int32_t end = 0;
      const int64_t sp = tries[t].shared_prefix(seq, len, &end);
      if (tries[t].count + (len - sp) <= capacity) {
        tries[t].count += len - sp;
        chosen = static_cast<int32_t>(t);
        shared = sp;
        at = end;
        break;
      }
    }
    if (chosen < 0) {
      tries.emplace_back();
      tries.back().nodes.reserve(trie_cap);
      chosen = static_cast<int32_t>(tries.size() - 1);
      tries.back().count = len;
    }
    tries[chosen].insert(seq, len, shared, at, path.data() + offsets[s]);
    tries[chosen].members.push_back(s);
    out.seq_tree[s] = chosen;
    out.causal_pairs += len * (len + 1) / 2;
  }

  // Trees are independent from here on: flatten them on a few threads (the
  // calling thread included), taking trees in order from a shared counter.
  out.trees.resize(tries.size());
  const int32_t n_trees = static_cast<int32_t>(tries.size());
  std::atomic<int32_t> next{0};
  std::exception_ptr failed;
  std::atomic<bool> any_failed{false};
  auto work = [&]() {
    for (int32_t t = next++; t < n_trees; t = next++) {
      try {
        flatten(tries[t], t, tokens, offsets, path, pad_to_maximum ? capacity : 0, out.trees[t]);
      } catch (...) {
        if (!any_failed.exchange(true)) failed = std::current_exception();
      }
    }
  };
  // at most 8 threads: callers may run several builds at once
  const int32_t hw = static_cast<int32_t>(std::min(8u, std::max(1u, std::thread::hardware_concurrency())));
  std::vector<std::thread> helpers;
  for (int32_t i = 1; i < std::min(n_trees, hw); ++i) {
    try {
      helpers.emplace_back(work);
    } catch (const std::system_error&) {
      break;  // no more threads: the others (and this one) take the rest
    }
  }
  work();
  for (std::thread& th : helpers) th.join();
  if (failed) std::rethrow_exception(failed);
  return kBuildOk;
}

}  // namespace pst
