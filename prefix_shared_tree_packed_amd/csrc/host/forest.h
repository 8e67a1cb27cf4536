// Host-side packing of sequences into compressed tries and the per-tree
// metadata the GPU kernels read.  Plain C++17, no HIP.
//
// The construction follows the AReaL tree-training page, section "树构建过程":
// sequences are inserted into tries first-fit-decreasing, linear chains are
// merged into single nodes (TrieNode, section "数据结构"), the trie is
// flattened in preorder and padded to the 128-token block, and the block
// structure of the ancestor mask is derived for the attention kernels.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace pst {

constexpr int32_t kBlock = 128;

struct Tree {
  int32_t id = 0;
  int32_t N = 0;    // real tree tokens
  int32_t Np = 0;   // N rounded up to a multiple of kBlock (or the capacity)
  int32_t nb = 0;   // Np / kBlock

  // per flat token [Np]
  std::vector<int32_t> token, pos, parent, se, node;
  // compressed nodes in preorder [n_nodes]
  std::vector<int32_t> node_start, node_end, node_parent;
  std::vector<int32_t> node_seq_ptr, node_seq_ids;
  // sequences of this tree, ascending input index
  std::vector<int32_t> seq_ids;
  std::vector<int64_t> seq_out_offsets;  // [n_seqs+1]
  std::vector<int32_t> seq_index;        // [n_out] flat index of each token
  // child-target CSR over real tokens
  std::vector<int32_t> child_ptr, child_idx;
  // 128x128 tile structure
  std::vector<int32_t> q_ptr, q_kb, q_full, kb_qhi, fwd_order, bwd_order;
  // per tile: class of each 32x32 sub-block (query sub-block qs, key sub-block
  // ks) in bits 2*(4*qs+ks) .. +1: 0 no visible pair, 1 some, 2 all
  std::vector<int32_t> q_cls;
  // gather map: for each real row, the outputs that read it
  std::vector<int32_t> row_out_ptr;  // [N+1]
  std::vector<int32_t> out_pos;      // [n_out] output slot
  std::vector<int32_t> out_tgt;      // [n_out] next token id, -1 for a sequence's last token
  int32_t min_target = 0, max_target = -1;

  int64_t n_pairs = 0;      // visible (query, key) pairs among real tokens
  int64_t orig_tokens = 0;  // sum of the lengths of the tree's sequences

  int64_t n_out() const { return static_cast<int64_t>(seq_index.size()); }
  int32_t n_tiles() const { return static_cast<int32_t>(q_kb.size()); }
};

struct Forest {
  std::vector<Tree> trees;
  int32_t n_seqs = 0;
  int32_t capacity = 0;
  std::vector<int32_t> seq_tree;  // tree of every input sequence
  int64_t orig_tokens = 0;
  int64_t causal_pairs = 0;
};

enum BuildStatus { kBuildOk = 0, kBuildInvalid = -1, kBuildCapacity = -2, kBuildBlock = -3 };

// Packs the sequences tokens[offsets[s] .. offsets[s+1]) into `out`.  Trees
// are padded to the next multiple of kBlock, or to `capacity` itself with
// pad_to_maximum.  Returns a BuildStatus; on failure `err` says why.
int build_forest(const int32_t* tokens, const int64_t* offsets, int32_t n_seqs,
                 int32_t capacity, bool pad_to_maximum, Forest& out, std::string& err);

}  // namespace pst
