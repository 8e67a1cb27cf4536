/*
 * pst.h -- C ABI of libpst, the MI355X (gfx950) hot path of prefix-shared
 * tree training.
 *
 * Sequences that share prefixes (several responses to one prompt, agent
 * trajectories that fork) are packed into compressed tries; every packed
 * token attends only to itself and its ancestors; per-sequence next-token
 * log-probabilities and entropies are read back from the packed logits.
 * The operations follow the AReaL tree-training page ("树训练"):
 *   - build:      section "树构建过程" (steps 1-4) and "数据结构 / TrieNode";
 *   - capacity:   section "必需配置" (max tokens per tree, a multiple of the
 *                 128-token BLOCK_SIZE);
 *   - attention:  section "树构建过程" (attention-mask column: a token attends
 *                 only to its ancestors) and "注意力机制" (128-token blocks);
 *   - gather:     section "对数概率计算";
 *   - accounting: section "指标和监控" (tree_token_ratio).
 *
 * Conventions (all entry points):
 *   - Every call returns PST_OK (0) or a negative status; pst_last_error()
 *     then returns a message for the calling thread.
 *   - Argument checks happen before any HIP call, so a bad argument never
 *     touches the GPU.
 *   - "host" pointers are ordinary CPU memory owned by the caller; "device"
 *     pointers are HBM allocations owned by the caller.  The library owns
 *     only pst_forest (host) and pst_tree_meta (device + pinned host).
 *   - Device work is enqueued on the given stream (a hipStream_t passed as
 *     void*, NULL for the null stream) and returns without waiting.
 *   - Tensors are dense and row-major: Q/O/dO/dQ [Np, Hq, d], K/V/dK/dV
 *     [Np, Hkv, d], LSE [Hq, Np] float32, logits [Np, V].  Device pointers
 *     must be 16-byte aligned.
 *   - There is no CPU fallback: a call that cannot run on the GPU fails.
 */
#ifndef PST_H
#define PST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PST_OK 0
#define PST_EINVAL (-1)     /* bad argument: null pointer, empty input, ... */
#define PST_ECAPACITY (-2)  /* a sequence is longer than max_tokens_per_mb */
#define PST_EBLOCK (-3)     /* max_tokens_per_mb is not a multiple of 128 */
#define PST_EDTYPE (-4)     /* unknown or unsupported dtype */
#define PST_ESHAPE (-5)     /* Hq % Hkv != 0, unsupported head_dim, misaligned */
#define PST_EHIP (-6)       /* a HIP runtime call or kernel launch failed */
#define PST_ENOMEM (-7)     /* host or device allocation failed */
#define PST_ERANGE (-8)     /* tree index out of range */

#define PST_BLOCK 128       /* BLOCK_SIZE: tile edge and padding unit */

typedef enum { PST_F32 = 0, PST_BF16 = 1 } pst_dtype;

typedef struct pst_forest pst_forest;        /* host, library-owned */
typedef struct pst_tree_meta pst_tree_meta;  /* device-resident, one per tree */

/* Sizes of one packed tree (all counts; N real tokens, Np = N rounded up
 * to a multiple of 128). */
typedef struct {
  int32_t n_tokens;    /* N: real tree tokens */
  int32_t n_padded;    /* Np */
  int32_t n_blocks;    /* Np / 128 */
  int32_t n_nodes;     /* compressed trie nodes (the virtual root excluded) */
  int32_t n_seqs;      /* sequences packed into this tree */
  int32_t n_edges;     /* parent->child token edges (child-target CSR entries) */
  int32_t n_tiles;     /* non-empty 128x128 attention tiles */
  int32_t n_node_seq;  /* total length of the per-node sequence-id lists */
  int64_t n_out;       /* sum of the lengths of the tree's sequences */
  int64_t n_pairs;     /* visible (query, key) pairs among real tokens */
} pst_tree_sizes;

/* Caller-owned host buffers for pst_forest_export_tree.  Any member may be
 * NULL to skip it; sizes come from pst_tree_sizes.  Flat indices follow the
 * preorder of the trie with children in first-insertion order. */
typedef struct {
  int32_t* token;           /* [n_padded] token id; 0 on pad rows */
  int32_t* pos;             /* [n_padded] depth = position inside every sequence
                               through the token (position_ids); 0 on pads */
  int32_t* parent;          /* [n_padded] flat index of the parent token; -1 at
                               depth 0 and on pads */
  int32_t* subtree_end;     /* [n_padded] last flat index of the token's subtree;
                               key j is visible to queries j..subtree_end[j] that
                               lie in its subtree (pads: themselves) */
  int32_t* node;            /* [n_padded] compressed node of the token; -1 on pads */
  int32_t* node_start;      /* [n_nodes] first flat index of the node (TrieNode.start_idx) */
  int32_t* node_end;        /* [n_nodes] last flat index, inclusive (end_idx) */
  int32_t* node_parent;     /* [n_nodes] parent node, -1 for children of the root */
  int32_t* node_seq_ptr;    /* [n_nodes+1] CSR into node_seq_ids */
  int32_t* node_seq_ids;    /* [n_node_seq] ascending ids of the sequences through
                               each node (TrieNode.sequence_ids) */
  int32_t* seq_ids;         /* [n_seqs] input indices of the tree's sequences, ascending */
  int64_t* seq_out_offsets; /* [n_seqs+1] offsets of each sequence in the outputs */
  int32_t* seq_index;       /* [n_out] flat index of every token of every sequence */
  int32_t* child_ptr;       /* [n_tokens+1] CSR into child_idx */
  int32_t* child_idx;       /* [n_edges] flat indices of each token's children, ascending */
  int32_t* q_ptr;           /* [n_blocks+1] CSR of non-empty tiles per query block */
  int32_t* q_kb;            /* [n_tiles] key block of each tile, descending per query block */
  int32_t* q_full;          /* [n_tiles] 1 if every pair of the tile is visible */
  int32_t* q_cls;           /* [n_tiles] class of each 32x32 sub-block of the tile,
                               2 bits at bit 2*(4*qs+ks) for query sub-block qs and
                               key sub-block ks: 0 no visible pair, 1 some, 2 all */
  int32_t* kb_qhi;          /* [n_blocks] last query block that sees each key block
                               (the visible query blocks are kb..kb_qhi[kb]) */
  int32_t* fwd_order;       /* [n_blocks] query blocks by descending tile count,
                               ties by index (a load-balancing order; the
                               kernels schedule by orders of their own that
                               pst_tree_meta builds at upload) */
  int32_t* bwd_order;       /* [n_blocks] key blocks by descending tile count,
                               ties by index (likewise) */
} pst_tree_arrays;

typedef struct {
  int32_t n_trees;
  int32_t n_seqs;
  int64_t orig_tokens;      /* sum of the input sequence lengths */
  int64_t tree_tokens;      /* sum over trees of N */
  int64_t padded_tokens;    /* sum over trees of Np */
  int64_t n_pairs;          /* visible pairs over all trees */
  int64_t causal_pairs;     /* pairs of unpacked causal attention: sum L(L+1)/2 */
  int64_t n_tiles;          /* non-empty tiles over all trees */
  double tree_token_ratio;  /* tree_tokens / orig_tokens ("指标和监控") */
} pst_stats;

/* ---- host: packing ------------------------------------------------------ */

/* Pack n_seqs sequences into compressed tries ("树构建过程" steps 1-3).
 *   tokens       host int32 [seq_offsets[n_seqs]]: the real tokens of every
 *                sequence, back to back (step 1 -- extracting them from a
 *                padded batch with its attention_mask -- is the caller's);
 *   seq_offsets  host int64 [n_seqs+1], seq_offsets[0] = 0, non-decreasing;
 *   max_tokens_per_mb  maximum real tokens per tree, a positive multiple of 128.
 * Sequences are taken longest first (ties by input index) and each goes into
 * the first tree, in creation order, whose token count after prefix sharing
 * stays within the capacity, else into a new tree.  Chains are compressed
 * into nodes that also end where a sequence ends; each tree is flattened in
 * preorder and padded to a multiple of 128.
 * Errors: PST_EINVAL (null pointer, n_seqs < 1, bad offsets, empty sequence,
 * max_tokens_per_mb <= 0), PST_EBLOCK, PST_ECAPACITY, PST_ENOMEM.
 * On success *out owns the forest; free it with pst_forest_free. */
int pst_build_tree(const int32_t* tokens, const int64_t* seq_offsets, int32_t n_seqs,
                   int32_t max_tokens_per_mb, pst_forest** out);

/* Build flags of pst_build_tree_ex. */
enum { PST_BUILD_PAD_TO_MAXIMUM = 1 };

/* pst_build_tree with flags.  PST_BUILD_PAD_TO_MAXIMUM pads every tree to
 * max_tokens_per_mb rows instead of the next multiple of 128 (the
 * pad_to_maximum setting of the tree-training page's configuration section:
 * every micro-batch then has the same shape).  The extra rows are pad rows:
 * token 0, position 0, parent -1, seeing only themselves.  Unknown flag bits:
 * PST_EINVAL.  Other arguments and errors as pst_build_tree. */
int pst_build_tree_ex(const int32_t* tokens, const int64_t* seq_offsets, int32_t n_seqs,
                      int32_t max_tokens_per_mb, int32_t flags, pst_forest** out);

int pst_forest_num_trees(const pst_forest* forest, int32_t* n_trees);
int pst_forest_tree_sizes(const pst_forest* forest, int32_t tree, pst_tree_sizes* out);
/* Copy tree `tree`'s arrays into the caller's host buffers (see pst_tree_arrays). */
int pst_forest_export_tree(const pst_forest* forest, int32_t tree, const pst_tree_arrays* out);
/* tree_of_seq: host int32 [n_seqs], the tree of every input sequence. */
int pst_forest_seq_tree(const pst_forest* forest, int32_t* tree_of_seq);
int pst_forest_stats(const pst_forest* forest, pst_stats* out);
void pst_forest_free(pst_forest* forest);

/* ---- device: per-tree metadata ----------------------------------------- */

/* Upload tree `tree`'s metadata (subtree_end, the tile lists and work orders,
 * the gather's row->output map) to the current HIP device: one device
 * allocation plus one asynchronous host-to-device copy on `stream`.  The role
 * of the block mask built from the trie ("树构建过程" step 4).
 * Errors: PST_EINVAL, PST_ERANGE, PST_ENOMEM, PST_EHIP. */
int pst_tree_meta_create(const pst_forest* forest, int32_t tree, void* stream,
                         pst_tree_meta** out);
/* The metadata of every tree of the forest at once, trees back to back in
 * tree order: the padded rows of tree t follow those of trees 0..t-1, and
 * its outputs (logprobs/entropy) follow theirs.  Attention never crosses
 * trees, so one call of the device entry points below then covers the whole
 * forest, with tensors of sum-over-trees Np rows.  Same errors as
 * pst_tree_meta_create; sizes (pst_tree_meta_sizes) are sums over trees. */
int pst_forest_meta_create(const pst_forest* forest, void* stream, pst_tree_meta** out);
int pst_tree_meta_sizes(const pst_tree_meta* meta, pst_tree_sizes* out);
/* Rebuild `meta` in place for `forest` (every tree, back to back, as
 * pst_forest_meta_create), for a training loop that packs a new batch every
 * step: the device allocation and the pinned staging memory are reused when
 * large enough and grown otherwise, so in steady state the call allocates
 * nothing and never synchronizes the device.  The upload is enqueued on
 * `stream`: work already enqueued on that stream that reads the old
 * metadata runs before the upload overwrites it (stream order); work on
 * other streams that reads it must have completed.  Two pinned staging
 * buffers alternate, so the host waits only for the upload issued two
 * updates earlier.  Growing the device allocation synchronizes the device
 * first.  If the call fails, `meta` is refused by every device entry point
 * until an update succeeds.  Errors: PST_EINVAL (NULL, other device),
 * PST_ENOMEM, PST_EHIP. */
int pst_forest_meta_update(const pst_forest* forest, void* stream, pst_tree_meta* meta);

/* Frees the metadata.  The caller first makes sure no work that reads it is
 * still queued (synchronize the stream it was used on). */
int pst_tree_meta_destroy(pst_tree_meta* meta);

/* ---- device: tree attention --------------------------------------------- */

/* Forward tree attention ("树构建过程": a token attends only to its ancestors,
 * itself included):
 *   O[i,h] = sum_j softmax_j(scale * Q[i,h].K[j,g]) V[j,g]  over j visible to i,
 *   g = h / (hq / hkv);  LSE[h,i] = natural-log log-sum-exp of the scores.
 *   q       device [Np, hq, head_dim]   dtype
 *   k, v    device [Np, hkv, head_dim]  dtype
 *   o       device [Np, hq, head_dim]   dtype (written)
 *   lse     device float32 [hq, Np]     (written)
 * Pad rows attend only to themselves.  Accumulation is float32; with
 * PST_BF16 the probabilities are rounded to bf16 before the P.V product.
 * softmax_scale <= 0 selects 1/sqrt(head_dim).  head_dim must be 64 or 128.
 * Errors: PST_EINVAL, PST_EDTYPE, PST_ESHAPE, PST_EHIP. */
int pst_tree_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      const pst_tree_meta* meta, int32_t hq, int32_t hkv, int32_t head_dim,
                      int32_t dtype, float softmax_scale, void* stream);

/* Bytes of device workspace pst_tree_attn_bwd needs for these shapes: the
 * float32 [hq, Np] per-row sums D = rowsum(dout * O).  The workspace is
 * scratch: its contents on entry do not matter and are overwritten.
 * Errors: PST_EINVAL (NULL), PST_ESHAPE, PST_EDTYPE. */
int pst_tree_attn_bwd_workspace_bytes(const pst_tree_meta* meta, int32_t hq, int32_t hkv,
                                      int32_t head_dim, int32_t dtype, size_t* bytes);

/* Backward tree attention (the tree page's "Megatron 引擎" section: training
 * through packed trees differentiates attention under the same ancestor
 * mask as "树构建过程"): gradients of sum(dout * O) with respect to q, k, v,
 * the softmax-attention vector-Jacobian product restricted to the tree mask.
 * dk/dv sum the contributions of all query heads of their group.  `o` and
 * `lse` are the forward outputs.  dq/dk/dv are written (not accumulated), in
 * `dtype`, from float32 accumulators; no atomics, so results are
 * deterministic.  workspace: device, >= pst_tree_attn_bwd_workspace_bytes.
 * Errors: as pst_tree_attn_fwd. */
int pst_tree_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                      const float* lse, const void* dout, void* dq, void* dk, void* dv,
                      void* workspace, size_t workspace_bytes, const pst_tree_meta* meta,
                      int32_t hq, int32_t hkv, int32_t head_dim, int32_t dtype,
                      float softmax_scale, void* stream);

/* pst_tree_attn_bwd for callers that cannot allocate device memory (code
 * under HIP graph capture, tight training loops, harnesses that forbid
 * hipMalloc): the same kernels and results, with the per-row sums that
 * pst_tree_attn_bwd keeps in the caller's workspace held instead in a
 * library-owned scratch array of 64 MiB per GPU (a static device array,
 * present from the library's first use on a GPU until the process ends).
 * The call allocates nothing; the caller still passes every input and
 * output.  Shapes whose scratch (pst_tree_attn_bwd_workspace_bytes) exceeds
 * 64 MiB -- hq * Np above 16 777 216 -- are refused with PST_ESHAPE before
 * any HIP call.  All calls on one GPU share its scratch: two calls that
 * overlap in time on one GPU (different streams, or host threads) race and
 * give wrong results; serialize them.  The scratch needs no clearing (it is
 * fully written before it is read).  Errors: as pst_tree_attn_bwd, and
 * PST_EHIP if the scratch address cannot be obtained. */
int pst_tree_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              const pst_tree_meta* meta, int32_t hq, int32_t hkv,
                              int32_t head_dim, int32_t dtype, float softmax_scale,
                              void* stream);

/* ---- device: log-probabilities and entropies ------------------------------ */

/* Per-sequence next-token log-probabilities and entropies from the packed
 * logits ("对数概率计算"): for every sequence of the tree (ascending input
 * index) and every position t of it, with row = the packed token holding t,
 *   logprobs[off+t] = log_softmax(logits[row])[s[t+1]]   (0 for the last t)
 *   entropy[off+t]  = -sum_v p_v log p_v,  p = softmax(logits[row])
 * where off = seq_out_offsets of that sequence.  Each real packed row is read
 * once, whatever the number of sequences through it.
 *   logits     device [Np, vocab] dtype (only the N real rows are read)
 *   logprobs   device float32 [n_out] (written)
 *   entropy    device float32 [n_out] (written)
 *   row_stats  device float32 [Np][2], 8-byte aligned, or NULL: when given,
 *              (log-sum-exp, entropy) of every real row is written (pad
 *              rows untouched), for pst_gather_tree_logprobs_entropy_bwd
 * Errors: PST_EINVAL, PST_EDTYPE, PST_ESHAPE, PST_EHIP. */
int pst_gather_tree_logprobs_entropy(const void* logits, int64_t vocab, int32_t dtype,
                                     const pst_tree_meta* meta, float* logprobs,
                                     float* entropy, float* row_stats, void* stream);

/* Gradient of the gather: d logits of
 *   sum_k dlogprobs[k] * logprobs[k] + dentropy[k] * entropy[k]
 * with logprobs/entropy as pst_gather_tree_logprobs_entropy defines them
 * (the loss path the "对数概率计算" section feeds).  For a row x serving
 * outputs k (next token t_k, none at a sequence's last position):
 *   dx_v = -p_v (A + B (log p_v + H)) + sum_{k: t_k = v} dlogprobs[k],
 *   A = sum over outputs with a next token of dlogprobs, B = sum of dentropy,
 * p = softmax(x), H its entropy (a zero probability contributes 0).  Each
 * real row is read once and written once when it fits a workgroup's
 * registers (up to 32768 bf16 / 16384 fp32 entries) or when row_stats is
 * given; otherwise twice (statistics, then gradient).  Rows no output reads
 * (pad rows) are written as zeros.  Deterministic.
 *   logits     device [Np, vocab] dtype
 *   dlogprobs  device float32 [n_out], dentropy device float32 [n_out]
 *   row_stats  NULL, or the row statistics that the forward gather wrote for
 *              these same logits (device float32 [Np][2], 8-byte aligned)
 *   dlogits    device [Np, vocab] dtype (written), same alignment as logits
 *              modulo 16 bytes
 * Errors: PST_EINVAL, PST_EDTYPE, PST_ESHAPE, PST_EHIP. */
int pst_gather_tree_logprobs_entropy_bwd(const void* logits, int64_t vocab, int32_t dtype,
                                         const pst_tree_meta* meta, const float* dlogprobs,
                                         const float* dentropy, const float* row_stats,
                                         void* dlogits, void* stream);

/* ---- device: tree-position rotary embedding -------------------------------- */

/* Rotary position embedding of packed tokens, in place, with position =
 * depth in the trie: the position the token has in every sequence through
 * it, which is what the position_ids that the tree-training page's "Archon
 * 引擎" section passes to the model alongside the tree metadata hold for a
 * packed tree.
 * For each row, head and i < head_dim/2, dims i and i + head_dim/2 are
 * rotated by a = pos * theta^(-2i/head_dim) (rotate-half pairing):
 *   y_i = x_i cos a - x_{i+d/2} sin a,   y_{i+d/2} = x_{i+d/2} cos a + x_i sin a
 * inverse != 0 rotates by -a (the backward of the forward rotation).  Angles
 * are formed and reduced modulo 2 pi in float64, their sine and cosine taken
 * in float; pad rows are left untouched (position 0).
 *   x   device [Np, n_heads, head_dim] dtype, 16-byte aligned (read and written)
 * theta <= 0 selects 10000.  head_dim: a multiple of 16 (bf16) or 8 (fp32),
 * at most 256.
 * Errors: PST_EINVAL, PST_EDTYPE, PST_ESHAPE, PST_EHIP. */
int pst_tree_rope(void* x, const pst_tree_meta* meta, int32_t n_heads, int32_t head_dim,
                  int32_t dtype, float theta, int32_t inverse, void* stream);

/* ---- device: dense mask export ------------------------------------------ */

/* Mask formats of pst_tree_dense_mask. */
enum { PST_MASK_U8 = 0, PST_MASK_ADD_F32 = 1, PST_MASK_ADD_BF16 = 2 };

/* Write the dense attention mask of the packed tree(s) behind `meta`, the
 * tensor form that the tree-training page's Megatron section uses instead of
 * a block mask so that it can be saved for gradient checkpointing.
 *   out  device [Np, Np], row = query i, column = key j, 16-byte aligned,
 *        Np = the metadata's padded rows (a forest's metadata gives its
 *        block-diagonal mask); caller-owned, fully overwritten.
 * Key j is visible to query i iff j is i or an ancestor of i (j <= i <=
 * subtree_end[j] in preorder); pad rows see only themselves.
 *   format  PST_MASK_U8: uint8, 1 visible, 0 hidden;
 *           PST_MASK_ADD_F32 / PST_MASK_ADD_BF16: additive, 0 visible, -inf hidden.
 * Any Np the metadata holds is covered (row groups are strided over a
 * capped grid).  Errors: PST_EINVAL, PST_EDTYPE (unknown format),
 * PST_ESHAPE (misaligned out), PST_EHIP. */
int pst_tree_dense_mask(const pst_tree_meta* meta, int32_t format, void* out, void* stream);

/* ---- host: micro-batch / rank allocation -------------------------------- */

/* Packing algorithms (article on AReaL's FFD/KK micro-batch packing). */
enum { PST_PACK_FFD = 0, PST_PACK_KK = 1 };

typedef struct {
  int32_t n_groups;
  int64_t total;          /* sum of all values */
  int64_t max_load;       /* largest group sum */
  int64_t min_load;       /* smallest group sum */
  int64_t spread;         /* max_load - min_load */
  int64_t wasted_tokens;  /* n_groups * capacity - total */
  double imbalance_ratio; /* max_load / mean (1 when the mean is 0) */
  double std_dev;         /* population standard deviation of the group sums */
  double cv;              /* std_dev / mean (0 when the mean is 0) */
  double utilization;     /* total / (n_groups * capacity) */
} pst_pack_metrics;

/* Allocate n weighted items (sequence lengths, per-tree costs) to groups
 * (micro-batches, data-parallel ranks), as the packing article's FFD and KK
 * sections describe.
 *   values      host int64 [n], non-negative, each at most `capacity`
 *   capacity    largest group sum allowed (a huge value balances without a
 *               capacity, as for assigning work to ranks)
 *   min_groups  at least this many groups (never more groups than items)
 *   divisor     the group count is rounded up to a multiple of it where the
 *               item count allows
 *   algorithm   PST_PACK_FFD: stable descending order, each item to the
 *               lightest group it fits (lowest index on ties), else a new
 *               group; the first min_groups items open groups.
 *               PST_PACK_KK: k-way Karmarkar-Karp largest differencing with
 *               k = max(min_groups, ceil(total / capacity)) rounded up to the
 *               divisor and capped at n; states pop by largest spread (push
 *               order on ties) and combine lightest-with-heaviest subsets.  If
 *               a group still exceeds the capacity, FFD is used instead.
 *   group_of    host int32 [n] out: the group of every item; KK numbers its
 *               groups in ascending order of their sums, FFD in creation order
 *   n_groups    out: the number of groups
 *   fell_back   out (may be NULL): 1 when KK fell back to FFD
 * Errors: PST_EINVAL (NULL, n < 1, capacity <= 0, min_groups or divisor < 1,
 * negative value, unknown algorithm), PST_ECAPACITY (an item above the
 * capacity), PST_ENOMEM. */
int pst_pack_allocate(const int64_t* values, int32_t n, int64_t capacity, int32_t min_groups,
                      int32_t divisor, int32_t algorithm, int32_t* group_of, int32_t* n_groups,
                      int32_t* fell_back);

/* Packing-quality metrics of an allocation (the packing article's metrics
 * section): spread, imbalance ratio, standard deviation, coefficient of
 * variation, utilization and wasted tokens of the group sums.
 *   values [n], group_of [n] (each in [0, n_groups)): host arrays.
 * Errors: PST_EINVAL, PST_ERANGE (a group index out of range). */
int pst_pack_metrics_compute(const int64_t* values, int32_t n, const int32_t* group_of,
                             int32_t n_groups, int64_t capacity, pst_pack_metrics* out);

/* Message of the last failed call on this thread ("" if none). */
const char* pst_last_error(void);

/* SHA-256, in hex, of the sources this library was built from (its C++ and
 * HIP sources, the headers under include/ and the build script), or
 * "unknown" for a build that did not record it.  A loader compares it with
 * the sources at hand to refuse a library built from other ones.  The
 * string is static; the call never fails. */
const char* pst_build_sources_sha256(void);

#ifdef __cplusplus
}
#endif

#endif /* PST_H */
