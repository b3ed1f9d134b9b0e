/*
 * tree_attn.h - C ABI of libtreeattn.so: tree-causal verification attention
 * for tree speculative decoding on AMD Instinct MI355X (gfx950).
 *
 * The operation.  A draft tree of B_s nodes per sequence s, given in
 * topological order (parent[i] < i), is verified by the target model in one
 * forward pass.  In that pass every tree node attends to the sequence's
 * whole input prefix and to its ancestors in the tree, never to its
 * descendants or to sibling branches (JETFLOW, gist.science 2606.18394,
 * section 2 "Arquitectura Central", bullet on the tree-causal attention
 * mask; the branch factorization printed under it makes the ancestor set
 * the root-to-node path).  The node itself is part of its own context, so a
 * pure chain is ordinary causal attention.  The pages name the kernel that
 * does this in their serving engine ("paged FlashAttention with tree-mask
 * staging", section 3, item 3) but do not describe it; this library is its
 * own design.  Topological order of the tree is also what DFlash-TfM
 * (gist.science 2607.06763, method section 3) sorts into before verifying.
 *
 * Conventions shared by every entry point:
 *  - Pointers marked "dev" are device pointers on the current HIP device.
 *    The caller owns every buffer.  The library never allocates or frees
 *    device memory and keeps no pointer after a call returns.
 *  - `stream` is a hipStream_t passed as void* (NULL = default stream).
 *    Calls only enqueue work on it; none synchronises.
 *  - Every status is returned synchronously.  Argument errors (every
 *    status but TREE_ATTN_ERR_HIP) are found before any HIP call: nothing
 *    was launched and nothing was written.  TREE_ATTN_ERR_HIP means that
 *    the HIP runtime refused one of the call's own launches (checked by
 *    each launch's return code; an error that an earlier, unrelated HIP
 *    call left pending on the thread is neither reported nor cleared).
 *    Calls that make two launches (tree_attn_verify with its separate
 *    merge launch, tree_attn_verify_ex with split partials) may return it
 *    after the first launch was enqueued: that launch then writes only
 *    the workspace's partials, and out and lse are left unspecified.
 *  - All arrays are contiguous and row-major.
 *  - bf16 is the 16-bit bfloat16 format (1 sign, 8 exponent, 7 mantissa).
 *
 * Indexing of a tree.  Sequence s owns nodes tree_offsets[s] ..
 * tree_offsets[s+1]-1 (global node indices).  parents[] holds LOCAL
 * indices: parents[tree_offsets[s] + i] is the local index of node i's
 * parent in the same tree, or -1 for a root.  Several roots (a forest) are
 * allowed; each root sees the prefix plus its own path.
 *
 * Where the tree's keys live.  Node j of sequence s has its key and value
 * cached at logical position prefix_lens[s] + j of that sequence's paged
 * cache, so the cache of sequence s holds prefix_lens[s] + B_s tokens.
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
enum tree_attn_status {
  TREE_ATTN_OK = 0,
  TREE_ATTN_ERR_NULL = 1,        /* a required pointer is NULL              */
  TREE_ATTN_ERR_SHAPE = 2,       /* inconsistent sizes                      */
  TREE_ATTN_ERR_UNSUPPORTED = 3, /* valid, but not supported by this build  */
  TREE_ATTN_ERR_WORKSPACE = 4,   /* workspace missing or too small          */
  TREE_ATTN_ERR_HIP = 5          /* a HIP runtime call or launch failed     */
};

/* Static, human-readable name of a status code (never NULL). */
const char* tree_attn_status_string(int status);

/* ABI version of this header (increases on any signature change). */
int tree_attn_abi_version(void);

/* Largest tree a sequence may hold in this build (nodes). */
#define TREE_ATTN_MAX_NODES 1024

/*
 * tree_attn_build_mask - per-node ancestor-or-self bitmasks.
 *
 * Row i (global node index) of `masks` has bit (j % 64) of 64-bit word
 * (j / 64) set iff local node j of the same tree lies on the root-to-node
 * path of node i (node i included).  All other bits of the row, including
 * every bit >= B_s, are zero.
 *
 *   parents       dev int32 [total_nodes]   local parent index, -1 = root
 *   tree_offsets  dev int32 [num_seqs + 1]  tree_offsets[0] = 0,
 *                                           tree_offsets[num_seqs] = total_nodes
 *   num_seqs      >= 0
 *   total_nodes   >= 0
 *   max_nodes     host upper bound on every B_s, <= TREE_ATTN_MAX_NODES
 *   mask_words    W, words per row; W * 64 >= max_nodes, 1 <= W <= 16
 *   masks         dev uint64 [total_nodes][mask_words]   (output)
 *   bad_node      dev int32 [num_seqs] (output): -1 when tree s is valid,
 *                 else the global index of its first node whose parent is
 *                 outside [-1, i), or of its first node past max_nodes.
 *                 The rows of an invalid tree are unspecified.
 *
 * Host-side errors: ERR_NULL (a NULL pointer with num_seqs > 0), ERR_SHAPE
 * (negative sizes, mask_words * 64 < max_nodes), ERR_UNSUPPORTED
 * (max_nodes > TREE_ATTN_MAX_NODES or mask_words > 16), ERR_HIP.
 */
int tree_attn_build_mask(const int32_t* parents, const int32_t* tree_offsets,
                         int32_t num_seqs, int32_t total_nodes,
                         int32_t max_nodes, int32_t mask_words,
                         uint64_t* masks, int32_t* bad_node, void* stream);

/*
 * tree_attn_workspace_size - bytes of device workspace tree_attn_verify
 * needs for these sizes (0 when the planned launch needs none).
 * Arguments as for tree_attn_verify.  num_splits: 0 lets the library plan
 * the split of the key range; n > 0 asks for n splits, clamped to what the
 * key range allows (at least 64 keys per split, at most 1039 pages per
 * split, at most 256 splits).  Returns 0 for invalid sizes as well.
 */
size_t tree_attn_workspace_size(int32_t num_seqs, int32_t total_nodes,
                                int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t max_prefix_len,
                                int32_t max_nodes, int32_t page_size,
                                int32_t num_splits);

/*
 * tree_attn_describe_plan - the launch tree_attn_verify would make for
 * these sizes, for tests and benchmarks.  Arguments as for
 * tree_attn_workspace_size; info is a host array of 5 int32 that receives
 * { waves per workgroup (4 or 8), query rows per workgroup (64, 128 or
 *   256), splits of the key range, keys per split, workgroups launched }.
 * Returns TREE_ATTN_OK, or the status tree_attn_verify would return for
 * these sizes (info untouched).
 */
int tree_attn_describe_plan(int32_t num_seqs, int32_t total_nodes,
                            int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t max_prefix_len,
                            int32_t max_nodes, int32_t page_size,
                            int32_t num_splits, int32_t* info);

/*
 * tree_attn_verify - tree-causal verification attention over a paged
 * bf16 KV cache, with the softmax log-sum-exp.
 *
 * For node i of sequence s (global row n = tree_offsets[s] + i) and query
 * head h, with g = h / (num_q_heads / num_kv_heads) (contiguous GQA
 * groups), the allowed keys are the logical cache positions
 *     { 0 .. prefix_lens[s]-1 }  and  { prefix_lens[s] + j : bit j of masks[n] }
 * and, with x_t = scale * <q[n,h,:], K_s[t,g,:]> over the allowed t,
 *     out[n,h,:] = sum_t exp(x_t) V_s[t,g,:] / sum_t exp(x_t)   (bf16, RNE)
 *     lse[n,h]   = ln sum_t exp(x_t)                             (fp32)
 * K_s[t] is read from physical page page_table[s][t / page_size], slot
 * t % page_size.
 *
 *   q             dev bf16 [total_nodes, num_q_heads, head_dim]
 *   k_cache       dev bf16 [num_pages, page_size, num_kv_heads, head_dim]
 *   v_cache       dev bf16 [num_pages, page_size, num_kv_heads, head_dim]
 *   page_table    dev int32 [num_seqs, max_pages_per_seq]: logical page ->
 *                 physical page; must cover prefix_lens[s] + B_s tokens
 *   page_size     power of two, 1 .. 4096
 *   prefix_lens   dev int32 [num_seqs], each 0 .. max_prefix_len
 *   tree_offsets  dev int32 [num_seqs + 1] (as for tree_attn_build_mask)
 *   masks         dev uint64 [total_nodes][mask_words], as written by
 *                 tree_attn_build_mask (any ancestor relation is accepted)
 *   max_prefix_len, max_nodes   host upper bounds of the device values;
 *                 they size the launch, so no device-to-host copy is made
 *   head_dim      128 in this build
 *   scale         softmax scale > 0 (1/sqrt(head_dim) for standard attention)
 *   num_splits    0 = planned by the library; n > 0 forces n splits
 *   out           dev bf16 [total_nodes, num_q_heads, head_dim]  (output)
 *   lse           dev fp32 [total_nodes, num_q_heads], natural log (output)
 *   workspace     dev scratch of tree_attn_workspace_size(...) bytes, 256-B
 *                 aligned; may be NULL when that size is 0.  Owned by the
 *                 caller and reusable across calls of any sizes, one call
 *                 at a time (calls that overlap on one workspace race).
 *                 Its first 64 KB hold arrival counters: they must be zero
 *                 before the workspace's first use (e.g. hipMemset once
 *                 after allocation), and every call that completes leaves
 *                 them at zero.  Nonzero counters give wrong output, never
 *                 a hang or an access outside the buffers.
 *
 * Launches.  One attention launch.  With more than one split, every split
 * workgroup leaves its partial in the workspace and the last one of a row
 * block to finish (a device-scope counter, no waiting) merges the block's
 * partials into out and lse.  Sizes with more than 16384 (sequence, kv
 * head, row block) triples merge in a second launch instead
 * (tree_attn_verify_merge); the results are the same bits either way.
 *
 * Precision.  Scores, softmax and the P*V products accumulate in fp32
 * (P rounded to bf16 for the matrix cores).  When the key range is split
 * (workspace size > 0), each split's output, normalised by its own row
 * sum, passes through the workspace in fp16 scaled by a power of two per
 * row (so any bf16 V keeps fp16's 11-bit precision relative to the row's
 * largest entry), before the log-sum-exp merge in fp32.
 *
 * Device values outside the stated bounds (a prefix longer than
 * max_prefix_len, a tree larger than max_nodes, page ids outside
 * [0, num_pages)) give unspecified output for the rows concerned, but no
 * access outside the buffers described above.
 *
 * Host-side errors: ERR_NULL, ERR_SHAPE (num_q_heads % num_kv_heads != 0,
 * mask_words * 64 < max_nodes, page_size not a power of two, scale not
 * finite and positive, negative sizes), ERR_UNSUPPORTED (head_dim != 128, max_nodes >
 * TREE_ATTN_MAX_NODES), ERR_WORKSPACE, ERR_HIP.
 */
int tree_attn_verify(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* page_table, int32_t max_pages_per_seq,
                     int32_t num_pages, int32_t page_size,
                     const int32_t* prefix_lens, const int32_t* tree_offsets,
                     const uint64_t* masks, int32_t mask_words,
                     int32_t num_seqs, int32_t total_nodes,
                     int32_t max_prefix_len, int32_t max_nodes,
                     int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, float scale, int32_t num_splits,
                     void* out, float* lse, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * tree_attn_verify_noalloc - tree_attn_verify for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).
 *
 * Same operation, arguments (minus workspace and workspace_bytes), checks
 * and kernels as tree_attn_verify.  The split partials and arrival
 * counters live in a device array inside the library, one per GPU, of
 * TREE_ATTN_NOALLOC_SCRATCH_BYTES bytes, held from the library's load to
 * the end of the process; the call itself allocates nothing (no hipMalloc,
 * no allocating library routine).  Sizes whose plan needs more than that
 * (tree_attn_workspace_size(...) > TREE_ATTN_NOALLOC_SCRATCH_BYTES) return
 * TREE_ATTN_ERR_WORKSPACE before any launch.  The first call on a device
 * clears the array's counter area with a kernel on `stream`; every call
 * that completes leaves it at zero again.  All calls on one GPU share the
 * array: calls that overlap (other streams, other threads) race and give
 * wrong output; calls made one after another on one stream do not.
 */
#define TREE_ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)

int tree_attn_verify_noalloc(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    int32_t page_size, const int32_t* prefix_lens,
    const int32_t* tree_offsets, const uint64_t* masks, int32_t mask_words,
    int32_t num_seqs, int32_t total_nodes, int32_t max_prefix_len,
    int32_t max_nodes, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float scale, int32_t num_splits, void* out, float* lse,
    void* stream);

/*
 * tree_attn_verify_attend, tree_attn_verify_merge - the two launches of
 * tree_attn_verify, for callers that schedule or time them separately.
 *
 * Same arguments and checks as tree_attn_verify.  _attend runs the split-KV
 * pass over the prefix with the tree block masked in registers; with one
 * planned split it writes out and lse itself, otherwise it leaves the
 * split partials in the workspace.  _merge then combines the partials into
 * out and lse (log-sum-exp merge), and launches nothing when the plan has
 * one split.  _attend followed by _merge on the same stream, with the same
 * arguments and workspace, gives exactly the results of tree_attn_verify.
 * Neither touches the workspace's arrival counters.
 */
int tree_attn_verify_attend(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    int32_t page_size, const int32_t* prefix_lens,
    const int32_t* tree_offsets, const uint64_t* masks, int32_t mask_words,
    int32_t num_seqs, int32_t total_nodes, int32_t max_prefix_len,
    int32_t max_nodes, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float scale, int32_t num_splits, void* out, float* lse,
    void* workspace, size_t workspace_bytes, void* stream);

int tree_attn_verify_merge(
    const void* q, const void* k_cache, const void* v_cache,
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    int32_t page_size, const int32_t* prefix_lens,
    const int32_t* tree_offsets, const uint64_t* masks, int32_t mask_words,
    int32_t num_seqs, int32_t total_nodes, int32_t max_prefix_len,
    int32_t max_nodes, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, float scale, int32_t num_splits, void* out, float* lse,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * tree_attn_build_tree - draft trees by best-first expansion, the step
 * before the verification.
 *
 * The drafting head emits logits for all tree depths at once; nodes are
 * ranked by their cumulative draft log-probability and best-first
 * expansion builds the tree up to a token budget (JETFLOW, gist.science
 * 2606.18394, section 2, bullet on tree construction).  Each step may take
 * the w best candidates at once and expand them together, which builds a
 * B-node tree in ceil(B / w) steps (DFlash-TfM, gist.science 2607.06763,
 * method section 2, tree construction).  The rule, per sequence s:
 *  - candidates at depth d = 1 .. depth are (parent, rank j) with
 *    tokens[s][d-1][j] and score = parent's score + logp[s][d-1][j] (fp32;
 *    a depth-1 candidate has no parent node and score logp[s][0][j]);
 *  - the candidate set starts with the topk depth-1 candidates; each step
 *    removes the best min(width, budget - size) candidates -- higher score
 *    first, then lower parent node index (none counts as -1), then lower
 *    rank -- appends them as nodes in that order, then adds the topk
 *    children of each of them (none past the last depth);
 *  - it stops at budget nodes or when no candidate is left.
 * Node indices are insertion order, so parents[i] < i (the topological
 * order tree_attn_build_mask takes; depth-1 nodes are roots).
 *
 *   logp       dev fp32 [num_seqs][depth][topk], every row non-increasing
 *              (as a top-k returns it) and finite
 *   tokens     dev int32 [num_seqs][depth][topk]
 *   depth      >= 0; topk 1 .. 64; depth * topk <= 8192
 *   budget     0 .. TREE_ATTN_MAX_NODES; width >= 1 (1 = strict best-first)
 *   parents, node_tokens, depths   dev int32 [num_seqs][budget] (outputs):
 *              parent node index (-1 for a depth-1 node), token, depth;
 *              past the tree's size: -1, -1, 0
 *   scores     dev fp32 [num_seqs][budget] (output): node scores, 0 past
 *              the size
 *   sizes      dev int32 [num_seqs] (output): nodes built,
 *              min(budget, number of nodes of the full tree)
 *
 * Rows that are not non-increasing, or not finite, give unspecified trees
 * for that sequence, but no access outside the buffers above.
 *
 * Host-side errors: ERR_SHAPE (negative sizes, topk < 1, width < 1),
 * ERR_UNSUPPORTED (budget > TREE_ATTN_MAX_NODES, topk > 64,
 * depth * topk > 8192), ERR_NULL, ERR_HIP.
 */
int tree_attn_build_tree(const float* logp, const int32_t* tokens,
                         int32_t num_seqs, int32_t depth, int32_t topk,
                         int32_t budget, int32_t width, int32_t* parents,
                         int32_t* node_tokens, int32_t* depths, float* scores,
                         int32_t* sizes, void* stream);

/*
 * tree_attn_accept - the accepted path of every verified draft tree.
 *
 * After the verification pass the target model has, for every tree node n,
 * the token it would emit next (target_tokens[n]) and, per sequence, the
 * token it would emit right after the prefix (root_tokens[s]).  Decoding
 * then keeps the accepted part of the tree, tau tokens per step (JETFLOW,
 * gist.science 2606.18394, section 4, where tau is reported per budget).
 * The pages do not spell out the acceptance rule; this library takes
 * exact match against the target's choices:
 *  - local node i of tree s matches when draft_tokens[n] (n the global
 *    index) equals the target's token after its parent: root_tokens[s] for
 *    a root, else target_tokens[tree_offsets[s] + parents[n]];
 *  - the accepted path is the longest root-to-node path whose nodes all
 *    match; among equally long ones, the one ending at the smallest local
 *    index.  With distinct draft tokens among siblings this is the usual
 *    walk down the one matching child.
 *
 *   parents, tree_offsets, num_seqs, total_nodes, max_nodes
 *                 as for tree_attn_build_mask
 *   masks, mask_words   the rows tree_attn_build_mask wrote for these trees
 *                 (W words per node; the path is read from them)
 *   draft_tokens  dev int32 [total_nodes]  token of each draft node
 *   target_tokens dev int32 [total_nodes]  target's token after each node
 *   root_tokens   dev int32 [num_seqs]     target's token after the prefix
 *   accept_len    dev int32 [num_seqs] (output): tau_s, 0 .. B_s
 *   accept_nodes  dev int32 [num_seqs][max_nodes] (output): the accepted
 *                 path as local node indices, root first, then -1 to the
 *                 end of the row
 *   bonus_tokens  dev int32 [num_seqs] (output): the target's token after
 *                 the last accepted node, root_tokens[s] when tau_s = 0
 *
 * Trees that tree_attn_build_mask reports invalid, or masks that are not
 * its rows for these trees, give unspecified output for that sequence but
 * no access outside the buffers above.
 *
 * Host-side errors: ERR_SHAPE (negative sizes, mask_words < 1,
 * mask_words * 64 < max_nodes), ERR_UNSUPPORTED (mask_words > 16,
 * max_nodes > TREE_ATTN_MAX_NODES), ERR_NULL (a NULL pointer that the
 * sizes make necessary), ERR_HIP.
 */
int tree_attn_accept(const int32_t* parents, const int32_t* tree_offsets,
                     const uint64_t* masks, int32_t mask_words,
                     const int32_t* draft_tokens, const int32_t* target_tokens,
                     const int32_t* root_tokens, int32_t num_seqs,
                     int32_t total_nodes, int32_t max_nodes,
                     int32_t* accept_len, int32_t* accept_nodes,
                     int32_t* bonus_tokens, void* stream);

/*
 * tree_attn_commit_kv - moves the accepted nodes' keys and values to the
 * front of the tree's region of the paged cache, in place.
 *
 * The cache commit waits until the accepted branch is known (DFlash-TfM,
 * gist.science 2607.06763, method section on rollback-free verification;
 * there for the recurrent state, here for the attention cache).  Node n of
 * sequence s sits at logical position prefix_lens[s] + n (as in
 * tree_attn_verify); for j = 0 .. accept_len[s]-1 the token row at
 * position prefix_lens[s] + accept_nodes[s][j] is copied to position
 * prefix_lens[s] + j, in k_cache and in v_cache, byte for byte.  Rows
 * already in place are not copied; every other row keeps its contents.
 * The result equals doing the copies one by one in increasing j, which
 * never reads a row an earlier copy wrote, provided accept_nodes[s] is
 * strictly increasing (as tree_attn_accept writes it).
 *
 *   k_cache, v_cache  dev [num_pages, page_size, token_bytes] bytes of any
 *                 element type (bf16 [.., num_kv_heads, head_dim] gives
 *                 token_bytes = num_kv_heads * head_dim * 2); 16-byte
 *                 aligned; read and written
 *   page_table    dev int32 [num_seqs, max_pages_per_seq]
 *   page_size     power of two
 *   prefix_lens   dev int32 [num_seqs]
 *   accept_len, accept_nodes   as written by tree_attn_accept
 *   max_nodes     columns of accept_nodes, <= TREE_ATTN_MAX_NODES
 *   token_bytes   bytes of one token row of one cache, a positive multiple
 *                 of 16, at most 1 MiB
 *
 * Pages that hold positions at or past prefix_lens[s] must belong to
 * sequence s alone.  A copy whose source or destination page lies outside
 * the page table or outside [0, num_pages) is skipped; a row list that is
 * not strictly increasing gives unspecified rows of that sequence, but no
 * access outside the buffers above.
 *
 * Host-side errors: ERR_SHAPE (negative sizes, page_size not a power of
 * two, token_bytes not a positive multiple of 16, caches not 16-byte
 * aligned), ERR_UNSUPPORTED (max_nodes > TREE_ATTN_MAX_NODES, token_bytes
 * > 1 MiB), ERR_NULL, ERR_HIP.
 */
int tree_attn_commit_kv(void* k_cache, void* v_cache,
                        const int32_t* page_table, int32_t max_pages_per_seq,
                        int32_t num_pages, int32_t page_size,
                        const int32_t* prefix_lens, const int32_t* accept_len,
                        const int32_t* accept_nodes, int32_t num_seqs,
                        int32_t max_nodes, int32_t token_bytes,
                        void* stream);

/*
 * tree_attn_accept_commit - tree_attn_accept followed by
 * tree_attn_commit_kv, in one launch.
 *
 * Arguments as for those two calls (token_bytes, the caches and the page
 * table as for tree_attn_commit_kv; the accepted lists are outputs here).
 * Results are identical to the two calls made in order: the path is found
 * on chip and the copies are planned from it without a round trip through
 * memory.
 *
 * Host-side errors: those of both calls.
 */
int tree_attn_accept_commit(
    const int32_t* parents, const int32_t* tree_offsets,
    const uint64_t* masks, int32_t mask_words, const int32_t* draft_tokens,
    const int32_t* target_tokens, const int32_t* root_tokens,
    int32_t num_seqs, int32_t total_nodes, int32_t max_nodes, void* k_cache,
    void* v_cache, const int32_t* page_table, int32_t max_pages_per_seq,
    int32_t num_pages, int32_t page_size, const int32_t* prefix_lens,
    int32_t token_bytes, int32_t* accept_len, int32_t* accept_nodes,
    int32_t* bonus_tokens, void* stream);

/* Largest tree tree_attn_gdn_verify takes (nodes). */
#define TREE_ATTN_GDN_MAX_NODES 128

/*
 * tree_attn_gdn_verify - rollback-free verification of a draft tree through
 * one Gated DeltaNet (GDN) layer.
 *
 * DFlash-TfM (gist.science 2607.06763, method section 3, rollback-free tree
 * verification for GDN) gives the GDN state recurrence
 *   S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
 * sorts the tree topologically and verifies it through a masked triangular
 * solve (I + X) U = beta V over ancestor relations, committing the state
 * only after acceptance.  The pages leave the per-node quantities open;
 * this call fixes them as follows.  Per node i and head h: alpha_i =
 * e^{g_i}; node i's state S_i is the recurrence run along its
 * root-to-node path starting from the committed state S0 of its sequence
 * (siblings and descendants play no part); the outputs are
 *   out_i = S_i^T q_i                          (after node i's own update)
 *   u_i   = beta_i (v_i - alpha_i S_parent^T k_i),
 * so that S_i = alpha_i S_parent + k_i u_i^T (S_parent = S0 for a root).
 * u is what tree_attn_gdn_commit needs.  A chain gives the ordinary
 * token-by-token recurrence.
 *
 *   q, k, v       dev bf16 [total_nodes][num_heads][head_dim]
 *   g             dev fp32 [total_nodes][num_heads]  log-decay (<= 0)
 *   beta          dev fp32 [total_nodes][num_heads]
 *   state         dev fp32 [num_seqs][num_heads][head_dim (k)][head_dim (v)]
 *                 S0 per sequence and head, k-major; read only
 *   tree_offsets  dev int32 [num_seqs + 1], as for tree_attn_build_mask
 *   masks, mask_words   as written by tree_attn_build_mask
 *   max_nodes     host upper bound on every B_s,
 *                 <= TREE_ATTN_GDN_MAX_NODES (128)
 *   num_heads     1 .. 16384 (q, k, v, g and beta all carry num_heads heads)
 *   head_dim      d_k = d_v; must be 128
 *   out           dev bf16 [total_nodes][num_heads][head_dim] (output)
 *   u             dev fp32 [total_nodes][num_heads][head_dim] (output)
 *
 * Precision: products run on the bf16 matrix cores; fp32 operands (S0 and
 * the triangular factors) are split into two bf16 parts, which keeps about
 * 16 mantissa bits per product; accumulation is fp32.  out is rounded to
 * bf16 once at the end.
 * A tree with more than 128 nodes (tree_offsets breaking max_nodes) is
 * skipped without writing.
 *
 * Host-side errors: ERR_SHAPE (negative sizes, num_heads < 1, mask_words *
 * 64 < max_nodes), ERR_UNSUPPORTED (head_dim != 128, max_nodes > 128,
 * num_heads > 16384, num_seqs * num_heads > 2^31 - 1), ERR_NULL, ERR_HIP.
 */
int tree_attn_gdn_verify(const void* q, const void* k, const void* v,
                         const float* g, const float* beta,
                         const float* state, const int32_t* tree_offsets,
                         const uint64_t* masks, int32_t mask_words,
                         int32_t num_seqs, int32_t total_nodes,
                         int32_t max_nodes, int32_t num_heads,
                         int32_t head_dim, void* out, float* u,
                         void* stream);

/*
 * tree_attn_gdn_commit - the deferred GDN state commit (DFlash-TfM,
 * gist.science 2607.06763, method section 3: the state is committed once
 * the accepted branch is known).
 *
 * For every sequence s and head h, state[s][h] is replaced, in place, by
 * the state of the last accepted node: with p_1 .. p_n the accepted path
 * (accept_nodes[s][0 .. n-1], n = accept_len[s], root first, as written
 * by tree_attn_accept) and G_j the sum of g over p_1 .. p_j,
 *   S_new = e^{G_n} S0 + sum_j e^{G_n - G_j} k_{p_j} u_{p_j}^T,
 * which equals the recurrence S <- alpha S + k u^T run along the path.
 * n = 0 leaves the state unchanged.  u is the output of
 * tree_attn_gdn_verify for the same tree.
 *
 *   k, u, g       as for tree_attn_gdn_verify (u as it wrote it)
 *   tree_offsets  dev int32 [num_seqs + 1]
 *   accept_len    dev int32 [num_seqs]
 *   accept_nodes  dev int32 [num_seqs][max_nodes], local node indices
 *   max_nodes     columns of accept_nodes, <= TREE_ATTN_MAX_NODES
 *   state         dev fp32 [num_seqs][num_heads][head_dim][head_dim],
 *                 updated in place
 *
 * Path entries outside the tree are skipped; accept_len is clamped to
 * [0, max_nodes].  Host-side errors: ERR_SHAPE (negative sizes,
 * num_heads < 1), ERR_UNSUPPORTED (head_dim != 128, max_nodes >
 * TREE_ATTN_MAX_NODES), ERR_NULL, ERR_HIP.
 */
int tree_attn_gdn_commit(const void* k, const float* u, const float* g,
                         const int32_t* tree_offsets,
                         const int32_t* accept_len,
                         const int32_t* accept_nodes, int32_t num_seqs,
                         int32_t max_nodes, int32_t num_heads,
                         int32_t head_dim, float* state, void* stream);

/* K/V element types of tree_attn_verify_ex. */
#define TREE_ATTN_KV_BF16 0     /* bfloat16 */
#define TREE_ATTN_KV_FP8_E4M3 1 /* OCP FP8 E4M3 (e4m3fn), scaled per kv head */

/*
 * tree_attn_verify_ex - tree_attn_verify for more cache formats and head
 * dimensions (the same operation, JETFLOW section 2 "Arquitectura
 * Central", bullet on the tree-causal mask).
 *
 * Arguments as for tree_attn_verify, plus:
 *   kv_dtype      TREE_ATTN_KV_BF16 or TREE_ATTN_KV_FP8_E4M3: the element
 *                 type of k_cache and v_cache ([num_pages][page_size]
 *                 [num_kv_heads][head_dim] elements, 1 or 2 bytes each)
 *   k_scale, v_scale
 *                 dev fp32 [num_kv_heads]: for FP8 the cached value of kv
 *                 head g stands for (E4M3 value) * scale[g]; NULL = 1.
 *                 Ignored for bf16.
 *   head_dim      64 or 128 (q, out: [total_nodes][num_q_heads][head_dim])
 * With bf16 and head_dim 128 this is exactly tree_attn_verify (the same
 * kernels).  FP8 with head_dim 128 runs the same kernels on FP8 tiles:
 * the DMA ring moves the codes, and each wave converts its operands to
 * bf16 (exactly: every E4M3 value is a bf16 value) as it reads them from
 * LDS; the K scale folds into the softmax scale and the V scale into the
 * output.  Head dim 64 runs the same kernels on rows of 128 bytes (bf16)
 * or 64 bytes (FP8), with split partials of 64 values per row.  The plan
 * is tree_attn_verify's, with one difference: where bf16 with head_dim
 * 128 replaces a split of the key range by 64-row blocks (pairs of at
 * most 128 rows, bandwidth-bound launches), these narrower rows keep
 * 128-row blocks and the split.  Workspace sizes come from
 * tree_attn_workspace_size_ex.
 *
 * The key range is cut into at most 256 splits of at most 1039 pages each
 * (the kernel copies a split's page ids to LDS), as for tree_attn_verify.
 *
 * Host-side errors: as tree_attn_verify; ERR_UNSUPPORTED also for
 * head_dim not 64 or 128, for an unknown kv_dtype, and for key ranges
 * longer than 256 splits of 1039 pages.
 */
int tree_attn_verify_ex(const void* q, const void* k_cache,
                        const void* v_cache, int32_t kv_dtype,
                        const float* k_scale, const float* v_scale,
                        const int32_t* page_table, int32_t max_pages_per_seq,
                        int32_t num_pages, int32_t page_size,
                        const int32_t* prefix_lens,
                        const int32_t* tree_offsets, const uint64_t* masks,
                        int32_t mask_words, int32_t num_seqs,
                        int32_t total_nodes, int32_t max_prefix_len,
                        int32_t max_nodes, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, float scale,
                        int32_t num_splits, void* out, float* lse,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/* Workspace bytes tree_attn_verify_ex needs for these sizes (0: none, or
 * sizes it would reject).  Same layout as tree_attn_verify's (the first
 * 64 KB are the counter area), so one workspace of the larger size serves
 * both. */
size_t tree_attn_workspace_size_ex(int32_t kv_dtype, int32_t num_seqs,
                                   int32_t total_nodes, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_prefix_len, int32_t max_nodes,
                                   int32_t page_size, int32_t num_splits);

/*
 * tree_attn_describe_plan_ex - tree_attn_describe_plan for the launches of
 * tree_attn_verify_ex (kv_dtype and head_dim as there).  Head dim 128
 * and 64, bf16 or FP8, run the tuned kernels with tree_attn_verify's
 * plan, except that rows narrower than 256 bytes keep a split where that
 * plan takes 64-row blocks without one.
 */
int tree_attn_describe_plan_ex(int32_t kv_dtype, int32_t num_seqs,
                               int32_t total_nodes, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim,
                               int32_t max_prefix_len, int32_t max_nodes,
                               int32_t page_size, int32_t num_splits,
                               int32_t* info);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H */
