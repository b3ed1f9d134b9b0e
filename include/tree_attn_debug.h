/*
 * tree_attn_debug.h - extra entry point of debug builds of libtreeattn.so
 * (compiled with -DTREE_ATTN_DEBUG; release builds do not export it).
 *
 * The verification kernels trust the device values the caller passes
 * (page ids, prefix lengths, tree offsets): out-of-range ones are clamped
 * where they are used, so no access leaves the buffers, and the rows
 * concerned get unspecified output (see tree_attn_verify in tree_attn.h,
 * whose operation is the tree-causal attention of JETFLOW, gist.science
 * 2606.18394, section 2 "Arquitectura Central").  This call checks host
 * copies of those values against the same bounds and reports the first
 * one the planned launch would have clamped.
 */
#ifndef TREE_ATTN_DEBUG_H
#define TREE_ATTN_DEBUG_H

#include <stdint.h>

#include "tree_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Kinds of report[0] written by tree_attn_debug_check_verify. */
enum tree_attn_debug_kind {
  TREE_ATTN_DEBUG_OK = 0,
  TREE_ATTN_DEBUG_OFFSETS = 1,    /* tree_offsets not 0 .. total_nodes, non-decreasing */
  TREE_ATTN_DEBUG_TREE_SIZE = 2,  /* a tree larger than max_nodes              */
  TREE_ATTN_DEBUG_PREFIX = 3,     /* prefix_lens[s] outside 0 .. max_prefix_len */
  TREE_ATTN_DEBUG_PARENT = 4,     /* parent[i] outside -1 .. i-1                */
  TREE_ATTN_DEBUG_TABLE = 5,      /* prefix + tree longer than the page table  */
  TREE_ATTN_DEBUG_PAGE_CACHE = 6, /* a split's pages exceed the kernel's LDS copy */
  TREE_ATTN_DEBUG_PAGE_ID = 7     /* a page id outside 0 .. num_pages-1        */
};

/*
 * tree_attn_debug_check_verify - the arguments of a tree_attn_verify call,
 * with HOST copies of page_table [num_seqs][max_pages_per_seq],
 * prefix_lens [num_seqs], tree_offsets [num_seqs+1] and parents
 * [total_nodes] (local indices, -1 = root), checked against every bound
 * the planned launch relies on: the size checks of tree_attn_verify, then
 * per sequence its offsets, tree size, prefix length, parents, table
 * length, and every page id each split of the plan reads.
 *
 *   report   host int32 [4], written: {kind, sequence, index, value} of
 *            the first problem (index: the node, logical page or offset
 *            slot concerned), or {TREE_ATTN_DEBUG_OK, -1, -1, -1}.
 *
 * Returns TREE_ATTN_OK when every value is in range, TREE_ATTN_ERR_SHAPE
 * when report names a problem, or the status tree_attn_verify would
 * return for bad sizes (ERR_SHAPE / ERR_UNSUPPORTED, report kind OK) or
 * a NULL array (ERR_NULL).  Reads only the host arrays; no HIP call.
 */
int tree_attn_debug_check_verify(
    const int32_t* page_table, int32_t max_pages_per_seq, int32_t num_pages,
    int32_t page_size, const int32_t* prefix_lens,
    const int32_t* tree_offsets, const int32_t* parents, int32_t mask_words,
    int32_t num_seqs, int32_t total_nodes, int32_t max_prefix_len,
    int32_t max_nodes, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t num_splits, int32_t* report);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_DEBUG_H */
