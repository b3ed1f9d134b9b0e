"""Tree-causal verification attention for AMD MI355X (gfx950).

The HIP library (libtreeattn.so, C ABI in include/tree_attn.h) does all the
work; ``api`` is its ctypes binding.  ``workloads`` draws seeded synthetic
inputs.  The binding is loaded on first use of one of its names, so the
input generator can be imported on machines without the built library.

One verification step, all tensors on the GPU (shapes in the docstrings
of the functions)::

    import tree_masked_attention_amd as tma
    masks, bad = tma.build_mask(parents, tree_offsets, max_nodes)
    out, lse = tma.verify(q, k_cache, v_cache, page_table, prefix_lens,
                          tree_offsets, masks, max_prefix_len, max_nodes,
                          scale, workspace=ws)   # ws: zero-filled once
    lens, nodes, bonus = tma.accept_commit(parents, tree_offsets, masks,
                                           draft_tokens, target_tokens,
                                           root_tokens, max_nodes, k_cache,
                                           v_cache, page_table, prefix_lens)

``tma.build_tree`` makes the draft trees from the drafting head's top-k
log-probabilities, ``tma.verify_ex`` takes FP8 E4M3 caches or head
dimension 64, and ``tma.gdn_verify`` / ``tma.gdn_commit`` verify and
commit Gated DeltaNet layers over the same trees.
"""

_API_NAMES = ("build_mask", "verify", "workspace_size", "describe_plan",
              "accept", "commit_kv", "accept_commit", "build_tree",
              "gdn_verify", "gdn_commit", "verify_ex",
              "status_string",
              "abi_version", "mask_words_for", "TreeAttnError")


def __getattr__(name):
    if name in _API_NAMES:
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
