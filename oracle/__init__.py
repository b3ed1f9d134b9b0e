"""CPU oracle for tree-causal verification attention, the draft-tree
construction before it, the acceptance / KV-commit step after it and the
Gated DeltaNet tree verification (test infrastructure only: imported by the tests, the smoke check and the benchmark's CPU
baseline, never by the library)."""

from .accept_oracle import accept, accept_tree, commit_kv
from .gdn_oracle import gdn_commit_tree, gdn_tree_verify, gdn_verify
from .tree_build_oracle import build_tree, build_trees
from .tree_oracle import (ancestor_masks, tree_attention, widen_bf16,
                          workload_attention, workload_masks)

__all__ = ["accept", "accept_tree", "build_tree", "build_trees", "commit_kv",
           "gdn_commit_tree", "gdn_tree_verify", "gdn_verify", "ancestor_masks", "tree_attention", "widen_bf16",
           "workload_attention", "workload_masks"]
