"""CPU oracle for tree-causal verification attention (test infrastructure
only: imported by the tests, the smoke check and the benchmark's CPU
baseline, never by the library)."""

from .tree_oracle import (ancestor_masks, tree_attention, widen_bf16,
                          workload_attention, workload_masks)

__all__ = ["ancestor_masks", "tree_attention", "widen_bf16",
           "workload_attention", "workload_masks"]
