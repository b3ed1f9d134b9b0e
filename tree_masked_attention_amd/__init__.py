"""Tree-causal verification attention for AMD MI355X (gfx950).

The HIP library (libtreeattn.so, C ABI in include/tree_attn.h) does all the
work; ``api`` is its ctypes binding.  ``workloads`` draws seeded synthetic
inputs.  The binding is loaded on first use of one of its names, so the
input generator can be imported on machines without the built library.
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
