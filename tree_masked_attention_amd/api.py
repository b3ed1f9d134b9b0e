"""Python binding of libtreeattn.so (argument marshalling only).

Every computation happens in the HIP library; torch supplies device
memory and the current stream.  The library must be built
(``python -m tree_masked_attention_amd._build``); without it, importing
this module raises.
"""

from __future__ import annotations

import ctypes
import functools
import inspect
import os
from typing import Optional, Tuple

import torch

from ._build import LIB_PATH

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(6)
MAX_NODES = 1024

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with "
        "`python -m tree_masked_attention_amd._build` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i = ctypes.c_int32
_lib.tree_attn_status_string.restype = ctypes.c_char_p
_lib.tree_attn_status_string.argtypes = [ctypes.c_int]
_lib.tree_attn_abi_version.restype = ctypes.c_int
_lib.tree_attn_abi_version.argtypes = []
_lib.tree_attn_build_mask.restype = ctypes.c_int
_lib.tree_attn_build_mask.argtypes = [_p, _p, _i, _i, _i, _i, _p, _p, _p]
_lib.tree_attn_workspace_size.restype = ctypes.c_size_t
_lib.tree_attn_workspace_size.argtypes = [_i] * 9
_lib.tree_attn_verify.restype = ctypes.c_int
_lib.tree_attn_verify.argtypes = (
    [_p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _i,
     ctypes.c_float, _i, _p, _p, _p, ctypes.c_size_t, _p])

_VERIFY_ARGS = ([_p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _i, _i, _i, _i, _i,
                 _i, _i, _i, ctypes.c_float, _i, _p, _p, _p, ctypes.c_size_t,
                 _p])
for _name in ("tree_attn_verify_attend", "tree_attn_verify_merge"):
    getattr(_lib, _name).restype = ctypes.c_int
    getattr(_lib, _name).argtypes = _VERIFY_ARGS

_lib.tree_attn_verify_noalloc.restype = ctypes.c_int
_lib.tree_attn_verify_noalloc.argtypes = _VERIFY_ARGS[:22] + [_p]
NOALLOC_SCRATCH_BYTES = 32 << 20

_lib.tree_attn_describe_plan.restype = ctypes.c_int
_lib.tree_attn_describe_plan.argtypes = [_i] * 9 + [_p]

_lib.tree_attn_accept.restype = ctypes.c_int
_lib.tree_attn_accept.argtypes = [_p, _p, _p, _i, _p, _p, _p, _i, _i, _i,
                                  _p, _p, _p, _p]
_lib.tree_attn_commit_kv.restype = ctypes.c_int
_lib.tree_attn_commit_kv.argtypes = [_p, _p, _p, _i, _i, _i, _p, _p, _p, _i,
                                     _i, _i, _p]

_lib.tree_attn_accept_commit.restype = ctypes.c_int
_lib.tree_attn_accept_commit.argtypes = [_p, _p, _p, _i, _p, _p, _p, _i, _i,
                                         _i, _p, _p, _p, _i, _i, _i, _p, _i,
                                         _p, _p, _p, _p]

_lib.tree_attn_build_tree.restype = ctypes.c_int
_lib.tree_attn_build_tree.argtypes = [_p, _p, _i, _i, _i, _i, _i, _p, _p, _p,
                                      _p, _p, _p]

_lib.tree_attn_gdn_verify.restype = ctypes.c_int
_lib.tree_attn_gdn_verify.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _i, _i,
                                      _i, _i, _i, _i, _p, _p, _p]
_lib.tree_attn_gdn_commit.restype = ctypes.c_int
_lib.tree_attn_gdn_commit.argtypes = [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i,
                                      _p, _p]

_lib.tree_attn_verify_ex.restype = ctypes.c_int
_lib.tree_attn_verify_ex.argtypes = (
    [_p, _p, _p, _i, _p, _p, _p, _i, _i, _i, _p, _p, _p, _i, _i, _i, _i, _i,
     _i, _i, _i, ctypes.c_float, _i, _p, _p, _p, ctypes.c_size_t, _p])
_lib.tree_attn_workspace_size_ex.restype = ctypes.c_size_t
_lib.tree_attn_workspace_size_ex.argtypes = [_i] * 10
_lib.tree_attn_describe_plan_ex.restype = ctypes.c_int
_lib.tree_attn_describe_plan_ex.argtypes = [_i] * 10 + [_p]

KV_BF16, KV_FP8_E4M3 = 0, 1

EXPORTED = ("tree_attn_status_string", "tree_attn_abi_version",
            "tree_attn_build_mask", "tree_attn_workspace_size",
            "tree_attn_describe_plan", "tree_attn_verify",
            "tree_attn_verify_attend", "tree_attn_verify_merge",
            "tree_attn_verify_noalloc",
            "tree_attn_accept", "tree_attn_commit_kv",
            "tree_attn_accept_commit", "tree_attn_build_tree",
            "tree_attn_gdn_verify", "tree_attn_gdn_commit",
            "tree_attn_verify_ex", "tree_attn_workspace_size_ex",
            "tree_attn_describe_plan_ex")
GDN_MAX_NODES = 128


class TreeAttnError(RuntimeError):
    pass


def status_string(code: int) -> str:
    return _lib.tree_attn_status_string(int(code)).decode()


def abi_version() -> int:
    return int(_lib.tree_attn_abi_version())


def _raise(code: int, what: str) -> None:
    if code == OK:
        return
    msg = f"{what}: {status_string(code)} (status {code})"
    if code in (ERR_NULL, ERR_SHAPE, ERR_WORKSPACE):
        raise ValueError(msg)
    if code == ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    raise TreeAttnError(msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _on_stream(fn):
    """Runs fn with its `stream` argument, when one is given, as torch's
    current stream: the buffers fn allocates (and zero-fills) are then
    ordered before its launches on that stream, and the caching allocator
    ties them to it, so they are not handed to other work while the
    launches still use them."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrapper(*args, **kw):
        stream = sig.bind(*args, **kw).arguments.get("stream")
        if stream is None:
            return fn(*args, **kw)
        with torch.cuda.stream(stream):
            return fn(*args, **kw)
    return wrapper


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dev(t: torch.Tensor, dtype, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def mask_words_for(max_nodes: int) -> int:
    return max(1, (int(max_nodes) + 63) // 64)


def build_mask_raw(parents, tree_offsets, num_seqs, total_nodes, max_nodes,
                   mask_words, masks, bad_node, stream=None) -> int:
    """Direct call of tree_attn_build_mask with raw device pointers."""
    return int(_lib.tree_attn_build_mask(
        parents, tree_offsets, num_seqs, total_nodes, max_nodes, mask_words,
        masks, bad_node, stream))


@_on_stream
def build_mask(parents: torch.Tensor, tree_offsets: torch.Tensor,
               max_nodes: int, mask_words: Optional[int] = None,
               masks: Optional[torch.Tensor] = None,
               bad_node: Optional[torch.Tensor] = None,
               stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Ancestor-or-self bitmasks of the draft trees.

    parents int32 [N] (local indices, -1 = root), tree_offsets int32 [S+1].
    Returns (masks int64 [N, W] holding the uint64 words, bad_node int32
    [S]: -1 per valid tree, else the first invalid global node).
    """
    _dev(parents, torch.int32, "parents")
    _dev(tree_offsets, torch.int32, "tree_offsets")
    S = tree_offsets.numel() - 1
    N = parents.numel()
    W = mask_words_for(max_nodes) if mask_words is None else int(mask_words)
    if masks is None:
        masks = torch.empty((N, W), dtype=torch.int64, device=parents.device)
    if bad_node is None:
        bad_node = torch.empty((max(S, 1),), dtype=torch.int32,
                               device=parents.device)
    _raise(build_mask_raw(_ptr(parents), _ptr(tree_offsets), S, N,
                          int(max_nodes), W, _ptr(masks), _ptr(bad_node),
                          _stream(stream)), "tree_attn_build_mask")
    return masks, bad_node


def workspace_size(num_seqs: int, total_nodes: int, num_q_heads: int,
                   num_kv_heads: int, head_dim: int, max_prefix_len: int,
                   max_nodes: int, page_size: int = 16,
                   num_splits: int = 0) -> int:
    return int(_lib.tree_attn_workspace_size(
        num_seqs, total_nodes, num_q_heads, num_kv_heads, head_dim,
        max_prefix_len, max_nodes, page_size, num_splits))


def describe_plan(num_seqs: int, total_nodes: int, num_q_heads: int,
                  num_kv_heads: int, head_dim: int, max_prefix_len: int,
                  max_nodes: int, page_size: int = 16,
                  num_splits: int = 0) -> dict:
    """The launch verify() makes for these sizes: waves per workgroup,
    query rows per workgroup, splits of the key range, keys per split,
    workgroups."""
    info = (ctypes.c_int32 * 5)()
    code = _lib.tree_attn_describe_plan(
        num_seqs, total_nodes, num_q_heads, num_kv_heads, head_dim,
        max_prefix_len, max_nodes, page_size, num_splits,
        ctypes.cast(info, ctypes.c_void_p))
    _raise(code, "tree_attn_describe_plan")
    return {"waves": info[0], "rows": info[1], "splits": info[2],
            "chunk": info[3], "workgroups": info[4]}


def describe_plan_ex(kv_dtype: int, num_seqs: int, total_nodes: int,
                     num_q_heads: int, num_kv_heads: int, head_dim: int,
                     max_prefix_len: int, max_nodes: int, page_size: int = 16,
                     num_splits: int = 0) -> dict:
    """The launch verify_ex() makes for these sizes (same keys as
    describe_plan)."""
    info = (ctypes.c_int32 * 5)()
    code = _lib.tree_attn_describe_plan_ex(
        kv_dtype, num_seqs, total_nodes, num_q_heads, num_kv_heads, head_dim,
        max_prefix_len, max_nodes, page_size, num_splits,
        ctypes.cast(info, ctypes.c_void_p))
    _raise(code, "tree_attn_describe_plan_ex")
    return {"waves": info[0], "rows": info[1], "splits": info[2],
            "chunk": info[3], "workgroups": info[4]}


@_on_stream
def verify(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           page_table: torch.Tensor, prefix_lens: torch.Tensor,
           tree_offsets: torch.Tensor, masks: torch.Tensor,
           max_prefix_len: int, max_nodes: int, scale: float,
           num_splits: int = 0, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None,
           stream=None, phase: str = "both") -> Tuple[torch.Tensor,
                                                      torch.Tensor]:
    """Tree-causal verification attention.

    q bf16 [N, Hq, d]; k_cache / v_cache bf16 [num_pages, page_size, Hkv, d];
    page_table int32 [S, max_pages_per_seq]; prefix_lens int32 [S];
    tree_offsets int32 [S+1]; masks int64 [N, W] (uint64 words from
    build_mask).  Returns (out bf16 [N, Hq, d], lse fp32 [N, Hq]).
    phase: "both" (tree_attn_verify), or "attend" / "merge" for its two
    launches (tree_attn_verify_attend / _merge; pass the same out, lse and
    workspace to both).  A workspace passed in must be zero-filled before
    its first use (its first bytes are the split launch's arrival counters,
    which every call leaves at zero); one allocated here is.
    """
    for t, dt, n in ((q, torch.bfloat16, "q"), (k_cache, torch.bfloat16, "k_cache"),
                     (v_cache, torch.bfloat16, "v_cache"),
                     (page_table, torch.int32, "page_table"),
                     (prefix_lens, torch.int32, "prefix_lens"),
                     (tree_offsets, torch.int32, "tree_offsets"),
                     (masks, torch.int64, "masks")):
        _dev(t, dt, n)
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [N, Hq, d] and k/v caches "
                         "[num_pages, page_size, Hkv, d]")
    N, Hq, d = q.shape
    num_pages, page_size, Hkv, dk = k_cache.shape
    if dk != d:
        raise ValueError("head_dim of q and the caches differ")
    S = prefix_lens.numel()
    if tree_offsets.numel() != S + 1 or page_table.dim() != 2 or \
            page_table.shape[0] != S:
        raise ValueError("page_table / tree_offsets do not match prefix_lens")
    if masks.dim() != 2 or masks.shape[0] != N:
        raise ValueError("masks must be [N, W]")
    W = masks.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((N, Hq), dtype=torch.float32, device=q.device)
    ws_bytes = workspace_size(S, N, Hq, Hkv, d, max_prefix_len, max_nodes,
                              page_size, num_splits)
    if phase != "both" and workspace is None and ws_bytes > 0:
        raise ValueError(f"phase {phase!r} needs the caller's workspace: "
                         "the attend and merge launches must share one")
    if workspace is None and ws_bytes > 0:
        workspace = torch.zeros((ws_bytes,), dtype=torch.uint8,
                                device=q.device)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    fn = {"both": _lib.tree_attn_verify,
          "attend": _lib.tree_attn_verify_attend,
          "merge": _lib.tree_attn_verify_merge}[phase]
    code = fn(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        page_table.shape[1], num_pages, page_size, _ptr(prefix_lens),
        _ptr(tree_offsets), _ptr(masks), W, S, N, int(max_prefix_len),
        int(max_nodes), Hq, Hkv, d, float(scale), int(num_splits), _ptr(out),
        _ptr(lse), _ptr(workspace), ws_len, _stream(stream))
    _raise(code, f"tree_attn_verify ({phase})")
    return out, lse


@_on_stream
def accept(parents: torch.Tensor, tree_offsets: torch.Tensor,
           masks: torch.Tensor, draft_tokens: torch.Tensor,
           target_tokens: torch.Tensor, root_tokens: torch.Tensor,
           max_nodes: int, accept_len: Optional[torch.Tensor] = None,
           accept_nodes: Optional[torch.Tensor] = None,
           bonus_tokens: Optional[torch.Tensor] = None,
           stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Accepted path of every draft tree (exact match on the target's
    tokens).  parents / tree_offsets / masks as for build_mask; draft and
    target tokens int32 [N], root_tokens int32 [S].  Returns (accept_len
    int32 [S], accept_nodes int32 [S, max_nodes] padded with -1,
    bonus_tokens int32 [S])."""
    for t, n in ((parents, "parents"), (tree_offsets, "tree_offsets"),
                 (draft_tokens, "draft_tokens"),
                 (target_tokens, "target_tokens"),
                 (root_tokens, "root_tokens")):
        _dev(t, torch.int32, n)
    _dev(masks, torch.int64, "masks")
    S = tree_offsets.numel() - 1
    N = parents.numel()
    if draft_tokens.numel() != N or target_tokens.numel() != N or \
            root_tokens.numel() != S:
        raise ValueError("token arrays do not match the trees")
    if masks.dim() != 2 or masks.shape[0] != N:
        raise ValueError("masks must be [N, W]")
    dev = parents.device
    if accept_len is None:
        accept_len = torch.empty((max(S, 1),), dtype=torch.int32, device=dev)
    if accept_nodes is None:
        accept_nodes = torch.empty((max(S, 1), int(max_nodes)),
                                   dtype=torch.int32, device=dev)
    if bonus_tokens is None:
        bonus_tokens = torch.empty((max(S, 1),), dtype=torch.int32,
                                   device=dev)
    code = _lib.tree_attn_accept(
        _ptr(parents), _ptr(tree_offsets), _ptr(masks), masks.shape[1],
        _ptr(draft_tokens), _ptr(target_tokens), _ptr(root_tokens), S, N,
        int(max_nodes), _ptr(accept_len), _ptr(accept_nodes),
        _ptr(bonus_tokens), _stream(stream))
    _raise(code, "tree_attn_accept")
    return accept_len[:S], accept_nodes[:S], bonus_tokens[:S]


def commit_kv(k_cache: torch.Tensor, v_cache: torch.Tensor,
              page_table: torch.Tensor, prefix_lens: torch.Tensor,
              accept_len: torch.Tensor, accept_nodes: torch.Tensor,
              stream=None) -> None:
    """Moves the accepted nodes' cache rows to positions P_s .. P_s+tau-1,
    in place.  k_cache / v_cache [num_pages, page_size, ...] of any dtype
    (same shape and dtype); accept_len / accept_nodes from accept()."""
    for t, n in ((page_table, "page_table"), (prefix_lens, "prefix_lens"),
                 (accept_len, "accept_len"), (accept_nodes, "accept_nodes")):
        _dev(t, torch.int32, n)
    _dev(k_cache, k_cache.dtype, "k_cache")
    _dev(v_cache, k_cache.dtype, "v_cache")
    if k_cache.shape != v_cache.shape or k_cache.dim() < 2:
        raise ValueError("k_cache and v_cache must both be "
                         "[num_pages, page_size, ...]")
    S = prefix_lens.numel()
    if page_table.dim() != 2 or page_table.shape[0] != S or \
            accept_len.numel() != S or accept_nodes.dim() != 2 or \
            accept_nodes.shape[0] != S:
        raise ValueError("page_table / accept arrays do not match prefix_lens")
    num_pages, page_size = k_cache.shape[0], k_cache.shape[1]
    token_bytes = _token_bytes(k_cache)
    code = _lib.tree_attn_commit_kv(
        _ptr(k_cache), _ptr(v_cache), _ptr(page_table), page_table.shape[1],
        num_pages, page_size, _ptr(prefix_lens), _ptr(accept_len),
        _ptr(accept_nodes), S, accept_nodes.shape[1], token_bytes,
        _stream(stream))
    _raise(code, "tree_attn_commit_kv")


def _token_bytes(k_cache: torch.Tensor) -> int:
    return (k_cache[0, 0].numel() * k_cache.element_size()
            if k_cache.shape[0] else 16)


@_on_stream
def accept_commit(parents: torch.Tensor, tree_offsets: torch.Tensor,
                  masks: torch.Tensor, draft_tokens: torch.Tensor,
                  target_tokens: torch.Tensor, root_tokens: torch.Tensor,
                  max_nodes: int, k_cache: torch.Tensor,
                  v_cache: torch.Tensor, page_table: torch.Tensor,
                  prefix_lens: torch.Tensor,
                  accept_len: Optional[torch.Tensor] = None,
                  accept_nodes: Optional[torch.Tensor] = None,
                  bonus_tokens: Optional[torch.Tensor] = None,
                  stream=None) -> Tuple[torch.Tensor, torch.Tensor,
                                        torch.Tensor]:
    """accept() then commit_kv() in one launch; same arguments and
    results (the caches are updated in place)."""
    for t, n in ((parents, "parents"), (tree_offsets, "tree_offsets"),
                 (draft_tokens, "draft_tokens"),
                 (target_tokens, "target_tokens"),
                 (root_tokens, "root_tokens"), (page_table, "page_table"),
                 (prefix_lens, "prefix_lens")):
        _dev(t, torch.int32, n)
    _dev(masks, torch.int64, "masks")
    _dev(k_cache, k_cache.dtype, "k_cache")
    _dev(v_cache, k_cache.dtype, "v_cache")
    S = tree_offsets.numel() - 1
    N = parents.numel()
    if draft_tokens.numel() != N or target_tokens.numel() != N or \
            root_tokens.numel() != S or prefix_lens.numel() != S:
        raise ValueError("token arrays / prefix_lens do not match the trees")
    if masks.dim() != 2 or masks.shape[0] != N:
        raise ValueError("masks must be [N, W]")
    if k_cache.shape != v_cache.shape or k_cache.dim() < 2 or \
            page_table.dim() != 2 or page_table.shape[0] != S:
        raise ValueError("caches must both be [num_pages, page_size, ...] "
                         "and page_table [S, max_pages_per_seq]")
    dev = parents.device
    if accept_len is None:
        accept_len = torch.empty((max(S, 1),), dtype=torch.int32, device=dev)
    if accept_nodes is None:
        accept_nodes = torch.empty((max(S, 1), int(max_nodes)),
                                   dtype=torch.int32, device=dev)
    if bonus_tokens is None:
        bonus_tokens = torch.empty((max(S, 1),), dtype=torch.int32,
                                   device=dev)
    code = _lib.tree_attn_accept_commit(
        _ptr(parents), _ptr(tree_offsets), _ptr(masks), masks.shape[1],
        _ptr(draft_tokens), _ptr(target_tokens), _ptr(root_tokens), S, N,
        int(max_nodes), _ptr(k_cache), _ptr(v_cache), _ptr(page_table),
        page_table.shape[1], k_cache.shape[0], k_cache.shape[1],
        _ptr(prefix_lens), _token_bytes(k_cache), _ptr(accept_len),
        _ptr(accept_nodes), _ptr(bonus_tokens), _stream(stream))
    _raise(code, "tree_attn_accept_commit")
    return accept_len[:S], accept_nodes[:S], bonus_tokens[:S]


@_on_stream
def build_tree(logp: torch.Tensor, tokens: torch.Tensor, budget: int,
               width: int = 1, stream=None) -> dict:
    """Draft trees by best-first expansion (width candidates per step).
    logp fp32 [S, D, K] (rows non-increasing), tokens int32 [S, D, K].
    Returns {"parents", "tokens", "depths": int32 [S, budget],
    "scores": fp32 [S, budget], "sizes": int32 [S]}."""
    _dev(logp, torch.float32, "logp")
    _dev(tokens, torch.int32, "tokens")
    if logp.dim() != 3 or tokens.shape != logp.shape:
        raise ValueError("logp and tokens must both be [S, D, K]")
    S, D, K = logp.shape
    dev = logp.device
    B = int(budget)
    out = {"parents": torch.empty((S, B), dtype=torch.int32, device=dev),
           "tokens": torch.empty((S, B), dtype=torch.int32, device=dev),
           "depths": torch.empty((S, B), dtype=torch.int32, device=dev),
           "scores": torch.empty((S, B), dtype=torch.float32, device=dev),
           "sizes": torch.empty((max(S, 1),), dtype=torch.int32, device=dev)}
    code = _lib.tree_attn_build_tree(
        _ptr(logp), _ptr(tokens), S, D, K, B, int(width),
        _ptr(out["parents"]), _ptr(out["tokens"]), _ptr(out["depths"]),
        _ptr(out["scores"]), _ptr(out["sizes"]), _stream(stream))
    _raise(code, "tree_attn_build_tree")
    out["sizes"] = out["sizes"][:S]
    return out


@_on_stream
def gdn_verify(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
               g: torch.Tensor, beta: torch.Tensor, state: torch.Tensor,
               tree_offsets: torch.Tensor, masks: torch.Tensor,
               max_nodes: int, out: Optional[torch.Tensor] = None,
               u: Optional[torch.Tensor] = None,
               stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Gated DeltaNet tree verification.  q, k, v bf16 [N, H, 128]; g, beta
    fp32 [N, H]; state fp32 [S, H, 128, 128] (S0, read only); masks from
    build_mask.  Returns (out bf16 [N, H, 128], u fp32 [N, H, 128])."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, torch.bfloat16, n)
    for t, n in ((g, "g"), (beta, "beta"), (state, "state")):
        _dev(t, torch.float32, n)
    _dev(tree_offsets, torch.int32, "tree_offsets")
    _dev(masks, torch.int64, "masks")
    if q.dim() != 3 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k and v must all be [N, H, d]")
    N, H, d = q.shape
    S = tree_offsets.numel() - 1
    if g.shape != (N, H) or beta.shape != (N, H) or \
            state.shape != (S, H, d, d):
        raise ValueError("g / beta must be [N, H] and state [S, H, d, d]")
    if masks.dim() != 2 or masks.shape[0] != N:
        raise ValueError("masks must be [N, W]")
    if out is None:
        out = torch.empty_like(q)
    if u is None:
        u = torch.empty((N, H, d), dtype=torch.float32, device=q.device)
    code = _lib.tree_attn_gdn_verify(
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state),
        _ptr(tree_offsets), _ptr(masks), masks.shape[1], S, N,
        int(max_nodes), H, d, _ptr(out), _ptr(u), _stream(stream))
    _raise(code, "tree_attn_gdn_verify")
    return out, u


def gdn_commit(k: torch.Tensor, u: torch.Tensor, g: torch.Tensor,
               tree_offsets: torch.Tensor, accept_len: torch.Tensor,
               accept_nodes: torch.Tensor, state: torch.Tensor,
               stream=None) -> None:
    """Deferred GDN state commit, in place on state fp32 [S, H, 128, 128]:
    the state of the last accepted node (accept_len / accept_nodes from
    accept()); k bf16 and u fp32 [N, H, 128], g fp32 [N, H]."""
    _dev(k, torch.bfloat16, "k")
    for t, n in ((u, "u"), (g, "g"), (state, "state")):
        _dev(t, torch.float32, n)
    for t, n in ((tree_offsets, "tree_offsets"), (accept_len, "accept_len"),
                 (accept_nodes, "accept_nodes")):
        _dev(t, torch.int32, n)
    if k.dim() != 3 or u.shape != k.shape:
        raise ValueError("k and u must both be [N, H, d]")
    N, H, d = k.shape
    S = tree_offsets.numel() - 1
    if g.shape != (N, H) or state.shape != (S, H, d, d) or \
            accept_len.numel() != S or accept_nodes.dim() != 2 or \
            accept_nodes.shape[0] != S:
        raise ValueError("g / state / accept arrays do not match")
    code = _lib.tree_attn_gdn_commit(
        _ptr(k), _ptr(u), _ptr(g), _ptr(tree_offsets), _ptr(accept_len),
        _ptr(accept_nodes), S, accept_nodes.shape[1], H, d, _ptr(state),
        _stream(stream))
    _raise(code, "tree_attn_gdn_commit")


@_on_stream
def verify_ex(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
              page_table: torch.Tensor, prefix_lens: torch.Tensor,
              tree_offsets: torch.Tensor, masks: torch.Tensor,
              max_prefix_len: int, max_nodes: int, scale: float,
              k_scale: Optional[torch.Tensor] = None,
              v_scale: Optional[torch.Tensor] = None, num_splits: int = 0,
              out: Optional[torch.Tensor] = None,
              lse: Optional[torch.Tensor] = None,
              workspace: Optional[torch.Tensor] = None,
              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """verify() for bf16 or FP8 E4M3 caches and head_dim 64 or 128.

    q bf16 [N, Hq, d]; k_cache / v_cache bf16, or uint8 /
    torch.float8_e4m3fn (E4M3 codes, with fp32 k_scale / v_scale [Hkv]),
    [num_pages, page_size, Hkv, d]; the rest as for verify()."""
    _dev(q, torch.bfloat16, "q")
    if k_cache.dtype == torch.bfloat16:
        kv = KV_BF16
    elif k_cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        kv = KV_FP8_E4M3
    else:
        raise ValueError(f"unsupported cache dtype {k_cache.dtype}")
    _dev(k_cache, k_cache.dtype, "k_cache")
    _dev(v_cache, k_cache.dtype, "v_cache")
    for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if t is not None:
            _dev(t, torch.float32, n)
    for t, dt, n in ((page_table, torch.int32, "page_table"),
                     (prefix_lens, torch.int32, "prefix_lens"),
                     (tree_offsets, torch.int32, "tree_offsets"),
                     (masks, torch.int64, "masks")):
        _dev(t, dt, n)
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [N, Hq, d] and k/v caches "
                         "[num_pages, page_size, Hkv, d]")
    N, Hq, d = q.shape
    num_pages, page_size, Hkv, dk = k_cache.shape
    if dk != d:
        raise ValueError("head_dim of q and the caches differ")
    S = prefix_lens.numel()
    if tree_offsets.numel() != S + 1 or page_table.dim() != 2 or \
            page_table.shape[0] != S:
        raise ValueError("page_table / tree_offsets do not match prefix_lens")
    if masks.dim() != 2 or masks.shape[0] != N:
        raise ValueError("masks must be [N, W]")
    for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        if t is not None and t.numel() != Hkv:
            raise ValueError(f"{n} must have num_kv_heads entries")
    W = masks.shape[1]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((N, Hq), dtype=torch.float32, device=q.device)
    ws_bytes = int(_lib.tree_attn_workspace_size_ex(
        kv, S, N, Hq, Hkv, d, int(max_prefix_len), int(max_nodes), page_size,
        int(num_splits)))
    if workspace is None and ws_bytes > 0:
        workspace = torch.zeros((ws_bytes,), dtype=torch.uint8,
                                device=q.device)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    code = _lib.tree_attn_verify_ex(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), kv, _ptr(k_scale),
        _ptr(v_scale), _ptr(page_table), page_table.shape[1], num_pages,
        page_size, _ptr(prefix_lens), _ptr(tree_offsets), _ptr(masks), W, S,
        N, int(max_prefix_len), int(max_nodes), Hq, Hkv, d, float(scale),
        int(num_splits), _ptr(out), _ptr(lse), _ptr(workspace), ws_len,
        _stream(stream))
    _raise(code, "tree_attn_verify_ex")
    return out, lse
