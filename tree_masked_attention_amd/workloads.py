"""Seeded synthetic inputs for tree-verification attention.

This module only draws random inputs; it holds none of the attention or
mask arithmetic, so both the CPU oracle (through the tests) and the HIP
path consume exactly the same arrays.

Workload shapes follow the JETFLOW pages (gist.science 2606.18394): a draft
tree of B nodes per sequence given in topological order (parent[i] < i,
section 2 "Construccion de Arboles", budgets 16 and 256), verified by the
target over a paged KV cache (section 3, item 3: paged FlashAttention with
tree-mask staging).  Model shapes are those of the models evaluated in
section 4 (Qwen3-8B: 32 q / 8 kv heads; Qwen3-30B-A3B: 32 q / 4 kv heads;
head dim 128).  No dataset item is used: every value is N(0, 1) noise.

Layouts (all row-major, contiguous):
  q          bf16 bits (uint16) [N, Hq, d]        N = sum of tree sizes
  k_cache    bf16 bits (uint16) [num_pages, page_size, Hkv, d]
  v_cache    bf16 bits (uint16) [num_pages, page_size, Hkv, d]
  page_table int32 [S, max_pages_per_seq]  logical page -> physical page,
             -1 in slots past the sequence's last page
  prefix_lens int32 [S]      tree node j of sequence s sits at logical
             position prefix_lens[s] + j of that sequence's cache
  tree_offsets int32 [S + 1] nodes of sequence s are rows
             tree_offsets[s] .. tree_offsets[s+1]-1 of q
  parents    int32 [N]       local parent index, -1 for a root

Draw order for one seed: a numpy PCG64 generator seeded with ``seed``
draws the prefix lengths, then each tree node by node, then the page
permutation.  The bulk arrays q, k, v (float32 N(0, 1)) and the optional
per-token key factors each come from their own child of
SeedSequence([seed, 1]), split into a fixed number of chunks with one
child stream per chunk (so the values do not depend on the thread count).
Values are rounded to bf16 with round-to-nearest-even.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence

import numpy as np

PAGE_SIZE = 16
_CHUNKS = 16
_THREADS = max(1, min(16, len(os.sched_getaffinity(0))))


def _chunk_bounds(n: int):
    return [int(x) for x in np.linspace(0, n, _CHUNKS + 1)]


def _parallel(fn, count: int) -> None:
    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fn, range(count)))


def _bulk_normal(ss: np.random.SeedSequence, shape) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    kids = ss.spawn(_CHUNKS)
    bnd = _chunk_bounds(n)

    def fill(i):
        np.random.default_rng(kids[i]).standard_normal(
            out=out[bnd[i]:bnd[i + 1]], dtype=np.float32)
    _parallel(fill, _CHUNKS)
    return out.reshape(shape)


def _bulk_uniform(ss: np.random.SeedSequence, shape, lo, hi) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    kids = ss.spawn(_CHUNKS)
    bnd = _chunk_bounds(n)

    def fill(i):
        out[bnd[i]:bnd[i + 1]] = np.random.default_rng(kids[i]).uniform(
            lo, hi, size=bnd[i + 1] - bnd[i])
    _parallel(fill, _CHUNKS)
    return out.reshape(shape)


# --------------------------------------------------------------------------
# bf16 helpers (storage conversion only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16.  Inputs here are finite.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1).view(np.uint32)
    out = np.empty(flat.shape[0], dtype=np.uint16)
    bnd = _chunk_bounds(flat.shape[0])

    def conv(i):
        u = flat[bnd[i]:bnd[i + 1]]
        lsb = (u >> np.uint32(16)) & np.uint32(1)
        out[bnd[i]:bnd[i + 1]] = ((u + np.uint32(0x7FFF) + lsb)
                                  >> np.uint32(16)).astype(np.uint16)
    _parallel(conv, _CHUNKS)
    return out.reshape(x.shape)


def quantize_e4m3(x: np.ndarray):
    """Per-kv-head FP8 E4M3 quantisation of a cache [pages, slots, Hkv, d]:
    scale_h = 2^ceil(log2(amax_h / 448)) (a power of two, so a stored code
    times its scale is exact in bf16 and fp32), codes = E4M3(x / scale_h)
    with round-to-nearest-even (torch's float8_e4m3fn conversion).  Returns
    (uint8 codes, fp32 scales [Hkv])."""
    import torch
    amax = np.abs(x).max(axis=(0, 1, 3)).astype(np.float64)
    amax = np.maximum(amax, 1e-30)
    scale = np.exp2(np.ceil(np.log2(amax / 448.0))).astype(np.float32)
    y = torch.from_numpy(np.ascontiguousarray(x / scale[None, None, :, None],
                                              dtype=np.float32))
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# tree shapes
# --------------------------------------------------------------------------

def draw_tree(rng: np.random.Generator, num_nodes: int, rule: str,
              p_chain: float = 0.5) -> np.ndarray:
    """Parent array of one draft tree in topological order.

    rule "pchain": parent[0] = -1; for i >= 1, parent[i] = i-1 with
      probability p_chain, else uniform in [0, i).  One uniform draw per
      node for the chain test, then one integer draw when it fails.
    rule "wide":  parent[i] uniform in [0, i) (one integer draw per node).
    rule "chain": parent[i] = i - 1 (no draws).
    rule "star":  parent[i] = 0 (no draws).
    """
    par = np.empty(num_nodes, dtype=np.int32)
    if num_nodes == 0:
        return par
    par[0] = -1
    for i in range(1, num_nodes):
        if rule == "pchain":
            if rng.random() < p_chain:
                par[i] = i - 1
            else:
                par[i] = int(rng.integers(0, i))
        elif rule == "wide":
            par[i] = int(rng.integers(0, i))
        elif rule == "chain":
            par[i] = i - 1
        elif rule == "star":
            par[i] = 0
        else:
            raise ValueError(f"unknown tree rule {rule!r}")
    return par


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    q: np.ndarray            # uint16 [N, Hq, d]
    k_cache: np.ndarray      # uint16 [num_pages, page_size, Hkv, d]
    v_cache: np.ndarray      # uint16 [num_pages, page_size, Hkv, d]
    page_table: np.ndarray   # int32 [S, max_pages_per_seq]
    prefix_lens: np.ndarray  # int32 [S]
    tree_offsets: np.ndarray  # int32 [S+1]
    parents: np.ndarray      # int32 [N]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    scale: float
    kv_format: str = "bf16"            # "bf16" (uint16 bits) or "e4m3" (uint8)
    k_scale: Optional[np.ndarray] = None  # fp32 [Hkv] for "e4m3"
    v_scale: Optional[np.ndarray] = None

    @property
    def num_seqs(self) -> int:
        return int(self.prefix_lens.shape[0])

    @property
    def total_nodes(self) -> int:
        return int(self.tree_offsets[-1])

    @property
    def tree_sizes(self) -> np.ndarray:
        return np.diff(self.tree_offsets).astype(np.int64)

    @property
    def max_nodes(self) -> int:
        sz = self.tree_sizes
        return int(sz.max()) if sz.size else 0

    @property
    def max_prefix_len(self) -> int:
        return int(self.prefix_lens.max()) if self.prefix_lens.size else 0

    @property
    def num_pages(self) -> int:
        return int(self.k_cache.shape[0])

    @property
    def max_pages_per_seq(self) -> int:
        return int(self.page_table.shape[1])

    def mask_words(self) -> int:
        return max(1, (self.max_nodes + 63) // 64)


def make_workload(seed: int, prefix_lens: Sequence[int] | None = None,
                  tree_sizes: Sequence[int] | None = None,
                  num_q_heads: int = 8, num_kv_heads: int = 2,
                  head_dim: int = 128, page_size: int = PAGE_SIZE,
                  tree_rules: Sequence[str] | str = "pchain",
                  p_chain: Sequence[float] | float = 0.5,
                  shuffle_pages: bool = True,
                  key_factor_range: Optional[tuple] = None,
                  prefix_range: Optional[tuple] = None,
                  num_seqs: Optional[int] = None,
                  extra_pages: int = 0,
                  kv_format: str = "bf16",
                  value_scale: float = 1.0,
                  name: str = "custom") -> Workload:
    """Draw one synthetic workload.

    Either ``prefix_lens`` is given, or ``prefix_range`` (inclusive integer
    bounds, drawn per sequence) together with ``num_seqs``.
    ``tree_rules`` / ``p_chain`` may be per-sequence lists.
    ``key_factor_range`` multiplies each cached token's key row (all kv
    heads) by a factor drawn uniformly from that range, in float32, before
    bf16 rounding.  ``extra_pages`` appends unused physical pages to the
    pool (filled with noise), so a page table can address a pool larger
    than the live tokens.
    ``value_scale`` multiplies every cached value row in float32 before the
    rounding (a power of two keeps the bf16 values exact multiples of the
    unscaled ones).
    """
    rng = np.random.default_rng(seed)
    if prefix_lens is None:
        if prefix_range is None or num_seqs is None:
            raise ValueError("need prefix_lens or (prefix_range, num_seqs)")
        lo, hi = prefix_range
        prefix = rng.integers(lo, hi + 1, size=num_seqs).astype(np.int32)
    else:
        prefix = np.asarray(prefix_lens, dtype=np.int32)
    S = int(prefix.shape[0])
    if tree_sizes is None:
        raise ValueError("tree_sizes required")
    sizes = np.asarray(tree_sizes, dtype=np.int64)
    if sizes.shape[0] == 1 and S > 1:
        sizes = np.full(S, int(sizes[0]), dtype=np.int64)
    if sizes.shape[0] != S:
        raise ValueError("tree_sizes must have one entry per sequence")
    rules = [tree_rules] * S if isinstance(tree_rules, str) else list(tree_rules)
    pcs = [p_chain] * S if np.isscalar(p_chain) else list(p_chain)

    parents: List[np.ndarray] = []
    for s in range(S):
        parents.append(draw_tree(rng, int(sizes[s]), rules[s], float(pcs[s])))
    par = (np.concatenate(parents).astype(np.int32) if S
           else np.zeros(0, np.int32))
    offsets = np.zeros(S + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(sizes)

    tokens = prefix.astype(np.int64) + sizes
    pages_per_seq = (tokens + page_size - 1) // page_size
    live_pages = int(pages_per_seq.sum())
    num_pages = max(1, live_pages + int(extra_pages))
    if shuffle_pages:
        perm = rng.permutation(num_pages).astype(np.int32)
    else:
        perm = np.arange(num_pages, dtype=np.int32)
    max_pps = max(1, int(pages_per_seq.max()) if S else 1)
    table = np.full((S, max_pps), -1, dtype=np.int32)
    cursor = 0
    for s in range(S):
        n = int(pages_per_seq[s])
        table[s, :n] = perm[cursor:cursor + n]
        cursor += n

    N = int(offsets[-1])
    ss_q, ss_k, ss_v, ss_f = np.random.SeedSequence([seed, 1]).spawn(4)
    q32 = _bulk_normal(ss_q, (N, num_q_heads, head_dim))
    kv_shape = (num_pages, page_size, num_kv_heads, head_dim)
    k32 = _bulk_normal(ss_k, kv_shape)
    if key_factor_range is not None:
        lo, hi = key_factor_range
        fac = _bulk_uniform(ss_f, (num_pages, page_size), lo, hi)
        k32 *= fac[:, :, None, None]
    v32 = _bulk_normal(ss_v, kv_shape)
    if value_scale != 1.0:
        v32 *= np.float32(value_scale)
    k_scale = v_scale = None
    if kv_format == "e4m3":
        k_cache, k_scale = quantize_e4m3(k32)
        v_cache, v_scale = quantize_e4m3(v32)
    elif kv_format == "bf16":
        k_cache, v_cache = f32_to_bf16_bits(k32), f32_to_bf16_bits(v32)
    else:
        raise ValueError(f"unknown kv_format {kv_format!r}")
    wl = Workload(
        name=name,
        q=f32_to_bf16_bits(q32),
        k_cache=k_cache,
        v_cache=v_cache,
        page_table=table,
        prefix_lens=prefix,
        tree_offsets=offsets,
        parents=par,
        num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads,
        head_dim=head_dim,
        page_size=page_size,
        scale=1.0 / math.sqrt(head_dim),
        kv_format=kv_format,
        k_scale=k_scale,
        v_scale=v_scale,
    )
    return wl


# --------------------------------------------------------------------------
# the five standard workloads
# --------------------------------------------------------------------------

# name -> (seed, keyword arguments of make_workload)
STANDARD: Dict[str, tuple] = {
    # one sequence, 256-token prefix, 16-node tree, 8 q / 2 kv heads,
    # contiguous cache (identity page table)
    "small-b16-p256": (1, dict(prefix_lens=[256], tree_sizes=[16],
                               num_q_heads=8, num_kv_heads=2,
                               tree_rules="pchain", p_chain=0.5,
                               shuffle_pages=False)),
    # Qwen3-8B attention shape, one sequence, 4096 prefix, 256-node tree
    "qwen3-8b-b256-p4k": (2, dict(prefix_lens=[4096], tree_sizes=[256],
                                  num_q_heads=32, num_kv_heads=8,
                                  tree_rules="pchain", p_chain=0.5,
                                  shuffle_pages=True)),
    # serving mix: 8 sequences, prefixes uniform in [1024, 8192], 64-node
    # trees alternating wide / deep (parent = i-1 with probability 0.9)
    "serving-mix-8x-b64": (3, dict(prefix_range=(1024, 8192), num_seqs=8,
                                   tree_sizes=[64], num_q_heads=32,
                                   num_kv_heads=8,
                                   tree_rules=["wide", "pchain"] * 4,
                                   p_chain=[0.0, 0.9] * 4,
                                   shuffle_pages=True)),
    # Qwen3-30B-A3B attention shape under load: 32 sequences, 2048 prefix,
    # 16-node trees
    "qwen3-30b-a3b-32x-b16-p2k": (4, dict(prefix_lens=[2048] * 32,
                                          tree_sizes=[16], num_q_heads=32,
                                          num_kv_heads=4,
                                          tree_rules="pchain", p_chain=0.5,
                                          shuffle_pages=True)),
    # long context, large budget: 4 sequences, 32768 prefix, 256-node
    # trees, key rows scaled per token by U[0.5, 2]
    "long-32k-4x-b256": (5, dict(prefix_lens=[32768] * 4, tree_sizes=[256],
                                 num_q_heads=32, num_kv_heads=8,
                                 tree_rules="pchain", p_chain=0.5,
                                 shuffle_pages=True,
                                 key_factor_range=(0.5, 2.0))),
}

STANDARD_ORDER = list(STANDARD.keys())


def draw_tokens(wl: Workload, seed: int, vocab: int = 8,
                p_agree: float = 0.7):
    """Synthetic tokens for the acceptance step: each node's draft token,
    the target's token after each node, and the target's token after each
    sequence's prefix.  With probability p_agree the target's token after a
    node (or after the prefix) is the draft token of one of the node's
    children (or of one of the roots), so that accepted paths of several
    nodes occur; otherwise it is uniform in [0, vocab)."""
    rng = np.random.default_rng([seed, 7])
    N, S = wl.total_nodes, wl.num_seqs
    draft = rng.integers(0, vocab, size=N).astype(np.int32)
    target = rng.integers(0, vocab, size=N).astype(np.int32)
    root = rng.integers(0, vocab, size=S).astype(np.int32)
    for s in range(S):
        a, b = int(wl.tree_offsets[s]), int(wl.tree_offsets[s + 1])
        children: Dict[int, List[int]] = {}
        for i in range(b - a):
            children.setdefault(int(wl.parents[a + i]), []).append(i)
        for n in [-1] + list(range(b - a)):
            ch = children.get(n)
            if ch and rng.random() < p_agree:
                tok = draft[a + ch[int(rng.integers(0, len(ch)))]]
                if n < 0:
                    root[s] = tok
                else:
                    target[a + n] = tok
    return draft, target, root


def draw_draft_topk(num_seqs: int, depth: int, topk: int, seed: int,
                    vocab: int = 32000, pool: int = 64):
    """Synthetic per-depth outputs of a drafting head for tree construction:
    for every sequence and depth, the top-k log-probabilities (fp32, sorted
    non-increasing) of a softmax over `pool` random logits with a random
    sharpness in [1, 4), and their tokens (distinct in [0, vocab))."""
    rng = np.random.default_rng([seed, 11])
    S, D, K = num_seqs, depth, topk
    z = rng.standard_normal((S, D, pool)) * rng.uniform(1.0, 4.0, (S, D, 1))
    z = z - z.max(axis=2, keepdims=True)
    lse = np.log(np.exp(z).sum(axis=2, keepdims=True))
    lp = np.sort(z - lse, axis=2)[:, :, ::-1][:, :, :K].astype(np.float32)
    lp = np.ascontiguousarray(lp)
    tok = np.empty((S, D, K), dtype=np.int32)
    for s in range(S):
        for d in range(D):
            tok[s, d] = rng.choice(vocab, size=K, replace=False)
    return lp, tok


def draw_gdn_inputs(num_seqs: int, total_nodes: int, seed: int,
                    heads: int = 8, dim: int = 128):
    """Synthetic Gated DeltaNet layer inputs for num_seqs trees with
    total_nodes nodes: per node and head q, k (unit length, then rounded to
    bf16), v (N(0, 1), bf16), log-decays g = -U(0.001, 0.1) (alpha = e^g
    near 1), write strengths beta = sigmoid(N(0, 1)) (fp32), and per
    sequence and head a committed state S0 with N(0, 0.25) entries (fp32).
    Returns bf16 arrays as uint16 bits and fp32 arrays:
    (q, k, v, g, beta, S0)."""
    rng = np.random.default_rng([seed, 13])
    N, S, H, d = int(total_nodes), int(num_seqs), int(heads), int(dim)
    q = rng.standard_normal((N, H, d), dtype=np.float32)
    k = rng.standard_normal((N, H, d), dtype=np.float32)
    q /= np.maximum(np.linalg.norm(q, axis=2, keepdims=True), 1e-30)
    k /= np.maximum(np.linalg.norm(k, axis=2, keepdims=True), 1e-30)
    v = rng.standard_normal((N, H, d), dtype=np.float32)
    g = (-rng.uniform(0.001, 0.1, size=(N, H))).astype(np.float32)
    beta = (1.0 / (1.0 + np.exp(-rng.standard_normal((N, H))))).astype(np.float32)
    S0 = rng.standard_normal((S, H, d, d), dtype=np.float32) * np.float32(0.5)
    return (f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v),
            g, beta, S0)


def gdn_trees(tree_sizes: Sequence[int], rules: Sequence[str] | str,
              seed: int, p_chain: float = 0.5):
    """Parent arrays and tree offsets of a batch of draft trees drawn with
    draw_tree (rules per tree or one for all)."""
    rng = np.random.default_rng([seed, 17])
    S = len(tree_sizes)
    rules = [rules] * S if isinstance(rules, str) else list(rules)
    par = [draw_tree(rng, int(b), r, p_chain) for b, r in zip(tree_sizes, rules)]
    offsets = np.zeros(S + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(tree_sizes)
    parents = (np.concatenate(par).astype(np.int32) if S
               else np.zeros(0, np.int32))
    return parents, offsets


def standard_workload(name: str, kv_format: str = "bf16",
                      head_dim: int = 128) -> Workload:
    """One of the standard workloads; kv_format / head_dim give the same
    workload with an FP8 E4M3 cache or head dimension 64 (the name gets a
    suffix, e.g. "qwen3-8b-b256-p4k+e4m3+d64")."""
    seed, kw = STANDARD[name]
    full = name + ("" if kv_format == "bf16" else "+" + kv_format) + \
        ("" if head_dim == 128 else f"+d{head_dim}")
    return make_workload(seed, name=full, kv_format=kv_format,
                         head_dim=head_dim, **kw)
