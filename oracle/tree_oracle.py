"""CPU oracle for tree-causal verification attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this module.  The HIP library
never calls it and shares no code with it.

What it computes is the plain definition, in float64, on the
bf16-rounded inputs:

* Tree-causal mask (JETFLOW, gist.science 2606.18394, section 2
  "Arquitectura Central", bullet on the tree-causal attention mask; the
  Korean page repeats it in its section 2): a draft-tree node attends to
  the whole input prefix and to its ancestors in the tree, never to its
  descendants or to sibling branches.  The branch factorization printed
  under that bullet, q(pi(v)|x) = prod over u in pi(v), fixes "ancestors"
  as the root-to-node path pi(v).  Reading taken here: the node's own
  position is part of its context (ancestor-or-self), so that a pure chain
  is ordinary causal attention, diagonal included.
* Nodes arrive in topological order, parent[i] < i (DFlash-TfM,
  gist.science 2607.06763, section 3 of the method: the tree is
  topologically sorted before verification).
* Attention over that key set is exact softmax attention; the log-sum-exp
  returned is the natural log of the sum of exp(scale * q.k) over the
  allowed keys.

Readings of points the pages leave open (each also listed in the design
notes): node j of sequence s is cached at logical position P_s + j of
that sequence's paged cache; parent indices are local to the sequence and
-1 marks a root (several roots are allowed); q head h reads kv head
h // (Hq / Hkv); masks are little-endian uint64 words, bit j % 64 of word
j // 64 of row i set iff node j is an ancestor-or-self of node i.

Parity pins live in tests/test_oracle_pins.py.
"""

from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Set, Tuple

import numpy as np


# --------------------------------------------------------------------------
# inputs
# --------------------------------------------------------------------------

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exact."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def widen_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3 (e4m3fn) codes (uint8) -> float64, exact, from the
    format's definition: sign bit, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 is subnormal, m/8 * 2^-6; S.1111.111 is NaN; there are
    no infinities (S.1111.110 = 448 is the largest finite value)."""
    b = np.asarray(codes).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6,
                   (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def _check_parents(parents_local: np.ndarray) -> None:
    for i, p in enumerate(parents_local.tolist()):
        if not (-1 <= p < i):
            raise ValueError(f"node {i}: parent {p} outside [-1, {i})")


# --------------------------------------------------------------------------
# ancestor sets and masks
# --------------------------------------------------------------------------

def _ancestor_sets(parents_local: np.ndarray) -> List[Set[int]]:
    """For each node, the set {i, parent(i), parent(parent(i)), ...}.

    Built by walking parent pointers up to a root, node by node (no reuse
    of other nodes' results).
    """
    _check_parents(parents_local)
    out: List[Set[int]] = []
    par = parents_local.tolist()
    for i in range(len(par)):
        s = set()
        j = i
        while j != -1:
            s.add(j)
            j = par[j]
        out.append(s)
    return out


def ancestor_masks(parents: np.ndarray, tree_offsets: np.ndarray,
                   mask_words: int) -> np.ndarray:
    """Per-node ancestor-or-self bitmasks, uint64 [N, mask_words].

    Bit j % 64 of word j // 64 in row i is set iff local node j lies on the
    root-to-node path of local node i.  All other bits are zero.
    """
    parents = np.asarray(parents, dtype=np.int64)
    offs = np.asarray(tree_offsets, dtype=np.int64)
    N = int(offs[-1])
    masks = np.zeros((N, mask_words), dtype=np.uint64)
    for s in range(len(offs) - 1):
        a, b = int(offs[s]), int(offs[s + 1])
        if b - a > 64 * mask_words:
            raise ValueError("mask_words too small for this tree")
        for i, anc in enumerate(_ancestor_sets(parents[a:b])):
            for j in anc:
                masks[a + i, j // 64] |= np.uint64(1) << np.uint64(j % 64)
    return masks


# --------------------------------------------------------------------------
# paged cache gather
# --------------------------------------------------------------------------

def _gather_tokens(cache_bits: np.ndarray, table_row: np.ndarray,
                   num_tokens: int, kv_format: str = "bf16",
                   head_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Logical tokens 0..num_tokens-1 of one sequence -> float64
    [num_tokens, Hkv, d], reading physical page table_row[t // page_size],
    slot t % page_size.  kv_format "bf16" (uint16 bit patterns) or "e4m3"
    (uint8 codes, each kv head's values times head_scale[head])."""
    num_pages, page_size = cache_bits.shape[0], cache_bits.shape[1]
    t = np.arange(num_tokens)
    pages = np.asarray(table_row, dtype=np.int64)[t // page_size]
    if num_tokens and (pages.min() < 0 or pages.max() >= num_pages):
        raise ValueError("page table entry outside the page pool")
    raw = cache_bits[pages, t % page_size]
    if kv_format == "bf16":
        return widen_bf16(raw)
    if kv_format != "e4m3":
        raise ValueError(f"unknown kv_format {kv_format!r}")
    vals = widen_e4m3(raw)
    if head_scale is not None:
        vals = vals * np.asarray(head_scale, np.float64)[None, :, None]
    return vals


def _kv_head_of(h: int, num_q_heads: int, num_kv_heads: int) -> int:
    """GQA grouping: contiguous groups of Hq / Hkv query heads."""
    return h // (num_q_heads // num_kv_heads)


def _allowed_keys(prefix_len: int, anc: Set[int], tree_size: int) -> np.ndarray:
    """Explicit boolean mask row over the prefix_len + tree_size positions."""
    row = np.zeros(prefix_len + tree_size, dtype=bool)
    row[:prefix_len] = True
    for j in anc:
        row[prefix_len + j] = True
    return row


def _masked_softmax_attention(scores: np.ndarray, allowed: np.ndarray,
                              values: np.ndarray
                              ) -> Tuple[np.ndarray, np.ndarray]:
    """rows: softmax over allowed columns of `scores`, applied to `values`.

    Returns (out [R, d], lse [R]) with lse the natural log of the sum of
    exp(score) over the allowed columns.
    """
    s = np.where(allowed, scores, -np.inf)
    m = s.max(axis=1, keepdims=True)
    w = np.where(allowed, np.exp(s - m), 0.0)
    l = w.sum(axis=1, keepdims=True)
    out = (w @ values) / l
    lse = (m + np.log(l))[:, 0]
    return out, lse


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def tree_attention(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray,
                   page_table: np.ndarray, prefix_lens: np.ndarray,
                   tree_offsets: np.ndarray, parents: np.ndarray,
                   scale: float,
                   seq_ids: Optional[Iterable[int]] = None,
                   kv_head_ids: Optional[Iterable[int]] = None,
                   kv_format: str = "bf16",
                   k_scale: Optional[np.ndarray] = None,
                   v_scale: Optional[np.ndarray] = None
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """Tree-causal verification attention, float64.

    q: bf16 bits [N, Hq, d]; k_cache / v_cache: bf16 bits (kv_format
    "bf16") or E4M3 codes with per-kv-head scales k_scale / v_scale
    (kv_format "e4m3") [num_pages, page_size, Hkv, d]; page_table int
    [S, max_pages];
    prefix_lens [S]; tree_offsets [S+1]; parents [N] (local, -1 = root).

    For node i of sequence s and query head h the allowed keys are the
    prefix positions 0..P_s-1 and the tree positions P_s + j for every j on
    the root-to-node path of i (i itself included).

    Returns (out [N, Hq, d], lse [N, Hq]) in float64.  With seq_ids /
    kv_head_ids only those sequences / kv-head groups are computed; the
    other entries are NaN.
    """
    q = np.asarray(q)
    N, Hq, d = q.shape
    Hkv = k_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    G = Hq // Hkv
    offs = np.asarray(tree_offsets, dtype=np.int64)
    prefix = np.asarray(prefix_lens, dtype=np.int64)
    parents = np.asarray(parents, dtype=np.int64)
    S = len(prefix)
    out = np.full((N, Hq, d), np.nan)
    lse = np.full((N, Hq), np.nan)
    seqs = range(S) if seq_ids is None else list(seq_ids)
    groups = range(Hkv) if kv_head_ids is None else list(kv_head_ids)
    for s in seqs:
        a, b = int(offs[s]), int(offs[s + 1])
        B, P = b - a, int(prefix[s])
        if B == 0:
            continue
        anc = _ancestor_sets(parents[a:b])
        allowed_nodes = np.stack([_allowed_keys(P, anc[i], B)
                                  for i in range(B)])          # [B, P+B]
        K = _gather_tokens(k_cache, page_table[s], P + B, kv_format,
                           k_scale)                              # [T, Hkv, d]
        V = _gather_tokens(v_cache, page_table[s], P + B, kv_format,
                           v_scale)
        qs = widen_bf16(q[a:b])                                  # [B, Hq, d]
        for g in groups:
            heads = [h for h in range(Hq)
                     if _kv_head_of(h, Hq, Hkv) == g]
            rows = qs[:, heads, :].reshape(B * len(heads), d)
            allowed = np.repeat(allowed_nodes, len(heads), axis=0)
            scores = scale * (rows @ K[:, g, :].T)
            o, l = _masked_softmax_attention(scores, allowed, V[:, g, :])
            out[a:b, heads, :] = o.reshape(B, len(heads), d)
            lse[a:b, heads] = l.reshape(B, len(heads))
    return out, lse


def workload_attention(wl, **kw):
    """tree_attention on an object with the workload attribute names."""
    return tree_attention(wl.q, wl.k_cache, wl.v_cache, wl.page_table,
                          wl.prefix_lens, wl.tree_offsets, wl.parents,
                          wl.scale, kv_format=wl.kv_format,
                          k_scale=wl.k_scale, v_scale=wl.v_scale, **kw)


def workload_masks(wl, mask_words: Optional[int] = None) -> np.ndarray:
    W = wl.mask_words() if mask_words is None else mask_words
    return ancestor_masks(wl.parents, wl.tree_offsets, W)
