"""CPU oracle for tree acceptance and KV commit, the step after the
verification attention.

TEST INFRASTRUCTURE ONLY.  Only the tests and the benchmark's CPU baseline
may import this module; the HIP library never calls it and shares no code
with it.

What the pages fix: after the target model has scored every draft-tree
node in one pass, decoding keeps the accepted prefix of the tree, tau
tokens per step (JETFLOW, gist.science 2606.18394, section 4 reports
tau ~= 10.7 accepted tokens at a 256-token budget), and the recurrent
state / cache commit is deferred until the accepted branch is known
(DFlash-TfM, gist.science 2607.06763, method section on rollback-free
verification: the state commit is delayed to the next decoding iteration,
once the accepted branch is known).

Readings of what the pages leave open (also listed in the design notes):
* Acceptance is exact-match on the target's choices: the target supplies,
  for every node i, the token it would emit after node i (target[i]) and,
  per sequence, the token it would emit after the prefix (root_token).
  Node i "matches" when its draft token equals the target's token after
  its parent (root_token for a root).  The accepted path is the longest
  root-to-node path all of whose nodes match; among equally long ones the
  one ending at the smallest node index.  tau is its length, the bonus
  token is the target's token after its last node (root_token if tau = 0).
  With distinct tokens among siblings this is the usual greedy walk.
* Commit: the K/V rows of the accepted nodes, cached at logical positions
  P_s + n_j (node n_j at position P_s + n_j, as in the attention), are
  moved to positions P_s + j, j = 0 .. tau-1, through the page table; all
  other positions keep their contents.  Since n_j >= j, copying in
  increasing j never reads a row that an earlier copy overwrote.
"""

from __future__ import annotations

from typing import List, Tuple

import numpy as np


def _node_matches(parents_local: np.ndarray, draft: np.ndarray,
                  target: np.ndarray, root_token: int) -> List[bool]:
    out = []
    for i, p in enumerate(parents_local):
        want = root_token if p < 0 else int(target[p])
        out.append(int(draft[i]) == want)
    return out


def accept_tree(parents_local: np.ndarray, draft: np.ndarray,
                target: np.ndarray, root_token: int) -> Tuple[List[int], int]:
    """Accepted path (local node indices, root first) and bonus token of
    one tree: walk every node's root path; keep the deepest fully matching
    node, the smallest index on ties."""
    matches = _node_matches(parents_local, draft, target, root_token)
    best, best_depth = -1, 0
    for i in range(len(parents_local)):
        path, ok, k = [], True, i
        while k >= 0:
            ok = ok and matches[k]
            path.append(k)
            k = int(parents_local[k])
        if ok and len(path) > best_depth:
            best, best_depth = i, len(path)
    if best < 0:
        return [], int(root_token)
    path, k = [], best
    while k >= 0:
        path.append(k)
        k = int(parents_local[k])
    return path[::-1], int(target[best])


def accept(parents: np.ndarray, tree_offsets: np.ndarray, draft: np.ndarray,
           target: np.ndarray, root_tokens: np.ndarray, max_nodes: int):
    """Per sequence: (accept_len [S], accept_nodes [S, max_nodes] with -1
    padding, bonus [S])."""
    S = len(tree_offsets) - 1
    lens = np.zeros(S, dtype=np.int32)
    nodes = np.full((S, max(max_nodes, 1)), -1, dtype=np.int32)
    bonus = np.zeros(S, dtype=np.int32)
    for s in range(S):
        a, b = int(tree_offsets[s]), int(tree_offsets[s + 1])
        path, bt = accept_tree(parents[a:b], draft[a:b], target[a:b],
                               int(root_tokens[s]))
        lens[s] = len(path)
        nodes[s, :len(path)] = path
        bonus[s] = bt
    return lens, nodes, bonus


def commit_kv(k_cache: np.ndarray, v_cache: np.ndarray,
              page_table: np.ndarray, prefix_lens: np.ndarray,
              accept_len: np.ndarray, accept_nodes: np.ndarray):
    """Copies of the caches after the commit ([num_pages, page_size, ...]
    arrays of any element type)."""
    k = k_cache.copy()
    v = v_cache.copy()
    page_size = k.shape[1]
    for s in range(len(prefix_lens)):
        P = int(prefix_lens[s])
        for j in range(int(accept_len[s])):
            src, dst = P + int(accept_nodes[s, j]), P + j
            sp, ss = int(page_table[s, src // page_size]), src % page_size
            dp, ds = int(page_table[s, dst // page_size]), dst % page_size
            k[dp, ds] = k[sp, ss]
            v[dp, ds] = v[sp, ss]
    return k, v
