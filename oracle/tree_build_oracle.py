"""CPU oracle for draft-tree construction, the step before the verification
attention.

TEST INFRASTRUCTURE ONLY.  Only the tests and the benchmark's CPU baseline
may import this module; the HIP library never calls it and shares no code
with it.

What the pages fix: the drafting head emits logits for every tree depth in
one pass; a branch score, by default the cumulative draft log-probability,
ranks the nodes, and best-first expansion builds the tree up to a token
budget such as 256 (JETFLOW, gist.science 2606.18394, section 2, bullet on
tree construction).  DFlash-TfM (gist.science 2607.06763, method section 2,
tree construction) takes the w best nodes off the candidate heap at once and
expands them together, which builds a B-node tree in ceil(B / w) sequential
steps.

Readings of what the pages leave open (also listed in the design notes):
* Inputs per sequence: for depths d = 1 .. D the head's top-K candidates,
  log-probabilities logp[d-1][0..K-1] (fp32, each row non-increasing, as a
  top-k returns them) and their tokens.  The same per-depth candidates
  serve every parent at that depth (the head's per-depth output).
* A candidate is (parent, rank j) at depth d; its score is the parent's
  score plus logp[d-1][j], added in fp32; depth-1 candidates have the
  prefix (score 0) as parent and no parent node (-1).
* Best-first: the candidate heap starts with the K depth-1 candidates.  A
  step removes the best min(w, B - size) candidates, appends them to the
  tree in that order (node index = order of insertion, so parents come
  first), then puts the K children of each of them, in insertion order,
  into the heap (none for a node at depth D).  w = 1 is strict best-first.
* Order of candidates: higher score first; equal scores by the parent's
  node index (the prefix as -1 first), then by rank j.  That is the order in
  which an eager heap would have created them.
"""

from __future__ import annotations

import heapq
from typing import Dict

import numpy as np


def build_tree(logp: np.ndarray, tokens: np.ndarray, budget: int,
               width: int) -> Dict[str, np.ndarray]:
    """One sequence: logp, tokens [D][K].  Returns parents, tokens, depths,
    scores (fp32) of the nodes in insertion order."""
    logp = np.asarray(logp, dtype=np.float32)
    D, K = logp.shape
    heap = []
    for j in range(K):
        sc = np.float32(logp[0, j])
        heapq.heappush(heap, (-float(sc), -1, j, 1, sc))
    parents, toks, depths, scores = [], [], [], []
    while len(parents) < budget and heap:
        take = min(width, budget - len(parents), len(heap))
        popped = [heapq.heappop(heap) for _ in range(take)]
        first = len(parents)
        for _, par, j, d, sc in popped:
            parents.append(par)
            toks.append(int(tokens[d - 1, j]))
            depths.append(d)
            scores.append(sc)
        for k, (_, par, j, d, sc) in enumerate(popped):
            if d >= D:
                continue
            v = first + k
            for c in range(K):
                csc = np.float32(sc + np.float32(logp[d, c]))
                heapq.heappush(heap, (-float(csc), v, c, d + 1, csc))
    return {"parents": np.array(parents, dtype=np.int32),
            "tokens": np.array(toks, dtype=np.int32),
            "depths": np.array(depths, dtype=np.int32),
            "scores": np.array(scores, dtype=np.float32)}


def build_trees(logp: np.ndarray, tokens: np.ndarray, budget: int,
                width: int) -> Dict[str, np.ndarray]:
    """All sequences: logp, tokens [S][D][K].  Returns [S][budget] arrays
    padded with parent -1, token -1, depth 0, score 0 past each tree's size,
    and the sizes [S]."""
    S = logp.shape[0]
    out = {"parents": np.full((S, budget), -1, dtype=np.int32),
           "tokens": np.full((S, budget), -1, dtype=np.int32),
           "depths": np.zeros((S, budget), dtype=np.int32),
           "scores": np.zeros((S, budget), dtype=np.float32),
           "sizes": np.zeros(S, dtype=np.int32)}
    for s in range(S):
        t = build_tree(logp[s], tokens[s], budget, width)
        n = len(t["parents"])
        out["sizes"][s] = n
        for k in ("parents", "tokens", "depths", "scores"):
            out[k][s, :n] = t[k]
    return out
