"""CPU oracle for rollback-free tree verification of Gated DeltaNet layers.

TEST INFRASTRUCTURE ONLY.  Only the tests and the benchmark's CPU baseline
may import this module; the HIP library never calls it and shares no code
with it.

What the pages fix (DFlash-TfM, gist.science 2607.06763, method section 3,
rollback-free tree verification for GDN): a GDN layer updates its state as
    S_t = alpha_t (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,
the tree is sorted topologically, verification is a masked triangular solve
(I + X) U = beta V over ancestor relations, and the state commit waits until
the accepted branch is known.

Readings of what the pages leave open (also listed in the design notes):
* Every draft node i, per head, carries q_i, k_i (d_k), v_i (d_v), a decay
  alpha_i = exp(g_i) (g_i <= 0 given) and beta_i.  Node i's state S_i is
  the recurrence run along its root-to-node path, starting from the
  committed state S_0 (d_k x d_v) of the prefix; siblings and descendants
  play no part.  The output is o_i = S_i^T q_i (after node i's update).
* u_i = beta_i (v_i - alpha_i S_parent(i)^T k_i) is node i's update vector
  (S_i = alpha_i S_parent(i) + k_i u_i^T); it depends on the path to i only,
  and is what the deferred commit needs.
* Commit: after acceptance, the new committed state is the state of the
  last accepted node, S_n = gamma_n S_0 + sum over the path of
  (gamma_n / gamma_j) k_j u_j^T, gamma the product of alphas along the path.

This oracle runs the recurrence itself, node by node, in float64 on the
given (bf16-rounded) inputs.
"""

from __future__ import annotations

import numpy as np


def _path(parents_local, i):
    p = []
    while i >= 0:
        p.append(i)
        i = int(parents_local[i])
    return p[::-1]


def gdn_tree_verify(parents_local, q, k, v, g, beta, S0):
    """One tree.  q, k [B, H, dk]; v [B, H, dv]; g, beta [B, H];
    S0 [H, dk, dv].  Returns (o [B, H, dv], u [B, H, dv]) in float64."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    g, beta = np.asarray(g, np.float64), np.asarray(beta, np.float64)
    S0 = np.asarray(S0, np.float64)
    B, H, _ = q.shape
    dv = v.shape[2]
    o = np.zeros((B, H, dv))
    u = np.zeros((B, H, dv))
    for i in range(B):
        for h in range(H):
            S = S0[h].copy()
            for t in _path(parents_local, i):
                a, bt, kt = np.exp(g[t, h]), beta[t, h], k[t, h]
                if t == i:
                    u[i, h] = bt * (v[t, h] - a * (S.T @ kt))
                # the recurrence as the pages write it
                S = a * (S - bt * np.outer(kt, kt @ S)) + bt * np.outer(kt, v[t, h])
            o[i, h] = S.T @ q[i, h]
    return o, u


def gdn_verify(parents, tree_offsets, q, k, v, g, beta, S0):
    """All sequences: node arrays over N nodes, S0 [S, H, dk, dv]."""
    N, H, _ = q.shape
    o = np.zeros((N, H, v.shape[2]))
    u = np.zeros_like(o)
    for s in range(len(tree_offsets) - 1):
        a, b = int(tree_offsets[s]), int(tree_offsets[s + 1])
        o[a:b], u[a:b] = gdn_tree_verify(parents[a:b], q[a:b], k[a:b],
                                         v[a:b], g[a:b], beta[a:b], S0[s])
    return o, u


def gdn_commit_tree(parents_local, k, v, g, beta, S0, last):
    """State after the accepted path ending at local node `last` (-1: none):
    the recurrence along that path from S0; [H, dk, dv] float64."""
    S = np.asarray(S0, np.float64).copy()
    k, v, g, beta = (np.asarray(x, np.float64) for x in (k, v, g, beta))
    if last < 0:
        return S
    for t in _path(parents_local, last):
        for h in range(S.shape[0]):
            a, bt, kt = np.exp(g[t, h]), beta[t, h], k[t, h]
            S[h] = a * (S[h] - bt * np.outer(kt, kt @ S[h])) + \
                bt * np.outer(kt, v[t, h])
    return S
