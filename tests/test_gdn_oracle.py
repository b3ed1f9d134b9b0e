"""Pins of the Gated DeltaNet tree-verification oracle (CPU).

* masked triangular form: the oracle's outputs and update vectors equal
  the solution of (I + X) U = beta (V - gamma K S0) over ancestor relations
  and O = gamma Q S0 + Y U, computed here with a dense linear solve (a
  different formulation from the oracle's node-by-node recurrence);
* closed forms: one node; beta = 0 and no decay leaves S0;
* a chain equals one sequential sweep of the recurrence over the tokens;
* a node's output does not depend on its siblings' subtrees;
* the committed state after a path equals gamma_n S0 + sum (gamma_n /
  gamma_j) k_j u_j^T over the path;
* planted mistakes in the oracle make some pin fail.
"""

import numpy as np
import pytest

from oracle import gdn_oracle as T


def _tree(rng, B, p_chain=0.5):
    par = [-1]
    for i in range(1, B):
        par.append(i - 1 if rng.random() < p_chain else int(rng.integers(-1, i)))
    return np.array(par, dtype=np.int32)


def _inputs(rng, B, H=2, dk=8, dv=6):
    q = rng.standard_normal((B, H, dk))
    k = rng.standard_normal((B, H, dk))
    k /= np.linalg.norm(k, axis=2, keepdims=True)
    v = rng.standard_normal((B, H, dv))
    g = -rng.uniform(0.0, 0.5, size=(B, H))
    beta = rng.uniform(0.1, 1.0, size=(B, H))
    S0 = rng.standard_normal((H, dk, dv)) * 0.5
    return q, k, v, g, beta, S0


def _anc(par):
    B = len(par)
    A = np.zeros((B, B), dtype=bool)  # A[i, j]: j is an ancestor-or-self of i
    for i in range(B):
        j = i
        while j >= 0:
            A[i, j] = True
            j = int(par[j])
    return A


def _triangular_form(par, q, k, v, g, beta, S0):
    B, H, _ = q.shape
    A = _anc(par)
    strict = A & ~np.eye(B, dtype=bool)
    G = (A * 1.0) @ g  # [B, H]: sum of log-decays on the root path
    O = np.zeros((B, H, v.shape[2]))
    U = np.zeros_like(O)
    for h in range(H):
        D = np.exp(G[:, h][:, None] - G[:, h][None, :])
        X = np.where(strict, beta[:, h][:, None] * D * (k[:, h] @ k[:, h].T), 0.0)
        R = beta[:, h][:, None] * (v[:, h] - np.exp(G[:, h])[:, None] * (k[:, h] @ S0[h]))
        U[:, h] = np.linalg.solve(np.eye(B) + X, R)
        Y = np.where(A, D * (q[:, h] @ k[:, h].T), 0.0)
        O[:, h] = np.exp(G[:, h])[:, None] * (q[:, h] @ S0[h]) + Y @ U[:, h]
    return O, U


def pin_triangular_form():
    rng = np.random.default_rng(41)
    for trial in range(25):
        B = int(rng.integers(1, 14))
        par = _tree(rng, B, p_chain=float(rng.uniform(0, 1)))
        x = _inputs(rng, B)
        o, u = T.gdn_tree_verify(par, *x)
        O, U = _triangular_form(par, *x)
        assert np.allclose(o, O, atol=1e-10, rtol=1e-10)
        assert np.allclose(u, U, atol=1e-10, rtol=1e-10)


def pin_closed_forms():
    rng = np.random.default_rng(42)
    q, k, v, g, beta, S0 = _inputs(rng, 1)
    o, u = T.gdn_tree_verify(np.array([-1]), q, k, v, g, beta, S0)
    for h in range(2):
        a = np.exp(g[0, h])
        S1 = a * (np.eye(8) - beta[0, h] * np.outer(k[0, h], k[0, h])) @ S0[h] \
            + beta[0, h] * np.outer(k[0, h], v[0, h])
        assert np.allclose(o[0, h], S1.T @ q[0, h], atol=1e-12)
    # no write and no decay: every node reads S0
    B = 9
    par = _tree(rng, B)
    q, k, v, g, beta, S0 = _inputs(rng, B)
    o, _ = T.gdn_tree_verify(par, q, k, v, np.zeros_like(g),
                             np.zeros_like(beta), S0)
    for h in range(2):
        assert np.allclose(o[:, h], q[:, h] @ S0[h], atol=1e-12)


def pin_chain_is_one_sweep():
    rng = np.random.default_rng(43)
    B = 11
    par = np.arange(-1, B - 1, dtype=np.int32)
    q, k, v, g, beta, S0 = _inputs(rng, B)
    o, _ = T.gdn_tree_verify(par, q, k, v, g, beta, S0)
    for h in range(2):
        S = S0[h].copy()
        for t in range(B):
            S = np.exp(g[t, h]) * (S - beta[t, h] * np.outer(k[t, h], k[t, h] @ S)) \
                + beta[t, h] * np.outer(k[t, h], v[t, h])
            assert np.allclose(o[t, h], S.T @ q[t, h], atol=1e-12)


def pin_siblings_do_not_matter():
    rng = np.random.default_rng(44)
    B = 8
    par = _tree(rng, B)
    x = _inputs(rng, B + 5)
    o_small, _ = T.gdn_tree_verify(par, *(a[:B] for a in x[:5]), x[5])
    # five more nodes hanging under random nodes of the tree
    par_big = np.concatenate([par, [int(rng.integers(-1, B + i)) for i in range(5)]])
    o_big, _ = T.gdn_tree_verify(par_big.astype(np.int32), *x)
    assert np.allclose(o_big[:B], o_small, atol=1e-12)


def pin_commit():
    rng = np.random.default_rng(45)
    for _ in range(10):
        B = int(rng.integers(1, 12))
        par = _tree(rng, B)
        q, k, v, g, beta, S0 = _inputs(rng, B)
        _, u = T.gdn_tree_verify(par, q, k, v, g, beta, S0)
        last = int(rng.integers(-1, B))
        S = T.gdn_commit_tree(par, k, v, g, beta, S0, last)
        want = S0.copy()
        if last >= 0:
            path, j = [], last
            while j >= 0:
                path.append(j)
                j = int(par[j])
            Gn = g[path].sum(axis=0)
            for h in range(2):
                want[h] = np.exp(Gn[h]) * S0[h]
                for j in path:
                    # decay from j to the end of the path
                    Gj = sum(g[t, h] for t in path if t <= j and _anc(par)[j, t])
                    want[h] += np.exp(Gn[h] - Gj) * np.outer(k[j, h], u[j, h])
        assert np.allclose(S, want, atol=1e-10)


PINS = [pin_triangular_form, pin_closed_forms, pin_chain_is_one_sweep,
        pin_siblings_do_not_matter, pin_commit]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_gdn_pin(pin):
    pin()


# ---- planted mistakes -----------------------------------------------------

def _mutant(kind):
    def verify(parents_local, q, k, v, g, beta, S0):
        q, k, v, g, beta, S0 = (np.asarray(a, np.float64)
                                for a in (q, k, v, g, beta, S0))
        B, H, _ = q.shape
        o = np.zeros((B, H, v.shape[2]))
        u = np.zeros_like(o)
        for i in range(B):
            for h in range(H):
                S = S0[h].copy()
                path = (list(range(i + 1)) if kind == "index_causal"
                        else T._path(parents_local, i))
                for t in path:
                    a, bt, kt = np.exp(g[t, h]), beta[t, h], k[t, h]
                    if t == i:
                        u[i, h] = bt * (v[t, h] - a * (S.T @ kt))
                        S_before = S.copy()
                    if kind == "write_not_decayed":
                        S = a * S - bt * np.outer(kt, kt @ S) + bt * np.outer(kt, v[t, h])
                    elif kind == "delta_sign":
                        S = a * (S + bt * np.outer(kt, kt @ S)) + bt * np.outer(kt, v[t, h])
                    else:
                        S = a * (S - bt * np.outer(kt, kt @ S)) + bt * np.outer(kt, v[t, h])
                o[i, h] = (S_before if kind == "read_before_write" else S).T @ q[i, h]
        return o, u
    return verify


@pytest.mark.parametrize("kind", ["index_causal", "write_not_decayed",
                                  "delta_sign", "read_before_write"])
def test_gdn_pins_catch_planted_mistake(kind, monkeypatch):
    monkeypatch.setattr(T, "gdn_tree_verify", _mutant(kind))
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0
