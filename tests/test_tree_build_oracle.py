"""Pins of the draft-tree construction oracle (CPU).

* golden: hand-derived cases in tests/golden/tree_build_tiny.json;
* brute force (w = 1): every node of the full tree (all paths up to depth
  D) is enumerated and ranked by its fp32 path score; the oracle's tree is
  the top B of them;
* rounds (w > 1): an independent simulation that keeps the candidates in a
  plain list and sorts it at every step gives the same tree;
* closed forms: one depth gives the row's first min(B, K) candidates; K = 1
  gives a chain; sizes are min(B, number of nodes of the full tree);
* planted mistakes in the oracle make some pin fail.
"""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import tree_build_oracle as T

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "tree_build_tiny.json")


def pin_golden():
    for c in json.load(open(GOLDEN))["cases"]:
        r = T.build_tree(np.array(c["logp"], np.float32),
                         np.array(c["tokens"], np.int32), c["budget"],
                         c["width"])
        assert r["parents"].tolist() == c["parents"], c["name"]
        assert r["tokens"].tolist() == c["out_tokens"], c["name"]
        assert r["depths"].tolist() == c["depths"], c["name"]
        assert r["scores"].tolist() == c["scores"], c["name"]


def _draw(rng, D, K):
    """sorted (non-increasing) log-probs and tokens that name (depth, rank)"""
    lp = -np.sort(rng.exponential(1.0, size=(D, K)).astype(np.float32), axis=1)
    lp = lp.astype(np.float32)
    tok = (np.arange(D)[:, None] * 100 + np.arange(K)[None, :]).astype(np.int32)
    return lp, tok


def _paths(r, tok):
    """each node's root path as a tuple of (depth, rank) from its tokens"""
    out = []
    for i in range(len(r["parents"])):
        p, k = [], i
        while k >= 0:
            t = int(r["tokens"][k])
            p.append((t // 100, t % 100))
            k = int(r["parents"][k])
        out.append(tuple(p[::-1]))
    return out


def pin_brute_force_strict():
    rng = np.random.default_rng(21)
    for trial in range(60):
        D = int(rng.integers(1, 5))
        K = int(rng.integers(1, 4))
        lp, tok = _draw(rng, D, K)
        allp = []
        for d in range(1, D + 1):
            for path in itertools.product(range(K), repeat=d):
                sc = np.float32(0)
                for t, j in enumerate(path):
                    sc = np.float32(sc + lp[t, j]) if t else np.float32(lp[0, j])
                allp.append((float(sc), tuple((t, j) for t, j in enumerate(path))))
        scores = [s for s, _ in allp]
        if len(set(scores)) != len(scores):
            continue  # ties: the ranking below would need the tie rule
        allp.sort(key=lambda x: -x[0])
        B = int(rng.integers(1, len(allp) + 3))
        r = T.build_tree(lp, tok, B, 1)
        want = allp[:B]
        assert len(r["parents"]) == len(want)
        assert set(_paths(r, tok)) == {p for _, p in want}
        assert r["scores"].tolist() == [s for s, _ in want]  # insertion order


def _rounds_by_sorting(lp, tok, B, w):
    D, K = lp.shape
    cand = [(np.float32(lp[0, j]), -1, j, 1) for j in range(K)]
    par, toks, deps, scs = [], [], [], []
    while len(par) < B and cand:
        cand.sort(key=lambda c: (-float(c[0]), c[1], c[2]))
        take = min(w, B - len(par), len(cand))
        step, cand = cand[:take], cand[take:]
        base = len(par)
        for sc, p, j, d in step:
            par.append(p); toks.append(int(tok[d - 1, j])); deps.append(d)
            scs.append(float(sc))
        for k, (sc, p, j, d) in enumerate(step):
            if d < D:
                cand += [(np.float32(sc + lp[d, c]), base + k, c, d + 1)
                         for c in range(K)]
    return par, toks, deps, scs


def pin_rounds_independent():
    rng = np.random.default_rng(22)
    for trial in range(80):
        D = int(rng.integers(1, 7))
        K = int(rng.integers(1, 5))
        lp, tok = _draw(rng, D, K)
        if trial % 3 == 0:  # force ties
            lp = np.round(lp * 2) / 2
            lp = -np.sort(-lp, axis=1).astype(np.float32)
        B = int(rng.integers(1, 60))
        w = int(rng.integers(1, 9))
        r = T.build_tree(lp, tok, B, w)
        par, toks, deps, scs = _rounds_by_sorting(lp, tok, B, w)
        assert r["parents"].tolist() == par
        assert r["tokens"].tolist() == toks
        assert r["depths"].tolist() == deps
        assert r["scores"].tolist() == scs


def pin_closed_forms():
    rng = np.random.default_rng(23)
    for _ in range(20):
        K = int(rng.integers(1, 9))
        lp, tok = _draw(rng, 1, K)
        B = int(rng.integers(1, 12))
        for w in (1, 3, 64):
            r = T.build_tree(lp, tok, B, w)
            n = min(B, K)
            assert r["parents"].tolist() == [-1] * n
            assert r["tokens"].tolist() == tok[0, :n].tolist()
        D = int(rng.integers(1, 9))
        lp, tok = _draw(rng, D, 1)
        r = T.build_tree(lp, tok, B, 1)
        n = min(B, D)
        assert r["parents"].tolist() == list(range(-1, n - 1))
        assert r["depths"].tolist() == list(range(1, n + 1))
    # sizes cap at the full tree
    lp, tok = _draw(rng, 3, 2)
    assert len(T.build_tree(lp, tok, 100, 5)["parents"]) == 2 + 4 + 8


PINS = [pin_golden, pin_brute_force_strict, pin_rounds_independent,
        pin_closed_forms]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_tree_build_pin(pin):
    pin()


def test_batched_padding():
    rng = np.random.default_rng(24)
    lp = np.stack([_draw(rng, 2, 2)[0], _draw(rng, 3, 3)[0][:2, :2]])
    tok = np.stack([_draw(rng, 2, 2)[1]] * 2)
    out = T.build_trees(lp, tok, 10, 2)
    assert out["sizes"].tolist() == [6, 6]
    assert (out["parents"][:, 6:] == -1).all() and (out["depths"][:, 6:] == 0).all()


# ---- planted mistakes -----------------------------------------------------

_orig = T.build_tree


def _mut_ties_reversed(logp, tokens, budget, width):
    """equal scores taken by the highest parent index first"""
    import heapq
    logp = np.asarray(logp, dtype=np.float32)
    D, K = logp.shape
    heap = [(-float(logp[0, j]), 1, -j, 1, np.float32(logp[0, j]), -1)
            for j in range(K)]
    heapq.heapify(heap)
    par, tk, dp, sc_ = [], [], [], []
    while len(par) < budget and heap:
        take = min(width, budget - len(par), len(heap))
        popped = [heapq.heappop(heap) for _ in range(take)]
        first = len(par)
        for _, _, nj, d, sc, p in popped:
            par.append(p); tk.append(int(tokens[d - 1, -nj])); dp.append(d)
            sc_.append(sc)
        for k, (_, _, nj, d, sc, p) in enumerate(popped):
            if d < D:
                for c in range(K):
                    csc = np.float32(sc + logp[d, c])
                    heapq.heappush(heap, (-float(csc), -(first + k), -c, d + 1,
                                          csc, first + k))
    return {"parents": np.array(par, np.int32), "tokens": np.array(tk, np.int32),
            "depths": np.array(dp, np.int32), "scores": np.array(sc_, np.float32)}


def _mut_children_now(logp, tokens, budget, width):
    """children enter the heap as soon as their parent is taken"""
    return _orig(logp, tokens, budget, 1)


def _mut_float64(logp, tokens, budget, width):
    """path scores accumulated in float64"""
    lp = np.asarray(logp, dtype=np.float64)
    r = _rounds_by_sorting_f64(lp, tokens, budget, width)
    return r


def _rounds_by_sorting_f64(lp, tok, B, w):
    D, K = lp.shape
    cand = [(lp[0, j], -1, j, 1) for j in range(K)]
    par, toks, deps, scs = [], [], [], []
    while len(par) < B and cand:
        cand.sort(key=lambda c: (-c[0], c[1], c[2]))
        take = min(w, B - len(par), len(cand))
        step, cand = cand[:take], cand[take:]
        base = len(par)
        for sc, p, j, d in step:
            par.append(p); toks.append(int(tok[d - 1, j])); deps.append(d)
            scs.append(sc)
        for k, (sc, p, j, d) in enumerate(step):
            if d < D:
                cand += [(sc + lp[d, c], base + k, c, d + 1) for c in range(K)]
    return {"parents": np.array(par, np.int32), "tokens": np.array(toks, np.int32),
            "depths": np.array(deps, np.int32), "scores": np.array(scs)}


@pytest.mark.parametrize("mutant", [_mut_ties_reversed, _mut_children_now,
                                    _mut_float64], ids=lambda f: f.__name__)
def test_tree_build_pins_catch_planted_mistake(mutant, monkeypatch):
    monkeypatch.setattr(T, "build_tree", mutant)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0
