"""Pins of the acceptance / KV-commit oracle (CPU).

* golden: hand-derived cases in tests/golden/accept_tiny.json;
* brute force: every parent array with B <= 5 and random binary tokens,
  against a top-down enumeration of all root paths (a different traversal
  from the oracle's bottom-up walk);
* greedy: with distinct tokens among siblings the result is the usual walk
  that follows the one matching child;
* commit: copying in increasing j equals copying from a snapshot (so the
  order of copies cannot matter), accepted rows land at P_s + j, every
  other position is unchanged;
* planted mistakes in the oracle make some pin fail.
"""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import accept_oracle as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accept_tiny.json")


def _golden():
    return json.load(open(GOLDEN))["cases"]


def pin_golden():
    for c in _golden():
        path, bonus = A.accept_tree(np.array(c["parents"], dtype=np.int32),
                                    np.array(c["draft"], dtype=np.int32),
                                    np.array(c["target"], dtype=np.int32),
                                    c["root_token"])
        assert path == c["accept"], c["name"]
        assert bonus == c["bonus"], c["name"]


def _all_paths_top_down(parents):
    """Every root path, enumerated from the roots down."""
    children = {}
    for i, p in enumerate(parents):
        children.setdefault(int(p), []).append(i)
    out = []

    def rec(node, path):
        path = path + [node]
        out.append(path)
        for c in children.get(node, []):
            rec(c, path)

    for r in children.get(-1, []):
        rec(r, [])
    return out


def _brute(parents, draft, target, root_token):
    best = []
    for path in _all_paths_top_down(parents):
        want, ok = root_token, True
        for n in path:
            ok = ok and int(draft[n]) == want
            want = int(target[n])
        if ok and (len(path) > len(best) or
                   (len(path) == len(best) and path[-1] < best[-1])):
            best = path
    bonus = int(target[best[-1]]) if best else int(root_token)
    return best, bonus


def pin_brute_force():
    rng = np.random.default_rng(11)
    for B in range(0, 6):
        for parents in itertools.product(*[range(-1, i) for i in range(B)]):
            parents = np.array(parents, dtype=np.int32)
            for _ in range(3):
                draft = rng.integers(0, 2, size=B)
                target = rng.integers(0, 2, size=B)
                root = int(rng.integers(0, 2))
                assert A.accept_tree(parents, draft, target, root) == \
                    _brute(parents, draft, target, root)


def pin_greedy_with_distinct_siblings():
    rng = np.random.default_rng(12)
    for _ in range(300):
        B = int(rng.integers(1, 40))
        parents = np.array([-1] + [int(rng.integers(0, i)) for i in
                                   range(1, B)], dtype=np.int32)
        children = {}
        for i, p in enumerate(parents):
            children.setdefault(int(p), []).append(i)
        draft = np.zeros(B, dtype=np.int32)
        for p, ch in children.items():  # distinct tokens among siblings
            for t, c in zip(rng.permutation(50)[:len(ch)], ch):
                draft[c] = t
        target = np.array([draft[children[i][int(rng.integers(0, len(children[i])))]]
                           if i in children and rng.random() < 0.8
                           else int(rng.integers(0, 50)) for i in range(B)],
                          dtype=np.int32)
        root = int(draft[0]) if rng.random() < 0.9 else 99
        cur, want, path = -1, root, []
        while True:  # follow the single matching child
            nxt = [c for c in children.get(cur, []) if draft[c] == want]
            if not nxt:
                break
            cur = nxt[0]
            path.append(cur)
            want = int(target[cur])
        bonus = want
        assert A.accept_tree(parents, draft, target, root) == (path, bonus)


def _commit_case(seed):
    rng = np.random.default_rng(seed)
    S, page = 3, 4
    P = rng.integers(0, 20, size=S)
    B = rng.integers(1, 12, size=S)
    pages = [int(np.ceil((P[s] + B[s]) / page)) for s in range(S)]
    num_pages = sum(pages) + 2
    perm = rng.permutation(num_pages)
    table = np.full((S, max(pages)), -1, dtype=np.int32)
    o = 0
    for s in range(S):
        table[s, :pages[s]] = perm[o:o + pages[s]]
        o += pages[s]
    k = rng.integers(0, 1 << 16, size=(num_pages, page, 2, 8)).astype(np.uint16)
    v = rng.integers(0, 1 << 16, size=(num_pages, page, 2, 8)).astype(np.uint16)
    lens = np.zeros(S, dtype=np.int32)
    nodes = np.full((S, 12), -1, dtype=np.int32)
    for s in range(S):
        tau = int(rng.integers(0, B[s] + 1))
        path = sorted(rng.choice(B[s], size=tau, replace=False).tolist())
        lens[s] = tau
        nodes[s, :tau] = path
    return k, v, table, P, lens, nodes, page


def pin_commit_semantics():
    for seed in range(20):
        k, v, table, P, lens, nodes, page = _commit_case(seed)
        k2, v2 = A.commit_kv(k, v, table, P, lens, nodes)
        # snapshot semantics: read every source from the original cache
        ks, vs = k.copy(), v.copy()
        touched = set()
        for s in range(len(P)):
            for j in range(lens[s]):
                src, dst = P[s] + nodes[s, j], P[s] + j
                sp, ss = table[s, src // page], src % page
                dp, ds = table[s, dst // page], dst % page
                ks[dp, ds] = k[sp, ss]
                vs[dp, ds] = v[sp, ss]
                touched.add((int(dp), int(ds)))
        assert np.array_equal(k2, ks) and np.array_equal(v2, vs)
        for p_ in range(k.shape[0]):
            for sl in range(page):
                if (p_, sl) not in touched:
                    assert np.array_equal(k2[p_, sl], k[p_, sl])


PINS = [pin_golden, pin_brute_force, pin_greedy_with_distinct_siblings,
        pin_commit_semantics]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_accept_pin(pin):
    pin()


def _largest_end(parents_local, draft, target, root_token):
    """tie-break on the largest end node"""
    m = A._node_matches(parents_local, draft, target, root_token)
    best, bd = -1, 0
    for i in range(len(parents_local)):
        k, ok, d = i, True, 0
        while k >= 0:
            ok = ok and m[k]
            d += 1
            k = int(parents_local[k])
        if ok and d >= bd:
            best, bd = i, d
    if best < 0:
        return [], int(root_token)
    path, k = [], best
    while k >= 0:
        path.append(k)
        k = int(parents_local[k])
    return path[::-1], int(target[best])


def _self_match(parents_local, draft, target, root_token):
    """compares a node's draft token with the target's token after itself"""
    return [int(draft[i]) == (root_token if p < 0 else int(target[i]))
            for i, p in enumerate(parents_local)]


MUTANTS = {
    "tie_break_largest": ("accept_tree", _largest_end),
    "match_against_self": ("_node_matches", _self_match),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_accept_pins_catch_planted_mistake(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(A, attr, fn)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, IndexError, KeyError):
            failed += 1
    assert failed > 0, f"no pin caught mutant {mutant}"


def _commit_shifted(k_cache, v_cache, page_table, prefix_lens, lens, nodes):
    """writes accepted row j to position P_s + j + 1"""
    k, v = k_cache.copy(), v_cache.copy()
    page = k.shape[1]
    for s in range(len(prefix_lens)):
        for j in range(int(lens[s])):
            src = prefix_lens[s] + nodes[s, j]
            dst = prefix_lens[s] + j + 1
            dp = page_table[s, dst // page] if dst // page < page_table.shape[1] else -1
            if dp < 0:
                continue
            sp = page_table[s, src // page]
            k[dp, dst % page] = k[sp, src % page]
            v[dp, dst % page] = v[sp, src % page]
    return k, v


def _commit_snapshot_missing(k_cache, v_cache, page_table, prefix_lens, lens,
                             nodes):
    """copies in decreasing j (reads rows an earlier copy overwrote)"""
    k, v = k_cache.copy(), v_cache.copy()
    page = k.shape[1]
    for s in range(len(prefix_lens)):
        for j in reversed(range(int(lens[s]))):
            src, dst = prefix_lens[s] + nodes[s, j], prefix_lens[s] + j
            sp, dp = page_table[s, src // page], page_table[s, dst // page]
            k[dp, dst % page] = k[sp, src % page]
            v[dp, dst % page] = v[sp, src % page]
    return k, v


@pytest.mark.parametrize("mutant", [_commit_shifted, _commit_snapshot_missing],
                         ids=lambda f: f.__name__)
def test_commit_pin_catches_planted_mistake(mutant, monkeypatch):
    monkeypatch.setattr(A, "commit_kv", mutant)
    with pytest.raises(AssertionError):
        pin_commit_semantics()
