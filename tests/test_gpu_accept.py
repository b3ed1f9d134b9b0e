"""Acceptance and KV commit: HIP path vs the CPU oracle, through the C ABI
(needs a gfx950 GPU).  Bar: bit-exact (accepted lengths, paths with their
-1 padding, bonus tokens; the whole K and V caches byte for byte)."""

import json
import os
import zlib

import numpy as np
import pytest
import torch

import oracle
from gpu_util import device_inputs, say
from tree_masked_attention_amd.workloads import (STANDARD_ORDER, draw_tokens,
                                                 make_workload,
                                                 standard_workload)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "accept_tiny.json")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import tree_masked_attention_amd.api  # noqa: F401  (fails loudly if unbuilt)


def _i32(a, dev="cuda:0"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)


def gpu_accept(parents, offsets, draft, target, root, max_nodes, W=None):
    import tree_masked_attention_amd.api as api
    W = W or api.mask_words_for(max_nodes)
    p, o = _i32(parents), _i32(offsets)
    masks, bad = api.build_mask(p, o, max(max_nodes, 1), W)
    lens, nodes, bonus = api.accept(p, o, masks, _i32(draft), _i32(target),
                                    _i32(root), max_nodes)
    torch.cuda.synchronize()
    return (lens.cpu().numpy(), nodes.cpu().numpy(), bonus.cpu().numpy(),
            bad.cpu().numpy()[:len(offsets) - 1])


def check_accept(parents, offsets, draft, target, root, max_nodes, label,
                 W=None):
    got = gpu_accept(parents, offsets, draft, target, root, max_nodes, W)
    ref = oracle.accept(np.asarray(parents), np.asarray(offsets),
                        np.asarray(draft), np.asarray(target),
                        np.asarray(root), max_nodes)
    S = len(offsets) - 1
    assert np.array_equal(got[0], ref[0]), f"{label}: accept_len"
    assert np.array_equal(got[1], ref[1][:S, :max_nodes]), f"{label}: nodes"
    assert np.array_equal(got[2], ref[2]), f"{label}: bonus"
    say(f"  {label}: tau = {got[0].tolist()[:8]}{' ...' if S > 8 else ''}")
    return got


def test_accept_golden():
    say("[gpu] accept: golden cases")
    for c in json.load(open(GOLDEN))["cases"]:
        B = len(c["parents"])
        got = gpu_accept(c["parents"], [0, B], c["draft"], c["target"],
                         [c["root_token"]], max(B, 1))
        assert got[0][0] == len(c["accept"]), c["name"]
        assert got[1][0, :len(c["accept"])].tolist() == c["accept"], c["name"]
        assert (got[1][0, len(c["accept"]):] == -1).all(), c["name"]
        assert got[2][0] == c["bonus"], c["name"]


ACCEPT_CASES = {
    # (prefix lens, tree sizes, rules, p_chain, vocab, p_agree, extra max)
    "ragged": ([3, 0, 9, 1], [1, 37, 130, 64], "pchain", 0.5, 8, 0.8, 0),
    "deep-chain": ([5], [300], "chain", 0.5, 4, 0.97, 0),
    "star": ([5], [200], "star", 0.5, 3, 0.9, 0),
    "wide-ties": ([1, 2], [100, 90], "wide", 0.0, 2, 0.6, 0),
    "max-1024": ([7], [1024], "pchain", 0.8, 2, 0.95, 0),
    "empty-middle": ([4, 4, 4], [9, 0, 12], "pchain", 0.5, 4, 0.9, 0),
    "spare-columns": ([4, 4], [20, 33], "pchain", 0.5, 4, 0.9, 40),
    "many-seqs": ([2] * 64, [16] * 64, "pchain", 0.5, 4, 0.85, 0),
}


@pytest.mark.parametrize("name", sorted(ACCEPT_CASES))
def test_accept_parity(name):
    pre, sizes, rule, pc, vocab, agree, extra = ACCEPT_CASES[name]
    wl = make_workload(zlib.crc32(name.encode()) % 1000 + 600, prefix_lens=pre,
                       tree_sizes=sizes, tree_rules=rule, p_chain=pc,
                       num_q_heads=2, num_kv_heads=1, name=name)
    for seed in range(3):
        d, t, r = draw_tokens(wl, seed, vocab=vocab, p_agree=agree)
        say(f"[gpu] accept {name} seed {seed}")
        check_accept(wl.parents, wl.tree_offsets, d, t, r,
                     max(wl.max_nodes, 1) + extra, f"{name}/{seed}")


def test_accept_forest():
    # several roots per tree: each root's subtree competes for the path
    r = np.random.default_rng(77)
    sizes = [40, 70, 5]
    parents = []
    for B in sizes:
        p = [-1] + [int(r.integers(-1, i)) if r.random() < 0.2 else
                    int(r.integers(max(0, i - 3), i)) for i in range(1, B)]
        parents += p
    offs = np.concatenate([[0], np.cumsum(sizes)])
    for seed in range(4):
        rr = np.random.default_rng(seed)
        d = rr.integers(0, 2, size=sum(sizes))
        t = rr.integers(0, 2, size=sum(sizes))
        root = rr.integers(0, 2, size=3)
        say(f"[gpu] accept forest seed {seed}")
        check_accept(parents, offs, d, t, root, 70, f"forest/{seed}")


def test_accept_invalid_tree_stays_in_bounds():
    # an invalid tree gives unspecified output for itself only
    parents = [-1, 0, 1, -1, 0, 5, 2]   # node 5 of tree 1 points at itself
    offs = [0, 3, 7]
    d = [1, 2, 3, 1, 2, 3, 4]
    t = [2, 3, 9, 2, 3, 4, 5]
    say("[gpu] accept with an invalid tree")
    lens, nodes, bonus, bad = gpu_accept(parents, offs, d, t, [1, 1], 4)
    assert bad.tolist() == [-1, 5]
    assert lens[0] == 3 and nodes[0].tolist() == [0, 1, 2, -1]
    assert bonus[0] == 9
    assert 0 <= lens[1] <= 4


@pytest.mark.parametrize("name", STANDARD_ORDER)
def test_accept_standard_workloads(name):
    say(f"[gpu] accept standard workload {name}")
    wl = standard_workload(name)
    d, t, r = draw_tokens(wl, 1)
    check_accept(wl.parents, wl.tree_offsets, d, t, r, wl.max_nodes, name)


# --------------------------------------------------------------------------
# commit
# --------------------------------------------------------------------------

def gpu_commit(k, v, table, prefix, lens, nodes):
    import tree_masked_attention_amd.api as api
    kd = torch.from_numpy(np.ascontiguousarray(k)).to("cuda:0")
    vd = torch.from_numpy(np.ascontiguousarray(v)).to("cuda:0")
    api.commit_kv(kd, vd, _i32(table), _i32(prefix), _i32(lens), _i32(nodes))
    torch.cuda.synchronize()
    return kd.cpu().numpy(), vd.cpu().numpy()


def check_commit(k, v, table, prefix, lens, nodes, label):
    gk, gv = gpu_commit(k, v, table, prefix, lens, nodes)
    rk, rv = oracle.commit_kv(k, v, table, prefix, lens, nodes)
    moved = int(sum(int((nodes[s, :lens[s]] != np.arange(lens[s])).sum())
                    for s in range(len(lens))))
    say(f"  {label}: rows moved {moved}")
    assert np.array_equal(gk, rk), f"{label}: k cache differs"
    assert np.array_equal(gv, rv), f"{label}: v cache differs"
    return moved


def _paged(rng, prefix, sizes, page, token_bytes, spare=3):
    S = len(prefix)
    pages = [-(-(prefix[s] + sizes[s]) // page) for s in range(S)]
    num = sum(pages) + spare
    perm = rng.permutation(num)
    table = np.full((S, max(pages) + 1), -1, dtype=np.int32)
    o = 0
    for s in range(S):
        table[s, :pages[s]] = perm[o:o + pages[s]]
        o += pages[s]
    k = rng.integers(0, 256, size=(num, page, token_bytes), dtype=np.uint8)
    v = rng.integers(0, 256, size=(num, page, token_bytes), dtype=np.uint8)
    return k, v, table


def _increasing(rng, B, tau):
    return np.sort(rng.choice(B, size=tau, replace=False)).astype(np.int32)


@pytest.mark.parametrize("page,token_bytes", [(1, 16), (4, 48), (16, 2048),
                                              (16, 4096 + 16), (64, 256),
                                              (2, 8192)])
def test_commit_random_lists(page, token_bytes):
    rng = np.random.default_rng(page * 7 + token_bytes)
    prefix = [0, 5, 33, 100]
    sizes = [40, 7, 300, 1]
    k, v, table = _paged(rng, prefix, sizes, page, token_bytes)
    max_nodes = 300
    for trial in range(3):
        lens = np.zeros(4, dtype=np.int32)
        nodes = np.full((4, max_nodes), -1, dtype=np.int32)
        for s in range(4):
            tau = int(rng.integers(0, sizes[s] + 1))
            lens[s] = tau
            nodes[s, :tau] = _increasing(rng, sizes[s], tau)
        say(f"[gpu] commit page {page} token_bytes {token_bytes} "
            f"trial {trial}")
        check_commit(k, v, table, prefix, lens, nodes,
                     f"p{page}/tb{token_bytes}/{trial}")


def test_commit_shifted_chain():
    # n_j = j + 1: every row written is the next row's source
    rng = np.random.default_rng(5)
    k, v, table = _paged(rng, [10], [1000], 16, 512)
    lens = np.array([999], dtype=np.int32)
    nodes = np.full((1, 1000), -1, dtype=np.int32)
    nodes[0, :999] = np.arange(1, 1000)
    say("[gpu] commit shifted chain of 999 rows")
    assert check_commit(k, v, table, [10], lens, nodes, "shift") == 999


def test_commit_in_place_rows_untouched():
    rng = np.random.default_rng(6)
    k, v, table = _paged(rng, [3, 8], [12, 12], 4, 64)
    lens = np.array([5, 12], dtype=np.int32)
    nodes = np.full((2, 12), -1, dtype=np.int32)
    nodes[0, :5] = [0, 1, 2, 3, 4]          # already in place
    nodes[1, :12] = np.arange(12)
    say("[gpu] commit of rows already in place")
    assert check_commit(k, v, table, [3, 8], lens, nodes, "in-place") == 0


def test_commit_skips_rows_outside_page_table():
    rng = np.random.default_rng(8)
    k, v, table = _paged(rng, [6], [10], 4, 32, spare=0)
    table[0, 3] = -1                       # positions 12..15 unmapped
    lens = np.array([3], dtype=np.int32)
    nodes = np.array([[0, 2, 9, -1, -1, -1, -1, -1, -1, -1]], dtype=np.int32)
    gk, gv = gpu_commit(k, v, table, [6], lens, nodes)
    # row 2 (source position 15) is unmapped: skipped; row 1 moves
    rk, rv = k.copy(), v.copy()
    src, dst = 6 + 2, 6 + 1
    rk[table[0, dst // 4], dst % 4] = k[table[0, src // 4], src % 4]
    rv[table[0, dst // 4], dst % 4] = v[table[0, src // 4], src % 4]
    assert np.array_equal(gk, rk) and np.array_equal(gv, rv)


def _run_path(mode, dev_parents, dev_offs, masks, d, t, r, max_nodes, kd, vd,
              table, prefix):
    import tree_masked_attention_amd.api as api
    if mode == "fused":
        out = api.accept_commit(dev_parents, dev_offs, masks, _i32(d),
                                _i32(t), _i32(r), max_nodes, kd, vd, table,
                                prefix)
    else:
        out = api.accept(dev_parents, dev_offs, masks, _i32(d), _i32(t),
                         _i32(r), max_nodes)
        api.commit_kv(kd, vd, table, prefix, out[0], out[1])
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in out]


@pytest.mark.parametrize("mode", ["separate", "fused"])
@pytest.mark.parametrize("name", STANDARD_ORDER)
def test_accept_commit_standard_workloads(name, mode):
    """build_mask -> accept -> commit on the workload's own bf16 caches."""
    import tree_masked_attention_amd.api as api
    say(f"[gpu] accept + commit ({mode}), standard workload {name}")
    wl = standard_workload(name)
    d, t, r = draw_tokens(wl, 2)
    dev = device_inputs(wl)
    masks, _ = api.build_mask(dev["parents"], dev["tree_offsets"],
                              wl.max_nodes, wl.mask_words())
    lens, nodes, bonus = _run_path(mode, dev["parents"], dev["tree_offsets"],
                                   masks, d, t, r, wl.max_nodes,
                                   dev["k_cache"], dev["v_cache"],
                                   dev["page_table"], dev["prefix_lens"])
    rl, rn, rb = oracle.accept(wl.parents, wl.tree_offsets, d, t, r,
                               wl.max_nodes)
    assert np.array_equal(lens, rl)
    assert np.array_equal(nodes, rn)
    assert np.array_equal(bonus, rb)
    rk, rv = oracle.commit_kv(wl.k_cache, wl.v_cache, wl.page_table,
                              wl.prefix_lens, rl, rn)
    gk = dev["k_cache"].view(torch.int16).cpu().numpy()
    gv = dev["v_cache"].view(torch.int16).cpu().numpy()
    assert np.array_equal(gk, rk.view(np.int16))
    assert np.array_equal(gv, rv.view(np.int16))
    say(f"  tau = {rl.tolist()[:8]}")


FUSED_CASES = {
    # (prefix lens, tree sizes, rule, page size, token bytes, vocab, agree)
    "ragged-small-rows": ([0, 5, 33, 100], [40, 7, 300, 1], "pchain", 4, 48,
                          3, 0.9),
    "two-slices": ([17, 3], [64, 90], "pchain", 16, 4096 + 16, 4, 0.95),
    "max-1024-deep": ([9], [1024], "pchain", 8, 512, 2, 0.99),
    "page1-wide": ([3, 0], [200, 30], "wide", 1, 32, 2, 0.8),
    "empty-trees": ([4, 4, 4], [0, 12, 0], "pchain", 16, 256, 4, 0.9),
}


@pytest.mark.parametrize("name", sorted(FUSED_CASES))
def test_accept_commit_fused_vs_oracle(name):
    import tree_masked_attention_amd.api as api
    pre, sizes, rule, page, tb, vocab, agree = FUSED_CASES[name]
    wl = make_workload(zlib.crc32(name.encode()) % 1000 + 1700,
                       prefix_lens=pre, tree_sizes=sizes, tree_rules=rule,
                       p_chain=0.6, num_q_heads=1, num_kv_heads=1,
                       page_size=page, name=name)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    k, v, table = _paged(rng, pre, sizes, page, tb)
    mb = max(wl.max_nodes, 1)
    for seed in range(2):
        d, t, r = draw_tokens(wl, seed, vocab=vocab, p_agree=agree)
        say(f"[gpu] fused accept + commit {name} seed {seed}")
        p, o = _i32(wl.parents), _i32(wl.tree_offsets)
        masks, _ = api.build_mask(p, o, mb, api.mask_words_for(mb))
        kd = torch.from_numpy(k.copy()).to("cuda:0")
        vd = torch.from_numpy(v.copy()).to("cuda:0")
        lens, nodes, bonus = _run_path("fused", p, o, masks, d, t, r, mb, kd,
                                       vd, _i32(table), _i32(pre))
        rl, rn, rb = oracle.accept(wl.parents, wl.tree_offsets, d, t, r, mb)
        assert np.array_equal(lens, rl) and np.array_equal(nodes, rn)
        assert np.array_equal(bonus, rb)
        rk, rv = oracle.commit_kv(k, v, table, pre, rl, rn)
        assert np.array_equal(kd.cpu().numpy(), rk)
        assert np.array_equal(vd.cpu().numpy(), rv)
        say(f"  tau = {rl.tolist()}")
