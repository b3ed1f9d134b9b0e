"""HIP path vs the CPU oracle, through the C ABI (needs a gfx950 GPU).

Bar: ancestor bitmasks bit-exact (padding words included); attention
output max |out - oracle| <= 2e-2 and lse max relative error <= 1e-3
(relative to max(|lse|, 1)).
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import (assert_parity, device_inputs, errors, run_gpu, say)
from tree_masked_attention_amd.workloads import (STANDARD_ORDER,
                                                 make_workload,
                                                 standard_workload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import tree_masked_attention_amd.api  # noqa: F401  (fails loudly if unbuilt)


def _case(name, seed, **kw):
    kw.setdefault("num_q_heads", 8)
    kw.setdefault("num_kv_heads", 2)
    return make_workload(seed, name=name, **kw)


SMALL_CASES = {
    "ragged-multi": lambda: _case("ragged-multi", 101,
                                  prefix_lens=[0, 77, 300, 1],
                                  tree_sizes=[1, 37, 130, 64],
                                  tree_rules="pchain", p_chain=0.5),
    "mha": lambda: _case("mha", 102, prefix_lens=[100], tree_sizes=[50],
                         num_q_heads=4, num_kv_heads=4),
    "gqa8": lambda: _case("gqa8", 103, prefix_lens=[513], tree_sizes=[16],
                          num_q_heads=32, num_kv_heads=4),
    "empty-tree-in-batch": lambda: _case("empty", 104, prefix_lens=[20, 40, 0],
                                         tree_sizes=[5, 0, 9]),
    "page1": lambda: _case("page1", 105, prefix_lens=[70, 3],
                           tree_sizes=[12, 7], page_size=1),
    "page64": lambda: _case("page64", 106, prefix_lens=[70, 200],
                            tree_sizes=[12, 70], page_size=64),
    "max-tree-1024": lambda: _case("b1024", 107, prefix_lens=[50],
                                   tree_sizes=[1024], num_q_heads=2,
                                   num_kv_heads=1, p_chain=0.7),
    "chain": lambda: _case("chain", 108, prefix_lens=[100], tree_sizes=[200],
                           tree_rules="chain"),
    "star": lambda: _case("star", 109, prefix_lens=[33], tree_sizes=[300],
                          tree_rules="star"),
    "no-prefix": lambda: _case("no-prefix", 110, prefix_lens=[0, 0],
                               tree_sizes=[64, 65]),
    "big-key-range": lambda: _case("keyscale", 111, prefix_lens=[900],
                                   tree_sizes=[40],
                                   key_factor_range=(0.25, 4.0)),
    "long-prefix-tiny-tree": lambda: _case("long-tail", 112,
                                           prefix_lens=[5000, 1234],
                                           tree_sizes=[3, 1]),
}


def _forest(wl):
    """Turn every 7th node into an extra root."""
    par = wl.parents.copy()
    for s in range(wl.num_seqs):
        a, b = wl.tree_offsets[s], wl.tree_offsets[s + 1]
        for i in range(7, b - a, 7):
            par[a + i] = -1
    wl.parents = par
    return wl


SMALL_CASES["forest"] = lambda: _forest(_case("forest", 113,
                                              prefix_lens=[10, 60],
                                              tree_sizes=[50, 90]))


@pytest.mark.parametrize("name", sorted(SMALL_CASES))
def test_small_case_parity(name):
    wl = SMALL_CASES[name]()
    say(f"[gpu] small case {name}: S={wl.num_seqs} P={list(wl.prefix_lens)} "
        f"B={list(wl.tree_sizes)} Hq={wl.num_q_heads} Hkv={wl.num_kv_heads} "
        f"page={wl.page_size}")
    got = run_gpu(wl)
    assert np.array_equal(got["masks"], oracle.workload_masks(wl))
    assert (got["bad"] == -1).all()
    ref_out, ref_lse = oracle.workload_attention(wl)
    assert_parity(got, ref_out, ref_lse, name)


# Cases sized so that the planner takes the eight-wave kernel (at least
# 256 query rows per kv head and at least 4096 keys per split).
EIGHT_WAVE_CASES = {
    "w8-ragged": (lambda: _case("w8-ragged", 140,
                                prefix_lens=[4100, 4500, 6000],
                                tree_sizes=[70, 1, 130], num_q_heads=16,
                                num_kv_heads=4), 1),
    "w8-page8": (lambda: _case("w8-page8", 141, prefix_lens=[4200],
                               tree_sizes=[64], page_size=8), 1),
    "w8-page4-slow-dma": (lambda: _case("w8-page4", 142, prefix_lens=[4000],
                                        tree_sizes=[96], page_size=4), 1),
    "w8-five-mask-words": (lambda: _case("w8-wide", 143, prefix_lens=[4000],
                                         tree_sizes=[300], num_q_heads=2,
                                         num_kv_heads=2), 1),
    "w8-two-splits": (lambda: _case("w8-2s", 144, prefix_lens=[9000, 8300],
                                    tree_sizes=[64, 90], num_q_heads=16,
                                    num_kv_heads=4), 2),
    "w8-chain": (lambda: _case("w8-chain", 145, prefix_lens=[4500],
                               tree_sizes=[128], tree_rules="chain"), 1),
}


@pytest.mark.parametrize("name", sorted(EIGHT_WAVE_CASES))
def test_eight_wave_parity(name):
    import tree_masked_attention_amd.api as api
    make, splits = EIGHT_WAVE_CASES[name]
    wl = make()
    plan = api.describe_plan(wl.num_seqs, wl.total_nodes, wl.num_q_heads,
                             wl.num_kv_heads, wl.head_dim,
                             wl.max_prefix_len, wl.max_nodes, wl.page_size,
                             splits)
    say(f"[gpu] eight-wave case {name}: P={list(wl.prefix_lens)} "
        f"B={list(wl.tree_sizes)} page={wl.page_size} plan={plan}")
    assert plan["waves"] == 8 and plan["rows"] == 256
    got = run_gpu(wl, num_splits=splits)
    assert np.array_equal(got["masks"], oracle.workload_masks(wl))
    ref_out, ref_lse = oracle.workload_attention(wl)
    assert_parity(got, ref_out, ref_lse, name)


@pytest.mark.parametrize("splits", [1, 2, 5, 64])
def test_forced_splits_parity(splits):
    wl = _case("splits", 120, prefix_lens=[1000, 64, 2500],
               tree_sizes=[33, 100, 7], num_q_heads=16, num_kv_heads=4)
    say(f"[gpu] forced splits={splits}")
    got = run_gpu(wl, num_splits=splits)
    ref_out, ref_lse = oracle.workload_attention(wl)
    assert_parity(got, ref_out, ref_lse, f"splits={splits}")


def test_split_count_changes_only_rounding():
    wl = _case("splitinv", 121, prefix_lens=[3000], tree_sizes=[64],
               num_q_heads=16, num_kv_heads=4)
    say("[gpu] split invariance")
    a = run_gpu(wl, num_splits=1)
    for n in (3, 11):
        b = run_gpu(wl, num_splits=n)
        assert np.abs(a["out"] - b["out"]).max() <= 8e-3
        assert np.abs(a["lse"] - b["lse"]).max() <= 1e-5 * 20


def test_page_permutation_bit_identical():
    wl = _case("perm", 122, prefix_lens=[700, 90], tree_sizes=[48, 20],
               shuffle_pages=False)
    say("[gpu] page permutation invariance")
    a = run_gpu(wl)
    perm = np.random.default_rng(5).permutation(wl.num_pages)
    inv = np.argsort(perm)
    wl.k_cache = np.ascontiguousarray(wl.k_cache[perm])
    wl.v_cache = np.ascontiguousarray(wl.v_cache[perm])
    wl.page_table = np.where(wl.page_table >= 0,
                             inv[np.maximum(wl.page_table, 0)],
                             -1).astype(np.int32)
    b = run_gpu(wl)
    assert np.array_equal(a["out_bits"], b["out_bits"])
    assert np.array_equal(a["lse"], b["lse"])


def test_deterministic():
    wl = standard_workload("qwen3-8b-b256-p4k")
    say("[gpu] determinism")
    dev = device_inputs(wl)
    a = run_gpu(wl, dev=dev)
    b = run_gpu(wl, dev=dev)
    assert np.array_equal(a["out_bits"], b["out_bits"])
    assert np.array_equal(a["lse"], b["lse"])
    assert np.array_equal(a["masks"], b["masks"])


def test_invalid_parents_reported():
    import tree_masked_attention_amd.api as api
    wl = _case("bad", 130, prefix_lens=[4, 4, 4], tree_sizes=[6, 5, 4])
    par = wl.parents.copy()
    par[0 + 3] = 3          # self loop in tree 0 (global node 3)
    par[6 + 2] = -2         # below -1 in tree 1 (global node 8)
    wl.parents = par
    say("[gpu] invalid parents")
    dev = device_inputs(wl)
    _, bad = api.build_mask(dev["parents"], dev["tree_offsets"], 6, 1)
    torch.cuda.synchronize()
    assert bad.cpu().tolist() == [3, 8, -1]
    # a tree larger than max_nodes is flagged at its first excess node
    wl2 = _case("big", 131, prefix_lens=[4], tree_sizes=[100])
    dev2 = device_inputs(wl2)
    masks, bad2 = api.build_mask(dev2["parents"], dev2["tree_offsets"], 64, 1)
    torch.cuda.synchronize()
    assert bad2.cpu().tolist() == [64]
    ref = oracle.ancestor_masks(wl2.parents[:64], np.array([0, 64]), 1)
    got = masks.cpu().numpy().view(np.uint64)
    assert np.array_equal(got[:64], ref)
    assert (got[64:] == 0).all()


# Cases sized so that the planner takes the 64-row kernel (pairs of at most
# 128 query rows, enough of them that 64-row blocks fill the CUs: no split).
def _r64(name, seed, **kw):
    kw.setdefault("num_q_heads", 32)
    kw.setdefault("num_kv_heads", 4)
    return make_workload(seed, name=name, **kw)


SIXTY_FOUR_ROW_CASES = {
    "r64-ragged": lambda: _r64("r64-ragged", 160, prefix_range=(0, 900),
                               num_seqs=32,
                               tree_sizes=[1 + (7 * s) % 16 for s in range(32)]),
    "r64-page4-slow-dma": lambda: _r64("r64-page4", 161,
                                       prefix_range=(100, 700), num_seqs=32,
                                       tree_sizes=[16], page_size=4),
    "r64-page64": lambda: _r64("r64-page64", 162, prefix_range=(600, 1200),
                               num_seqs=32, tree_sizes=[16], page_size=64),
    "r64-forest": lambda: _forest(_r64("r64-forest", 163,
                                       prefix_range=(600, 900), num_seqs=32,
                                       tree_sizes=[16])),
    "r64-g4-b32": lambda: _r64("r64-g4-b32", 164, prefix_range=(520, 900),
                               num_seqs=32, tree_sizes=[32], num_q_heads=16,
                               num_kv_heads=4, tree_rules="chain"),
}


@pytest.mark.parametrize("name", sorted(SIXTY_FOUR_ROW_CASES))
def test_sixty_four_row_parity(name):
    import tree_masked_attention_amd.api as api
    wl = SIXTY_FOUR_ROW_CASES[name]()
    plan = api.describe_plan(wl.num_seqs, wl.total_nodes, wl.num_q_heads,
                             wl.num_kv_heads, 128, wl.max_prefix_len,
                             wl.max_nodes, wl.page_size, 0)
    say(f"[gpu] 64-row case {name}: plan {plan}")
    assert plan["rows"] == 64 and plan["waves"] == 4 and plan["splits"] == 1
    got = run_gpu(wl)
    assert np.array_equal(got["masks"], oracle.workload_masks(wl))
    ref_out, ref_lse = oracle.workload_attention(wl)
    assert_parity(got, ref_out, ref_lse, name)
    # the same inputs with forced splits take the 128-row kernel
    two = run_gpu(wl, num_splits=2)
    assert_parity(two, ref_out, ref_lse, f"{name}, 2 splits")


# Pairs of at most 64 query rows take 64-row blocks whatever the split
# count: the planned launch (balanced over the sequences) and forced
# uniform splits, with the merge of the last split workgroup.
SIXTY_FOUR_ROW_SPLIT_CASES = {
    "r64s-g4-b16": lambda: _r64("r64s-g4-b16", 165, prefix_lens=[5000] * 4,
                                tree_sizes=[16], num_q_heads=16,
                                num_kv_heads=4),
    "r64s-ragged": lambda: _r64("r64s-ragged", 166, prefix_range=(300, 7000),
                                num_seqs=6, tree_sizes=[1 + (5 * s) % 16
                                                        for s in range(6)],
                                num_q_heads=16, num_kv_heads=4),
    "r64s-g8-b8-page4": lambda: _r64("r64s-g8-b8-page4", 167,
                                     prefix_range=(2000, 3000), num_seqs=3,
                                     tree_sizes=[8], page_size=4),
}


@pytest.mark.parametrize("name", sorted(SIXTY_FOUR_ROW_SPLIT_CASES))
def test_sixty_four_row_split_parity(name):
    import tree_masked_attention_amd.api as api
    wl = SIXTY_FOUR_ROW_SPLIT_CASES[name]()
    ref_out, ref_lse = oracle.workload_attention(wl)
    for req in (0, 3):
        plan = api.describe_plan(wl.num_seqs, wl.total_nodes,
                                 wl.num_q_heads, wl.num_kv_heads, 128,
                                 wl.max_prefix_len, wl.max_nodes,
                                 wl.page_size, req)
        say(f"[gpu] 64-row split case {name}, requested {req}: plan {plan}")
        assert plan["rows"] == 64 and plan["waves"] == 4
        assert plan["splits"] > 1
        got = run_gpu(wl, num_splits=req)
        assert np.array_equal(got["masks"], oracle.workload_masks(wl))
        assert_parity(got, ref_out, ref_lse, f"{name}, requested {req}")


# --------------------------------------------------------------------------
# the five standard workloads at full size, planned launch (as benchmarked)
# --------------------------------------------------------------------------

# Workloads whose oracle runs in worker processes, one task per
# (sequence, kv head) pair, so that every row is compared with the oracle
# within the test's time limit.
POOLED = {"long-32k-4x-b256"}


@pytest.mark.parametrize("name", STANDARD_ORDER)
def test_standard_workload_parity(name):
    say(f"[gpu] standard workload {name}: drawing inputs")
    wl = standard_workload(name)
    got = run_gpu(wl)
    assert np.array_equal(got["masks"], oracle.workload_masks(wl))
    assert np.isfinite(got["out"]).all() and np.isfinite(got["lse"]).all()
    if name in POOLED:
        from oracle_pool import oracle_by_pairs
        pairs = [(s, g) for s in range(wl.num_seqs)
                 for g in range(wl.num_kv_heads)]
        say(f"  oracle over {len(pairs)} (sequence, kv head) pairs")
        ro, rl = oracle_by_pairs(wl, pairs, workers=8)
        assert not np.isnan(rl).any()
        for s, g in pairs:
            a, b = wl.tree_offsets[s], wl.tree_offsets[s + 1]
            G = wl.num_q_heads // wl.num_kv_heads
            sl = (slice(a, b), slice(g * G, (g + 1) * G))
            part = dict(out=got["out"][sl], lse=got["lse"][sl])
            assert_parity(part, ro[sl], rl[sl], f"{name} seq {s} kv head {g}")
        assert_parity(got, ro, rl, f"{name} all rows")
        # the planned split against a single split, every row
        one = run_gpu(wl, num_splits=1)
        d_out = np.abs(one["out"] - got["out"]).max()
        d_lse = np.abs(one["lse"] - got["lse"]).max()
        say(f"  planned vs 1 split: max|dout|={d_out:.3e} max|dlse|={d_lse:.3e}")
        assert d_out <= 1e-2 and d_lse <= 1e-3
    else:
        ro, rl = oracle.workload_attention(wl)
        assert_parity(got, ro, rl, name)


# --------------------------------------------------------------------------
# randomised shapes: seeded draws of heads, page size, prefixes, tree sizes
# and shapes, split count (both kernel shapes get drawn)
# --------------------------------------------------------------------------

def _random_case(seed, wide=False):
    """wide: shapes that take the 256-row kernel (>= 256 rows per kv head,
    long key ranges, one or planned splits)."""
    r = np.random.default_rng(seed)
    hkv = int(r.choice([1, 2, 4]))
    g = int(r.choice([4, 8]) if wide else r.choice([1, 2, 4, 8]))
    s = int(r.integers(1, 5))
    long_keys = wide or bool(r.integers(0, 2))
    hi = 5000 if long_keys else 1500
    prefix = [int(x) for x in r.integers(2500 if wide else 0, hi, size=s)]
    sizes = [int(x) for x in r.integers(0, 300, size=s)]
    if wide:
        sizes[0] = max(sizes[0], 256 // g)
    if max(sizes) == 0:
        sizes[0] = 1
    rules = [str(x) for x in r.choice(["pchain", "wide", "chain", "star"], size=s)]
    page = int(r.choice([2, 4, 8, 16, 32, 64]))
    splits = int(r.choice([0, 1] if wide else [0, 0, 1, 1, 2, 3, 7]))
    wl = make_workload(seed, prefix_lens=prefix, tree_sizes=sizes,
                       num_q_heads=g * hkv, num_kv_heads=hkv, page_size=page,
                       tree_rules=rules, p_chain=float(r.uniform(0.2, 0.95)),
                       name=f"random-{seed}")
    return wl, splits


@pytest.mark.parametrize("seed", list(range(500, 524)))
def test_random_shapes_parity(seed):
    import tree_masked_attention_amd.api as api
    wl, splits = _random_case(seed, wide=seed >= 516)
    plan = api.describe_plan(wl.num_seqs, wl.total_nodes, wl.num_q_heads,
                             wl.num_kv_heads, wl.head_dim,
                             wl.max_prefix_len, wl.max_nodes, wl.page_size,
                             splits)
    say(f"[gpu] random case {seed}: P={[int(x) for x in wl.prefix_lens]} "
        f"B={[int(x) for x in wl.tree_sizes]} Hq={wl.num_q_heads} "
        f"Hkv={wl.num_kv_heads} "
        f"page={wl.page_size} splits={splits} plan={plan}")
    got = run_gpu(wl, num_splits=splits)
    assert np.array_equal(got["masks"], oracle.workload_masks(wl))
    assert (got["bad"] == -1).all()
    ref_out, ref_lse = oracle.workload_attention(wl)
    assert_parity(got, ref_out, ref_lse, f"random-{seed}")


# --------------------------------------------------------------------------
# the two launches of a verify call, made separately
# --------------------------------------------------------------------------

@pytest.mark.parametrize("splits", [0, 1, 3])
def test_attend_then_merge_equals_verify(splits):
    import tree_masked_attention_amd.api as api
    wl = _case("phases", 140, prefix_lens=[300, 77, 1500], tree_sizes=[40, 9, 70])
    say(f"[gpu] attend + merge vs verify, splits={splits}")
    dev = device_inputs(wl)
    masks, _ = api.build_mask(dev["parents"], dev["tree_offsets"],
                              wl.max_nodes, wl.mask_words())
    args = (dev["q"], dev["k_cache"], dev["v_cache"], dev["page_table"],
            dev["prefix_lens"], dev["tree_offsets"], masks, wl.max_prefix_len,
            wl.max_nodes, wl.scale)
    out1, lse1 = api.verify(*args, num_splits=splits)
    nbytes = api.workspace_size(wl.num_seqs, wl.total_nodes, wl.num_q_heads,
                                wl.num_kv_heads, wl.head_dim,
                                wl.max_prefix_len, wl.max_nodes,
                                wl.page_size, splits)
    ws = torch.empty((max(nbytes, 256),), dtype=torch.uint8, device="cuda:0")
    out2 = torch.empty_like(out1)
    lse2 = torch.empty_like(lse1)
    api.verify(*args, num_splits=splits, out=out2, lse=lse2, workspace=ws,
               phase="attend")
    api.verify(*args, num_splits=splits, out=out2, lse=lse2, workspace=ws,
               phase="merge")
    torch.cuda.synchronize()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1, lse2)


def test_one_launch_merge_reuses_workspace():
    # One zero-filled workspace for a run of calls of different shapes,
    # kernels (128 and 256 rows per workgroup) and split counts: every call
    # gives the bits of the two-launch form (attention kernel writing the
    # partials, then the merge kernel) and leaves the arrival counters at
    # zero for the next one.
    import tree_masked_attention_amd.api as api
    cases = [
        (_case("reuse-a", 150, prefix_lens=[300, 77, 1500],
               tree_sizes=[40, 9, 70]), 3),
        (_case("reuse-w8", 151, prefix_lens=[9000, 8300],
               tree_sizes=[64, 90], num_q_heads=16, num_kv_heads=4), 2),
        (_case("reuse-b", 152, prefix_lens=[2000, 0, 5],
               tree_sizes=[128, 31, 1]), 0),
        (_case("reuse-a2", 153, prefix_lens=[300, 77, 1500],
               tree_sizes=[40, 9, 70]), 7),
    ]
    sizes = []
    for wl, splits in cases:
        sizes.append(api.workspace_size(wl.num_seqs, wl.total_nodes,
                                        wl.num_q_heads, wl.num_kv_heads,
                                        wl.head_dim, wl.max_prefix_len,
                                        wl.max_nodes, wl.page_size, splits))
    ws = torch.zeros((max(sizes),), dtype=torch.uint8, device="cuda:0")
    for (wl, splits), nbytes in zip(cases, sizes):
        plan = api.describe_plan(wl.num_seqs, wl.total_nodes, wl.num_q_heads,
                                 wl.num_kv_heads, wl.head_dim,
                                 wl.max_prefix_len, wl.max_nodes,
                                 wl.page_size, splits)
        say(f"[gpu] workspace reuse {wl.name}: plan {plan}")
        assert plan["splits"] > 1
        dev = device_inputs(wl)
        masks, _ = api.build_mask(dev["parents"], dev["tree_offsets"],
                                  wl.max_nodes, wl.mask_words())
        args = (dev["q"], dev["k_cache"], dev["v_cache"], dev["page_table"],
                dev["prefix_lens"], dev["tree_offsets"], masks,
                wl.max_prefix_len, wl.max_nodes, wl.scale)
        out1, lse1 = api.verify(*args, num_splits=splits, workspace=ws)
        ws2 = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda:0")
        out2 = torch.empty_like(out1)
        lse2 = torch.empty_like(lse1)
        api.verify(*args, num_splits=splits, out=out2, lse=lse2,
                   workspace=ws2, phase="attend")
        api.verify(*args, num_splits=splits, out=out2, lse=lse2,
                   workspace=ws2, phase="merge")
        torch.cuda.synchronize()
        assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
        assert torch.equal(lse1, lse2)
        assert int(ws[:65536].count_nonzero()) == 0, "counters left set"
        ref_out, ref_lse = oracle.workload_attention(wl)
        eo, el = errors(out1.float().cpu().numpy().astype(np.float64),
                        lse1.cpu().numpy().astype(np.float64), ref_out,
                        ref_lse)
        say(f"  max|dout| {eo:.2e}, lse rel {el:.2e}")
        assert eo <= 2e-2 and el <= 1e-3


def _split_case_inputs(name, seed, splits):
    import tree_masked_attention_amd.api as api
    wl = _case(name, seed, prefix_lens=[2500, 700, 64], tree_sizes=[64, 17, 3])
    dev = device_inputs(wl)
    masks, _ = api.build_mask(dev["parents"], dev["tree_offsets"],
                              wl.max_nodes, wl.mask_words())
    args = (dev["q"], dev["k_cache"], dev["v_cache"], dev["page_table"],
            dev["prefix_lens"], dev["tree_offsets"], masks, wl.max_prefix_len,
            wl.max_nodes, wl.scale)
    nbytes = api.workspace_size(wl.num_seqs, wl.total_nodes, wl.num_q_heads,
                                wl.num_kv_heads, wl.head_dim,
                                wl.max_prefix_len, wl.max_nodes,
                                wl.page_size, splits)
    assert nbytes > 65536
    return wl, dev, args, nbytes


def test_overlapping_calls_with_own_workspaces():
    # two calls on two streams at the same time, each with its own
    # workspace (the arrival counters live in the workspace): each gives
    # the bits of the same call made alone
    import tree_masked_attention_amd.api as api
    splits = 4
    wl, dev, args, nbytes = _split_case_inputs("overlap", 160, splits)
    say("[gpu] overlapping verify calls on two streams")
    ref_out, ref_lse = api.verify(*args, num_splits=splits)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for st in streams:
        ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda:0")
        outs.append((torch.empty_like(ref_out), torch.empty_like(ref_lse), ws))
    torch.cuda.synchronize()  # the zero fills are done before the streams
    for rep in range(3):
        for st, (o, l, ws) in zip(streams, outs):
            with torch.cuda.stream(st):
                for _ in range(4):
                    api.verify(*args, num_splits=splits, out=o, lse=l,
                               workspace=ws, stream=st)
        torch.cuda.synchronize()
        for o, l, ws in outs:
            assert torch.equal(o.view(torch.int16), ref_out.view(torch.int16))
            assert torch.equal(l, ref_lse)
            assert int(ws[:65536].count_nonzero()) == 0


def test_side_stream_without_workspace():
    # verify on a stream that is not torch's current one, with the binding
    # allocating the (zero-filled) workspace and the outputs: the fills are
    # ordered before the launches on that stream, and the result equals the
    # call on the current stream bit for bit, in a loop that keeps the
    # allocator busy on the current stream meanwhile
    import tree_masked_attention_amd.api as api
    splits = 4
    wl, dev, args, nbytes = _split_case_inputs("side", 161, splits)
    say("[gpu] verify on a side stream, workspace allocated by the binding")
    ref_out, ref_lse = api.verify(*args, num_splits=splits)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(4):
        out, lse = api.verify(*args, num_splits=splits, stream=side)
        # unrelated allocations and work on the current stream
        junk = torch.full((1 << 20,), 7, dtype=torch.int32, device="cuda:0")
        junk.add_(1)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), rep
        assert torch.equal(lse, ref_lse), rep
        del junk


def test_two_phases_without_workspace_rejected():
    # the attend and merge launches must share a workspace: asking for a
    # phase of a split call without one is an error, not a silent zero merge
    import tree_masked_attention_amd.api as api
    splits = 4
    wl, dev, args, nbytes = _split_case_inputs("phase-ws", 162, splits)
    with pytest.raises(ValueError):
        api.verify(*args, num_splits=splits, phase="attend")


def test_graph_capture_replays():
    # tree_attn_verify (with split partials merged in its last workgroups)
    # captured in a graph: every replay, with eager work and a sync between
    # replays, gives the bits of the eager call; the arrival counters are
    # back at zero after each replay
    import tree_masked_attention_amd.api as api
    splits = 3
    wl, dev, args, nbytes = _split_case_inputs("graph", 161, splits)
    say("[gpu] graph capture of verify, 4 replays")
    ref_out, ref_lse = api.verify(*args, num_splits=splits)
    torch.cuda.synchronize()
    out = torch.empty_like(ref_out)
    lse = torch.empty_like(ref_lse)
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        # warm call outside the capture on the capture stream
        api.verify(*args, num_splits=splits, out=out, lse=lse, workspace=ws,
                   stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.verify(*args, num_splits=splits, out=out, lse=lse, workspace=ws,
                   stream=torch.cuda.current_stream())
    for rep in range(4):
        out.zero_()
        lse.zero_()
        scratch = torch.randn(1 << 20, device="cuda:0") * 2.0  # eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), rep
        assert torch.equal(lse, ref_lse), rep
        assert int(ws[:65536].count_nonzero()) == 0
        del scratch


def test_many_row_blocks_take_the_merge_launch():
    # 4200 one-node trees x 4 kv heads = 16800 row blocks, more than the
    # workspace's 16384 arrival counters: tree_attn_verify then merges in a
    # second launch. Its results equal the two-launch entry points' bit for
    # bit, and the counter area is not touched. (Inputs drawn on the GPU:
    # this branch is about the launch choice; parity of the two-launch form
    # with the oracle is covered above.)
    import tree_masked_attention_amd.api as api
    S, P, H, d, page = 4200, 100, 4, 128, 64
    npp = (P + 1 + page - 1) // page
    g = torch.Generator(device="cuda:0").manual_seed(170)
    kw = dict(device="cuda:0", generator=g)
    q = torch.randn((S, H, d), **kw).to(torch.bfloat16)
    k = torch.randn((S * npp, page, H, d), **kw).to(torch.bfloat16)
    v = torch.randn((S * npp, page, H, d), **kw).to(torch.bfloat16)
    i32 = dict(dtype=torch.int32, device="cuda:0")
    table = torch.arange(S * npp, **i32).view(S, npp)
    prefix = torch.full((S,), P, **i32)
    offs = torch.arange(S + 1, **i32)
    parents = torch.full((S,), -1, **i32)
    masks, bad = api.build_mask(parents, offs, 1)
    args = (q, k, v, table, prefix, offs, masks, P, 1, d ** -0.5)
    plan = api.describe_plan(S, S, H, H, d, P, 1, page, 2)
    say(f"[gpu] {S} one-node trees x {H} kv heads, plan {plan}")
    assert plan["splits"] == 2
    nbytes = api.workspace_size(S, S, H, H, d, P, 1, page, 2)
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda:0")
    out1, lse1 = api.verify(*args, num_splits=2, workspace=ws)
    ws2 = torch.zeros_like(ws)
    out2 = torch.empty_like(out1)
    lse2 = torch.empty_like(lse1)
    api.verify(*args, num_splits=2, out=out2, lse=lse2, workspace=ws2,
               phase="attend")
    api.verify(*args, num_splits=2, out=out2, lse=lse2, workspace=ws2,
               phase="merge")
    torch.cuda.synchronize()
    assert (bad.cpu() == -1).all()
    assert torch.equal(out1.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse1, lse2)
    assert torch.isfinite(lse1).all()
    assert int(ws[:65536].count_nonzero()) == 0


@pytest.mark.parametrize("seed", list(range(700, 716)))
def test_random_split_merge_repeated(seed):
    # random shapes (both kernels) with random forced splits, three calls in
    # a row on one workspace: every call gives the two-launch form's bits
    # and leaves the arrival counters at zero
    import tree_masked_attention_amd.api as api
    wl, _ = _random_case(seed, wide=bool(seed % 2))
    splits = int(np.random.default_rng(seed + 1).integers(2, 9))
    dev = device_inputs(wl)
    masks, _ = api.build_mask(dev["parents"], dev["tree_offsets"],
                              max(wl.max_nodes, 1), wl.mask_words())
    args = (dev["q"], dev["k_cache"], dev["v_cache"], dev["page_table"],
            dev["prefix_lens"], dev["tree_offsets"], masks, wl.max_prefix_len,
            wl.max_nodes, wl.scale)
    plan = api.describe_plan(wl.num_seqs, wl.total_nodes, wl.num_q_heads,
                             wl.num_kv_heads, wl.head_dim, wl.max_prefix_len,
                             wl.max_nodes, wl.page_size, splits)
    say(f"[gpu] random split merge {seed}: P={list(wl.prefix_lens)} "
        f"B={list(wl.tree_sizes)} plan={plan}")
    nbytes = api.workspace_size(wl.num_seqs, wl.total_nodes, wl.num_q_heads,
                                wl.num_kv_heads, wl.head_dim,
                                wl.max_prefix_len, wl.max_nodes,
                                wl.page_size, splits)
    ws2 = torch.zeros((max(nbytes, 256),), dtype=torch.uint8, device="cuda:0")
    ref_out, ref_lse = api.verify(*args, num_splits=splits, workspace=ws2,
                                  phase="attend")
    api.verify(*args, num_splits=splits, out=ref_out, lse=ref_lse,
               workspace=ws2, phase="merge")
    ws = torch.zeros_like(ws2)
    for rep in range(3):
        out, lse = api.verify(*args, num_splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), rep
        assert torch.equal(lse, ref_lse), rep
        assert int(ws[:65536].count_nonzero()) == 0


# --------------------------------------------------------------------------
# device-balanced split plans: a split launch over 2 .. 64 sequences sizes
# its splits on the device from each sequence's own key range (one shared
# split length, as many splits per sequence as its keys need), so short
# sequences take few workgroups and long ones many
# --------------------------------------------------------------------------

def _balanced_many(seed, S):
    r = np.random.default_rng(seed)
    return _case(f"bal-{S}", seed,
                 prefix_lens=[int(x) for x in r.integers(0, 3000, size=S)],
                 tree_sizes=[int(x) for x in r.integers(0, 40, size=S)],
                 num_q_heads=8, num_kv_heads=1)


BALANCED_CASES = {
    # lengths 12x apart; 128-row kernel
    "bal-ragged": (lambda: _case("bal-ragged", 180,
                                 prefix_lens=[300, 4000, 12000],
                                 tree_sizes=[40, 9, 70]), True),
    # sequences without tree nodes (no units) and one without prefix
    "bal-empty-trees": (lambda: _case("bal-empty", 181,
                                      prefix_lens=[0, 2500, 6000, 10],
                                      tree_sizes=[0, 30, 0, 5]), True),
    # 256-row kernel, two and three sequences of different lengths, one
    # with fewer rows than a block
    "bal-256": (lambda: _case("bal-256", 182, prefix_lens=[16000, 9000],
                              tree_sizes=[64, 70], num_q_heads=32,
                              num_kv_heads=8), True),
    "bal-256-ragged": (lambda: _case("bal-256r", 183,
                                     prefix_lens=[17000, 300, 6000],
                                     tree_sizes=[64, 3, 70], num_q_heads=32,
                                     num_kv_heads=8, page_size=32), True),
    # the largest batch the device plan takes, and one sequence more (the
    # host's uniform plan)
    "bal-64-seqs": (lambda: _balanced_many(184, 64), True),
    "uniform-65-seqs": (lambda: _balanced_many(185, 65), False),
}


def _balanced_inputs(name):
    import tree_masked_attention_amd.api as api
    make, balanced = BALANCED_CASES[name]
    wl = make()
    plan = api.describe_plan(wl.num_seqs, wl.total_nodes, wl.num_q_heads,
                             wl.num_kv_heads, wl.head_dim, wl.max_prefix_len,
                             wl.max_nodes, wl.page_size, 0)
    say(f"[gpu] {name}: S={wl.num_seqs} P={[int(x) for x in wl.prefix_lens]} "
        f"B={[int(x) for x in wl.tree_sizes]} Hq={wl.num_q_heads} "
        f"Hkv={wl.num_kv_heads} page={wl.page_size} plan={plan}")
    assert plan["splits"] > 1
    assert (2 <= wl.num_seqs <= 64) == balanced
    return wl, plan


@pytest.mark.parametrize("name", sorted(BALANCED_CASES))
def test_balanced_plan_parity(name):
    wl, _ = _balanced_inputs(name)
    got = run_gpu(wl)
    assert (got["bad"] == -1).all()
    ref_out, ref_lse = oracle.workload_attention(wl)
    assert_parity(got, ref_out, ref_lse, name)


@pytest.mark.parametrize("name", sorted(BALANCED_CASES))
def test_balanced_plan_two_launches_and_repeats(name):
    # the one-call form (last split workgroup merges) equals the two-launch
    # form (attention kernel, then merge kernel) bit for bit, on three
    # calls in a row over one workspace, each leaving the arrival counters
    # at zero
    import tree_masked_attention_amd.api as api
    wl, _ = _balanced_inputs(name)
    dev = device_inputs(wl)
    masks, _ = api.build_mask(dev["parents"], dev["tree_offsets"],
                              max(wl.max_nodes, 1), wl.mask_words())
    args = (dev["q"], dev["k_cache"], dev["v_cache"], dev["page_table"],
            dev["prefix_lens"], dev["tree_offsets"], masks, wl.max_prefix_len,
            wl.max_nodes, wl.scale)
    nbytes = api.workspace_size(wl.num_seqs, wl.total_nodes, wl.num_q_heads,
                                wl.num_kv_heads, wl.head_dim,
                                wl.max_prefix_len, wl.max_nodes,
                                wl.page_size, 0)
    ws2 = torch.zeros((max(nbytes, 256),), dtype=torch.uint8, device="cuda:0")
    ref_out, ref_lse = api.verify(*args, workspace=ws2, phase="attend")
    api.verify(*args, out=ref_out, lse=ref_lse, workspace=ws2, phase="merge")
    ws = torch.zeros_like(ws2)
    for rep in range(3):
        out, lse = api.verify(*args, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), rep
        assert torch.equal(lse, ref_lse), rep
        assert int(ws[:65536].count_nonzero()) == 0


# --------------------------------------------------------------------------
# status contract: an error left pending by an unrelated HIP call
# --------------------------------------------------------------------------

def test_stale_hip_error_not_reported_by_verify():
    """A failed, unchecked HIP call made just before a valid verify call
    (hipSetDevice on an ordinal that does not exist) does not turn the
    verify call's status into ERR_HIP; the call runs and matches the
    oracle."""
    import ctypes
    import tree_masked_attention_amd.api as api
    wl = SMALL_CASES["gqa8"]()
    dev = device_inputs(wl)
    W = wl.mask_words()
    masks, bad = api.build_mask(dev["parents"], dev["tree_offsets"],
                                max(wl.max_nodes, 1), W)
    N, Hq, d = wl.q.shape
    out = torch.empty((N, Hq, d), dtype=torch.bfloat16, device="cuda:0")
    lse = torch.empty((N, Hq), dtype=torch.float32, device="cuda:0")
    ws_bytes = api.workspace_size(wl.num_seqs, N, Hq, wl.num_kv_heads, d,
                                  wl.max_prefix_len, wl.max_nodes,
                                  wl.page_size, 0)
    ws = torch.zeros((max(ws_bytes, 256),), dtype=torch.uint8,
                     device="cuda:0")
    torch.cuda.synchronize()
    hip = ctypes.CDLL("libamdhip64.so.7")
    planted = hip.hipSetDevice(ctypes.c_int(1 << 20))
    assert planted != 0
    code = api._lib.tree_attn_verify(
        dev["q"].data_ptr(), dev["k_cache"].data_ptr(),
        dev["v_cache"].data_ptr(), dev["page_table"].data_ptr(),
        wl.max_pages_per_seq, wl.num_pages, wl.page_size,
        dev["prefix_lens"].data_ptr(), dev["tree_offsets"].data_ptr(),
        masks.data_ptr(), W, wl.num_seqs, N, wl.max_prefix_len,
        wl.max_nodes, Hq, wl.num_kv_heads, d, wl.scale, 0, out.data_ptr(),
        lse.data_ptr(), ws.data_ptr(), ws.numel(),
        torch.cuda.current_stream().cuda_stream)
    pending = hip.hipGetLastError()  # consume what is left for torch
    say(f"  planted error {planted}; verify status {code}; pending after "
        f"the call {pending}")
    assert code == api.OK
    torch.cuda.synchronize()
    got = dict(out=out.float().cpu().numpy().astype(np.float64),
               lse=lse.cpu().numpy().astype(np.float64))
    ref_out, ref_lse = oracle.workload_attention(wl)
    assert_parity(got, ref_out, ref_lse, "after a stale HIP error")
