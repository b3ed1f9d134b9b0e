"""Cache-format and head-dimension variants of the verification attention
(tree_attn_verify_ex): head_dim 64, and FP8 E4M3 K/V pages with per-kv-head
scales, against the CPU oracle through the C ABI (needs a gfx950 GPU).
Bar: out max-abs <= 2e-2, lse relative <= 1e-3 (the oracle decodes the same
E4M3 codes, so the cache format adds no error of its own)."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_RTOL, OUT_ATOL, say
from tree_masked_attention_amd.workloads import (make_workload,
                                                 standard_workload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import tree_masked_attention_amd.api  # noqa: F401  (fails loudly if unbuilt)


def run_ex(wl, num_splits=0, W=None):
    import tree_masked_attention_amd.api as api
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    if wl.kv_format == "bf16":
        k, v = bf(wl.k_cache), bf(wl.v_cache)
        ks = vs = None
    else:
        k = torch.from_numpy(wl.k_cache).to(dev)
        v = torch.from_numpy(wl.v_cache).to(dev)
        ks = torch.from_numpy(wl.k_scale).to(dev)
        vs = torch.from_numpy(wl.v_scale).to(dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    masks, bad = api.build_mask(i32(wl.parents), i32(wl.tree_offsets),
                                max(wl.max_nodes, 1), W)
    out, lse = api.verify_ex(bf(wl.q), k, v, i32(wl.page_table),
                             i32(wl.prefix_lens), i32(wl.tree_offsets), masks,
                             wl.max_prefix_len, wl.max_nodes, wl.scale, ks, vs,
                             num_splits=num_splits)
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy().astype(np.float64)


def check(wl, label, num_splits=0, **okw):
    out, lse = run_ex(wl, num_splits)
    ref_o, ref_l = oracle.workload_attention(wl, **okw)
    sel = ~np.isnan(ref_l)
    eo = np.abs(out - ref_o)[sel].max() if sel.any() else 0.0
    el = (np.abs(lse - ref_l) / np.maximum(np.abs(ref_l), 1))[sel].max() \
        if sel.any() else 0.0
    say(f"  {label}: max|dout| {eo:.2e}, max rel dlse {el:.2e}")
    assert eo <= OUT_ATOL and el <= LSE_RTOL, label


def _case(name, seed, fmt, d, **kw):
    kw.setdefault("num_q_heads", 8)
    kw.setdefault("num_kv_heads", 2)
    return make_workload(seed, name=name, kv_format=fmt, head_dim=d, **kw)


CASES = {
    "ragged-multi": dict(prefix_lens=[0, 77, 300, 1],
                         tree_sizes=[1, 37, 130, 64]),
    "gqa8": dict(prefix_lens=[513], tree_sizes=[16], num_q_heads=32,
                 num_kv_heads=4),
    "empty-tree-in-batch": dict(prefix_lens=[20, 40, 0], tree_sizes=[5, 0, 9]),
    "page1": dict(prefix_lens=[70, 3], tree_sizes=[12, 7], page_size=1),
    # page size 1 over 3000 keys: a split holds at most 1039 page ids, so
    # the plan makes at least three splits whatever is asked
    "page1-long": dict(prefix_lens=[3000, 1500], tree_sizes=[40, 9],
                       page_size=1),
    "page64": dict(prefix_lens=[70, 200], tree_sizes=[12, 70], page_size=64),
    "max-tree-1024": dict(prefix_lens=[50], tree_sizes=[1024], num_q_heads=2,
                          num_kv_heads=1, p_chain=0.7),
    "star": dict(prefix_lens=[33], tree_sizes=[300], tree_rules="star"),
    "long-prefix": dict(prefix_lens=[5000, 1234], tree_sizes=[3, 40]),
    "big-key-range": dict(prefix_lens=[900], tree_sizes=[40],
                          key_factor_range=(0.25, 4.0)),
    # the draft head's use of the mask (JETFLOW's parallel drafter): its own
    # short KV, a budget-256 tree, the target's head shape
    "draft-head": dict(prefix_lens=[600, 1500], tree_sizes=[256, 256],
                       num_q_heads=32, num_kv_heads=8),
}
FORMATS = [("bf16", 64), ("e4m3", 64), ("e4m3", 128)]


@pytest.mark.parametrize("fmt,d", FORMATS, ids=lambda x: str(x))
@pytest.mark.parametrize("name", sorted(CASES))
def test_variant_parity(name, fmt, d):
    seed = sum(map(ord, name)) + d
    say(f"[gpu] verify_ex {name} {fmt} d={d}")
    check(_case(name, seed, fmt, d, **CASES[name]), f"{name}/{fmt}/d{d}")


@pytest.mark.parametrize("splits", [1, 2, 5])
@pytest.mark.parametrize("fmt,d", FORMATS, ids=lambda x: str(x))
def test_variant_forced_splits(fmt, d, splits):
    wl = _case("splits", 41, fmt, d, prefix_lens=[2000, 300],
               tree_sizes=[64, 17])
    say(f"[gpu] verify_ex splits={splits} {fmt} d={d}")
    check(wl, f"splits{splits}/{fmt}/d{d}", num_splits=splits)


def test_draft_head_bf16_d128_is_the_tuned_path():
    # bf16, d = 128 through verify_ex runs tree_attn_verify's kernels
    wl = _case("draft-head", 7, "bf16", 128, **CASES["draft-head"])
    say("[gpu] verify_ex draft-head bf16 d=128")
    check(wl, "draft-head/bf16/d128")


@pytest.mark.parametrize("name", ["qwen3-30b-a3b-32x-b16-p2k",
                                  "long-32k-4x-b256"])
@pytest.mark.parametrize("fmt,d", [("e4m3", 128), ("bf16", 64)],
                         ids=lambda x: str(x))
def test_variant_full_size_sampled(name, fmt, d):
    wl = standard_workload(name, kv_format=fmt, head_dim=d)
    say(f"[gpu] verify_ex full size {wl.name}")
    out, lse = run_ex(wl)
    rng = np.random.default_rng(5)
    seqs = [int(rng.integers(0, wl.num_seqs))]
    heads = [int(rng.integers(0, wl.num_kv_heads))]
    ref_o, ref_l = oracle.workload_attention(wl, seq_ids=seqs,
                                             kv_head_ids=heads)
    sel = ~np.isnan(ref_l)
    eo = np.abs(out - ref_o)[sel].max()
    el = (np.abs(lse - ref_l) / np.maximum(np.abs(ref_l), 1))[sel].max()
    say(f"  {wl.name} seqs {seqs} kv head {heads}: max|dout| {eo:.2e}, "
        f"max rel dlse {el:.2e}")
    assert eo <= OUT_ATOL and el <= LSE_RTOL


def test_workspace_reuse_across_formats():
    # One zero-filled workspace for calls of different formats, head dims
    # and split counts in a row: each call matches the oracle and leaves
    # the counter area (the first 64 KB, which tree_attn_verify's launches
    # use) at zero, so one workspace serves both entry points.
    import tree_masked_attention_amd.api as api
    dev = torch.device("cuda:0")
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    to_dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    runs = [(_case("reuse-e4m3", 60, "e4m3", 128, prefix_lens=[700, 90],
                   tree_sizes=[40, 70]), 3),
            (_case("reuse-d64", 61, "bf16", 64, prefix_lens=[2000, 0, 31],
                   tree_sizes=[100, 16, 1]), 5),
            (_case("reuse-e4m3-d64", 62, "e4m3", 64, prefix_lens=[1500],
                   tree_sizes=[64]), 0)]
    ws = torch.zeros((64 << 20,), dtype=torch.uint8, device=dev)
    for wl, splits in runs:
        kvd = api.KV_FP8_E4M3 if wl.kv_format == "e4m3" else api.KV_BF16
        need = int(api._lib.tree_attn_workspace_size_ex(
            kvd, wl.num_seqs, wl.total_nodes, wl.num_q_heads,
            wl.num_kv_heads, wl.head_dim, wl.max_prefix_len, wl.max_nodes,
            wl.page_size, splits))
        assert 65536 < need <= ws.numel()
        if wl.kv_format == "bf16":
            k, v, ks, vs = bf(wl.k_cache), bf(wl.v_cache), None, None
        else:
            k, v = to_dev(wl.k_cache), to_dev(wl.v_cache)
            ks, vs = to_dev(wl.k_scale), to_dev(wl.v_scale)
        masks, _ = api.build_mask(to_dev(wl.parents), to_dev(wl.tree_offsets),
                                  wl.max_nodes)
        say(f"[gpu] variant workspace reuse {wl.name}, splits {splits}")
        out, lse = api.verify_ex(bf(wl.q), k, v, to_dev(wl.page_table),
                                 to_dev(wl.prefix_lens), to_dev(wl.tree_offsets),
                                 masks, wl.max_prefix_len, wl.max_nodes,
                                 wl.scale, ks, vs, num_splits=splits,
                                 workspace=ws)
        torch.cuda.synchronize()
        assert int(ws[:65536].count_nonzero()) == 0, "counters left set"
        ref_o, ref_l = oracle.workload_attention(wl)
        sel = ~np.isnan(ref_l)
        o = out.float().cpu().numpy()
        l = lse.cpu().numpy().astype(np.float64)
        eo = np.abs(o - ref_o)[sel].max()
        el = (np.abs(l - ref_l) / np.maximum(np.abs(ref_l), 1))[sel].max()
        say(f"  max|dout| {eo:.2e}, max rel dlse {el:.2e}")
        assert eo <= OUT_ATOL and el <= LSE_RTOL


# FP8 K/V with head dim 128 runs the tuned kernels (128 or 64 query rows
# per workgroup, fp8 tiles converted to bf16 as the matrix cores read
# them).  Shapes that take the 64-row kernel (pairs of at most 64 rows),
# pairs of 65-128 rows on 128-row blocks with a key split (where bf16
# takes 64-row blocks without one), the device-balanced split plan (2 to
# 64 sequences with splits), and the slow DMA path (pages of 4 keys).
def _fp8(name, seed, **kw):
    kw.setdefault("num_q_heads", 32)
    kw.setdefault("num_kv_heads", 4)
    return make_workload(seed, name=name, kv_format="e4m3", **kw)


FP8_TUNED_CASES = {
    "fp8-r128-split-ragged": (lambda: _fp8("fp8-r128s", 190,
                                           prefix_range=(0, 900),
                                           num_seqs=32,
                                           tree_sizes=[1 + (7 * s) % 16
                                                       for s in range(32)]),
                              128),
    "fp8-r128-split-page4": (lambda: _fp8("fp8-r128s-p4", 191,
                                          prefix_range=(100, 700),
                                          num_seqs=32, tree_sizes=[16],
                                          page_size=4), 128),
    "fp8-r64-ragged": (lambda: _fp8("fp8-r64", 197, prefix_range=(0, 900),
                                    num_seqs=32, num_q_heads=16,
                                    tree_sizes=[1 + (7 * s) % 16
                                                for s in range(32)]), 64),
    "fp8-r64-page4": (lambda: _fp8("fp8-r64-p4", 198,
                                   prefix_range=(100, 700), num_seqs=32,
                                   num_q_heads=16, tree_sizes=[16],
                                   page_size=4), 64),
    "fp8-balanced": (lambda: _fp8("fp8-bal", 192,
                                  prefix_lens=[300, 4000, 9000],
                                  tree_sizes=[40, 9, 70], num_q_heads=8,
                                  num_kv_heads=2), 128),
    "fp8-page8-chain": (lambda: _fp8("fp8-p8", 193, prefix_lens=[2500],
                                     tree_sizes=[100], page_size=8,
                                     num_q_heads=8, num_kv_heads=2,
                                     tree_rules="chain"), 128),
    # 256-row kernel on FP8 tiles (balanced plan over two sequences)
    "fp8-r256-balanced": (lambda: _fp8("fp8-r256", 195,
                                       prefix_lens=[16000, 9000],
                                       tree_sizes=[64, 70], num_q_heads=32,
                                       num_kv_heads=8), 256),
}


@pytest.mark.parametrize("name", sorted(FP8_TUNED_CASES))
def test_fp8_tuned_parity(name):
    import tree_masked_attention_amd.api as api
    make, rows = FP8_TUNED_CASES[name]
    wl = make()
    plan = api.describe_plan_ex(api.KV_FP8_E4M3, wl.num_seqs,
                                wl.total_nodes, wl.num_q_heads,
                                wl.num_kv_heads, 128, wl.max_prefix_len,
                                wl.max_nodes, wl.page_size, 0)
    say(f"[gpu] fp8 tuned {name}: plan {plan}")
    assert plan["rows"] == rows
    if name == "fp8-balanced" or "split" in name:
        assert plan["splits"] > 1  # the device-balanced plan
    check(wl, name)
    check(wl, f"{name}, 3 splits", num_splits=3)


# Head dim 64 runs the same three tuned kernel shapes: bf16 K/V in rows of
# 128 bytes (like the FP8 tiles of head dim 128), FP8 K/V in rows of 64
# bytes (one DMA op per wave per tile on the 8-wave shapes)
def _d64(name, seed, fmt="bf16", **kw):
    kw.setdefault("num_q_heads", 32)
    kw.setdefault("num_kv_heads", 4)
    return make_workload(seed, name=name, kv_format=fmt, head_dim=64, **kw)


D64_TUNED_CASES = {
    "d64-r128-split-ragged": (180, dict(prefix_range=(0, 900), num_seqs=32,
                                        tree_sizes=[1 + (7 * s) % 16
                                                    for s in range(32)]),
                              128),
    "d64-r64-ragged": (187, dict(prefix_range=(0, 900), num_seqs=32,
                                 num_q_heads=16,
                                 tree_sizes=[1 + (7 * s) % 16
                                             for s in range(32)]), 64),
    "d64-r64-split": (181, dict(prefix_lens=[5000] * 4, tree_sizes=[16],
                                num_q_heads=16), 64),
    "d64-balanced": (182, dict(prefix_lens=[300, 4000, 9000],
                               tree_sizes=[40, 9, 70], num_q_heads=8,
                               num_kv_heads=2), 128),
    "d64-page4-chain": (183, dict(prefix_lens=[2500], tree_sizes=[100],
                                  page_size=4, num_q_heads=8, num_kv_heads=2,
                                  tree_rules="chain"), 128),
    "d64-r256-balanced": (185, dict(prefix_lens=[16000, 9000],
                                    tree_sizes=[64, 70], num_kv_heads=8), 256),
    "d64-r256-page4": (186, dict(prefix_lens=[3900], tree_sizes=[64],
                                 page_size=4, num_q_heads=16), 256),
}


@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
@pytest.mark.parametrize("name", sorted(D64_TUNED_CASES))
def test_d64_tuned_parity(name, fmt):
    import tree_masked_attention_amd.api as api
    seed, kw, rows = D64_TUNED_CASES[name]
    wl = _d64(f"{name}-{fmt}", seed, fmt, **kw)
    kvd = api.KV_BF16 if fmt == "bf16" else api.KV_FP8_E4M3
    req = 1 if name == "d64-r256-page4" else 0
    plan = api.describe_plan_ex(kvd, wl.num_seqs, wl.total_nodes,
                                wl.num_q_heads, wl.num_kv_heads, 64,
                                wl.max_prefix_len, wl.max_nodes,
                                wl.page_size, req)
    say(f"[gpu] {fmt} d=64 tuned {name}: plan {plan}")
    assert plan["rows"] == rows
    check(wl, f"{name}/{fmt}", num_splits=req)
    check(wl, f"{name}/{fmt}, 3 splits", num_splits=3)


def _random_d64(seed):
    """Seeded random shapes for bf16 head dim 64 (all three kernel shapes
    get drawn: narrow and wide GQA groups, short and long key ranges)."""
    r = np.random.default_rng(seed)
    wide = seed % 2 == 1
    hkv = int(r.choice([1, 2, 4]))
    g = int(r.choice([4, 8]) if wide else r.choice([1, 2, 4, 8]))
    s = int(r.integers(1, 5))
    prefix = [int(x) for x in r.integers(2500 if wide else 0,
                                          5000 if wide else 1500, size=s)]
    sizes = [int(x) for x in r.integers(0, 300, size=s)]
    if wide:
        sizes[0] = max(sizes[0], 256 // g)
    if max(sizes) == 0:
        sizes[0] = 1
    rules = [str(x) for x in r.choice(["pchain", "wide", "chain", "star"],
                                      size=s)]
    page = int(r.choice([2, 4, 8, 16, 32, 64]))
    splits = int(r.choice([0, 1] if wide else [0, 0, 1, 2, 3, 7]))
    wl = make_workload(seed, prefix_lens=prefix, tree_sizes=sizes,
                       num_q_heads=g * hkv, num_kv_heads=hkv, page_size=page,
                       tree_rules=rules, p_chain=float(r.uniform(0.2, 0.95)),
                       kv_format="bf16", head_dim=64, name=f"d64-random-{seed}")
    return wl, splits


@pytest.mark.parametrize("seed", list(range(600, 612)))
def test_d64_random_shapes_parity(seed):
    import tree_masked_attention_amd.api as api
    wl, splits = _random_d64(seed)
    plan = api.describe_plan_ex(api.KV_BF16, wl.num_seqs, wl.total_nodes,
                                wl.num_q_heads, wl.num_kv_heads, 64,
                                wl.max_prefix_len, wl.max_nodes,
                                wl.page_size, splits)
    say(f"[gpu] d64 random {seed}: P={[int(x) for x in wl.prefix_lens]} "
        f"B={[int(x) for x in wl.tree_sizes]} Hq={wl.num_q_heads} "
        f"Hkv={wl.num_kv_heads} page={wl.page_size} splits={splits} "
        f"plan={plan}")
    check(wl, f"d64-random-{seed}", num_splits=splits)


def test_d64_many_row_blocks_take_the_merge_launch():
    # 4200 one-node trees x 4 kv heads = 16800 row blocks with 2 splits,
    # more than the workspace's 16384 arrival counters: the head-dim-64
    # partials are merged by the merge kernel's d = 64 instantiation in a
    # second launch; sampled sequences against the oracle
    import tree_masked_attention_amd.api as api
    wl = make_workload(171, prefix_lens=[100] * 4200, tree_sizes=[1],
                       num_q_heads=4, num_kv_heads=4, page_size=64,
                       head_dim=64, kv_format="bf16", name="d64-many-blocks")
    plan = api.describe_plan_ex(api.KV_BF16, wl.num_seqs, wl.total_nodes, 4,
                                4, 64, wl.max_prefix_len, wl.max_nodes,
                                wl.page_size, 2)
    say(f"[gpu] d64 with 16800 row blocks: plan {plan}")
    assert plan["splits"] == 2 and plan["rows"] == 64
    out, lse = run_ex(wl, 2)
    assert np.isfinite(lse).all()
    seqs = [0, 1, 777, 2048, 4198, 4199]
    ref_o, ref_l = oracle.workload_attention(wl, seq_ids=seqs)
    rows = np.array(seqs)  # one node per sequence
    eo = np.abs(out[rows] - ref_o[rows]).max()
    el = (np.abs(lse[rows] - ref_l[rows]) /
          np.maximum(np.abs(ref_l[rows]), 1)).max()
    say(f"  sampled sequences {seqs}: max|dout| {eo:.2e}, "
        f"max rel dlse {el:.2e}")
    assert eo <= OUT_ATOL and el <= LSE_RTOL


@pytest.mark.parametrize("page", [4, 16])
def test_fp8_256_rows_one_split(page):
    # one split of 3964 keys on the 256-row kernel (within the 1039 page
    # ids a split can hold at 4 keys per page): the tree tile's mask, the
    # slow DMA path (pages of 4 keys) and the fast one
    import tree_masked_attention_amd.api as api
    wl = _fp8(f"fp8-r256-p{page}", 196, prefix_lens=[3900], tree_sizes=[64],
              page_size=page, num_q_heads=16, num_kv_heads=4)
    plan = api.describe_plan_ex(api.KV_FP8_E4M3, wl.num_seqs, wl.total_nodes,
                                wl.num_q_heads, wl.num_kv_heads, 128,
                                wl.max_prefix_len, wl.max_nodes, wl.page_size,
                                1)
    say(f"[gpu] fp8 256 rows, one split, page {page}: plan {plan}")
    assert plan["rows"] == 256 and plan["splits"] == 1
    check(wl, f"fp8-r256-p{page}", num_splits=1)


@pytest.mark.parametrize("splits", [2, 5, 64])
def test_fp8_large_v_scale_splits(splits):
    # v_scale times 2^20: decoded values reach about 448 * 2^13, far past
    # fp16's range; split partials keep them through their per-row
    # power-of-two scale
    wl = _case("fp8-bigv", 194, "e4m3", 128, prefix_lens=[3000, 700],
               tree_sizes=[30, 64])
    wl.v_scale = (wl.v_scale * np.float32(2.0 ** 20)).astype(np.float32)
    from oracle.tree_oracle import widen_e4m3
    assert float(np.nanmax(np.abs(widen_e4m3(wl.v_cache))) *
                 wl.v_scale.max()) > 1e6
    say(f"[gpu] fp8 large v_scale, splits {splits}")
    out, lse = run_ex(wl, splits)
    ref_o, ref_l = oracle.workload_attention(wl)
    sel = ~np.isnan(ref_l)
    assert np.isfinite(out).all()
    rel = np.abs(out - ref_o)[sel].max() / np.abs(ref_o[sel]).max()
    el = (np.abs(lse - ref_l) / np.maximum(np.abs(ref_l), 1))[sel].max()
    say(f"  max|dout| / max|out| {rel:.2e}, max rel dlse {el:.2e}")
    # the bar relative to the output's scale (2e-2 of unit-scale outputs)
    assert rel <= OUT_ATOL / 4 and el <= LSE_RTOL


@pytest.mark.parametrize("d", [64, 128])
def test_fp8_decode_exact_through_the_path(d):
    # One node per sequence, no prefix: the node's only key is itself, its
    # softmax weight is exactly 1, so out is its V row decoded (times
    # v_scale = 1), bit for bit in bf16 -- every E4M3 value is a bf16
    # value.  The V rows hold all 256 codes; out must equal the oracle's
    # decoding from the format definition (NaN where the code is NaN).
    import tree_masked_attention_amd.api as api
    dev = torch.device("cuda:0")
    S = 256 // d
    codes = np.arange(256, dtype=np.uint8).reshape(S, d)
    page = 16
    k = np.full((S, page, 1, d), 0x38, dtype=np.uint8)  # 1.0 everywhere
    v = np.full((S, page, 1, d), 0x38, dtype=np.uint8)
    v[:, 0, 0, :] = codes
    q = torch.ones((S, 1, d), dtype=torch.bfloat16, device=dev)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    table = t(np.arange(S, dtype=np.int32).reshape(S, 1))
    prefix = t(np.zeros(S, dtype=np.int32))
    offs = t(np.arange(S + 1, dtype=np.int32))
    parents = t(np.full(S, -1, dtype=np.int32))
    masks, _ = api.build_mask(parents, offs, 1)
    ones = t(np.ones(1, dtype=np.float32))
    say(f"[gpu] fp8 decode through the path, d = {d}")
    out, lse = api.verify_ex(q, t(k), t(v), table, prefix, offs, masks, 0,
                             1, 1.0 / np.sqrt(d), ones, ones)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().reshape(S, d)
    from oracle.tree_oracle import widen_e4m3
    want = widen_e4m3(codes)
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert np.array_equal(got[~nan], want[~nan])
    assert np.isfinite(lse.cpu().numpy()).all()
