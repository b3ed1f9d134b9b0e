"""The C-ABI library on the CPU: it loads, exports every function the header
declares, and rejects bad arguments before any launch (no GPU needed: each
call below fails its host-side checks before touching HIP)."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tree_attn.h")

api = pytest.importorskip("tree_masked_attention_amd.api")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tree_attn_[a-z_]+)\s*\(", text)))


def test_header_functions_exported():
    lib = ctypes.CDLL(api.LIB_PATH)
    names = declared_functions()
    assert set(names) == set(api.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    assert api.status_string(0) == "ok"
    for c in range(1, 6):
        assert api.status_string(c) not in ("ok", "unknown status")
    assert api.status_string(99) == "unknown status"
    assert api.abi_version() >= 1


def test_build_mask_rejects_bad_sizes():
    f = api.build_mask_raw
    assert f(1, 1, -1, 4, 4, 1, 1, 1, None) == api.ERR_SHAPE
    assert f(1, 1, 1, 4, 4, 0, 1, 1, None) == api.ERR_SHAPE
    assert f(1, 1, 1, 200, 200, 2, 1, 1, None) == api.ERR_SHAPE   # 128 < 200
    assert f(1, 1, 1, 2000, 2000, 32, 1, 1, None) == api.ERR_UNSUPPORTED
    assert f(None, 1, 1, 4, 4, 1, 1, 1, None) == api.ERR_NULL
    assert f(1, None, 1, 4, 4, 1, 1, 1, None) == api.ERR_NULL
    assert f(1, 1, 1, 4, 4, 1, None, 1, None) == api.ERR_NULL
    assert f(1, 1, 1, 4, 4, 1, 1, None, None) == api.ERR_NULL
    assert f(None, None, 0, 0, 0, 1, None, None, None) == api.OK  # no-op


def _verify(**over):
    args = dict(q=1, k=1, v=1, table=1, max_pps=20, num_pages=20,
                page_size=16, prefix=1, offs=1, masks=1, W=1, S=1, N=16,
                max_p=256, max_b=16, Hq=8, Hkv=2, d=128, scale=0.088,
                splits=0, out=1, lse=1, ws=None, ws_bytes=0)
    args.update(over)
    a = args
    return int(api._lib.tree_attn_verify(
        a["q"], a["k"], a["v"], a["table"], a["max_pps"], a["num_pages"],
        a["page_size"], a["prefix"], a["offs"], a["masks"], a["W"], a["S"],
        a["N"], a["max_p"], a["max_b"], a["Hq"], a["Hkv"], a["d"],
        a["scale"], a["splits"], a["out"], a["lse"], a["ws"], a["ws_bytes"],
        None))


@pytest.mark.parametrize("over,code", [
    (dict(Hkv=3), api.ERR_SHAPE),
    (dict(d=64), api.ERR_UNSUPPORTED),
    (dict(max_b=2048, W=32), api.ERR_UNSUPPORTED),
    (dict(max_b=65, W=1), api.ERR_SHAPE),
    (dict(page_size=12), api.ERR_SHAPE),
    (dict(page_size=0), api.ERR_SHAPE),
    (dict(max_pps=-1), api.ERR_SHAPE),
    (dict(S=-1), api.ERR_SHAPE),
    (dict(splits=-2), api.ERR_SHAPE),
    (dict(scale=float("nan")), api.ERR_SHAPE),
    (dict(scale=0.0), api.ERR_SHAPE),
    (dict(scale=-0.5), api.ERR_SHAPE),
    (dict(q=None), api.ERR_NULL),
    (dict(k=None), api.ERR_NULL),
    (dict(table=None), api.ERR_NULL),
    (dict(masks=None), api.ERR_NULL),
    (dict(out=None), api.ERR_NULL),
    (dict(lse=None), api.ERR_NULL),
    (dict(splits=4), api.ERR_WORKSPACE),        # forced split needs scratch
    (dict(splits=4, ws=256, ws_bytes=16), api.ERR_WORKSPACE),
])
def test_verify_rejects(over, code):
    assert _verify(**over) == code


def test_verify_empty_is_noop():
    assert _verify(S=0, N=0, q=None, k=None, v=None) == api.OK
    assert _verify(N=0) == api.OK


def test_workspace_size_rules():
    # one split needs no workspace; forced splits need partial rows
    ws1 = api.workspace_size(1, 16, 8, 2, 128, 256, 16, 16, 1)
    ws4 = api.workspace_size(1, 16, 8, 2, 128, 1024, 16, 16, 4)
    assert ws1 == 0
    # 64 KB of arrival counters, then one slot of partial rows per work
    # unit (4 splits x 2 kv heads x 1 row block of 64 rows: pairs of 64
    # rows take 64-row blocks): per row the fp16 output (256 B) and two
    # 32-bit statistics, each part rounded up to 256 B
    plan = api.describe_plan(1, 16, 8, 2, 128, 1024, 16, 16, 4)
    assert plan["rows"] == 64 and plan["splits"] == 4
    rows = 4 * 2 * 64
    part_o = -(-rows * 256 // 256) * 256
    part_ml = -(-rows * 8 // 256) * 256
    assert ws4 == 65536 + part_o + part_ml
    assert api.workspace_size(1, 16, 8, 3, 128, 256, 16, 16, 0) == 0  # invalid
    assert api.workspace_size(1, 16, 8, 2, 128, 256, 16, 12, 0) == 0  # page
    # tiny pages force more splits (each split's page slice is bounded)
    assert api.workspace_size(1, 16, 8, 2, 128, 5000, 16, 1, 1) >= \
        5 * 2 * 64 * (128 * 2 + 2 * 4)


def test_describe_plan():
    # pairs of at most 64 rows: 64-row blocks (four waves)
    p = api.describe_plan(1, 16, 8, 2, 128, 256, 16, 16, 0)
    assert p["waves"] == 4 and p["rows"] == 64 and p["splits"] >= 1
    assert p["chunk"] % 64 == 0 and p["chunk"] * p["splits"] >= 256 + 16
    # 96 rows per pair: 128-row blocks (eight waves: four row groups x two
    # key halves); the key range is split to fill the CUs
    p = api.describe_plan(1, 24, 8, 2, 128, 2048, 24, 16, 0)
    assert p["waves"] == 8 and p["rows"] == 128 and p["splits"] > 1
    # 1024 rows per kv head and one long split: eight waves
    p = api.describe_plan(4, 1024, 32, 8, 128, 32768, 256, 16, 0)
    assert p["waves"] == 8 and p["rows"] == 256 and p["splits"] == 2
    assert p["workgroups"] == 4 * 8 * 4 * 2
    # short splits of the same rows stay on 128-row blocks
    p = api.describe_plan(1, 256, 32, 8, 128, 4096, 256, 16, 0)
    assert p["rows"] == 128
    # forced split count is honoured, clamped by the key range
    p = api.describe_plan(1, 64, 16, 4, 128, 6000, 64, 16, 1)
    assert p["splits"] == 1 and p["waves"] == 8 and p["chunk"] >= 6064
    with pytest.raises(ValueError):
        api.describe_plan(1, 16, 8, 3, 128, 256, 16, 16, 0)
    with pytest.raises(NotImplementedError):
        api.describe_plan(1, 16, 8, 2, 64, 256, 16, 16, 0)


def _narrow_row_plan(sizes):
    """The plan tree_attn_verify_ex takes for rows narrower than 256 bytes
    (fp8, or head dim 64): tree_attn_verify's plan, except where that plan
    replaces a key split by 64-row blocks (pairs of 65 .. 128 rows, no
    requested split): the split is kept, on 128-row blocks."""
    bf = api.describe_plan(*sizes)
    S, N, Hq, Hkv, d, P, B, page, req = sizes
    rows = Hq // Hkv * B
    if bf["rows"] == 64 and 64 < rows <= 128 and req == 0:
        two = api.describe_plan(*sizes[:8], 2)
        # the 128-row plan that the substitution replaced has >= 2 splits
        assert two["rows"] == 128
        return None
    return bf


def test_describe_plan_ex():
    # every format and head dim runs the tuned kernels with
    # tree_attn_verify's plan (FP8 with head dim 128 with its workspace,
    # head dim 64 with partials of 64 values per row), except that rows
    # narrower than 256 bytes keep the key split where bf16 with head dim
    # 128 takes 64-row blocks without one
    for sizes in [(1, 16, 8, 2, 128, 256, 16, 16, 0),
                  (4, 1024, 32, 8, 128, 32768, 256, 16, 0),
                  (32, 512, 32, 4, 128, 2048, 16, 16, 0),
                  (3, 119, 8, 2, 128, 9000, 70, 16, 0),
                  (1, 64, 16, 4, 128, 6000, 64, 16, 3)]:
        bf = api.describe_plan(*sizes)
        want = _narrow_row_plan(sizes)
        f8 = api.describe_plan_ex(api.KV_FP8_E4M3, *sizes)
        d64 = sizes[:4] + (64,) + sizes[5:]
        plans = [(api.KV_FP8_E4M3, sizes, f8)] + [
            (kvd, d64, api.describe_plan_ex(kvd, *d64))
            for kvd in (api.KV_BF16, api.KV_FP8_E4M3)]
        for kvd, sz, pl in plans:
            if want is not None:
                assert pl == want, (sizes, kvd)
            else:
                assert pl["rows"] == 128 and pl["waves"] == 8, (sizes, kvd)
                assert pl["splits"] >= 2, (sizes, kvd)
            ws = api._lib.tree_attn_workspace_size_ex(kvd, *sz)
            per_row = 2 * sz[4] + 8
            if pl["splits"] == 1:
                assert ws == 0
            else:
                assert 65536 < ws <= \
                    65536 + pl["workgroups"] * pl["rows"] * per_row + 512
        if want is not None:
            assert api._lib.tree_attn_workspace_size_ex(
                api.KV_FP8_E4M3, *sizes) == \
                api._lib.tree_attn_workspace_size(*sizes)
    with pytest.raises(NotImplementedError):
        api.describe_plan_ex(api.KV_BF16, 1, 16, 8, 2, 96, 256, 16, 16, 0)
    with pytest.raises(NotImplementedError):
        api.describe_plan_ex(7, 1, 16, 8, 2, 128, 256, 16, 16, 0)


def test_plan_invariants_random_shapes():
    # host planning over random shapes: tile-multiple chunks covering the
    # key range, at most 256 splits, a kernel shape for every row count,
    # the 64-row shape only without a split, a workspace exactly when the
    # key range is split, and the workgroup count of the unit grid
    rng = np.random.default_rng(3)
    for _ in range(400):
        S = int(rng.integers(1, 80))
        hkv = int(rng.choice([1, 2, 4, 8]))
        G = int(rng.choice([1, 2, 4, 8]))
        max_b = int(rng.integers(1, 1025))
        max_p = int(rng.integers(0, 40000))
        page = int(rng.choice([1, 4, 16, 64, 256]))
        splits = int(rng.choice([0, 0, 0, 1, 2, 7]))
        N = S * max_b
        args = (S, N, G * hkv, hkv, 128, max_p, max_b, page, splits)
        try:
            p = api.describe_plan(*args)
        except NotImplementedError:
            continue  # key ranges beyond 256 splits of 1039 pages
        T = max_p + max_b
        assert p["chunk"] % 64 == 0 and 1 <= p["splits"] <= 256, args
        assert p["chunk"] * p["splits"] >= T, args
        assert (p["chunk"] - 64) * p["splits"] < T or p["splits"] == 1, args
        assert (p["waves"], p["rows"]) in ((4, 64), (8, 128), (8, 256)), args
        if p["rows"] == 64:
            assert G * max_b <= 64 or (p["splits"] == 1 and
                                       G * max_b <= 128), args
        if p["rows"] == 256:
            assert G * max_b >= 256 and p["chunk"] >= 2048, args
        if splits > 0:
            assert p["splits"] >= min(splits, -(-T // p["chunk"])), args
        mblocks = -(-G * max_b // p["rows"])
        units = S * hkv * mblocks * p["splits"]
        assert p["workgroups"] == 8 * -(-units // 8), args
        ws = api.workspace_size(*args)
        assert (ws > 0) == (p["splits"] > 1), args


def _accept(**over):
    a = dict(parents=1, offs=1, masks=1, W=1, draft=1, target=1, root=1, S=1,
             N=16, max_b=16, lens=1, nodes=1, bonus=1)
    a.update(over)
    return int(api._lib.tree_attn_accept(
        a["parents"], a["offs"], a["masks"], a["W"], a["draft"], a["target"],
        a["root"], a["S"], a["N"], a["max_b"], a["lens"], a["nodes"],
        a["bonus"], None))


@pytest.mark.parametrize("over,code", [
    (dict(S=-1), api.ERR_SHAPE),
    (dict(N=-1), api.ERR_SHAPE),
    (dict(W=0), api.ERR_SHAPE),
    (dict(max_b=65, W=1), api.ERR_SHAPE),
    (dict(max_b=2000, W=32), api.ERR_UNSUPPORTED),
    (dict(max_b=16, W=17), api.ERR_UNSUPPORTED),
    (dict(parents=None), api.ERR_NULL),
    (dict(masks=None), api.ERR_NULL),
    (dict(draft=None), api.ERR_NULL),
    (dict(target=None), api.ERR_NULL),
    (dict(root=None), api.ERR_NULL),
    (dict(lens=None), api.ERR_NULL),
    (dict(nodes=None), api.ERR_NULL),
    (dict(bonus=None), api.ERR_NULL),
])
def test_accept_rejects(over, code):
    assert _accept(**over) == code


def test_accept_empty_is_noop():
    assert _accept(S=0, parents=None, offs=None, masks=None, lens=None,
                   nodes=None) == api.OK


def _commit(**over):
    a = dict(k=256, v=512, table=1, max_pps=4, num_pages=8, page_size=16,
             prefix=1, lens=1, nodes=1, S=1, max_b=16, token_bytes=4096)
    a.update(over)
    return int(api._lib.tree_attn_commit_kv(
        a["k"], a["v"], a["table"], a["max_pps"], a["num_pages"],
        a["page_size"], a["prefix"], a["lens"], a["nodes"], a["S"],
        a["max_b"], a["token_bytes"], None))


@pytest.mark.parametrize("over,code", [
    (dict(S=-1), api.ERR_SHAPE),
    (dict(max_pps=-1), api.ERR_SHAPE),
    (dict(num_pages=-1), api.ERR_SHAPE),
    (dict(page_size=12), api.ERR_SHAPE),
    (dict(token_bytes=0), api.ERR_SHAPE),
    (dict(token_bytes=24), api.ERR_SHAPE),
    (dict(k=8), api.ERR_SHAPE),                 # not 16-byte aligned
    (dict(token_bytes=(1 << 20) + 16), api.ERR_UNSUPPORTED),
    (dict(max_b=2048), api.ERR_UNSUPPORTED),
    (dict(k=None), api.ERR_NULL),
    (dict(v=None), api.ERR_NULL),
    (dict(table=None), api.ERR_NULL),
    (dict(prefix=None), api.ERR_NULL),
    (dict(lens=None), api.ERR_NULL),
    (dict(nodes=None), api.ERR_NULL),
])
def test_commit_rejects(over, code):
    assert _commit(**over) == code


def test_commit_empty_is_noop():
    assert _commit(S=0, k=None, v=None) == api.OK
    assert _commit(max_b=0, k=None) == api.OK


def _fused(**over):
    a = dict(parents=1, offs=1, masks=1, W=1, draft=1, target=1, root=1, S=1,
             N=16, max_b=16, k=256, v=512, table=1, max_pps=4, num_pages=8,
             page_size=16, prefix=1, token_bytes=4096, lens=1, nodes=1,
             bonus=1)
    a.update(over)
    return int(api._lib.tree_attn_accept_commit(
        a["parents"], a["offs"], a["masks"], a["W"], a["draft"], a["target"],
        a["root"], a["S"], a["N"], a["max_b"], a["k"], a["v"], a["table"],
        a["max_pps"], a["num_pages"], a["page_size"], a["prefix"],
        a["token_bytes"], a["lens"], a["nodes"], a["bonus"], None))


@pytest.mark.parametrize("over,code", [
    (dict(W=0), api.ERR_SHAPE),
    (dict(max_b=65, W=1), api.ERR_SHAPE),
    (dict(page_size=3), api.ERR_SHAPE),
    (dict(token_bytes=8), api.ERR_SHAPE),
    (dict(v=8), api.ERR_SHAPE),
    (dict(W=17), api.ERR_UNSUPPORTED),
    (dict(token_bytes=1 << 21), api.ERR_UNSUPPORTED),
    (dict(masks=None), api.ERR_NULL),
    (dict(nodes=None), api.ERR_NULL),
    (dict(k=None), api.ERR_NULL),
    (dict(prefix=None), api.ERR_NULL),
])
def test_accept_commit_rejects(over, code):
    assert _fused(**over) == code


def test_accept_commit_empty_is_noop():
    assert _fused(S=0, parents=None, k=None, v=None, lens=None) == api.OK


@pytest.mark.parametrize("fn", ["tree_attn_verify_attend", "tree_attn_verify_merge"])
def test_verify_phases_check_like_verify(fn):
    f = getattr(api._lib, fn)
    base = dict(q=1, k=1, v=1, table=1, max_pps=20, num_pages=20,
                page_size=16, prefix=1, offs=1, masks=1, W=1, S=1, N=16,
                max_p=256, max_b=16, Hq=8, Hkv=2, d=128, scale=0.088,
                splits=0, out=1, lse=1, ws=None, ws_bytes=0)
    for over, code in ((dict(Hkv=3), api.ERR_SHAPE), (dict(d=64), api.ERR_UNSUPPORTED),
                       (dict(q=None), api.ERR_NULL), (dict(splits=4), api.ERR_WORKSPACE)):
        a = dict(base, **over)
        assert int(f(a["q"], a["k"], a["v"], a["table"], a["max_pps"],
                     a["num_pages"], a["page_size"], a["prefix"], a["offs"],
                     a["masks"], a["W"], a["S"], a["N"], a["max_p"], a["max_b"],
                     a["Hq"], a["Hkv"], a["d"], a["scale"], a["splits"],
                     a["out"], a["lse"], a["ws"], a["ws_bytes"], None)) == code


def _tree(**over):
    a = dict(logp=1, tokens=1, S=1, D=4, K=4, B=16, w=1, par=1, tok=1,
             dep=1, sc=1, sizes=1)
    a.update(over)
    return int(api._lib.tree_attn_build_tree(
        a["logp"], a["tokens"], a["S"], a["D"], a["K"], a["B"], a["w"],
        a["par"], a["tok"], a["dep"], a["sc"], a["sizes"], None))


@pytest.mark.parametrize("over,code", [
    (dict(S=-1), api.ERR_SHAPE),
    (dict(D=-1), api.ERR_SHAPE),
    (dict(K=0), api.ERR_SHAPE),
    (dict(B=-1), api.ERR_SHAPE),
    (dict(w=0), api.ERR_SHAPE),
    (dict(B=1025), api.ERR_UNSUPPORTED),
    (dict(K=65), api.ERR_UNSUPPORTED),
    (dict(D=1025, K=8), api.ERR_UNSUPPORTED),
    (dict(logp=None), api.ERR_NULL),
    (dict(tokens=None), api.ERR_NULL),
    (dict(par=None), api.ERR_NULL),
    (dict(sc=None), api.ERR_NULL),
    (dict(sizes=None), api.ERR_NULL),
])
def test_build_tree_rejects(over, code):
    assert _tree(**over) == code


def test_build_tree_empty_is_noop():
    assert _tree(S=0, logp=None, sizes=None) == api.OK


def _gdn(**over):
    a = dict(q=1, k=1, v=1, g=1, beta=1, st=1, offs=1, masks=1, W=2, S=2,
             N=20, max_b=128, H=4, d=128, out=1, u=1)
    a.update(over)
    return int(api._lib.tree_attn_gdn_verify(
        a["q"], a["k"], a["v"], a["g"], a["beta"], a["st"], a["offs"],
        a["masks"], a["W"], a["S"], a["N"], a["max_b"], a["H"], a["d"],
        a["out"], a["u"], None))


@pytest.mark.parametrize("over,code", [
    (dict(S=-1), api.ERR_SHAPE),
    (dict(N=-1), api.ERR_SHAPE),
    (dict(H=0), api.ERR_SHAPE),
    (dict(W=0), api.ERR_SHAPE),
    (dict(W=1, max_b=65), api.ERR_SHAPE),
    (dict(d=64), api.ERR_UNSUPPORTED),
    (dict(max_b=129, W=3), api.ERR_UNSUPPORTED),
    (dict(H=16385), api.ERR_UNSUPPORTED),
    (dict(S=1 << 20, H=1 << 12), api.ERR_UNSUPPORTED),
    (dict(q=None), api.ERR_NULL),
    (dict(beta=None), api.ERR_NULL),
    (dict(st=None), api.ERR_NULL),
    (dict(masks=None), api.ERR_NULL),
    (dict(out=None), api.ERR_NULL),
    (dict(u=None), api.ERR_NULL),
])
def test_gdn_verify_rejects(over, code):
    assert _gdn(**over) == code


def test_gdn_verify_empty_is_noop():
    assert _gdn(S=0, q=None) == api.OK
    assert _gdn(N=0, q=None) == api.OK


def _gdn_commit(**over):
    a = dict(k=1, u=1, g=1, offs=1, alen=1, anodes=1, S=2, max_b=16, H=4,
             d=128, st=1)
    a.update(over)
    return int(api._lib.tree_attn_gdn_commit(
        a["k"], a["u"], a["g"], a["offs"], a["alen"], a["anodes"], a["S"],
        a["max_b"], a["H"], a["d"], a["st"], None))


@pytest.mark.parametrize("over,code", [
    (dict(S=-1), api.ERR_SHAPE),
    (dict(max_b=-1), api.ERR_SHAPE),
    (dict(H=0), api.ERR_SHAPE),
    (dict(d=256), api.ERR_UNSUPPORTED),
    (dict(max_b=1025), api.ERR_UNSUPPORTED),
    (dict(S=1 << 20, H=1 << 12), api.ERR_UNSUPPORTED),
    (dict(k=None), api.ERR_NULL),
    (dict(alen=None), api.ERR_NULL),
    (dict(anodes=None), api.ERR_NULL),
    (dict(st=None), api.ERR_NULL),
])
def test_gdn_commit_rejects(over, code):
    assert _gdn_commit(**over) == code


def test_gdn_commit_empty_is_noop():
    assert _gdn_commit(S=0, k=None) == api.OK
    assert _gdn_commit(max_b=0, k=None) == api.OK


def _vex(**over):
    a = dict(q=1, k=1, v=1, kv=1, ks=None, vs=None, table=1, max_pps=4,
             num_pages=8, page_size=16, prefix=1, offs=1, masks=1, W=1, S=1,
             N=8, max_p=40, max_b=8, Hq=8, Hkv=2, d=64, scale=0.125,
             splits=0, out=1, lse=1, ws=None, ws_bytes=0)
    a.update(over)
    return int(api._lib.tree_attn_verify_ex(
        a["q"], a["k"], a["v"], a["kv"], a["ks"], a["vs"], a["table"],
        a["max_pps"], a["num_pages"], a["page_size"], a["prefix"], a["offs"],
        a["masks"], a["W"], a["S"], a["N"], a["max_p"], a["max_b"], a["Hq"],
        a["Hkv"], a["d"], a["scale"], a["splits"], a["out"], a["lse"],
        a["ws"], a["ws_bytes"], None))


@pytest.mark.parametrize("over,code", [
    (dict(S=-1), api.ERR_SHAPE),
    (dict(Hq=6, Hkv=4), api.ERR_SHAPE),
    (dict(page_size=24), api.ERR_SHAPE),
    (dict(W=0), api.ERR_SHAPE),
    (dict(W=1, max_b=65), api.ERR_SHAPE),
    (dict(scale=0.0), api.ERR_SHAPE),
    (dict(num_pages=0), api.ERR_SHAPE),
    (dict(d=96), api.ERR_UNSUPPORTED),
    (dict(d=256), api.ERR_UNSUPPORTED),
    (dict(kv=2), api.ERR_UNSUPPORTED),
    (dict(max_b=1025, W=17), api.ERR_UNSUPPORTED),
    (dict(q=None), api.ERR_NULL),
    (dict(k=None), api.ERR_NULL),
    (dict(masks=None), api.ERR_NULL),
    (dict(lse=None), api.ERR_NULL),
    (dict(max_p=100000, S=64, N=64), api.ERR_WORKSPACE),
    # more than 256 splits of 1039 pages (page size 1): not supported
    (dict(max_p=300000, page_size=1), api.ERR_UNSUPPORTED),
])
def test_verify_ex_rejects(over, code):
    assert _vex(**over) == code


def test_verify_ex_bf16_d128_checks_like_verify():
    # the bf16 / d = 128 combination is tree_attn_verify itself
    assert _vex(kv=0, d=128, q=None) == api.ERR_NULL
    assert _vex(kv=0, d=128, page_size=24) == api.ERR_SHAPE


def test_verify_ex_empty_is_noop():
    assert _vex(S=0, q=None) == api.OK
    assert _vex(N=0, q=None) == api.OK


def test_workspace_size_ex_rules():
    f = api._lib.tree_attn_workspace_size_ex
    # one sequence with a short range: a single split, no workspace
    assert f(1, 1, 8, 8, 2, 64, 40, 8, 16, 1) == 0
    # forced splits: fp16 partials (N * Hq * d * 2 per split) + (m, l)
    n = f(1, 1, 8, 8, 2, 64, 4000, 8, 16, 4)
    assert n >= 4 * 8 * 8 * 64 * 2 + 4 * 8 * 8 * 8
    # bf16 / d = 128 uses the tuned path's size
    assert f(0, 1, 8, 8, 2, 128, 4000, 8, 16, 4) == \
        api._lib.tree_attn_workspace_size(1, 8, 8, 2, 128, 4000, 8, 16, 4)
    assert f(1, 1, 8, 8, 2, 96, 4000, 8, 16, 4) == 0   # rejected sizes
    # a split's page ids fit the kernel's LDS copy: page size 1 and 4000
    # keys need at least 4 splits (1039 pages each), so one is not enough
    one = f(1, 1, 8, 8, 2, 64, 4000, 8, 1, 1)
    assert one >= 4 * 8 * 8 * 64 * 2
    assert f(1, 1, 8, 8, 2, 64, 300000, 8, 1, 0) == 0  # > 256 x 1039 pages


def _noalloc(**over):
    args = dict(q=1, k=1, v=1, table=1, max_pps=20, num_pages=20,
                page_size=16, prefix=1, offs=1, masks=1, W=1, S=1, N=16,
                max_p=256, max_b=16, Hq=8, Hkv=2, d=128, scale=0.088,
                splits=0, out=1, lse=1)
    args.update(over)
    a = args
    return int(api._lib.tree_attn_verify_noalloc(
        a["q"], a["k"], a["v"], a["table"], a["max_pps"], a["num_pages"],
        a["page_size"], a["prefix"], a["offs"], a["masks"], a["W"], a["S"],
        a["N"], a["max_p"], a["max_b"], a["Hq"], a["Hkv"], a["d"],
        a["scale"], a["splits"], a["out"], a["lse"], None))


@pytest.mark.parametrize("over,code", [
    (dict(Hkv=3), api.ERR_SHAPE),
    (dict(d=64), api.ERR_UNSUPPORTED),
    (dict(max_b=65, W=1), api.ERR_SHAPE),
    (dict(page_size=12), api.ERR_SHAPE),
    (dict(scale=0.0), api.ERR_SHAPE),
    (dict(q=None), api.ERR_NULL),
    (dict(lse=None), api.ERR_NULL),
    # a plan whose partials exceed the library's device scratch
    (dict(S=1, N=256, max_p=30000, max_b=256, W=4, Hq=32, Hkv=8,
          splits=256), api.ERR_WORKSPACE),
])
def test_verify_noalloc_rejects(over, code):
    assert _noalloc(**over) == code


def test_verify_noalloc_empty_is_noop():
    assert _noalloc(S=0, N=0, q=None, k=None, v=None) == api.OK
    assert _noalloc(N=0) == api.OK


def test_noalloc_scratch_limit_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define TREE_ATTN_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)",
                  text)
    assert m and int(m.group(1)) << int(m.group(2)) == api.NOALLOC_SCRATCH_BYTES
