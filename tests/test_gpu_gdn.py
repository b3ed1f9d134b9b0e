"""Gated DeltaNet tree verification and state commit: HIP path vs the CPU
oracle, through the C ABI (needs a gfx950 GPU).

Tolerances.  The oracle runs in fp64 on the same bf16-rounded q, k, v and
fp32 g, beta, S0.  The kernel computes in fp32 with every product on the
bf16 matrix cores, fp32 operands split into two bf16 parts (about 16
mantissa bits kept per product), so its fp32 results carry errors of order
2^-16 relative to the operand sizes (|u|, |o| are O(1) here): 2e-4 bounds
them with a wide margin.  out is then rounded to bf16 once, which adds at
most half an ulp, 2^-8 |out|.  Hence
  |u_gpu - u_ref|     <= 2e-4 (1 + |u_ref|)
  |out_gpu - out_ref| <= 2^-8 |out_ref| + 2e-4
  |S_gpu - S_ref|     <= 2e-4 (1 + |S_ref|)   (the commit, fp32 sums)
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import say
from tree_masked_attention_amd.workloads import (bf16_bits_to_f32,
                                                 draw_gdn_inputs, gdn_trees)

pytestmark = pytest.mark.gpu

U_TOL = 2e-4
O_REL = 2.0 ** -8
O_ABS = 2e-4
S_TOL = 2e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import tree_masked_attention_amd.api  # noqa: F401  (fails loudly if unbuilt)


def _dev_inputs(parents, offsets, x):
    q, k, v, g, beta, S0 = x
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(
        torch.bfloat16).cuda()
    return dict(q=bf(q), k=bf(k), v=bf(v), g=torch.from_numpy(g).cuda(),
                beta=torch.from_numpy(beta).cuda(),
                state=torch.from_numpy(np.ascontiguousarray(S0)).cuda(),
                parents=torch.from_numpy(parents).cuda(),
                offsets=torch.from_numpy(offsets).cuda())


def gpu_verify(parents, offsets, x, max_nodes=128):
    import tree_masked_attention_amd.api as api
    d = _dev_inputs(parents, offsets, x)
    masks, bad = api.build_mask(d["parents"], d["offsets"], max_nodes)
    out, u = api.gdn_verify(d["q"], d["k"], d["v"], d["g"], d["beta"],
                            d["state"], d["offsets"], masks, max_nodes)
    torch.cuda.synchronize()
    assert (bad.cpu().numpy() == -1).all()
    return out.float().cpu().numpy(), u.cpu().numpy(), d


def f32(x):
    q, k, v, g, beta, S0 = x
    return (bf16_bits_to_f32(q), bf16_bits_to_f32(k), bf16_bits_to_f32(v),
            g, beta, S0)


def check_outputs(o, u, ro, ru, label, rows=None):
    sel = slice(None) if rows is None else rows
    eu = np.abs(u[sel] - ru[sel])
    eo = np.abs(o[sel] - ro[sel])
    say(f"  {label}: max|du| {eu.max() if eu.size else 0:.2e}, "
        f"max|dout| {eo.max() if eo.size else 0:.2e}")
    assert (eu <= U_TOL * (1 + np.abs(ru[sel]))).all(), f"{label}: u"
    assert (eo <= O_REL * np.abs(ro[sel]) + O_ABS).all(), f"{label}: out"


CASES = {
    # name: (tree sizes, rules, heads)
    "one-node": ([1], "pchain", 2),
    "b16-pchain": ([16, 16, 16], "pchain", 3),
    "ragged-tails": ([1, 5, 31, 32, 33, 63, 64, 65], "pchain", 2),
    "b64-wide": ([64, 64], "wide", 2),
    "b96-deep": ([96], "pchain", 2),
    "b128-pchain": ([128, 128], "pchain", 2),
    "b128-chain": ([128], "chain", 2),
    "b128-star": ([128], "star", 2),
    "mixed-rules": ([100, 97, 128, 7], ["wide", "chain", "pchain", "star"], 2),
    "empty-trees": ([0, 7, 0, 12, 0], "pchain", 2),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_gdn_verify_parity(name):
    sizes, rules, H = CASES[name]
    seed = sum(map(ord, name))
    parents, offsets = gdn_trees(sizes, rules, seed,
                                 p_chain=0.9 if name == "b96-deep" else 0.5)
    x = draw_gdn_inputs(len(sizes), int(offsets[-1]), seed, heads=H)
    say(f"[gpu] gdn verify {name}: sizes {sizes} heads {H}")
    o, u, _ = gpu_verify(parents, offsets, x)
    ro, ru = oracle.gdn_verify(parents, offsets, *f32(x))
    check_outputs(o, u, ro, ru, name)


def test_gdn_verify_forest():
    # several roots per tree: each root path starts from S0
    parents, offsets = gdn_trees([40, 128], "pchain", 5)
    parents = parents.copy()
    parents[::9] = -1
    x = draw_gdn_inputs(2, int(offsets[-1]), 5, heads=2)
    say("[gpu] gdn verify forest")
    o, u, _ = gpu_verify(parents, offsets, x)
    ro, ru = oracle.gdn_verify(parents, offsets, *f32(x))
    check_outputs(o, u, ro, ru, "forest")


def test_gdn_verify_extreme_gates():
    # beta at 0 and 1, no decay and strong decay, zero state
    parents, offsets = gdn_trees([70, 50], "pchain", 6)
    q, k, v, g, beta, S0 = draw_gdn_inputs(2, int(offsets[-1]), 6, heads=4)
    beta[:, 0] = 0.0
    beta[:, 1] = 1.0
    g[:, 2] = 0.0
    g[:, 3] = -3.0
    S0[1] = 0.0
    x = (q, k, v, g, beta, S0)
    say("[gpu] gdn verify extreme gates")
    o, u, _ = gpu_verify(parents, offsets, x)
    ro, ru = oracle.gdn_verify(parents, offsets, *f32(x))
    check_outputs(o, u, ro, ru, "extreme-gates")


def test_gdn_verify_full_size_sampled():
    # the benchmark's shape: 16 trees of 128 nodes, 32 heads; the oracle
    # checks sampled (sequence, head) pairs one by one
    S, B, H = 16, 128, 32
    parents, offsets = gdn_trees([B] * S, "pchain", 11)
    x = draw_gdn_inputs(S, S * B, 11, heads=H)
    say("[gpu] gdn verify full size 16 x 128 nodes x 32 heads")
    o, u, _ = gpu_verify(parents, offsets, x)
    q, k, v, g, beta, S0 = f32(x)
    rng = np.random.default_rng(12)
    for s, h in zip(rng.integers(0, S, 4), rng.integers(0, H, 4)):
        a, b = int(offsets[s]), int(offsets[s + 1])
        hs = slice(int(h), int(h) + 1)
        ro, ru = oracle.gdn_tree_verify(parents[a:b], q[a:b, hs], k[a:b, hs],
                                        v[a:b, hs], g[a:b, hs], beta[a:b, hs],
                                        S0[s, hs])
        check_outputs(o[a:b, hs], u[a:b, hs], ro, ru, f"seq {s} head {h}")


def _random_paths(parents, offsets, rng, max_nodes):
    S = len(offsets) - 1
    lens = np.zeros(S, np.int32)
    nodes = np.full((S, max_nodes), -1, np.int32)
    last = np.full(S, -1)
    for s in range(S):
        a, b = int(offsets[s]), int(offsets[s + 1])
        if b == a or rng.random() < 0.15:
            continue  # nothing accepted
        j = int(rng.integers(0, b - a))
        last[s] = j
        path = []
        while j >= 0:
            path.append(j)
            j = int(parents[a + j])
        path = path[::-1]
        lens[s] = len(path)
        nodes[s, :len(path)] = path
    return lens, nodes, last


@pytest.mark.parametrize("name", ["b16-pchain", "ragged-tails",
                                  "b128-chain", "mixed-rules",
                                  "empty-trees"])
def test_gdn_commit_parity(name):
    import tree_masked_attention_amd.api as api
    sizes, rules, H = CASES[name]
    seed = sum(map(ord, name)) + 1
    parents, offsets = gdn_trees(sizes, rules, seed)
    x = draw_gdn_inputs(len(sizes), int(offsets[-1]), seed, heads=H)
    say(f"[gpu] gdn commit {name}")
    d = _dev_inputs(parents, offsets, x)
    masks, _ = api.build_mask(d["parents"], d["offsets"], 128)
    _, u = api.gdn_verify(d["q"], d["k"], d["v"], d["g"], d["beta"],
                          d["state"], d["offsets"], masks, 128)
    rng = np.random.default_rng(seed)
    max_nodes = 128
    lens, nodes, last = _random_paths(parents, offsets, rng, max_nodes)
    state = d["state"].clone()
    api.gdn_commit(d["k"], u, d["g"], d["offsets"],
                   torch.from_numpy(lens).cuda(),
                   torch.from_numpy(nodes).cuda(), state)
    torch.cuda.synchronize()
    got = state.cpu().numpy()
    q, k, v, g, beta, S0 = f32(x)
    worst = 0.0
    for s in range(len(sizes)):
        a, b = int(offsets[s]), int(offsets[s + 1])
        if lens[s] == 0:
            # nothing accepted: untouched, bit for bit
            assert np.array_equal(got[s], S0[s]), f"{name}: seq {s} changed"
            continue
        ref = oracle.gdn_commit_tree(parents[a:b], k[a:b], v[a:b], g[a:b],
                                     beta[a:b], S0[s], int(last[s]))
        err = np.abs(got[s] - ref)
        worst = max(worst, float(err.max()))
        assert (err <= S_TOL * (1 + np.abs(ref))).all(), f"{name}: seq {s}"
    say(f"  {name}: accepted {lens.tolist()}, max|dS| {worst:.2e}")


def test_gdn_commit_after_accept():
    # the path tree_attn_accept finds, committed; equals the oracle's
    # recurrence along the same path
    import tree_masked_attention_amd.api as api
    S, B, H = 4, 64, 2
    parents, offsets = gdn_trees([B] * S, "pchain", 21)
    x = draw_gdn_inputs(S, S * B, 21, heads=H)
    d = _dev_inputs(parents, offsets, x)
    masks, _ = api.build_mask(d["parents"], d["offsets"], B)
    _, u = api.gdn_verify(d["q"], d["k"], d["v"], d["g"], d["beta"],
                          d["state"], d["offsets"], masks, B)
    rng = np.random.default_rng(22)
    draft = rng.integers(0, 3, S * B).astype(np.int32)
    target = rng.integers(0, 3, S * B).astype(np.int32)
    root = rng.integers(0, 3, S).astype(np.int32)
    i32 = lambda a: torch.from_numpy(a).cuda()
    lens, nodes, _ = api.accept(d["parents"], d["offsets"], masks, i32(draft),
                                i32(target), i32(root), B)
    state = d["state"].clone()
    api.gdn_commit(d["k"], u, d["g"], d["offsets"], lens, nodes, state)
    torch.cuda.synchronize()
    got, lens, nodes = state.cpu().numpy(), lens.cpu().numpy(), nodes.cpu().numpy()
    q, k, v, g, beta, S0 = f32(x)
    say(f"[gpu] gdn commit after accept: tau {lens.tolist()}")
    for s in range(S):
        a, b = int(offsets[s]), int(offsets[s + 1])
        last = int(nodes[s, lens[s] - 1]) if lens[s] else -1
        ref = oracle.gdn_commit_tree(parents[a:b], k[a:b], v[a:b], g[a:b],
                                     beta[a:b], S0[s], last)
        assert (np.abs(got[s] - ref) <= S_TOL * (1 + np.abs(ref))).all()
