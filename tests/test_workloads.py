"""Seeded synthetic inputs: determinism, shapes, validity."""

import numpy as np
import pytest
import torch

from tree_masked_attention_amd import workloads as W


def test_bf16_rounding_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.5 - 2**-8,
                                  0.0, -0.0, 3.0e38], np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(ours, ref.view(np.uint16))
    assert np.array_equal(W.bf16_bits_to_f32(ours),
                          torch.from_numpy(x).to(torch.bfloat16)
                          .to(torch.float32).numpy())


def test_draw_is_deterministic():
    a = W.make_workload(7, prefix_lens=[20, 3], tree_sizes=[9, 4],
                        num_q_heads=4, num_kv_heads=2, head_dim=8)
    b = W.make_workload(7, prefix_lens=[20, 3], tree_sizes=[9, 4],
                        num_q_heads=4, num_kv_heads=2, head_dim=8)
    for f in ("q", "k_cache", "v_cache", "page_table", "parents"):
        assert np.array_equal(getattr(a, f), getattr(b, f))


@pytest.mark.parametrize("name", ["small-b16-p256", "qwen3-8b-b256-p4k",
                                  "serving-mix-8x-b64"])
def test_standard_workload_structure(name):
    wl = W.standard_workload(name)
    S = wl.num_seqs
    sizes = wl.tree_sizes
    assert wl.q.shape == (wl.total_nodes, wl.num_q_heads, wl.head_dim)
    assert wl.k_cache.shape == wl.v_cache.shape
    assert wl.k_cache.shape[1:] == (16, wl.num_kv_heads, 128)
    # trees: topological, parent[0] = -1
    for s in range(S):
        a, b = wl.tree_offsets[s], wl.tree_offsets[s + 1]
        par = wl.parents[a:b]
        assert par[0] == -1
        assert all(-1 <= p < i for i, p in enumerate(par))
    # every live logical page maps to a distinct physical page
    live = []
    for s in range(S):
        n = -(-(int(wl.prefix_lens[s]) + int(sizes[s])) // 16)
        row = wl.page_table[s]
        assert (row[:n] >= 0).all() and (row[n:] == -1).all()
        live.extend(row[:n].tolist())
    assert len(set(live)) == len(live) == wl.num_pages
    if name == "small-b16-p256":
        assert np.array_equal(wl.page_table[0], np.arange(wl.num_pages))
    if name == "serving-mix-8x-b64":
        assert ((wl.prefix_lens >= 1024) & (wl.prefix_lens <= 8192)).all()
        # deep trees (odd sequences) are mostly chains, wide ones are not
        deep = [np.mean(wl.parents[wl.tree_offsets[s] + 1:
                                   wl.tree_offsets[s + 1]]
                        == np.arange(63)) for s in range(8)]
        assert min(deep[1::2]) > 0.75 and max(deep[0::2]) < 0.5


def test_draw_tokens_gives_multi_node_paths():
    from oracle import accept
    from tree_masked_attention_amd.workloads import draw_tokens, make_workload
    wl = make_workload(3, prefix_lens=[5, 0, 17, 2], tree_sizes=[40, 1, 64, 9],
                       num_q_heads=4, num_kv_heads=2)
    d, t, r = draw_tokens(wl, 3)
    assert d.shape == t.shape == (wl.total_nodes,) and r.shape == (4,)
    lens, nodes, _ = accept(wl.parents, wl.tree_offsets, d, t, r, wl.max_nodes)
    assert lens.max() >= 3
    d2, t2, r2 = draw_tokens(wl, 3)
    assert (d == d2).all() and (t == t2).all() and (r == r2).all()


def test_draw_draft_topk_sorted_and_seeded():
    from tree_masked_attention_amd.workloads import draw_draft_topk
    lp, tok = draw_draft_topk(3, 5, 4, seed=9)
    assert lp.shape == tok.shape == (3, 5, 4) and lp.dtype == np.float32
    assert (np.diff(lp, axis=2) <= 0).all() and (lp <= 0).all()
    assert np.isclose(np.exp(lp).sum(axis=2), 1.0).sum() == 0  # top-k only
    lp2, tok2 = draw_draft_topk(3, 5, 4, seed=9)
    assert (lp == lp2).all() and (tok == tok2).all()
