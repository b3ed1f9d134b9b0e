"""Draft-tree construction: HIP path vs the CPU oracle, through the C ABI
(needs a gfx950 GPU).  Bar: bit-exact (parents, tokens, depths, scores as
fp32 bits, sizes, padding)."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
from gpu_util import say
from tree_masked_attention_amd.workloads import draw_draft_topk

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden",
                      "tree_build_tiny.json")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import tree_masked_attention_amd.api  # noqa: F401  (fails loudly if unbuilt)


def gpu_build(lp, tok, budget, width):
    import tree_masked_attention_amd.api as api
    out = api.build_tree(torch.from_numpy(np.ascontiguousarray(lp)).cuda(),
                         torch.from_numpy(np.ascontiguousarray(tok)).cuda(),
                         budget, width)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def check(lp, tok, budget, width, label):
    got = gpu_build(lp, tok, budget, width)
    ref = oracle.build_trees(lp, tok, budget, width)
    assert np.array_equal(got["sizes"], ref["sizes"]), f"{label}: sizes"
    for k in ("parents", "tokens", "depths"):
        assert np.array_equal(got[k], ref[k]), f"{label}: {k}"
    assert np.array_equal(got["scores"].view(np.int32),
                          ref["scores"].view(np.int32)), f"{label}: scores"
    say(f"  {label}: sizes {got['sizes'].tolist()[:6]} max depth "
        f"{int(got['depths'].max()) if got['depths'].size else 0}")
    return got


def test_tree_build_golden():
    say("[gpu] tree build: golden cases")
    for c in json.load(open(GOLDEN))["cases"]:
        lp = np.array([c["logp"]], np.float32)
        tok = np.array([c["tokens"]], np.int32)
        got = gpu_build(lp, tok, c["budget"], c["width"])
        n = len(c["parents"])
        assert got["sizes"].tolist() == [n], c["name"]
        assert got["parents"][0, :n].tolist() == c["parents"], c["name"]
        assert got["tokens"][0, :n].tolist() == c["out_tokens"], c["name"]
        assert got["depths"][0, :n].tolist() == c["depths"], c["name"]
        assert got["scores"][0, :n].tolist() == c["scores"], c["name"]


CASES = {
    # name: (S, D, K, budget, widths)
    "b16-k4": (8, 8, 4, 16, (1, 4, 16)),
    "b64-k8": (4, 16, 8, 64, (1, 8)),
    "b256-k8": (2, 16, 8, 256, (1, 16, 64)),
    "b256-deep": (1, 256, 2, 256, (1, 3)),
    "b150-k8": (3, 16, 8, 150, (1, 5)),      # 3 slots per lane
    "b300-k8": (2, 16, 8, 300, (1, 9)),      # 5 slots per lane
    "b350-k6": (2, 20, 6, 350, (1, 2)),      # 6 slots per lane
    "b1024-k16": (2, 64, 16, 1024, (1, 32)),
    "b1024-k64-d128": (1, 128, 64, 1024, (7,)),
    "b63-edge": (3, 5, 3, 63, (1, 2)),
    "b64-edge": (3, 5, 3, 64, (1,)),
    "b65-edge": (3, 5, 3, 65, (1, 64)),
    "budget-above-tree": (2, 3, 3, 200, (1, 5)),
    "one-depth": (4, 1, 16, 10, (1, 3)),
    "topk-1-chain": (2, 40, 1, 30, (1, 4)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_tree_build_parity(name):
    S, D, K, B, widths = CASES[name]
    lp, tok = draw_draft_topk(S, D, K, seed=sum(map(ord, name)))
    for w in widths:
        say(f"[gpu] tree build {name} width {w}")
        check(lp, tok, B, w, f"{name}/w{w}")


def test_tree_build_ties():
    # log-probs on a coarse grid: many equal scores, the tie rule decides
    rng = np.random.default_rng(31)
    S, D, K = 4, 6, 5
    lp = -np.sort(rng.integers(0, 4, size=(S, D, K)) * 0.5, axis=2)
    lp = np.ascontiguousarray(-np.sort(-lp, axis=2)).astype(np.float32)
    tok = rng.integers(0, 1000, size=(S, D, K)).astype(np.int32)
    for w in (1, 2, 7):
        say(f"[gpu] tree build ties width {w}")
        check(lp, tok, 100, w, f"ties/w{w}")


@pytest.mark.parametrize("budget", (150, 300, 350, 1000))
def test_tree_build_ties_many_slots(budget):
    # equal scores between slots held in different registers of a lane
    # (slot sigma and sigma + 64 m share lane sigma mod 64)
    rng = np.random.default_rng(budget)
    S, D, K = 2, 14, 6
    lp = -np.sort(rng.integers(0, 3, size=(S, D, K)) * 0.25, axis=2)
    lp = np.ascontiguousarray(-np.sort(-lp, axis=2)).astype(np.float32)
    tok = rng.integers(0, 1000, size=(S, D, K)).astype(np.int32)
    for w in (1, 4):
        say(f"[gpu] tree build ties budget {budget} width {w}")
        check(lp, tok, budget, w, f"ties-{budget}/w{w}")


def test_tree_build_zero_budget_and_depth():
    lp, tok = draw_draft_topk(2, 3, 4, seed=5)
    got = gpu_build(lp, tok, 0, 1)
    assert got["sizes"].tolist() == [0, 0]
    got = gpu_build(lp[:, :0], tok[:, :0], 8, 1)
    assert got["sizes"].tolist() == [0, 0]
    assert (got["parents"] == -1).all() and (got["depths"] == 0).all()
