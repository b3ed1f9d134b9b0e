"""tree_attn_verify_noalloc (device scratch inside the library) against
tree_attn_verify with a caller workspace, through the C ABI (needs a
gfx950 GPU): two calls in a row, the second on a smaller input, each
bit-identical to the existing entry point's result and within the oracle
bar; oversized plans are refused before any launch."""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import assert_parity, device_inputs, say
from tree_masked_attention_amd.workloads import (make_workload,
                                                 standard_workload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import tree_masked_attention_amd.api  # noqa: F401  (fails loudly if unbuilt)


def _call(api, fn_name, wl, dev, masks, splits, with_ws):
    N, Hq, d = wl.q.shape
    out = torch.full((N, Hq, d), float("nan"), dtype=torch.bfloat16,
                     device="cuda:0")
    lse = torch.full((N, Hq), float("nan"), dtype=torch.float32,
                     device="cuda:0")
    args = [dev["q"].data_ptr(), dev["k_cache"].data_ptr(),
            dev["v_cache"].data_ptr(), dev["page_table"].data_ptr(),
            wl.max_pages_per_seq, wl.num_pages, wl.page_size,
            dev["prefix_lens"].data_ptr(), dev["tree_offsets"].data_ptr(),
            masks.data_ptr(), masks.shape[1], wl.num_seqs, N,
            wl.max_prefix_len, wl.max_nodes, Hq, wl.num_kv_heads, d,
            wl.scale, splits, out.data_ptr(), lse.data_ptr()]
    ws = None
    if with_ws:
        nb = api.workspace_size(wl.num_seqs, N, Hq, wl.num_kv_heads, d,
                                wl.max_prefix_len, wl.max_nodes,
                                wl.page_size, splits)
        ws = torch.zeros((max(nb, 256),), dtype=torch.uint8, device="cuda:0")
        args += [ws.data_ptr(), ws.numel()]
    args.append(torch.cuda.current_stream().cuda_stream)
    code = getattr(api._lib, fn_name)(*args)
    torch.cuda.synchronize()
    return code, out, lse


def test_noalloc_matches_verify_twice():
    import tree_masked_attention_amd.api as api
    cases = [
        (standard_workload("qwen3-8b-b256-p4k"), 0),
        (make_workload(401, name="smaller", prefix_lens=[700, 300, 33],
                       tree_sizes=[40, 20, 64], num_q_heads=8,
                       num_kv_heads=2), 3),
    ]
    for wl, splits in cases:
        plan = api.describe_plan(wl.num_seqs, wl.total_nodes, wl.num_q_heads,
                                 wl.num_kv_heads, 128, wl.max_prefix_len,
                                 wl.max_nodes, wl.page_size, splits)
        say(f"[gpu] noalloc vs verify on {wl.name}: plan {plan}")
        assert plan["splits"] > 1  # the scratch holds partials and counters
        dev = device_inputs(wl)
        masks, _ = api.build_mask(dev["parents"], dev["tree_offsets"],
                                  max(wl.max_nodes, 1), wl.mask_words())
        c0, out0, lse0 = _call(api, "tree_attn_verify", wl, dev, masks,
                               splits, True)
        c1, out1, lse1 = _call(api, "tree_attn_verify_noalloc", wl, dev,
                               masks, splits, False)
        assert c0 == api.OK and c1 == api.OK, (c0, c1)
        assert torch.equal(out0.view(torch.int16), out1.view(torch.int16))
        assert torch.equal(lse0.view(torch.int32), lse1.view(torch.int32))
        ref_o, ref_l = oracle.workload_attention(wl)
        got = dict(out=out1.float().cpu().numpy().astype(np.float64),
                   lse=lse1.cpu().numpy().astype(np.float64))
        assert_parity(got, ref_o, ref_l, f"noalloc {wl.name}")


def test_noalloc_refuses_plans_beyond_its_scratch():
    import tree_masked_attention_amd.api as api
    wl = make_workload(402, name="many-splits", prefix_lens=[30000],
                       tree_sizes=[256], num_q_heads=32, num_kv_heads=8)
    nb = api.workspace_size(1, wl.total_nodes, 32, 8, 128, wl.max_prefix_len,
                            wl.max_nodes, 16, 256)
    assert nb > api.NOALLOC_SCRATCH_BYTES
    dev = device_inputs(wl)
    masks, _ = api.build_mask(dev["parents"], dev["tree_offsets"], 256,
                              wl.mask_words())
    code, out, _ = _call(api, "tree_attn_verify_noalloc", wl, dev, masks,
                         256, False)
    assert code == api.ERR_WORKSPACE
    assert torch.isnan(out.float()).all()  # nothing was launched
