"""Split partials keep bf16's range (needs a gfx950 GPU).

Values far beyond fp16's finite range (|v| up to about 5e5) go through
forced key-range splits, whose partials travel in fp16 with a power-of-two
scale per row, on the tuned kernels (bf16 and FP8 K/V, head dims 128
and 64).  The
attention output is linear in V, so the bar scales with V: max |out -
oracle| <= 2e-2 * value_scale; the lse does not depend on V (1e-3
relative, as everywhere).  The scale is a power of two, so the scaled bf16
values are exact multiples of the unscaled ones.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import LSE_RTOL, OUT_ATOL, errors, run_gpu, say
from tree_masked_attention_amd.workloads import make_workload

pytestmark = pytest.mark.gpu

VSCALE = 2.0 ** 17


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    import tree_masked_attention_amd.api  # noqa: F401  (fails loudly if unbuilt)


def _check(label, got_out, got_lse, ref_out, ref_lse):
    eo, el = errors(got_out, got_lse, ref_out, ref_lse)
    say(f"  {label}: max|dout|/scale={eo / VSCALE:.3e} max rel dlse={el:.3e}")
    assert np.isfinite(got_out).all() and np.isfinite(got_lse).all(), label
    assert eo <= OUT_ATOL * VSCALE, f"{label}: out error {eo}"
    assert el <= LSE_RTOL, f"{label}: lse error {el}"


# (workload kwargs, forced split counts, rows per workgroup expected)
TUNED = {
    "128-rows": (dict(prefix_lens=[900, 317], tree_sizes=[40, 70],
                      num_q_heads=8, num_kv_heads=2), (2, 5, 64), 128),
    "256-rows": (dict(prefix_lens=[9000], tree_sizes=[64], num_q_heads=16,
                      num_kv_heads=4), (2, 4), 256),
}


@pytest.mark.parametrize("name", sorted(TUNED))
def test_large_values_tuned_kernels(name):
    import tree_masked_attention_amd.api as api
    kw, split_list, rows = TUNED[name]
    wl = make_workload(301, name=name, value_scale=VSCALE, **kw)
    vmax = np.abs(oracle.widen_bf16(wl.v_cache)).max()
    say(f"[gpu] large V ({name}): max|v| = {vmax:.3e}")
    assert vmax > 4 * 65504
    ref_o, ref_l = oracle.workload_attention(wl)
    for splits in split_list:
        plan = api.describe_plan(wl.num_seqs, wl.total_nodes, wl.num_q_heads,
                                 wl.num_kv_heads, 128, wl.max_prefix_len,
                                 wl.max_nodes, wl.page_size, splits)
        assert plan["splits"] > 1 and plan["rows"] == rows, plan
        got = run_gpu(wl, num_splits=splits)
        _check(f"{name} {plan['splits']} splits", got["out"], got["lse"],
               ref_o, ref_l)


@pytest.mark.parametrize("fmt,d", [("bf16", 64), ("e4m3", 128),
                                   ("e4m3", 64)])
def test_large_values_other_formats(fmt, d):
    from test_gpu_variants import run_ex
    wl = make_workload(302, name=f"big-v-{fmt}-{d}", prefix_lens=[700, 90],
                       tree_sizes=[33, 64], num_q_heads=8, num_kv_heads=2,
                       kv_format=fmt, head_dim=d, value_scale=VSCALE)
    ref_o, ref_l = oracle.workload_attention(wl)
    say(f"[gpu] large V {fmt} d={d}: "
        f"max|v| = {np.nanmax(np.abs(ref_o)):.3e} (output)")
    for splits in (2, 5):
        out, lse = run_ex(wl, num_splits=splits)
        _check(f"{fmt} d={d} {splits} splits", out.astype(np.float64), lse,
               ref_o, ref_l)
