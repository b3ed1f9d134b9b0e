"""Helpers for the GPU tests: move a workload to the device, run the HIP
path through the C ABI, compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

OUT_ATOL = 2e-2      # max |out_gpu - out_oracle|
LSE_RTOL = 1e-3      # max |lse_gpu - lse_oracle| / max(|lse_oracle|, 1)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def device_inputs(wl, device="cuda:0"):
    d = torch.device(device)
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(d)
    return dict(
        q=bf(wl.q), k_cache=bf(wl.k_cache), v_cache=bf(wl.v_cache),
        page_table=torch.from_numpy(wl.page_table).to(d),
        prefix_lens=torch.from_numpy(wl.prefix_lens).to(d),
        tree_offsets=torch.from_numpy(wl.tree_offsets).to(d),
        parents=torch.from_numpy(wl.parents).to(d),
    )


def run_gpu(wl, num_splits=0, dev=None, mask_words=None):
    """build_mask + verify through the C ABI; returns numpy results."""
    import tree_masked_attention_amd.api as api
    dev = dev or device_inputs(wl)
    W = mask_words or wl.mask_words()
    masks, bad = api.build_mask(dev["parents"], dev["tree_offsets"],
                                max(wl.max_nodes, 1), W)
    out, lse = api.verify(dev["q"], dev["k_cache"], dev["v_cache"],
                          dev["page_table"], dev["prefix_lens"],
                          dev["tree_offsets"], masks, wl.max_prefix_len,
                          wl.max_nodes, wl.scale, num_splits=num_splits)
    torch.cuda.synchronize()
    return dict(
        masks=masks.cpu().numpy().view(np.uint64),
        bad=bad.cpu().numpy()[:wl.num_seqs],
        out=out.float().cpu().numpy().astype(np.float64),
        lse=lse.cpu().numpy().astype(np.float64),
        out_bits=out.view(torch.int16).cpu().numpy(),
    )


def errors(got_out, got_lse, ref_out, ref_lse):
    """(max abs out error, max relative lse error) over computed entries."""
    sel = ~np.isnan(ref_lse)
    eo = np.abs(got_out[sel] - ref_out[sel]).max() if sel.any() else 0.0
    el = (np.abs(got_lse[sel] - ref_lse[sel]) /
          np.maximum(np.abs(ref_lse[sel]), 1.0)).max() if sel.any() else 0.0
    return float(eo), float(el)


def assert_parity(got, ref_out, ref_lse, label=""):
    assert np.isfinite(got["out"]).all(), f"{label}: non-finite output"
    assert np.isfinite(got["lse"]).all(), f"{label}: non-finite lse"
    eo, el = errors(got["out"], got["lse"], ref_out, ref_lse)
    say(f"  {label}: max|dout|={eo:.3e} max rel dlse={el:.3e}")
    assert eo <= OUT_ATOL, f"{label}: out error {eo}"
    assert el <= LSE_RTOL, f"{label}: lse error {el}"
    return eo, el
