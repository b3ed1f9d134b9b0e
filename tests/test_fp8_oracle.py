"""Pins of the oracle's FP8 (E4M3) cache support (CPU).

* the decoder matches torch's float8_e4m3fn conversion on all 256 codes
  (a library routine standing in for the format's published table), and
  hand values from the format definition;
* attention over an E4M3 cache with power-of-two per-head scales equals
  attention over a bf16 cache holding the dequantised values (exact: an
  E4M3 value times a power of two is a bf16 value);
* planted mistakes (bias 8 as in the FNUZ variant, scales ignored,
  subnormals flushed, the K scale applied to V) each fail a pin.
"""

import numpy as np
import pytest
import torch

import oracle.tree_oracle as T
from tree_masked_attention_amd.workloads import (f32_to_bf16_bits,
                                                 make_workload)


def pin_decoder_vs_library():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    got = T.widen_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(got[~nan], ref[~nan].astype(np.float64))


def pin_decoder_hand_values():
    cases = {0x38: 1.0, 0x7E: 448.0, 0xFE: -448.0, 0x01: 2.0 ** -9,
             0x08: 2.0 ** -6, 0x07: 7 * 2.0 ** -9, 0x80: -0.0, 0x3C: 1.5,
             0x40: 2.0, 0x30: 0.5}
    got = T.widen_e4m3(np.array(list(cases), dtype=np.uint8))
    assert got.tolist() == list(cases.values())
    assert np.isnan(T.widen_e4m3(np.array([0x7F, 0xFF], np.uint8))).all()


def _as_bf16_workload(wl):
    """The same workload with the dequantised caches stored as bf16."""
    import copy
    b = copy.copy(wl)
    k = T.widen_e4m3(wl.k_cache) * wl.k_scale[None, None, :, None]
    v = T.widen_e4m3(wl.v_cache) * wl.v_scale[None, None, :, None]
    b.k_cache = f32_to_bf16_bits(k.astype(np.float32))
    b.v_cache = f32_to_bf16_bits(v.astype(np.float32))
    # exact: the bf16 round trip must not change any value
    assert np.array_equal(T.widen_bf16(b.k_cache), k)
    assert np.array_equal(T.widen_bf16(b.v_cache), v)
    b.kv_format, b.k_scale, b.v_scale = "bf16", None, None
    return b


def pin_fp8_equals_dequantised_bf16():
    for seed, d in ((1, 128), (2, 64)):
        wl = make_workload(seed, prefix_lens=[37, 5], tree_sizes=[9, 14],
                           num_q_heads=4, num_kv_heads=2, head_dim=d,
                           kv_format="e4m3")
        # different scales per head, so a swapped or ignored scale shows
        wl.k_scale = (wl.k_scale * np.array([1.0, 4.0], np.float32))
        wl.v_scale = (wl.v_scale * np.array([0.5, 2.0], np.float32))
        o8, l8 = T.workload_attention(wl)
        ob, lb = T.workload_attention(_as_bf16_workload(wl))
        assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


def pin_scale_moves_lse():
    # scaling every K of a head by 2 doubles its scores: softmax changes, so
    # the lse must differ from the unscaled one
    wl = make_workload(3, prefix_lens=[20], tree_sizes=[6], num_q_heads=2,
                       num_kv_heads=1, kv_format="e4m3")
    _, l1 = T.workload_attention(wl)
    wl.k_scale = wl.k_scale * 2
    _, l2 = T.workload_attention(wl)
    assert not np.allclose(l1, l2)


PINS = [pin_decoder_vs_library, pin_decoder_hand_values,
        pin_fp8_equals_dequantised_bf16, pin_scale_moves_lse]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_fp8_pin(pin):
    pin()


_orig_widen = T.widen_e4m3
_orig_gather = T._gather_tokens


def _mut_bias8(codes):
    b = np.asarray(codes).astype(np.int64)
    v = _orig_widen(codes)
    return np.where((b & 0x78) != 0, v / 2.0, v)


def _mut_flush_subnormals(codes):
    b = np.asarray(codes).astype(np.int64)
    v = _orig_widen(codes)
    return np.where((b & 0x78) == 0, 0.0 * v, v)


def _mut_scale_ignored(cache, row, n, kv_format="bf16", head_scale=None):
    return _orig_gather(cache, row, n, kv_format, None)


@pytest.mark.parametrize("target,mutant", [
    ("widen_e4m3", _mut_bias8),
    ("widen_e4m3", _mut_flush_subnormals),
    ("_gather_tokens", _mut_scale_ignored),
], ids=["bias8", "flush-subnormals", "scale-ignored"])
def test_fp8_pins_catch_planted_mistake(target, mutant, monkeypatch):
    monkeypatch.setattr(T, target, mutant)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0
