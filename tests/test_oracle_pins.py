"""The CPU oracle against its pins, and the pins against planted mistakes.

A planted mistake is a plausible slip in the oracle (self excluded from
the ancestor set, siblings leaking in, wrong GQA grouping, page table
ignored, log base 2, no normalisation, mask bits reversed).  Each one is
planted in the oracle on the CPU through monkeypatching, and at least one
pin must then fail.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.tree_oracle as T
import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def _excl_self(parents_local):
    return [s - {i} for i, s in enumerate(_ORIG["anc"](parents_local))]


def _index_causal(prefix_len, anc, tree_size):
    row = np.zeros(prefix_len + tree_size, dtype=bool)
    row[:prefix_len + max(anc) + 1] = True
    return row


def _shift_one(prefix_len, anc, tree_size):
    row = np.zeros(prefix_len + tree_size, dtype=bool)
    row[:prefix_len] = True
    for j in anc:
        row[prefix_len + j - 1] = True
    return row


def _gqa_modulo(h, hq, hkv):
    return h % hkv


def _no_table(cache_bits, table_row, num_tokens, kv_format="bf16",
              head_scale=None):
    ps = cache_bits.shape[1]
    t = np.arange(num_tokens)
    first = int(table_row[0])
    return T.widen_bf16(cache_bits[(first + t // ps) % cache_bits.shape[0],
                                   t % ps])


def _log2_lse(scores, allowed, values):
    o, l = _ORIG["sm"](scores, allowed, values)
    return o, l / math.log(2.0)


def _unnormalised(scores, allowed, values):
    s = np.where(allowed, scores, -np.inf)
    m = s.max(axis=1, keepdims=True)
    w = np.where(allowed, np.exp(s - m), 0.0)
    return w @ values, (m + np.log(w.sum(axis=1, keepdims=True)))[:, 0]


def _reversed_bits(parents, tree_offsets, mask_words):
    m = _ORIG["masks"](parents, tree_offsets, mask_words)
    out = np.zeros_like(m)
    for b in range(64):
        out |= ((m >> np.uint64(b)) & np.uint64(1)) << np.uint64(63 - b)
    return out


_ORIG = {"anc": T._ancestor_sets, "sm": T._masked_softmax_attention,
         "masks": T.ancestor_masks}

MUTANTS = {
    "self_excluded": ("_ancestor_sets", _excl_self),
    "siblings_leak": ("_allowed_keys", _index_causal),
    "tree_position_off_by_one": ("_allowed_keys", _shift_one),
    "gqa_modulo": ("_kv_head_of", _gqa_modulo),
    "page_table_ignored": ("_gather_tokens", _no_table),
    "lse_base2": ("_masked_softmax_attention", _log2_lse),
    "no_normalisation": ("_masked_softmax_attention", _unnormalised),
    "mask_bits_reversed": ("ancestor_masks", _reversed_bits),
}


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_planted_mistake(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(T, attr, fn)
    if attr == "ancestor_masks":
        monkeypatch.setattr(oracle, "ancestor_masks", fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(oracle)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {mutant}"
