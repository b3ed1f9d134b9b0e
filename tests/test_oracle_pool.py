"""The pooled oracle runs (tests/oracle_pool.py) equal the oracle on the
whole workload, bit for bit: the (sequence, kv head) pieces carry every
input those rows depend on, in the order the page table gives."""

import numpy as np

import oracle
from oracle_pool import oracle_by_pairs
from tree_masked_attention_amd.workloads import make_workload


def test_pieces_equal_whole():
    wl = make_workload(7, prefix_lens=[37, 0, 130], tree_sizes=[9, 5, 20],
                       num_q_heads=8, num_kv_heads=2, page_size=8,
                       key_factor_range=(0.5, 2.0))
    ref_o, ref_l = oracle.workload_attention(wl)
    pairs = [(s, g) for s in range(3) for g in range(2)]
    got_o, got_l = oracle_by_pairs(wl, pairs, workers=2)
    assert np.array_equal(got_o, ref_o)
    assert np.array_equal(got_l, ref_l)


def test_pieces_equal_whole_e4m3():
    wl = make_workload(8, prefix_lens=[20, 50], tree_sizes=[6, 11],
                       num_q_heads=4, num_kv_heads=2, kv_format="e4m3")
    ref_o, ref_l = oracle.workload_attention(wl)
    got_o, got_l = oracle_by_pairs(wl, [(0, 0), (0, 1), (1, 0), (1, 1)],
                                   workers=2)
    assert np.array_equal(got_o, ref_o)
    assert np.array_equal(got_l, ref_l)
