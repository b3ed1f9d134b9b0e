"""Oracle runs in worker processes, for the full-size parity tests.

Test infrastructure.  The oracle's rows of one (sequence s, kv head g)
pair depend only on that sequence's cached tokens of kv head g, the q rows
of g's query-head group and the sequence's tree.  So each task carries
just those inputs -- the sequence's pages gathered in logical order with an
identity page table, one kv head, G query heads -- and the worker calls
oracle.tree_attention on them unchanged.  The pages are taken in the order
the page table lists them, which is the gather the oracle itself performs;
tests/test_oracle_pool.py checks on small inputs that the pieces equal the
oracle run on the whole workload, bit for bit.
"""

from __future__ import annotations

import math
import multiprocessing
import os
from typing import Iterable, List, Tuple

import numpy as np


def sub_problem(wl, s: int, g: int) -> dict:
    """Keyword arguments of oracle.tree_attention for pair (s, g) alone."""
    a, b = int(wl.tree_offsets[s]), int(wl.tree_offsets[s + 1])
    G = wl.num_q_heads // wl.num_kv_heads
    P = int(wl.prefix_lens[s])
    npg = max(1, math.ceil((P + b - a) / wl.page_size))
    pages = wl.page_table[s, :npg]
    kw = dict(q=np.ascontiguousarray(wl.q[a:b, g * G:(g + 1) * G]),
              k_cache=np.ascontiguousarray(wl.k_cache[pages][:, :, g:g + 1]),
              v_cache=np.ascontiguousarray(wl.v_cache[pages][:, :, g:g + 1]),
              page_table=np.arange(npg, dtype=np.int64)[None, :],
              prefix_lens=np.array([P]),
              tree_offsets=np.array([0, b - a]),
              parents=np.ascontiguousarray(wl.parents[a:b]),
              scale=wl.scale, kv_format=wl.kv_format)
    if wl.k_scale is not None:
        kw["k_scale"] = wl.k_scale[g:g + 1]
        kw["v_scale"] = wl.v_scale[g:g + 1]
    return kw


def _run(kw):
    import oracle
    return oracle.tree_attention(**kw)


def oracle_by_pairs(wl, pairs: Iterable[Tuple[int, int]], workers: int = 8
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """Oracle (out [N, Hq, d], lse [N, Hq]) with the given pairs filled in
    (NaN elsewhere), computed by `workers` spawned processes."""
    pairs = list(pairs)
    tasks = [sub_problem(wl, s, g) for s, g in pairs]
    N, Hq, d = wl.q.shape
    G = wl.num_q_heads // wl.num_kv_heads
    out = np.full((N, Hq, d), np.nan)
    lse = np.full((N, Hq), np.nan)
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS",
                                            "OPENBLAS_NUM_THREADS")}
    os.environ["OMP_NUM_THREADS"] = os.environ["OPENBLAS_NUM_THREADS"] = "2"
    try:
        ctx = multiprocessing.get_context("spawn")
        with ctx.Pool(max(1, min(workers, len(tasks)))) as pool:
            results: List = pool.map(_run, tasks, chunksize=1)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    for (s, g), (o, l) in zip(pairs, results):
        a, b = int(wl.tree_offsets[s]), int(wl.tree_offsets[s + 1])
        out[a:b, g * G:(g + 1) * G] = o
        lse[a:b, g * G:(g + 1) * G] = l
    return out, lse
