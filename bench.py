#!/usr/bin/env python3
"""Benchmark of the tree-verification attention hot path on one MI355X.

One step = one pass of the whole path over one batch: ancestor-bitmask
build (tree_attn_build_mask) + verification attention (tree_attn_verify,
split-KV pass with the tree keys masked in registers, then the LSE merge).
Inputs are resident in HBM before timing; the input sets are rotated over
enough copies (>= 1 GiB in total) that no step finds its K/V in the 256 MB
Infinity Cache left there by the previous step.

Warmup runs the requested W steps and keeps going, back to back, until the
path has run for about 0.3 s.

--stage accept-commit times the step after the verification instead:
tree acceptance and the commit of the accepted rows' K/V (one fused launch,
with the two-launch form beside it), on tokens drawn for the workload.
--stage tree-build times the draft-tree construction before it.
--stage gdn times tree verification through a Gated DeltaNet layer
(tree_attn_gdn_verify) on its own synthetic workload (--gdn-seqs trees of
--gdn-nodes nodes, --gdn-heads heads of d_k = d_v = 128), with the
deferred state commit of an accepted path timed beside it.

Prints one JSON line on stdout.  Everything else goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

DEFAULT_WORKLOAD = "long-32k-4x-b256"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
ROTATE_BYTES = 1 << 30
WARM_SECONDS = 0.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--splits", type=int, default=0,
                    help="0 = planned by the library")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", action="store_true",
                    help="verify: time the chosen workload alone (by "
                         "default the other standard workloads are timed "
                         "after it and summarised in the same line)")
    ap.add_argument("--phases", action="store_true",
                    help="also time the two-launch form of the verification "
                         "(attention kernel writing split partials, then "
                         "the merge kernel)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle baseline")
    ap.add_argument("--stage", choices=("verify", "accept-commit",
                                        "tree-build", "gdn"),
                    default="verify",
                    help="verify: the verification path (default); "
                         "accept-commit: tree acceptance + KV commit, the "
                         "step after it; tree-build: draft-tree "
                         "construction, the step before it; gdn: tree "
                         "verification through a Gated DeltaNet layer "
                         "(and its state commit)")
    ap.add_argument("--gdn-seqs", type=int, default=16,
                    help="gdn: draft trees (sequences)")
    ap.add_argument("--gdn-nodes", type=int, default=128,
                    help="gdn: nodes per tree (<= 128)")
    ap.add_argument("--gdn-heads", type=int, default=32,
                    help="gdn: heads (d_k = d_v = 128)")
    ap.add_argument("--kv", choices=("bf16", "e4m3"), default="bf16",
                    help="verify: K/V cache element type (e4m3: FP8 with "
                         "per-kv-head scales, through tree_attn_verify_ex)")
    ap.add_argument("--head-dim", type=int, choices=(64, 128), default=128,
                    help="verify: head dimension (64 runs through "
                         "tree_attn_verify_ex)")
    ap.add_argument("--width", type=int, default=1,
                    help="tree-build: candidates taken per step (1 = strict "
                         "best-first)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 512 MiB device copies (the "
                         "reference kernel for scaling HBM byte counters)")
    return ap.parse_args()


HERE = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(HERE, "profiles", "hbm_traffic.txt")


# HIP sources of each measured kernel: HBM counters taken on other sources
# of that kernel are not reported
KERNEL_SOURCES = {
    "attn_fwdh_kernel<8>": ("common.hpp", "split_plan.hpp", "attn_merge.hpp",
                            "attn_fwd.hpp", "attn_fwd128h.hpp"),
    "attn_fwdh_kernel<4>": ("common.hpp", "split_plan.hpp", "attn_merge.hpp",
                            "attn_fwd.hpp", "attn_fwd128h.hpp"),
    "attn_fwd256_kernel": ("common.hpp", "split_plan.hpp", "attn_merge.hpp",
                           "attn_fwd.hpp", "attn_fwd8.hpp"),
    "attn_merge_kernel": ("common.hpp", "split_plan.hpp", "attn_merge.hpp"),
    "gdn_verify_kernel": ("common.hpp", "gdn.hpp"),
}


def kernel_source_hash(kernel):
    """Hash of the HIP sources a kernel is built from."""
    import hashlib
    csrc = os.path.join(HERE, "tree_masked_attention_amd", "csrc")
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def copy_bandwidth(torch, dev, stream, mib=512, reps=10):
    """HBM bandwidth of a plain device-to-device copy (bytes read + bytes
    written per second, GB/s), the practical ceiling the attention
    kernel's HBM figure is also compared with."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del src, dst
    return 2 * n / sec / 1e9


def measured_traffic(workload, kernel):
    """HBM bytes per launch of one kernel from the committed counter
    summary, when it was taken on the kernel's current sources; else
    None."""
    try:
        lines = open(TRAFFIC_FILE).read().splitlines()
    except OSError:
        return None
    for ln in lines:
        f = ln.split()
        if len(f) < 2 or f[0] != workload:
            continue
        for x in f[1:]:
            if x.startswith(kernel + ":"):
                parts = dict(y.split("=") for y in x[len(kernel) + 1:].split(","))
                if parts.get("sources") != kernel_source_hash(kernel):
                    return None
                try:
                    return float(parts["fetch"]) + float(parts["write"])
                except (KeyError, ValueError):
                    return None
    return None


def copy_calibration(torch):
    dev = torch.device("cuda:0")
    n = 512 << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n,
                      "launches": 5}), flush=True)
    return 0


# --------------------------------------------------------------------------
# algorithmic work of one verify launch
# --------------------------------------------------------------------------

def algorithmic_work(wl, with_output=True, kv_bytes=None):
    """(bytes, flops) the method must move / compute for one verify call.

    bytes: K and V of every cached token read once, q read and out written
    once (bf16), lse written (fp32), the ancestor masks and the page-table
    entries read once (without out and lse when with_output is False: the
    split pass of a split call leaves them to the merge).  flops: 4*d per
    allowed (query, key) pair (2*d for q.k, 2*d for p*v); masked-out tree
    pairs are not counted.
    """
    d, Hq, Hkv, ps = wl.head_dim, wl.num_q_heads, wl.num_kv_heads, wl.page_size
    if kv_bytes is None:
        kv_bytes = 1 if wl.kv_format == "e4m3" else 2
    P = wl.prefix_lens.astype(np.int64)
    B = wl.tree_sizes
    N = wl.total_nodes
    W = wl.mask_words()
    tokens = P + B
    nbytes = (int(tokens.sum()) * Hkv * d * kv_bytes * 2 + N * Hq * d * 2 +
              N * W * 8 + 4 * int(((tokens + ps - 1) // ps).sum()))
    if with_output:
        nbytes += N * Hq * d * 2 + N * Hq * 4
    pairs = 0
    for s in range(wl.num_seqs):
        a, b = int(wl.tree_offsets[s]), int(wl.tree_offsets[s + 1])
        par = wl.parents[a:b]
        depth = np.zeros(b - a, dtype=np.int64)
        for i in range(b - a):
            depth[i] = 0 if par[i] < 0 else depth[par[i]] + 1
        pairs += int(P[s]) * (b - a) + int((depth + 1).sum())
    flops = 4 * d * Hq * pairs
    return nbytes, flops


# --------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on the host cores
# --------------------------------------------------------------------------

def cpu_model():
    """Model name of the host CPU (for the baseline's record)."""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()]
                   or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_baseline(wl, target_s):
    """The oracle as it stands (mask build + fp64 attention) on whole
    sequences of the workload, in order and cycling, until about target_s
    seconds have passed (at least one sequence, at most about 30 s); the
    rate is the tree tokens of the sequences done per second."""
    import oracle
    threads = blas_threads()
    S = wl.num_seqs
    W = wl.mask_words()
    done, seqs, t = 0, 0, 0.0
    t0 = time.perf_counter()
    while True:
        s = seqs % S
        a, b = int(wl.tree_offsets[s]), int(wl.tree_offsets[s + 1])
        oracle.ancestor_masks(wl.parents[a:b], np.array([0, b - a]), W)
        oracle.workload_attention(wl, seq_ids=[s])
        done += b - a
        seqs += 1
        t = time.perf_counter() - t0
        if t >= target_s or t / seqs * (seqs + 1) > 30.0:
            break
    return {"value": done / t, "unit": "tree tokens/s",
            "cores": int(threads), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{seqs} sequence(s) of workload {wl.name}, in "
                      f"order and cycling ({done} tree tokens; one pass of "
                      f"the workload has {wl.total_nodes}): mask build + "
                      f"fp64 attention over all kv heads, {t:.1f} s"}


def cpu_baseline_accept(wl, tokens, target_s):
    import oracle
    d, t, r = tokens
    reps, el = 0, 0.0
    t0 = time.perf_counter()
    while True:
        lens, nodes, _ = oracle.accept(wl.parents, wl.tree_offsets, d, t, r,
                                       wl.max_nodes)
        oracle.commit_kv(wl.k_cache, wl.v_cache, wl.page_table,
                         wl.prefix_lens, lens, nodes)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or el / reps * (reps + 1) > 30.0:
            break
    return {"value": wl.total_nodes * reps / el, "unit": "tree tokens/s",
            "cores": 1, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{reps} full pass(es) of workload {wl.name} "
                      f"(acceptance + commit on copies of the caches), "
                      f"{el:.1f} s"}


def accept_commit_stage(args, torch, api, wl, sets, stream):
    """Times the step after the verification: tree_attn_accept +
    tree_attn_commit_kv (two launches) and tree_attn_accept_commit (one
    launch, the reported value).  Masks are built once per input copy
    beforehand."""
    from tree_masked_attention_amd.workloads import draw_tokens
    dev = torch.device("cuda:0")
    N, S, W = wl.total_nodes, wl.num_seqs, wl.mask_words()
    max_b = max(wl.max_nodes, 1)
    tokens = draw_tokens(wl, 1)
    tok = [torch.from_numpy(a).to(dev) for a in tokens]
    lens = torch.empty((max(S, 1),), dtype=torch.int32, device=dev)
    nodes = torch.empty((max(S, 1), max_b), dtype=torch.int32, device=dev)
    bonus = torch.empty((max(S, 1),), dtype=torch.int32, device=dev)
    token_bytes = wl.num_kv_heads * wl.head_dim * 2
    sptr = stream.cuda_stream
    calls = []
    for c in sets:
        masks, _ = api.build_mask(c["parents"], c["offs"], max_b, W)
        c["masks"] = masks
        acc = (c["parents"].data_ptr(), c["offs"].data_ptr(),
               masks.data_ptr(), W, tok[0].data_ptr(), tok[1].data_ptr(),
               tok[2].data_ptr(), S, N, max_b, lens.data_ptr(),
               nodes.data_ptr(), bonus.data_ptr(), sptr)
        com = (c["k"].data_ptr(), c["v"].data_ptr(), c["table"].data_ptr(),
               wl.max_pages_per_seq, wl.num_pages, wl.page_size,
               c["prefix"].data_ptr(), lens.data_ptr(), nodes.data_ptr(), S,
               max_b, token_bytes, sptr)
        calls.append((acc, com))
    f_acc = api._lib.tree_attn_accept
    f_com = api._lib.tree_attn_commit_kv
    f_fused = api._lib.tree_attn_accept_commit

    def step_accept(i):
        return f_acc(*calls[i % len(calls)][0])

    def step_commit(i):
        return f_com(*calls[i % len(calls)][1])

    def step_separate(i):
        return step_accept(i) | step_commit(i)

    def step_fused(i):
        a, cm = calls[i % len(calls)]
        # tree_attn_accept_commit takes the accept arguments, then the
        # cache arguments of tree_attn_commit_kv, then the outputs
        return f_fused(*a[:10], cm[0], cm[1], cm[2], cm[3], cm[4], cm[5],
                       cm[6], cm[11], *a[10:])

    def loop_ms(step):
        """per-step time of K back-to-back steps after a warmup"""
        n_warm = 0
        t_w = time.perf_counter()
        while n_warm < max(args.warmup, 1) or time.perf_counter() - t_w < 0.1:
            if step(n_warm) != 0:
                raise RuntimeError("tree_attn call failed during warmup")
            n_warm += 1
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(args.steps):
            step(i)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps, n_warm

    acc_ms, _ = loop_ms(step_accept)
    com_ms, _ = loop_ms(step_commit)
    sep_ms, _ = loop_ms(step_separate)
    ms_per_step, n_warm = loop_ms(step_fused)

    # The fused kernel runs for a few microseconds, about what the host
    # needs to issue a launch from Python, so this per-launch figure is
    # bounded by the launch rate; the kernel trace gives the kernel's own
    # time.  (A HIP graph of the launches is no way out: its kernels
    # overlapped, 0.9 us per launch for a 3.6 us kernel.)
    fused_ms = ms_per_step

    L = lens[:S].cpu().numpy()
    nd = nodes[:S].cpu().numpy()
    moved = int(sum(int((nd[s, :L[s]] != np.arange(L[s])).sum())
                    for s in range(S)))
    # commit: each moved row read once and written once, in K and in V;
    # the accepted lists and page-table entries read once
    com_bytes = moved * token_bytes * 2 * 2 + S * (max_b * 4 + 12) + \
        8 * moved
    # accept: per node its parent, draft and target token, the target token
    # of its parent and its mask row; per sequence the outputs
    acc_bytes = N * (16 + W * 8) + S * (max_b * 4 + 12)
    log(f"[bench] back-to-back launches: accept {acc_ms * 1e3:.1f} us, "
        f"commit {com_ms * 1e3:.1f} us, both {sep_ms * 1e3:.1f} us, fused "
        f"{ms_per_step * 1e3:.1f} us; tau {L.tolist()[:8]}, {moved} rows "
        f"moved")
    fused_bytes = com_bytes + acc_bytes
    achieved = fused_bytes / (fused_ms * 1e-3) / 1e9
    result = {
        "metric": "tree acceptance + KV commit, tree tokens/s",
        "value": N / (ms_per_step * 1e-3),
        "unit": "tree tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_warm,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int32",
        "data": "synthetic",
        "config": {
            "workload": wl.name, "stage": "accept-commit", "num_seqs": S,
            "tree_nodes_per_seq": int(wl.max_nodes),
            "token_bytes": token_bytes, "accepted": [int(x) for x in L][:8],
            "rows_moved": moved,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "tree_attn_accept_commit (accept_commit_kernel)",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": None,
            "alg_bytes_per_launch": fused_bytes,
            "avg_launch_us": fused_ms * 1e3,
        },
        "separate_ms_per_step": sep_ms,
        "accept_us": acc_ms * 1e3,
        "accept_alg_bytes": acc_bytes,
        "commit_us": com_ms * 1e3,
        "commit_alg_bytes": com_bytes,
    }
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline_accept(wl, tokens,
                                                     args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


TREE_DEPTH, TREE_TOPK = 16, 8  # per-depth head outputs for tree building


def tree_build_stage(args, torch, api, wl, stream):
    """Times tree_attn_build_tree for the workload's trees: num_seqs trees
    of its budget from synthetic per-depth top-k head outputs."""
    from tree_masked_attention_amd.workloads import draw_draft_topk
    import oracle
    dev = torch.device("cuda:0")
    S, B = wl.num_seqs, int(wl.max_nodes)
    D, K = TREE_DEPTH, TREE_TOPK
    lp, tok = draw_draft_topk(S, D, K, seed=3)
    lp_d, tok_d = torch.from_numpy(lp).to(dev), torch.from_numpy(tok).to(dev)
    outs = [torch.empty((S, B), dtype=dt, device=dev)
            for dt in (torch.int32, torch.int32, torch.int32, torch.float32)]
    sizes = torch.empty((S,), dtype=torch.int32, device=dev)
    f = api._lib.tree_attn_build_tree
    argv = (lp_d.data_ptr(), tok_d.data_ptr(), S, D, K, B, args.width,
            outs[0].data_ptr(), outs[1].data_ptr(), outs[2].data_ptr(),
            outs[3].data_ptr(), sizes.data_ptr(), stream.cuda_stream)
    n_warm = 0
    t_w = time.perf_counter()
    while n_warm < max(args.warmup, 1) or time.perf_counter() - t_w < 0.1:
        if f(*argv) != 0:
            raise RuntimeError("tree_attn_build_tree failed")
        n_warm += 1
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        f(*argv)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # check the last result against the oracle before reporting
    ref = oracle.build_trees(lp, tok, B, args.width)
    if not (np.array_equal(outs[0].cpu().numpy(), ref["parents"]) and
            np.array_equal(sizes.cpu().numpy(), ref["sizes"])):
        raise RuntimeError("tree build differs from the oracle")
    alg_bytes = S * D * K * 8 + S * B * 16 + 4 * S
    log(f"[bench] tree build: {S} x {B} nodes (depth {D}, top-{K}, width "
        f"{args.width}): {ms * 1e3:.2f} us per launch")
    result = {
        "metric": "draft-tree construction, tree nodes/s",
        "value": S * B / (ms * 1e-3),
        "unit": "tree nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_warm,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "stage": "tree-build",
                   "num_seqs": S, "budget": B, "depth": D, "topk": K,
                   "width": args.width},
        "roofline": {
            "bound": "latency",
            "kernel": "build_tree_kernel (tree_attn_build_tree)",
            "achieved": alg_bytes / (ms * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": alg_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
            "traffic": None,
            "alg_bytes_per_launch": alg_bytes,
            "avg_launch_us": ms * 1e3,
            "note": "one wave per tree, B dependent extraction steps",
        },
    }
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle)")
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.build_trees(lp, tok, B, args.width)
            reps += 1
            el = time.perf_counter() - t0
            if el >= min(args.cpu_seconds, 5.0) or el / reps * (reps + 1) > 30:
                break
        result["cpu_baseline"] = {
            "value": S * B * reps / el, "unit": "tree nodes/s", "cores": 1,
            "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{reps} full pass(es) of the same {S} trees, {el:.1f} s"}
    print(json.dumps(result), flush=True)
    return 0


# --------------------------------------------------------------------------
# Gated DeltaNet tree verification
# --------------------------------------------------------------------------

def gdn_work(S, B, H, depth_sum, W, d=128):
    """(bytes, flops) of one tree_attn_gdn_verify call that the method
    needs: q, k, v read once (bf16), g and beta (fp32), the ancestor masks
    (once per tree), S0 (fp32, d x d per sequence and head), out (bf16) and
    u (fp32) written once.  flops: K S0 and Q S0 (2 * 2 B d^2), the Gram
    products over ancestor-or-self pairs (2 * 2 d each), the triangular
    solve over strict-ancestor pairs and the output over ancestor-or-self
    pairs (2 d each), per sequence and head; depth_sum = sum over all
    nodes of the number of ancestor-or-self nodes."""
    N = S * B
    nbytes = (N * H * d * 2 * 3 + N * H * 4 * 2 + N * W * 8 +
              S * H * d * d * 4 + N * H * d * (2 + 4))
    anc_self = depth_sum
    strict = depth_sum - N
    flops = H * (2 * 2 * N * d * d + 2 * 2 * anc_self * d +
                 2 * strict * d + 2 * anc_self * d)
    return nbytes, flops


def gdn_stage(args, torch, api):
    """Times tree_attn_gdn_verify (and tree_attn_gdn_commit) on synthetic
    Gated DeltaNet inputs: --gdn-seqs trees of --gdn-nodes nodes drawn with
    the pchain rule, --gdn-heads heads."""
    from tree_masked_attention_amd.workloads import (draw_gdn_inputs,
                                                     gdn_trees)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    S, B, H, d = args.gdn_seqs, args.gdn_nodes, args.gdn_heads, 128
    N = S * B
    name = f"gdn-h{H}-b{B}-x{S}"
    parents, offsets = gdn_trees([B] * S, "pchain", 7)
    x = draw_gdn_inputs(S, N, 7, heads=H)
    depth = np.zeros(N, np.int64)
    for i in range(N):
        p = int(parents[i])
        local = i - int(offsets[i // B])
        depth[i] = 1 if p < 0 else depth[i - local + p] + 1
    W = api.mask_words_for(B)
    alg_bytes, alg_flops = gdn_work(S, B, H, int(depth.sum()), W, d)
    # input copies rotated so that no launch finds its inputs in the
    # 256 MB Infinity Cache
    copies = max(2, min(16, int(math.ceil(ROTATE_BYTES / alg_bytes))))
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    par_d = torch.from_numpy(parents).to(dev)
    off_d = torch.from_numpy(offsets).to(dev)
    masks, _ = api.build_mask(par_d, off_d, B)
    sets = []
    for c in range(copies):
        q, k, v = (bf(a).to(dev) for a in x[:3])
        g, beta, S0 = (torch.from_numpy(np.ascontiguousarray(a)).to(dev)
                       for a in x[3:])
        out = torch.empty((N, H, d), dtype=torch.bfloat16, device=dev)
        u = torch.empty((N, H, d), dtype=torch.float32, device=dev)
        sets.append((q, k, v, g, beta, S0, out, u))
    f = api._lib.tree_attn_gdn_verify
    argv = [(t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(),
             t[3].data_ptr(), t[4].data_ptr(), t[5].data_ptr(),
             off_d.data_ptr(), masks.data_ptr(), W, S, N, B, H, d,
             t[6].data_ptr(), t[7].data_ptr(), stream.cuda_stream)
            for t in sets]
    n_warm = 0
    t_w = time.perf_counter()
    while n_warm < max(args.warmup, 1) or time.perf_counter() - t_w < \
            WARM_SECONDS:
        if f(*argv[n_warm % copies]) != 0:
            raise RuntimeError("tree_attn_gdn_verify failed")
        n_warm += 1
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        f(*argv[i % copies])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # the commit of one accepted root path per tree (depth-first to the
    # deepest node of the tree), back to back on the same stream
    rng = np.random.default_rng(8)
    lens = np.zeros(S, np.int32)
    nodes = np.full((S, B), -1, np.int32)
    for s in range(S):
        a = int(offsets[s])
        j = int(np.argmax(depth[a:a + B]))
        path = []
        while j >= 0:
            path.append(j)
            j = int(parents[a + j])
        lens[s] = len(path)
        nodes[s, :len(path)] = path[::-1]
    lens_d = torch.from_numpy(lens).to(dev)
    nodes_d = torch.from_numpy(nodes).to(dev)
    fc = api._lib.tree_attn_gdn_commit
    cargv = [(t[1].data_ptr(), t[7].data_ptr(), t[3].data_ptr(),
              off_d.data_ptr(), lens_d.data_ptr(), nodes_d.data_ptr(), S, B,
              H, d, t[5].data_ptr(), stream.cuda_stream) for t in sets]
    for i in range(3):
        fc(*cargv[i % copies])
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        if fc(*cargv[i % copies]) != 0:
            raise RuntimeError("tree_attn_gdn_commit failed")
    e1.record(stream)
    torch.cuda.synchronize()
    commit_ms = e0.elapsed_time(e1) / args.steps
    commit_bytes = S * H * d * d * 4 * 2 + int(lens.sum()) * H * (d * 6 + 4)

    # check one (sequence, head) of the last launch against the oracle
    import oracle
    from tree_masked_attention_amd.workloads import bf16_bits_to_f32
    sets[0][5].copy_(torch.from_numpy(x[5]))  # the commits changed S0
    f(*argv[0])
    torch.cuda.synchronize()
    o_gpu = sets[0][6][:B, 0].float().cpu().numpy()
    u_gpu = sets[0][7][:B, 0].cpu().numpy()
    q32, k32, v32 = (bf16_bits_to_f32(a)[:B, :1] for a in x[:3])
    ro, ru = oracle.gdn_tree_verify(parents[:B], q32, k32, v32, x[3][:B, :1],
                                    x[4][:B, :1], x[5][0, :1])
    if not (np.abs(u_gpu - ru[:, 0]).max() <= 2e-4 * (1 + np.abs(ru).max()) and
            np.abs(o_gpu - ro[:, 0]).max() <= 2 ** -8 * np.abs(ro).max() + 2e-4):
        raise RuntimeError("GDN verify differs from the oracle")

    sec = ms * 1e-3
    ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
    NT = (B + 31) // 32
    T1 = NT * (NT + 1) // 2
    mfma_per_wg = 4 * (NT * 8 * 4 + 6 * (NT * (NT - 1) // 2) + 6 * NT +
                       6 * T1) + 2 * T1 * 8
    exec_flops = S * H * mfma_per_wg * 32 * 32 * 16 * 2
    log(f"[bench] gdn verify {name}: {ms * 1e3:.1f} us per launch "
        f"({alg_bytes / sec / 1e9:.0f} GB/s algorithmic, "
        f"{alg_flops / sec / 1e12:.1f} TFLOP/s algorithmic, "
        f"{exec_flops / sec / 1e12:.1f} TFLOP/s executed on MFMA); "
        f"commit {commit_ms * 1e3:.1f} us")
    result = {
        "metric": "GDN tree-verify tree tokens/s + achieved HBM GB/s",
        "value": N / sec,
        "unit": "tree tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_warm,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 in, f32 math",
        "data": "synthetic",
        "config": {"workload": name, "stage": "gdn", "num_seqs": S,
                   "tree_nodes_per_seq": B, "heads": H, "d_k": d, "d_v": d,
                   "tree_rule": "pchain 0.5", "input_copies_rotated": copies},
        "roofline": {
            "bound": "hbm" if alg_flops / alg_bytes < ridge else "mfma",
            "kernel": "gdn_verify_kernel (tree_attn_gdn_verify)",
            "achieved": alg_bytes / sec / 1e9,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": alg_bytes / sec / 1e9 / HBM_PEAK_GBPS,
            "traffic": measured_traffic(name, "gdn_verify_kernel"),
            "alg_bytes_per_launch": alg_bytes,
            "alg_flops_per_launch": alg_flops,
            "avg_launch_us": ms * 1e3,
            "executed_mfma_tflops": exec_flops / sec / 1e12,
            "executed_mfma_frac": exec_flops / sec / 1e12 /
                                  MFMA_BF16_PEAK_TFLOPS,
        },
        "commit_us": commit_ms * 1e3,
        "commit_hbm_gbps": commit_bytes / (commit_ms * 1e-3) / 1e9,
        "commit_path_lens": f"{int(lens.min())}..{int(lens.max())}",
    }
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle)")
        q32, k32, v32 = (bf16_bits_to_f32(a) for a in x[:3])
        pairs, t0 = 0, time.perf_counter()
        while pairs < S * H:
            sq, hd = divmod(pairs, H)
            a, hs = sq * B, slice(hd, hd + 1)
            oracle.gdn_tree_verify(parents[a:a + B], q32[a:a + B, hs],
                                   k32[a:a + B, hs], v32[a:a + B, hs],
                                   x[3][a:a + B, hs], x[4][a:a + B, hs],
                                   x[5][sq, hs])
            pairs += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or el / pairs * (pairs + 1) > 30:
                break
        el = time.perf_counter() - t0
        result["cpu_baseline"] = {
            "value": B * pairs / H / el, "unit": "tree tokens/s",
            "cores": 1, "cpu_model": cpu_model(), "kind": "oracle",
            "sample": f"{pairs} (tree, head) pairs of {B} nodes, first "
                      f"trees first, all heads of a tree in turn, {el:.1f} s"}
    print(json.dumps(result), flush=True)
    return 0


# --------------------------------------------------------------------------
# GPU timing
# --------------------------------------------------------------------------

# --------------------------------------------------------------------------
# verification timing
# --------------------------------------------------------------------------

def device_sets(torch, wl, dev):
    """Copies of the workload's inputs on the device, enough of them
    (>= 1 GiB in all) that no step finds its K/V in the 256 MB Infinity
    Cache left there by the previous step."""
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    if wl.kv_format == "bf16":
        kv_host = dict(k=bf(wl.k_cache), v=bf(wl.v_cache))
    else:
        kv_host = dict(k=torch.from_numpy(wl.k_cache),
                       v=torch.from_numpy(wl.v_cache),
                       ks=torch.from_numpy(wl.k_scale),
                       vs=torch.from_numpy(wl.v_scale))
    host = dict(q=bf(wl.q), **kv_host,
                table=torch.from_numpy(wl.page_table),
                prefix=torch.from_numpy(wl.prefix_lens),
                offs=torch.from_numpy(wl.tree_offsets),
                parents=torch.from_numpy(wl.parents))
    per_copy = sum(t.numel() * t.element_size() for t in host.values())
    copies = int(min(256, max(2, math.ceil(ROTATE_BYTES / per_copy))))
    log(f"[bench] {wl.name}: {per_copy / 2**20:.1f} MiB per input set, "
        f"{copies} copies")
    sets = [{k: t.to(dev) for k, t in host.items()} for _ in range(copies)]
    return sets, copies


def per_launch(torch, stream, fn, pick, steps):
    """Milliseconds per call of K calls back to back on the launch stream
    between one pair of events (input copies rotated): the kernel's own
    time plus the dispatch gap between consecutive launches."""
    for i in range(3):
        fn(*pick(i))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        if fn(*pick(i)) != 0:
            raise RuntimeError("tree_attn call failed")
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def per_call(torch, stream, fn, pick, reps=20):
    """Median and minimum over single calls: an event between every two
    consecutive calls of a back-to-back run (input copies rotated), so
    each interval is one call plus its dispatch gap, without the host's
    launch latency."""
    for i in range(3):
        fn(*pick(i))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(reps):
        if fn(*pick(i)) != 0:
            raise RuntimeError("tree_attn call failed")
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    times = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps))
    return {"median": times[len(times) // 2], "min": times[0], "calls": reps}


class VerifyBench:
    """Pre-marshalled C-ABI calls of one workload (mask build + verify),
    one argument list per input copy."""

    def __init__(self, torch, api, wl, sets, splits, stream):
        self.torch, self.api, self.wl, self.stream = torch, api, wl, stream
        dev = sets[0]["q"].device
        N, Hq, d = wl.q.shape
        S, W = wl.num_seqs, wl.mask_words()
        max_b = max(wl.max_nodes, 1)
        self.variant = wl.kv_format != "bf16" or wl.head_dim != 128
        self.masks = torch.empty((N, W), dtype=torch.int64, device=dev)
        self.bad = torch.empty((max(S, 1),), dtype=torch.int32, device=dev)
        self.out = torch.empty((N, Hq, d), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((N, Hq), dtype=torch.float32, device=dev)
        kvd = api.KV_FP8_E4M3 if wl.kv_format == "e4m3" else api.KV_BF16
        self.ws_bytes = int(api._lib.tree_attn_workspace_size_ex(
            kvd, S, N, Hq, wl.num_kv_heads, d, wl.max_prefix_len,
            wl.max_nodes, wl.page_size, splits))
        # zero-filled once: the split launch's arrival counters start at 0
        self.ws = torch.zeros((max(self.ws_bytes, 256),), dtype=torch.uint8,
                              device=dev)
        sptr = stream.cuda_stream
        ws, masks = self.ws, self.masks
        self.calls = []
        for c in sets:
            mask_args = (c["parents"].data_ptr(), c["offs"].data_ptr(), S, N,
                         max_b, W, masks.data_ptr(), self.bad.data_ptr(),
                         sptr)
            if self.variant:
                ver_args = (c["q"].data_ptr(), c["k"].data_ptr(),
                            c["v"].data_ptr(), kvd,
                            c["ks"].data_ptr() if "ks" in c else None,
                            c["vs"].data_ptr() if "vs" in c else None,
                            c["table"].data_ptr(), wl.max_pages_per_seq,
                            wl.num_pages, wl.page_size,
                            c["prefix"].data_ptr(), c["offs"].data_ptr(),
                            masks.data_ptr(), W, S, N, wl.max_prefix_len,
                            wl.max_nodes, Hq, wl.num_kv_heads, d, wl.scale,
                            splits, self.out.data_ptr(), self.lse.data_ptr(),
                            ws.data_ptr(), ws.numel(), sptr)
            else:
                ver_args = (c["q"].data_ptr(), c["k"].data_ptr(),
                            c["v"].data_ptr(), c["table"].data_ptr(),
                            wl.max_pages_per_seq, wl.num_pages, wl.page_size,
                            c["prefix"].data_ptr(), c["offs"].data_ptr(),
                            masks.data_ptr(), W, S, N, wl.max_prefix_len,
                            wl.max_nodes, Hq, wl.num_kv_heads, d, wl.scale,
                            splits, self.out.data_ptr(), self.lse.data_ptr(),
                            ws.data_ptr(), ws.numel(), sptr)
            self.calls.append((mask_args, ver_args))
        self.f_mask = api._lib.tree_attn_build_mask
        self.f_ver = (api._lib.tree_attn_verify_ex if self.variant
                      else api._lib.tree_attn_verify)
        if self.variant:
            # fp8 K/V or head dim 64: the same tuned kernels and plan
            self.plan = api.describe_plan_ex(kvd, S, N, Hq, wl.num_kv_heads,
                                             d, wl.max_prefix_len,
                                             wl.max_nodes, wl.page_size,
                                             splits)
        else:
            self.plan = api.describe_plan(S, N, Hq, wl.num_kv_heads, d,
                                          wl.max_prefix_len, wl.max_nodes,
                                          wl.page_size, splits)

    def mask_args(self, i):
        return self.calls[i % len(self.calls)][0]

    def ver_args(self, i):
        return self.calls[i % len(self.calls)][1]

    def step(self, i):
        return self.f_mask(*self.mask_args(i)) | self.f_ver(*self.ver_args(i))

    def warm(self, warmup):
        """W warmup steps, then as many more as fill WARM_SECONDS, enqueued
        back to back like the timed steps.  Under sustained back-to-back
        load the GPU's power management lowers clocks, so the whole-step
        figure is the sustained rate; the per-launch figures, taken with
        small gaps between launches, run at higher clocks."""
        torch = self.torch
        t_w = time.perf_counter()
        n = 0
        for _ in range(max(warmup, 1)):
            if self.step(n) != 0:
                raise RuntimeError("tree_attn call failed during warmup")
            n += 1
        torch.cuda.synchronize()
        per = (time.perf_counter() - t_w) / n
        extra = int(max(0.0, WARM_SECONDS - (time.perf_counter() - t_w)) /
                    per)
        for _ in range(extra):
            self.step(n)
            n += 1
        torch.cuda.synchronize()
        log(f"[bench] warmup: {n} steps ({warmup} requested), "
            f"{time.perf_counter() - t_w:.2f} s")
        return n

    def kernel_name(self):
        return {256: "attn_fwd256_kernel", 128: "attn_fwdh_kernel<8>",
                64: "attn_fwdh_kernel<4>"}[self.plan["rows"]]

    def measure(self, steps):
        """Per-launch verify and mask-build times and the verify launch's
        algorithmic rates (the one attention launch does all the method's
        flops and bytes, its merge included)."""
        torch, st = self.torch, self.stream
        mask_ms = per_launch(torch, st, self.f_mask, self.mask_args, steps)
        ver_ms = per_launch(torch, st, self.f_ver, self.ver_args, steps)
        call = per_call(torch, st, self.f_ver, self.ver_args)
        nbytes, flops = algorithmic_work(self.wl)
        ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBPS * 1e9)
        sec = ver_ms * 1e-3
        return {"verify_us": ver_ms * 1e3, "verify_call_us": call,
                "mask_build_us": mask_ms * 1e3, "alg_bytes": nbytes,
                "alg_flops": flops,
                "bound": "mfma" if flops / nbytes > ridge else "hbm",
                "tflops": flops / sec / 1e12, "hbm_gbps": nbytes / sec / 1e9,
                "plan": self.plan}


def summary_entry(wl, m):
    """One workload's line of the all-workload summary."""
    return {"verify_us": m["verify_us"],
            "verify_call_median_us": m["verify_call_us"]["median"],
            "tree_tokens_per_s": wl.total_nodes / (m["verify_us"] * 1e-6),
            "bound": m["bound"],
            "tflops": m["tflops"],
            "frac_mfma_bf16": m["tflops"] / MFMA_BF16_PEAK_TFLOPS,
            "hbm_gbps": m["hbm_gbps"],
            "frac_hbm": m["hbm_gbps"] / HBM_PEAK_GBPS,
            "alg_bytes": m["alg_bytes"], "alg_flops": m["alg_flops"],
            "plan": m["plan"]}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only "
              f"(--gpus {args.gpus} requested); nothing was run.",
              file=sys.stderr)
        return 2
    import torch
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import tree_masked_attention_amd.api as api
    from tree_masked_attention_amd.workloads import (STANDARD_ORDER,
                                                     standard_workload)

    assert torch.cuda.is_available(), "bench.py needs a ROCm GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        return copy_calibration(torch)

    if args.stage == "gdn":
        return gdn_stage(args, torch, api)
    log(f"[bench] drawing workload {args.workload}")
    wl = standard_workload(args.workload, kv_format=args.kv,
                           head_dim=args.head_dim)
    if args.stage == "tree-build":
        return tree_build_stage(args, torch, api, wl,
                                torch.cuda.current_stream())
    stream = torch.cuda.current_stream()
    sets, copies = device_sets(torch, wl, dev)
    if args.stage == "accept-commit":
        return accept_commit_stage(args, torch, api, wl, sets, stream)

    vb = VerifyBench(torch, api, wl, sets, args.splits, stream)
    n_warm = vb.warm(args.warmup)
    # checked on the host: a torch comparison/reduction here would be the
    # process's first launch of those kernels, and their module load was
    # measured to slow the next ~25 ms of launches (the timed loop) by ~10%
    if (vb.bad[:wl.num_seqs].cpu().numpy() != -1).any():
        raise RuntimeError("invalid tree in benchmark input")

    # (1) whole-step throughput: K back-to-back steps (mask build + verify)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        vb.step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # (2) per-launch durations of the mask build and of the verify launch
    m = vb.measure(args.steps)
    phases = None
    if args.phases and not vb.variant:
        # the two-launch form (attention kernel writing partials, then the
        # merge kernel); its attention launches carry the same kernel name,
        # so a kernel trace of such a run mixes the two forms
        f_att = api._lib.tree_attn_verify_attend
        f_mer = api._lib.tree_attn_verify_merge
        att_ms = per_launch(torch, stream, f_att, vb.ver_args, args.steps)
        mer_ms = (per_launch(torch, stream, f_mer, vb.ver_args, args.steps)
                  if vb.plan["splits"] > 1 else 0.0)
        phases = {"attend_us": att_ms * 1e3, "merge_us": mer_ms * 1e3}
    log(f"[bench] {wl.name}: step {ms_per_step * 1e3:.1f} us; mask build "
        f"{m['mask_build_us']:.1f} us; verify {m['verify_us']:.1f} us back "
        f"to back, single calls median {m['verify_call_us']['median']:.1f} "
        f"/ min {m['verify_call_us']['min']:.1f} us"
        + (f" (two-launch form: attend {phases['attend_us']:.1f} us + merge "
           f"{phases['merge_us']:.1f} us)" if phases else ""))

    N, Hq, d = wl.q.shape
    S = wl.num_seqs
    kname = vb.kernel_name()
    bound = m["bound"]
    frac_m = m["tflops"] / MFMA_BF16_PEAK_TFLOPS
    frac_h = m["hbm_gbps"] / HBM_PEAK_GBPS
    if bound == "hbm":
        achieved, peak, unit, frac = (m["hbm_gbps"], HBM_PEAK_GBPS, "GB/s",
                                      frac_h)
    else:
        achieved, peak, unit, frac = (m["tflops"], MFMA_BF16_PEAK_TFLOPS,
                                      "TFLOP/s", frac_m)
    result = {
        "metric": "tree-verify attention tree tokens/s + achieved HBM GB/s "
                  "/ MFMA% of peak",
        "value": N / (ms_per_step * 1e-3),
        "unit": "tree tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": n_warm,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.kv_format == "bf16" else "bf16 q, e4m3 kv",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "kv_format": wl.kv_format,
            "num_seqs": S,
            "prefix_lens": ([int(x) for x in wl.prefix_lens] if S <= 8
                            else f"{S} x {int(wl.prefix_lens[0])}"),
            "tree_nodes_per_seq": int(wl.max_nodes),
            "q_heads": Hq, "kv_heads": wl.num_kv_heads, "head_dim": d,
            "page_size": wl.page_size,
            "splits_requested": args.splits or "planned",
            "plan": vb.plan,
            "input_copies_rotated": copies,
        },
        "roofline": {
            "bound": bound,
            "kernel": (f"{kname} with its merge (tree_attn_verify_ex, one "
                       f"call)" if vb.variant
                       else f"{kname} (tree_attn_verify, one launch)"),
            "achieved": achieved,
            "peak": peak,
            "unit": unit,
            "frac": frac,
            "traffic": measured_traffic(wl.name, kname),
            "tflops": m["tflops"],
            "frac_mfma_bf16": frac_m,
            "hbm_gbps": m["hbm_gbps"],
            "frac_hbm": frac_h,
            "alg_bytes_per_launch": m["alg_bytes"],
            "alg_flops_per_launch": m["alg_flops"],
            "avg_launch_us": m["verify_us"],
        },
        "verify_us": m["verify_us"],
        "verify_call_us": m["verify_call_us"],
        "mask_build_us": m["mask_build_us"],
        "verify_tflops": m["tflops"],
        "verify_hbm_gbps": m["hbm_gbps"],
    }
    if phases:
        result["two_launch_form"] = phases
    if bound == "hbm":
        cp = copy_bandwidth(torch, dev, stream)
        result["roofline"]["measured_copy_gbps"] = cp
        result["roofline"]["frac_of_measured_copy"] = achieved / cp
    if not args.only and not vb.variant and args.splits == 0:
        # the other standard workloads, timed the same way (per launch,
        # inputs rotated), each with both roofline fractions
        del vb, sets
        torch.cuda.empty_cache()
        summary = {wl.name: summary_entry(wl, m)}
        for name in STANDARD_ORDER:
            if name == wl.name:
                continue
            log(f"[bench] workload {name}")
            w2 = standard_workload(name)
            sets2, _ = device_sets(torch, w2, dev)
            vb2 = VerifyBench(torch, api, w2, sets2, 0, stream)
            vb2.warm(args.warmup)
            summary[name] = summary_entry(w2, vb2.measure(args.steps))
            log(f"[bench]   verify {summary[name]['verify_us']:.1f} us, "
                f"{summary[name]['tflops']:.0f} TFLOP/s "
                f"({summary[name]['frac_mfma_bf16']:.3f}), "
                f"{summary[name]['hbm_gbps']:.0f} GB/s "
                f"({summary[name]['frac_hbm']:.3f})")
            del vb2, sets2
            torch.cuda.empty_cache()
        result["workloads"] = summary
    if not args.no_cpu_baseline:
        log("[bench] CPU baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
