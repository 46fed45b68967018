#!/usr/bin/env python3
"""Benchmark of the shared-index decode step on one MI355X.

One step = one pass of the whole hot path over one batch: the indexer scores
every cached key once, the top-k keeps k positions per query, and each of the
N layers runs gathered sparse attention with that one index (CLSA: one
indexer, N cross-decoder layers over one shared KV cache). Default workload:
the 128K-context decode (B=4, kv_len=131072, 64x128 bf16 indexer, k=2048,
16 layers, 32 q / 8 KV heads, dim 128, 1% needle keys), synthetic seeded
inputs resident in HBM before the timed region starts. Consecutive timed steps
cycle through N_ROT sets of queries (same caches), so each step computes a new
index, as consecutive decode steps do.

Prints one JSON line: tokens/s for the step (K timed steps, nothing enqueued
between them), the step's spread and its cold-cache time, and the roofline
of the dominant kernel (the one with the larger share of the step): for the
sparse-attention call, algorithmic bytes (decode) or flops (chunk) over its
GPU time per call (back-to-back calls replayed from a HIP graph between one
event pair), warm and with the caches evicted before each call, plus the
HBM traffic rocprofv3 measured for it; for a chunk's indexer, its flops over
its time per call, with the attention call's figures nested beside it;
per-kernel times; a dense-gather run
of the same call (k = kv_len) for the speedup; and the CPU oracle timed on
one pinned host core on a bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--config decode128k]
"""

from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix cores
MFMA_FP8_PEAK_TFLOPS = 5000.0    # MI355X dense fp8 matrix cores
N_ROT = 4                        # query sets the timed steps cycle through
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sparse_attn_decode128k_traffic.txt")
ATTN_SOURCE = os.path.join(ROOT, "token_sparse_attention_clsa_amd", "csrc", "sparse_attn.hip")


def measured_traffic(config_name):
    """HBM bytes per attention call from the committed rocprofv3 counter summary
    (FETCH_SIZE + WRITE_SIZE, calibrated on a copy kernel), if that summary was
    taken on the current kernel source and this workload; else None."""
    import hashlib
    try:
        fields = dict(line.split("=", 1) for line in open(TRAFFIC_FILE).read().split("\n")
                      if "=" in line and not line.startswith("#"))
    except OSError:
        return None
    sha = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()
    if fields.get("source_sha256", "").strip() != sha or fields.get("workload", "").strip() != config_name:
        return None
    return float(fields["bytes_per_call"])


def algorithmic_bytes(wl):
    """Bytes each kernel of the step must move at least (its algorithmic traffic)."""
    bt = wl.B * wl.T
    e_kv = 2 if wl.dtype == 1 else 4
    e_idx = {0: 4, 1: 2, 2: 1}[wl.idx_dtype]
    vis_keys = sum(wl.kv_len - wl.T + t + 1 for t in range(wl.T)) * wl.B
    index_score = (vis_keys * wl.D_I * e_idx + bt * wl.H_I * wl.D_I * e_idx + bt * wl.H_I * 4
                   + bt * wl.kv_len * 4)
    topk = bt * wl.kv_len * 4 + bt * wl.k * 4
    attn = (bt * wl.k * wl.Hkv * wl.D * e_kv * 2      # gathered K and V rows
            + bt * wl.k * 4                            # index
            + 2 * bt * wl.Hq * wl.D * e_kv + bt * wl.Hq * 4)  # q, out, lse
    return {"index_score": index_score, "topk": topk, "sparse_attn": attn}


def host_cpu():
    """Host core count available to this process and the CPU model."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return len(os.sched_getaffinity(0)), model


def cpu_baseline(wl, X, budget_s=12.0):
    """The oracle's decode step (all layers, one indexer pass) on host copies of
    the same inputs, single-threaded and pinned to one core, one batch element
    per call, cycling over the batch until the time budget is spent (at least
    one call). For a chunk (T > 1) each call is one query of the chunk (T = 1
    with that query's visible length), queries taken evenly over the chunk."""
    import oracle
    from token_sparse_attention_clsa_amd import inputs as inp

    host = []
    for b in range(wl.B):
        memo = {}  # layers share one cache: copy each distinct tensor once

        def sl(t, tq=None):
            if t is None:
                return None
            key = (id(t), tq)
            if key not in memo:
                memo[key] = inp.raw(t[b:b + 1] if tq is None else t[b:b + 1, tq:tq + 1])
            return memo[key]

        host.append(sl)
    queries = [None] if wl.T == 1 else [int(i * (wl.T - 1) / 15) for i in range(16)]
    n_cores, model = host_cpu()
    old_aff = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {min(old_aff)})
    done, t_total = 0, 0.0
    try:
        while done == 0 or t_total < budget_s:
            sl = host[done % wl.B]
            tq = queries[(done // wl.B) % len(queries)]
            kv = wl.kv_len if tq is None else wl.kv_len - wl.T + tq + 1
            args = ([sl(t, tq) for t in X.q], [sl(t) for t in X.k_cache], [sl(t) for t in X.v_cache],
                    [sl(t, tq) for t in X.q_idx], [sl(t) for t in X.k_idx], [sl(t, tq) for t in X.w])
            t0 = time.perf_counter()
            oracle.decode_step(wl.layer_src, args[0], args[1], args[2], wl.dtype, args[3], args[4], args[5],
                               wl.idx_dtype, kv, wl.k)
            t_total += time.perf_counter() - t0
            done += 1
            if done >= 64 * len(queries) * wl.B:
                break
    finally:
        os.sched_setaffinity(0, old_aff)
    what = ("single-batch-element decode steps" if wl.T == 1 else
            f"single-query steps (16 queries spread over the {wl.T}-query chunk, each with its visible length)")

    # The same oracle over independent units on every host core: one thread
    # per core (the ctypes call releases the GIL; the oracle's decode tables
    # were filled by the single-core run above and are only read from here).
    from concurrent.futures import ThreadPoolExecutor
    n_thr = max(1, min(len(old_aff), 16))
    par_budget = budget_s / 2

    def worker(wid):
        calls, t_end = 0, time.perf_counter() + par_budget
        while calls == 0 or time.perf_counter() < t_end:
            u = wid + calls * n_thr
            sl = host[u % wl.B]
            tq = queries[(u // wl.B) % len(queries)]
            kv = wl.kv_len if tq is None else wl.kv_len - wl.T + tq + 1
            oracle.decode_step(wl.layer_src, [sl(t, tq) for t in X.q], [sl(t) for t in X.k_cache],
                               [sl(t) for t in X.v_cache], wl.dtype, [sl(t, tq) for t in X.q_idx],
                               [sl(t) for t in X.k_idx], [sl(t, tq) for t in X.w], wl.idx_dtype, kv, wl.k)
            calls += 1
        return calls

    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=n_thr) as ex:
        par_calls = sum(ex.map(worker, range(n_thr)))
    par_wall = time.perf_counter() - t0
    return {
        "value": done / t_total,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{done} {what} ({wl.n_layers} layers, {len(wl.f_layers)} indexer pass, "
                  f"kv_len {wl.kv_len}) of the same inputs, {t_total:.1f} s of CPU time on one "
                  f"pinned core",
        "host_cores": n_cores,
        "host_cpu": model,
        "parallel": {"value": par_calls / par_wall, "unit": "tokens/s", "threads": n_thr,
                     "sample": f"{par_calls} of the same units on {n_thr} threads, "
                               f"{par_wall:.1f} s wall"},
    }


def evict_caches(scratch):
    """Evicts the L2s and the 256 MB Infinity Cache: a 1 GiB fill and a read
    of it. The read leaves clean lines behind, so no write-back of the fill
    lands inside what runs next (after a fill alone a 128K decode attention
    call measured 24.9 us, after a fill and a read 17.3 us)."""
    scratch.fill_(1.0)
    scratch.sum()


def profile_attn(wl, X, step, mode, reps):
    """R attention calls of the step's first layer shapes over the step's
    index: back to back ("warm": a workgroup finds part of its rows in the L2
    of the XCD it ran on in the previous call, the rest in the Infinity
    Cache), each after a 64 MiB read ("l2flush": the L2s hold other data, the
    Infinity Cache still holds the rows) or each after evict_caches ("cold":
    rows come from HBM). Used under rocprofv3, whose per-kernel averages then
    describe that state."""
    import torch
    import token_sparse_attention_clsa_amd as clsa
    n = wl.n_layers
    ws = torch.empty(max(256, clsa.workspace_bytes(1, B=wl.B, T=wl.T, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, k=wl.k)),
                     dtype=torch.uint8, device="cuda")
    out = [torch.empty_like(X.q[l]) for l in range(n)]
    lse = [torch.empty((wl.B, wl.T, wl.Hq), dtype=torch.float32, device="cuda") for _ in range(n)]
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if mode == "cold" else None
    flush = torch.zeros(1 << 24, dtype=torch.float32, device="cuda") if mode == "l2flush" else None
    torch.cuda.synchronize()
    for i in range(reps):
        if scratch is not None:
            evict_caches(scratch)
        if flush is not None:
            flush.sum()
        clsa.sparse_attn(X.q[i % n], X.k_cache[i % n], X.v_cache[i % n], step.idx, kv_len=wl.kv_len,
                         out=out[i % n], lse=lse[i % n], ws=ws)
        if scratch is not None:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    print(f"[bench] {reps} {mode} attention calls done", file=sys.stderr, flush=True)


def measured_gemm_tflops():
    """The bf16 matrix-core rate a library GEMM reaches on this device: torch.mm
    (hipBLASLt) of two contiguous 8192 x 8192 bf16 operands, median of 5
    event-timed calls after 3 warm-up calls. The measured counterpart of the
    2.5 PFLOP/s spec peak, as the device copy is for HBM."""
    import torch
    n = 8192
    a = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    b = torch.randn((n, n), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((n, n), dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        torch.mm(a, b, out=c)
    ts = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.mm(a, b, out=c)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3)
    del a, b, c
    torch.cuda.empty_cache()
    return 2.0 * n ** 3 / statistics.median(ts) / 1e12


def contrast_indexers(wl, X, variant, device):
    """Indexer inputs for every layer: the workload's own on its F layers,
    new seeded ones (same recipe) on the others."""
    from token_sparse_attention_clsa_amd import inputs as inp
    qi, ki, w = [], [], []
    for l in range(wl.n_layers):
        if X.q_idx[l] is not None:
            qi.append(X.q_idx[l]); ki.append(X.k_idx[l]); w.append(X.w[l])
            continue
        base = 77000 + 4 * l
        if variant == "int":
            qi.append(inp.randint(X.q_idx[0].shape, -8, 8, wl.idx_dtype, base, device))
            ki.append(inp.randint(X.k_idx[0].shape, -8, 8, wl.idx_dtype, base + 1, device))
        else:
            qi.append(inp.randn(X.q_idx[0].shape, wl.idx_dtype, base, device))
            ki.append(inp.randn(X.k_idx[0].shape, wl.idx_dtype, base + 1, device))
        w.append(inp.weights(X.w[0].shape, variant, base + 2, device, bits=wl.weight_bits))
    return qi, ki, w


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="decode128k")
    ap.add_argument("--variant", default="gauss", choices=["gauss", "int"])
    ap.add_argument("--idx-dtype", default=None, choices=["bf16", "fp8"],
                    help="indexer query/key storage type (default: the workload's own)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-graph", action="store_true", help="skip the HIP-graph replay timing")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run 3 plain device copies of this many MiB first (counter calibration)")
    ap.add_argument("--profile-attn", choices=["warm", "l2flush", "cold"], default=None,
                    help="only run the step once, then R attention calls (back to back, each after "
                         "a 64 MiB read that replaces the L2s' contents, or each after evicting "
                         "every cache) and exit: the run a profiler wraps")
    ap.add_argument("--no-contrast", action="store_true",
                    help="skip the per-layer-indexer (every layer F) step used as the method's contrast")
    ap.add_argument("--batch-curve", type=lambda x: [int(v) for v in x.split(",") if v], default=[4, 8, 16, 32, 64],
                    help="batch sizes of the attention-call curve (decode; empty to skip)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the library runs the shared-index decode step on one GPU and does not shard it",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import token_sparse_attention_clsa_amd as clsa
    from token_sparse_attention_clsa_amd import inputs as inp

    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    clsa.load()
    wl = inp.config(args.config)
    if args.idx_dtype is not None:
        wl = inp.config(args.config, idx_dtype={"bf16": inp.BF16, "fp8": inp.FP8_E4M3FN}[args.idx_dtype])
    print(f"[bench] workload {wl.name}: B={wl.B} T={wl.T} kv_len={wl.kv_len} layers={wl.n_layers} "
          f"F={len(wl.f_layers)} k={wl.k}", file=sys.stderr, flush=True)
    if args.calib_copy_mib:
        src = torch.empty(args.calib_copy_mib << 18, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    X = inp.make(wl, args.variant, seed=7, device="cuda")
    n = wl.n_layers
    K, W = args.steps, args.warmup
    # Consecutive decode steps see new queries, hence a new index each step:
    # the timed steps cycle through N_ROT sets of attention and indexer
    # queries (same caches), so a step's first layer does not find its rows
    # in the caches from the step before, as it would if one step repeated.
    qsets = [(X.q, X.q_idx, X.w)]
    for r in range(1, N_ROT):
        qsets.append(([inp.randn(t.shape, wl.dtype, 9000 + 97 * r + l, "cuda") for l, t in enumerate(X.q)],
                      [None if t is None else inp.randn(t.shape, wl.idx_dtype, 9500 + 97 * r + l, "cuda")
                       for l, t in enumerate(X.q_idx)],
                      [None if t is None else inp.weights(t.shape, args.variant, 9900 + 97 * r + l, "cuda",
                                                          bits=wl.weight_bits)
                       for l, t in enumerate(X.w)]))
    if args.variant == "int":  # integer indexer queries, as in the first set
        qsets = qsets[:1] + [(q, [None if t is None else inp.randint(t.shape, -8, 8, wl.idx_dtype, 9700 + 97 * r + l,
                                                                       "cuda")
                                  for l, t in enumerate(qi)], w) for r, (q, qi, w) in enumerate(qsets[1:], 1)]

    def make_steps(**kw):
        return [clsa.DecodeStep(wl.layer_src, q, X.k_cache, X.v_cache, qi, X.k_idx, w, wl.k, kv_len=wl.kv_len, **kw)
                for q, qi, w in qsets]

    steps = make_steps()
    step = steps[0]
    for i in range(W):
        steps[i % N_ROT].run()
    torch.cuda.synchronize()
    print(f"[bench] warmup done ({W} steps)", file=sys.stderr, flush=True)
    if args.profile_attn:
        profile_attn(wl, X, step, args.profile_attn, max(K, 20))
        return

    # Timed region: exactly K steps, nothing else enqueued between them.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for i in range(K):
        steps[i % N_ROT].run()
    e1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / K
    ms_per_step_events = e0.elapsed_time(e1) / K
    print(f"[bench] timed {K} steps: {ms_per_step * 1e3:.1f} us/step (events {ms_per_step_events * 1e3:.1f})",
          file=sys.stderr, flush=True)

    # The N_ROT steps captured once in a HIP graph and replayed (one launch
    # per N_ROT steps instead of one per kernel; the work is identical).
    graph_ms = None
    if not args.no_graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for st in steps:
                st.run()  # the steps issue no allocations and no memset nodes
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for st in steps:
                st.run()
        reps = max(1, K // N_ROT)
        for _ in range(max(1, W // N_ROT)):
            g.replay()
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t2) * 1e3 / (reps * N_ROT)
        print(f"[bench] graph replay: {graph_ms * 1e3:.1f} us/step", file=sys.stderr, flush=True)

    # Where a step's time goes: the same steps with events recorded between
    # their stages (before each F layer's indexer, between it and its top-k,
    # around every attention call), one step at a time, medians over the
    # steps. Each recorded event adds about 1-2 us, so the stages sum to more
    # than the step.
    stage_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4 * n)] for _ in range(N_ROT)]
    st_ev = [clsa.DecodeStep(wl.layer_src, q, X.k_cache, X.v_cache, qi, X.k_idx, w, wl.k, kv_len=wl.kv_len,
                             events=stage_ev[i]) for i, (q, qi, w) in enumerate(qsets)]
    for st in st_ev:
        st.run()
    torch.cuda.synchronize()
    f_layers_ev = [l for l in range(n) if wl.layer_src[l] == l]
    t_idx, t_topk, t_a0, t_arest = [], [], [], []
    for i in range(max(N_ROT, min(K, 40))):
        st_ev[i % N_ROT].run()
        torch.cuda.synchronize()
        e = stage_ev[i % N_ROT]
        t_idx.append(sum(e[4 * l].elapsed_time(e[4 * l + 1]) for l in f_layers_ev) * 1e3)
        t_topk.append(sum(e[4 * l + 1].elapsed_time(e[4 * l + 2]) for l in f_layers_ev) * 1e3)
        t_a0.append(e[2].elapsed_time(e[3]) * 1e3)
        if n > 1:
            t_arest.append(statistics.mean(e[4 * l + 2].elapsed_time(e[4 * l + 3]) for l in range(1, n)) * 1e3)
    step_stages = {"indexer_us": statistics.median(t_idx), "topk_us": statistics.median(t_topk),
                   "attn_first_layer_us": statistics.median(t_a0),
                   "attn_other_layers_mean_us": statistics.median(t_arest) if t_arest else None,
                   "steps": len(t_idx),
                   "note": "per step: indexer and top-k summed over the F layers; events between the "
                           "stages, one step at a time: each recorded event adds about 1-2 us, so the "
                           "stages sum to more than ms_per_step"}
    del st_ev, stage_ev
    print(f"[bench] step stages: indexer {step_stages['indexer_us']:.1f} us, top-k {step_stages['topk_us']:.1f} us, "
          f"attention {step_stages['attn_first_layer_us']:.1f} us (first layer)", file=sys.stderr, flush=True)

    # The same step with a per-query count of kept positions (the dynamic-k
    # reading), counts drawn uniformly from [k/4, k] (seeded): GPU time of K
    # back-to-back steps between one event pair (the wall clock of the first
    # pass after this step's warmup has shown a one-off stall of ~16 ms before
    # the GPU starts, outside the steps themselves).
    gk = torch.Generator().manual_seed(17)
    kpq = torch.randint(wl.k // 4, wl.k + 1, (wl.B, wl.T), generator=gk, dtype=torch.int32).to("cuda")
    step_dk = make_steps(k_per_query=kpq)
    for i in range(W):
        step_dk[i % N_ROT].run()
    torch.cuda.synchronize()
    e3a, e3b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e3a.record()
    for i in range(K):
        step_dk[i % N_ROT].run()
    e3b.record()
    torch.cuda.synchronize()
    dynamic_k = {"k_per_query": f"uniform [{wl.k // 4}, {wl.k}]", "mean_k": float(kpq.float().mean()),
                 "ms_per_step_events": e3a.elapsed_time(e3b) / K}
    del step_dk

    # The same step with ordered skipping: the margin is the median over the
    # first full layer's queries of (best score - score at rank k/2), so the
    # median query keeps about half of its k positions. Same timing as above.
    f0 = wl.f_layers[0]
    sc = clsa.index_score(X.q_idx[f0], X.k_idx[f0], X.w[f0], kv_len=wl.kv_len)
    top = torch.topk(sc.view(wl.B * wl.T, wl.kv_len), min(wl.k, wl.kv_len - wl.T + 1), dim=1).values
    margin = float((top[:, 0] - top[:, top.shape[1] // 2 - 1]).median())
    _, kept = clsa.topk_margin(sc, wl.k, margin)
    del sc, top
    step_os = make_steps(skip_margin=margin)
    for i in range(W):
        step_os[i % N_ROT].run()
    torch.cuda.synchronize()
    e4a, e4b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e4a.record()
    for i in range(K):
        step_os[i % N_ROT].run()
    e4b.record()
    torch.cuda.synchronize()
    ordered_skip = {"margin": margin, "rule": "median query keeps ~k/2 of its top-k",
                    "mean_kept": float(kept.float().mean()), "ms_per_step_events": e4a.elapsed_time(e4b) / K}
    del step_os

    # The method's contrast on this GPU: the same step with every layer an F
    # layer (its own indexer inputs, indexer pass and top-k, as a DSA model
    # without index reuse runs it), against the workload's own layer map.
    contrast = None
    if not args.no_contrast and len(wl.f_layers) < n:
        qi_all, ki_all, w_all = contrast_indexers(wl, X, args.variant, "cuda")
        st_all = clsa.DecodeStep(list(range(n)), X.q, X.k_cache, X.v_cache, qi_all, ki_all, w_all, wl.k,
                                 kv_len=wl.kv_len)
        for _ in range(max(1, W // 2)):
            st_all.run()
        torch.cuda.synchronize()
        kc = max(5, K // 4)
        e5a, e5b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e5a.record()
        for _ in range(kc):
            st_all.run()
        e5b.record()
        torch.cuda.synchronize()
        ms_all = e5a.elapsed_time(e5b) / kc
        contrast = {
            "every_layer_indexer": {"indexer_passes": n, "ms_per_step_events": ms_all, "steps": kc},
            "this_layer_map": {"indexer_passes": len(wl.f_layers), "ms_per_step_events": ms_per_step_events},
            "step_speedup_from_index_reuse": ms_all / ms_per_step_events,
            "indexer_passes_removed": 1.0 - len(wl.f_layers) / n,
        }
        del st_all, qi_all, ki_all, w_all
        torch.cuda.empty_cache()
        print(f"[bench] every-layer-indexer step: {ms_all * 1e3:.1f} us", file=sys.stderr, flush=True)

    # Per-kernel averages: R back-to-back calls of one entry point, same
    # shapes and inputs as the step. The R calls are captured once in a HIP
    # graph and replayed between one event pair on the replay stream, so the
    # figure is GPU time per call (the gap between a call's kernels
    # included) without the Python call overhead; --no-graph times the
    # direct calls instead (host-bound for short kernels).
    f0 = wl.f_layers[0]
    R = max(4 * K, 64)
    scores = torch.empty((wl.B, wl.T, wl.kv_len), dtype=torch.float32, device="cuda")
    idx = step.idx
    topk_ws = torch.empty(clsa.workspace_bytes(0, B=wl.B, T=wl.T, kv_len=wl.kv_len, k=wl.k),
                          dtype=torch.uint8, device="cuda")
    attn_ws = torch.zeros(max(256, clsa.workspace_bytes(1, B=wl.B, T=wl.T, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D,
                                                        k=wl.k)), dtype=torch.uint8, device="cuda")
    out = [torch.empty_like(X.q[l]) for l in range(n)]
    lse = [torch.empty((wl.B, wl.T, wl.Hq), dtype=torch.float32, device="cuda") for _ in range(n)]

    def per_launch_us(fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if args.no_graph:
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            a.record()
            for i in range(R):
                fn(i)
            b.record()
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / R
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(3):
                fn(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(R):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / R

    us_index = per_launch_us(lambda i: clsa.index_score(X.q_idx[f0], X.k_idx[f0], X.w[f0], kv_len=wl.kv_len,
                                                        out=scores))
    us_topk = per_launch_us(lambda i: clsa.topk(scores, wl.k, out=idx, ws=topk_ws))
    us_attn = per_launch_us(lambda i: clsa.sparse_attn(X.q[i % n], X.k_cache[i % n], X.v_cache[i % n], idx,
                                                       kv_len=wl.kv_len, out=out[i % n], lse=lse[i % n],
                                                       ws=attn_ws))
    # Cache append of the step's new tokens (rows kv_len-T .. kv_len-1 written
    # again with copies of themselves, so the caches do not change).
    pos = wl.kv_len - wl.T
    new_rows = [X.k_cache[0][:, pos:wl.kv_len].clone(), X.v_cache[0][:, pos:wl.kv_len].clone(),
                X.k_idx[f0][:, pos:wl.kv_len].clone()]
    us_append = per_launch_us(lambda i: clsa.cache_append(new_rows[0], new_rows[1], X.k_cache[0],
                                                          X.v_cache[0], pos, new_rows[2], X.k_idx[f0]))
    del new_rows

    alg = algorithmic_bytes(wl)
    attn_gbs = alg["sparse_attn"] / (us_attn * 1e-6) / 1e9

    # Cold figures: a 1 GiB fill and a read of it before each timed call (or
    # step) evict the L2s and the 256 MB Infinity Cache. The read leaves them
    # holding clean lines: after a fill alone, the write-back of its dirty
    # lines lands inside the timed call (measured: 24.9 us per decode128k
    # attention call after a fill, 17.3 us after a fill and a read). The
    # flush also keeps the GPU busy while the host enqueues the event pair
    # and the call, so the pair brackets GPU time only. Median over the
    # repetitions.
    scratch = torch.empty(1 << 28, dtype=torch.float32, device="cuda")

    def cold_us(fn, reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for i in range(reps + 2):
            evict_caches(scratch)
            a.record()
            fn(i)
            b.record()
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(a.elapsed_time(b) * 1e3)
        return statistics.median(ts)

    us_attn_cold = cold_us(lambda i: clsa.sparse_attn(X.q[i % n], X.k_cache[i % n], X.v_cache[i % n], idx,
                                                      kv_len=wl.kv_len, out=out[i % n], lse=lse[i % n],
                                                      ws=attn_ws), 20)

    # The first layer of a real step finds its index and queries in cache
    # (the top-k and the previous layer just wrote them) and only its rows
    # cold: the same eviction, then the index and the query re-read.
    def cold_rows_only(i):
        evict_caches(scratch)
        idx.sum()
        X.q[i % n].float().sum()

    def cold_rows_us(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for i in range(reps + 2):
            cold_rows_only(i)
            a.record()
            clsa.sparse_attn(X.q[i % n], X.k_cache[i % n], X.v_cache[i % n], idx, kv_len=wl.kv_len,
                             out=out[i % n], lse=lse[i % n], ws=attn_ws)
            b.record()
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(a.elapsed_time(b) * 1e3)
        return statistics.median(ts)

    us_attn_cold_rows = cold_rows_us(20) if wl.T == 1 else None

    # As cold_rows_only, and the call's kernels run once on a tiny input
    # first, so their code and launch path are warm as in a step (every
    # layer runs the same two kernels); only the rows come from HBM.
    us_attn_cold_rows_warm_code = None
    if wl.T == 1:
        kt = inp.randn((wl.B, 64, wl.Hkv, wl.D), wl.dtype, 35000, "cuda")
        vt = inp.randn((wl.B, 64, wl.Hkv, wl.D), wl.dtype, 35001, "cuda")
        it = torch.arange(64, dtype=torch.int32, device="cuda").repeat(wl.B, 1, wl.k // 64 + 1)[..., :wl.k]
        it = torch.sort(it, dim=-1).values.contiguous()
        ot, lt = torch.empty_like(X.q[0]), torch.empty((wl.B, 1, wl.Hq), dtype=torch.float32, device="cuda")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for i in range(22):
            cold_rows_only(i)
            clsa.sparse_attn(X.q[i % n], kt, vt, it, kv_len=64, out=ot, lse=lt, ws=attn_ws)
            a.record()
            clsa.sparse_attn(X.q[i % n], X.k_cache[i % n], X.v_cache[i % n], idx, kv_len=wl.kv_len,
                             out=out[i % n], lse=lse[i % n], ws=attn_ws)
            b.record()
            torch.cuda.synchronize()
            if i >= 2:
                ts.append(a.elapsed_time(b) * 1e3)
        us_attn_cold_rows_warm_code = statistics.median(ts)
        del kt, vt, it, ot, lt
    us_step_cold = cold_us(lambda i: step.run(), 10)

    # Measured memory ceiling on this device: a plain device-to-device copy of
    # 256 MiB (torch's copy kernel), bytes read + written over its time.
    csrc = scratch[: 1 << 26]
    cdst = scratch[1 << 26: 2 << 26]
    for _ in range(3):
        cdst.copy_(csrc)
    a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a_ev.record()
    for _ in range(10):
        cdst.copy_(csrc)
    b_ev.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * csrc.numel() * 4 * 10 / (a_ev.elapsed_time(b_ev) * 1e-3) / 1e9

    # Per-step spread: one event before each of K steps (none between kernels).
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(K):
        steps[i % N_ROT].run()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(K))
    pct = lambda f: per_step[min(K - 1, int(f * K))]

    # Speedup context: the same attention call over every visible position
    # (idx = 0..kv_len-1, a dense gather), decode only.
    dense = None
    if wl.T == 1:
        idx_all = torch.arange(wl.kv_len, dtype=torch.int32, device="cuda").expand(wl.B, 1, wl.kv_len).contiguous()
        ws_all = torch.empty(max(256, clsa.workspace_bytes(1, B=wl.B, T=1, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D,
                                                           k=wl.kv_len)), dtype=torch.uint8, device="cuda")
        us_dense = per_launch_us(lambda i: clsa.sparse_attn(X.q[0], X.k_cache[0], X.v_cache[0], idx_all,
                                                            kv_len=wl.kv_len, out=out[0], lse=lse[0],
                                                            ws=ws_all))
        dense_bytes = wl.B * wl.kv_len * wl.Hkv * wl.D * (2 if wl.dtype == 1 else 4) * 2
        dense = {"k": wl.kv_len, "us": us_dense, "gbs": dense_bytes / (us_dense * 1e-6) / 1e9,
                 "speedup_sparse_vs_dense": us_dense / us_attn}
        del idx_all, ws_all
    # Attention call against batch size at this context and k (decode): the
    # call's fixed costs (launch, index latency, split merge) amortise over
    # more gathered rows as B grows. Caches of B sequences, Gaussian, rows
    # from a seeded random index; warm (back-to-back) and cold per call.
    batch_curve = None
    if wl.T == 1 and args.batch_curve:
        batch_curve = []
        for Bc in args.batch_curve:
            kc_b = inp.randn((Bc, wl.kv_len, wl.Hkv, wl.D), wl.dtype, 31000 + Bc, "cuda")
            vc_b = inp.randn((Bc, wl.kv_len, wl.Hkv, wl.D), wl.dtype, 32000 + Bc, "cuda")
            q_b = inp.randn((Bc, 1, wl.Hq, wl.D), wl.dtype, 33000 + Bc, "cuda")
            g = torch.Generator(device="cuda").manual_seed(34000 + Bc)
            idx_b = torch.sort(torch.rand((Bc, 1, wl.kv_len), generator=g, device="cuda").argsort(dim=-1)[..., :wl.k]
                               .to(torch.int32), dim=-1).values.contiguous()
            ws_b = torch.zeros(max(256, clsa.workspace_bytes(1, B=Bc, T=1, Hq=wl.Hq, Hkv=wl.Hkv, D=wl.D, k=wl.k)),
                               dtype=torch.uint8, device="cuda")
            out_b = torch.empty_like(q_b)
            lse_b = torch.empty((Bc, 1, wl.Hq), dtype=torch.float32, device="cuda")
            fn = lambda i: clsa.sparse_attn(q_b, kc_b, vc_b, idx_b, kv_len=wl.kv_len, out=out_b, lse=lse_b, ws=ws_b)
            warm = per_launch_us(fn)
            cold = cold_us(fn, 10)
            byt = (Bc * wl.k * wl.Hkv * wl.D * (2 if wl.dtype == 1 else 4) * 2 + Bc * wl.k * 4
                   + 2 * Bc * wl.Hq * wl.D * (2 if wl.dtype == 1 else 4) + Bc * wl.Hq * 4)
            batch_curve.append({"B": Bc, "warm_us": warm, "cold_us": cold,
                                "cold_gbs": byt / (cold * 1e-6) / 1e9,
                                "cold_frac": byt / (cold * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                "warm_gbs": byt / (warm * 1e-6) / 1e9})
            del kc_b, vc_b, q_b, idx_b, ws_b, out_b, lse_b
            torch.cuda.empty_cache()
        print("[bench] attention batch curve: " + ", ".join(
            f"B={c['B']} {c['warm_us']:.1f}/{c['cold_us']:.1f} us" for c in batch_curve), file=sys.stderr, flush=True)
    del scratch
    step_bytes = len(wl.f_layers) * (alg["index_score"] + alg["topk"]) + n * alg["sparse_attn"]
    f_layers = wl.f_layers

    comparator = None
    if wl.T > 1:
        # Block-union comparator on the same chunk: union table of the step's
        # index (64-token blocks), then dense attention over the table.
        block = 64
        indptr, indices = clsa.block_union_build(idx, wl.kv_len, block, wl.Hkv)
        torch.cuda.synchronize()
        n_blocks = int(indptr[1].item() - indptr[0].item())
        out_b = torch.empty_like(X.q[0])
        lse_b = torch.empty((wl.B, wl.T, wl.Hq), dtype=torch.float32, device="cuda")
        us_union = per_launch_us(lambda i: clsa.block_union_build(idx, wl.kv_len, block, wl.Hkv))
        us_paged = per_launch_us(lambda i: clsa.block_paged_attn(X.q[0], X.k_cache[0], X.v_cache[0], indptr,
                                                                 indices, block, kv_len=wl.kv_len, out=out_b,
                                                                 lse=lse_b))
        # The same comparator over head-major copies of the caches.
        kh = X.k_cache[0].transpose(1, 2).contiguous()
        vh = X.v_cache[0].transpose(1, 2).contiguous()
        us_paged_hm = per_launch_us(lambda i: clsa.block_paged_attn(X.q[0], kh, vh, indptr, indices, block,
                                                                    kv_len=wl.kv_len, out=out_b, lse=lse_b,
                                                                    head_major=True))
        del kh, vh
        pos = min(n_blocks * block, wl.kv_len)
        vis_sum = sum(min(pos, wl.kv_len - wl.T + t + 1) for t in range(wl.T))  # upper bound of keys seen
        flops = 4.0 * wl.B * wl.Hq * wl.D * vis_sum
        comparator = {
            "block": block,
            "union_blocks_per_group": n_blocks,
            "block_union_build_us": us_union,
            "block_paged_attn_us": us_paged,
            "block_paged_attn_head_major_us": us_paged_hm,
            "block_paged_attn_tflops_upper": flops / (us_paged * 1e-6) / 1e12,
            "sparse_attn_us": us_attn,
        }

    # Roofline of the sparse-attention call. A decode query gathers its own
    # rows once per layer: HBM-bound, priced by the algorithmic bytes. In a
    # chunk, the queries' index rows overlap and the repeated gathers are
    # served by L2 / Infinity Cache, so the call is priced by its bf16
    # matrix-core flops instead (q.K and P.V: 4 flops per (query head, entry,
    # element)).
    # A decode call is graded cold: every cache evicted before the call, so
    # its rows come from HBM. Back to back over one index (the 15 layers after
    # a step's first, with one shared cache) a workgroup runs on the same XCD
    # as in the previous call and finds part of its rows in that XCD's L2;
    # that warm rate is reported separately and is not an HBM figure.
    if wl.T == 1:
        cold_gbs = alg["sparse_attn"] / (us_attn_cold * 1e-6) / 1e9
        attn_roof = {"bound": "hbm", "achieved": cold_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": cold_gbs / HBM_PEAK_GBS, "traffic": measured_traffic(wl.name)}
    else:
        attn_tflops = 4.0 * wl.B * wl.T * wl.k * wl.Hq * wl.D / (us_attn * 1e-6) / 1e12
        attn_roof = {"bound": "mfma", "achieved": attn_tflops, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": attn_tflops / MFMA_BF16_PEAK_TFLOPS, "traffic": None,
                     # the rate at which the call gathers its rows through the L2s (their
                     # repeats across queries come from L2 / Infinity Cache, not HBM)
                     "l2_gather_gbs": attn_gbs}
    split_kernel = "attn_split_mfma" if wl.dtype == 1 else "attn_split_kernel"
    attn_roof.update({"kernel": f"sparse_attn call ({split_kernel} + attn_combine_kernel)",
                      "bytes_per_launch": alg["sparse_attn"]})
    if wl.T == 1:
        attn_roof.update({
            "avg_launch_us": us_attn_cold,
            "launch_state": "cold: L2s and Infinity Cache evicted before each call (median of 20)",
            "measured_copy_gbs": copy_gbs,
            "frac_of_measured_copy": cold_gbs / copy_gbs,
            "warm_caches": {
                "avg_launch_us": us_attn, "achieved": attn_gbs, "unit": "GB/s",
                "state": "back-to-back calls over one index, as for the 15 layers after a step's "
                         "first: part of the rows come from the XCDs' L2s (each workgroup runs on "
                         "the XCD it ran on in the previous call), the rest from the Infinity "
                         "Cache; not HBM traffic"},
            "cold_rows_hot_index": {
                "avg_launch_us": us_attn_cold_rows,
                "achieved": alg["sparse_attn"] / (us_attn_cold_rows * 1e-6) / 1e9, "unit": "GB/s",
                "state": "caches evicted, then the index and the query re-read: a step's first layer"},
            "cold_rows_warm_code": {
                "avg_launch_us": us_attn_cold_rows_warm_code,
                "achieved": alg["sparse_attn"] / (us_attn_cold_rows_warm_code * 1e-6) / 1e9, "unit": "GB/s",
                "state": "as cold_rows_hot_index, and the two kernels first run once on a 64-row cache "
                         "(their code and launch path warm, as for every layer of a step)"},
            "batch_curve": batch_curve,
        })
    else:
        attn_roof.update({"avg_launch_us": us_attn, "cold_launch_us": us_attn_cold})
    # The dominant kernel is the one with the larger share of the step: the
    # attention call (n layers) or the indexer (F layers). A chunk's indexer
    # is a contraction priced by its flops (2 * H_I * D_I per visible key);
    # a decode indexer streams its keys and is priced by its bytes.
    roofline = attn_roof
    if us_index * len(wl.f_layers) > us_attn * n and wl.idx_dtype != 0:
        vis_keys = wl.B * sum(wl.kv_len - wl.T + t + 1 for t in range(wl.T))
        if wl.T > 1:
            tf = 2.0 * wl.H_I * wl.D_I * vis_keys / (us_index * 1e-6) / 1e12
            peak = MFMA_FP8_PEAK_TFLOPS if wl.idx_dtype == 2 else MFMA_BF16_PEAK_TFLOPS
            roofline = {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s",
                        "frac": tf / peak, "traffic": None}
            if wl.idx_dtype == 1:
                gemm = measured_gemm_tflops()
                roofline.update({"measured_gemm_tflops": gemm, "frac_of_measured_gemm": tf / gemm,
                                 "measured_gemm": "torch.mm bf16 8192^3 (hipBLASLt), median of 5"})
        else:
            gbs = alg["index_score"] / (us_index * 1e-6) / 1e9
            roofline = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": gbs / HBM_PEAK_GBS, "traffic": None}
        kname = "idx_score_multi" if wl.T >= 8 else "idx_score_mfma"
        roofline.update({"kernel": f"index_score ({kname})", "avg_launch_us": us_index,
                         "sparse_attn": attn_roof})

    tokens_per_step = wl.B * wl.T
    result = {
        "metric": "decode tokens/sec + achieved HBM GB/s, sparse-attn step @128K ctx, top-k 2048",
        "value": tokens_per_step / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == 1 else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{wl.name}: {'decode' if wl.T == 1 else 'prefill chunk'} B={wl.B}, T={wl.T}, "
                        f"kv_len={wl.kv_len}, indexer {wl.H_I}x{wl.D_I} {inp.DTYPE_NAME[wl.idx_dtype]}, "
                        f"top-k {wl.k}, {n} layers, {len(f_layers)} indexer "
                        f"pass{'es' if len(f_layers) > 1 else ''} (each F layer's index serves the layers "
                        f"up to the next F layer), GQA {wl.Hq}q/{wl.Hkv}kv x {wl.D}, "
                        f"{'one KV cache shared by every layer' if wl.shared_kv else 'a KV cache per layer'}",
            "variant": args.variant,
            "query_sets": N_ROT,
            "global_batch": wl.B,
            "seq_len": wl.kv_len,
            "parallelism": "single GPU",
        },
        # algorithmic bytes of the whole step over its time; with one shared
        # cache the layers after the first re-gather the rows the first one
        # gathered, part of them from the L2s, so this is not HBM traffic
        "algorithmic_gbs_step": step_bytes / (ms_per_step * 1e-3) / 1e9,
        "roofline": roofline,
        "kernels_us": {
            "sparse_attn": us_attn,
            "index_score": us_index,
            "topk": us_topk,
            "cache_append": us_append,
            "index_score_gbs": alg["index_score"] / (us_index * 1e-6) / 1e9,
            "topk_gbs": alg["topk"] / (us_topk * 1e-6) / 1e9,
        },
        "ms_per_step_events": ms_per_step_events,
        "ms_per_step_p10_p50_p90": [pct(0.1), pct(0.5), pct(0.9)],
        "ms_per_step_cold": us_step_cold * 1e-3,
        "dense_gather_context": dense,
        "dynamic_k": dynamic_k,
        "ordered_skip": ordered_skip,
        "method_contrast": contrast,
        "ms_per_step_graph_replay": graph_ms,
        "step_stages_us": step_stages,
    }
    if comparator is not None:
        result["block_union_comparator"] = comparator
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, X, args.cpu_budget)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
