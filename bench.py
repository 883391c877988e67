"""Benchmark of the lightning-indexer decode step on one MI355X.

A step is one decode step of the whole hot path over one batch: for each of
the 21 CSA layers, in sequence, the indexer scores (a1), the exact top-512
(a2) and the sparse MQA attention over the selected rows plus the 128-row
window (a3), for 32 sequences at 64K context (16384 compressed entries each).
One query = one sequence x one layer x one decode step; value = queries/s.

Inputs are synthetic (seeded, generated on the GPU) and resident in HBM before
the timed region. The step is captured once in a HIP graph (checked against
the eager result) and replayed. Besides the headline line the JSON carries:
  roofline     : the dominant kernel (indexer scores) - algorithmic bytes per
                 launch / its average launch time, measured with HIP events on
                 the stream it runs on, against the 8 TB/s HBM peak;
  cpu_baseline : the CPU oracle on a bounded sample of the same queries;
  others       : the whole attention step of a token (2 SWA + 21 CSA + 20
                 HCA layers) at 64K and 500K, the 64K batch-1 latency, the
                 500K batch-4 step (distinct layers rotated so every replay
                 streams from HBM), the LSA cold-pool fetch, the lookahead
                 golden and the recall chain (gate, gated and native top-1024,
                 vote labels) at the gate workload's shapes.
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--only lookahead|prefill|offload|recall|ctx500k]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode queries/sec (indexer+top-512+sparse attn) at 64K/500K ctx; % HBM roofline"


def algo_bytes_per_query(N, H, k, window, Hq, kv_row_bytes=1024):
    """Algorithmic HBM bytes of one query of the path (score + select + attend)."""
    keys = N * 128 * 2
    rows = min(N, k + window) * kv_row_bytes
    small = H * 128 * 2 + H * 4 + Hq * 512 * 2 + Hq * 512 * 4 + k * 4
    return keys + rows + small


def idx_score_bytes_per_query(N, H):
    """Algorithmic bytes of one query of the indexer-score kernel: the bf16 keys
    and queries, the fp32 weights, the fp32 scores written and the hints written
    (one key-norm bound per 256 entries, one score maximum per 16 entries)."""
    return N * 128 * 2 + H * 128 * 2 + H * 4 + N * 4 + ((-(-N // 256)) + (-(-N // 16))) * 4


def capture(fn):
    """Captures fn(stream) into a graph; returns the graph."""
    import torch

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(torch.cuda.current_stream().cuda_stream)  # warm (attributes, code objects)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        fn(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return g


def time_graph(g, reps):
    import torch

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(reps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / 1e3  # seconds


# the sources the indexer-score kernel is compiled from
IDX_SCORE_SOURCES = ("lightning_indexer_top_idx_amd/csrc/idx_score.hip", "lightning_indexer_top_idx_amd/csrc/lit_common.h",
                     "include/lit.h")


def source_hash(paths=IDX_SCORE_SOURCES):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()


def stored_traffic(workload):
    """Per-launch HBM bytes of the indexer-score kernel from the committed
    rocprofv3 counter summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"idx_score_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        if rec.get("source_sha256") != source_hash():
            return None
        return rec.get("hbm_bytes_per_launch")
    except Exception:
        return None


def cpu_model():
    """The host CPU's model name, from /proc/cpuinfo."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_share():
    """Host threads the oracle may use: the process's CPU affinity, capped at
    the CPU share a one-GPU job is given (OMP_NUM_THREADS when set, else 16)."""
    aff = len(os.sched_getaffinity(0))
    try:
        share = int(os.environ.get("OMP_NUM_THREADS", "16"))
    except ValueError:
        share = 16
    return max(1, min(aff, share)), aff


def cpu_baseline(layers, wl, k, window, scale, budget_s, max_queries, threads, gpu_paths, single_s=None):
    """The oracle, as it stands, on a bounded sample of the same queries: on
    `threads` host threads (the value) and on one thread (single_core)."""
    import numpy as np
    import oracle

    oracle.build()
    jobs, keys = [], []
    n_layers, B = len(layers), layers[0].idx.k_idx.shape[0]
    picks = [(l, (7 * l + 3) % B) for l in range(n_layers)][:max_queries]
    for l, b in picks:
        L = layers[l]
        jobs.append(dict(q_idx=oracle.np_of(L.idx.q_idx[b]), w=oracle.np_of(L.idx.w[b]).copy(),
                         k_idx=oracle.np_of(L.idx.k_idx[b]), k=k, q=oracle.np_of(L.q[b]), kv_dtype=oracle.BF16,
                         data=oracle.np_of(L.kv.data[b]), window=window, scale_f=scale))
        keys.append((l, b))
    # parity of the timed path on the sample (ids bit-exact, outputs within 2e-2)
    t0 = time.perf_counter()
    res = oracle.decode_queries(jobs, threads=threads)
    done, elapsed = len(jobs), time.perf_counter() - t0
    while elapsed < budget_s:
        t1 = time.perf_counter()
        oracle.decode_queries(jobs, threads=threads)
        done += len(jobs)
        elapsed += time.perf_counter() - t1
    # one thread: whole queries until about single_s has passed
    single_s = budget_s / 2 if single_s is None else single_s
    n1, t1 = 0, time.perf_counter()
    while True:
        oracle.decode_queries([jobs[n1 % len(jobs)]], threads=1)
        n1 += 1
        e1 = time.perf_counter() - t1
        if e1 >= single_s:
            break
    ids_ok, worst = True, 0.0
    for (l, b), (c, rids, rout, _) in zip(keys, res):
        P = gpu_paths[l]
        ids_ok &= bool(np.array_equal(P.ids[b].cpu().numpy(), rids))
        o = P.out[b].double().cpu().numpy()
        worst = max(worst, float((np.abs(o - rout).max(-1) / np.abs(rout).max(-1)).max()))
    share, aff = cpu_share()
    return {"value": done / elapsed, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(jobs)} distinct queries of the timed workload (one sequence per layer), "
                      f"score+exact top-{k}+attention in fp64 C, {done} query runs in {elapsed:.1f} s",
            "single_core": {"value": n1 / e1, "unit": "queries/s", "cores": 1,
                            "sample": f"{n1} query runs of the same sample in {e1:.1f} s"},
            "cpu_model": cpu_model(), "affinity_cores": aff,
            "parity_on_sample": {"ids_bit_exact": ids_ok, "attn_max_rel_err": worst}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 512 MiB device copy (reference for HBM byte counters)")
    ap.add_argument("--only", choices=["lookahead", "prefill", "offload", "recall", "ctx500k"],
                    help="run one secondary measurement alone and print its JSON (for profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; --gpus above 1 is not supported "
                                   "(the path shards by sequence with no communication; see the design notes)"}))
        sys.exit(2)

    import numpy as np
    import torch

    import lightning_indexer_top_idx_amd as lit
    from lightning_indexer_top_idx_amd import workloads as W
    from lightning_indexer_top_idx_amd.step import CsaLayer

    lit.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        # copies of known size (512 MiB read, 512 MiB written): their counter
        # readings per byte scale the kernels' readings. One is the runtime's
        # blit copy, one a vectorized elementwise kernel (16-byte accesses).
        src = torch.ones(512 << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    scale = 1.0 / math.sqrt(512)
    if args.only:
        fn = {"lookahead": lookahead, "prefill": lambda lit, W, dev, scale: prefill(lit, W, dev),
              "offload": offload, "recall": gate_recall,
              "ctx500k": lambda lit, W, dev, scale: ctx500k(lit, W, dev, scale)[0]}[args.only]
        print(json.dumps({args.only: fn(lit, W, dev, scale)}))
        return
    wl = W.CTX64K_B
    print(f"[bench] generating {wl.name}: {wl.layers} layers x {wl.B} sequences x N={wl.N}", file=sys.stderr,
          flush=True)
    layers = [W.layer_inputs(wl, l, dev) for l in range(wl.layers)]
    paths = [CsaLayer(L, wl.k, wl.window, scale, dev) for L in layers]
    torch.cuda.synchronize()

    def step(stream):
        for P in paths:
            P.run(stream)

    # eager reference, then the captured step; every replay must match it
    step(torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    # a negative count would mean a violated rounding bound (nothing selected)
    assert all(bool((P.count == wl.k).all()) for P in paths), "a sequence selected fewer than k entries"
    ref_ids = [P.ids.clone() for P in paths]
    ref_out = [P.out.clone() for P in paths]
    g = capture(step)
    for _ in range(2):
        for P in paths:
            P.ids.fill_(-7)
            P.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        for P, ri, ro in zip(paths, ref_ids, ref_out):
            assert torch.equal(P.ids, ri) and torch.equal(P.out, ro), "graph replay differs from the eager step"
    print("[bench] graph replay matches the eager step", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    secs = time_graph(g, args.steps)
    wall = time.perf_counter() - t0
    q_per_step = wl.B * wl.layers
    value = q_per_step * args.steps / secs
    ms_per_step = secs / args.steps * 1e3
    per_query = algo_bytes_per_query(wl.N, wl.H, wl.k, wl.window, wl.Hq)
    print(f"[bench] {ms_per_step:.3f} ms/step, {value:.0f} queries/s", file=sys.stderr, flush=True)

    # dominant kernel: the indexer scores, 21 launches back to back in one graph
    gs = capture(lambda s: [P.score(s) for P in paths])
    reps = 10
    sec_s = time_graph(gs, reps)
    launch_s = sec_s / (reps * len(paths))
    score_bytes = idx_score_bytes_per_query(wl.N, wl.H) * wl.B
    achieved = score_bytes / launch_s / 1e9
    traffic = stored_traffic(wl.name)
    roofline = {"bound": "hbm", "kernel": "idx_score (indexer scores, MFMA bf16)",
                "scope": "this kernel alone; the whole path's fraction is path_roofline.frac",
                "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "avg_launch_us": round(launch_s * 1e6, 2),
                "algorithmic_bytes_per_launch": score_bytes}

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "ctx64k_b: 32 sequences x 21 CSA layers run in sequence, 64K context "
                               "(N=16384 compressed entries), 64x128 index heads, exact top-512 + SWA 128, "
                               "64-head MQA over 512-wide bf16 rows",
                   "global_batch": wl.B, "seq_len": 65536, "layers": wl.layers, "parallelism": "none (1 GPU)"},
        "path_roofline": {"algorithmic_bytes_per_query": per_query,
                          "achieved_GBs": round(per_query * value / 1e9, 1),
                          "frac": round(per_query * value / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "wall_s_timed": round(wall, 3),
    }

    if not args.no_cpu_baseline:
        threads, _ = cpu_share()
        print(f"[bench] CPU oracle on {threads} threads", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(layers, wl, wl.k, wl.window, scale, args.cpu_seconds, wl.layers,
                                           threads, paths)

    if not args.no_others:
        print("[bench] token step at 64K", file=sys.stderr, flush=True)
        out["others"] = {"token_step_64k": token_step(W, dev, scale, paths, 65536)}
        print("[bench] multi-query indexer: MTP at 64K", file=sys.stderr, flush=True)
        out["others"]["mtp_64k_indexer"] = mtp(lit, W, dev, layers, paths, wl)
        out["others"].update(others(lit, W, dev, scale))

    del g, gs
    print(json.dumps(out))


def token_step(W, dev, scale, csa, T, hca_kv=None, reps=10):
    """All 43 attention layers of one decode step ([ARCH] (A), the layer table):
    SWA on layers 0-1 (the last 128 uncompressed rows), CSA on the even layers
    2-42 (the `csa` layers given, reused in turn when fewer than 21), HCA on the
    odd layers 3-41 (ceil(T/128) rows read densely; the rows of `hca_kv` =
    (q, [rows...]) reused in turn when given). Returns the step time for the
    CSA layers' B sequences and the tokens/s it gives."""
    import torch
    from lightning_indexer_top_idx_amd.step import DenseLayer, TokenSchedule, layer_kind

    B, Hq = csa[0].B, csa[0].Hq
    swa = [DenseLayer(*W.dense_layer_inputs(B, 128, Hq, l, dev), scale, dev) for l in range(2)]
    if hca_kv is None:
        hca = [DenseLayer(*W.dense_layer_inputs(B, -(-T // 128), Hq, l, dev), scale, dev) for l in range(3, 42, 2)]
    else:
        hca = [DenseLayer(hca_kv[0], hca_kv[1][i % len(hca_kv[1])], scale, dev) for i in range(20)]
    order = []
    for l in range(43):
        kind = layer_kind(l)
        order.append(swa[l] if kind == "swa" else csa[((l - 2) // 2) % len(csa)] if kind == "csa"
                     else hca[(l - 3) // 2])
    sched = TokenSchedule(order)
    g = capture(sched.run)
    g.replay()
    sec = time_graph(g, reps) / reps
    # the CSA layers alone, in the same order, for their share of the step
    gc = capture(lambda s: [Ly.run(s) for l, Ly in enumerate(order) if layer_kind(l) == "csa"])
    gc.replay()
    csa_sec = time_graph(gc, reps) / reps
    del g, gc, swa, hca
    torch.cuda.empty_cache()
    return {"sequences": B, "context_tokens": T, "layers": "2 SWA (128 rows) + 21 CSA + 20 HCA "
                                                          f"({-(-T // 128)} rows)",
            "token_step_us": round(sec * 1e6, 1), "tokens_per_s": round(B / sec, 1),
            "csa_layers_us": round(csa_sec * 1e6, 1), "csa_share": round(csa_sec / sec, 3)}


MFMA_BF16_PEAK_TFLOPS = 2500.0


def cpu_baseline_rate(fn, gpu_s_per_unit, unit, sample, budget_s=4.0, max_units=50):
    """The cpu_baseline leg of a secondary measurement: the CPU oracle (one
    thread, as it stands) on a bounded sample of the same work. fn() does one
    unit and is run until about budget_s has passed. Returned as units/s, with
    the GPU's units/s beside it."""
    import oracle

    oracle.build()
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= max_units:
            break
    return {"value": round(n / el, 3), "unit": unit, "cores": 1, "kind": "oracle",
            "sample": f"{sample}, {n} runs in {el:.1f} s", "gpu_value": round(1.0 / gpu_s_per_unit, 1)}


def mtp(lit, W, dev, layers, paths, wl):
    """The multi-query indexer at depth-1 MTP (the current token and its draft,
    Q = 2) on the timed workload's 21 layers: score both queries against the
    keys in one pass, then each query's exact top-512. Next to it the same
    layers' single-query indexer (score + select of the timed step). Query 0
    of each sequence is the timed step's query, so its selection must equal
    the timed step's ids (checked)."""
    import torch

    Q = W.MTP_Q
    C = lit.load()
    bufs = []
    for l, (L, P) in enumerate(zip(layers, paths)):
        q, w = W.extra_queries(L.idx, Q, l, dev)
        d = lit.idx_in_mq(q, w, L.idx.k_idx)
        B, N = P.B, P.N
        sc = torch.empty(B, Q, N, dtype=torch.float32, device=dev)
        hi = torch.empty(B, Q, lit.hints_len(N), dtype=torch.float32, device=dev)
        ids = torch.empty(B, Q, wl.k, dtype=torch.int32, device=dev)
        cnt = torch.empty(B, Q, dtype=torch.int32, device=dev)
        ws = torch.empty(C.lit_topk_workspace_bytes(B * Q, N, wl.k), dtype=torch.uint8, device=dev)
        bufs.append((q, w, d, sc, hi, ids, cnt, ws, B, N))

    def score(s):
        for (q, w, d, sc, hi, ids, cnt, ws, B, N) in bufs:
            assert C.lit_idx_score_mq(ctypes.byref(d), Q, None, None, B, N, sc.data_ptr(), hi.data_ptr(), s) == 0, \
                lit.last_error()

    def select(s):
        for (q, w, d, sc, hi, ids, cnt, ws, B, N) in bufs:
            assert C.lit_topk_select_mq(sc.data_ptr(), B, Q, N, wl.k, ctypes.byref(d), hi.data_ptr(), ids.data_ptr(),
                                        cnt.data_ptr(), None, ws.data_ptr(), ws.numel(), s) == 0, lit.last_error()

    g2 = capture(lambda s: (score(s), select(s)))
    g2.replay()
    torch.cuda.synchronize()
    same = all(torch.equal(b[5][:, 0], P.ids) for b, P in zip(bufs, paths))
    gs = capture(score)
    g1 = capture(lambda s: [(P.score(s), P.select(s)) for P in paths])
    reps = 10
    t2 = time_graph(g2, reps) / (reps * len(paths))
    ts = time_graph(gs, reps) / (reps * len(paths))
    t1 = time_graph(g1, reps) / (reps * len(paths))
    B, N = paths[0].B, paths[0].N
    score_bytes = B * (N * 128 * 2 + Q * (wl.H * 128 * 2 + wl.H * 4) + Q * N * 4
                       + Q * ((-(-N // 256)) + (-(-N // 16))) * 4)
    del g2, gs, g1, bufs
    torch.cuda.empty_cache()
    return {"sequences": B, "queries_per_sequence": Q, "entries": N,
            "indexer_us_per_layer_q2": round(t2 * 1e6, 2), "indexer_us_per_layer_q1": round(t1 * 1e6, 2),
            "indexer_us_per_query_q2": round(t2 * 1e6 / (B * Q), 3),
            "indexer_us_per_query_q1": round(t1 * 1e6 / B, 3),
            "score_us_per_layer_q2": round(ts * 1e6, 2),
            "score_hbm_frac_q2": round(score_bytes / ts / 1e9 / HBM_PEAK_GBS, 4),
            "query0_equals_single_query_step": same,
            "note": "score + exact top-512 of both queries per layer, 21 layers in one graph; the keys are read "
                    "once for the two queries"}


def prefill(lit, W, dev):
    """The multi-query indexer on a prefill chunk: the last 2048 tokens of a 64K
    prompt (one sequence, 16384 entries, 64 index heads), each token seeing the
    entries complete before it (causal lengths). The scoring is a [2048*64 x
    128] x [128 x 16384] product on the matrix cores; algorithmic flops count
    the visible entries only. Then every token's exact top-512."""
    import torch

    wl = W.CTX64K
    Q = W.PREFILL_Q
    idx = W.mq_inputs(wl, Q, 0, dev)
    q, w, k = idx.q_idx, idx.w, idx.k_idx
    lengths = W.causal_lengths(1, Q, W.PREFILL_T - Q, dev)
    C = lit.load()
    d = lit.idx_in_mq(q, w, k)
    N = wl.N
    sc = torch.empty(1, Q, N, dtype=torch.float32, device=dev)
    hi = torch.empty(1, Q, lit.hints_len(N), dtype=torch.float32, device=dev)
    ids = torch.empty(1, Q, wl.k, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, Q, dtype=torch.int32, device=dev)
    ws = torch.empty(C.lit_topk_workspace_bytes(Q, N, wl.k), dtype=torch.uint8, device=dev)

    def score(s):
        assert C.lit_idx_score_mq(ctypes.byref(d), Q, lengths.data_ptr(), None, 1, N, sc.data_ptr(), hi.data_ptr(),
                                  s) == 0, lit.last_error()

    def select(s):
        assert C.lit_topk_select_mq(sc.data_ptr(), 1, Q, N, wl.k, ctypes.byref(d), hi.data_ptr(), ids.data_ptr(),
                                    cnt.data_ptr(), None, ws.data_ptr(), ws.numel(), s) == 0, lit.last_error()

    gs, gt = capture(score), capture(select)
    reps = 10
    ts = time_graph(gs, reps) / reps
    tt = time_graph(gt, reps) / reps
    flops = 2.0 * wl.H * 128 * float(lengths.sum().item())
    tflops = flops / ts / 1e12
    ok = bool((cnt == wl.k).all().item())
    import oracle

    qc, wc, kc, lc = q[:, :1].cpu(), w[:, :1].cpu(), k.cpu(), lengths[:, :1].cpu()
    orc = cpu_baseline_rate(lambda: oracle.topk_mq(oracle.idx_score_mq(qc, wc, kc, lc), wl.k), (ts + tt) / Q,
                            "query rows/s", "query 0 of the chunk (fp64 scores over its 15873 visible entries, "
                            "exact top-512)")
    del gs, gt
    torch.cuda.empty_cache()
    return {"queries": Q, "entries": N, "score_us": round(ts * 1e6, 1), "score_TFLOPs": round(tflops, 1),
            "mfma_bf16_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "topk_us": round(tt * 1e6, 1),
            "topk_us_per_query": round(tt * 1e6 / Q, 3), "tokens_per_s_indexer": round(Q / (ts + tt), 1),
            "all_counts_k": ok, "cpu_baseline": orc}


FP64_PEAK_TFLOPS = 78.6


def lookahead(lit, W, dev, scale):
    """The lookahead golden at the gate workload's shapes (8 sequences, 16384
    entries, FP8 rows, 64 heads, top-1024) over a tau = 64 step horizon: the
    fp64 logits of 64 x 64 query rows against every row (a [4096 x 512] x [512
    x 16384] product per sequence on the fp64 matrix cores), each step's
    golden top-1024, and their union. Reported: the logits kernel's rate
    against the fp64 matrix-core peak, the whole call, and how much of the
    horizon's union three selections of the current step cover (the LSA gate
    at layers 10/12/20, the native top-1024 at layer 10, the current step's
    golden) -- on synthetic data, so these coverages describe the inputs, not
    the model. The rate counts the logits' flops over the whole call (the
    softmax, top-k and union passes included)."""
    import torch

    wl = W.GATE64K
    T = W.TAU
    keys = [W.layer_inputs(wl, l, dev).idx.k_idx for l in W.GATE_LAYERS]
    gl = [W.gate_layer(wl, l, kk, dev) for l, kk in zip(W.GATE_LAYERS, keys)]
    gate, _ = lit.lsa_gate(gl, 0.5)
    del gl, keys
    L = W.layer_inputs(wl, 10, dev)
    q = W.horizon_queries(L.q, T, 10, dev)
    s_, h_ = lit.idx_score(L.idx.q_idx, L.idx.w, L.idx.k_idx)
    _, _, native = lit.topk_select(s_, wl.k, exact=(L.idx.q_idx, L.idx.w, L.idx.k_idx), hints=h_)
    C = lit.load()
    B, Hq, N, k = wl.B, wl.Hq, wl.N, wl.k
    ws = torch.empty(C.lit_lookahead_workspace_bytes(B, T, Hq, N, k), dtype=torch.uint8, device=dev)
    hits = torch.empty(B, N, dtype=torch.int32, device=dev)
    um = torch.empty(B, N, dtype=torch.uint8, device=dev)
    uc = torch.empty(B, dtype=torch.int32, device=dev)
    sids = torch.empty(B, T, k, dtype=torch.int32, device=dev)
    desc = lit.kv_desc(L.kv)

    def call(s):
        assert C.lit_lookahead_golden(q.data_ptr(), lit.LIT_BF16, T, Hq, ctypes.byref(desc), B, scale, k,
                                      sids.data_ptr(), hits.data_ptr(), um.data_ptr(), uc.data_ptr(), None,
                                      ws.data_ptr(), ws.numel(), s) == 0, lit.last_error()

    s0 = torch.cuda.current_stream().cuda_stream
    call(s0)
    torch.cuda.synchronize()
    reps = 3
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call(s0)
    e1.record()
    torch.cuda.synchronize()
    total_s = e0.elapsed_time(e1) / 1e3 / reps
    flops = 2.0 * B * T * Hq * 512 * N
    first = sids[:, 0]
    gold0 = torch.zeros(B, N, dtype=torch.uint8, device=dev)
    gold0.scatter_(1, first.clamp(min=0).long(), 1)
    cov = {}
    for name, m in (("lsa_gate", gate), ("native_top1024", native), ("current_golden", gold0)):
        inter, _, cu = lit.recall(m, um)
        cov[name] = round(float(inter.sum().item()) / float(cu.sum().item()), 4)
    import oracle
    from lightning_indexer_top_idx_amd import synth

    kv0 = synth.KVRows("fp8", L.kv.data[:1].cpu(), L.kv.rope[:1].cpu(), L.kv.scale[:1].cpu())
    q00 = q[:1, :1].cpu()
    orc = cpu_baseline_rate(lambda: oracle.lookahead_golden(q00, kv0, scale, k), total_s / (B * T),
                            "horizon steps/s", "one horizon step of sequence 0 (dense fp64 softmax over 16384 FP8 "
                            "rows, 64 heads, top-1024)")
    res = {"sequences": B, "entries": N, "horizon": T, "heads": Hq, "k": k,
           "call_ms": round(total_s * 1e3, 2), "logits_flops": flops, "cpu_baseline": orc,
           "call_TFLOPs_fp64": round(flops / total_s / 1e12, 1),
           "call_fp64_mfma_frac": round(flops / total_s / 1e12 / FP64_PEAK_TFLOPS, 4),
           "union_mean": round(float(uc.float().mean().item()), 1),
           "union_over_k": round(float(uc.float().mean().item()) / k, 3),
           "union_coverage": cov}
    del ws
    torch.cuda.empty_cache()
    return res


def ctx500k(lit, W, dev, scale):
    """The 500K batch-4 figures: one CSA layer step and one HCA layer; returns
    them with the layers' inputs (for the token step)."""
    import torch
    from lightning_indexer_top_idx_amd.step import CsaLayer

    # 500K, batch 4: one CSA layer (N=125000) + one HCA layer (3907 rows read
    # densely). Distinct layers are rotated (3 CSA layers, 384 MB of keys; 24
    # copies of the HCA rows, 384 MB) so that no replay finds its data in the
    # 256 MB cache.
    wl = W.CTX500K
    n_csa, n_hca = 3, 24
    csa_paths = [CsaLayer(W.layer_inputs(wl, l, dev), wl.k, wl.window, scale, dev) for l in range(n_csa)]
    hq, hkv0 = W.hca_inputs(wl, dev)
    hkvs = [hkv0] + [type(hkv0)(hkv0.dtype, hkv0.data.clone()) for _ in range(n_hca - 1)]
    hout = torch.empty(wl.B, wl.Hq, 512, dtype=torch.float32, device=dev)
    C = lit.load()
    hws = torch.empty(C.lit_attn_workspace_bytes(wl.B, wl.Hq, wl.hca_N), dtype=torch.uint8, device=dev)
    hdescs = [lit.kv_desc(h) for h in hkvs]

    def hca(s):
        for hdesc in hdescs:
            st = C.lit_sparse_attn_decode(hq.data_ptr(), lit.LIT_BF16, wl.Hq, ctypes.byref(hdesc), wl.B, None, None, 0,
                                          0, scale, hout.data_ptr(), None, hws.data_ptr(), hws.numel(), s)
            assert st == 0, lit.last_error()

    gc = capture(lambda s: [P.run(s) for P in csa_paths])
    gh = capture(hca)
    csa_s = time_graph(gc, 10) / (10 * n_csa)
    hca_s = time_graph(gh, 10) / (10 * n_hca)
    per_query = algo_bytes_per_query(wl.N, wl.H, wl.k, wl.window, wl.Hq)
    r = {"csa_step_us": round(csa_s * 1e6, 2), "queries_per_s": round(wl.B / csa_s, 1),
         "hbm_frac": round(per_query * wl.B / csa_s / 1e9 / HBM_PEAK_GBS, 4),
         "hca_layer_us": round(hca_s * 1e6, 2),
         "hca_hbm_frac": round(wl.B * wl.hca_N * 1024 / hca_s / 1e9 / HBM_PEAK_GBS, 4)}
    del gc, gh, hout, hws
    return r, csa_paths, hq, hkvs


def others(lit, W, dev, scale):
    """Secondary figures: 64K batch-1 latency and the 500K batch-4 step."""
    import torch
    from lightning_indexer_top_idx_amd.step import CsaLayer

    res = {}
    # 64K, batch 1: 32 independent layers rotated so the data exceeds the 256 MB cache
    wl = W.CTX64K
    n_rot = 32
    layers = [W.layer_inputs(wl, 100 + l, dev) for l in range(n_rot)]
    paths = [CsaLayer(L, wl.k, wl.window, scale, dev) for L in layers]
    g = capture(lambda s: [P.run(s) for P in paths])
    g.replay()
    sec = time_graph(g, 5)
    per_q = sec / (5 * n_rot)
    res["ctx64k_b1"] = {"us_per_query": round(per_q * 1e6, 2), "queries_per_s": round(1 / per_q, 1),
                        "note": "batch 1, one query per step; 32 distinct layers replayed back to back in a graph"}
    del g, paths, layers
    torch.cuda.empty_cache()
    res["ctx500k_b4"], csa_paths, hq, hkvs = ctx500k(lit, W, dev, scale)
    # the whole attention step of a token at 500K: the three CSA layers above
    # in turn, the 24 copies of the HCA rows in turn
    print("[bench] token step at 500K", file=sys.stderr, flush=True)
    res["token_step_500k"] = token_step(W, dev, scale, csa_paths, 500000, hca_kv=(hq, hkvs))
    del csa_paths, hkvs
    torch.cuda.empty_cache()
    res["gate64k_offload"] = offload(lit, W, dev, scale)
    print("[bench] multi-query indexer: prefill chunk", file=sys.stderr, flush=True)
    res["prefill_chunk_indexer"] = prefill(lit, W, dev)
    print("[bench] lookahead golden", file=sys.stderr, flush=True)
    res["lookahead_golden_gate64k"] = lookahead(lit, W, dev, scale)
    print("[bench] gate-stress recall chain", file=sys.stderr, flush=True)
    res["gate64k_recall"] = gate_recall(lit, W, dev, scale)
    return res


def gate_recall(lit, W, dev, scale):
    """The gate-stress workload's reported figures: 8 sequences x 16384 entries,
    FP8 rows, top-1024 over the 21 CSA layers; the gate of layers 10/12/20
    (d_model 4096, rank 2048), the native and the gated exact top-1024 of every
    layer, the vote labels (top-p 0.6, at least 3 of 21 layers) from the
    indexer logits (R1) and from dense attention (R2), and the recalls of the
    gated selection against each label set and against the native selection.
    Synthetic inputs: the planted entries are aligned with the index queries
    only, so R1 labels follow the indexer and R2 labels (dense attention over
    unplanted rows) do not; these recalls describe the inputs, not the model."""
    import torch
    from lightning_indexer_top_idx_amd import labels

    wl = W.GATE64K
    keys = [W.layer_inputs(wl, l, dev).idx.k_idx for l in W.GATE_LAYERS]
    gl = [W.gate_layer(wl, l, kk, dev) for l, kk in zip(W.GATE_LAYERS, keys)]
    del keys
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r = labels.run_chain([(lambda l=l: W.layer_inputs(wl, l, dev)) for l in W.CSA_LAYERS], gl, wl.k, scale=scale)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    res = {"sequences": wl.B, "entries": wl.N, "layers": len(W.CSA_LAYERS), "k": wl.k,
           "gate_layers": list(W.GATE_LAYERS), "top_p": 0.6, "min_votes": 3}
    res.update(labels.summary(r, wl.N))
    res["chain_s_with_input_generation"] = round(el, 2)
    res["data"] = "synthetic: recalls describe the generated inputs, not the model's"
    del r, gl
    torch.cuda.empty_cache()
    return res


def offload(lit, W, dev, scale):
    """The LSA cold-pool fetch at the gate workload's shapes (8 sequences, N =
    16384, FP8 rows, top-1024, gate at layers 10/12/20): one CSA layer's index
    keys and latent rows live in pinned host memory; the gate's kept entries
    (plus the window) are gathered over the host link into a compact pool, and
    the decode step runs on that pool. Reported: the fetch (per layer, and per
    tau = 64 steps for the 21 CSA layers), the link rate it reaches next to a
    plain pinned-to-device copy, and the step on the compact pool next to the
    same step on the resident arrays with the gate as the allowed set (the two
    are checked equal first)."""
    import torch
    from lightning_indexer_top_idx_amd import synth
    from lightning_indexer_top_idx_amd.step import CsaLayer

    wl = W.GATE64K
    keys = [W.layer_inputs(wl, l, dev).idx.k_idx for l in W.GATE_LAYERS]
    gl = [W.gate_layer(wl, l, kk, dev) for l, kk in zip(W.GATE_LAYERS, keys)]
    gate, gcnt = lit.lsa_gate(gl, 0.5)
    # the gate itself (a8): three layers' projections and entry scores
    g0 = gl[0]
    gws = lit.workspace(lit.load().lit_gate_workspace_bytes(3, wl.B, g0.w_proj.shape[0], g0.wq_a.shape[0], wl.N), dev)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        lit.lsa_gate(gl, 0.5, ws=gws)
    e1.record()
    torch.cuda.synchronize()
    gate_s = e0.elapsed_time(e1) / 1e3 / 5
    gate_bytes = sum(Ly.wq_a.numel() * 2 + Ly.wq_b.numel() * 2 + Ly.w_proj.numel() * 2 + Ly.k.numel() * 2
                     + Ly.h.numel() * 4 for Ly in gl) + 2 * wl.B * wl.N
    import oracle

    one = [{"h": Ly.h[:1].cpu(), "wq_a": Ly.wq_a.cpu(), "wq_b": Ly.wq_b.cpu(), "w_proj": Ly.w_proj.cpu(),
            "k": Ly.k[:1].cpu()} for Ly in gl]
    gate_orc = cpu_baseline_rate(lambda: oracle.lsa_gate(one, 0.5), gate_s / wl.B, "sequences/s",
                                 "sequence 0's gate over layers 10/12/20 (fp64 projections, 16384 entries)")
    del gl, keys, gws
    L = W.layer_inputs(wl, 10, dev)
    # the pool holds the largest kept set (a first plan at full size counts them)
    _, pc, _ = lit.pool_plan(gate, wl.window, wl.N)
    C = min(wl.N, int((pc.max().item() + 63) // 64 * 64))
    m, pc, ac = lit.pool_plan(gate, wl.window, C)
    host = [t.cpu().pin_memory() for t in (L.idx.k_idx, L.kv.data, L.kv.rope, L.kv.scale)]
    bufs = [torch.empty((wl.B, C) + tuple(t.shape[2:]), dtype=t.dtype, device=dev) for t in host]
    row_bytes = sum(t[0, 0].numel() * t.element_size() for t in host)

    def fetch():
        for t, o in zip(host, bufs):
            lit.pool_gather(t, m, out=o)

    fetch()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        fetch()
    e1.record()
    torch.cuda.synchronize()
    fetch_s = e0.elapsed_time(e1) / 1e3 / reps
    link_bytes = int(pc.sum().item()) * row_bytes
    # a plain copy of as many bytes from pinned memory (the runtime's DMA engines)
    cp_src = torch.empty(link_bytes, dtype=torch.uint8).pin_memory()
    cp_dst = torch.empty(link_bytes, dtype=torch.uint8, device=dev)
    cp_dst.copy_(cp_src, non_blocking=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        cp_dst.copy_(cp_src, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    copy_s = e0.elapsed_time(e1) / 1e3 / reps
    # the decode step, resident (gate as allowed) and on the compact pool
    Pr = CsaLayer(L, wl.k, wl.window, scale, dev, allowed=gate)
    Lc = W.LayerInputs(synth.IndexerInputs(L.idx.q_idx, L.idx.w, bufs[0]), L.q,
                       synth.KVRows("fp8", bufs[1], bufs[2], bufs[3]))
    Pc = CsaLayer(Lc, wl.k, wl.window, scale, dev, allowed=ac)
    s0 = torch.cuda.current_stream().cuda_stream
    Pr.run(s0)
    Pc.run(s0)
    ids_o = lit.pool_remap_ids(Pc.ids, Pc.count, m)
    torch.cuda.synchronize()
    same = bool(torch.equal(ids_o, Pr.ids) and torch.equal(Pc.count, Pr.count) and torch.equal(Pc.out, Pr.out))
    gr, gcp = capture(Pr.run), capture(Pc.run)
    resident_s = time_graph(gr, 20) / 20
    compact_s = time_graph(gcp, 20) / 20
    return {"sequences": wl.B, "entries": wl.N, "keep_frac": round(float(gcnt.float().mean().item()) / wl.N, 4),
            "gate_us_3_layers": round(gate_s * 1e6, 1), "gate_hbm_frac": round(gate_bytes / gate_s / 1e9 / HBM_PEAK_GBS, 4),
            "gate_us_per_step_amortized": round(gate_s * 1e6 / 64, 2), "gate_cpu_baseline": gate_orc,
            "pool_rows": C, "row_bytes": row_bytes, "fetch_bytes_per_layer": link_bytes,
            "fetch_us_per_layer": round(fetch_s * 1e6, 1), "link_GBs": round(link_bytes / fetch_s / 1e9, 2),
            "pinned_copy_GBs": round(link_bytes / copy_s / 1e9, 2),
            "fetch_ms_per_tau_21_layers": round(21 * fetch_s * 1e3, 2),
            "fetch_us_per_step_amortized": round(21 * fetch_s * 1e6 / 64, 1),
            "step_us_resident_gated": round(resident_s * 1e6, 2), "step_us_compact_pool": round(compact_s * 1e6, 2),
            "compact_equals_resident": same,
            "note": "one CSA layer's keys + FP8 rows (840 B per entry) fetched from pinned host memory by the "
                    "gather kernel; per-tau and per-step figures scale it to the 21 CSA layers"}


if __name__ == "__main__":
    main()
