"""Benchmark of the DynamicRad block-sparse attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--mode static|dynamic|token|decay-static] [--preset low|mid|high]

One step = one pass of the whole hot path over one batch of synthetic input
already resident in HBM: candidate build (asynchronous form), block mean
pooling + scoring + selection, the choice of query-block grouping, and
block-sparse flash attention (--graph: the step's launches replayed from a
HIP graph). The dense
kernel is timed separately as the speedup denominator. Per-stage times come
from HIP events on the launch stream: stage_ms is the mean over
--stage-iters launches (the roofline uses it), stage_ms_median the median of
the per-launch times. Prints one JSON line.

--mode decay-static: the paper's content-free static-ratio selector (Eq. 8);
its mask depends on no tensor, so it is built once (timed separately as
stage_ms.mask_build) and a step is the sparse attention over it.

Metric: sparse-attention effective TFLOP/s (4 * B_s^2 * D per kept block,
kept blocks only) with the speedup over the on-GPU dense kernel, on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn effective TFLOP/s + speedup vs dense at ≥80% sparsity, 1 GPU"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan14b_720p")
    ap.add_argument("--mode", default="static", choices=["static", "dynamic", "token", "decay-static"],
                    help="block-level static-ratio / dynamic-threshold selection, the paper's token-level "
                         "dynamic-threshold selector (dr_token_select) or its decay-state static-ratio "
                         "selector (dr_static_select), the last two with a Table 2 preset")
    ap.add_argument("--preset", default="mid", choices=["low", "mid", "high"],
                    help="Table 2 preset (dynamic rows for --mode token, static rows for --mode decay-static)")
    ap.add_argument("--seed", type=int, default=2024, help="sampling seed of --mode decay-static")
    ap.add_argument("--block-size", type=int, default=None, help="override the workload's block size (32, 64, 128)")
    ap.add_argument("--stage-iters", type=int, default=100, help="timed launches per stage (mean and median)")
    ap.add_argument("--dense-iters", type=int, default=50, help="timed launches of the dense kernel")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step's HIP graph instead of eager launches")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-groups", action="store_true",
                    help="consecutive query blocks per attention workgroup (skip dr_query_groups)")
    ap.add_argument("--cpu-blocks", type=int, default=960, help="query blocks in the CPU oracle sample")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run one plain 1 GiB device copy (the reference for HBM byte counters)")
    return ap.parse_args()


def event_ms(fn, iters, torch, medians=None, name=None):
    """Average ms per call from HIP events on the current stream (the stream
    the library launches on): the first launch's start to the last one's end,
    over iters. With `medians`, also the median of the per-launch times,
    stored under `name`."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(iters):
        fn()
        ev[i + 1].record()
    ev[-1].synchronize()
    if medians is not None:
        medians[name] = round(float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(iters)])), 4)
    return ev[0].elapsed_time(ev[-1]) / iters


def traffic_record(workload, mode):
    """HBM bytes per sparse-attention launch from committed rocprofv3 PMC
    counters, if they were taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", "sparse_attn_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p)).get(f"{workload}/{mode}")
    from block_sparse_attention_candidates_amd.profsum import attention_source_digest
    if not rec or rec.get("attention_src_sha256") != attention_source_digest():
        return None
    return rec


def host_info():
    """Threads the oracle's BLAS uses, CPUs this process may run on, CPU model."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas = 1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return int(blas), len(os.sched_getaffinity(0)), model


def cpu_baseline(w, mode, ratio, tau, n_blocks):
    """The CPU oracle, untuned, on a bounded sample: one head, n_blocks query
    blocks spread over the sequence; every step of the path for those blocks
    (candidate rows, pooling, scores, selection, attention), each timed."""
    import workloads
    from oracle import dynrad_oracle as O
    cores, host_cpus, model = host_info()
    if mode == "token":
        res = cpu_baseline_token(w, tau, cores)
    elif mode == "decay-static":
        res = cpu_baseline_decay_static(w, tau, cores)
    else:
        q, k, v = (x.astype(np.float64) for x in workloads.head_qkv(w, 0, 0))
        Sb = w.num_blocks
        blocks = np.unique(np.linspace(0, Sb - 1, n_blocks).astype(int))
        t0 = time.perf_counter()
        table = O.distance_table(w.num_frames, w.tokens_per_frame, w.block_size, w.gamma, w.lam)
        rows = {int(a): O.candidate_row(int(a), w.num_frames, w.tokens_per_frame, w.block_size, w.gamma, w.lam,
                                        w.theta_c, w.theta_m, table=table) for a in blocks}
        t1 = time.perf_counter()
        qbar, kbar = O.pool_blocks(q, w.block_size), O.pool_blocks(k, w.block_size)
        t2 = time.perf_counter()
        kept = {}
        for a in blocks:
            cols = rows[int(a)]
            s = (kbar[cols] @ qbar[a]) / math.sqrt(w.head_dim)
            kept[int(a)] = O.select_row(s, cols, mode, ratio=ratio, tau=tau)
        t3 = time.perf_counter()
        klist = [kept.get(a, np.zeros(0, dtype=np.int64)) for a in range(Sb)]
        O.sparse_attention_rows(q, k, v, w.block_size, klist, [int(a) for a in blocks])
        t4 = time.perf_counter()
        dt = t4 - t0
        flops = 4.0 * w.block_size ** 2 * w.head_dim * sum(len(kept[int(a)]) for a in blocks)
        res = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
               "seconds": round(dt, 3),
               "stage_ms": {"candidate_rows": round((t1 - t0) * 1e3, 2), "pooling": round((t2 - t1) * 1e3, 2),
                            "scores_selection": round((t3 - t2) * 1e3, 2), "attention": round((t4 - t3) * 1e3, 2)},
               "sample": f"{w.name} head 0, {len(blocks)} of {Sb} query blocks (evenly spaced), all stages "
                         f"(candidate rows, pooling of the whole head, scores, {mode} selection, attention), "
                         f"float64 NumPy"}
    res["host_cpus"] = host_cpus
    res["cpu_model"] = model
    return res


def cpu_baseline_token(w, taus, cores):
    """Token-level mode: the query blocks lying in frame N_f/2, with the
    statistics of the frame pairs they need (that frame against every key
    frame), their selection and their attention, on heads 0-1 (H_f = 2)."""
    import workloads
    from oracle import dynrad_oracle as O
    heads = [workloads.head_qkv(w, 0, h) for h in range(2)]
    qh = [x[0].astype(np.float64) for x in heads]
    kh = [x[1].astype(np.float64) for x in heads]
    v0 = heads[0][2].astype(np.float64)
    Nf, Nt, Bs = w.num_frames, w.tokens_per_frame, w.block_size
    frames = [Nf // 2]
    blocks = sorted({a for f in frames for a in range(f * Nt // Bs, ((f + 1) * Nt - 1) // Bs + 1)
                     if a * Bs // Nt == f and ((a + 1) * Bs - 1) // Nt == f})
    t0 = time.perf_counter()
    sub = O.token_frame_stats(qh, kh, Nf, Nt, Bs, w.gamma, w.lam, taus[0], taus[1], query_frames=frames)
    t1 = time.perf_counter()
    kept = O.token_select_rows(qh, kh, blocks, Nf, Nt, Bs, w.gamma, w.lam, taus[0], taus[1], w.theta_c, w.theta_m,
                               stats=sub)
    t2 = time.perf_counter()
    klist = [np.zeros(0, dtype=np.int64)] * w.num_blocks
    for a, ks in zip(blocks, kept):
        klist[a] = ks
    O.sparse_attention_rows(qh[0], kh[0], v0, Bs, klist, blocks)
    t3 = time.perf_counter()
    dt = t3 - t0
    flops = 4.0 * Bs ** 2 * w.head_dim * sum(len(x) for x in kept)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "seconds": round(dt, 3),
            "stage_ms": {"frame_pair_statistics": round((t1 - t0) * 1e3, 2),
                         "token_selection": round((t2 - t1) * 1e3, 2), "attention": round((t3 - t2) * 1e3, 2)},
            "sample": f"{w.name}: the {len(blocks)} query blocks inside frames {frames}, all stages (statistics "
                      f"of those frames' frame pairs, token-level selection on heads 0-1, attention on head 0), "
                      f"float64 NumPy"}


def cpu_baseline_decay_static(w, rho_seed, cores, n_blocks=16):
    """Decay-state static mode: n_blocks query blocks evenly spaced inside
    frame N_f/2, with the sample cuts of that frame's frame pairs, their
    selection and their attention on head 0."""
    import workloads
    from oracle import dynrad_oracle as O
    rn, rf, seed = rho_seed
    q, k, v = (x.astype(np.float64) for x in workloads.head_qkv(w, 0, 0))
    Nf, Nt, Bs = w.num_frames, w.tokens_per_frame, w.block_size
    f = Nf // 2
    inside = [a for a in range(f * Nt // Bs, ((f + 1) * Nt - 1) // Bs + 1)
              if a * Bs // Nt == f and ((a + 1) * Bs - 1) // Nt == f]
    blocks = [inside[int(x)] for x in np.unique(np.linspace(0, len(inside) - 1, n_blocks).astype(int))]
    t0 = time.perf_counter()
    th = O.static_frame_thresholds(Nf, Nt, Bs, w.gamma, w.lam, rn, rf, seed, query_frames=[f])
    t1 = time.perf_counter()
    kept = O.static_select_rows(blocks, Nf, Nt, Bs, w.gamma, w.lam, rn, rf, seed, w.theta_c, w.theta_m,
                                thresholds=th)
    t2 = time.perf_counter()
    klist = [np.zeros(0, dtype=np.int64)] * w.num_blocks
    for a, ks in zip(blocks, kept):
        klist[a] = ks
    O.sparse_attention_rows(q, k, v, Bs, klist, blocks)
    t3 = time.perf_counter()
    dt = t3 - t0
    flops = 4.0 * Bs ** 2 * w.head_dim * sum(len(x) for x in kept)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "seconds": round(dt, 3),
            "stage_ms": {"sample_cuts": round((t1 - t0) * 1e3, 2), "decay_static_selection": round((t2 - t1) * 1e3, 2),
                         "attention": round((t3 - t2) * 1e3, 2)},
            "sample": f"{w.name}: {len(blocks)} query blocks inside frame {f}, all stages (sample cuts of that "
                      f"frame's {len(th)} sampled frame pairs, decay-state static selection, attention on head 0), "
                      f"float64 NumPy"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the attention path here is a "
              f"single-GPU kernel; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_attention_candidates_amd as dr
    import workloads
    from block_sparse_attention_candidates_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_attention_candidates_amd import build
        build.build()
    w = workloads.get_workload(args.workload)
    taus = rhos = None
    if args.mode == "token":
        w, taus = workloads.token_workload(args.workload, args.preset)
    if args.mode == "decay-static":
        w, rhos = workloads.static_workload(args.workload, args.preset)
    if args.block_size:
        import dataclasses
        w = dataclasses.replace(w, name=f"{w.name}+bs{args.block_size}", block_size=args.block_size)
    ratio = w.static_ratio if args.mode == "static" else 1.0
    tau = w.dynamic_tau if args.mode == "dynamic" else 1.0
    print(f"# generating {w.name}: B={w.batch} H={w.heads} S={w.seq_len} D={w.head_dim}", file=sys.stderr, flush=True)
    qb, kb, vb = workloads.qkv_bits_parallel(w, workers=16)
    q, k, v = (torch.from_numpy(x).view(torch.bfloat16).cuda() for x in (qb, kb, vb))
    del qb, kb, vb
    cfg = dr.radial_cfg(w.num_frames, w.tokens_per_frame, w.block_size, w.gamma, w.lam, w.theta_c, w.theta_m)
    cand = dr.build_candidates(cfg)           # setup: sizes the buffers (reports nnz)
    import ctypes
    L = _lib.lib()
    dims = _lib.Dims(w.batch, w.heads, w.head_dim, 0)
    wsb = ctypes.c_size_t(0)
    ms_mask = None
    if args.mode == "decay-static":
        # content-free mask, built once (cached across layers and steps)
        kept = dr.static_select(cand, rhos[0], rhos[1], args.seed, batch=w.batch, heads=w.heads)
        # wall clock of the whole build (candidate CSR, whose size the host reads, and the mask)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(3):
            c2 = dr.build_candidates(cfg)
            dr.static_select(c2, rhos[0], rhos[1], args.seed, batch=w.batch, heads=w.heads)
        torch.cuda.synchronize()
        ms_mask = (time.perf_counter() - t0) * 1e3 / 3
    elif args.mode == "token":
        kept = dr.token_select(q, k, cand, taus[0], taus[1])
        tokc = _lib.TokenCfg(2, 0, float(taus[0]), float(taus[1]), 1e-6)
        _lib.check(L.dr_token_select_workspace(ctypes.byref(dims), ctypes.byref(cfg), ctypes.byref(tokc), cand.nnz,
                                               ctypes.byref(wsb)))
    else:
        kept = dr.score_select(q, k, cand, mode=args.mode, ratio=ratio, tau=tau)
        selc = dr._select_cfg(args.mode, ratio, tau, 0)
        _lib.check(L.dr_score_select_workspace(ctypes.byref(dims), ctypes.byref(cfg), ctypes.byref(selc),
                                               cand.nnz, ctypes.byref(wsb)))
    out = torch.empty_like(q)
    # preallocated buffers for the timed step (no allocation inside it)
    ws = torch.empty(wsb.value, dtype=torch.uint8, device="cuda")
    row_ptr = torch.empty_like(cand.row_ptr)
    cols = torch.empty_like(cand.cols)
    kept_col, kept_cnt = torch.empty_like(kept.kept_col), torch.empty_like(kept.kept_cnt)
    gwsb = ctypes.c_size_t(0)
    _lib.check(L.dr_query_groups_workspace(ctypes.byref(dims), ctypes.byref(gwsb)))
    gws = torch.empty(gwsb.value, dtype=torch.uint8, device="cuda")
    gmodes = torch.zeros(w.batch * w.heads, dtype=torch.int32, device="cuda")
    scale = 1.0 / math.sqrt(w.head_dim)

    def stream():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step_candidates():
        _lib.check(L.dr_build_candidates(ctypes.byref(cfg), row_ptr.data_ptr(), cols.data_ptr(), cand.nnz, None,
                                         stream()))

    def step_select():
        if args.mode == "token":
            _lib.check(L.dr_token_select(ctypes.byref(dims), ctypes.byref(cfg), ctypes.byref(tokc), q.data_ptr(),
                                         k.data_ptr(), row_ptr.data_ptr(), cols.data_ptr(), cand.nnz,
                                         kept_col.data_ptr(), kept_cnt.data_ptr(), ws.data_ptr(), ws.numel(),
                                         stream()))
            return
        _lib.check(L.dr_score_select(ctypes.byref(dims), ctypes.byref(cfg), ctypes.byref(selc), q.data_ptr(),
                                     k.data_ptr(), row_ptr.data_ptr(), cols.data_ptr(), cand.nnz,
                                     kept_col.data_ptr(), kept_cnt.data_ptr(), None, ws.data_ptr(), ws.numel(),
                                     stream()))

    def step_groups():
        if args.no_groups:
            return
        _lib.check(L.dr_query_groups(ctypes.byref(dims), ctypes.byref(cfg), row_ptr.data_ptr(), cand.nnz,
                                     kept_col.data_ptr(), kept_cnt.data_ptr(), gmodes.data_ptr(), gws.data_ptr(),
                                     gws.numel(), stream()))

    def step_attn():
        if args.no_groups:
            _lib.check(L.dr_sparse_attn(ctypes.byref(dims), ctypes.byref(cfg), q.data_ptr(), k.data_ptr(),
                                        v.data_ptr(), row_ptr.data_ptr(), cand.nnz, kept_col.data_ptr(),
                                        kept_cnt.data_ptr(), ctypes.c_float(scale), out.data_ptr(), stream()))
            return
        _lib.check(L.dr_sparse_attn_grouped(ctypes.byref(dims), ctypes.byref(cfg), q.data_ptr(), k.data_ptr(),
                                            v.data_ptr(), row_ptr.data_ptr(), cand.nnz, kept_col.data_ptr(),
                                            kept_cnt.data_ptr(), gmodes.data_ptr(), ctypes.c_float(scale),
                                            out.data_ptr(), stream()))

    if args.mode == "decay-static":
        # the cached mask and its grouping
        row_ptr.copy_(cand.row_ptr)
        cols.copy_(cand.cols)
        kept_col.copy_(kept.kept_col)
        kept_cnt.copy_(kept.kept_cnt)
        step_groups()

    def step():
        if args.mode == "decay-static":   # the mask is cached: attention only
            step_attn()
            return
        step_candidates()
        step_select()
        step_groups()
        step_attn()

    # --graph: the step's launches recorded once in a HIP graph and replayed
    # (no host launch overhead per kernel; measured no faster than eager
    # launches, which the GPU never waits for); eager if capture fails.
    run_step, launch = step, "eager"
    if args.graph:
        try:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            torch.cuda.synchronize()
            run_step, launch = graph.replay, "hip_graph"
        except Exception as exc:   # noqa: BLE001 - report and time the eager launches
            print(f"# graph capture failed ({exc}); timing eager launches", file=sys.stderr, flush=True)
            torch.cuda.synchronize()

    for _ in range(args.warmup):
        run_step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # per-stage HIP-event timing on the launch stream
    med = {}
    sel_name = "token_select" if args.mode == "token" else "score_select"
    ms_cand = event_ms(step_candidates, args.stage_iters, torch, med, "build_candidates") if ms_mask is None else None
    ms_sel = event_ms(step_select, args.stage_iters, torch, med, sel_name) if ms_mask is None else None
    ms_groups = event_ms(step_groups, args.stage_iters, torch, med, "query_groups") if not args.no_groups else None
    ms_attn = event_ms(step_attn, args.stage_iters, torch, med, "sparse_attn")
    modes_used = np.bincount(gmodes.cpu().numpy(), minlength=3).tolist() if not args.no_groups else None
    kept_total = int(kept_cnt.sum().item())
    Sb = cand.num_blocks
    flops = 4.0 * w.block_size ** 2 * w.head_dim * kept_total
    sparsity = 1.0 - kept_total / (w.batch * w.heads * Sb * Sb)
    ms_dense = None
    if not args.no_dense:
        dense_out = torch.empty_like(q)
        dr.attn(q, k, v, out=dense_out)
        ms_dense = event_ms(lambda: dr.attn(q, k, v, out=dense_out), args.dense_iters, torch, med, "dense_attn")
    dense_flops = 4.0 * w.batch * w.heads * w.seq_len ** 2 * w.head_dim
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (ms_attn * 1e-3) / 1e12
    tr = traffic_record(w.name, args.mode)
    res = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "mode": args.mode, "ratio": ratio if args.mode == "static" else None,
                   "tau": tau if args.mode == "dynamic" else None,
                   "tau_near_far": list(taus) if taus else None,
                   "rho_near_far": list(rhos) if rhos else None, "seed": args.seed if rhos else None,
                   "theta_c": w.theta_c, "theta_m": w.theta_m,
                   "batch": w.batch, "heads": w.heads,
                   "seq_len": w.seq_len, "head_dim": w.head_dim, "block_size": w.block_size, "gamma": w.gamma,
                   "lambda": w.lam, "parallelism": "single-gpu", "launch": launch},
        "sparsity": round(sparsity, 4),
        "candidate_density": round(cand.nnz / Sb ** 2, 4),
        "kept_blocks": kept_total,
        "speedup_vs_dense": round(ms_dense / ms_step, 3) if ms_dense else None,
        "speedup_vs_dense_attention_only": round(ms_dense / ms_attn, 3) if ms_dense else None,
        # selection + attention, the candidate set counted as a cached setup cost
        "speedup_vs_dense_select_attn": (round(ms_dense / (ms_sel + ms_attn), 3)
                                         if ms_dense and ms_sel is not None else None),
        "stage_ms": ({"mask_build": round(ms_mask, 4)} if ms_mask is not None else
                     {"build_candidates": round(ms_cand, 4),
                      ("token_select" if args.mode == "token" else "score_select"): round(ms_sel, 4)}) |
                    ({"query_groups": round(ms_groups, 4)} if ms_groups is not None else {}) |
                    {"sparse_attn": round(ms_attn, 4), "dense_attn": round(ms_dense, 3) if ms_dense else None},
        "stage_ms_median": med,
        "query_grouping": ({"heads_per_mode": modes_used} if modes_used is not None else "consecutive"),
        "dense_tflops": round(dense_flops / (ms_dense * 1e-3) / 1e12, 2) if ms_dense else None,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": tr["hbm_bytes_per_launch"] if tr else None,
                     "kernel": "dr_sparse_attn (attn_kernel<128,B_s,sparse>)"},
    }
    if args.calib_copy:
        # a plain copy kernel of known size: its FETCH_SIZE / WRITE_SIZE readings
        # scale the attention kernel's counters to bytes
        # (an elementwise kernel, so that the copy runs on the shader engines)
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu:
        print("# timing the CPU oracle sample", file=sys.stderr, flush=True)
        extra = taus if args.mode == "token" else ((rhos[0], rhos[1], args.seed) if rhos else tau)
        res["cpu_baseline"] = cpu_baseline(w, args.mode, ratio, extra, args.cpu_blocks)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
