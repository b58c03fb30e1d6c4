"""Throughput of one local-cluster-attention step on one MI355X.

A step is one pass of the whole hot path over one batch: neighbour-list
build, forward (O + LSE) and backward (dQ, dK, dV), on the stage-1
pre-training shape (32 images x 2048 visible tokens of a 64x64 Perlin-masked
patch grid, 4 heads x 32 dims, bf16, clusters of 8, 48 key slots).

Inputs are resident in HBM before the timed region.  Steps rotate over
several copies of the batch whose combined footprint exceeds the 256 MB
last-level cache, so no step reads data a recent step left in cache (the
"warm" figure, every step on one copy, is reported beside it).

Prints one JSON line.  Usage:
    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config stage1]

Other configurations (parity-test workloads of the wider rows, measured the
same way): stage2, stage3, stage4, highres, stress (2D attention), varlen
(packed images), volume, volume_hr (3D tokens), knn_decoder (KNN-cache
sampler), merge_stages (token merging).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor figure
# kernels behind each entry point on the bf16/f16 path (the roofline is per
# entry point; the committed kernel trace splits it per kernel)
ENTRY_KERNELS = {
    "build": ["build_small_kernel (N <= 4096) | segsort_kernel, merge_round_kernel, "
              "centroid_box_kernel, select_box_kernel (N > 4096)"],
    "plan": ["plan_small_kernel (images <= 4096 tokens) | plan_init/inv/count/scan/place/sort_kernel"],
    "fwd": ["fwd_lds_kernel"],
    "bwd": ["bwd_q_lds_kernel", "bwd_kv_lds_kernel"],
}
MERGE_ENTRY_KERNELS = {
    "plan": ["merge_assign_kernel, merge_members_kernel (images <= 4096 tokens) | merge_select_kernel, "
             "merge_abucket_count/place_kernel, merge_assign_wide_kernel, merge_gcount/gplace/grank_kernel, "
             "zero_i32_kernel, segment_scan_kernel (larger)"],
    "fwd": ["merge_fwd_kernel"],
    "bwd": ["merge_bwd_kernel"]}
SAMPLER_ENTRY_KERNELS = {
    "table": ["knn_table_kernel (images <= 4096 tokens) | knn_bucket_count/place_kernel, "
              "segment_scan_kernel, knn_table_search_kernel (larger)"],
    "fwd": ["knn_fwd_kernel"],
    "bwd": ["knn_bwd_query_kernel", "knn_pcount_kernel (partition counts and walk order)",
            "knn_pprefix_kernel", "segment_scan_kernel", "knn_pplace_kernel",
            "knn_dfeat_kernel (feature gradient and dp); larger images: zero_i32_kernel, "
            "knn_lplace/lrank_kernel, knn_bucket_count/place_kernel in place of the partition kernels"],
}
BF16_MFMA_PEAK_TFLOPS = 2500.0  # dense


def algorithmic(cfg):
    """Compulsory bytes and matmul flops of each entry point (every tensor
    touched once; gathered re-reads, workspace and atomics not counted)."""
    T, H, D, nk = cfg.tokens, cfg.H, cfg.D, cfg.nk
    C = cfg.B * cfg.C
    return algorithmic_tc(T, C, H, D, nk, cfg.k, cfg.cs, cfg.dtype)


def algorithmic_tc(T, C, H, D, nk, k, cs, dtype):
    """The same for T tokens in C clusters (a partial cluster counts as one)."""
    es = 4 if dtype == "f32" else 2
    t = T * H * D * es                  # one [tokens, H, D] tensor
    lse = T * H * 4
    idx = C * cs * 4 + C * nk * 4       # q_idx + key_idx
    return {
        "build": {"bytes": T * 8 + C * cs * 4 + C * k * 4 + C * nk * 4, "flops": 0},
        # lists in; per key cluster one entry per referencing cluster out
        # (counted at one per list slot group: 48 B of entry, tokens, mults)
        "plan": {"bytes": idx + C * (nk // cs) * 48, "flops": 0},
        "fwd": {"bytes": 3 * t + t + lse + idx, "flops": T * H * 4 * nk * D},
        "bwd": {"bytes": 5 * t + lse + 3 * t + idx, "flops": T * H * 10 * nk * D},
    }


def formulation_bytes(cfg, dom, alg, dur):
    """The matrix-core backward (bf16/f16, 48 slots) takes Delta from P and
    dP and reads no O, so it must move one [tokens, H, D] tensor fewer than
    the algorithmic bytes above (which count O as a backward input);
    reported beside the roofline so that its fraction can be read on either
    count."""
    if dom != "bwd" or cfg.dtype == "f32" or cfg.nk != 48:
        return {}
    b = alg["bwd"]["bytes"] - cfg.tokens * cfg.H * cfg.D * 2
    gbps = b / (dur["bwd"] * 1e-6) / 1e9
    return {"bytes_this_formulation_moves": b, "frac_on_those_bytes": gbps / HBM_PEAK_GBPS}


def copy_bandwidth(torch, ca, nbytes=1 << 30, reps=10):
    """Achievable HBM bandwidth: the library's plain copy kernel
    (cluster_attn_device_copy) moving `nbytes` (1 GiB read + 1 GiB written),
    median over `reps` timed copies; torch's own copy_ beside it."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    ca.device_copy(dst, src)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        ca.device_copy(dst, src)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(reps))
    med = ms[reps // 2]
    assert torch.equal(dst[:4096], src[:4096])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    torch_gbps = 2 * nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    del src, dst
    return {"GBps": 2 * nbytes / (med * 1e-3) / 1e9, "bytes_moved": 2 * nbytes,
            "kernel": "cluster_attn_device_copy (copy16_kernel)", "median_of": reps,
            "torch_copy_GBps": torch_gbps}


def entry_times(torch, calls, n_ev, n_sets):
    """Per-launch durations of each entry point: HIP events on the launch
    stream recorded between n_ev back-to-back calls (rotating input copies),
    so every call has its own event pair while the queue stays full.
    Returns name -> {mean, median, p10, p90} in microseconds."""
    out = {}
    for name, call in calls.items():
        call(0)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev + 1)]
        ev[0].record()
        for i in range(n_ev):
            call(i % n_sets)
            ev[i + 1].record()
        torch.cuda.synchronize()
        d = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n_ev))
        q = lambda f: d[min(n_ev - 1, int(round(f * (n_ev - 1))))]
        out[name] = {"mean": ev[0].elapsed_time(ev[n_ev]) * 1e3 / n_ev, "median": q(0.5),
                     "p10": q(0.1), "p90": q(0.9)}
    return out


def entry_times_stream(torch, calls, n_sets, blocks=20):
    """Back-to-back eager calls in blocks of one rotation (n_sets calls, one
    per input copy) with HIP events only between blocks: nothing waits
    between the calls of a block, so while the host issues calls faster than
    the GPU runs them this is the GPU's time per call in a full queue (the
    kernels and the gaps between them).  Returns name -> {mean, median, p10,
    p90} (per call, microseconds, statistics over the blocks)."""
    out = {}
    for name, call in calls.items():
        for i in range(n_sets):
            call(i)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(blocks + 1)]
        ev[0].record()
        for b in range(blocks):
            for i in range(n_sets):
                call(i)
            ev[b + 1].record()
        torch.cuda.synchronize()
        d = sorted(ev[b].elapsed_time(ev[b + 1]) * 1e3 / n_sets for b in range(blocks))
        q = lambda f: d[min(blocks - 1, int(round(f * (blocks - 1))))]
        out[name] = {"mean": ev[0].elapsed_time(ev[blocks]) * 1e3 / (blocks * n_sets),
                     "median": q(0.5), "p10": q(0.1), "p90": q(0.9)}
    return out


def pick_timing(names, graph, stream):
    """Per-launch figure of each entry point: the lower mean of the graph
    replay (when its outputs matched an eager call's) and the eager stream;
    both are real launch modes of the same work.  Returns (stats, how)."""
    stats, how = {}, {}
    for name in names:
        g, s = (graph or {}).get(name), stream[name]
        if g is not None and g["mean"] <= s["mean"]:
            stats[name], how[name] = g, ("graph: one call per rotating copy captured, 10 "
                                         "replays, every captured call bitwise equal to an "
                                         "eager call (faster than the eager stream)")
        else:
            stats[name], how[name] = s, ("stream: blocks of back-to-back eager calls over the "
                                         "rotating copies, events between blocks only"
                                         + (" (faster than the graph replay)" if g is not None
                                            else " (no bitwise-matching graph replay: the plan "
                                            "buffer also holds scratch whose contents vary)"
                                            if graph is not None else ""))
    return stats, how


def entry_times_graph(torch, calls, n_sets, replays=10):
    """The same entry points launched from a HIP graph: one call per
    rotating copy captured once, the graph replayed `replays` times with HIP
    events around each replay, so the time is the GPU's (kernels and the
    gaps between them) without the Python launch cost.  Every captured
    call's outputs are compared bit for bit with an eager call on the same
    inputs after the first replay; an entry point whose graph does not match
    is reported as None.  Returns name -> {mean, median, p10, p90} (per call,
    microseconds) or None."""
    out = {}
    for name, call in calls.items():
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            call(0)                       # warm-up on the capture stream
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            got = [call(i) for i in range(n_sets)]
        g.replay()
        torch.cuda.synchronize()
        flat = lambda r: [t for t in (r if isinstance(r, (tuple, list)) else (r,))
                          if hasattr(t, "is_cuda")]
        ok = True
        for i in range(n_sets):
            ref = flat(call(i))
            torch.cuda.synchronize()
            ok = ok and all(torch.equal(a, b) for a, b in zip(flat(got[i]), ref))
        if not ok:
            out[name] = None
            continue
        ts = []
        for _ in range(replays):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / n_sets)
        ts.sort()
        q = lambda f: ts[min(len(ts) - 1, int(round(f * (len(ts) - 1))))]
        out[name] = {"mean": sum(ts) / len(ts), "median": q(0.5), "p10": q(0.1), "p90": q(0.9)}
        del g, got
    return out


def rotation_copies(requested, tensor_bytes, tensors_read=3, llc_bytes=256 << 20):
    """Rotating input copies so that every timed entry point walks at least
    twice the 256 MB last-level cache before it reads a copy again (the
    forward reads three tensors of a copy; the backward more)."""
    if requested:
        return requested
    return max(4, -(-2 * llc_bytes // (tensors_read * tensor_bytes)))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _oracle_images(args):
    """Worker of the all-cores baseline: the oracle's gathered forward +
    backward on some images, one thread per worker process."""
    from threadpoolctl import threadpool_limits

    import oracle as O

    q, k, v, do, q_idx, key_idx, scale = args
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.attn_fwd_gathered(q, k, v, q_idx, key_idx, scale)
        O.attn_bwd_gathered(q, k, v, do, q_idx, key_idx, scale)
        return time.perf_counter() - t0


def cpu_baseline(cfg, case, images: int, single_images: int = 8, runs: int = 3):
    """The fp64 oracle (gathered form, forward + backward; neighbour build
    excluded) timed on the host: single-threaded on `single_images` images
    and on all cores (one worker process per core, capped at 16, each taking
    whole images) over `images` images; median of `runs` runs each."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import statistics

    import numpy as np

    import oracle as O

    build = O.build_neighbors_3d if case["coords"].shape[-1] == 3 else O.build_neighbors
    perm, _, key_idx = build(case["coords"][:images], cfg.G)
    q_idx = perm.reshape(images, cfg.C, cfg.cs)
    arrs = [case[n][:images].float().numpy() for n in ("q", "k", "v", "do")]
    scale = 1.0 / math.sqrt(cfg.D)
    job = lambda lo, hi: tuple(a[lo:hi] for a in arrs) + (q_idx[lo:hi], key_idx[lo:hi], scale)

    one = [_oracle_images(job(0, single_images)) for _ in range(runs)]
    t1 = statistics.median(one)
    workers = max(1, min(16, os.cpu_count() or 1, images))
    per = -(-images // workers)
    parts = [job(lo, min(images, lo + per)) for lo in range(0, images, per)]
    alls = []
    with cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
        list(ex.map(_oracle_images, parts[:1]))         # start the workers (imports) untimed
        for _ in range(runs):
            t0 = time.perf_counter()
            list(ex.map(_oracle_images, parts))
            alls.append(time.perf_counter() - t0)
    ta = statistics.median(alls)
    del np
    return {
        "value": images * cfg.N / ta,
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{images} of {cfg.B} images ({images * cfg.N} tokens), fp64 gathered "
                  f"forward+backward, {workers} worker processes x 1 thread, median of {runs}: "
                  f"{ta:.2f} s",
        "single_thread": {"value": single_images * cfg.N / t1, "unit": "tokens/s", "cores": 1,
                          "sample": f"{single_images} images, median of {runs}: {t1:.2f} s"},
        "host_cpu": cpu_model(),
        "os_cpu_count": os.cpu_count(),
    }


# the kernel sources whose rocprofv3 counter summaries bench.py reports
KERNEL_SOURCES = ("attn_mfma.hip", "attn_valu.hip", "mfma_util.h", "common.h", "bwd_plan.hip",
                  "neighbors.hip", "dpp_scan.h")


SAMPLER_SOURCES = ("knn_sampler.hip", "scan.hip", "common.h")
MERGE_SOURCES = ("token_merge.hip", "scan.hip", "common.h")


def kernel_source_hash(files=KERNEL_SOURCES) -> str:
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "gathered_local_attention_amd", "csrc")
    for name in files:
        h.update(name.encode())
        with open(os.path.join(d, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_summary(config: str, files=KERNEL_SOURCES):
    """The committed rocprofv3 summary of a configuration
    (profiles/<config>_hbm_traffic.json or _counters.json) if it was taken on
    the current kernel sources (same hash), else None."""
    for suffix in ("hbm_traffic", "counters"):
        path = os.path.join(ROOT, "profiles", f"{config}_{suffix}.json")
        if os.path.exists(path):
            with open(path) as f:
                rec = json.load(f)
            if rec.get("source_sha256") == kernel_source_hash(files):
                return rec
    return None


def measured_traffic(config: str, entry: str, files=KERNEL_SOURCES):
    """HBM bytes per launch of an entry point from FETCH_SIZE / WRITE_SIZE
    (calibrated against the copy kernel) in the committed summary, or None."""
    rec = counter_summary(config, files)
    e = None if rec is None else rec.get("entries", {}).get(entry)
    return None if e is None else e["traffic_bytes"]


def measured_mfma(config: str, dur_us: dict):
    """MFMA utilisation per entry point from the committed summary's MFMA
    counters (MfmaUtil, SQ_INSTS_VALU_MFMA_MOPS_BF16), with the flops over
    this run's entry time; None without a current summary."""
    rec = counter_summary(config)
    if rec is None or "mfma" not in rec:
        return None
    out = {}
    for entry, m in rec["mfma"].items():
        tf = m["bf16_flops"] / (dur_us[entry] * 1e-6) / 1e12 if entry in dur_us else None
        out[entry] = {"mfma_busy_pct": m["busy_pct"], "bf16_flops_per_launch": m["bf16_flops"],
                      "TFLOPs": tf,
                      "frac_of_bf16_peak": None if tf is None else tf / BF16_MFMA_PEAK_TFLOPS}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="stage1")
    ap.add_argument("--copies", type=int, default=0,
                    help="rotating input copies (default: enough that every timed entry point "
                         "walks at least twice the 256 MB last-level cache)")
    ap.add_argument("--cpu-images", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(images shard across GPUs with no communication; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import gathered_local_attention_amd as ca
    from gen import (MERGE_CONFIGS, RAGGED_CONFIGS, SAMPLER_CONFIGS, VOLUME_CONFIGS, make_case,
                     make_volume_case)

    if args.config in RAGGED_CONFIGS:
        bench_varlen(args, torch, ca)
        return
    if args.config in SAMPLER_CONFIGS:
        bench_sampler(args, torch, ca)
        return
    if args.config in MERGE_CONFIGS:
        bench_merge(args, torch, ca)
        return
    case = make_volume_case(args.config) if args.config in VOLUME_CONFIGS else make_case(args.config)
    cfg = case["cfg"]
    scale = 1.0 / math.sqrt(cfg.D)
    dev = "cuda"
    # The host baseline runs first, before anything touches the GPU: its
    # worker processes are started while this process holds no GPU state.
    cpu_line = None
    if not args.no_cpu_baseline:
        cpu_line = cpu_baseline(cfg, case, min(args.cpu_images, cfg.B))
    tensor_bytes = case["q"].numel() * case["q"].element_size()
    args.copies = rotation_copies(args.copies, tensor_bytes)
    ca._lib.load()

    # rotating copies of the batch, all resident in HBM
    sets = []
    for r in range(args.copies):
        s = {"coords": torch.from_numpy(case["coords"]).to(dev)}
        for n in ("q", "k", "v", "do"):
            s[n] = case[n].to(dev)
        sets.append(s)
    bws = torch.empty(ca.build_workspace_bytes(cfg.B, cfg.N, cfg.cs, cfg.k) or 1,
                      dtype=torch.uint8, device=dev)
    gws = torch.empty(ca.bwd_workspace_bytes(case["q"].dtype, cfg.B, cfg.N, cfg.H, cfg.D,
                                             cfg.cs, cfg.nk), dtype=torch.uint8, device=dev)

    # A step runs the lists' whole life once: neighbour build, the
    # backward's transposed lists (plan), forward, backward on that plan.
    # In a model the build and the plan serve every layer of a stage.
    def step(s):
        perm, nbr, key = ca.build_neighbors(s["coords"], cfg.G, cfg.cs, cfg.k, workspace=bws)
        plan = ca.bwd_plan(perm, key, cfg.N)
        o, lse = ca.fwd(s["q"], s["k"], s["v"], perm, key, scale)
        dq, dk, dv = ca.bwd(s["q"], s["k"], s["v"], o, s["do"], lse, perm, key, scale,
                            workspace=gws, plan=plan)
        return dq

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # per-entry-point durations: HIP events on the launch stream around
    # n_ev back-to-back calls of one entry point (rotating copies), so the
    # per-launch average compares with the kernel trace (the gaps between
    # back-to-back kernels, ~1-2 us each, are included)
    n_ev = min(args.steps, 100)
    outs = []
    for s in sets:
        perm, nbr, key = ca.build_neighbors(s["coords"], cfg.G, cfg.cs, cfg.k, workspace=bws)
        o, lse = ca.fwd(s["q"], s["k"], s["v"], perm, key, scale)
        outs.append((perm, key, o, lse, ca.bwd_plan(perm, key, cfg.N)))
    calls = {
        "build": lambda i: ca.build_neighbors(sets[i]["coords"], cfg.G, cfg.cs, cfg.k,
                                              workspace=bws),
        "plan": lambda i: ca.bwd_plan(outs[i][0], outs[i][1], cfg.N),
        "fwd": lambda i: ca.fwd(sets[i]["q"], sets[i]["k"], sets[i]["v"], outs[i][0],
                                outs[i][1], scale),
        "bwd": lambda i: ca.bwd(sets[i]["q"], sets[i]["k"], sets[i]["v"], outs[i][2],
                                sets[i]["do"], outs[i][3], outs[i][0], outs[i][1], scale,
                                workspace=gws, plan=outs[i][4]),
        # the self-planning backward (plan + passes in one call), for reference
        "bwd_with_plan": lambda i: ca.bwd(sets[i]["q"], sets[i]["k"], sets[i]["v"], outs[i][2],
                                          sets[i]["do"], outs[i][3], outs[i][0], outs[i][1],
                                          scale, workspace=gws),
    }
    eager = entry_times(torch, calls, n_ev, len(sets))
    graph = entry_times_graph(torch, calls, len(sets))
    stream = entry_times_stream(torch, calls, len(sets))
    # per-launch figures: the faster of the graph replay (where it matched
    # the eager results) and the eager stream; the per-call-event figures
    # (an event between every two calls) are kept beside them
    stats, how = pick_timing(calls, graph, stream)
    dur = {name: st["mean"] for name, st in stats.items()}   # microseconds per launch

    # warm-cache variant: every step on the same copy
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[0])
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t0) * 1e3 / args.steps

    alg = algorithmic(cfg)
    dom = max(("build", "plan", "fwd", "bwd"), key=lambda k: dur[k])
    achieved = alg[dom]["bytes"] / (dur[dom] * 1e-6) / 1e9
    fb_us = dur["fwd"] + dur["bwd"]
    fb_bytes = alg["fwd"]["bytes"] + alg["bwd"]["bytes"]
    fb_flops = alg["fwd"]["flops"] + alg["bwd"]["flops"]
    copy = copy_bandwidth(torch, ca)
    copy_gbps = copy["GBps"]
    fb_gbps = fb_bytes / (fb_us * 1e-6) / 1e9
    fb_med = stats["fwd"]["median"] + stats["bwd"]["median"]

    line = {
        "metric": "cluster-attention fwd+bwd tokens/sec and % of HBM roofline (stage-1 shape)"
                  if cfg.name == "stage1" else
                  f"cluster-attention fwd+bwd tokens/sec and % of HBM roofline ({cfg.name} shape)",
        "value": cfg.tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f32": "f32", "bf16": "bf16", "f16": "f16"}[cfg.dtype],
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: B={cfg.B} {'volumes' if case['coords'].shape[-1] == 3 else 'images'}"
                        f" x N={cfg.N} tokens ({case['coords'].shape[-1]}D coordinates), "
                        f"H={cfg.H}x{cfg.D}, clusters of {cfg.cs} ({cfg.C} per image), {cfg.nk} key "
                        f"slots, {cfg.dtype}; step = neighbour build + backward plan + forward + "
                        "backward",
            "B": cfg.B, "N": cfg.N, "H": cfg.H, "D": cfg.D, "cs": cfg.cs, "nk": cfg.nk,
            "geometry": cfg.geometry, "seed": cfg.seed, "rotating_copies": args.copies,
            "rotation_footprint_MB": {
                "fwd": round(args.copies * 3 * tensor_bytes / 1e6, 1),
                "bwd": round(args.copies * 6 * tensor_bytes / 1e6, 1),
                "step": round(args.copies * 4 * tensor_bytes / 1e6, 1)},
        },
        "roofline": {
            "bound": "hbm",
            "kernel": {"build": "cluster_attn_build_neighbors", "plan": "cluster_attn_bwd_plan",
                       "fwd": "cluster_attn_fwd", "bwd": "cluster_attn_bwd_planned"}[dom],
            "entry_point_kernels": ENTRY_KERNELS[dom],
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": measured_traffic(cfg.name, dom),
            "algorithmic_bytes": alg[dom]["bytes"],
            "avg_us": dur[dom],
            **formulation_bytes(cfg, dom, alg, dur),
        },
        "fwd_bwd": {
            "note": "forward + backward on built lists and plan (both depend on the coordinates "
                    "only and serve every layer of a stage); the self-planning backward is "
                    "entry_us.bwd_with_plan",
            "us": fb_us,
            "us_median": fb_med,
            "tokens_per_s": cfg.tokens / (fb_us * 1e-6),
            "effective_GBps": fb_gbps,
            "hbm_frac": fb_gbps / HBM_PEAK_GBPS,
            "copy_frac": fb_gbps / copy_gbps,
            "effective_TFLOPs": fb_flops / (fb_us * 1e-6) / 1e12,
            "mfma_bf16_frac": fb_flops / (fb_us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
        },
        "entry_us": dur,
        "entry_us_stats": stats,
        "entry_timing": how,
        "entry_us_graph": {name: (st["mean"] if st else None) for name, st in graph.items()},
        "entry_us_stream": {name: st["mean"] for name, st in stream.items()},
        "entry_us_eager": {name: st["mean"] for name, st in eager.items()},
        "entry_us_stats_eager": eager,
        "mfma_counters": measured_mfma(cfg.name, dur),
        "warm_ms_per_step": warm_ms,
        "copy_GBps": copy_gbps,
        "copy": copy,
        "roofline_vs_copy": achieved / copy_gbps,
        "cpu_baseline": cpu_line,
    }
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# Packed batches of images of different sizes: --config varlen
# ---------------------------------------------------------------------------

def varlen_cpu_baseline(cfg, case, images: int):
    """The fp64 oracle (gathered forward + backward) on the first `images`
    images of the packed batch, single-threaded; build excluded."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O

    n = sum(case["lengths"][:images])
    q_idx, _, key_idx, _, _ = O.build_neighbors_varlen(case["coords"][:n], case["lengths"][:images],
                                                        cfg.G)
    args = [case[x][:n][None] for x in ("q", "k", "v", "do")]
    scale = 1.0 / math.sqrt(cfg.D)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        O.attn_fwd_gathered(*args[:3], q_idx[None], key_idx[None], scale)
        O.attn_bwd_gathered(*args, q_idx[None], key_idx[None], scale)
        dt = time.perf_counter() - t0
    return {
        "value": n / dt,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{images} of {cfg.B} images ({n} tokens), fp64 gathered forward+backward, "
                  f"{dt:.1f} s",
    }


def bench_varlen(args, torch, ca):
    ca._lib.load()
    args.copies = args.copies or 4
    from gen import make_varlen_case

    case = make_varlen_case(args.config)
    cfg = case["cfg"]
    lengths = case["lengths"]
    T = case["coords"].shape[0]
    tok, clu = ca.varlen_offsets(lengths, cfg.cs)
    Ct = clu[-1]
    scale = 1.0 / math.sqrt(cfg.D)
    dev = "cuda"
    offsets = (torch.tensor(tok, dtype=torch.int32).to(dev),
               torch.tensor(clu, dtype=torch.int32).to(dev))
    sets = []
    for r in range(args.copies):
        s = {"coords": torch.from_numpy(case["coords"]).to(dev)}
        for n in ("q", "k", "v", "do"):
            s[n] = case[n].to(dev)
        sets.append(s)
    max_n = max(lengths)
    lib = ca._lib.load()
    bws = torch.empty(max(1, lib.cluster_attn_build_neighbors_varlen_workspace(
        cfg.B, T, Ct, max_n, cfg.cs, cfg.k)), dtype=torch.uint8, device=dev)
    dt = {"f32": 0, "bf16": 1, "f16": 2}[cfg.dtype]
    gws = torch.empty(lib.cluster_attn_bwd_varlen_workspace(dt, T, Ct, cfg.H, cfg.D, cfg.cs, cfg.nk),
                      dtype=torch.uint8, device=dev)

    def build(s):
        return ca.build_neighbors_varlen(s["coords"], lengths, cfg.G, cfg.cs, cfg.k, workspace=bws,
                                         offsets=offsets)

    def plan_of(q_idx, key):
        return ca.bwd_plan_varlen(q_idx, key, lengths, offsets=offsets)

    def step(s):
        q_idx, _, key, _, _ = build(s)
        plan = plan_of(q_idx, key)
        o, lse = ca.fwd_varlen(s["q"], s["k"], s["v"], q_idx, key, scale)
        return ca.bwd_varlen(s["q"], s["k"], s["v"], o, s["do"], lse, q_idx, key, scale,
                             workspace=gws, plan=plan)

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    n_ev = min(args.steps, 100)
    outs = []
    for s in sets:
        q_idx, _, key, _, _ = build(s)
        o, lse = ca.fwd_varlen(s["q"], s["k"], s["v"], q_idx, key, scale)
        outs.append((q_idx, key, o, lse, plan_of(q_idx, key)))
    calls = {
        "build": lambda i: build(sets[i]),
        "plan": lambda i: plan_of(outs[i][0], outs[i][1]),
        "fwd": lambda i: ca.fwd_varlen(sets[i]["q"], sets[i]["k"], sets[i]["v"], outs[i][0],
                                       outs[i][1], scale),
        "bwd": lambda i: ca.bwd_varlen(sets[i]["q"], sets[i]["k"], sets[i]["v"], outs[i][2],
                                       sets[i]["do"], outs[i][3], outs[i][0], outs[i][1], scale,
                                       workspace=gws, plan=outs[i][4]),
        "bwd_with_plan": lambda i: ca.bwd_varlen(sets[i]["q"], sets[i]["k"], sets[i]["v"],
                                                 outs[i][2], sets[i]["do"], outs[i][3], outs[i][0],
                                                 outs[i][1], scale, workspace=gws),
    }
    eager = entry_times(torch, calls, n_ev, len(sets))
    stats, how = pick_timing(calls, None, entry_times_stream(torch, calls, len(sets)))
    dur = {name: st["mean"] for name, st in stats.items()}

    alg = algorithmic_tc(T, Ct, cfg.H, cfg.D, cfg.nk, cfg.k, cfg.cs, cfg.dtype)
    dom = max(("build", "plan", "fwd", "bwd"), key=lambda k: dur[k])
    achieved = alg[dom]["bytes"] / (dur[dom] * 1e-6) / 1e9
    fb_us = dur["fwd"] + dur["bwd"]
    fb_bytes = alg["fwd"]["bytes"] + alg["bwd"]["bytes"]
    fb_flops = alg["fwd"]["flops"] + alg["bwd"]["flops"]
    line = {
        "metric": "cluster-attention fwd+bwd tokens/sec and % of HBM roofline "
                  f"(packed batch, {cfg.name})",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: B={cfg.B} images of {min(lengths)}..{max(lengths)} tokens "
                        f"(T={T}, {Ct} clusters), H={cfg.H}x{cfg.D}, {cfg.nk} key slots, "
                        f"{cfg.dtype}; step = packed neighbour build + backward plan + forward + "
                        "backward",
            "B": cfg.B, "T": T, "clusters": Ct, "H": cfg.H, "D": cfg.D, "geometry": cfg.geometry,
            "seed": cfg.seed, "rotating_copies": args.copies,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": {"build": "cluster_attn_build_neighbors_varlen", "plan": "cluster_attn_bwd_plan_varlen",
                       "fwd": "cluster_attn_fwd_varlen", "bwd": "cluster_attn_bwd_planned"}[dom],
            "entry_point_kernels": ENTRY_KERNELS[dom],
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": None,
            "algorithmic_bytes": alg[dom]["bytes"],
            "avg_us": dur[dom],
        },
        "fwd_bwd": {
            "us": fb_us,
            "tokens_per_s": T / (fb_us * 1e-6),
            "effective_GBps": fb_bytes / (fb_us * 1e-6) / 1e9,
            "hbm_frac": fb_bytes / (fb_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
            "effective_TFLOPs": fb_flops / (fb_us * 1e-6) / 1e12,
            "mfma_bf16_frac": fb_flops / (fb_us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS,
        },
        "entry_us": dur,
        "entry_us_stats": stats,
        "entry_timing": how,
        "entry_us_eager": {name: st["mean"] for name, st in eager.items()},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = varlen_cpu_baseline(cfg, case, min(args.cpu_images, cfg.B))
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# KNN-cache point sampler (decoder): --config knn_decoder
# ---------------------------------------------------------------------------

def sampler_algorithmic(cfg):
    """Compulsory bytes per entry point, summed over the levels (every tensor
    touched once; table rows re-read by several queries, workspace and the
    token-major entry lists not counted)."""
    es = 4 if cfg.dtype == "f32" else 2
    B, M, G, K = cfg.B, cfg.M, cfg.G, cfg.K
    tab = G * G * K * 4
    out = {"table": 0, "fwd": 0, "bwd": 0}
    for N, C in cfg.levels:
        out["table"] += B * (N * 8 + tab)
        out["fwd"] += B * (M * 8 + tab + N * 8 + N * C * es + M * C * es)
        out["bwd"] += B * (M * 8 + tab + N * 8 + N * C * es + M * C * es + N * C * es + M * 8) + 4
    return out


def sampler_cpu_baseline(cfg, case, images: int):
    """The fp64 oracle's sampler forward + backward on `images` images, all
    levels, single-threaded.  The table rows the queries use are ranked by
    the oracle beforehand, outside the timing (only the queries' cells: the
    other cells are never read)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle as O

    def rows_of(coords, q):
        i, j = O.query_cells(q, cfg.G)
        cells = np.unique(i * cfg.G + j)
        t = np.full((cfg.G, cfg.G, cfg.K), -1, dtype=np.int64)
        t[cells // cfg.G, cells % cfg.G] = O.knn_table_cells(coords, cfg.G, cfg.K, cells // cfg.G,
                                                            cells % cfg.G)
        return t

    tabs = [[rows_of(case["coords"][li][b], case["queries"][b]) for b in range(images)]
            for li in range(len(cfg.levels))]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for li in range(len(cfg.levels)):
            F = case["feats"][li].double().numpy()
            dO = case["dout"][li].double().numpy()
            for b in range(images):
                c, q = case["coords"][li][b], case["queries"][b]
                O.knn_sample_fwd(c, F[b], q, tabs[li][b], cfg.p)
                O.knn_sample_bwd(c, F[b], q, tabs[li][b], cfg.p, dO[b])
        dt = time.perf_counter() - t0
    return {
        "value": images * cfg.M / dt,
        "unit": "queries/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{images} of {cfg.B} images ({images * cfg.M} queries x {len(cfg.levels)} "
                  f"levels), fp64 forward+backward, tables excluded, {dt:.1f} s",
    }


def bench_sampler(args, torch, ca):
    ca._lib.load()
    args.copies = args.copies or 4
    from gen import make_sampler_case

    case = make_sampler_case(args.config)
    cfg = case["cfg"]
    dev = "cuda"
    L = len(cfg.levels)
    sets = []
    for r in range(args.copies):
        s = {"q": torch.from_numpy(case["queries"]).to(dev), "lv": []}
        for li in range(L):
            s["lv"].append({"coords": torch.from_numpy(case["coords"][li]).to(dev),
                            "feats": case["feats"][li].to(dev), "dout": case["dout"][li].to(dev)})
        sets.append(s)
    wss = [torch.empty(max(1, ca.knn_bwd_workspace_bytes(cfg.B, N, cfg.M, cfg.K)),
                       dtype=torch.uint8, device=dev) for N, _ in cfg.levels]
    tws = [torch.empty(max(1, ca.knn_table_workspace_bytes(cfg.B, N, cfg.G)),
                       dtype=torch.uint8, device=dev) for N, _ in cfg.levels]

    def step(s):
        for li in range(L):
            lv = s["lv"][li]
            table = ca.knn_table(lv["coords"], cfg.G, cfg.K, workspace=tws[li])
            ca.knn_sample_fwd(lv["feats"], lv["coords"], s["q"], table, cfg.p)
            ca.knn_sample_bwd(lv["feats"], lv["coords"], s["q"], table, cfg.p, lv["dout"],
                              workspace=wss[li])

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # per-entry-point durations (all levels of one step), HIP events on the
    # launch stream around back-to-back calls
    n_ev = min(args.steps, 100)
    tables = [[ca.knn_table(s["lv"][li]["coords"], cfg.G, cfg.K, workspace=tws[li]) for li in range(L)]
              for s in sets]
    calls = {
        "table": lambda i: [ca.knn_table(sets[i]["lv"][li]["coords"], cfg.G, cfg.K, workspace=tws[li])
                            for li in range(L)],
        "fwd": lambda i: [ca.knn_sample_fwd(sets[i]["lv"][li]["feats"], sets[i]["lv"][li]["coords"],
                                            sets[i]["q"], tables[i][li], cfg.p) for li in range(L)],
        "bwd": lambda i: [ca.knn_sample_bwd(sets[i]["lv"][li]["feats"], sets[i]["lv"][li]["coords"],
                                            sets[i]["q"], tables[i][li], cfg.p,
                                            sets[i]["lv"][li]["dout"], workspace=wss[li])
                          for li in range(L)],
    }
    eager = entry_times(torch, calls, n_ev, len(sets))
    stats, how = pick_timing(calls, None, entry_times_stream(torch, calls, len(sets)))
    dur = {name: st["mean"] for name, st in stats.items()}
    alg = sampler_algorithmic(cfg)
    dom = max(("table", "fwd", "bwd"), key=lambda k: dur[k])
    achieved = alg[dom] / (dur[dom] * 1e-6) / 1e9
    fb_us = dur["fwd"] + dur["bwd"]
    queries = cfg.B * cfg.M
    line = {
        "metric": "KNN-cache point sampler fwd+bwd queries/sec and % of HBM roofline "
                  "(decoder, 4 levels)",
        "value": queries / (ms_per_step * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: B={cfg.B} images x M={cfg.M} queries, G={cfg.G}, K={cfg.K}, "
                        f"levels (N, C) = {list(cfg.levels)}, {cfg.dtype}; step = per level "
                        "table build + forward + backward",
            "B": cfg.B, "M": cfg.M, "G": cfg.G, "K": cfg.K, "p": cfg.p,
            "levels": [list(x) for x in cfg.levels], "seed": cfg.seed,
            "rotating_copies": args.copies,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": {"table": "cluster_attn_knn_table", "fwd": "cluster_attn_knn_sample_fwd",
                       "bwd": "cluster_attn_knn_sample_bwd"}[dom],
            "entry_point_kernels": SAMPLER_ENTRY_KERNELS[dom],
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": measured_traffic(cfg.name, dom, SAMPLER_SOURCES),
            "algorithmic_bytes": alg[dom],
            "avg_us": dur[dom],
        },
        "fwd_bwd": {
            "us": fb_us,
            "queries_per_s": queries / (fb_us * 1e-6),
            "effective_GBps": (alg["fwd"] + alg["bwd"]) / (fb_us * 1e-6) / 1e9,
            "hbm_frac": (alg["fwd"] + alg["bwd"]) / (fb_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        },
        "entry_us": dur,
        "entry_us_stats": stats,
        "entry_timing": how,
        "entry_us_eager": {name: st["mean"] for name, st in eager.items()},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        # about 24576 queries per level (12 images of the decoder workload)
        line["cpu_baseline"] = sampler_cpu_baseline(cfg, case, max(1, min(cfg.B, 24576 // cfg.M)))
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------------------
# Adaptive token merging: --config merge_stages
# ---------------------------------------------------------------------------

def merge_algorithmic(cfg):
    """Compulsory bytes per entry point, summed over the levels."""
    es = 4 if cfg.dtype == "f32" else 2
    B = cfg.B
    out = {"plan": 0, "fwd": 0, "bwd": 0}
    for N, k, C in cfg.levels:
        plan_io = N * 12 + k * 4 + N * 8 + (k + 1) * 4
        lists = N * 4 + (k + 1) * 4
        out["plan"] += B * plan_io
        out["fwd"] += B * (N * C * es + N * 12 + lists + k * C * es + k * 8)
        out["bwd"] += B * (N * C * es + N * 12 + lists + k * C * es + k * 8 + N * C * es + N * 12)
    return out


def merge_cpu_baseline(cfg, case, images: int):
    """The fp64 oracle (plan + forward + backward, all levels) on `images`
    images, single-threaded."""
    from threadpoolctl import threadpool_limits

    import oracle as O

    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for li, (N, k, C) in enumerate(cfg.levels):
            F = case["feats"][li].double().numpy()
            dF = case["dfeat"][li].double().numpy()
            for b in range(images):
                c, s = case["coords"][li][b], case["scores"][li][b]
                anchors = O.merge_anchors(s, k)
                # the per-token scan, or its k-d tree form on large images
                assign = (O.merge_assign if N <= 4096 else O.merge_assign_tree)(c, anchors, cfg.G)
                O.merge_fwd(F[b], c, s, assign, k)
                O.merge_bwd(F[b], c, s, assign, k, dF[b], case["dcoord"][li][b])
        dt = time.perf_counter() - t0
    tokens = images * cfg.levels[0][0]
    return {
        "value": tokens / dt,
        "unit": "tokens/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"{images} of {cfg.B} images ({tokens} first-level tokens, {len(cfg.levels)} levels), "
                  f"fp64 plan+forward+backward, {dt:.1f} s",
    }


def bench_merge(args, torch, ca):
    ca._lib.load()
    args.copies = args.copies or 4
    from gen import make_merge_case

    case = make_merge_case(args.config)
    cfg = case["cfg"]
    dev = "cuda"
    L = len(cfg.levels)
    sets = []
    for r in range(args.copies):
        sets.append([{"coords": torch.from_numpy(case["coords"][li]).to(dev),
                      "scores": torch.from_numpy(case["scores"][li]).to(dev),
                      "feats": case["feats"][li].to(dev), "dfeat": case["dfeat"][li].to(dev),
                      "dcoord": torch.from_numpy(case["dcoord"][li]).to(dev)} for li in range(L)])

    pws = [torch.empty(max(1, ca.merge_plan_workspace_bytes(cfg.B, N, k)), dtype=torch.uint8,
                       device=dev) for N, k, _ in cfg.levels]

    def step(s):
        for li, (N, k, C) in enumerate(cfg.levels):
            lv = s[li]
            _, _, mem, off = ca.merge_plan(lv["coords"], lv["scores"], k, cfg.G, workspace=pws[li])
            ca.merge_fwd(lv["feats"], lv["coords"], lv["scores"], mem, off)
            ca.merge_bwd(lv["feats"], lv["coords"], lv["scores"], mem, off, lv["dfeat"], lv["dcoord"])

    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    n_ev = min(args.steps, 100)
    plans = [[ca.merge_plan(s[li]["coords"], s[li]["scores"], k, cfg.G, workspace=pws[li])
              for li, (N, k, C) in enumerate(cfg.levels)] for s in sets]
    calls = {
        "plan": lambda i: [ca.merge_plan(sets[i][li]["coords"], sets[i][li]["scores"], k, cfg.G,
                                         workspace=pws[li])
                           for li, (N, k, C) in enumerate(cfg.levels)],
        "fwd": lambda i: [ca.merge_fwd(sets[i][li]["feats"], sets[i][li]["coords"], sets[i][li]["scores"],
                                       plans[i][li][2], plans[i][li][3]) for li in range(L)],
        "bwd": lambda i: [ca.merge_bwd(sets[i][li]["feats"], sets[i][li]["coords"], sets[i][li]["scores"],
                                       plans[i][li][2], plans[i][li][3], sets[i][li]["dfeat"],
                                       sets[i][li]["dcoord"]) for li in range(L)],
    }
    eager = entry_times(torch, calls, n_ev, len(sets))
    stats, how = pick_timing(calls, None, entry_times_stream(torch, calls, len(sets)))
    dur = {name: st["mean"] for name, st in stats.items()}
    alg = merge_algorithmic(cfg)
    dom = max(("plan", "fwd", "bwd"), key=lambda k: dur[k])
    achieved = alg[dom] / (dur[dom] * 1e-6) / 1e9
    fb_us = dur["fwd"] + dur["bwd"]
    tokens = cfg.B * cfg.levels[0][0]
    line = {
        "metric": "adaptive token merging plan+fwd+bwd tokens/sec and % of HBM roofline "
                  "(3 stage transitions)",
        "value": tokens / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: B={cfg.B} images, levels (N, k, C) = {list(cfg.levels)}, G={cfg.G}, "
                        f"{cfg.dtype}; step = per level plan + forward + backward",
            "B": cfg.B, "levels": [list(x) for x in cfg.levels], "G": cfg.G, "seed": cfg.seed,
            "rotating_copies": args.copies,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": {"plan": "cluster_attn_merge_plan", "fwd": "cluster_attn_merge_fwd",
                       "bwd": "cluster_attn_merge_bwd"}[dom],
            "entry_point_kernels": MERGE_ENTRY_KERNELS[dom],
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": measured_traffic(cfg.name, dom, MERGE_SOURCES),
            "algorithmic_bytes": alg[dom],
            "avg_us": dur[dom],
        },
        "fwd_bwd": {
            "us": fb_us,
            "effective_GBps": (alg["fwd"] + alg["bwd"]) / (fb_us * 1e-6) / 1e9,
            "hbm_frac": (alg["fwd"] + alg["bwd"]) / (fb_us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
        },
        "entry_us": dur,
        "entry_us_stats": stats,
        "entry_timing": how,
        "entry_us_eager": {name: st["mean"] for name, st in eager.items()},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = merge_cpu_baseline(cfg, case, max(1, min(cfg.B, 65536 // cfg.levels[0][0])))
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
