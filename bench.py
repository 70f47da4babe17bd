#!/usr/bin/env python3
"""Throughput of the QuantWM 2-bit KV-cache hot path on one MI355X.

Default workload: the streaming-insert step. A 100,000-token cache of 40
heads (head_dim 128, 256 centroids, PSAC rank 16, 9 calibration epochs
refreshed every 8 frames) is built once, untimed, with GPU calibration at
every epoch boundary. One step is
  1. quantize_append  -- QSAC assignment, INT2 residual, PSAC coefficients
                         and INT2 Values of one new 1,560-token frame;
  2. attend           -- a 1,560-Query chunk attends to all 101,560 cached
                         tokens (PSAC logit term per epoch).
Before every timed step a write of --flush-mib MiB (default 1024) evicts the
L2 caches and the 256 MB MALL, outside the timed region; each step is timed
with HIP events on the library's stream. The every-8-frames refresh (subspace
from 12,480 historical Queries, 10-iteration centroid build) is timed apart
and reported per refresh and per frame.

Other workloads (--workload): video_chunk (a whole step of calibration,
quantize-append of 7,040 tokens and attention of 880 Queries with their own
K/V; --mode picks QVG and the ablations), wm_layer, long_horizon (attention
over a prebuilt 131,072-token cache; with --nq <= 48 the decode kernel runs,
and up to 64 Queries the launch is priced against HBM, past that against MFMA).

Prints ONE JSON line. `value` = cache token-heads attended per second of
step time (H * N_kv / t_step). `roofline` reports the kernel with the most
time per step against the MI355X peak of the unit that bounds it; its
average launch time comes from HIP events the library records on its own
stream. `cpu_baseline` is the CPU oracle timed on the host's cores on a
stated sample of the same step.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

METRIC = "KV tokens attended/s over 2-bit cache + quantize GB/s; % of HBM roofline"
HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
# VALU: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.32 T lane-instructions/s.
# The QSAC cost loop retires 3 elementary ops (sub, max, min) per channel in
# 2 lane-instructions (v_sub + half a v_max3 + half a v_min3), so its
# arithmetic peak is 1.5 x 39.32 = 58.98 T ops/s.
VALU_LANE_INSTR_PER_S = 256 * 4 * 16 * 2.4e9
QSAC_OPS_PEAK = 1.5 * VALU_LANE_INSTR_PER_S
# The nearest-centroid cost retires its 3 ops per channel (sub, mul, add) as
# 3 lane-instructions.
NEAREST_OPS_PEAK = VALU_LANE_INSTR_PER_S

MODES = {  # objective, PSAC on
    "quantwm": ("qsac", True),
    "qvg": ("nearest", False),
    "qsac": ("qsac", False),
    "nearest-psac": ("nearest", True),
    "postq": ("postq", True),
}

KERNELS = ["quantize", "attend", "merge", "qu", "gram", "eigen", "assign", "update", "other"]
# The sources each kernel class is compiled from: its file(s) and the headers
# every kernel includes (device helpers and the internal constants).
_HEADERS = ("qwm_dev.h", "qwm_internal.h")
KERNEL_SOURCES = {
    "quantize": ("kern_quant.hip",) + _HEADERS, "assign": ("kern_quant.hip",) + _HEADERS,
    "update": ("kern_quant.hip",) + _HEADERS, "other": ("kern_quant.hip",) + _HEADERS,
    # the attention class: the general kernel, the bf16 head_dim-128 kernel and the decode kernel
    "attend": ("kern_attend.hip", "kern_attend_bf16.hip", "kern_decode.hip", "qwm_codes.h") + _HEADERS,
    "merge": ("kern_attend.hip",) + _HEADERS, "qu": ("kern_attend.hip",) + _HEADERS,
    "gram": ("kern_calib.hip",) + _HEADERS, "eigen": ("kern_calib.hip",) + _HEADERS,
    "diag": ("kern_calib.hip",) + _HEADERS,
    "decode": ("kern_decode.hip", "qwm_codes.h") + _HEADERS, "qc": ("kern_decode.hip", "qwm_codes.h") + _HEADERS,
}


def source_hash(kernel: str) -> str:
    """First 16 hex digits of a SHA-256 over the source file(s) of a kernel class."""
    files = KERNEL_SOURCES[kernel]
    h = hashlib.sha256()
    for f in (files,) if isinstance(files, str) else files:
        with open(os.path.join(ROOT, "video_world_model_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, profile: str):
    """HBM bytes per launch of `kernel` from profiles/<kernel>_<profile>_pmc.json
    (two rocprofv3 --pmc runs, scaled by the copy probe), or None when there is
    no such file or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{profile}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        pmc = json.load(f)
    if pmc.get("source_sha256_16") != source_hash(kernel):
        return None
    return pmc.get("hbm_bytes_per_launch")


def bytes_per_token_head(d, g, r):
    return 2 * (d // 4) + 2 * (d // g) * 4 + 1 + 2 * r


def models(w: W.Workload, r: int):
    """Algorithmic work per launch of each kernel class (PSAC rank r)."""
    H, d, g, m = w.heads, w.head_dim, w.group, w.n_centroids
    N, Nq, Ns, M = w.n_kv, w.n_q, w.n_self, w.n_hist
    esz = 2 if w.dtype == "bf16" else 4
    B = bytes_per_token_head(d, g, r)
    return {
        "quantize": dict(ops=H * N * 3 * m * d, bytes=H * N * (2 * d * esz + B)),
        "assign": dict(ops=H * N * 3 * m * d, bytes=H * N * (d * esz + 1)),
        "attend": dict(flops=H * Nq * (N * (4 * d + 2 * r) + Ns * 4 * d),
                       bytes=H * (N * B + Nq * d * esz + Nq * d * 4 + Ns * 2 * d * esz)),
        "gram": dict(flops=2 * H * M * d * d, bytes=H * M * d * esz),
    }


# ----------------------------------------------------------------- CPU oracle

def _oracle_head(args):
    name, head, objective, r = args
    from threadpoolctl import threadpool_limits

    import oracle.qwm_oracle as O
    w = W.workload(name)
    hg = W.HeadGen(w, head)
    keys, vals = hg.cache_keys(), hg.cache_values()
    qh, q = hg.hist_queries(), hg.current_queries()
    ks = vs = None
    if w.n_self:
        ks, vs = hg.self_keys(), hg.self_values()
    with threadpool_limits(1):
        t0 = time.perf_counter()
        if objective == "qsac" or r > 0:
            S = O.sensitivity(qh, w.group)
        else:
            S = np.zeros(w.head_dim // w.group, np.float32)
        U = O.subspace(qh, r)
        C = O.build_centroids(keys, S, w.n_centroids, w.group, w.kmeans_iters, w.dtype, objective=objective)
        hc = O.HeadCache(w.group, w.dtype, objective)
        hc.add_epoch(C, S, U)
        hc.append(keys, vals)
        O.attend(q, hc, ks, vs, mask=w.self_mask)
        return time.perf_counter() - t0


def cpu_baseline(w: W.Workload, n_heads: int, objective: str, r: int):
    """The oracle's full step on `n_heads` heads, one forked worker per head
    (run before the GPU is initialized), scaled to cache tokens/s."""
    import multiprocessing as mp
    n_heads = min(n_heads, w.heads)
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(n_heads) as pool:
        times = pool.map(_oracle_head, [(w.name, h, objective, r) for h in range(n_heads)])
    wall = time.perf_counter() - t0
    busy = max(times)
    return {
        "value": n_heads * w.n_kv / busy,
        "unit": "KV tokens/s",
        "cores": n_heads,
        "kind": "oracle",
        "sample": (f"one full {w.name} step ({objective} rule, rank {r}: subspace, {w.kmeans_iters}-iteration "
                   f"centroid build, quantize of "
                   f"{w.n_kv} tokens, attention of {w.n_q} Queries) on {n_heads} of {w.heads} heads, one forked "
                   f"process per head, BLAS 1 thread; slowest head {busy:.2f} s, pool wall {wall:.2f} s"),
        "host_cpus": len(os.sched_getaffinity(0)),
        "numpy": np.__version__,
    }


def _oracle_stream_epoch(args):
    """One epoch of one head of the streaming cache, built by the oracle
    (untimed set-up): calibration from the epoch's historical Queries and
    first frame, then its tokens of the 100,000-token base cache."""
    name, head, e = args
    from threadpoolctl import threadpool_limits

    import oracle.qwm_oracle as O
    w = W.workload(name)
    hg = W.HeadGen(w, head)
    base = w.n_kv - w.n_append
    s0, s1 = w.epoch_start(e), min(w.epoch_end(e), base)
    a0, a1 = w.centroid_keys_range(e)
    with threadpool_limits(1):
        qh = hg.hist_queries(e)
        S = O.sensitivity(qh, w.group)
        U = O.subspace(qh, w.rank)
        C = O.build_centroids(hg.keys(a0, a1), S, w.n_centroids, w.group, w.kmeans_iters, w.dtype)
        hc = O.HeadCache(w.group, w.dtype)
        hc.add_epoch(C, S, U)
        hc.append(hg.keys(s0, s1), hg.values(s0, s1))
    return head, e, (C, S, U), hc.records[0][1]


# Oracle head caches of the streaming base cache, filled before the step
# workers are forked (they inherit them).
_STREAM_CACHES = {}


def _oracle_stream_step(args):
    """The timed oracle work of one (head, slice) of a streaming step: the
    append of the slice's share of the new frame (HeadCache.append:
    quantize-on-insert of those tokens), then the attention of the slice's
    share of the Query chunk over the whole 101,560-token cache. Between the
    two, untimed, the frame is appended whole in token order so that the
    attention sees the GPU step's cache."""
    name, head, j, nsl, nq = args
    from threadpoolctl import threadpool_limits

    import oracle.qwm_oracle as O
    w = W.workload(name)
    hg = W.HeadGen(w, head)
    hc = _STREAM_CACHES[head]
    base = w.n_kv - w.n_append
    cuts = [base + (w.n_append * i) // nsl for i in range(nsl + 1)]
    qcuts = [(nq * i) // nsl for i in range(nsl + 1)]
    q = hg.queries(W.Q_CURRENT, nq)[qcuts[j]:qcuts[j + 1]]
    tq = 0.0
    with threadpool_limits(1):
        if w.n_append:
            k = [hg.keys(cuts[i], cuts[i + 1]) for i in range(nsl)]
            v = [hg.values(cuts[i], cuts[i + 1]) for i in range(nsl)]
            n_rec = len(hc.records)
            t0 = time.perf_counter()
            hc.append(k[j], v[j])
            tq = time.perf_counter() - t0
            del hc.records[n_rec:]
            hc.length = base
            for i in range(nsl):
                hc.append(k[i], v[i])
        t0 = time.perf_counter()
        O.attend(q, hc)
        ta = time.perf_counter() - t0
    return tq, ta


def cpu_baseline_streaming(w: W.Workload, n_heads: int, cores: int, nq: int = 0):
    """The oracle's step of a multi-epoch workload (streaming: append one
    frame and attend; long_horizon: attend only) on `n_heads` heads over
    `cores` forked processes (one per core, run before the GPU is
    initialized): each head's frame and Query chunk are cut into
    cores / n_heads slices, one process per (head, slice). Each head's base
    cache is built first by the oracle, untimed, one process per (head,
    epoch)."""
    nq = nq or w.n_q
    import multiprocessing as mp

    import oracle.qwm_oracle as O
    n_heads = max(1, min(n_heads, w.heads))
    nsl = max(1, cores // n_heads)
    ctx = mp.get_context("fork")
    base = w.n_kv - w.n_append
    n_ep = -(-base // w.epoch_tokens)
    t0 = time.perf_counter()
    with ctx.Pool(cores) as pool:
        parts = pool.map(_oracle_stream_epoch, [(w.name, h, e) for h in range(n_heads) for e in range(n_ep)])
    t_setup = time.perf_counter() - t0
    for h in range(n_heads):
        # the oracle's HeadCache, filled with the per-epoch results in order
        # (what add_epoch and append would have produced one after the other)
        hc = O.HeadCache(w.group, w.dtype)
        for hh, e, cal, rec in sorted(parts, key=lambda x: (x[0], x[1])):
            if hh != h:
                continue
            hc.epochs.append((hc.length, *cal))
            rec["epoch"] = np.full(len(rec["ids"]), e, np.int64)
            hc.records.append((hc.length, rec))
            hc.length += len(rec["ids"])
        assert hc.length == base
        _STREAM_CACHES[h] = hc
    del parts
    t0 = time.perf_counter()
    with ctx.Pool(n_heads * nsl) as pool:
        res = pool.map(_oracle_stream_step, [(w.name, h, j, nsl, nq) for h in range(n_heads) for j in range(nsl)])
    wall = time.perf_counter() - t0
    _STREAM_CACHES.clear()
    per = [tq + ta for tq, ta in res]
    busy = max(per)
    return {
        "value": n_heads * w.n_kv / busy,
        "unit": "KV tokens/s",
        "cores": n_heads * nsl,
        "kind": "oracle",
        "sample": (f"the {w.name} step ("
                   + (f"quantize-append of the {w.n_append}-token frame, " if w.n_append else "")
                   + f"attention of {nq} Queries over {w.n_kv} tokens) on {n_heads} of {w.heads} heads; each head's "
                   f"work cut into {nsl} slices, one forked process per (head, slice), BLAS 1 thread; "
                   f"value = {n_heads} heads x {w.n_kv} tokens / slowest process ({busy:.2f} s: append "
                   f"{max(r[0] for r in res):.2f} s + attention {max(r[1] for r in res):.2f} s at most); "
                   f"pool wall {wall:.2f} s; the oracle built the {base}-token base caches first "
                   f"({t_setup:.1f} s, untimed)"),
        "host_cpus": len(os.sched_getaffinity(0)),
        "numpy": np.__version__,
    }


# ----------------------------------------------------------------- GPU

def _build_epochs(cache, w, gens, dev, n_tokens):
    """Cache of the first n_tokens stream tokens, epoch by epoch, calibrated on
    the GPU from each epoch's historical Queries and first frame."""
    import torch
    for e in range(w.n_epochs):
        s0, s1 = w.epoch_start(e), min(w.epoch_end(e), n_tokens)
        if s1 <= s0:
            break
        a0, a1 = w.centroid_keys_range(e)
        cache.build_subspace(dev([g.hist_queries(e) for g in gens]))
        cache.build_centroids(dev([g.keys(a0, a1) for g in gens]), w.kmeans_iters)
        cache.quantize_append(dev([g.keys(s0, s1) for g in gens]), dev([g.values(s0, s1) for g in gens]))
        torch.cuda.synchronize()


def _bf16_dev(x_list):
    import torch
    x = np.ascontiguousarray(np.stack(x_list))
    return torch.from_numpy(W.bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16)


def _kernel_times(cache, steps):
    kern = {}
    for k in KERNELS:
        ms, n = cache.profile_read(k)
        if n:
            kern[k] = dict(ms_per_step=ms / steps, launches_per_step=n / steps, avg_launch_ms=ms / n)
    return kern


def _copy_probe(args):
    """One plain elementwise copy (torch.neg) of --copy-probe-mib MiB: a kernel
    of known traffic (read and write that many bytes) whose FETCH_SIZE and
    WRITE_SIZE, in the same profiled run, calibrate the counters."""
    import torch
    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib * (1 << 18), dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst


def _event_timer(stream, flush):
    """timed(fn, n): mean milliseconds of n runs of fn, each between two HIP
    events on `stream`; before each run (outside its events) the flush
    buffer is rewritten, so the L2 caches and the MALL hold none of the
    step's data."""
    import torch

    def timed(fn, n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            for i, (e0, e1) in enumerate(evs):
                if flush is not None:
                    flush.fill_(i & 0xFF)
                e0.record(stream)
                fn()
                e1.record(stream)
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in evs) / n

    def profiled(cache, fn, n):
        """n runs of fn with the library's event timing on, flushed the same way."""
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            cache.profile_enable(True)
            for i in range(n):
                if flush is not None:
                    flush.fill_(i & 0xFF)
                fn()
        torch.cuda.synchronize()
        kern = _kernel_times(cache, n)
        cache.profile_enable(False)
        return kern

    return timed, profiled


def bench_streaming(args, w):
    """The streaming-insert step on the 100,000-token cache (built once,
    untimed, with GPU calibration at every epoch boundary): quantize-append
    one 1,560-token frame, then attention of a 1,560-Query chunk over all
    101,560 tokens. The calibration refresh (every 8 frames: subspace from
    the last 8 frames' 12,480 Queries, 10-iteration centroid build on the
    refresh frame) is timed on its own and reported per refresh and per
    frame."""
    cpu = None
    if args.cpu_heads > 0:
        cpu = cpu_baseline_streaming(w, args.cpu_heads, args.cpu_cores or len(os.sched_getaffinity(0)))
    import torch
    from video_world_model_amd import Cache
    from video_world_model_amd import qwm as Q
    src_hash = Q.check_build()
    torch.cuda.set_device(0)
    _copy_probe(args)
    gens = [W.HeadGen(w, h) for h in range(w.heads)]
    base = w.n_kv - w.n_append
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        cache = Cache(w.heads, w.head_dim, w.n_centroids, w.rank, w.n_kv, dtype=torch.bfloat16,
                      max_epochs=w.n_epochs, max_query_tokens=w.n_q, max_build_tokens=w.frame_tokens)
        _build_epochs(cache, w, gens, _bf16_dev, base)
        kf = _bf16_dev([g.keys(base, w.n_kv) for g in gens])
        vf = _bf16_dev([g.values(base, w.n_kv) for g in gens])
        q = _bf16_dev([g.current_queries() for g in gens])
        e_last = w.n_epochs - 1
        qh = _bf16_dev([g.hist_queries(e_last) for g in gens])
        a0, a1 = w.centroid_keys_range(e_last)
        kref = _bf16_dev([g.keys(a0, a1) for g in gens])
        out = torch.empty((w.heads, w.n_q, w.head_dim), dtype=torch.float32, device="cuda")
        flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device="cuda") if args.flush_mib > 0 else None
    torch.cuda.synchronize()
    timed, profiled = _event_timer(stream, flush)

    def step():
        cache.truncate(base)
        cache.quantize_append(kf, vf)
        cache.attend(q, out=out)

    refresh_at = w.epoch_start(e_last)  # the last refresh point: an epoch boundary

    def refresh():
        # rewind to the boundary (the epoch there keeps no token and is replaced)
        cache.truncate(refresh_at)
        cache.build_subspace(qh)
        cache.build_centroids(kref, w.kmeans_iters)

    n_ref = max(1, args.steps // 4)
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            refresh()
    ms_refresh = timed(refresh, n_ref)
    kref_t = profiled(cache, refresh, n_ref)
    # back to the 100,000-token cache: the last epoch rebuilt the same way
    with torch.cuda.stream(stream):
        cache.truncate(refresh_at)
        cache.quantize_append(_bf16_dev([g.keys(refresh_at, base) for g in gens]),
                              _bf16_dev([g.values(refresh_at, base) for g in gens]))
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    # timed region: exactly `steps` steps, each flushed before its events
    ms_step = timed(step, args.steps)
    kern = profiled(cache, step, args.steps)
    assert cache.length() == w.n_kv and cache.epochs() == w.n_epochs
    rb, tb = cache.storage_bytes()

    B = bytes_per_token_head(w.head_dim, w.group, w.rank)
    tq = kern["quantize"]["avg_launch_ms"] * 1e-3
    ta = sum(kern[k]["ms_per_step"] for k in ("qu", "attend", "merge") if k in kern) * 1e-3
    ta_k = kern["attend"]["avg_launch_ms"] * 1e-3
    q_bytes = w.heads * w.n_append * (2 * w.head_dim * 2 + B)
    q_ops = w.heads * w.n_append * 3 * w.n_centroids * w.head_dim
    a_flops = w.heads * w.n_q * w.n_kv * (4 * w.head_dim + 2 * w.rank)
    a_bytes = w.heads * (w.n_kv * B + w.n_q * w.head_dim * 2 + w.n_q * w.head_dim * 4)
    dom = max(kern, key=lambda k: kern[k]["ms_per_step"])
    if dom == "attend":
        achieved = a_flops / ta_k / 1e12
        roof = dict(bound="mfma", achieved=achieved, peak=MFMA_F16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=achieved / MFMA_F16_PEAK_TFLOPS, kernel="attend",
                    traffic=measured_traffic("attend", w.name),
                    work=f"{w.heads} heads x {w.n_q} Queries x {w.n_kv} tokens x (4*{w.head_dim} + 2*{w.rank}) "
                         f"flops = {a_flops:.4g} per launch")
    else:
        achieved = q_ops / tq / 1e12
        roof = dict(bound="alu", achieved=achieved, peak=QSAC_OPS_PEAK / 1e12, unit="Top/s",
                    frac=achieved * 1e12 / QSAC_OPS_PEAK, kernel=dom, traffic=measured_traffic(dom, w.name))
    rec = {
        "metric": METRIC,
        "value": w.heads * w.n_kv / (ms_step * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32-valu+f16-mfma",
        "data": "synthetic",
        "config": {"workload": w.name, "step": "quantize-append 1 frame + attend 1 chunk", "heads": w.heads,
                   "head_dim": w.head_dim, "n_centroids": w.n_centroids, "rank": w.rank, "n_kv": w.n_kv,
                   "n_append": w.n_append, "n_q": w.n_q, "epochs": w.n_epochs, "input_dtype": w.dtype,
                   "flush_mib": args.flush_mib},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kern,
        "phases": {
            "quantize": dict(ms=tq * 1e3, GBps=q_bytes / tq / 1e9, hbm_frac=q_bytes / tq / 1e9 / HBM_PEAK_GBPS,
                             alu_frac=q_ops / tq / QSAC_OPS_PEAK),
            "attend": dict(ms=ta * 1e3, kv_tokens_per_s=w.heads * w.n_kv / ta,
                           mfma_frac=a_flops / ta_k / 1e12 / MFMA_F16_PEAK_TFLOPS,
                           hbm_frac=a_bytes / ta_k / 1e9 / HBM_PEAK_GBPS),
            "refresh": dict(ms=ms_refresh, ms_per_frame=ms_refresh / (w.epoch_tokens // w.frame_tokens),
                            kernels=kref_t),
        },
        "storage": dict(bytes_per_token_head=B, record_bytes=rb, table_bytes=tb,
                        compression_vs_bf16=w.heads * w.n_kv * 4 * w.head_dim / (rb + tb)),
        "lib_source_hash": src_hash,
    }
    print(json.dumps(rec), flush=True)


def bench_long_horizon(args, w):
    """Attention over the long-horizon cache (built once per epoch from the
    epoch's historical Queries and first frame, untimed): a step is one
    qwm_attend of n_q Queries per head, no self segment, flushed before its
    events like the streaming step."""
    nq = args.nq or w.n_q
    cpu = None
    if args.cpu_heads > 0:
        cpu = cpu_baseline_streaming(w, args.cpu_heads, args.cpu_cores or len(os.sched_getaffinity(0)), nq)
    import torch
    from video_world_model_amd import Cache
    from video_world_model_amd import qwm as Q
    src_hash = Q.check_build()
    torch.cuda.set_device(0)
    _copy_probe(args)
    gens = [W.HeadGen(w, h) for h in range(w.heads)]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        cache = Cache(w.heads, w.head_dim, w.n_centroids, w.rank, w.n_kv, dtype=torch.bfloat16,
                      max_epochs=w.n_epochs, max_query_tokens=max(nq, 16), max_build_tokens=w.frame_tokens)
        _build_epochs(cache, w, gens, _bf16_dev, w.n_kv)
        q = _bf16_dev([g.queries(W.Q_CURRENT, nq) for g in gens])
        out = torch.empty((w.heads, nq, w.head_dim), dtype=torch.float32, device="cuda")
        flush = torch.empty(args.flush_mib << 20, dtype=torch.uint8, device="cuda") if args.flush_mib > 0 else None
        for _ in range(args.warmup):
            cache.attend(q, out=out)
    torch.cuda.synchronize()
    timed, profiled = _event_timer(stream, flush)

    def step():
        cache.attend(q, out=out)

    ms_step = timed(step, args.steps)
    kern = profiled(cache, step, args.steps)
    rb, tb = cache.storage_bytes()
    B = bytes_per_token_head(w.head_dim, w.group, w.rank)
    attend_bytes = w.heads * (w.n_kv * B + nq * w.head_dim * 2 + nq * w.head_dim * 4)
    attend_flops = w.heads * nq * w.n_kv * (4 * w.head_dim + 2 * w.rank)
    ta = kern["attend"]["avg_launch_ms"] * 1e-3
    # the packed cache's bytes bound the launch up to about 79 Queries per head
    # (2.5 PFLOP/s over 8 TB/s against 4 * 128 flops per Query and ~130 B per
    # token); 64 is the round cut used here
    hbm_bound = nq <= 64
    if hbm_bound:
        achieved = attend_bytes / ta / 1e9
        roof = dict(bound="hbm", achieved=achieved, peak=HBM_PEAK_GBPS, unit="GB/s", frac=achieved / HBM_PEAK_GBPS,
                    work=f"{w.heads} heads x ({w.n_kv} tokens x {B} B + {nq} Queries x {w.head_dim} x (2 + 4) B) "
                         f"= {attend_bytes:.4g} B per launch")
    else:
        achieved = attend_flops / ta / 1e12
        roof = dict(bound="mfma", achieved=achieved, peak=MFMA_F16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=achieved / MFMA_F16_PEAK_TFLOPS,
                    work=f"{w.heads} heads x {nq} Queries x {w.n_kv} tokens x (4*{w.head_dim} + 2*{w.rank}) flops "
                         f"= {attend_flops:.4g} per launch")
    # the library's dispatch: bf16 head_dim-128 calls of at most 48 Queries
    # and no self segment run the decode kernel
    roof["kernel"] = "decode" if nq <= 48 else "attend"
    roof["traffic"] = measured_traffic(roof["kernel"], f"{w.name}_nq{nq}" if args.nq else w.name)
    rec = {
        "metric": METRIC,
        "value": w.heads * w.n_kv / (ms_step * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32-valu+f16-mfma",
        "data": "synthetic",
        "config": {"workload": w.name, "step": "attend", "heads": w.heads, "head_dim": w.head_dim,
                   "n_centroids": w.n_centroids, "rank": w.rank, "n_kv": w.n_kv, "n_q": nq, "epochs": w.n_epochs,
                   "input_dtype": w.dtype, "flush_mib": args.flush_mib},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kern,
        "phases": {"attend": dict(GBps=attend_bytes / ta / 1e9, hbm_frac=attend_bytes / ta / 1e9 / HBM_PEAK_GBPS,
                                  mfma_frac=attend_flops / ta / 1e12 / MFMA_F16_PEAK_TFLOPS,
                                  ms=ta * 1e3, pair_per_s=w.heads * nq * w.n_kv / (ms_step * 1e-3))},
        "storage": dict(bytes_per_token_head=B, record_bytes=rb, table_bytes=tb,
                        compression_vs_bf16=w.heads * w.n_kv * 4 * w.head_dim / (rb + tb)),
        "lib_source_hash": src_hash,
    }
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="streaming",
                    choices=["tiny", "video_chunk", "wm_layer", "streaming", "long_horizon"],
                    help="streaming: the 100,000-token cache is built once (untimed); a step appends one "
                         "1,560-token frame and attends with 1,560 Queries; the every-8-frames refresh is timed "
                         "apart. long_horizon: the 131,072-token, 11-epoch cache is built once (untimed) and a "
                         "step is one attention of --nq Queries per head over it (decode kernel when --nq <= 48)")
    ap.add_argument("--nq", type=int, default=0, help="Queries per head for long_horizon (default: the workload's)")
    ap.add_argument("--mode", default="quantwm", choices=sorted(MODES))
    ap.add_argument("--graph", type=int, default=0,
                    help="1: capture one step in a HIP graph (through torch.cuda.graph) and time its replays; "
                         "0: time eager calls")
    ap.add_argument("--cpu-heads", type=int, default=4,
                    help="heads in the oracle's timed sample of the streaming, long_horizon and wm_layer steps "
                         "(tiny and video_chunk take one head per core); 0: skip the oracle")
    ap.add_argument("--cpu-cores", type=int, default=0,
                    help="processes of the oracle sample (default: one per available core)")
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="MiB written before every timed step, outside its events, to evict the L2 caches and "
                         "the 256 MB MALL (streaming and long_horizon; 0: no flush)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one plain elementwise copy (torch.neg) over this many MiB first, as a known-size "
                         "reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this path uses no cross-GPU work); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    w = W.workload(args.workload)
    if w.name == "long_horizon":
        return bench_long_horizon(args, w)
    if w.name == "streaming":
        return bench_streaming(args, w)
    objective, psac = MODES[args.mode]
    r = w.rank if psac else 0
    needs_queries = psac or objective == "qsac"  # QVG uses no historical Queries
    cpu = None
    if args.cpu_heads > 0:
        # the small workloads: one head per host core (all 12 of video_chunk
        # on a 16-core host); wm_layer's oracle step takes about a minute per
        # head, so it keeps --cpu-heads
        cores = args.cpu_cores or len(os.sched_getaffinity(0))
        n_cpu = min(w.heads, cores) if w.name in ("tiny", "video_chunk") else args.cpu_heads
        cpu = cpu_baseline(w, n_cpu, objective, r)

    import torch
    from video_world_model_amd import Cache
    from video_world_model_amd import qwm as Q

    src_hash = Q.check_build()
    torch.cuda.set_device(0)
    _copy_probe(args)
    gens = [W.HeadGen(w, h) for h in range(w.heads)]

    def dev(arrs):
        x = np.ascontiguousarray(np.stack(arrs))
        if w.dtype == "bf16":
            return torch.from_numpy(W.bf16_bits(x).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(x).cuda()

    keys = dev([g.cache_keys() for g in gens])
    vals = dev([g.cache_values() for g in gens])
    qh = dev([g.hist_queries() for g in gens])
    q = dev([g.current_queries() for g in gens])
    ks = vs = None
    if w.n_self:
        ks = dev([g.self_keys() for g in gens])
        vs = dev([g.self_values() for g in gens])
    # the library works on the stream current at create: a stream of our own,
    # which is also the one a graph is captured on
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        cache = Cache(w.heads, w.head_dim, w.n_centroids, r, w.n_kv,
                      dtype=torch.bfloat16 if w.dtype == "bf16" else torch.float32,
                      max_query_tokens=w.n_q, max_build_tokens=w.n_kv, objective=objective)
        out = torch.empty((w.heads, w.n_q, w.head_dim), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def step():
        cache.truncate(0)
        if needs_queries:
            cache.build_subspace(qh)
        cache.build_centroids(keys, w.kmeans_iters)
        cache.quantize_append(keys, vals)
        cache.attend(q, ks, vs, mask=w.self_mask, out=out)

    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            step()
        torch.cuda.synchronize()
        graph.replay()  # one untimed replay
        torch.cuda.synchronize()

    # timed region: K steps, nothing else on the stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    with torch.cuda.stream(stream):
        for _ in range(args.steps):
            if graph is not None:
                graph.replay()
            else:
                step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / args.steps

    # per-kernel times: the same number of eager steps with the library's
    # HIP events around every launch (outside the timed region)
    with torch.cuda.stream(stream):
        cache.profile_enable(True)
        for _ in range(args.steps):
            step()
    torch.cuda.synchronize()
    kern = {}
    for k in KERNELS:
        ms, n = cache.profile_read(k)
        if n:
            kern[k] = dict(ms_per_step=ms / args.steps, launches_per_step=n / args.steps, avg_launch_ms=ms / n)
            if k in ("quantize", "assign"):
                # channel evaluations the launches made (the pruned k-means
                # pass counts its own), 3 elementary ops each
                kern[k]["ops_per_launch"] = 3.0 * cache.profile_work(k) / n
    cache.profile_enable(False)
    # the article's "Table 1" diagnostic, outside the timed region
    with torch.cuda.stream(stream):
        top_cache = cache.attend_top1(q)
        top_full = cache.attend_top1(q, keys)
    torch.cuda.synchronize()
    top1_rate = float((top_cache != top_full).float().mean().item())

    ops_peak = QSAC_OPS_PEAK if objective in ("qsac", "postq") else NEAREST_OPS_PEAK
    mdl = models(w, r)
    dom = max(kern, key=lambda k: kern[k]["ms_per_step"])
    avg_s = kern[dom]["avg_launch_ms"] * 1e-3
    if dom in ("quantize", "assign") and objective == "postq":
        # the 3 m d op count describes the range and distance rules only
        roof = dict(bound="alu", achieved=None, peak=None, unit=None, frac=None)
    elif dom in ("quantize", "assign"):
        ops = kern[dom]["ops_per_launch"]
        achieved = ops / avg_s / 1e12
        roof = dict(bound="alu", achieved=achieved, peak=ops_peak / 1e12, unit="Top/s",
                    frac=achieved * 1e12 / ops_peak,
                    work=f"{ops:.4g} ops per launch: 3 per channel evaluation counted by the library "
                         f"(a full pass: {w.heads} heads x {w.n_kv} tokens x {w.n_centroids} centroids x "
                         f"{w.head_dim} channels = {mdl[dom]['ops'] / 3:.4g} evaluations)")
    elif dom == "attend":
        achieved = mdl[dom]["flops"] / avg_s / 1e12
        roof = dict(bound="mfma", achieved=achieved, peak=MFMA_F16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=achieved / MFMA_F16_PEAK_TFLOPS)
    else:
        roof = dict(bound="alu", achieved=None, peak=None, unit=None, frac=None)
    roof["kernel"] = dom
    suffix = "" if args.mode == "quantwm" else f"_{args.mode}"
    roof["traffic"] = measured_traffic(dom, f"{w.name}{suffix}")

    extras = {}
    if "quantize" in kern:
        t = kern["quantize"]["avg_launch_ms"] * 1e-3
        gbps = mdl["quantize"]["bytes"] / t / 1e9
        extras["quantize"] = dict(GBps=gbps, hbm_frac=gbps / HBM_PEAK_GBPS,
                                  alu_frac=mdl["quantize"]["ops"] / t / ops_peak, ms=t * 1e3)
    if "attend" in kern:
        t = sum(kern[k]["ms_per_step"] for k in ("qu", "attend", "merge") if k in kern) * 1e-3
        ta = kern["attend"]["avg_launch_ms"] * 1e-3
        extras["attend"] = dict(kv_tokens_per_s=w.heads * w.n_kv / t, ms=t * 1e3,
                                pair_per_s=w.heads * w.n_q * (w.n_kv + w.n_self) / t,
                                mfma_frac=mdl["attend"]["flops"] / ta / 1e12 / MFMA_F16_PEAK_TFLOPS,
                                hbm_frac=mdl["attend"]["bytes"] / ta / 1e9 / HBM_PEAK_GBPS)
    extras["calibration_ms"] = sum(kern[k]["ms_per_step"] for k in ("gram", "eigen", "assign", "update", "other")
                                   if k in kern)

    rec = {
        "metric": METRIC,
        "value": w.heads * w.n_kv / (ms_step * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32-valu+f16-mfma",
        "data": "synthetic",
        "config": {"workload": w.name, "mode": args.mode, "hip_graph": bool(args.graph), "objective": objective, "heads": w.heads,
                   "head_dim": w.head_dim, "group": w.group,
                   "n_centroids": w.n_centroids, "rank": r, "n_kv": w.n_kv, "n_q": w.n_q,
                   "n_self": w.n_self, "n_hist": w.n_hist, "kmeans_iters": w.kmeans_iters,
                   "input_dtype": w.dtype, "query_alpha": W.QUERY_ALPHA},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kern,
        "phases": extras,
        "diagnostics": {"top1_change_rate": top1_rate},
        "storage": dict(zip(("record_bytes", "table_bytes"), cache.storage_bytes()),
                        compression_vs_bf16=cache.compression_ratio()),
        "lib_source_hash": src_hash,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
