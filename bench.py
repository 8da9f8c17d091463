#!/usr/bin/env python3
"""Benchmark of one MLA decode step on one MI355X.

A step is one whole mla_decode call (query absorption, split attention over
the paged latent cache, log-sum-exp merge, W_UV up-projection) for a batch of
B sequences: it produces one new token per sequence, so tokens/s = B / step.

Inputs are seeded and synthetic (mla_inputs) and resident in HBM before the
timed region.  Several copies of the cache pool are rotated from step to step
so that the steps together touch more than 2x the 256 MB Infinity Cache and
the latent-cache reads come from HBM.

The latent-cache writer (one new token per sequence appended to the paged
cache, mla_cache_write) is measured on its own under `extra`: a HIP graph of
64 calls, each on its own copy of the projection weights (over 512 MB, so they
are read from HBM), is replayed and timed with events; reported are the time
per call and its algorithmic bytes (weights, hidden states, the rows written)
per second against the 8 TB/s peak.

The DSA sparse decode step (lightning indexer, top-k, decode over the
selected tokens; mla_dsa_decode) is measured the same way under `extra` on
its own workloads, with each stage also timed alone.

The step is timed over K plain mla_decode calls, and again over the same K
calls captured into one HIP graph and replayed (`ms_per_step_graph`; the
replay's output is checked bit for bit against the eager step).  The attention
kernel is then timed alone over K more steps with HIP events recorded on its
stream around its launch (mla_decode_timed); `roofline.achieved` is the
algorithmic latent-cache bytes of one launch over that average duration.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix-core peak
FP8_PEAK_TFLOPS = 5000.0    # dense fp8 matrix-core peak
METRIC = "MLA decode tokens/s + latent-cache HBM GB/s (% of peak), DSV3 shape @32K ctx"
CSRC = os.path.join(ROOT, "head_latent_attention_10_amd", "csrc")


def attn_source(workload: str) -> str:
    """The source file of the attention kernel that serves `workload`: the fp8
    kernel's for an fp8 cache, the bf16 matrix-core kernel's otherwise."""
    from mla_inputs import CONFIGS
    cfg = CONFIGS.get(workload)
    fp8 = cfg is not None and cfg.cache_dtype == "e4m3"
    return os.path.join(CSRC, "mla_attend_fp8.hip" if fp8 else "mla_attend_mfma.hip")


def attn_source_hash(workload: str) -> str:
    with open(attn_source(workload), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_counters(workload: str):
    """The committed rocprofv3 counter summary of the attention kernel on
    `workload` (profiles/attend_<workload>_counters.json), if it was taken on
    the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"attend_{workload}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != attn_source_hash(workload):
        return None
    return rec


def measured_traffic(workload: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"attend_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_sha256_16") != attn_source_hash(workload):
        return None
    return rec.get("hbm_bytes_per_launch")


def attention_roof(r) -> dict:
    """The attention kernel's own bound for a measured workload: the larger of
    its HBM time (the cache bytes at 8 TB/s) and its matrix-core time.  Per
    cached token and head the bf16 kernel multiplies 2 (d_c + d_r) score and
    2 d_c value flops at the bf16 rate; the fp8 kernel runs the latent scores
    on two E4M3 query terms at the fp8 rate (2 x 2 d_c) and the rope scores and
    the values (widened to bf16) at the bf16 rate."""
    cfg = r["cfg"]
    th = r["total_tokens"] * cfg.heads
    if cfg.cache_dtype == "e4m3":
        mfma_s = th * (2 * cfg.d_rope + 2 * cfg.d_latent) / (BF16_PEAK_TFLOPS * 1e12) + \
                 th * (2 * 2 * cfg.d_latent) / (FP8_PEAK_TFLOPS * 1e12)
    else:
        mfma_s = th * (2 * (cfg.d_latent + cfg.d_rope) + 2 * cfg.d_latent) / (BF16_PEAK_TFLOPS * 1e12)
    hbm_s = r["cache_bytes"] / (HBM_PEAK_GBPS * 1e9)
    roof_us = max(hbm_s, mfma_s) * 1e6
    return {"attn_roof_us": round(roof_us, 1), "attn_roof_bound": "hbm" if hbm_s >= mfma_s else "mfma",
            "attn_hbm_us": round(hbm_s * 1e6, 1), "attn_mfma_floor_us": round(mfma_s * 1e6, 1),
            "attn_frac_of_roof": round(roof_us / (r["attn_ms"] * 1e3), 4)}


def measure(workload: str, steps: int, warmup: int, num_splits: int = 0):
    import torch

    from head_latent_attention_10_amd import _lib
    from head_latent_attention_10_amd.device import Decoder, DeviceInputs
    from mla_inputs import CONFIGS, generate

    cfg = CONFIGS[workload]
    t0 = time.time()
    inp = generate(cfg)
    dev = DeviceInputs(inp)
    dec = Decoder(dev, num_splits=num_splits)
    pool_bytes = dev.c_kv.numel() * dev.c_kv.element_size() + dev.k_rope.numel() * dev.k_rope.element_size()
    copies = max(2, math.ceil(768e6 / pool_bytes))
    c_copies = [dev.c_kv] + [dev.c_kv.clone() for _ in range(copies - 1)]
    r_copies = [dev.k_rope] + [dev.k_rope.clone() for _ in range(copies - 1)]
    s_copies = [dev.c_kv_scale] * copies
    if dev.c_kv_scale is not None:
        s_copies = [dev.c_kv_scale] + [dev.c_kv_scale.clone() for _ in range(copies - 1)]
    torch.cuda.synchronize()
    print(f"[bench] {workload}: inputs ready in {time.time() - t0:.1f}s, "
          f"{copies} cache copies of {pool_bytes / 1e6:.0f} MB", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream()
    p = dec.p

    def step(k, evb=None, eva=None, on=None):
        i = k % copies
        if evb is None:
            _lib.mla_decode(p, dev.q, c_copies[i], s_copies[i], r_copies[i], dev.block_table,
                            dev.seq_lens, dev.W_UK, dev.W_UV, dec.out, dec.workspace, dec.ws_bytes,
                            stream if on is None else on)
        else:
            _lib.mla_decode_timed(p, dev.q, c_copies[i], s_copies[i], r_copies[i], dev.block_table,
                                  dev.seq_lens, dev.W_UK, dev.W_UV, dec.out, dec.workspace,
                                  dec.ws_bytes, stream, evb, eva)

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    # the step: plain mla_decode calls between two events
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for k in range(steps):
        step(warmup + k)
    stop.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(stop)
    want = dec.out.clone()
    # The same K steps captured once into a HIP graph (kernel launches only:
    # the step allocates nothing and sets no memory) and replayed, as a
    # serving loop may run them.  One untimed replay first (the graph's
    # upload), then the timed one; every copy of the cache holds the same
    # values, so the output must equal the eager step's bit for bit.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for k in range(steps):
            step(warmup + k, on=cap)
    graph.replay()
    torch.cuda.synchronize()
    start.record(stream)
    graph.replay()
    stop.record(stream)
    torch.cuda.synchronize()
    graph_ms = start.elapsed_time(stop)
    if not torch.equal(dec.out.view(torch.uint8), want.view(torch.uint8)):
        raise RuntimeError(f"{workload}: graph replay of the decode step differs from the eager step")
    del graph
    # the attention kernel alone: the same steps again, with events around it
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:            # torch creates the HIP events on first record
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for k in range(steps):
        step(warmup + k, *evs[k])
    torch.cuda.synchronize()
    attn_ms = [a.elapsed_time(b) for a, b in evs]
    attn_avg = sum(attn_ms) / len(attn_ms)
    # per-step spread: the same steps once more, each between two events
    sevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(steps)]
    for a, b in sevs:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    for k in range(steps):
        sevs[k][0].record(stream)
        step(warmup + k)
        sevs[k][1].record(stream)
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in sevs]
    cache_bytes = inp.cache_bytes()
    ms_per_step = total_ms / steps
    return {
        "ms_per_step_graph": graph_ms / steps,
        "workload": workload, "cfg": cfg, "batch": cfg.batch,
        "total_tokens": int(inp.seq_lens.astype("int64").sum()),
        "ms_per_step": ms_per_step,
        "tokens_per_s": cfg.batch / (ms_per_step * 1e-3),
        "attn_ms": attn_avg,
        "attn_ms_min": min(attn_ms),
        "attn_ms_pct": percentiles(attn_ms),
        "step_ms_pct": percentiles(step_ms),
        "cache_bytes": cache_bytes,
        "attn_gbps": cache_bytes / (attn_avg * 1e-3) / 1e9,
        "step_cache_gbps": cache_bytes / (ms_per_step * 1e-3) / 1e9,
        "splits": _lib.mla_decode_num_splits(p),
        "copies": copies,
        "inp": inp,
    }


def percentiles(xs):
    """Median, 10th and 90th percentile (ms) of per-call times."""
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def copy_bandwidth(mib: int = 1024, reps: int = 10):
    """A plain device-to-device copy of `mib` MiB, timed with events over
    `reps` copies: (read + written bytes) / time in GB/s, the median call."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(b))
    del src, dst
    times.sort()
    ms = times[len(times) // 2]
    return {"GBps": round(2 * n / (ms * 1e-3) / 1e9, 1), "bytes": 2 * n, "ms_median": round(ms, 4),
            "how": f"torch copy_ of {mib} MiB device to device, median of {reps}, read + write bytes"}


def host_cpu():
    """(logical CPUs, CPU model) of the host."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count(), model


def cpu_baseline(inp, seconds: float):
    """The oracle as it stands, on a bounded sample of the same workload:
    (sequence, group of up to 32 heads) calls in order until about `seconds` of CPU time
    have passed, extrapolated to the full step by the token x head count."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import oracle_from_inputs

    cfg = inp.cfg
    lens = inp.seq_lens.astype(np.int64)
    chunk = min(cfg.heads, 32)
    pairs, work_done, passes = 0, 0, 0
    t_start = time.perf_counter()
    while time.perf_counter() - t_start < seconds:     # repeat whole steps if one is short
        for b in range(cfg.batch):
            for i0 in range(0, cfg.heads, chunk):
                if time.perf_counter() - t_start >= seconds:
                    break
                heads = list(range(i0, min(i0 + chunk, cfg.heads)))
                oracle_from_inputs(inp, batches=[b], heads=heads)
                pairs += len(heads)
                work_done += int(lens[b]) * len(heads)
        passes += 1
    elapsed = time.perf_counter() - t_start
    work_full = int(lens.sum()) * cfg.heads
    t_full = elapsed * work_full / max(work_done, 1)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("user_api") == "blas"] or [1])
    nproc, model = host_cpu()
    return {
        "value": cfg.batch / t_full, "unit": "tokens/s", "cores": threads, "kind": "oracle",
        "threads": threads, "nproc": nproc, "cpu_model": model,
        "sample": (f"{pairs} (sequence, head) pairs in order over {passes} pass(es) of the "
                   f"step ({work_done} token-heads; one step is {work_full}) in {elapsed:.1f} s, "
                   f"fp64 numpy oracle, scaled by token-heads to one step"),
    }


def _counter_rows(directory: str):
    """(dispatch id, kernel name, counter name, value) rows of a rocprofv3
    csv counter collection found under `directory`."""
    import csv
    import glob

    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], r["Counter_Name"],
                             float(r["Counter_Value"])))
    if not rows:
        raise SystemExit(f"no counter collection under {directory}")
    return rows


def measure_writer(name: str, steps: int, warmup: int, copies: int = 64):
    """Time mla_cache_write on the writer workload `name` (weights rotated)."""
    import torch
    from head_latent_attention_10_amd import _lib
    from head_latent_attention_10_amd.device import to_device_array
    from mla_inputs.writer import WRITER_CONFIGS, generate_writer

    cfg = WRITER_CONFIGS[name]
    w = generate_writer(cfg)
    dev = torch.device("cuda")
    d = {k: to_device_array(getattr(w, k), dev)
         for k in ("x", "gamma", "positions", "block_table", "c_kv", "k_rope")}
    scale = None if w.c_kv_scale is None else to_device_array(w.c_kv_scale, dev)
    wd = [to_device_array(w.W_DKV, dev) for _ in range(copies)]
    wr = [to_device_array(w.W_KR, dev) for _ in range(copies)]
    p = _lib.make_write_params(cfg.batch, cfg.d_model, cfg.d_latent, cfg.d_rope, cfg.page_size,
                               w.block_table.shape[1], w.num_blocks, cfg.x_dtype, cfg.weight_dtype,
                               cfg.cache_dtype, cfg.rope_dtype, cfg.rms_eps, cfg.rope_base)
    nbytes = _lib.mla_cache_write_workspace_size(p)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def call(k, stream):
        _lib.mla_cache_write(p, d["x"], wd[k % copies], d["gamma"], wr[k % copies],
                             d["positions"], d["block_table"], d["c_kv"], scale, d["k_rope"],
                             ws, nbytes, stream)

    # the eager result, for checking the graph replays below
    call(0, torch.cuda.current_stream())
    torch.cuda.synchronize()
    want = [t.clone() for t in (d["c_kv"], d["k_rope"], scale) if t is not None]
    # one HIP graph of `copies` calls (kernel launches only), replayed, so that
    # the time is the GPU's and not the host's launch path
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for k in range(warmup):
            call(k, side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for k in range(copies):
            call(k, torch.cuda.current_stream())
    reps = max(1, steps // copies)
    graph.replay()
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        graph.replay()
    stop.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / (reps * copies)
    got = [t for t in (d["c_kv"], d["k_rope"], scale) if t is not None]
    # bitwise: untouched slots hold NaN
    if not all(torch.equal(u.view(torch.uint8), v.view(torch.uint8)) for u, v in zip(got, want)):
        raise RuntimeError("graph replays of the cache writer differ from the eager call")
    esz = {"f32": 4, "bf16": 2, "e4m3": 1}
    n_out = cfg.d_latent + cfg.d_rope
    alg = (n_out * cfg.d_model + cfg.d_latent) * esz[cfg.weight_dtype] \
        + cfg.batch * cfg.d_model * esz[cfg.x_dtype] \
        + cfg.batch * (cfg.d_latent * esz[cfg.cache_dtype] + cfg.d_rope * esz[cfg.rope_dtype]
                       + (4 if cfg.cache_dtype == "e4m3" else 0))
    gbps = alg / (ms * 1e-3) / 1e9
    return {"us_per_call": round(ms * 1e3, 2), "algorithmic_bytes": int(alg),
            "GBps": round(gbps, 1), "frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "batch": cfg.batch, "d_model": cfg.d_model, "cache_dtype": cfg.cache_dtype,
            "weight_copies_rotated": copies}


def measure_dsa(name: str, steps: int, warmup: int):
    """Time the DSA decode step (mla_dsa_decode: indexer, top-k, decode over the
    selection) on the workload `name`, with copies of the indexer keys and the
    latent cache rotated so that every step reads them from HBM; then each
    stage alone (its entry point between two events)."""
    import numpy as np
    import torch

    from head_latent_attention_10_amd import _lib
    from head_latent_attention_10_amd.device import DeviceInputs, out_torch_dtype, to_device_array
    from mla_inputs.dsa import DSA_CONFIGS, generate_dsa

    dcfg = DSA_CONFIGS[name]
    t0 = time.time()
    inp = generate_dsa(dcfg)
    cfg, k = inp.cfg, dcfg.topk
    dev = DeviceInputs(inp.dense)
    ix = {f: to_device_array(getattr(inp, f), dev.device)
          for f in ("q_I", "q_I_scale", "w_I", "k_I", "k_I_scale")}
    p = dev.params()
    d = _lib.make_dsa_params(dcfg.index_heads, dcfg.index_dim, k)
    lens = inp.seq_lens.astype(np.int64)
    sel = np.minimum(lens, k)
    touched = int(lens.sum()) * (dcfg.index_dim + 4) + int(sel.sum()) * 1152
    copies = max(2, math.ceil(768e6 / touched))
    c_copies = [dev.c_kv] + [dev.c_kv.clone() for _ in range(copies - 1)]
    r_copies = [dev.k_rope] + [dev.k_rope.clone() for _ in range(copies - 1)]
    s_copies = [dev.c_kv_scale] * copies
    if dev.c_kv_scale is not None:
        s_copies = [dev.c_kv_scale] + [dev.c_kv_scale.clone() for _ in range(copies - 1)]
    k_copies = [ix["k_I"]] + [ix["k_I"].clone() for _ in range(copies - 1)]
    ks_copies = [ix["k_I_scale"]] + [ix["k_I_scale"].clone() for _ in range(copies - 1)]
    ws_bytes = _lib.mla_dsa_decode_workspace_size(p, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev.device)
    out = torch.empty((cfg.batch, cfg.heads, cfg.d_v), dtype=out_torch_dtype(cfg.out_dtype),
                      device=dev.device)
    torch.cuda.synchronize()
    print(f"[bench] {name}: inputs ready in {time.time() - t0:.1f}s, {copies} copies",
          file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream()

    def step(j):
        i = j % copies
        _lib.mla_dsa_decode(p, d, dev.q, c_copies[i], s_copies[i], r_copies[i], dev.block_table,
                            dev.seq_lens, ix["q_I"], ix["q_I_scale"], ix["w_I"], k_copies[i],
                            ks_copies[i], dev.W_UK, dev.W_UV, out, None, ws, ws_bytes, stream)

    for j in range(warmup):
        step(j)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for j in range(steps):
        step(warmup + j)
    stop.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(stop) / steps

    # the stages alone, each between two events (marker events: a few us of
    # launch overhead included)
    cap = int(inp.block_table.shape[1] * cfg.page_size)
    scores = torch.empty((cfg.batch, cap), dtype=torch.float32, device=dev.device)
    idx = torch.empty((cfg.batch, k), dtype=torch.int32, device=dev.device)
    cnt = torch.empty((cfg.batch,), dtype=torch.int32, device=dev.device)
    sws = _lib.mla_decode_sparse_workspace_size(p, k)
    sw = torch.empty(sws, dtype=torch.uint8, device=dev.device)

    def stage(fn, n=steps):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for j, (a, b) in enumerate(evs):
            a.record(stream)
            fn(j)
            b.record(stream)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / n

    t_idx = stage(lambda j: _lib.mla_indexer_scores(
        p, d, ix["q_I"], ix["q_I_scale"], ix["w_I"], k_copies[j % copies], ks_copies[j % copies],
        dev.block_table, dev.seq_lens, scores, cap, stream))
    t_topk = stage(lambda j: _lib.mla_topk_select(scores, cap, dev.seq_lens, cfg.batch, k, idx, k,
                                                  cnt, stream))
    tws = _lib.mla_topk_select_split_workspace_size(cfg.batch, cap)
    tw = torch.empty(tws, dtype=torch.uint8, device=dev.device)
    t_topk_split = stage(lambda j: _lib.mla_topk_select_split(
        scores, cap, dev.seq_lens, cfg.batch, k, idx, k, cnt, tw, tws, stream))
    t_dec = stage(lambda j: _lib.mla_decode_sparse(
        p, dev.q, c_copies[j % copies], s_copies[j % copies], r_copies[j % copies],
        dev.block_table, idx, k, cnt, dev.W_UK, dev.W_UV, out, sw, sws, stream))
    esz = 1 if cfg.cache_dtype == "e4m3" else 2
    row = cfg.d_latent * esz + cfg.d_rope * 2 + (4 if cfg.cache_dtype == "e4m3" else 0)
    idx_bytes = int(lens.sum()) * (dcfg.index_dim + 4 + 4)
    dec_bytes = int(sel.sum()) * row + 2 * cfg.heads * cfg.d_latent * cfg.d_nope * 2
    alg = idx_bytes + int(lens.sum()) * 4 + int(sel.sum()) * 4 + dec_bytes
    return {"us_per_step": round(ms * 1e3, 2), "tokens_per_s": round(cfg.batch / (ms * 1e-3), 1),
            "batch": cfg.batch, "topk": k, "context_tokens": int(lens.sum()),
            "selected_tokens": int(sel.sum()), "cache_dtype": cfg.cache_dtype,
            "algorithmic_bytes": alg, "GBps": round(alg / (ms * 1e-3) / 1e9, 1),
            "stage_us": {"indexer": round(t_idx * 1e3, 2), "topk": round(t_topk * 1e3, 2),
                         "topk_split": round(t_topk_split * 1e3, 2),
                         "sparse_decode": round(t_dec * 1e3, 2)},
            "topk_in_step": "split" if cfg.batch <= 64 else "one work group per sequence",
            "indexer_key_GBps": round(idx_bytes / (t_idx * 1e-3) / 1e9, 1),
            "copies_rotated": copies}


def measure_tpla(workload: str, shards: int, steps: int, warmup: int):
    """Time the TPLA decode step (mla_tpla_decode, `shards` latent shards on
    one GPU) on `workload`, cache copies rotated as for the dense step."""
    import torch

    from head_latent_attention_10_amd import _lib
    from head_latent_attention_10_amd.device import DeviceInputs, out_torch_dtype
    from mla_inputs import CONFIGS, generate

    cfg = CONFIGS[workload]
    inp = generate(cfg)
    dev = DeviceInputs(inp)
    p = dev.params()
    t = _lib.make_tpla_params(shards)
    pool = dev.c_kv.numel() * dev.c_kv.element_size() + dev.k_rope.numel() * dev.k_rope.element_size()
    copies = max(2, math.ceil(768e6 / pool))
    c_copies = [dev.c_kv] + [dev.c_kv.clone() for _ in range(copies - 1)]
    r_copies = [dev.k_rope] + [dev.k_rope.clone() for _ in range(copies - 1)]
    s_copies = [dev.c_kv_scale] * copies
    if dev.c_kv_scale is not None:
        s_copies = [dev.c_kv_scale] + [dev.c_kv_scale.clone() for _ in range(copies - 1)]
    n = _lib.mla_tpla_decode_workspace_size(p, t)
    ws = torch.empty(n, dtype=torch.uint8, device=dev.device)
    out = torch.empty((cfg.batch, cfg.heads, cfg.d_v), dtype=out_torch_dtype(cfg.out_dtype),
                      device=dev.device)
    stream = torch.cuda.current_stream()

    def step(j):
        i = j % copies
        _lib.mla_tpla_decode(p, t, dev.q, c_copies[i], s_copies[i], r_copies[i], dev.block_table,
                             dev.seq_lens, dev.W_UK, dev.W_UV, out, ws, n, stream)

    for j in range(warmup):
        step(j)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for j in range(steps):
        step(warmup + j)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    cache = inp.cache_bytes()
    return {"us_per_step": round(ms * 1e3, 2), "tokens_per_s": round(cfg.batch / (ms * 1e-3), 1),
            "shards": shards, "shard_heads": cfg.heads * shards, "cache_bytes": cache,
            "cache_GBps_step": round(cache / (ms * 1e-3) / 1e9, 1), "copies_rotated": copies}


def measure_grouped(workload: str, groups: int, steps: int, warmup: int):
    """Time the grouped-MLA decode step (mla_grouped_decode, `groups` latent
    pools) on `workload`, copies of the pools rotated."""
    import torch

    from head_latent_attention_10_amd import _lib
    from head_latent_attention_10_amd.device import DeviceInputs, out_torch_dtype, to_device_array
    from mla_inputs import CONFIGS
    from mla_inputs.grouped import generate_grouped

    cfg = CONFIGS[workload]
    gi = generate_grouped(cfg, groups)
    dev = DeviceInputs(gi.dense)
    pools = to_device_array(gi.c_pools, dev.device)
    scales = None if gi.scale_pools is None else to_device_array(gi.scale_pools, dev.device)
    p = dev.params()
    size = pools.numel() * pools.element_size() + dev.k_rope.numel() * dev.k_rope.element_size()
    copies = max(2, math.ceil(768e6 / size))
    c_copies = [pools] + [pools.clone() for _ in range(copies - 1)]
    r_copies = [dev.k_rope] + [dev.k_rope.clone() for _ in range(copies - 1)]
    s_copies = [scales] * copies if scales is None else [scales] + [scales.clone() for _ in range(copies - 1)]
    n = _lib.mla_decode_workspace_size(p)
    ws = torch.empty(n, dtype=torch.uint8, device=dev.device)
    out = torch.empty((cfg.batch, cfg.heads, cfg.d_v), dtype=out_torch_dtype(cfg.out_dtype),
                      device=dev.device)
    stream = torch.cuda.current_stream()

    def step(j):
        i = j % copies
        _lib.mla_grouped_decode(p, groups, dev.q, c_copies[i], s_copies[i], r_copies[i],
                                dev.block_table, dev.seq_lens, dev.W_UK, dev.W_UV, out, ws, n,
                                stream)

    for j in range(warmup):
        step(j)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for j in range(steps):
        step(warmup + j)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    per_tok = groups * cfg.d_latent * (1 if cfg.cache_dtype == "e4m3" else 2) + cfg.d_rope * 2
    cache = int(gi.seq_lens.astype("int64").sum()) * per_tok
    return {"us_per_step": round(ms * 1e3, 2), "tokens_per_s": round(cfg.batch / (ms * 1e-3), 1),
            "latent_groups": groups, "kv_rank": groups * cfg.d_latent + cfg.d_rope,
            "cache_bytes": cache, "cache_GBps_step": round(cache / (ms * 1e-3) / 1e9, 1),
            "copies_rotated": copies}


def prefill_flops(seq_lens, q_lens, heads, d_qk=192, d_v=128, d_c=512):
    """Algorithmic flops of one MHA-mode prefill call: the reconstruction of the
    keys (no rope part) and values of every cached token (2 d_c flops per output
    value), and per query the score and value products over the positions it
    sees (2 (d_qk + d_v) per head and key)."""
    dec = 0
    att = 0
    for T, L in zip(seq_lens, q_lens):
        T, L = int(T), int(min(L, T))
        dec += T * heads * 2 * d_c * ((d_qk - 64) + d_v)
        keys = L * (T - L) + L * (L + 1) // 2
        att += keys * heads * 2 * (d_qk + d_v)
    return dec, att


def measure_prefill(spec: str, steps: int, warmup: int):
    """Time MHA-mode prefill (mla_prefill) on the DeepSeek-V3 shape: spec
    'batch:context:chunk[:fp8]' = `batch` sequences of `context` cached tokens
    whose last `chunk` are the new query tokens, over a bf16 (or fp8) cache."""
    import torch

    from head_latent_attention_10_amd import _lib
    from head_latent_attention_10_amd.device import DeviceInputs, out_torch_dtype, to_device_array
    from mla_inputs import CONFIGS
    from mla_inputs.prefill import generate_prefill

    parts = spec.split(":")
    B, T, L = (int(x) for x in parts[:3])
    cache = "e4m3" if parts[3:] == ["fp8"] else "bf16"
    cfg = CONFIGS["dsv3_b8_32k"].replace(batch=B, seq_len=T, out_dtype="bf16", seed=1200,
                                         cache_dtype=cache)
    pi = generate_prefill(cfg, L)
    dev = DeviceInputs(pi.dense)
    q = to_device_array(pi.q, dev.device)
    ql = to_device_array(pi.q_lens, dev.device)
    p = dev.params()
    n = _lib.mla_prefill_workspace_size(p)
    unit = _lib.prefill_unit_bytes(dev.max_blocks_per_seq, cfg.page_size)
    out = torch.empty((B, L, cfg.heads, cfg.d_v), dtype=out_torch_dtype(cfg.out_dtype),
                      device=dev.device)
    stream = torch.cuda.current_stream()

    def timed(nbytes):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev.device)

        def step():
            _lib.mla_prefill(p, L, q, ql, dev.c_kv, dev.c_kv_scale, dev.k_rope, dev.block_table,
                             dev.seq_lens, dev.W_UK, dev.W_UV, out, ws, nbytes, stream)

        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            step()
        b.record(stream)
        torch.cuda.synchronize()
        del ws
        return a.elapsed_time(b) / steps

    # the default workspace (the call in chunks of (sequence, head) units once
    # every unit's keys and values pass its size), then one holding them all
    ms = timed(n)
    units = B * cfg.heads
    ms_one_pass = timed(units * unit) if units * unit != n else ms
    dec, att = prefill_flops(pi.seq_lens, pi.q_lens, cfg.heads)
    return {"ms_per_call": round(ms, 4), "new_tokens_per_s": round(B * L / (ms * 1e-3), 1),
            "decompress_tflop": round(dec / 1e12, 4), "attention_tflop": round(att / 1e12, 4),
            "TFLOPs": round((dec + att) / (ms * 1e-3) / 1e12, 1),
            "frac_of_bf16_peak": round((dec + att) / (ms * 1e-3) / BF16_PEAK_TFLOPS / 1e12, 4),
            "workspace_bytes": n, "units": units, "units_per_chunk_max": n // unit,
            "ms_per_call_one_pass": round(ms_one_pass, 4),
            "workspace_bytes_one_pass": units * unit}


def kernel_class(name: str):
    """The decode-step stage a rocprofv3 kernel name belongs to (None: other)."""
    for key, cls in (("attend64_kernel", "attention"), ("attend64_fp8_kernel", "attention"),
                     ("attend_mfma_kernel", "attention"),
                     ("attend_fp8_kernel", "attention"), ("attend_simt_kernel", "attention"),
                     ("absorb", "absorb"), ("up16_mfma_kernel<true", "merge_up"),
                     ("up16_mfma_kernel<false", "up_project"), ("merge_kernel", "combine"),
                     ("combine", "combine"), ("up_project", "up_project"),
                     ("plan_kernel", "plan"), ("copyBuffer", "copy")):
        if key in name:
            return cls
    return None


def summarize_traffic(workload: str, fetch_dir: str, write_dir: str, copy_mb: int, commands):
    """HBM bytes per launch of every stage of the decode step from two
    rocprofv3 --pmc runs of `bench.py --calibrate-copy-mb copy_mb` (FETCH_SIZE,
    then WRITE_SIZE, KiB per dispatch).  Each counter is scaled by what it reads
    for the plain copy of copy_mb MiB that ends the run (its last copy
    dispatch); the attention launch's bytes go to hbm_bytes_per_launch."""
    import statistics

    out = {}
    for name, directory in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in _counter_rows(directory) if r[2] == name]
        copies = [(d, v) for d, k, _, v in rows if kernel_class(k) == "copy"]
        if not copies:
            raise SystemExit(f"{name}: copy dispatch missing")
        copy_kib = max(copies)[1]   # the calibration copy is the run's last dispatch
        factor = copy_mb * 1024.0 / copy_kib
        per = {}
        for cls in ("attention", "absorb", "merge_up", "combine", "up_project", "plan"):
            vals = [v for _, k, _, v in rows if kernel_class(k) == cls]
            if vals:
                per[cls] = {"kib_median": statistics.median(vals), "dispatches": len(vals),
                            "bytes_per_launch": round(statistics.median(vals) * 1024.0 * factor)}
        if "attention" not in per:
            raise SystemExit(f"{name}: attention dispatches missing")
        out[name] = {"copy_kib": copy_kib, "factor": factor, "kernels": per}
    fetch, write = out["FETCH_SIZE"], out["WRITE_SIZE"]
    step = {cls: fetch["kernels"].get(cls, {}).get("bytes_per_launch", 0) +
            write["kernels"].get(cls, {}).get("bytes_per_launch", 0)
            for cls in set(fetch["kernels"]) | set(write["kernels"])}
    rec = {
        "workload": workload,
        "kernel_source": os.path.basename(attn_source(workload)),
        "kernel_source_sha256_16": attn_source_hash(workload),
        "copy_calibration_mib": copy_mb,
        "fetch": fetch,
        "write": write,
        "hbm_bytes_per_launch": step["attention"],
        "hbm_bytes_per_step_by_stage": step,
        "hbm_bytes_per_step": sum(step.values()),
        "commands": commands,
    }
    path = os.path.join(ROOT, "profiles", f"attend_{workload}_traffic.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def summarize_counters(workload: str, dirs, commands):
    """Median per dispatch of every counter in rocprofv3 --pmc runs of this
    script (`dirs`), per decode-step stage, into
    profiles/attend_<workload>_counters.json.  MfmaUtil (rocprofv3's
    SQ_VALU_MFMA_BUSY_CYCLES summed over SIMDs / (GRBM_GUI_ACTIVE x SIMDs), in
    percent) becomes mfma_util, a fraction, for the attention kernel."""
    import statistics

    rows = []
    for d in dirs:
        rows += _counter_rows(d)
    per = {}
    for _, k, c, v in rows:
        cls = kernel_class(k)
        if cls and cls != "copy":
            per.setdefault(cls, {}).setdefault(c, []).append(v)
    stages = {cls: {c: statistics.median(vs) for c, vs in cs.items()} for cls, cs in per.items()}
    if "attention" not in stages:
        raise SystemExit("no attention dispatches in the counter runs")
    att = stages["attention"]
    rec = {
        "workload": workload,
        "kernel_source": os.path.basename(attn_source(workload)),
        "kernel_source_sha256_16": attn_source_hash(workload),
        "mfma_util": round(att["MfmaUtil"] / 100.0, 4) if "MfmaUtil" in att else None,
        "stages": stages,
        "commands": commands,
    }
    path = os.path.join(ROOT, "profiles", f"attend_{workload}_counters.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dsv3_ragged_32k")
    ap.add_argument("--also", default="dsv3_b8_32k,dsv3_b64_4k,transmla_llama2_7b,dsv3_fp8_16k",
                    help="other workloads reported under 'extra' (comma list, may be empty)")
    ap.add_argument("--num-splits", type=int, default=0)
    ap.add_argument("--writers", default="writer_dsv3_b8,writer_dsv3_b64,writer_dsv3_fp8_b32",
                    help="latent-cache writer workloads reported under 'extra' (comma list)")
    ap.add_argument("--writer-only", action="store_true",
                    help="measure only the latent-cache writer workloads (for profiling)")
    ap.add_argument("--dsa", default="dsa_dsv3_ragged_32k,dsa_dsv3_b4_128k,dsa_dsv3_fp8_16k",
                    help="DSA sparse-decode workloads reported under 'extra' (comma list)")
    ap.add_argument("--dsa-only", action="store_true",
                    help="measure only the DSA workloads (for profiling)")
    ap.add_argument("--tpla", default="dsv3_ragged_32k:2",
                    help="TPLA workloads workload:shards reported under 'extra' (comma list)")
    ap.add_argument("--grouped", default="dsv3_ragged_32k:2",
                    help="grouped-MLA workloads workload:groups reported under 'extra' (comma list)")
    ap.add_argument("--prefill", default="2:16384:4096,2:16384:4096:fp8",
                    help="MHA-mode prefill workloads batch:context:chunk[:fp8] (DeepSeek-V3 shape) "
                         "reported under 'extra' (comma list)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="measure only the prefill workloads (for profiling)")
    ap.add_argument("--tpla-only", action="store_true",
                    help="measure only the TPLA workloads (for profiling)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="after the measurement, copy this many MiB once (a plain copy of known "
                         "size for scaling rocprofv3 byte counters)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/attend_<workload>_traffic.json from two rocprofv3 --pmc "
                         "runs (FETCH_SIZE, WRITE_SIZE) of this script; no GPU needed")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="write profiles/attend_<workload>_counters.json from rocprofv3 --pmc runs "
                         "of this script (one directory per run); no GPU needed")
    ap.add_argument("--profile-command", action="append", default=[],
                    help="command line recorded with --summarize-traffic (repeatable)")
    args = ap.parse_args()

    if args.summarize_traffic:
        summarize_traffic(args.workload, args.summarize_traffic[0], args.summarize_traffic[1],
                          args.calibrate_copy_mb, args.profile_command)
        return
    if args.summarize_counters:
        summarize_counters(args.workload, args.summarize_counters, args.profile_command)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures the decode step on one GPU only; the multi-GPU path is a "
              "design (batch or context-parallel sharding) and is not built. Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)

    if args.writer_only:
        out = {w: measure_writer(w, max(320, args.steps), args.warmup)
               for w in args.writers.split(",") if w}
        print(json.dumps({"cache_writer": out}))
        return

    if args.tpla_only:
        out = {w: measure_tpla(w.split(":")[0], int(w.split(":")[1]), args.steps, args.warmup)
               for w in args.tpla.split(",") if w}
        print(json.dumps({"tpla": out}))
        return

    if args.prefill_only:
        out = {w: measure_prefill(w, max(3, args.steps), args.warmup)
               for w in args.prefill.split(",") if w}
        print(json.dumps({"prefill": out}))
        return

    if args.dsa_only:
        out = {w: measure_dsa(w, args.steps, args.warmup) for w in args.dsa.split(",") if w}
        print(json.dumps({"dsa": out}))
        return

    main_run = measure(args.workload, args.steps, args.warmup, args.num_splits)
    extra = {}
    for w in [w for w in args.also.split(",") if w]:
        r = measure(w, max(10, args.steps // 2), max(3, args.warmup // 2), args.num_splits)
        extra[w] = {"tokens_per_s": round(r["tokens_per_s"], 1),
                    "ms_per_step": round(r["ms_per_step"], 4),
                    "ms_per_step_graph": round(r["ms_per_step_graph"], 4),
                    "ms_per_step_pct": r["step_ms_pct"],
                    "attn_kernel_ms": round(r["attn_ms"], 4),
                    "attn_kernel_ms_pct": r["attn_ms_pct"],
                    "attn_cache_GBps": round(r["attn_gbps"], 1),
                    "attn_frac_of_hbm_peak": round(r["attn_gbps"] / HBM_PEAK_GBPS, 4),
                    **attention_roof(r)}
        # committed counter summaries of this workload's attention kernel, if
        # taken on its current source
        wc = measured_counters(w)
        if wc:
            extra[w]["attn_mfma_util"] = wc.get("mfma_util")
        wt = measured_traffic(w)
        if wt:
            extra[w]["attn_hbm_bytes_per_launch"] = wt
        del r
    for w in [w for w in args.writers.split(",") if w]:
        extra["cache_" + w] = measure_writer(w, max(320, args.steps), max(5, args.warmup))
    for w in [w for w in args.dsa.split(",") if w]:
        extra[w] = measure_dsa(w, max(10, args.steps // 2), max(3, args.warmup // 2))
    for w in [w for w in args.grouped.split(",") if w]:
        name, g = w.split(":")
        extra[f"grouped_{name}_G{g}"] = measure_grouped(name, int(g), max(10, args.steps // 2),
                                                        max(3, args.warmup // 2))
    for w in [w for w in args.tpla.split(",") if w]:
        name, g = w.split(":")
        extra[f"tpla_{name}_g{g}"] = measure_tpla(name, int(g), max(10, args.steps // 2),
                                                  max(3, args.warmup // 2))

    for w in [w for w in args.prefill.split(",") if w]:
        extra[f"prefill_dsv3_{w.replace(':', '_')}"] = measure_prefill(w, 5, 2)

    cfg = main_run["cfg"]
    traffic = measured_traffic(args.workload)
    counters = measured_counters(args.workload)
    copy = copy_bandwidth()
    roofline = {
        "bound": "hbm",
        "achieved": round(main_run["attn_gbps"], 1),
        "peak": HBM_PEAK_GBPS,
        "unit": "GB/s",
        "frac": round(main_run["attn_gbps"] / HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "kernel": "attend64_kernel" if cfg.heads % 64 == 0 else "attend_mfma_kernel<1>",
        "algorithmic_bytes_per_launch": main_run["cache_bytes"],
        "kernel_ms": round(main_run["attn_ms"], 4),
        "kernel_ms_pct": main_run["attn_ms_pct"],
        # a second denominator: what a plain copy reaches on this GPU in this run
        "copy_GBps": copy["GBps"],
        "frac_of_copy": round(main_run["attn_gbps"] / copy["GBps"], 4),
        "copy": copy,
        # matrix-core busy share of the kernel (SQ_VALU_MFMA_BUSY_CYCLES over
        # every SIMD's active cycles) from the committed counter run, if taken
        # on this kernel source
        "mfma_util": counters.get("mfma_util") if counters else None,
        # the kernel's own bound: max(HBM time, matrix-core time) and its share
        "own_roof": attention_roof(main_run),
    }
    if args.calibrate_copy_mb > 0:
        # the last copy dispatch of the run: a plain copy of known size that
        # scales the byte counters of a rocprofv3 --pmc run
        n = args.calibrate_copy_mb << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(main_run["inp"], args.cpu_seconds)
    line = {
        "metric": METRIC,
        "value": round(main_run["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_run["ms_per_step"], 4),
        # the same K steps captured into one HIP graph and replayed
        "ms_per_step_graph": round(main_run["ms_per_step_graph"], 4),
        "ms_per_step_pct": main_run["step_ms_pct"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.workload, "batch": cfg.batch, "heads": cfg.heads,
            "d_nope": cfg.d_nope, "d_latent": cfg.d_latent, "d_rope": cfg.d_rope, "d_v": cfg.d_v,
            "page_size": cfg.page_size, "cache_dtype": cfg.cache_dtype,
            "seq_lens": (f"uniform [{cfg.seq_len_range[0]}, {cfg.seq_len_range[1]}], seed {cfg.seed}"
                         if cfg.seq_len_range else f"{cfg.seq_len} each"),
            "total_tokens": main_run["total_tokens"], "splits": main_run["splits"],
            "cache_copies_rotated": main_run["copies"],
        },
        "latent_cache_GBps_step": round(main_run["step_cache_gbps"], 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
