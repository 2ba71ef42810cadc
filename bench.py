"""Throughput of the candidate-consuming sparse MQA-logits indexer on one MI355X.

One step = the whole hot path over one batch: the candidate expansion (the shared
sparse-column schedule) and the consuming layers (paged gather, MX-scaled MFMA, ReLU +
fp32 head reduce, per-row top-k) in one idx_expand_and_score_layers call for a step's
layers (--separate-expansion: idx_expand_candidates, then one
idx_sparse_mqa_logits_topk_layers call).  The default workload is the largest one that
fits one GPU, the long-context decode batch (256 rows, contexts 32k-128k, 128 candidate
blocks of 64 tokens, top-2048, 4 consuming layers sharing one schedule).  Inputs are seeded and
synthetic and already resident in HBM when the timed region starts; the step rotates
through enough copies of them (distinct device buffers) that no step finds its K
pages in the 256 MB Infinity Cache.

Prints one JSON line: candidate columns scored per second (and rows/s), the
dominant kernel's roofline (algorithmic bytes per launch / average launch time,
timed with HIP events attached to at least 50 of its launches on the bench stream,
in a pass after the timed steps), the step-level bandwidth, the prefill chunk's
MX-FP4 roofline from the same run, and the CPU oracle timed on a bounded sample.
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
sys.path.insert(0, ROOT)

METRIC = "candidate cols scored/s & rows/s incl. top-k; % of HBM / MXFP4-MFMA roofline"
HBM_PEAK_GBS = 8000.0
MXFP4_PEAK_TFLOPS = 10066.0
VALU_PEAK_TLANEOPS = 256 * 4 * 16 * 2.4e9 / 1e12   # 39.3: one op a lane a cycle, every SIMD
EVENT_STEPS = 64           # steps of the event-timed pass (each times its scoring launches)
KERNEL_SOURCE_DIR = "sparse_attention_indexer_candidate_amd/csrc"


def kernel_source_hash() -> str:
    """Hash of every library source (csrc/*.hip, csrc/*.h), which a stored traffic count
    must match to be reported."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, KERNEL_SOURCE_DIR)
    for name in sorted(os.listdir(d)):
        if name.endswith((".hip", ".h")):
            with open(os.path.join(d, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(case, q_format: str, ends: np.ndarray, with_output: bool = True,
                      score_format: str = "fp32") -> int:
    """Bytes the scoring of one layer must move: 68 B of K per valid column (64 B
    e2m1 + 4 B UE8M0), and per row its query (4352 B MXFP4 / 8196 B fp8 with its
    row scale), its 64 weights (fp32, or bf16 in the bf16 scoring format), ~12 B per
    candidate block (candidate id, schedule entry, block-table entry) and, when the same
    kernel selects, the 4-byte top-k output slots."""
    s = case.spec
    per_col = s.head_dim // 2 + s.head_dim // 32
    q = s.num_heads * (s.head_dim // 2 + s.head_dim // 32) if q_format == "mxfp4" \
        else s.num_heads * s.head_dim + 4
    wbytes = 2 if score_format == "bf16" else 4
    per_row = q + wbytes * s.num_heads + 12 * s.nb + (4 * s.topk if with_output else 0)
    return int(ends.astype(np.int64).sum()) * per_col + case.num_rows * per_row


def host_cpu() -> dict:
    """The host CPU the oracle runs on: model name, logical CPUs, CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = os.cpu_count() or 1
    return {"cpu_model": model, "nproc": os.cpu_count() or 1, "cpus_allowed": allowed}


def cpu_baseline(case, q_format: str, seconds: float, threads: int = 1):
    """The oracle (unchanged) over chunks of 4 of the workload's rows of layer 0, taken in
    order and wrapping around, until `seconds` of wall time have passed.  threads == 1:
    on the calling thread pinned to one CPU (restored afterwards).  threads > 1: the same
    calls on that many threads at once (the C oracle releases the GIL and keeps no state
    between calls), i.e. the rows split across the host cores."""
    import threading

    import oracle

    pool = case.layers[0].host_pool(case.spec.page_bytes)
    oracle.indexer_rows(case, 0, np.zeros(1, np.int32), q_format, pool=pool, with_logits=False)
    lock = threading.Lock()
    state = {"next": 0, "rows": 0, "cols": 0}
    t_end = time.perf_counter() + seconds

    def worker():
        while time.perf_counter() < t_end:
            with lock:
                i = state["next"]
                state["next"] = (i + 4) % case.num_rows
            chunk = (np.arange(i, i + 4) % case.num_rows).astype(np.int32)
            res = oracle.indexer_rows(case, 0, chunk, q_format, pool=pool, with_logits=False)
            with lock:
                state["rows"] += chunk.size
                state["cols"] += int(res.count.sum())

    pinned = None
    t0 = time.perf_counter()
    if threads == 1:
        try:
            old = os.sched_getaffinity(0)
            pinned = min(old)
            os.sched_setaffinity(0, {pinned})
        except (AttributeError, OSError):
            old = None
        try:
            worker()
        finally:
            if old is not None:
                os.sched_setaffinity(0, old)
    else:
        ts = [threading.Thread(target=worker) for _ in range(threads)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
    wall = time.perf_counter() - t0
    where = f"pinned to CPU {pinned}" if pinned is not None else f"{threads} thread(s)"
    return dict(value=state["cols"] / wall, unit="cols/s", cores=threads, kind="oracle",
                rows_per_s=state["rows"] / wall, **host_cpu(),
                sample=f"{state['rows']} row-scorings of layer 0 ({state['cols']} candidate cols, "
                       f"{case.num_rows} rows wrapping), C oracle on {threads} thread(s), "
                       f"{where}, {wall:.1f} s wall")


def measured_peaks(stream) -> dict:
    """The chip's measured ceilings for the roofline, from the library's reference
    kernels timed with events on the bench stream (median of 5 after a warm-up): a read
    stream over 2 GiB (larger than the caches, so every byte comes from HBM) and an
    MFMA-only loop on the MX-FP4 instruction the scoring uses."""
    import torch

    import sparse_attention_indexer_candidate_amd as idx

    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=stream.device)
    sink = torch.empty(idx.IDX_MEASURE_WGS * 4, dtype=torch.float32, device=stream.device)
    iters = 4096

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) / 1e3)
        return float(np.median(ts))

    t_read = timed(lambda: idx.idx_measure_read(buf, nbytes, sink, stream=stream.cuda_stream))
    t_mfma = timed(lambda: idx.idx_measure_mfma(iters, sink, stream=stream.cuda_stream))
    t_relu = timed(lambda: idx.idx_measure_mfma_relu(iters // 4, sink,
                                                      stream=stream.cuda_stream))
    del buf
    return {"read_gbs": nbytes / t_read / 1e9,
            "mxfp4_tflops": idx.idx_measure_mfma_flops(iters) / t_mfma / 1e12,
            "mxfp4_relu_epilogue_tflops": idx.idx_measure_mfma_flops(iters // 4) / t_relu / 1e12,
            "how": "idx_measure_read over 2 GiB; idx_measure_mfma (8 independent MX-FP4 "
                   "16x16x128 MFMA chains a wave, 4096 x 256 threads, operands in registers); "
                   "idx_measure_mfma_relu (the same MFMAs, each product through the ReLU-weight "
                   "epilogue, 9 VALU operations per MFMA); median of 5 launches timed with events"}


def gather_workload(case):
    """(table rows, request lengths, algorithmic bytes a launch) of the gather benchmark:
    one request per table row, of its rows' largest ke.  A launch reads and writes each
    position's D/2 value and D/32 scale bytes, reads one block-table entry a page, and
    reads cu and the request table (8 B a request)."""
    spec = case.spec
    tables = np.unique(case.row_table)
    lens = np.array([int(case.row_ke[case.row_table == t].max()) for t in tables], np.int64)
    pages = int(sum((n + spec.page_size - 1) // spec.page_size for n in lens))
    per_pos = spec.head_dim // 2 + spec.head_dim // 32
    return tables, lens, int(lens.sum()) * per_pos * 2 + pages * 4 + 8 * len(lens)


def bench_gather(args, idx, case, cfg, dev, gen_s):
    """The packed K workspace gather: one request per table row, its positions [0, ke)
    (the largest ke of the rows on it), layer 0's pool, every step one launch."""
    import torch

    from workloads.device import to_device

    spec = case.spec
    tables, lens, launch_bytes = gather_workload(case)
    cu = np.r_[0, np.cumsum(lens)].astype(np.int32)
    total, max_seq = int(cu[-1]), int(lens.max())
    base = to_device(case, dev, layers=[0])
    pool_bytes = base.layers[0].pool.numel()
    nrep = args.replicas if args.replicas > 0 else max(2, math.ceil(1.5e9 / launch_bytes))
    nrep = max(1, min(nrep, int(40e9 // max(pool_bytes, 1))))
    pools = [base.layers[0].pool] + [base.layers[0].pool.clone() for _ in range(nrep - 1)]
    d_cu = torch.from_numpy(cu).to(dev)
    d_req = torch.from_numpy(tables.astype(np.int32)).to(dev)
    vals = torch.empty((total, spec.head_dim // 2), dtype=torch.uint8, device=dev)
    scs = torch.empty((total, spec.head_dim // 32), dtype=torch.uint8, device=dev)
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    calls = [idx.bind_gather_k_workspace(
        cfg, idx.make_kcache(p, spec.page_size, spec.head_dim, base.block_table), d_cu, vals,
        scs, max_seq, req_table=d_req, stream=stream.cuda_stream) for p in pools]
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(max(EVENT_STEPS, 1))]
    for a, b in ev:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    ev_raw = [(idx.event_handle(a), idx.event_handle(b)) for a, b in ev]
    set_events = idx.lib.idx_set_timing_events
    for i in range(args.warmup):
        calls[i % nrep]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        calls[i % nrep]()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # event-timed pass (not part of the timed steps): every launch carries its events
    for i, pair in enumerate(ev_raw):
        set_events(*pair)
        calls[i % nrep]()
        set_events(None, None)
    torch.cuda.synchronize()
    kernel_ms = [a.elapsed_time(b) for a, b in ev]
    avg_s = float(np.mean(kernel_ms)) / 1e3
    achieved = launch_bytes / avg_s / 1e9
    peaks = measured_peaks(stream)
    traffic = traffic_for("gather_k_kernel", f"gather_{spec.name}", "mxfp4")
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": "gather_k_kernel",
            "measured_peak": peaks["read_gbs"], "frac_of_measured": achieved / peaks["read_gbs"],
            "avg_launch_us": avg_s * 1e6,
            "launch_us_p10": float(np.percentile(kernel_ms, 10)) * 1e3,
            "launch_us_p90": float(np.percentile(kernel_ms, 90)) * 1e3,
            "timed_launches": len(kernel_ms), "algorithmic_bytes_per_launch": launch_bytes}
    out = {"metric": "K positions gathered into the packed workspace/s", "value": total * args.steps / elapsed,
           "unit": "positions/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": elapsed / args.steps * 1e3, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "u8", "data": "synthetic",
           "config": {"workload": f"gather_{spec.name}", "requests": len(lens), "positions": total,
                      "page_size": spec.page_size, "path": "gather", "input_copies": nrep,
                      "seed": args.seed},
           "roofline": roof, "measured_peaks": peaks}
    if not args.no_cpu_baseline:
        import oracle

        pool = case.layers[0].host_pool(spec.page_bytes)
        n, t0 = 0, time.perf_counter()
        for r in range(len(lens)):   # whole requests until the time budget is spent
            oracle.gather_k_workspace(pool, spec.page_size, spec.head_dim, case.block_table,
                                      [0, int(lens[r])], req_table=[int(tables[r])])
            n += int(lens[r])
            if time.perf_counter() - t0 > args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": n / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
                               "sample": f"{n} positions of the first {r + 1} requests, one thread"}
    print(f"# generated inputs in {gen_s:.1f} s; {nrep} input copies", file=sys.stderr)
    print(json.dumps(out), flush=True)


def source_bytes(case, q_format: str, max_ctx: int, score_format: str = "fp32") -> int:
    """Bytes the candidate-source layer must move a launch pair: 68 B of K for every
    context token of each row's [ks, ke), the row's query and weights (as for the sparse
    path), one 4-byte part key per min(cbs, 64) positions of max_ctx written by the scoring
    kernel and read by the selection, and NB published block ids."""
    s = case.spec
    ctx = (case.row_ke - case.row_ks).astype(np.int64)
    per_col = s.head_dim // 2 + s.head_dim // 32
    q = s.num_heads * (s.head_dim // 2 + s.head_dim // 32) if q_format == "mxfp4" \
        else s.num_heads * s.head_dim + 4
    wbytes = 2 if score_format == "bf16" else 4
    parts = (max_ctx + 63) // 64 * (64 // min(64, s.cbs))
    per_row = q + wbytes * s.num_heads + 2 * 4 * parts + 4 * s.nb
    return int(ctx.sum()) * per_col + case.num_rows * per_row


def bench_source(args, idx, W, dev, stream):
    """The candidate-source layer (idx_publish_candidates): every context token of every
    row scored, blocks pooled by their largest logit, NB blocks published a row."""
    import torch

    from workloads.device import to_device

    spec = W.config(args.config)
    t0 = time.time()
    case = W.generate(spec, args.seed)
    gen_s = time.time() - t0
    sfmt = args.score_format
    cfg = idx.make_config(spec.num_heads, spec.head_dim,
                          idx.IDX_Q_MXFP4 if args.q_format == "mxfp4" else idx.IDX_Q_FP8_E4M3_ROWSCALE,
                          spec.page_size, spec.cbs, 0, spec.nb, spec.topk,
                          idx.IDX_SCORE_BF16 if sfmt == "bf16" else idx.IDX_SCORE_FP32)
    R = case.num_rows
    max_ctx = int(case.row_ke.max())
    launch_bytes = source_bytes(case, args.q_format, max_ctx, sfmt)
    base = to_device(case, dev, layers=[0])
    pool_bytes = base.layers[0].pool.numel()
    nrep = args.replicas if args.replicas > 0 else max(2, math.ceil(1.5e9 / launch_bytes))
    nrep = max(1, min(nrep, int(40e9 // max(pool_bytes, 1))))
    reps = [base.layers[0]] + [type(base.layers[0])(
        pool=base.layers[0].pool.clone(), weights=base.layers[0].weights.clone(),
        weights_bf16=base.layers[0].weights_bf16.clone(),
        q_values=None if base.layers[0].q_values is None else base.layers[0].q_values.clone(),
        q_scales=None if base.layers[0].q_scales is None else base.layers[0].q_scales.clone(),
        q_fp8=None if base.layers[0].q_fp8 is None else base.layers[0].q_fp8.clone(),
        q_rowscale=None if base.layers[0].q_rowscale is None else base.layers[0].q_rowscale.clone())
        for _ in range(nrep - 1)]
    rows = idx.make_rows(base.row_ke, base.row_ks, base.row_table, spec.next_n)
    cand = torch.empty((R, spec.nb), dtype=torch.int32, device=dev)
    ws = torch.empty(max(4, idx.idx_publish_workspace_bytes(cfg, R, max_ctx)), dtype=torch.uint8,
                     device=dev)
    sh = stream.cuda_stream
    calls = []
    for L in reps:
        qv, qs = L.q(args.q_format)
        kc = idx.make_kcache(L.pool, spec.page_size, spec.head_dim, base.block_table)
        calls.append(idx.bind_publish_candidates(cfg, rows, max_ctx, qv, qs, L.w(sfmt), kc, cand,
                                                 cand.stride(0), None, 0, ws, ws.numel(),
                                                 stream=sh))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(EVENT_STEPS)]
    for a, b in ev:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    ev_raw = [(idx.event_handle(a), idx.event_handle(b)) for a, b in ev]
    set_events = idx.lib.idx_set_timing_events
    for i in range(args.warmup):
        calls[i % nrep]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        calls[i % nrep]()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    for i, pair in enumerate(ev_raw):
        set_events(*pair)
        calls[i % nrep]()
        set_events(None, None)
    torch.cuda.synchronize()
    kernel_ms = [a.elapsed_time(b) for a, b in ev]
    avg_s = float(np.mean(kernel_ms)) / 1e3
    step_s = elapsed / args.steps
    peaks = measured_peaks(stream)
    ctx_cols = int((case.row_ke - case.row_ks).astype(np.int64).sum())
    # the scoring kernel's share: everything but the selection's read of the part keys
    # and the published ids
    parts = (max_ctx + 63) // 64 * (64 // min(64, spec.cbs))
    score_bytes = launch_bytes - R * (4 * parts + 4 * spec.nb)
    achieved = score_bytes / avg_s / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "step_gbs": launch_bytes / step_s / 1e9,
            "step_frac": launch_bytes / step_s / 1e9 / HBM_PEAK_GBS,
            "traffic": traffic_for("score_pool_kernel", f"source_{spec.name}", args.q_format,
                                   args.score_format),
            "kernel": "score_pool_kernel", "measured_peak": peaks["read_gbs"],
            "frac_of_measured": achieved / peaks["read_gbs"], "avg_launch_us": avg_s * 1e6,
            "launch_us_p10": float(np.percentile(kernel_ms, 10)) * 1e3,
            "launch_us_p90": float(np.percentile(kernel_ms, 90)) * 1e3,
            "timed_launches": len(kernel_ms),
            "timing": "dispatch events on the scoring launch, in an event pass after the timed "
                      "steps",
            "algorithmic_bytes_per_launch": score_bytes}
    out = {"metric": "context cols scored/s by the candidate-source layer (candidate blocks "
                     "published)",
           "value": ctx_cols / step_s, "unit": "cols/s", "rows_per_s": R / step_s,
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": step_s * 1e3, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None,
           "dtype": "mxfp4" if args.q_format == "mxfp4" else "fp8e4m3xmxfp4", "data": "synthetic",
           "config": {"workload": f"source_{spec.name}", "rows": R, "max_ctx": max_ctx,
                      "candidate_blocks": spec.nb, "candidate_block_size": spec.cbs,
                      "q_format": args.q_format, "score_format": sfmt, "path": "source",
                      "input_copies": nrep, "seed": args.seed},
           "roofline": roof, "measured_peaks": peaks}
    if not args.no_cpu_baseline:
        import oracle

        pool = case.layers[0].host_pool(spec.page_bytes)
        n, cols, t0 = 0, 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds:   # whole rows, one thread
            r = n % R
            oracle.source_candidates(case, 0, np.array([r], np.int32), spec.nb, args.q_format,
                                     sfmt, pool=pool)
            cols += int(case.row_ke[r] - case.row_ks[r])
            n += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = dict(value=cols / dt, unit="cols/s", cores=1, kind="oracle",
                                   rows_per_s=n / dt, **host_cpu(),
                                   sample=f"{n} rows ({cols} context cols), one thread, "
                                          f"{dt:.1f} s wall")
    print(f"# generated inputs in {gen_s:.1f} s; {nrep} input copies", file=sys.stderr)
    print(json.dumps(out), flush=True)


def traffic_file(kernel_name: str, workload: str, q_format: str, score_format: str = "fp32"):
    """profiles/ file of the FETCH_SIZE / WRITE_SIZE counters of one kernel on one workload
    (its full name: rows, sizes and layer count) in one query and scoring format."""
    sfx = "_bf16" if score_format == "bf16" else ""
    return os.path.join(ROOT, "profiles", f"traffic_{kernel_name}_{workload}_{q_format}{sfx}.json")


def traffic_for(kernel_name: str, workload: str, q_format: str, score_format: str = "fp32"):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE counters of this
    kernel on this workload, or None when none were taken for the current kernel sources."""
    tfile = traffic_file(kernel_name, workload, q_format, score_format)
    if not os.path.exists(tfile):
        return None
    with open(tfile) as f:
        t = json.load(f)
    return t.get("bytes_per_launch") if t.get("kernel_source_hash") == kernel_source_hash() else None


def run_workload(idx, W, config: int, args, dev, stream, steps: int, warmup: int,
                 layers: int = 0, per_layer_calls: bool = False, graph: bool = False,
                 rows: int = 0, separate_expansion: bool = False):
    """Generates one workload, times `steps` steps (after `warmup`) with nothing attached,
    then an event pass of EVENT_STEPS steps whose scoring launches carry dispatch events.
    Returns the measurements and the accounting the report needs.  layers / rows (> 0)
    replace the workload's layer and row counts (its other parameters unchanged)."""
    import dataclasses

    import torch

    from workloads.device import to_device

    spec = W.config(config)
    if args.q_format == "fp8" and "fp8" not in spec.q_formats:
        spec = W.config(config, q_formats=("mxfp4", "fp8"))
    if layers > 0 and layers != spec.layers:
        spec = dataclasses.replace(spec, layers=layers, name=f"{spec.name}_l{layers}")
    if rows > 0 and rows != spec.num_rows:
        spec = dataclasses.replace(spec, num_rows=rows, name=f"{spec.name}_rows{rows}")
    t0 = time.time()
    case = W.generate(spec, args.seed)
    gen_s = time.time() - t0
    cfg = idx.make_config(spec.num_heads, spec.head_dim,
                          idx.IDX_Q_MXFP4 if args.q_format == "mxfp4" else idx.IDX_Q_FP8_E4M3_ROWSCALE,
                          spec.page_size, spec.cbs, 0, spec.nb, spec.topk,
                          idx.IDX_SCORE_BF16 if args.score_format == "bf16" else idx.IDX_SCORE_FP32)
    R = case.num_rows
    sfmt = args.score_format

    # Touched bytes per step decide how many copies defeat the Infinity Cache.
    sched0 = idx.Schedule(cfg, R, dev)
    base = to_device(case, dev)
    kc0 = idx.make_kcache(base.layers[0].pool, spec.page_size, spec.head_dim, base.block_table)
    rows0 = idx.make_rows(base.row_ke, base.row_ks, base.row_table, spec.next_n)
    idx.idx_expand_candidates(cfg, rows0, kc0, base.candidate_blocks,
                              base.candidate_blocks.stride(0), sched0.struct)
    torch.cuda.synchronize()
    ends = sched0.end.cpu().numpy()
    ctx = (case.row_ke - (case.row_ks if case.row_ks is not None else 0)).astype(np.int64)
    max_ctx = int(case.row_ke.max()) if R else 0

    # The step's consuming layers go to the library in one call; the library reports
    # which kernels that call launches (one rule for the launch and this accounting).
    dense = args.path == "dense"
    # The step's expansion goes into the same call (idx_expand_and_score_layers) unless
    # asked to keep its own launch (idx_expand_candidates first).
    expand_in_call = not dense and not per_layer_calls and not separate_expansion
    layers_call = not dense and (spec.layers > 1 or expand_in_call) and not per_layer_calls
    ncols = idx.idx_num_sparse_blocks(cfg) * cfg.sparse_block_kv
    ws_rows_all = R * spec.layers
    plan = idx.idx_sparse_plan(cfg, R, spec.layers if layers_call else 1, logits_home=True)
    if dense:
        kernel_name, fused, launch_layers = "score_dense_kernel", False, 1
    else:
        kernel_name = plan["expand_and_score_kernel" if expand_in_call else "scoring_kernel"]
        fused = plan["selects_in_scoring_kernel"]
        launch_layers = plan["layers_per_scoring_launch"]
    calls_per_step = 1 if layers_call else spec.layers
    if dense:
        # every context token's K, the row's query state, the logits row written
        kernel_bytes = algorithmic_bytes(case, args.q_format, ctx, with_output=False,
                                         score_format=sfmt) + R * 4 * max_ctx
        step_bytes = (kernel_bytes + R * 4 * spec.topk) * spec.layers
    else:
        kernel_bytes = algorithmic_bytes(case, args.q_format, ends, with_output=fused,
                                         score_format=sfmt)
        step_bytes = algorithmic_bytes(case, args.q_format, ends, score_format=sfmt) * spec.layers
    pool_bytes = sum(L.pool.numel() for L in base.layers)
    if args.replicas > 0:
        nrep = args.replicas
    else:
        nrep = max(2, math.ceil(1.5e9 / step_bytes))
        nrep = max(1, min(nrep, int(40e9 // max(pool_bytes, 1))))

    reps = [base]
    for _ in range(nrep - 1):
        reps.append(type(base)(
            row_ks=base.row_ks.clone(), row_ke=base.row_ke.clone(), row_table=base.row_table.clone(),
            block_table=base.block_table.clone(), candidate_blocks=base.candidate_blocks.clone(),
            layers=[type(L)(pool=L.pool.clone(), weights=L.weights.clone(),
                            weights_bf16=L.weights_bf16.clone(),
                            q_values=None if L.q_values is None else L.q_values.clone(),
                            q_scales=None if L.q_scales is None else L.q_scales.clone(),
                            q_fp8=None if L.q_fp8 is None else L.q_fp8.clone(),
                            q_rowscale=None if L.q_rowscale is None else L.q_rowscale.clone())
                    for L in base.layers]))

    # a multi-layer call on fewer rows than CUs keeps every layer's logits (one launch
    # scores them all)
    ws_rows = ws_rows_all if layers_call else R
    ws_bytes = idx.idx_workspace_bytes(cfg, ws_rows, max_ctx if dense else 0)
    plans = []
    for d in reps:
        plans.append(dict(
            d=d, rows=idx.make_rows(d.row_ke, d.row_ks, d.row_table, spec.next_n),
            kc=[idx.make_kcache(L.pool, spec.page_size, spec.head_dim, d.block_table) for L in d.layers],
            sched=idx.Schedule(cfg, R, dev),
            out=torch.empty((R, spec.topk), dtype=torch.int32, device=dev),
            out_l=[torch.empty((R, spec.topk), dtype=torch.int32, device=dev)
                   for _ in range(spec.layers)],
            ws=torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)))
    sh = stream.cuda_stream
    n_events = EVENT_STEPS * calls_per_step
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_events)]
    for a, b in ev:            # materialise the HIP events before the timed region
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    ev_raw = [(idx.event_handle(a), idx.event_handle(b)) for a, b in ev]

    # Every launch of a step is bound once (arguments marshalled ahead), as a serving
    # loop would: a step then costs the host one foreign call per launch, so short
    # steps are not bound by Python.
    for p in plans:
        d = p["d"]
        p["expand"] = None if expand_in_call else idx.bind_expand_candidates(
            cfg, p["rows"], p["kc"][0], d.candidate_blocks, d.candidate_blocks.stride(0),
            p["sched"].struct, stream=sh)
        p["layers"] = []
        if layers_call:
            entries = [(*L.q(args.q_format), L.w(sfmt), p["kc"][layer], p["out_l"][layer], None)
                       for layer, L in enumerate(d.layers)]
            if expand_in_call:
                p["layers"].append(idx.bind_expand_and_score_layers(
                    cfg, p["rows"], d.candidate_blocks, d.candidate_blocks.stride(0),
                    p["sched"].struct, entries, spec.topk, p["ws"], p["ws"].numel(), stream=sh))
            else:
                p["layers"].append(idx.bind_sparse_mqa_logits_topk_layers(
                    cfg, p["rows"], p["sched"].struct, entries, spec.topk, p["ws"],
                    p["ws"].numel(), stream=sh))
        for layer, L in enumerate([] if layers_call else d.layers):
            qv, qs = L.q(args.q_format)
            if dense:
                call = idx.bind_dense_masked_logits_topk(
                    cfg, p["rows"], max_ctx, qv, qs, L.w(sfmt), p["kc"][layer], p["sched"].struct,
                    p["out"], p["out"].stride(0), None, 0, p["ws"], p["ws"].numel(), stream=sh)
            else:
                call = idx.bind_sparse_mqa_logits_topk(
                    cfg, p["rows"], qv, qs, L.w(sfmt), p["kc"][layer], p["sched"].struct,
                    p["out"], p["out"].stride(0), None, p["ws"], p["ws"].numel(), stream=sh)
            p["layers"].append(call)
    set_events = idx.lib.idx_set_timing_events

    def launch(p, events=None):
        if p["expand"] is not None:
            p["expand"]()
        for c, call in enumerate(p["layers"]):
            if events is not None:
                set_events(*events[c])
            call()
            if events is not None:
                set_events(None, None)

    for i in range(warmup):
        launch(plans[i % nrep])
    torch.cuda.synchronize()
    if graph:
        for p in plans:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                launch(p)
            p["graph"] = g
        for i in range(warmup):
            plans[i % nrep]["graph"].replay()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        p = plans[i % nrep]
        if graph:
            p["graph"].replay()
        else:
            launch(p)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # Event pass, after the timed steps and not counted in them: the events ride on the
    # scoring dispatch itself (hipExtLaunchKernel), which costs the host ~20 us a launch.
    for i in range(EVENT_STEPS):
        launch(plans[i % nrep], ev_raw[i * calls_per_step:(i + 1) * calls_per_step])
    torch.cuda.synchronize()
    kernel_ms = [a.elapsed_time(b) for a, b in ev]
    return dict(spec=spec, case=case, cfg=cfg, ends=ends, ctx=ctx, max_ctx=max_ctx, R=R,
                gen_s=gen_s, kernel_name=kernel_name, fused=fused, launch_layers=launch_layers,
                layers_call=layers_call, expand_in_call=expand_in_call, plan=plan,
                kernel_bytes=kernel_bytes,
                step_bytes=step_bytes, nrep=nrep, elapsed=elapsed, steps=steps,
                kernel_ms=kernel_ms)


def roofline(m, config: int, q_format: str, peaks: dict, dense: bool,
             score_format: str = "fp32") -> dict:
    """The scoring kernel's roofline object from run_workload's measurements."""
    spec, kernel_ms = m["spec"], m["kernel_ms"]
    avg_s = float(np.mean(kernel_ms)) / 1e3
    cols_per_layer = int(m["ends"].astype(np.int64).sum())
    scored = int(m["ctx"].sum()) if dense else cols_per_layer
    launch_bytes = m["kernel_bytes"] * m["launch_layers"]
    achieved_gbs = launch_bytes / avg_s / 1e9
    flops = 2 * spec.num_heads * spec.head_dim * scored * m["launch_layers"]
    step_s = m["elapsed"] / m["steps"]
    if spec.mode == "prefill":
        # Prefill chunks share each K tile among many rows (K comes from L2), so the MX-FP4
        # MFMA rate bounds them; decode rows each stream their own K from HBM.
        roof = {"bound": "mfma", "achieved": flops / avg_s / 1e12, "peak": MXFP4_PEAK_TFLOPS,
                "unit": "TFLOP/s"}
        # What actually bounds the contraction here: its ReLU-weight epilogue, one integer
        # max and one fp32 FMA per (head, column) element on the vector ALUs, whose peak is
        # 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz lane-operations per second.
        lane_ops = 2 * spec.num_heads * scored * m["launch_layers"]
        roof["epilogue_valu"] = {"achieved": lane_ops / avg_s / 1e12, "peak": VALU_PEAK_TLANEOPS,
                                 "unit": "T lane-ops/s",
                                 "frac": lane_ops / avg_s / 1e12 / VALU_PEAK_TLANEOPS}
        roof["step_tflops"] = flops / m["launch_layers"] * spec.layers / step_s / 1e12
        roof["step_frac"] = roof["step_tflops"] / MXFP4_PEAK_TFLOPS
        # The per-row byte count reads a request's K once per row; what must cross HBM is
        # that K once per request (the longest row of each block table) plus the per-row
        # query, weights, schedule and output.
        case = m["case"]
        per_col = spec.head_dim // 2 + spec.head_dim // 32
        uniq_cols = sum(int(case.row_ke[case.row_table == t].max())
                        for t in np.unique(case.row_table))
        uniq_bytes = (m["kernel_bytes"] - int(m["ends"].astype(np.int64).sum()) * per_col
                      + uniq_cols * per_col) * m["launch_layers"]
        roof["unique_bytes_per_launch"] = uniq_bytes
    else:
        roof = {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
        # the whole step (expansion + every layer's launches) against the same peak
        roof["step_gbs"] = m["step_bytes"] / step_s / 1e9
        roof["step_frac"] = roof["step_gbs"] / HBM_PEAK_GBS
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["measured_peak"] = peaks["mxfp4_tflops"] if roof["bound"] == "mfma" else peaks["read_gbs"]
    roof["frac_of_measured"] = roof["achieved"] / roof["measured_peak"]
    if roof["bound"] == "mfma":
        # the MFMA rate left once the same SIMDs issue the ReLU-weight epilogue
        roof["epilogue_ceiling"] = peaks["mxfp4_relu_epilogue_tflops"]
        roof["frac_of_epilogue_ceiling"] = roof["achieved"] / roof["epilogue_ceiling"]
    roof.update({"traffic": traffic_for(m["kernel_name"], spec.name, q_format, score_format),
                 "kernel": m["kernel_name"], "avg_launch_us": avg_s * 1e6,
                 "launch_us_p10": float(np.percentile(kernel_ms, 10)) * 1e3,
                 "launch_us_p90": float(np.percentile(kernel_ms, 90)) * 1e3,
                 "timed_launches": len(kernel_ms),
                 "timing": "dispatch events on the scoring launch, in an event pass after the "
                           "timed steps",
                 "algorithmic_bytes_per_launch": launch_bytes, "hbm_gbs": achieved_gbs,
                 "mxfp4_tflops": flops / avg_s / 1e12})
    if "unique_bytes_per_launch" in roof:
        roof["operand_gbs"] = achieved_gbs
        roof["hbm_gbs"] = roof["unique_bytes_per_launch"] / avg_s / 1e9
    return roof


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=4,
                    help="workload 1-5 (default 4, the long-context decode batch); 6: decode "
                         "with two rows per request")
    ap.add_argument("--q-format", default="mxfp4", choices=["mxfp4", "fp8"])
    ap.add_argument("--score-format", default="fp32", choices=["fp32", "bf16"],
                    help="fp32 weights and logits (default), or bf16 weights with bf16-rounded "
                         "logits")
    ap.add_argument("--path", default="sparse", choices=["sparse", "dense", "gather", "source"],
                    help="sparse: the indexer; dense: the comparator "
                         "idx_dense_masked_logits_topk (scores the whole context); gather: "
                         "idx_gather_k_workspace of every table row's context [0, ke); source: "
                         "the candidate-source layer idx_publish_candidates")
    ap.add_argument("--replicas", type=int, default=0, help="input copies (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the prefill chunk's MX-FP4 roofline (reported beside the "
                         "long-context decode workload's, the default)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--layers", type=int, default=0,
                    help="consuming layers a step (0: the workload's own); each layer gets its "
                         "own K pool, query and weights, all sharing one schedule")
    ap.add_argument("--rows", type=int, default=0,
                    help="query rows a step (0: the workload's own; sparse and dense paths), "
                         "e.g. --config 6 --rows 512 for 256 requests of two decode rows")
    ap.add_argument("--per-layer-calls", action="store_true",
                    help="one sparse call per layer instead of one multi-layer call")
    ap.add_argument("--separate-expansion", action="store_true",
                    help="the expansion in its own call (idx_expand_candidates) before the "
                         "scoring call, instead of idx_expand_and_score_layers")
    ap.add_argument("--graph", action="store_true",
                    help="replay each timed step as a captured HIP graph (measured slower than "
                         "direct launches on this stack: 21.7 vs 14.8 us a decode-batch step)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MB",
                    help="only run a plain device copy of MB megabytes 5 times (the reference "
                         "for scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    if args.calibrate_copy:
        import torch

        n = args.calibrate_copy << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 5}))
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(rows would shard across GPUs with no exchange)", file=sys.stderr)
        sys.exit(2)

    if args.rows and args.path in ("gather", "source"):
        print("--rows applies to the sparse and dense paths", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_attention_indexer_candidate_amd as idx
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.path == "gather":
        spec = W.config(args.config)
        t0 = time.time()
        case = W.generate(spec, args.seed)
        cfg = idx.make_config(spec.num_heads, spec.head_dim, idx.IDX_Q_MXFP4, spec.page_size,
                              spec.cbs, 0, spec.nb, spec.topk)
        return bench_gather(args, idx, case, cfg, dev, time.time() - t0)
    # A stream of the bench's own (default priority), current for the rest of the run.
    stream = torch.cuda.Stream()
    torch.cuda.set_stream(stream)
    if args.path == "source":
        return bench_source(args, idx, W, dev, stream)
    dense = args.path == "dense"
    m = run_workload(idx, W, args.config, args, dev, stream, args.steps, args.warmup,
                     layers=args.layers, per_layer_calls=args.per_layer_calls, graph=args.graph,
                     rows=args.rows, separate_expansion=args.separate_expansion)
    spec, R = m["spec"], m["R"]
    peaks = measured_peaks(stream)
    roof = roofline(m, args.config, args.q_format, peaks, dense, args.score_format)
    cols_per_step = int(m["ends"].astype(np.int64).sum()) * spec.layers
    ctx_cols_per_step = int(m["ctx"].sum()) * spec.layers
    elapsed = m["elapsed"]
    out = {
        "metric": METRIC,
        "value": cols_per_step * args.steps / elapsed,
        "unit": "cols/s",
        "rows_per_s": R * spec.layers * args.steps / elapsed,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": elapsed / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4" if args.q_format == "mxfp4" else "fp8e4m3xmxfp4",
        "data": "synthetic",
        "config": {"workload": spec.name, "rows": R, "candidate_blocks": spec.nb,
                   "candidate_block_size": spec.cbs, "topk": spec.topk, "layers": spec.layers,
                   "heads": spec.num_heads, "head_dim": spec.head_dim, "page_size": spec.page_size,
                   "valid_cols_per_step": cols_per_step, "q_format": args.q_format,
                   "score_format": args.score_format,
                   "path": args.path,
                   "calls": "one call for all layers" if m["layers_call"] else "one call per layer",
                   "expansion": ("in the scoring kernel" if m["plan"]["expansion_in_scoring_kernel"]
                                 else "own launch, in the same call") if m["expand_in_call"]
                                else "own call",
                   "launch": "HIP graph per step" if args.graph else "direct",
                   "input_copies": m["nrep"], "seed": args.seed},
        "roofline": roof,
        "measured_peaks": peaks,
    }
    if dense:
        out["context_cols_per_s"] = ctx_cols_per_step * args.steps / elapsed
    if not args.no_prefill and not dense and args.config == 4 and args.q_format == "mxfp4":
        # the prefill chunk (4096 rows of one request), whose bound is the MX-FP4 MFMA rate
        pm = run_workload(idx, W, 3, args, dev, stream, max(args.steps, 20), args.warmup)
        pr = roofline(pm, 3, args.q_format, peaks, False, args.score_format)
        pcols = int(pm["ends"].astype(np.int64).sum())
        out["prefill"] = {"workload": pm["spec"].name, "rows": pm["R"],
                          "ms_per_step": pm["elapsed"] / pm["steps"] * 1e3,
                          "cols_per_s": pcols * pm["steps"] / pm["elapsed"],
                          "rows_per_s": pm["R"] * pm["steps"] / pm["elapsed"],
                          "steps": pm["steps"], "input_copies": pm["nrep"], "roofline": pr}
        del pm
    if not args.no_cpu_baseline:
        case = m["case"]
        out["cpu_baseline"] = cpu_baseline(case, args.q_format, args.cpu_seconds)
        allowed = host_cpu()["cpus_allowed"]
        out["cpu_baseline_all_cores"] = cpu_baseline(case, args.q_format, args.cpu_seconds,
                                                     threads=max(1, min(16, allowed)))
    print(f"# generated inputs in {m['gen_s']:.1f} s; {m['nrep']} input copies", file=sys.stderr)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
