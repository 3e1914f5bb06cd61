#!/usr/bin/env python3
"""Benchmark of the DeepSeek-V4 hybrid sparse MQA attention path on one GPU.

One step = one dsv4_attn_forward call (gather + fused split kernel + merge)
over one batch of a synthetic workload already resident in HBM.  The default
is workload 3 (C128 decode, 64 requests x 128K tokens, 84 MB per call), the
largest of the five.  To keep the 256 MB Infinity Cache from serving repeated
steps, the step rotates over several GPU copies of the inputs (same values,
different addresses) whose referenced bytes together exceed the cache three
times (workload 5, whose call touches only ~4 MB, rotates its C4 index lists
over one set of pools instead).

Prints ONE JSON line: tokens (query rows) per second of the whole job over a
timed HIP-graph replay of exactly --steps calls; a roofline object for the
dominant kernel (the split kernel: the bytes it must read -- Q, C4 index
lists and every unique KV row -- over its average duration from HIP events
recorded on its stream around each kernel of a timed run of eager calls on
the same rotating inputs, queued behind a spin kernel so that they run back
to back; inside a graph replay event nodes add about a microsecond to each
interval, and host-paced eager calls add the launch gaps); the whole path's
achieved GB/s per step; and the fp64
oracle timed on the host cores on a bounded sample of the same workload, with
all threads and with one.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

METRIC = "decode attention tokens/s + achieved HBM GB/s (% peak), C4/C128 at batch×ctx"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 matrix peak of MI355X
RIDGE_FLOP_PER_BYTE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
MALL_BYTES = 256 << 20
KV_ROW_BYTES = {"bf16": 1024, "fp8": 584}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = [os.path.join(ROOT, "hybrid_sparse_mqa_amd", "csrc", f)
                  for f in ("dsv4_attn_kernels.hip", "dsv4_device.h", "dsv4_launch.h")]



# Split-kernel variant (DSV4_KERNEL_* of dsv4_attn_plan) -> (name as rocprofv3 prints it, heads per workgroup).
# (name as rocprofv3 prints it, without the namespace: the second template
# argument is the key-recording switch, off in every timed call; heads per
# workgroup)
SPLIT_KERNELS = {1: ("attn_narrow_kernel<false>", 16), 2: ("attn_wide_kernel<1, false>", 32),
                 3: ("attn_ws_kernel<1, false>", 32), 4: ("attn_wide_kernel<2, false>", 64),
                 5: ("attn_fp8_kernel<2, false>", 64), 6: ("attn_fp8_kernel<1, false>", 32)}


def split_kernel_name(kernel: int) -> str:
    """Name (as rocprofv3 prints it) of the split kernel that runs."""
    return SPLIT_KERNELS[kernel][0]


def kernel_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def algorithmic_bytes(case) -> dict:
    """Bytes one call must move: Q, out, lse, C4 index lists and every unique
    KV row it reads (SWA window rows and visible/selected compressed rows)."""
    T, H = case.T, case.H
    q = T * H * 512 * 2
    out = T * H * 512 * 2
    lse = T * H * 4
    idx = T * case.K * 4 if case.R == 4 else 0
    swa_rows = 0
    ext_rows = 0
    for r in range(case.B):
        lo_t, hi_t = int(case.qo_indptr[r]), int(case.qo_indptr[r + 1])
        n_q = hi_t - lo_t
        if n_q == 0:
            continue
        L = int(case.seq_lens[r])
        p_first, p_last = L - n_q, L - 1
        swa_rows += p_last - max(0, p_first - case.W + 1) + 1
        if case.R == 128:
            ext_rows += (p_last + 1) // 128
        elif case.R == 4:
            ids = case.c4_indices[lo_t:hi_t]
            ext_rows += len(np.unique(ids[ids >= 0]))
    kv = (swa_rows + ext_rows) * KV_ROW_BYTES[case.kv]
    return dict(total=q + out + lse + idx + kv, kv=kv, q=q, out=out, lse=lse, idx=idx,
                kv_rows=swa_rows + ext_rows, flops=attention_flops(case))


def attention_flops(case) -> int:
    """Multiply-add work of one call: per query row and key, 2*H*512 for the
    scores and 2*H*512 for P.V (keys: the window plus the used C4 entries or
    the visible C128 entries of the row)."""
    total_keys = 0
    for r in range(case.B):
        lo_t, hi_t = int(case.qo_indptr[r]), int(case.qo_indptr[r + 1])
        n_q = hi_t - lo_t
        L = int(case.seq_lens[r])
        for t in range(lo_t, hi_t):
            p = L - n_q + (t - lo_t)
            keys = min(case.W, p + 1)
            if case.R == 128:
                keys += (p + 1) // 128
            elif case.R == 4:
                keys += int((case.c4_indices[t] >= 0).sum())
            total_keys += keys
    return 4 * case.H * 512 * total_keys


def describe_workload(n, case) -> dict:
    sl = case.seq_lens
    return {
        "workload": case.name,
        "batch": int(case.B),
        "query_rows": int(case.T),
        "seq_len": int(sl[0]) if np.all(sl == sl[0]) else f"{int(sl.min())}-{int(sl.max())}",
        "q_heads": int(case.H),
        "kv_heads": 1,
        "head_dim": 512,
        "window": int(case.W),
        "compress_ratio": int(case.R),
        "c4_topk": int(case.K) if case.R == 4 else None,
        "kv_format": case.kv,
        "page_size": 256,
    }


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_rate(orc, case, target_s: float, threads: int):
    """Rows per second of the fp64 oracle with `threads` OpenMP threads over
    a seeded sample of the workload's rows, repeated for about target_s."""
    t0 = time.perf_counter()
    orc.attention(case, rows=[0], nthreads=1)
    per_row_1 = max(time.perf_counter() - t0, 1e-6)
    n = int(max(1, min(case.T, target_s * threads / per_row_1)))
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(case.T, size=n, replace=False)).astype(np.int32)
    reps = 0
    t0 = time.perf_counter()
    while True:  # repeat the sample until about target_s seconds of CPU work
        orc.attention(case, rows=rows, nthreads=threads)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= target_s:
            break
    return reps * n / dt, n, reps, dt


def cpu_baseline(case, target_s: float):
    """The fp64 oracle on the host cores over a bounded sample of rows: with
    every thread OpenMP gets (the reported value) and with one thread."""
    import oracle

    orc = oracle.Oracle()
    omp_threads = int(orc.max_threads())
    threads = max(1, min(omp_threads, case.T))
    v_all, n, reps, dt = _oracle_rate(orc, case, target_s / 2, threads)
    v_one, n1, reps1, dt1 = _oracle_rate(orc, case, target_s / 2, 1)
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    per_row = algorithmic_bytes(case)["total"] / case.T  # the call's algorithmic bytes per query row
    return {
        "value": v_all,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "effective_gbs": v_all * per_row / 1e9,  # the same algorithmic bytes per row, at the oracle's rate
        "sample": f"{n} of {case.T} query rows of the same workload x {reps} repetitions "
                  f"(fp64 C, OpenMP over rows, {threads} threads), {dt:.1f} s",
        "one_thread": {"value": v_one, "unit": "tokens/s", "cores": 1, "effective_gbs": v_one * per_row / 1e9,
                       "sample": f"{n1} rows x {reps1} repetitions, {dt1:.1f} s"},
        "host": {"cpu_model": cpu_model(), "nproc": os.cpu_count(), "affinity": affinity,
                 "omp_threads": omp_threads},
    }


def copy_calibration(mib: int) -> int:
    """A plain device-to-device copy of `mib` MiB, ten times (for scaling the
    FETCH_SIZE / WRITE_SIZE counters against a kernel of known traffic)."""
    import torch

    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {mib} MiB x 10", flush=True)
    return 0


def _counter_per_dispatch(csv_dir: str, counter: str) -> dict:
    """Mean value of `counter` per dispatch, by kernel name, from a rocprofv3
    --pmc run written with --output-format csv."""
    import csv
    import glob

    vals = {}
    for f in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row["Counter_Name"] != counter:
                continue
            vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in vals.items()}


def record_traffic(config: int, split_keys: int, fetch_dir: str, write_dir: str, copy_fetch_dir: str,
                   copy_write_dir: str, copy_mib: int, commands: list) -> int:
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of the
    attention, and of a plain copy of known size) into HBM bytes per launch of
    the split kernel, stored with a hash of the kernel sources."""
    from synth import make_config, tile_requests

    case = make_config(config)
    from hybrid_sparse_mqa_amd import dsv4_attn_plan

    _, _, kernel = dsv4_attn_plan(case.T, case.H, case.R, case.W, case.K,
                               0 if case.extra_page_table is None else case.extra_page_table.shape[1],
                               kv_fp8=case.kv == "fp8")
    name = split_kernel_name(kernel)

    def pick(d, key):
        hits = {k: v for k, v in d.items() if key in k}
        if len(hits) != 1:
            raise SystemExit(f"expected one kernel matching {key!r}, found {sorted(hits)}")
        return next(iter(hits.values()))

    copy_bytes = float(copy_mib << 20)
    f_copy = pick(_counter_per_dispatch(copy_fetch_dir, "FETCH_SIZE"), "copyBuffer") * 1024.0
    w_copy = pick(_counter_per_dispatch(copy_write_dir, "WRITE_SIZE"), "copyBuffer") * 1024.0
    f_attn = pick(_counter_per_dispatch(fetch_dir, "FETCH_SIZE"), name) * 1024.0
    w_attn = pick(_counter_per_dispatch(write_dir, "WRITE_SIZE"), name) * 1024.0
    f_scale, w_scale = copy_bytes / f_copy, copy_bytes / w_copy
    rec = {
        "kernel_sha": kernel_sha(),
        "split_keys": split_keys,
        "hbm_bytes_per_launch": f_attn * f_scale + w_attn * w_scale,
        "fetch_bytes_per_launch": f_attn * f_scale,
        "write_bytes_per_launch": w_attn * w_scale,
        "raw_fetch_kib": f_attn / 1024.0,
        "raw_write_kib": w_attn / 1024.0,
        "copy_calibration": {"bytes": copy_bytes, "fetch_scale": f_scale, "write_scale": w_scale},
        "algorithmic_bytes_per_launch": None,
        "commands": commands,
    }
    ab = algorithmic_bytes(case)
    rec["algorithmic_bytes_per_launch"] = ab["q"] + ab["idx"] + ab["kv"]
    data = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
    data[f"{name}/{case.name}"] = rec
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    print(json.dumps({f"{name}/{case.name}": rec}, indent=1))
    return 0


def bench_pack(args) -> int:
    """The KV store kernel (dsv4_kv_pack_fp8) on its own: `args.pack` bf16 K
    rows quantised into packed FP8 records at a random permutation of the
    pool's slots, timed as one HIP graph replay of `steps` calls rotating over
    enough input copies that they do not stay in the MALL."""
    import torch

    from hybrid_sparse_mqa_amd import dsv4_kv_pack_fp8
    from synth.workloads import FP8_PAGE_BYTES, _to_bf16_bits

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    n = int(args.pack)
    pages = (n + 255) // 256
    rng = np.random.default_rng(0)
    k = rng.standard_normal((n, 512), dtype=np.float32)
    k *= np.exp(rng.uniform(np.log(1e-3), np.log(1e2), (n, 1))).astype(np.float32)
    k_bits = _to_bf16_bits(k)
    slots = rng.permutation(pages * 256)[:n].astype(np.int32)
    set_bytes = n * 1024 + pages * FP8_PAGE_BYTES
    n_sets = int(min(16, max(2, -(-3 * MALL_BYTES // set_bytes))))
    kt = torch.from_numpy(k_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    st = torch.from_numpy(slots).to(dev)
    sets = [(kt if i == 0 else kt.clone(), torch.zeros((pages, FP8_PAGE_BYTES), dtype=torch.uint8, device=dev))
            for i in range(n_sets)]
    # Algorithmic bytes per call: K rows read, slots read, records and scales written.
    nbytes = n * (1024 + 4 + 576 + 4)

    def step(i):
        kk, pool = sets[i % n_sets]
        dsv4_kv_pack_fp8(kk, st, pool)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(args.steps):
                step(i)
        g.replay()  # warm replay (untimed)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    achieved = nbytes / (ms * 1e-3) / 1e9
    result = {
        "metric": "KV store rows/s (bf16 K -> packed FP8 records) + achieved HBM GB/s (% peak)",
        "value": n / (ms * 1e-3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16->fp8",
        "data": "synthetic",
        "config": {"workload": f"fp8_kv_pack_n{n}", "rows": n, "pages": pages, "input_sets": n_sets,
                   "cache": "cold-rotated", "timed": "HIP graph replay, events around it on the kernels' stream",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "pack_fp8_kernel<4>" if n >= 16384 else "pack_fp8_kernel<1>",
                     "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": ms},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle

        o = oracle.Oracle()
        m = min(n, 2048)
        pool = np.zeros(((m + 255) // 256 + 1, FP8_PAGE_BYTES), np.uint8)
        sl = np.arange(m, dtype=np.int32)
        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds / 2:
            o.pack_fp8(k_bits[:m], sl, pool)
            reps += 1
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": reps * m / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
                                  "sample": f"{m} of {n} rows x {reps} repetitions (C, one thread), {dt:.1f} s"}
    print(json.dumps(result), flush=True)
    return 0


def bench_topk(args) -> int:
    """The C4 top-k kernel (dsv4_c4_topk) on its own: `args.topk` rows of
    2^18 candidate scores each (the C4 entries of a 1M-token context), K = 512,
    timed as one HIP graph replay of `steps` calls rotating over enough score
    copies that they do not stay in the MALL."""
    import torch

    from hybrid_sparse_mqa_amd import dsv4_c4_topk

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    T, n, K = int(args.topk), 1 << 18, 512
    rng = np.random.default_rng(0)
    scores = rng.standard_normal((T, n), dtype=np.float32)
    n_sets = int(min(32, max(2, -(-3 * MALL_BYTES // (T * n * 4)))))
    st = torch.from_numpy(scores).to(dev)
    sets = [st if i == 0 else st.clone() for i in range(n_sets)]
    nc = torch.full((T,), n, dtype=torch.int32, device=dev)
    outs = [torch.empty((T, K), dtype=torch.int32, device=dev) for _ in range(2)]
    nbytes = T * n * 4 + T * K * 4  # scores read once, indices written

    def step(i):
        dsv4_c4_topk(sets[i % n_sets], nc, K, indices=outs[i & 1])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(args.steps):
                step(i)
        g.replay()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    achieved = nbytes / (ms * 1e-3) / 1e9
    result = {
        "metric": "C4 top-512 selections/s (query rows over 2^18 candidates) + achieved HBM GB/s (% peak)",
        "value": T / (ms * 1e-3), "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"c4_topk512_b{T}_n262144", "rows": T, "candidates": n, "k": K,
                   "input_sets": n_sets, "cache": "cold-rotated",
                   "timed": "HIP graph replay, events around it on the kernels' stream", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": "topk_chunk_kernel + topk_finish_kernel (one call)",
                     "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": ms},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        from oracle.topk import topk_select

        reps, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds / 2:
            topk_select(scores, np.full(T, n), K)
            reps += 1
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": reps * T / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
                                  "sample": f"all {T} rows x {reps} repetitions (numpy lexsort), {dt:.1f} s"}
    print(json.dumps(result), flush=True)
    return 0


def plain_read_ms(nbytes: int, reps: int = 50, workgroups: int = 1024) -> float:
    """Average duration of the library's plain streaming read of `nbytes`
    bytes (dsv4_read_probe), each call bracketed by its own event pair and all
    of them queued behind a spin kernel, as the split kernel's durations are;
    successive calls read disjoint windows of a buffer four times larger than
    the 256 MB MALL, so that every call reads from HBM."""
    import torch

    from hybrid_sparse_mqa_amd import dsv4_read_probe

    nbytes = (nbytes + 255) // 256 * 256
    span = max(4 * nbytes, 1 << 30)
    buf = torch.ones(span + nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(16, dtype=torch.uint8, device="cuda")
    stride = nbytes + 4096  # no two consecutive windows share a line
    offsets = [(i * stride) % span // 256 * 256 for i in range(reps)]
    for o in offsets[:3]:
        dsv4_read_probe(buf[o:], nbytes, workgroups, sink)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in offsets]
    torch.cuda._sleep(1 << 24)
    for (e0, e1), o in zip(evs, offsets):
        e0.record()
        dsv4_read_probe(buf[o:], nbytes, workgroups, sink)
        e1.record()
    torch.cuda.synchronize()
    ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / reps
    del buf
    return ms


def bench_stream(args) -> int:
    """Achievable HBM bandwidth on this device, for context beside the 8 TB/s
    peak the roofline fractions use: torch's own kernels reading (a sum over
    a 1 GiB bf16 tensor), writing (a fill) and copying (read + write), each
    far larger than the 256 MB MALL, timed with events over repeated calls."""
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    n = 1 << 29  # bf16 elements: 1 GiB
    x = torch.randn(n, dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x)
    acc = torch.empty((), dtype=torch.float32, device=dev)

    def timed(fn, nbytes, reps=args.steps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return nbytes / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9

    read = timed(lambda: torch.sum(x, dim=0, dtype=torch.float32, out=acc), 2 * n)
    write = timed(lambda: y.fill_(1.0), 2 * n)
    copy = timed(lambda: y.copy_(x), 4 * n)
    del x, y
    # The library's plain streaming read at a range of sizes: small reads
    # cannot reach the large-read rate (launch, ramp-up and drain are fixed).
    probe = {}
    for nbytes in (1 << 30, 256 << 20, 80 << 20, 24 << 20, 4 << 20):
        ms = plain_read_ms(nbytes, reps=20 if nbytes >= (256 << 20) else 50)
        probe[str(nbytes)] = {"us": ms * 1e3, "gbs": nbytes / (ms * 1e-3) / 1e9,
                              "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    print(json.dumps({
        "metric": "achievable HBM bandwidth (torch kernels, 1 GiB operands; plain read probe by size)",
        "unit": "GB/s", "read_gbs": read, "write_gbs": write, "copy_gbs": copy,
        "read_frac": read / HBM_PEAK_GBS, "write_frac": write / HBM_PEAK_GBS, "copy_frac": copy / HBM_PEAK_GBS,
        "plain_read_probe": probe, "peak": HBM_PEAK_GBS, "reps": args.steps,
    }), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3,
                    help="workload 1..7 (default 3: C128 decode, batch 64 x 128K, the largest decode workload; "
                         "6 and 7 are the C4 and C128 sparse-prefill workloads)")
    ap.add_argument("--sets", type=int, default=0, help="input copies to rotate over (0 = auto)")
    ap.add_argument("--batch", type=int, default=0,
                    help="requests per call: workloads 2-4, B requests of the workload's shape; workload 5, a "
                         "multiple of 8 (copies of the 8 requests, each copy reading through its own C4 index lists)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample size target")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--split-keys", type=int, default=0, help="force keys per split (0 = library plan)")
    ap.add_argument("--kernel", type=int, default=0,
                    help="force a bf16 split-kernel variant (DSV4_KERNEL_*, 0 = library choice)")
    ap.add_argument("--sample-every", type=int, default=10,
                    help="time the kernels of every N-th call of the timed replay with HIP events")
    ap.add_argument("--pack", type=int, default=0, metavar="ROWS",
                    help="time the FP8 KV store kernel on ROWS rows instead of the attention")
    ap.add_argument("--topk", type=int, default=0, metavar="ROWS",
                    help="time the C4 top-512 kernel on ROWS rows of 2^18 candidates instead of the attention")
    ap.add_argument("--stream", action="store_true",
                    help="measure achievable HBM read / write / copy bandwidth with torch kernels")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--traffic-from", nargs=4, metavar=("FETCH", "WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="rocprofv3 --pmc output folders to turn into profiles/traffic_counters.json")
    ap.add_argument("--copy-mib", type=int, default=1024, help="size of the calibration copy in MiB")
    ap.add_argument("--commands", nargs="*", default=[], help="commands recorded with --traffic-from")
    args = ap.parse_args()

    if args.traffic_from:
        return record_traffic(args.config, args.split_keys, *args.traffic_from, args.copy_mib, args.commands)
    if args.copy_calibration:
        return copy_calibration(args.copy_calibration)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported (the attention shards by "
              "request, so N GPUs run N independent copies of this benchmark)", file=sys.stderr)
        return 2

    if args.stream:
        return bench_stream(args)
    if args.pack:
        return bench_pack(args)
    if args.topk:
        return bench_topk(args)

    import torch

    from hybrid_sparse_mqa_amd import (dsv4_attn_forward, dsv4_attn_plan, dsv4_attn_set_kernel,
                                       dsv4_attn_set_split_keys, dsv4_attn_timing_enable, dsv4_attn_timing_read)
    from synth import make_config, tile_requests

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # Workload 5's call touches only ~4 MB per 8 requests, so its cold
    # rotation varies the C4 index lists (and Q) over disjoint sets drawn
    # from the same pools.  --batch B runs B/8 copies of the 8 requests, copy
    # k reading through its own index set (synth.tile_requests), so that the
    # batch sweep at 1M tokens needs no per-request pools.
    # For workloads 2-4, --batch B draws B requests of the same shape (a
    # batch sweep of the bf16 decode and verify kernels).
    copies = 1
    batch = None
    if args.batch:
        if args.config == 5 and args.batch % 8 == 0:
            copies = args.batch // 8
        elif args.config in (2, 3, 4) and args.batch > 0:
            batch = args.batch
        else:
            print("--batch applies to workloads 2-4 (any B > 0) and 5 (a multiple of 8)", file=sys.stderr)
            return 2
    idx_sets = 0
    if args.config == 5:
        # distinct bytes per rotation step: C4 rows (8 x 512 x 584 B) and Q per copy
        steps_needed = int(-(-3 * MALL_BYTES // (copies * (8 * 512 * 584 + 8 * 64 * 1024))))
        idx_sets = (args.sets or max(2, steps_needed)) * copies
    case = make_config(args.config, index_sets=max(1, idx_sets), batch=batch)
    if copies > 1:
        case = tile_requests(case, copies)
    ab = algorithmic_bytes(case)
    bf = torch.bfloat16

    def up(a, dt=None):
        if a is None:
            return None
        x = torch.from_numpy(np.ascontiguousarray(a))
        return (x.view(dt) if dt is not None else x).to(dev)

    def pool(a):
        return None if a is None else (up(a.view(np.int16), bf) if case.kv == "bf16" else up(a))

    base = dict(q=up(case.q.view(np.int16), bf), swa_pool=pool(case.swa_pool), extra_pool=pool(case.extra_pool))
    meta = dict(swa_page_table=up(case.swa_page_table), extra_page_table=up(case.extra_page_table),
                c4_indices=up(case.c4_indices), seq_lens=up(case.seq_lens), qo_indptr=up(case.qo_indptr),
                sink=up(case.sink))
    if idx_sets:
        # Same pools; per set its own Q copy and its own C4 index lists.
        c4_sets = case.meta["c4_sets"]
        n_sets = len(c4_sets)
        sets = [dict(q=base["q"] if i == 0 else base["q"].clone(), swa_pool=base["swa_pool"],
                     extra_pool=base["extra_pool"], c4_indices=up(c4_sets[i])) for i in range(n_sets)]
        # Distinct bytes per set: Q, out, lse, indices and the C4 rows (the
        # window rows are shared by every set).
        swa_kv = case.T * min(case.W, int(case.seq_lens.min())) * KV_ROW_BYTES[case.kv]
        cold = n_sets * (ab["total"] - swa_kv) > 2 * MALL_BYTES
    else:
        set_bytes = sum(x.numel() * x.element_size() for x in base.values() if x is not None)
        n_sets = args.sets or int(min(64, max(2, -(-3 * MALL_BYTES // max(ab["total"], 1)))))
        n_sets = max(1, min(n_sets, int((48 << 30) // max(set_bytes, 1))))
        sets = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()} for _ in range(n_sets - 1)]
        for st in sets:
            st["c4_indices"] = meta["c4_indices"]
        cold = n_sets * ab["total"] > 2 * MALL_BYTES
    outs = [torch.empty((case.T, case.H, 512), dtype=bf, device=dev) for _ in range(2)]
    lses = [torch.empty((case.T, case.H), dtype=torch.float32, device=dev) for _ in range(2)]

    if args.split_keys:
        dsv4_attn_set_split_keys(args.split_keys)
    if args.kernel:
        dsv4_attn_set_kernel(args.kernel)
    splits, chunk, kernel = dsv4_attn_plan(case.T, case.H, case.R, case.W, case.K,
                                   0 if case.extra_page_table is None else case.extra_page_table.shape[1],
                                   kv_fp8=case.kv == "fp8")

    def step(i):
        s = sets[i % n_sets]
        dsv4_attn_forward(s["q"], s["swa_pool"], meta["swa_page_table"], s["extra_pool"], meta["extra_page_table"],
                          s["c4_indices"], meta["seq_lens"], meta["qo_indptr"], meta["sink"], case.R, case.W,
                          case.scale, out=outs[i & 1], lse=lses[i & 1])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] workload {case.name}: T={case.T} H={case.H} splits={splits} keys/split={chunk} "
          f"sets={n_sets} ({'cold' if cold else 'warm'}) algorithmic {ab['total'] / 1e6:.2f} MB/call",
          file=sys.stderr, flush=True)

    # Kernel durations: a timed run of eager calls on the same rotating inputs,
    # each kernel bracketed by HIP events on the stream it runs on (the
    # library's timing hook).  The calls are queued behind a spin kernel that
    # outlasts the host's queueing, so that they run back to back and each
    # interval holds its kernel, not the host's launch gaps.
    n_eager = min(args.steps, 100)
    t0 = time.perf_counter()
    for i in range(n_eager):  # the host's queueing time (the GPU work is warm-up)
        step(i)
    host_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    sl0, sl1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sl0.record()
    torch.cuda._sleep(1 << 22)
    sl1.record()
    torch.cuda.synchronize()
    cycles_per_ms = (1 << 22) / max(sl0.elapsed_time(sl1), 1e-3)
    dsv4_attn_timing_read()  # clear
    torch.cuda._sleep(int(cycles_per_ms * (2.0 * host_ms + 2.0)))
    spin_end = torch.cuda.Event()
    spin_end.record()
    dsv4_attn_timing_enable(True)
    for i in range(n_eager):
        step(i)
    dsv4_attn_timing_enable(False)
    queued_ahead = not spin_end.query()  # the spin still ran when the last call was queued
    torch.cuda.synchronize()
    e_split, e_merge, e_calls = dsv4_attn_timing_read()
    if not queued_ahead:
        print("[bench] the host queued the timed eager calls slower than the spin kernel ran; "
              "their event intervals may hold launch gaps", file=sys.stderr)

    # Timed region: one replay of a HIP graph holding exactly `steps` calls
    # (rotating over the input sets), bracketed by two events.  Every N-th
    # call (--sample-every) is captured with the library's timing on, which
    # adds event-record nodes before its split kernel, between split and
    # merge kernel and after the merge kernel (for context: inside the graph
    # each interval also holds the nodes' own cost).
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    every = args.sample_every
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(args.steps):
                sampled = every > 0 and i % every == every // 2
                if sampled:
                    dsv4_attn_timing_enable(True)
                step(i)
                if sampled:
                    dsv4_attn_timing_enable(False)
        g.replay()  # warm replay (untimed)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        ev0.record(stream)
        g.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    event_ms = ev0.elapsed_time(ev1)
    g_split_ms, g_merge_ms, g_calls = dsv4_attn_timing_read()  # the timed replay's sampled calls
    expected = sum(1 for i in range(args.steps) if every > 0 and i % every == every // 2)
    if g_calls != expected or e_calls != n_eager or n_eager == 0:
        print(f"[bench] expected {n_eager} eager and {expected} sampled calls, the library recorded {e_calls} "
              f"and {g_calls}", file=sys.stderr)
        return 1

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    tokens_per_s = case.T / (ms_per_step / 1e3)
    split_avg_ms = e_split / n_eager
    merge_avg_ms = e_merge / n_eager
    kernel_bytes = ab["q"] + ab["idx"] + ab["kv"] + (ab["out"] + ab["lse"] if splits == 1 else 0)
    achieved = kernel_bytes / (split_avg_ms * 1e-3) / 1e9
    tflops = ab["flops"] / (split_avg_ms * 1e-3) / 1e12
    # The bound the split kernel sits under: HBM below the ridge point
    # (decode and verify), the bf16 MFMA peak above it (prefill: 2048 rows
    # per request bring 64 KiB of Q and of out per row and ~1 MFLOP per key).
    mfma_bound = ab["flops"] / max(kernel_bytes, 1) > RIDGE_FLOP_PER_BYTE
    kernel_name = split_kernel_name(kernel)

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE)).get(f"{kernel_name}/{case.name}")
        if rec and rec.get("kernel_sha") == kernel_sha() and rec.get("split_keys", 0) == args.split_keys:
            traffic = rec.get("hbm_bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": dict(describe_workload(args.config, case), splits=int(splits), keys_per_split=int(chunk),
                       heads_per_workgroup=SPLIT_KERNELS[kernel][1], split_kernel=kernel_name,
                       input_sets=int(n_sets), cache="cold-rotated" if cold else "warm-rotated",
                       rotation="C4 index lists and Q (window rows shared)" if idx_sets else "all inputs",
                       timed="HIP graph replay", parallelism="single GPU"),
        "path": {
            "algorithmic_bytes_per_call": ab["total"],
            "achieved_gbs_per_step": ab["total"] / (ms_per_step * 1e-3) / 1e9,
            "frac_per_step": ab["total"] / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "split_kernel_ms": split_avg_ms,
            "merge_kernel_ms": merge_avg_ms,
            "kernel_timing": f"HIP events around each kernel of {n_eager} eager calls queued back to back "
                             f"behind a spin kernel ({'queued ahead' if queued_ahead else 'NOT queued ahead'})",
            "kernels_per_step_frac": (split_avg_ms + merge_avg_ms) / ms_per_step,
            "graph_event_ms_per_step": event_ms / args.steps,
            "graph_sampled_calls": g_calls,
            "graph_sampled_split_interval_ms": g_split_ms / g_calls if g_calls else None,
            "graph_sampled_merge_interval_ms": g_merge_ms / g_calls if g_calls else None,
            "host_queue_ms_per_call": host_ms / n_eager,
        },
        "roofline": ({
            "bound": "mfma",
            "kernel": kernel_name,
            "achieved": tflops,
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": tflops / MFMA_BF16_PEAK_TFLOPS,
            "traffic": traffic,
            "algorithmic_flops_per_launch": ab["flops"],
            "algorithmic_bytes_per_launch": kernel_bytes,
            "hbm_gbs": achieved,
            "avg_launch_ms": split_avg_ms,
        } if mfma_bound else {
            "bound": "hbm",
            "kernel": kernel_name,
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kernel_bytes,
            "algorithmic_flops_per_launch": ab["flops"],
            "mfma_tflops": tflops,
            "avg_launch_ms": split_avg_ms,
        }),
        "cpu_baseline": None,
    }
    if not mfma_bound:
        # Context, not the roofline: the same bytes read by a plain streaming
        # kernel (no metadata, no arithmetic, no stores), timed the same way.
        pr_ms = plain_read_ms(kernel_bytes)
        result["roofline"]["plain_read_same_bytes"] = {
            "us": pr_ms * 1e3, "gbs": kernel_bytes / (pr_ms * 1e-3) / 1e9,
            "frac": kernel_bytes / (pr_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "split_kernel_vs_plain_read": pr_ms / split_avg_ms,
        }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, args.cpu_seconds)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
