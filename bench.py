"""Benchmark of DFlash block attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c3_global_d512]

A step is one whole dflash_block_attn call (attention kernel + split-KV
combine) over one batch of the named synthetic workload, inputs resident in
HBM.  Between steps a 1 GiB buffer is read by the library's streaming-read
kernel (outside the timed events) so that the 256 MB Infinity Cache does not
hold K/V from the previous step.  The flush only reads: a flush that writes
leaves up to 256 MB of dirty lines whose write-back would then be charged to
the timed kernel.  The same streaming read, timed, is the measured achievable
read bandwidth the K/V rate is also compared with.

The K timed steps run the call as a user would, with no events inside it;
each is followed by one more call (flushed the same way) that records events
around the attention kernel alone, for the kernel's duration (each recorded
event adds about 6 us between kernels, which is why the call is not timed
from those calls).

Printed (one JSON line): query-tokens/s over the timed steps, the achieved
K/V HBM bandwidth of the attention kernel against the 8 TB/s peak and against
the measured streaming read, and the fp64 CPU oracle timed on a bounded sample
of the same workload.

    python bench.py --graph-latency
measures one draft step (block K/V append + attention, one call) at the
block-aligned capture sizes 9/18/36/72 (B = 1/2/4/8 requests x block 9) for
the C1 and C2 request shapes, launched eagerly and as a replayed HIP graph;
it prints its own JSON line instead of the throughput line.

    python bench.py --conv
times DFlash2's in-block grouped dynamic depthwise convolution (dflash_block_conv)
at draft-step shapes and prints its own JSON line.

    python bench.py --summarize-pmc FETCH_CSV WRITE_CSV
turns two rocprofv3 counter runs of this script (FETCH_SIZE, then WRITE_SIZE)
into the HBM-traffic record the "traffic" field reads.

    python bench.py --summarize-trace KERNEL_TRACE_CSV
prints kernel durations from a rocprofv3 kernel trace, per kernel and per phase.
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

METRIC = "query-tokens/s + K/V HBM GB/s (% of peak) for block attention, 1 MI355X"
HBM_PEAK_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_mfma_c3_global_d512.json")
FLUSH_BYTES = 1 << 30
SETTLE_STEPS = 25  # untimed steps (warm-up included) before the timed ones
KERNEL_SOURCES = ["attn_mfma_kernel.h", "attn_mfma.hip", "device_common.h", "decomp.h", "merge.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "non_causal_block_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def visible_kv_bytes(wl) -> int:
    """Algorithmic K/V bytes: every key some query of the block can see, K and V
    rows of every kv-head read once.  With a window only keys from the first
    query's window start onward count; otherwise all L + n keys."""
    import numpy as np

    L = wl.ctx_lens.astype(np.int64)
    n = wl.block_lens.astype(np.int64)
    lo = np.maximum(0, L - wl.window + 1) if wl.window > 0 else np.zeros_like(L)
    U = np.where(n > 0, L + n - lo, 0)
    return int(U.sum()) * wl.Hkv * wl.D * 2 * 2


def cpu_model() -> str:
    """The host CPU's model name (Linux), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s: float = 12.0, spans=None) -> dict:
    """The fp64 oracle (unchanged) on a bounded sample of the workload's rows (with the
    call's bidirectional spans, if any)."""
    import numpy as np

    import oracle

    # the oracle library is compiled before the GPU is touched (main); a compiler must not
    # be started from this process now
    if not oracle.is_built():
        raise RuntimeError("the oracle library is missing or stale; build it before initialising the GPU")
    threads = oracle.default_threads()
    rng = np.random.default_rng(0)
    all_rows = wl.total_q * wl.Hq
    # calibrate on a few rows, then size the sample for ~budget_s of work
    probe = rng.choice(all_rows, size=min(all_rows, max(threads, 8)), replace=False)
    t0 = time.perf_counter()
    oracle.run_workload(wl, rows=probe, threads=threads, spans=spans)
    dt = max(time.perf_counter() - t0, 1e-4)
    per_row = dt / len(probe)
    n_rows = int(min(all_rows, max(len(probe), budget_s / per_row)))
    rows = np.sort(rng.choice(all_rows, size=n_rows, replace=False))
    t0 = time.perf_counter()
    oracle.run_workload(wl, rows=rows, threads=threads, spans=spans)
    dt = time.perf_counter() - t0
    tokens = n_rows / wl.Hq  # one query token = Hq output rows
    return {"value": tokens / dt, "unit": "query-tokens/s", "cores": threads, "kind": "oracle", "cpu": cpu_model(),
            "sample": f"{n_rows} of {all_rows} (token, q-head) output rows drawn uniformly from {wl.name}"
                      f"{' with its spans' if spans is not None else ''}, fp64, {dt:.1f} s on {threads} threads"}


def traffic_for(kernel_hash: str, launches_bytes: float):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they were
    taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    if rec.get("kernel_sha") != kernel_hash:
        return None
    return rec.get("bytes_per_launch")


def _pmc_means(path: str, counter: str) -> dict:
    """Mean counter value per dispatch, per kernel name, from a rocprofv3 counter CSV."""
    import csv

    acc = {}
    with open(path) as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            acc.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_trace(csv_path: str) -> dict:
    """Kernel durations from a rocprofv3 --kernel-trace CSV, per kernel name and per
    phase (phases are separated by idle gaps of more than 5 ms, e.g. the eager calls
    and the graph replays of --graph-latency)."""
    import csv

    import numpy as np

    rows = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"])
                  for r in csv.DictReader(open(csv_path)))
    phases, cur, last_end = [], [], None
    for s, e, n in rows:
        if last_end is not None and s - last_end > 5_000_000:
            phases.append(cur)
            cur = []
        cur.append((s, e, n))
        last_end = e if last_end is None else max(last_end, e)
    phases.append(cur)
    out = []
    for i, ph in enumerate(phases):
        per = {}
        for s, e, n in ph:
            per.setdefault(n.split("(")[0][:120], []).append((e - s) / 1e3)
        out.append({"phase": i, "kernels": {n: {"count": len(v), "mean_us": float(np.mean(v)),
                                                "median_us": float(np.median(v)),
                                                "p10_us": float(np.percentile(v, 10)),
                                                "p90_us": float(np.percentile(v, 90))} for n, v in per.items()}})
    return {"trace": csv_path, "phases": out}


def summarize_timeline(stamps, call_us, tile_bytes: int) -> dict:
    """Per-workgroup timeline of the attention kernel from the timeline build's stamps.

    stamps: [calls][P][8] of the 100 MHz wall clock (words 0-3: start, first tile
    loop, last tile loop end, end of the last epilogue; word 4: key tiles), call_us:
    the events around each of those calls.  Per call, medians over the workgroups
    that have tiles; reported as medians over calls.  Logical workgroup k runs on
    XCD k // (P / 8) when P is a multiple of 8 (the kernel's XCD-major order)."""
    import numpy as np

    S = np.asarray(stamps, dtype=np.float64)
    calls, P, _ = S.shape
    keys = ["setup_us", "loop_us", "per_tile_us", "per_tile_p90_us", "epilogue_us", "last_after_median_us",
            "span_us", "events_minus_span_us", "tiles_median", "tiles_max"]
    rows = {k: [] for k in keys}
    per_xcd = []
    for c in range(calls):
        s = S[c]
        t0 = s[s[:, 0] > 0, 0].min()
        rel = (s[:, :4] - t0) / 100.0
        tiles = s[:, 4]
        act = tiles > 0
        setup = rel[act, 1] - rel[act, 0]
        loop = rel[act, 2] - rel[act, 1]
        per_tile = loop / tiles[act]
        end = rel[s[:, 0] > 0, 3]
        rows["setup_us"].append(np.median(setup))
        rows["loop_us"].append(np.median(loop))
        rows["per_tile_us"].append(np.median(per_tile))
        rows["per_tile_p90_us"].append(np.percentile(per_tile, 90))
        rows["epilogue_us"].append(np.median(rel[act, 3] - rel[act, 2]))
        rows["last_after_median_us"].append(end.max() - np.median(end))
        rows["span_us"].append(end.max())
        rows["events_minus_span_us"].append(call_us[c] - end.max())
        rows["tiles_median"].append(np.median(tiles[act]))
        rows["tiles_max"].append(tiles.max())
        if P % 8 == 0:
            pt = np.full(P, np.nan)
            pt[act] = per_tile
            per = P // 8
            per_xcd.append([np.nanmedian(pt[x * per:(x + 1) * per]) for x in range(8)])
    out = {k: float(np.median(v)) for k, v in rows.items()}
    out["calls"] = calls
    out["workgroups"] = P
    out["call_us"] = float(np.median(call_us))
    out["loop_rate_gbps"] = P * tile_bytes / (out["per_tile_us"] * 1e-6) / 1e9
    if per_xcd:
        out["per_xcd_per_tile_us"] = [float(v) for v in np.median(np.asarray(per_xcd), axis=0)]
    return out


def gpu_info() -> dict:
    """Device name and CU count (no clocks: reading them would need a helper process,
    which must not be started from a process that has initialised the GPU)."""
    import torch

    props = torch.cuda.get_device_properties(0)
    return {"name": props.name, "cus": props.multi_processor_count}


def summarize_pmc(fetch_csv: str, write_csv: str, config: str) -> dict:
    """HBM bytes per launch of the attention kernel from FETCH_SIZE / WRITE_SIZE runs.

    Each counter (KiB per dispatch) is scaled by what it reads for a kernel of
    known size in the same run: the 1 GiB streaming-read flush for FETCH_SIZE,
    the 1 GiB fill that initialises the flush buffer for WRITE_SIZE."""
    import workloads

    fetch = _pmc_means(fetch_csv, "FETCH_SIZE")
    write = _pmc_means(write_csv, "WRITE_SIZE")

    def pick(table, key):
        names = [k for k in table if key in k]
        if len(names) != 1:
            raise SystemExit(f"expected one kernel matching {key!r}, found {names}")
        return names[0], table[names[0]]

    attn_name, attn_fetch = pick(fetch, "attn_mfma_kernel")
    _, attn_write = pick(write, "attn_mfma_kernel")
    _, read_cal = pick(fetch, "stream_read_kernel")
    _, write_cal = pick(write, "FillFunctor<float>")  # the flush buffer (float); other fills are tiny
    f_read = FLUSH_BYTES / (read_cal * 1024.0)
    f_write = FLUSH_BYTES / (write_cal * 1024.0)
    fetch_b = attn_fetch * 1024.0 * f_read
    write_b = attn_write * 1024.0 * f_write
    kv = visible_kv_bytes(workloads.make(config, poison=False))
    return {
        "kernel": attn_name, "workload": config, "kernel_sha": kernel_source_hash(),
        "fetch_kib_per_launch": attn_fetch, "write_kib_per_launch": attn_write,
        "read_calibration": {"kernel": "dflash stream_read", "known_bytes": FLUSH_BYTES, "fetch_kib": read_cal,
                             "factor": f_read},
        "write_calibration": {"kernel": "torch fill_ (flush buffer init)", "known_bytes": FLUSH_BYTES,
                              "write_kib": write_cal, "factor": f_write},
        "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
        "bytes_per_launch": fetch_b + write_b, "algorithmic_kv_bytes": kv,
        "over_fetch_ratio": fetch_b / kv,
    }


def _graph_node_types(graph) -> list:
    """Node types of a captured HIP graph (torch CUDAGraph kept with keep_graph=True),
    read with the HIP runtime torch loaded."""
    import ctypes

    import torch

    hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
    P = ctypes.c_void_p
    hip.hipGraphGetNodes.argtypes = [P, ctypes.POINTER(P), ctypes.POINTER(ctypes.c_size_t)]
    hip.hipGraphNodeGetType.argtypes = [P, ctypes.POINTER(ctypes.c_int)]
    names = {0: "kernel", 1: "memcpy", 2: "memset", 3: "host", 4: "graph", 5: "empty", 6: "wait_event",
             7: "event_record", 10: "mem_alloc", 11: "mem_free"}
    g = P(graph.raw_cuda_graph())
    n = ctypes.c_size_t(0)
    if hip.hipGraphGetNodes(g, None, ctypes.byref(n)) != 0:
        return ["?"]
    arr = (P * n.value)()
    hip.hipGraphGetNodes(g, arr, ctypes.byref(n))
    out = []
    for i in range(n.value):
        t = ctypes.c_int(-1)
        hip.hipGraphNodeGetType(arr[i], ctypes.byref(t))
        out.append(names.get(t.value, str(t.value)))
    return out


def graph_latency(reps: int = 200, only: str = "", layers: int = 1) -> dict:
    """Per-step latency of dflash_block_attn_append, eager vs graph replay.

    A step is ``layers`` consecutive calls (one per layer of a draft model; the
    same buffers serve every layer), made one by one from Python or captured
    together as one graph.  Each step is timed alone from the host (launch to
    completion, warm caches: a draft step re-reads the context it just read) and
    on the GPU (events).  The captured graph's node types are listed, and a
    control -- one trivial torch kernel, eager vs replayed graph -- measures what
    a graph replay costs on this runtime by itself.  ``only`` ("c1:1", ...)
    restricts the shapes."""
    import numpy as np
    import torch

    import non_causal_block_amd as nb
    import workloads

    dev = torch.device("cuda", 0)
    shapes = {  # request shapes of C1 and C2 (block 9 = 1 + 8 speculative tokens)
        "c1": dict(Hq=8, Hkv=2, D=128, ctx=lambda rng, B: np.full(B, 512)),
        "c2": dict(Hq=32, Hkv=8, D=256, ctx=lambda rng, B: rng.integers(1024, 4097, size=B)),
    }

    def t16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    side = torch.cuda.Stream()

    def timed(fn):
        host, gpu = [], []
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(reps + 10):
            t0 = time.perf_counter()
            e0.record(side)
            fn()
            e1.record(side)
            side.synchronize()
            t1 = time.perf_counter()
            if i >= 10:
                host.append((t1 - t0) * 1e6)
                gpu.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(host)), float(np.median(gpu))

    results = []
    for name, sh in shapes.items():
        for B in (1, 2, 4, 8):
            if only and f"{name}:{B}" != only:
                continue
            rng = np.random.default_rng(2000 + B)
            ctx = sh["ctx"](rng, B)
            wl = workloads.build(B, sh["Hq"], sh["Hkv"], sh["D"], ctx, np.full(B, 9), np.zeros(B, dtype=np.uint8),
                                 seed=2100 + B, poison=False)
            k_new, v_new, kc, vc = workloads.split_block_kv(wl)
            q, kn, vn, kp, vp = t16(wl.q), t16(k_new), t16(v_new), t16(kc), t16(vc)
            pt, cl, bl = (torch.from_numpy(a).to(dev) for a in (wl.page_table, wl.ctx_lens, wl.block_lens))
            out = torch.empty((wl.total_q, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
            desc = nb.make_desc(num_reqs=B, total_q=wl.total_q, max_block_len=9, total_kv_len=wl.total_kv,
                                page_size=wl.page_size, max_pages_per_req=wl.max_pages_per_req,
                                num_pages=wl.num_pages)
            ws = torch.zeros(max(nb.dflash_block_attn_workspace_size(desc, wl.Hq, wl.Hkv, wl.D), 256),
                             dtype=torch.uint8, device=dev)
            desc.workspace, desc.workspace_bytes = ws.data_ptr(), ws.numel()
            plan = nb.dflash_block_attn_plan(desc, wl.Hq, wl.Hkv, wl.D)

            def call_one():
                st = nb.dflash_block_attn_append(q, kn, vn, kp, vp, pt, cl, bl, wl.Hq, wl.Hkv, wl.D, None, 0,
                                                 wl.scale, out, side.cuda_stream, desc)
                if st != nb.DFLASH_OK:
                    raise nb.DFlashError(st, nb.dflash_last_error_message())

            def call():
                for _ in range(layers):
                    call_one()

            with torch.cuda.stream(side):
                for _ in range(10):
                    call()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph(keep_graph=True)
            with torch.cuda.graph(g, stream=side):
                call()
            g.instantiate()
            torch.cuda.synchronize()
            nodes = _graph_node_types(g)
            with torch.cuda.stream(side):
                eager_host, eager_gpu = timed(call)
                torch.cuda.synchronize()
                time.sleep(0.01)  # separates the eager calls from the replays in a kernel trace
                graph_host, graph_gpu = timed(g.replay)
            results.append({"shape": name, "B": B, "layers": layers, "query_tokens": wl.total_q, "Hq": wl.Hq,
                            "Hkv": wl.Hkv,
                            "head_dim": wl.D, "total_kv_tokens": wl.total_kv, "attn_workgroups": plan.num_workgroups,
                            "merge_in_kernel": bool(plan.merge_in_kernel), "graph_nodes": nodes,
                            "eager_us": eager_host, "graph_us": graph_host,
                            "eager_gpu_us": eager_gpu, "graph_gpu_us": graph_gpu})
            print(f"[graph] {name} B={B} x {layers} layer(s): eager {eager_host:.1f} us (gpu {eager_gpu:.1f}), "
                  f"graph {graph_host:.1f} us (gpu {graph_gpu:.1f}), nodes {nodes if layers == 1 else len(nodes)}",
                  file=sys.stderr, flush=True)
    # control: one trivial torch kernel, eager vs replayed graph
    x = torch.zeros(16, device=dev)
    with torch.cuda.stream(side):
        for _ in range(10):
            x.add_(1)
    torch.cuda.synchronize()
    gc = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gc, stream=side):
        x.add_(1)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        ctl_eager = timed(lambda: x.add_(1))
        ctl_graph = timed(gc.replay)
    control = {"what": "one trivial torch kernel (x.add_(1)), eager vs replayed graph",
               "eager_us": ctl_eager[0], "graph_us": ctl_graph[0], "eager_gpu_us": ctl_eager[1],
               "graph_gpu_us": ctl_graph[1]}
    print(f"[graph] control: eager gpu {ctl_eager[1]:.1f} us, graph gpu {ctl_graph[1]:.1f} us", file=sys.stderr,
          flush=True)
    return {"metric": f"draft-step latency: block K/V append + attention, {layers} call(s) per step, us (median)",
            "higher_is_better": False, "n_gpus": 1, "data": "synthetic", "reps": reps, "results": results,
            "control": control}


def conv_bench(reps: int = 200, cpu_baseline_leg: bool = True) -> dict:
    """DFlash2 block convolution: GPU time per call and algorithmic bytes per second.

    Shapes are readings (the pages give the formula, not the model sizes): blocks
    of 1 + 15 positions, 5120 channels in 32 groups, 16 taps (the whole block)."""
    import numpy as np
    import torch

    import non_causal_block_amd as nb
    import workloads

    dev = torch.device("cuda", 0)
    res = []
    for B in (8, 64):
        blocks = [16] * B
        C, G, taps = 5120, 32, 16
        x, base, delta = workloads.block_conv_inputs(blocks, C, G, taps, seed=3000 + B)

        def t16(a):
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

        tx, tb, td = t16(x), t16(base), t16(delta)
        bl = torch.tensor(blocks, dtype=torch.int32, device=dev)
        out = torch.empty_like(tx)
        stream = torch.cuda.current_stream(dev)
        for _ in range(10):
            nb.block_conv(tx, tb, td, bl, groups=G, out=out)
        # one call alone between two events: includes the launch reaching an idle GPU
        e0 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        e1 = [torch.cuda.Event(enable_timing=True) for _ in range(reps)]
        for i in range(reps):
            e0[i].record(stream)
            nb.block_conv(tx, tb, td, bl, groups=G, out=out)
            e1[i].record(stream)
        torch.cuda.synchronize()
        call_us = float(np.median([e0[i].elapsed_time(e1[i]) * 1e3 for i in range(reps)]))
        # calls back to back (the host runs ahead): GPU time per call in a stream of them
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(reps):
            nb.block_conv(tx, tb, td, bl, groups=G, out=out)
        b1.record(stream)
        torch.cuda.synchronize()
        b2b_us = b0.elapsed_time(b1) * 1e3 / reps
        # 20 calls captured in one HIP graph, replayed: GPU time per call without the host's
        # launch cost (a Python call here costs more host time than the kernel takes)
        per_graph, replays = 20, 20
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            nb.block_conv(tx, tb, td, bl, groups=G, out=out)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(per_graph):
                nb.block_conv(tx, tb, td, bl, groups=G, out=out)
        g.replay()
        torch.cuda.synchronize()
        b0.record(stream)
        for _ in range(replays):
            g.replay()
        b1.record(stream)
        torch.cuda.synchronize()
        us = b0.elapsed_time(b1) * 1e3 / (replays * per_graph)
        nbytes = (x.size + out.numel() + base.size + delta.size) * 2
        gbps = nbytes / (us * 1e-6) / 1e9
        row = {"B": B, "block": 16, "channels": C, "groups": G, "taps": taps, "gpu_us": us,
               "back_to_back_us": b2b_us, "call_us": call_us, "algorithmic_bytes": nbytes, "gbps": gbps,
               "positions_per_s": B * 16 / (us * 1e-6),
               "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                            "frac": gbps / HBM_PEAK_GBPS,
                            "basis": "algorithmic bytes (x, out, base, delta once) / GPU time per call in a "
                                     "replayed graph of 20 calls"}}
        if cpu_baseline_leg:
            # the sequential fp64 oracle on the same inputs (every position of the batch)
            from oracle.block_conv import block_conv_f64

            f = lambda a: (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
            xf, bf, df = f(x), f(base), f(delta)
            t0 = time.perf_counter()
            block_conv_f64(xf, bf, df, blocks, G)
            dt = time.perf_counter() - t0
            row["cpu_baseline"] = {"value": B * 16 / dt, "unit": "positions/s", "cores": 1, "kind": "oracle",
                                   "sample": f"all {B * 16} positions of the {B}-request batch, fp64 numpy, "
                                             f"{dt:.2f} s on one thread"}
        res.append(row)
        print(f"[conv] B={B}: {us:.1f} us per call in a graph of {per_graph} ({b2b_us:.1f} us back to back, "
              f"{call_us:.1f} us alone), {nbytes/1e6:.1f} MB -> {nbytes/(us*1e-6)/1e9:.0f} GB/s",
              file=sys.stderr, flush=True)
    # known-size traffic for scaling FETCH_SIZE / WRITE_SIZE in counter runs of this mode:
    # one fill of 256 MiB (a write) and one streaming read of it
    cal_bytes = 256 << 20
    cal = torch.empty(cal_bytes // 4, dtype=torch.float32, device=dev)
    cal.fill_(1.0)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    st = nb.dflash_stream_read(cal, cal_bytes, sink, stream.cuda_stream)
    if st != nb.DFLASH_OK:
        raise RuntimeError(f"stream_read failed: {nb.dflash_last_error_message()}")
    torch.cuda.synchronize()
    return {"metric": "DFlash2 in-block grouped dynamic depthwise convolution, GPU us per call (20 calls per replayed graph)",
            "higher_is_better": False, "n_gpus": 1, "data": "synthetic", "reps": reps, "results": res}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    # The attention kernel runs slower for the first ~30 flushed calls of a process on these
    # GPUs (a transient: C3 132-140 us per call, then 121-124 us from about call 40 on), so
    # the default warm-up (two calls per step) runs past it; with fewer warm-up steps the
    # bench adds untimed settle steps up to SETTLE_STEPS and reports them.
    ap.add_argument("--warmup", type=int, default=SETTLE_STEPS)
    ap.add_argument("--config", default="c3_global_d512")
    ap.add_argument("--kernel", choices=["auto", "mfma", "ref"], default="auto")
    ap.add_argument("--num-workgroups", type=int, default=0)
    ap.add_argument("--no-flush", action="store_true")
    ap.add_argument("--merge", choices=["auto", "combine", "in-kernel"], default="auto",
                    help="how split-KV pieces are merged (desc->merge_mode)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV")
    ap.add_argument("--graph-latency", action="store_true")
    ap.add_argument("--graph-shape", default="", help="with --graph-latency: only this shape, e.g. c1:1")
    ap.add_argument("--graph-reps", type=int, default=200)
    ap.add_argument("--graph-layers", type=int, default=1, help="with --graph-latency: calls per step (layers)")
    ap.add_argument("--conv", action="store_true")
    ap.add_argument("--spans", action="store_true",
                    help="call dflash_block_attn_spans with seeded bidirectional spans (causal requests)")
    ap.add_argument("--timeline", action="store_true",
                    help="per-workgroup timeline of the attention kernel (the timeline build of the library)")
    args = ap.parse_args(argv)

    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace), indent=1))
        return 0

    if args.summarize_pmc:
        rec = summarize_pmc(*args.summarize_pmc, args.config)
        rec["command"] = ("cd /tmp && rocprofv3 --pmc FETCH_SIZE (then WRITE_SIZE) --kernel-include-regex "
                          "'attn_mfma|stream_read|FillFunctor' -f csv -d <dir> -o run -- "
                          f"python3 bench.py --config {args.config} --steps 5 --warmup 2 --no-cpu-baseline")
        with open(TRAFFIC_FILE, "w") as fh:
            json.dump(rec, fh, indent=1)
        print(json.dumps(rec, indent=1))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the work shards by request / kv-head with no communication)", file=sys.stderr)
        return 2

    if not args.no_cpu_baseline and not (args.graph_latency or args.conv):
        # compile the oracle (if stale) now: a compiler must not be started from this
        # process once it has initialised the GPU
        import oracle

        oracle.build()

    import non_causal_block_amd as nb

    if args.timeline:
        # the library built with stamps; built (if missing) before this process touches the GPU
        if not os.path.exists(nb._lib.TIMELINE_LIB_PATH):
            from non_causal_block_amd import build as hipbuild
            hipbuild.build(timeline=True)
        nb._lib.LIB_PATH = nb._lib.TIMELINE_LIB_PATH

    import numpy as np
    import torch

    import workloads

    if args.graph_latency or args.conv:
        assert torch.cuda.is_available(), "bench.py needs a GPU"
        print(json.dumps(graph_latency(args.graph_reps, args.graph_shape, args.graph_layers) if args.graph_latency
                         else conv_bench(cpu_baseline_leg=not args.no_cpu_baseline)), flush=True)
        return 0

    if not os.path.exists(nb._lib.LIB_PATH):
        from non_causal_block_amd import build as hipbuild
        hipbuild.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda", 0)
    kernel = {"auto": nb.DFLASH_KERNEL_AUTO, "mfma": nb.DFLASH_KERNEL_MFMA, "ref": nb.DFLASH_KERNEL_REFERENCE}[
        args.kernel]

    print(f"[bench] generating {args.config}", file=sys.stderr, flush=True)
    wl = workloads.make(args.config, poison=False)

    def t16(x):
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)

    q, kp, vp = t16(wl.q), t16(wl.k_pages), t16(wl.v_pages)
    span_offs = span_tab = None
    n_spans = 0
    if args.spans:
        lists = workloads.draw_spans(wl.ctx_lens, wl.block_lens, seed=wl.seed + 7)
        offs = np.zeros(wl.B + 1, dtype=np.int32)
        offs[1:] = np.cumsum([len(x) for x in lists])
        flat = np.asarray([p for x in lists for p in x], dtype=np.int32).reshape(-1, 2)
        n_spans = int(flat.shape[0])
        span_offs = torch.from_numpy(offs).to(dev)
        span_tab = torch.from_numpy(np.ascontiguousarray(flat)).to(dev) if n_spans else None
    pt = torch.from_numpy(wl.page_table).to(dev)
    ctx = torch.from_numpy(wl.ctx_lens).to(dev)
    blk = torch.from_numpy(wl.block_lens).to(dev)
    causal = torch.from_numpy(wl.causal).to(dev)
    out = torch.empty((wl.total_q, wl.Hq, wl.D), dtype=torch.bfloat16, device=dev)
    desc = nb.make_desc(num_reqs=wl.B, total_q=wl.total_q, max_block_len=int(wl.block_lens.max()),
                        total_kv_len=wl.total_kv, page_size=wl.page_size, max_pages_per_req=wl.max_pages_per_req,
                        num_pages=wl.num_pages, kernel=kernel, num_workgroups=args.num_workgroups,
                        merge_mode={"auto": nb.DFLASH_MERGE_AUTO, "combine": nb.DFLASH_MERGE_COMBINE_KERNEL,
                                    "in-kernel": nb.DFLASH_MERGE_IN_KERNEL}[args.merge])
    plan = nb.dflash_block_attn_plan(desc, wl.Hq, wl.Hkv, wl.D)
    ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device=dev)
    desc.workspace, desc.workspace_bytes = ws.data_ptr(), ws.numel()
    flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush.fill_(1.0)  # also the known-size write the WRITE_SIZE counter is calibrated with
    sink = torch.zeros(1, dtype=torch.int32, device=dev)  # receives the XOR of each pass
    stream = torch.cuda.current_stream(dev)

    tl_buf, tl_snaps = None, []
    if args.timeline:
        tl_buf = torch.zeros(plan.num_workgroups * 8, dtype=torch.int64, device=dev)
        st = nb.dflash_timeline_set_buffer(tl_buf, tl_buf.numel() * 8)
        if st != nb.DFLASH_OK:
            raise nb.DFlashError(st, nb.dflash_last_error_message())

    def stream_read():
        st = nb.dflash_stream_read(flush, FLUSH_BYTES, sink, stream.cuda_stream)
        if st != nb.DFLASH_OK:
            raise nb.DFlashError(st, nb.dflash_last_error_message())

    n_ev = args.warmup + args.steps
    call0 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    call1 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    att0 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    att1 = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
    for ev in att0 + att1:
        ev.record(stream)  # torch creates the HIP event on first record; the library re-records it
    torch.cuda.synchronize()

    def step(i, instrumented):
        if not args.no_flush:
            stream_read()
        # The call's own throughput is timed without events inside it (each recorded event
        # adds a few microseconds between the kernels); the attention kernel's duration
        # comes from a second pass whose calls record events around that kernel.
        if instrumented:
            desc.event_attn_begin, desc.event_attn_end = att0[i].cuda_event, att1[i].cuda_event
        else:
            desc.event_attn_begin, desc.event_attn_end = None, None
            call0[i].record(stream)
        if args.spans:
            st = nb.dflash_block_attn_spans(q, kp, vp, pt, ctx, blk, wl.Hq, wl.Hkv, wl.D, causal, span_offs,
                                            span_tab, n_spans, wl.window, wl.scale, out, stream.cuda_stream, desc)
        else:
            st = nb.dflash_block_attn(q, kp, vp, pt, ctx, blk, wl.Hq, wl.Hkv, wl.D, causal, wl.window, wl.scale,
                                      out, stream.cuda_stream, desc)
        if not instrumented:
            call1[i].record(stream)
        if st != nb.DFLASH_OK:
            raise nb.DFlashError(st, nb.dflash_last_error_message())

    print(f"[bench] plan: kernel={plan.kernel} workgroups={plan.num_workgroups} rows/unit={plan.rows_per_unit} "
          f"merge_in_kernel={plan.merge_in_kernel} combine={plan.combine_workgroups} "
          f"workspace={plan.workspace_bytes}", file=sys.stderr, flush=True)
    settle = max(0, SETTLE_STEPS - args.warmup)
    for _ in range(settle):  # untimed, past the GPU's slow first calls (see --warmup)
        step(0, False)
        step(0, True)
    for i in range(args.warmup):
        step(i, False)
        step(i, True)
    torch.cuda.synchronize()
    # each timed step is followed by one instrumented call, so that both see the same
    # state of the chip (clocks drift over a run of back-to-back calls)
    t_wall0 = time.perf_counter()
    for i in range(args.warmup, n_ev):
        step(i, False)
        if tl_buf is not None:
            tl_snaps.append(tl_buf.clone())  # this call's stamps, before the next call's
        step(i, True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall0

    # measured achievable read bandwidth: the same streaming read, timed on its own
    sr0 = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    sr1 = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    for i in range(6):
        sr0[i].record(stream)
        stream_read()
        sr1[i].record(stream)
    torch.cuda.synchronize()
    stream_gbps = FLUSH_BYTES / (np.mean([sr0[i].elapsed_time(sr1[i]) for i in range(1, 6)]) / 1e3) / 1e9

    call_ms = np.array([call0[i].elapsed_time(call1[i]) for i in range(args.warmup, n_ev)])
    att_ms = np.array([att0[i].elapsed_time(att1[i]) for i in range(args.warmup, n_ev)])
    tokens = wl.total_q
    value = tokens * args.steps / (call_ms.sum() / 1e3)
    kv_bytes = visible_kv_bytes(wl)
    att_s = att_ms.mean() / 1e3
    achieved = kv_bytes / att_s / 1e9
    call_gbps = kv_bytes / (call_ms.mean() / 1e3) / 1e9
    print(f"[bench] call mean {call_ms.mean()*1e3:.1f} us (p10 {np.percentile(call_ms,10)*1e3:.1f}, "
          f"p90 {np.percentile(call_ms,90)*1e3:.1f}); attention kernel mean {att_ms.mean()*1e3:.1f} us; "
          f"K/V {kv_bytes/1e6:.1f} MB -> {achieved:.0f} GB/s kernel, {call_gbps:.0f} GB/s call; "
          f"wall {t_wall:.3f} s; streaming read {stream_gbps:.0f} GB/s", file=sys.stderr, flush=True)

    if tl_buf is not None:
        stamps = torch.stack(tl_snaps).view(len(tl_snaps), plan.num_workgroups, 8).cpu().numpy()
        tl = summarize_timeline(stamps, call_ms * 1e3, tile_bytes=plan.tile_keys * wl.D * 2 * 2)
        print(json.dumps({"workload": args.config, "build": "timeline (libdflash_attn_timeline.so)",
                          "kernel_sha": kernel_source_hash(), "attention_kernel_us": float(att_ms.mean() * 1e3),
                          "timeline": tl, "gpu": gpu_info()}), flush=True)
        return 0

    khash = kernel_source_hash()
    traffic = traffic_for(khash, kv_bytes)
    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(wl, spans=lists if args.spans else None)

    cfg = workloads.CONFIGS[args.config]
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle,
        "ms_per_step": float(call_ms.mean()),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": args.config, "description": cfg.description, "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv,
            "head_dim": wl.D, "query_tokens": tokens, "total_kv_tokens": wl.total_kv, "window": wl.window,
            "page_size": wl.page_size, "seed": wl.seed, "kernel": args.kernel,
            "attn_workgroups": plan.num_workgroups, "kv_bytes": kv_bytes,
            **({"spans": n_spans} if args.spans else {}),
        },
        "kv_hbm_gbps": call_gbps,
        "kv_hbm_frac_of_peak": call_gbps / HBM_PEAK_GBPS,
        "kv_hbm_basis": "whole dflash_block_attn call (attention + split-KV combine), mean over the timed calls",
        "stream_read_gbps": stream_gbps,
        "attn_kv_frac_of_stream_read": achieved / stream_gbps,
        "roofline": {
            "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
            "basis": "attention kernel alone: mean of HIP events around it on its launch stream",
            "call_frac": call_gbps / HBM_PEAK_GBPS,
            "kernel": "attn_mfma_kernel" if plan.kernel == nb.DFLASH_KERNEL_MFMA else "attn_ref_kernel",
            "kernel_sha": khash,
        },
        "cpu_baseline": cpu,
        "timing_us": {
            "call": {"mean": float(call_ms.mean() * 1e3), "median": float(np.median(call_ms) * 1e3),
                     "p10": float(np.percentile(call_ms, 10) * 1e3), "p90": float(np.percentile(call_ms, 90) * 1e3)},
            "attention_kernel": {"mean": float(att_ms.mean() * 1e3), "median": float(np.median(att_ms) * 1e3),
                                 "p10": float(np.percentile(att_ms, 10) * 1e3),
                                 "p90": float(np.percentile(att_ms, 90) * 1e3)},
        },
        "gpu": gpu_info(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
