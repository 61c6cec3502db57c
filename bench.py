"""Benchmark of the MXFP4 routed-expert linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
    python bench.py --router softmax|sigmoid --workload NAME   (the router alone)

A step is one call of the whole layer (bucketing, dequant-GEMV or grouped
GEMM, combine) on one batch of the workload's synthetic inputs, all resident
in HBM before the timed region. Step i uses routing draw i mod R (R = 64
distinct (sel, p) draws), so consecutive calls read different experts and
the Infinity Cache cannot serve the weights from the previous call.

The K timed steps are captured once in a HIP graph and replayed; the timed
region is bracketed by device synchronisation, and HIP events on the replay
stream give its duration. One JSON line goes to stdout; details to stderr.

value:
  decode-shaped workloads: algorithmic weight bytes per second, where a call
    reads U * O * G * 17 bytes (16 packed + 1 scale byte per 32-weight
    group of each of the U distinct selected experts; 4.25 bits per weight);
  prefill-shaped workloads: 2 * T * K * O * I flops per second;
  the SwiGLU expert block: 2 * T * K * (2F * I + O * F) flops per second.
cpu_baseline: the float64 oracle timed on the host on a bounded sample of
  the same workload.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "packed-weight GB/s (decode) & TFLOP/s (prefill), % of MI355X roofline"
HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 MFMA, published
MFMA_FP8_PEAK_TFLOPS = 5033.2   # MI355X dense fp8 MFMA, published (the fp4 x fp8 scaled MFMA runs at this rate)
N_ROUTING_SETS = 64
DECODE_WORKLOADS = ("tiny", "decode", "decode8")
KERNEL_SOURCES = {
    "gemv": ["mxfp4_block_scaled_amd/csrc/gemv_rows.hip", "mxfp4_block_scaled_amd/csrc/device_common.h",
             "mxfp4_block_scaled_amd/csrc/wave_routing.h"],
    "gemm": ["mxfp4_block_scaled_amd/csrc/gemm.hip", "mxfp4_block_scaled_amd/csrc/device_common.h"],
    "swiglu": ["mxfp4_block_scaled_amd/csrc/gemm.hip", "mxfp4_block_scaled_amd/csrc/device_common.h"],
    "mx": ["mxfp4_block_scaled_amd/csrc/gemm_mx.hip", "mxfp4_block_scaled_amd/csrc/device_common.h"],
    "gemmp": ["mxfp4_block_scaled_amd/csrc/gemm_regdec.hip", "mxfp4_block_scaled_amd/csrc/device_common.h"],
}
KERNEL_NAMES = {"gemv": "gemv_rows_kernel", "gemm": "gemm_bf16_kernel", "gemmp": "gemm_regdec_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sources_sha(kind: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(workload: str, kind: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha") != sources_sha(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


def copy_calibration(mib: int, reps: int = 8):
    """A plain elementwise kernel of known traffic (reads and writes mib MiB
    per launch): the calibration run for the HBM byte counters."""
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} launches of a {mib} MiB read + {mib} MiB write")


def _counter_means(run_dir: str, counter: str, kernel_part: str):
    """Mean of one rocprofv3 counter over the dispatches of the kernels whose
    name contains kernel_part, from the counter_collection.csv files under
    run_dir."""
    import csv
    import glob

    vals = []
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") == counter and kernel_part in row.get("Kernel_Name", ""):
                    vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} values for kernels named *{kernel_part}* under {run_dir}")
    return float(np.mean(vals)), len(vals)


def record_traffic(args):
    """Turn four rocprofv3 --pmc runs (FETCH_SIZE and WRITE_SIZE of the
    workload's dominant kernel, the same two of the copy calibration) into
    HBM bytes per launch, stored in profiles/traffic.json with the hash of
    the kernel's sources; prints a summary."""
    w = workloads.WORKLOADS[args.workload]
    kind = "gemv" if args.workload in DECODE_WORKLOADS else ("gemmp" if args.prepared else "gemm")
    kname = KERNEL_NAMES[kind]
    fdir, wdir, cfdir, cwdir = args.record_traffic
    copy_kib = args.copy_mib * 1024.0
    k_fetch, n_f = _counter_means(fdir, "FETCH_SIZE", kname)
    k_write, n_w = _counter_means(wdir, "WRITE_SIZE", kname)
    c_fetch, _ = _counter_means(cfdir, "FETCH_SIZE", "neg_kernel")
    c_write, _ = _counter_means(cwdir, "WRITE_SIZE", "neg_kernel")
    f_fac, w_fac = copy_kib / c_fetch, copy_kib / c_write
    hbm = (k_fetch * f_fac + k_write * w_fac) * 1024.0
    rec = {"kernel": kname, "source_sha": sources_sha(kind), "hbm_bytes_per_launch": round(hbm),
           "fetch_kib_per_dispatch": round(k_fetch, 1), "write_kib_per_dispatch": round(k_write, 1),
           "dispatches": [n_f, n_w], "copy_mib": args.copy_mib,
           "copy_fetch_kib": round(c_fetch, 1), "copy_write_kib": round(c_write, 1),
           "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    key = w.name + ("-prepared" if kind == "gemmp" else "")
    allrec[key] = rec
    with open(path, "w") as f:
        json.dump(allrec, f, indent=1, sort_keys=True)
        f.write("\n")
    print(json.dumps({key: rec}))


def _kind(w, variant=None, prepared=False) -> str:
    if variant == "mxfp8":
        if w.F or w.dtype != "bf16":
            raise SystemExit("the MXFP8 variant runs the bf16 routed linear workloads only")
        return "mx"
    if w.F:
        return "swiglup" if prepared else "swiglu"
    if w.name in DECODE_WORKLOADS:
        return "gemvp" if prepared else "gemv"
    return "gemmp" if prepared else "gemm"


def cpu_baseline(inp, kind, sample_seconds):
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([int(i.get("num_threads", 1)) for i in threadpool_info()] + [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS threads unknown
        threads = os.cpu_count() or 1
    w = inp.workload
    if kind in ("swiglu", "swiglup"):
        # one token's full SwiGLU (all K pairs) on a sample of output rows
        rows_per_call = 16
        done_flops, calls, t0 = 0.0, 0, time.perf_counter()
        rng = np.random.default_rng(0)
        while True:
            t = calls % w.T
            rows = np.sort(rng.choice(w.O, rows_per_call, replace=False))
            oracle.expert_swiglu_rows(inp.x[t:t + 1], inp.packed, inp.scales, inp.dn_packed, inp.dn_scales,
                                      inp.sel[t:t + 1], inp.p[t:t + 1], inp.shared[t:t + 1], rows)
            done_flops += 2.0 * w.K * (2 * w.F * w.I + rows_per_call * w.F)
            calls += 1
            if time.perf_counter() - t0 >= sample_seconds:
                break
        dt = time.perf_counter() - t0
        return {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                "sample": f"{calls} tokens (all {w.K} pairs each) x {rows_per_call} output rows of the {w.name} "
                          "workload", "seconds": round(dt, 2)}
    if kind in ("gemv", "gemvp"):
        done_bytes, calls, t0 = 0.0, 0, time.perf_counter()
        while True:
            sel, p = inp.routing_sets[calls % len(inp.routing_sets)]
            oracle.expert_linear(inp.x, inp.packed, inp.scales, sel, p, inp.shared)
            done_bytes += len(np.unique(sel)) * w.O * w.G * 17
            calls += 1
            if time.perf_counter() - t0 >= sample_seconds:
                break
        dt = time.perf_counter() - t0
        return {"value": done_bytes / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": f"{calls} full calls of the {w.name} workload (routing draws 0..{calls - 1})",
                "seconds": round(dt, 2)}
    # prefill: all tokens, a sample of output rows
    rows_per_call = 16
    done_flops, calls, t0 = 0.0, 0, time.perf_counter()
    rng = np.random.default_rng(0)
    while True:
        rows = np.sort(rng.choice(w.O, rows_per_call, replace=False))
        rows_fn = oracle.expert_linear_mxfp8_rows if kind == "mx" else oracle.expert_linear_rows
        rows_fn(inp.x, inp.packed, inp.scales, inp.sel, inp.p, inp.shared, rows)
        done_flops += 2.0 * w.P * rows_per_call * w.I
        calls += 1
        if time.perf_counter() - t0 >= sample_seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{calls} x {rows_per_call} output rows of the {w.name} workload, all {w.T} tokens",
            "seconds": round(dt, 2)}


def _path_name(mx, w, kind) -> str:
    if kind == "mx":
        return "MXFP8 variant (bucketing, quantisation, scaled-MFMA grouped GEMM, combine)"
    if kind == "gemvp":
        return "decode-shaped MFMA kernel on prepared weights (routing, dequant-GEMV, combine in one launch)"
    if kind == "gemmp":
        return "GEMM on prepared weights (bucketing, register-decode grouped GEMM, combine)"
    if kind == "swiglu":
        return "SwiGLU block (bucketing, gate/up GEMM, down GEMM, combine)"
    if kind == "swiglup":
        return "SwiGLU block on prepared weights (bucketing, register-decode gate/up and down GEMMs, combine)"
    return "GEMV" if mx.select_path(w.T, w.E, w.O, w.G, w.K, 0 if w.dtype == "fp32" else 1) == 1 else "GEMM"


def bench_router(args, w):
    """The router alone (mxfp4_moe_route) at the workload's T, E and K.
    Algorithmic bytes per launch: the fp32 logits (T * E * 4), the bias
    (E * 4, sigmoid only) and the outputs (T * K * 8). Successive steps read
    different logits buffers, together larger than the 256 MB Infinity Cache,
    so the logits come from HBM."""
    import torch

    import mxfp4_block_scaled_amd as mx
    import oracle

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mode = args.router
    T, E, K = w.T, w.E, w.K
    per_set = T * E * 4
    n_sets = max(2, min(256, -(-512 * 2**20 // per_set)))
    t_gen = time.perf_counter()
    logits = torch.empty((n_sets, T, E), dtype=torch.float32, device=dev)
    host = []
    for i in range(n_sets):
        lg, bias = workloads.router_logits(T, E, seed=100 + i, std=2.0, bias_std=0.1 if mode == "sigmoid" else None)
        logits[i].copy_(torch.from_numpy(lg))
        if i == 0:
            host = (lg, bias)
    dbias = None if host[1] is None else torch.from_numpy(host[1]).to(dev)
    sel = torch.empty((T, K), dtype=torch.int32, device=dev)
    p = torch.empty((T, K), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"[bench] router {mode} at {w.name} (T={T} E={E} K={K}): {n_sets} logits buffers of "
        f"{per_set / 1e6:.1f} MB drawn in {time.perf_counter() - t_gen:.1f} s")

    def step(i):
        mx.route(logits[i % n_sets], K, mode, dbias, 1.0, sel=sel, p=p)

    step((args.steps - 1) % n_sets)
    torch.cuda.synchronize()
    sel_eager, p_eager = sel.clone(), p.clone()
    for i in range(args.warmup):
        step(i)
    stream = torch.cuda.Stream(device=dev)
    stream.wait_stream(torch.cuda.current_stream())
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            step(0)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(args.steps):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
        if not (torch.equal(sel, sel_eager) and torch.equal(p, p_eager)):
            raise SystemExit("graph replay result differs from the eager call")
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for i in range(args.steps):
                step(i)
        ev1.record(stream)
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    nbytes = T * E * 4 + (E * 4 if mode == "sigmoid" else 0) + T * K * 8
    value = nbytes / (ms_step * 1e-3) / 1e9
    roof = {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None, "kernel": "route_kernel",
            "launch_ms": round(ms_step, 6), "per_launch": {"bytes": nbytes}}
    log(f"[bench] router: {ms_step * 1e3:.2f} us per launch, {value:.1f} GB/s, "
        f"{T / (ms_step * 1e-3) / 1e6:.1f} M tokens/s")
    out = {
        "metric": f"router ({mode}) logits GB/s, % of HBM roofline", "value": round(value, 2), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"router-{mode}-{w.name}", "T": T, "E": E, "K": K, "logits_buffers": n_sets,
                   "graph": graph is not None},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        threads = os.cpu_count() or 1
        fn = (lambda: oracle.route_softmax(host[0], K)) if mode == "softmax" else \
             (lambda: oracle.route_sigmoid(host[0], host[1], K))
        calls, t0 = 0, time.perf_counter()
        while True:
            fn()
            calls += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(calls * nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "sample": f"{calls} full router calls on one logits buffer",
                               "seconds": round(dt, 2)}
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="decode", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--no-graph", action="store_true", help="time eager calls instead of a graph replay")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU work for the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run only the copy calibration kernel of this size (for the byte counters)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="host only: turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of --workload and of "
                         "the copy calibration (--copy-mib) into profiles/traffic.json")
    ap.add_argument("--variant", choices=["mxfp8"],
                    help="time the block-scaled variant (MXFP8 activations on the scaled MFMA) instead of the layer")
    ap.add_argument("--prepared", action="store_true",
                    help="weights repacked once (outside the timed region) by prepare_bf16: the bf16 GEMM on "
                         "prepared weights, or with --variant mxfp8 the variant's")
    ap.add_argument("--router", choices=["softmax", "sigmoid"],
                    help="time the router alone at the workload's T, E and K instead of the layer")
    args = ap.parse_args()
    if args.record_traffic:
        if args.copy_mib <= 0:
            raise SystemExit("--record-traffic needs the --copy-mib size the calibration ran with")
        record_traffic(args)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "multi-GPU runs are not part of this build.", file=sys.stderr)
        sys.exit(2)

    if args.copy_mib > 0:
        copy_calibration(args.copy_mib)
        return
    if args.router:
        bench_router(args, workloads.WORKLOADS[args.workload])
        return

    import torch

    import mxfp4_block_scaled_amd as mx

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.WORKLOADS[args.workload]
    kind = _kind(w, args.variant, args.prepared)
    td = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    t_gen = time.perf_counter()
    inp = workloads.make_inputs(w, n_routing_sets=N_ROUTING_SETS)
    packed = torch.empty(inp.packed.shape, dtype=torch.uint8, device=dev)
    scales = torch.empty(inp.scales.shape, dtype=torch.uint8, device=dev)
    for e in range(w.E):
        packed[e].copy_(torch.from_numpy(inp.packed[e]))
        scales[e].copy_(torch.from_numpy(inp.scales[e]))
    dn_packed = dn_scales = None
    if kind in ("swiglu", "swiglup"):
        dn_packed = torch.empty(inp.dn_packed.shape, dtype=torch.uint8, device=dev)
        dn_scales = torch.empty(inp.dn_scales.shape, dtype=torch.uint8, device=dev)
        for e in range(w.E):
            dn_packed[e].copy_(torch.from_numpy(inp.dn_packed[e]))
            dn_scales[e].copy_(torch.from_numpy(inp.dn_scales[e]))
    x = torch.from_numpy(inp.x).to(dev).to(td)
    shared = torch.from_numpy(inp.shared).to(dev).to(td)
    sels = torch.from_numpy(np.stack([s for s, _ in inp.routing_sets])).to(dev)
    ps = torch.from_numpy(np.stack([p for _, p in inp.routing_sets])).to(dev)
    y = torch.empty_like(shared)
    if kind in ("swiglu", "swiglup"):
        ws_bytes = mx.swiglu_workspace_size(w.T, w.E, w.F, w.G, w.O, w.K)
    elif kind == "mx":
        ws_bytes = mx.mxfp8_workspace_size(w.T, w.E, w.O, w.G, w.K)
    elif kind == "gemmp":
        ws_bytes = mx.workspace_size(w.T, w.E, w.O, w.G, w.K, mx.DTYPE_BF16, mx.FLAG_FORCE_GEMM)
    elif kind == "gemvp":
        ws_bytes = mx.workspace_size(w.T, w.E, w.O, w.G, w.K, 0 if w.dtype == "fp32" else 1, mx.FLAG_FORCE_GEMV)
    else:
        ws_bytes = mx.workspace_size(w.T, w.E, w.O, w.G, w.K, 0 if w.dtype == "fp32" else 1)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    prepared = None
    if args.prepared:
        prepared = (mx.prepare_swiglu(packed, scales, dn_packed, dn_scales) if kind == "swiglup"
                    else mx.prepare_bf16(packed, scales) if kind == "gemmp" else mx.prepare_mx(packed, scales))
    torch.cuda.synchronize()
    log(f"[bench] {w.name}: inputs drawn and resident in {time.perf_counter() - t_gen:.1f} s; "
        f"packed {packed.numel() / 1e9:.2f} GB, workspace {ws.numel() / 1e6:.1f} MB, "
        f"path {_path_name(mx, w, kind)}")

    def step(i):
        r = i % N_ROUTING_SETS
        if kind == "swiglu":
            mx.moe_swiglu(x, packed, scales, dn_packed, dn_scales, sels[r], ps[r], shared, out=y, workspace=ws)
        elif kind == "swiglup":
            mx.moe_swiglu_prepared(x, prepared, sels[r], ps[r], shared, out=y, workspace=ws)
        elif kind == "mx" and prepared is not None:
            mx.moe_linear_mxfp8_prepared(x, prepared, sels[r], ps[r], shared, out=y, workspace=ws)
        elif kind == "mx":
            mx.moe_linear_mxfp8(x, packed, scales, sels[r], ps[r], shared, out=y, workspace=ws)
        elif kind == "gemmp":
            mx.moe_linear_prepared(x, prepared, sels[r], ps[r], shared, out=y, workspace=ws)
        elif kind == "gemvp":
            mx.moe_decode_prepared(x, prepared, sels[r], ps[r], shared, out=y, workspace=ws)
        else:
            mx.moe_linear(x, packed, scales, sels[r], ps[r], shared, out=y, workspace=ws)

    # eager reference of the last timed step, for the graph replay check
    last = (args.steps - 1) % N_ROUTING_SETS
    step(last)
    torch.cuda.synchronize()
    y_eager = y.clone()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.Stream(device=dev)
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            step(0)  # the binding allocates nothing here; this call only settles the stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(args.steps):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(y, y_eager):
            raise SystemExit("graph replay result differs from the eager call")
        log("[bench] graph replay matches the eager call bit for bit")

    # timed region
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for i in range(args.steps):
                step(i)
        ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    if not torch.equal(y, y_eager):
        raise SystemExit("timed steps ended with a result that differs from the eager call")

    gemm_ms = None
    if kind in ("gemm", "gemmp"):
        def gemm_alone():
            if kind == "gemmp":
                mx.gemm_stage_prepared(x, prepared, w.K, ws)
            else:
                mx.gemm_stage(x, packed, scales, w.K, ws)

        # the grouped GEMM alone, on the bucketing the last timed step left in
        # the workspace: K launches captured in a graph, timed like the steps
        r_last = (args.steps - 1) % N_ROUTING_SETS
        with torch.cuda.stream(stream):
            gemm_alone()
        torch.cuda.synchronize()
        g2 = None
        if graph is not None:
            g2 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g2, stream=stream):
                for _ in range(args.steps):
                    gemm_alone()
            g2.replay()
            torch.cuda.synchronize()
        e2a = torch.cuda.Event(enable_timing=True)
        e2b = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e2a.record(stream)
            if g2 is not None:
                g2.replay()
            else:
                for _ in range(args.steps):
                    gemm_alone()
            e2b.record(stream)
        torch.cuda.synchronize()
        gemm_ms = e2a.elapsed_time(e2b) / args.steps
        log(f"[bench] grouped GEMM alone (routing draw {r_last}): {gemm_ms * 1e3:.1f} us per launch")

    uniq = [len(np.unique(inp.routing_sets[i % N_ROUTING_SETS][0])) for i in range(args.steps)]
    bytes_per_step = float(np.mean(uniq)) * w.O * w.G * 17
    flops_per_step = 2.0 * w.P * w.O * w.I
    if kind in ("swiglu", "swiglup"):
        flops_per_step = 2.0 * w.P * (2 * w.F * w.I + w.O * w.F)
    if kind == "mx":
        # the variant's grouped GEMM on the scaled MFMA is its work; timed as
        # the whole call (bucketing, quantisation and combine included)
        value = flops_per_step / (ms_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        roof = {"bound": "mfma", "achieved": round(value, 1), "peak": MFMA_FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(value / MFMA_FP8_PEAK_TFLOPS, 4)}
        roof["kernel"] = "gemm_mx_kernel<%s> (whole call)" % ("true" if prepared is not None else "false")
        roof["launch_ms"] = round(ms_step, 6)
    elif kind in ("swiglu", "swiglup"):
        # the block's two grouped GEMMs are its work; timed here as the whole
        # call (bucketing and combine included), a lower bound on the GEMMs
        value = flops_per_step / (ms_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        roof = {"bound": "mfma", "achieved": round(value, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(value / MFMA_BF16_PEAK_TFLOPS, 4)}
        roof["kernel"] = ("gemm_regdec_kernel<1> + gemm_regdec_kernel<2> (whole call)" if kind == "swiglup"
                          else "gemm_bf16_kernel<1> + gemm_bf16_kernel<2> (whole call)")
        roof["launch_ms"] = round(ms_step, 6)
    elif kind in ("gemv", "gemvp"):
        # one launch per step: the fused kernel is the whole call
        value = bytes_per_step / (ms_step * 1e-3) / 1e9
        unit = "GB/s"
        roof = {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(value / HBM_PEAK_GBS, 4)}
        roof["kernel"] = "decode_fused_kernel<prepared>" if kind == "gemvp" else "gemv_rows_kernel"
        roof["launch_ms"] = round(ms_step, 6)
    else:
        value = flops_per_step / (ms_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        ach = flops_per_step / (gemm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
        roof["kernel"] = KERNEL_NAMES[kind]
        roof["launch_ms"] = round(gemm_ms, 6)
    roof["per_launch"] = ({"bytes": bytes_per_step} if kind in ("gemv", "gemvp") else {"flops": flops_per_step})
    if kind in ("swiglu", "swiglup", "mx", "gemvp"):
        roof["traffic"] = None
    else:
        roof["traffic"] = committed_traffic(w.name + ("-prepared" if kind == "gemmp" else ""), kind)
    log(f"[bench] {args.steps} steps in {ms_total:.3f} ms: {ms_step * 1e3:.2f} us/step, "
        f"{value:.1f} {unit} ({100 * roof['frac']:.1f}% of peak); mean distinct experts {np.mean(uniq):.1f}")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp4xfp8" if kind == "mx" else ("f32" if w.dtype == "fp32" else "bf16"),
        "data": "synthetic",
        "config": {"workload": w.name + ("-mxfp8" if kind == "mx" else "") + ("-prepared" if prepared is not None else ""),
                   "T": w.T, "E": w.E, "K": w.K, "G": w.G, "I": w.I, "O": w.O,
                   **({"F": w.F} if w.F else {}),
                   "x_dtype": w.dtype, "routing": w.routing if w.routing == "uniform" else f"zipf({w.zipf_s})",
                   "routing_draws": N_ROUTING_SETS, "graph": graph is not None},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(inp, kind, args.cpu_seconds)
        out["cpu_baseline"] = cb
        log(f"[bench] oracle on the host: {cb['value']:.4g} {cb['unit']} with {cb['cores']} threads ({cb['sample']})")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
