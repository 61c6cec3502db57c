"""Benchmark of the MXFP4 routed-expert linear on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]          (the full suite)
    python bench.py --workload NAME [--steps K] [--warmup W]     (one workload)
    python bench.py --router softmax|sigmoid --workload NAME      (the router alone)

A step is one call of the whole layer (bucketing, dequant-GEMV or grouped
GEMM, combine) on one batch of the workload's synthetic inputs, all resident
in HBM before the timed region. Step i uses routing draw i mod R (R = 64
distinct (sel, p) draws for the decode-shaped workloads, 4 for the
prefill-shaped ones, which read every expert in every call), so consecutive
calls read different experts and the Infinity Cache cannot serve the weights
from the previous call.

The K timed steps are captured once in a HIP graph and replayed; the timed
region is bracketed by device synchronisation, and HIP events on the replay
stream give its duration. One JSON line goes to stdout; details to stderr.

Without --workload the line is the decode workload's (T1 E128 K4 G90 O5760,
fp32) and carries a "suite" object with one record per other workload
(tiny, decode8, prefill, skewed; each with its own roofline and oracle
baseline) and the plain streaming-read ceiling of the same bytes.

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
MFMA_FP4_PEAK_TFLOPS = 10066.4  # MI355X dense fp4 MFMA, published (both operands of the scaled MFMA in fp4)
N_ROUTING_SETS = 64
DECODE_WORKLOADS = ("tiny", "decode", "decode8")
KERNEL_SOURCES = {
    "gemv": ["mxfp4_block_scaled_amd/csrc/gemv_rows.hip", "mxfp4_block_scaled_amd/csrc/gemv_one.hip",
             "mxfp4_block_scaled_amd/csrc/device_common.h", "mxfp4_block_scaled_amd/csrc/wave_routing.h"],
    "gemm": ["mxfp4_block_scaled_amd/csrc/gemm_regdec.hip", "mxfp4_block_scaled_amd/csrc/device_common.h"],
    "swiglu": ["mxfp4_block_scaled_amd/csrc/gemm_regdec.hip", "mxfp4_block_scaled_amd/csrc/device_common.h"],
    "mx": ["mxfp4_block_scaled_amd/csrc/gemm_mx.hip", "mxfp4_block_scaled_amd/csrc/device_common.h"],
    "mx4": ["mxfp4_block_scaled_amd/csrc/gemm_mx.hip", "mxfp4_block_scaled_amd/csrc/device_common.h"],
    "gemmp": ["mxfp4_block_scaled_amd/csrc/gemm_regdec.hip", "mxfp4_block_scaled_amd/csrc/device_common.h"],
}
# the dominant kernel per path: bf16 prefill-shaped calls on canonical weights
# run the register-decode GEMM's canonical-layout instantiation
KERNEL_NAMES = {"gemv": "gemv_rows_kernel", "gemm": "gemm_regdec_kernel<0, true>",
                "gemmp": "gemm_regdec_kernel<0, false>"}


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
    kname = "gemv_one_kernel" if (kind == "gemv" and w.T == 1) else KERNEL_NAMES[kind]
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
    if variant in ("mxfp8", "mxfp4"):
        if w.F or w.dtype != "bf16":
            raise SystemExit("the block-scaled variants run the bf16 routed linear workloads only")
        return "mx" if variant == "mxfp8" else "mx4"
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
        rows_fn = {"mx": oracle.expert_linear_mxfp8_rows,
                   "mx4": oracle.expert_linear_mxfp4act_rows}.get(kind, oracle.expert_linear_rows)
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
    if kind == "mx4":
        return "MXFP4-activation variant (bucketing, quantisation, FP4 x FP4 scaled-MFMA grouped GEMM, combine)"
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

    def one_pass():
        if graph is not None:
            graph.replay()
        else:
            for i in range(args.steps):
                step(i)

    settle_passes(one_pass, stream, args.steps, args.settle_ms)
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


def host_info():
    """The host the oracle baseline runs on: cores this process may use, CPU
    model, the BLAS NumPy calls and its thread count."""
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", cores
    try:
        from threadpoolctl import threadpool_info

        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
            threads = int(libs[0].get("num_threads", cores))
    except Exception:  # threadpoolctl missing: BLAS unknown
        pass
    return {"host_cores": cores, "cpu_model": model, "blas": blas, "blas_threads": threads}


def device_info():
    import torch

    pr = torch.cuda.get_device_properties(0)
    info = {"name": pr.name, "arch": getattr(pr, "gcnArchName", "?"), "compute_units": pr.multi_processor_count}
    clk = getattr(pr, "clock_rate", None)
    if clk:
        info["clock_mhz"] = round(clk / 1000.0)
    return info


def _upload_experts(t, arr, E):
    for e in range(E):  # the expert tensors are drawn expert by expert
        t[e].copy_(torch_from(arr[e]))


def torch_from(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a))


def settle_passes(one_pass, stream, steps, settle_ms):
    """Untimed passes over the timed steps until about settle_ms have gone by,
    so that the timed region does not start on GPU clocks that are still
    ramping up after host-side work. Returns each pass's ms per step."""
    import torch

    per_step = []
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_ms * 1e-3:
        e_a, e_b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e_a.record(stream)
            one_pass()
            e_b.record(stream)
        torch.cuda.synchronize()
        per_step.append(e_a.elapsed_time(e_b) / steps)
    return per_step


def measure(args, w, kind, steps, warmup, cpu_seconds, n_sets):
    """Time `steps` graph-replayed calls of workload w on the path `kind`;
    returns the JSON record (without the top-level contract keys)."""
    import torch

    import mxfp4_block_scaled_amd as mx

    dev = torch.device("cuda:0")
    td = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    t_gen = time.perf_counter()
    inp = workloads.make_inputs(w, n_routing_sets=n_sets)
    packed = torch.empty(inp.packed.shape, dtype=torch.uint8, device=dev)
    scales = torch.empty(inp.scales.shape, dtype=torch.uint8, device=dev)
    _upload_experts(packed, inp.packed, w.E)
    _upload_experts(scales, inp.scales, w.E)
    dn_packed = dn_scales = None
    if kind in ("swiglu", "swiglup"):
        dn_packed = torch.empty(inp.dn_packed.shape, dtype=torch.uint8, device=dev)
        dn_scales = torch.empty(inp.dn_scales.shape, dtype=torch.uint8, device=dev)
        _upload_experts(dn_packed, inp.dn_packed, w.E)
        _upload_experts(dn_scales, inp.dn_scales, w.E)
    x = torch.from_numpy(inp.x).to(dev).to(td)
    shared = torch.from_numpy(inp.shared).to(dev).to(td)
    sels = torch.from_numpy(np.stack([s for s, _ in inp.routing_sets])).to(dev)
    ps = torch.from_numpy(np.stack([p for _, p in inp.routing_sets])).to(dev)
    y = torch.empty_like(shared)
    dt = 0 if w.dtype == "fp32" else 1
    if kind in ("swiglu", "swiglup"):
        ws_bytes = mx.swiglu_workspace_size(w.T, w.E, w.F, w.G, w.O, w.K)
    elif kind == "mx":
        ws_bytes = mx.mxfp8_workspace_size(w.T, w.E, w.O, w.G, w.K)
    elif kind == "mx4":
        ws_bytes = mx.mxfp4act_workspace_size(w.T, w.E, w.O, w.G, w.K)
    elif kind == "gemmp":
        ws_bytes = mx.workspace_size(w.T, w.E, w.O, w.G, w.K, mx.DTYPE_BF16, mx.FLAG_FORCE_GEMM)
    elif kind == "gemvp":
        ws_bytes = mx.workspace_size(w.T, w.E, w.O, w.G, w.K, dt, mx.FLAG_FORCE_GEMV)
    else:
        ws_bytes = mx.workspace_size(w.T, w.E, w.O, w.G, w.K, dt)
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
        r = i % n_sets
        if kind == "swiglu":
            mx.moe_swiglu(x, packed, scales, dn_packed, dn_scales, sels[r], ps[r], shared, out=y, workspace=ws)
        elif kind == "swiglup":
            mx.moe_swiglu_prepared(x, prepared, sels[r], ps[r], shared, out=y, workspace=ws)
        elif kind == "mx" and prepared is not None:
            mx.moe_linear_mxfp8_prepared(x, prepared, sels[r], ps[r], shared, out=y, workspace=ws)
        elif kind == "mx":
            mx.moe_linear_mxfp8(x, packed, scales, sels[r], ps[r], shared, out=y, workspace=ws)
        elif kind == "mx4" and prepared is not None:
            mx.moe_linear_mxfp4act_prepared(x, prepared, sels[r], ps[r], shared, out=y, workspace=ws)
        elif kind == "mx4":
            mx.moe_linear_mxfp4act(x, packed, scales, sels[r], ps[r], shared, out=y, workspace=ws)
        elif kind == "gemmp":
            mx.moe_linear_prepared(x, prepared, sels[r], ps[r], shared, out=y, workspace=ws)
        elif kind == "gemvp":
            mx.moe_decode_prepared(x, prepared, sels[r], ps[r], shared, out=y, workspace=ws)
        else:
            mx.moe_linear(x, packed, scales, sels[r], ps[r], shared, out=y, workspace=ws)

    # eager reference of the last timed step, for the graph replay check
    last = (steps - 1) % n_sets
    step(last)
    torch.cuda.synchronize()
    y_eager = y.clone()
    for i in range(warmup):
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
            for i in range(steps):
                step(i)
        graph.replay()
        torch.cuda.synchronize()
        if not torch.equal(y, y_eager):
            raise SystemExit(f"{w.name}: graph replay result differs from the eager call")
        log(f"[bench] {w.name}: graph replay matches the eager call bit for bit")

    def one_pass():
        if graph is not None:
            graph.replay()
        else:
            for i in range(steps):
                step(i)

    settle = settle_passes(one_pass, stream, steps, args.settle_ms)
    if settle:
        log(f"[bench] {w.name}: settle: {len(settle)} untimed passes, {settle[0] * 1e3:.2f} us/step first, "
            f"{settle[-1] * 1e3:.2f} us/step last")

    # timed region: HIP events recorded on the stream the kernels run on
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        ev0.record(stream)
        if graph is not None:
            graph.replay()
        else:
            for i in range(steps):
                step(i)
        ev1.record(stream)
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / steps
    if not torch.equal(y, y_eager):
        raise SystemExit(f"{w.name}: timed steps ended with a result that differs from the eager call")

    gemm_ms = None
    # the grouped GEMM alone (its stage entry points take bf16 activations);
    # fp32 activations: the whole call is timed
    if kind == "gemmp" or (kind == "gemm" and w.dtype == "bf16"):
        def gemm_alone():
            if kind == "gemmp":
                mx.gemm_stage_prepared(x, prepared, w.K, ws)
            else:
                mx.gemm_stage(x, packed, scales, w.K, ws)

        # the grouped GEMM alone, on the bucketing the last timed step left in
        # the workspace: `steps` launches captured in a graph, timed like the steps
        with torch.cuda.stream(stream):
            gemm_alone()
        torch.cuda.synchronize()
        g2 = None
        if graph is not None:
            g2 = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g2, stream=stream):
                for _ in range(steps):
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
                for _ in range(steps):
                    gemm_alone()
            e2b.record(stream)
        torch.cuda.synchronize()
        gemm_ms = e2a.elapsed_time(e2b) / steps
        log(f"[bench] {w.name}: grouped GEMM alone (routing draw {last}): {gemm_ms * 1e3:.1f} us per launch")

    uniq = [len(np.unique(inp.routing_sets[i % n_sets][0])) for i in range(steps)]
    bytes_per_step = float(np.mean(uniq)) * w.O * w.G * 17
    flops_per_step = 2.0 * w.P * w.O * w.I
    if kind in ("swiglu", "swiglup"):
        flops_per_step = 2.0 * w.P * (2 * w.F * w.I + w.O * w.F)
    extra = {}
    if kind in ("mx", "mx4"):
        # the variant's grouped GEMM on the scaled MFMA is its work; timed as
        # the whole call (bucketing, quantisation and combine included)
        value = flops_per_step / (ms_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        peak = MFMA_FP8_PEAK_TFLOPS if kind == "mx" else MFMA_FP4_PEAK_TFLOPS
        roof = {"bound": "mfma", "achieved": round(value, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(value / peak, 4)}
        roof["kernel"] = "gemm_mx_kernel<%s, %s> (whole call)" % ("true" if prepared is not None else "false",
                                                                  "true" if kind == "mx4" else "false")
        roof["launch_ms"] = round(ms_step, 6)
    elif kind in ("swiglu", "swiglup"):
        # the block's two grouped GEMMs are its work; timed here as the whole
        # call (bucketing and combine included), a lower bound on the GEMMs
        value = flops_per_step / (ms_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        roof = {"bound": "mfma", "achieved": round(value, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(value / MFMA_BF16_PEAK_TFLOPS, 4)}
        roof["kernel"] = ("gemm_regdec_kernel<1, false> + gemm_regdec_kernel<2, false> (whole call)"
                          if kind == "swiglup"
                          else "gemm_regdec_kernel<1, true> + gemm_regdec_kernel<2, true> (whole call)")
        roof["launch_ms"] = round(ms_step, 6)
    elif kind in ("gemv", "gemvp"):
        # one launch per step: the fused kernel is the whole call
        value = bytes_per_step / (ms_step * 1e-3) / 1e9
        unit = "GB/s"
        roof = {"bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(value / HBM_PEAK_GBS, 4)}
        roof["kernel"] = ("decode_fused_kernel<prepared>" if kind == "gemvp"
                          else "gemv_one_kernel" if w.T == 1 else KERNEL_NAMES["gemv"])
        roof["launch_ms"] = round(ms_step, 6)
        packed_only = float(np.mean(uniq)) * w.O * w.G * 16 / (ms_step * 1e-3) / 1e9
        extra["packed_only_GBs"] = round(packed_only, 1)
    else:
        value = flops_per_step / (ms_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        g_ms = gemm_ms if gemm_ms is not None else ms_step
        ach = flops_per_step / (g_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
        roof["kernel"] = KERNEL_NAMES[kind] if gemm_ms is not None else "gemm_bf16_kernel<0, 3> (whole call)"
        roof["launch_ms"] = round(g_ms, 6)
        extra["whole_call_frac"] = round(value / MFMA_BF16_PEAK_TFLOPS, 4)
        extra["weight_GBs_whole_call"] = round(w.E * w.O * w.G * 17 / (ms_step * 1e-3) / 1e9, 1) \
            if len(np.unique(inp.sel)) == w.E else None
    roof["per_launch"] = ({"bytes": bytes_per_step} if kind in ("gemv", "gemvp") else {"flops": flops_per_step})
    if kind in ("swiglu", "swiglup", "mx", "mx4", "gemvp"):
        roof["traffic"] = None
    else:
        roof["traffic"] = committed_traffic(w.name + ("-prepared" if kind == "gemmp" else ""), kind)
    log(f"[bench] {w.name}: {steps} steps in {ms_total:.3f} ms: {ms_step * 1e3:.2f} us/step, "
        f"{value:.1f} {unit} ({100 * roof['frac']:.1f}% of peak for the timed kernel); "
        f"mean distinct experts {np.mean(uniq):.1f}")
    rec = {
        "value": round(value, 2), "unit": unit, "ms_per_step": round(ms_step, 6), "steps": steps,
        "dtype": {"mx": "fp4xfp8", "mx4": "fp4xfp4"}.get(kind, "f32" if w.dtype == "fp32" else "bf16"),
        "config": {"workload": w.name + {"mx": "-mxfp8", "mx4": "-mxfp4"}.get(kind, "")
                               + ("-prepared" if prepared is not None else ""),
                   "T": w.T, "E": w.E, "K": w.K, "G": w.G, "I": w.I, "O": w.O,
                   **({"F": w.F} if w.F else {}),
                   "x_dtype": w.dtype, "routing": w.routing if w.routing == "uniform" else f"zipf({w.zipf_s})",
                   "routing_draws": n_sets, "graph": graph is not None},
        "path": _path_name(mx, w, kind),
        "roofline": roof, **extra,
    }
    if cpu_seconds > 0:
        cb = cpu_baseline(inp, kind, cpu_seconds)
        cb.update(host_info())
        rec["cpu_baseline"] = cb
        log(f"[bench] {w.name}: oracle on the host: {cb['value']:.4g} {cb['unit']} with {cb['cores']} threads "
            f"({cb['sample']})")
    del packed, scales, dn_packed, dn_scales, x, shared, sels, ps, y, ws, prepared, graph
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def stream_ceiling(window_bytes, steps, warmup, settle_ms):
    """The plain streaming-read kernel (mxfp4_stream_read) on windows of
    window_bytes taken in turn from a buffer of 64 such windows (larger than
    the Infinity Cache), in a graph of `steps` launches; and on one 1 GiB
    read. The practical read ceiling of the bytes a decode call moves."""
    import torch

    import mxfp4_block_scaled_amd as mx

    dev = torch.device("cuda:0")
    win = (int(window_bytes) + 4095) // 4096 * 4096
    n_win = 64
    buf = torch.randint(0, 255, (n_win * win,), dtype=torch.uint8, device=dev)
    sink = torch.zeros(65536, dtype=torch.int32, device=dev)
    out = {}
    for label, nbytes, views in (("decode_call_bytes", win, [buf[i * win:(i + 1) * win] for i in range(n_win)]),
                                 ("one_GiB", 1 << 30, [buf[:1 << 30]])):
        best = None
        for blocks in STREAM_BLOCKS:  # the best of a few grid sizes is the ceiling
            def step(i):
                mx.stream_read(views[i % len(views)], sink, blocks)

            for i in range(warmup):
                step(i)
            stream = torch.cuda.Stream(device=dev)
            stream.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(stream):
                step(0)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(steps):
                    step(i)
            g.replay()
            torch.cuda.synchronize()
            settle_passes(g.replay, stream, steps, settle_ms)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / steps
            if best is None or ms < best[0]:
                best = (ms, blocks)
            del g
        ms, blocks = best
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[label] = {"bytes": nbytes, "ms_per_launch": round(ms, 6), "GBs": round(gbs, 1),
                      "frac": round(gbs / HBM_PEAK_GBS, 4), "workgroups": blocks}
        log(f"[bench] streaming read of {nbytes / 1e6:.1f} MB: {ms * 1e3:.2f} us, {gbs:.0f} GB/s "
            f"({100 * gbs / HBM_PEAK_GBS:.1f}% of 8 TB/s; best of {len(STREAM_BLOCKS)} grids: {blocks} workgroups)")
    del buf, sink
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"kernel": "stream_read_kernel", **out}


def dense_gemm_ceiling(names, steps, settle_ms):
    """The vendor library's dense bf16 GEMM (torch.matmul on hipBLASLt) at
    each prefill workload's M = T K pairs, N = O, K = I, bf16 weights stored
    [O, I] like the experts' rows: no gather, no decode, no expert groups.
    A context figure for the grouped GEMM's MFMA fraction on this GPU (clock
    and power included), not part of the layer."""
    import torch

    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    out = {}
    for name in names:
        w = workloads.WORKLOADS[name]
        M, N, K = w.T * w.K, w.O, w.I
        a = torch.randn((M, K), generator=gen, device=dev, dtype=torch.bfloat16)
        wt = torch.randn((N, K), generator=gen, device=dev, dtype=torch.bfloat16)
        c = torch.empty((M, N), device=dev, dtype=torch.bfloat16)

        def one_pass():
            for _ in range(steps):
                torch.matmul(a, wt.t(), out=c)

        stream = torch.cuda.Stream(device=dev)
        stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(stream):
            one_pass()
        torch.cuda.synchronize()
        settle_passes(one_pass, stream, steps, settle_ms)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            one_pass()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        out[name] = {"M": M, "N": N, "K": K, "ms_per_launch": round(ms, 6), "TFLOPs": round(tf, 1),
                     "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}
        log(f"[bench] dense bf16 GEMM {M}x{N}x{K} (library): {ms * 1e3:.1f} us, {tf:.0f} TFLOP/s "
            f"({100 * tf / MFMA_BF16_PEAK_TFLOPS:.1f}% of the bf16 MFMA peak)")
        del a, wt, c
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"kernel": "torch.matmul (bf16, hipBLASLt)", **out}


SUITE = ("tiny", "decode8", "prefill", "skewed")
STREAM_BLOCKS = (512, 2048, 8192)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", choices=sorted(workloads.WORKLOADS),
                    help="time one workload (default: the decode workload, with the whole suite as sub-records)")
    ap.add_argument("--no-suite", action="store_true", help="without --workload: the decode workload only")
    ap.add_argument("--no-graph", action="store_true", help="time eager calls instead of a graph replay")
    ap.add_argument("--settle-ms", type=float, default=250.0,
                    help="untimed passes over the timed steps before the timed one, for about this long")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU work for the oracle baseline")
    ap.add_argument("--suite-cpu-seconds", type=float, default=4.0, help="CPU work per suite workload's baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="run only the copy calibration kernel of this size (for the byte counters)")
    ap.add_argument("--record-traffic", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="host only: turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs of --workload and of "
                         "the copy calibration (--copy-mib) into profiles/traffic.json")
    ap.add_argument("--variant", choices=["mxfp8", "mxfp4"],
                    help="time a block-scaled variant (activations quantised to MXFP8 or MXFP4, multiplied on "
                         "the scaled MFMA) instead of the layer")
    ap.add_argument("--prepared", action="store_true",
                    help="weights repacked once (outside the timed region) by prepare_bf16: the bf16 GEMM on "
                         "prepared weights, or with --variant the variant's")
    ap.add_argument("--router", choices=["softmax", "sigmoid"],
                    help="time the router alone at the workload's T, E and K instead of the layer")
    ap.add_argument("--stream", action="store_true", help="time only the plain streaming-read ceiling")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="time only the library's dense bf16 GEMM at the prefill workloads' sizes")
    args = ap.parse_args()
    if args.record_traffic:
        if args.copy_mib <= 0:
            raise SystemExit("--record-traffic needs the --copy-mib size the calibration ran with")
        if not args.workload:
            raise SystemExit("--record-traffic needs --workload")
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
        bench_router(args, workloads.WORKLOADS[args.workload or "decode"])
        return

    import torch

    torch.cuda.set_device(torch.device("cuda:0"))
    dec = workloads.WORKLOADS["decode"]
    if args.stream:
        st = stream_ceiling(dec.K * dec.O * dec.G * 17, args.steps, args.warmup, args.settle_ms)
        print(json.dumps({"stream_ceiling": st}), flush=True)
        return
    if args.gemm_ceiling:
        print(json.dumps({"dense_gemm_ceiling": dense_gemm_ceiling(("prefill", "skewed"), args.steps,
                                                                   args.settle_ms)}), flush=True)
        return
    suite = not args.workload and not args.no_suite
    w = workloads.WORKLOADS[args.workload or "decode"]
    kind = _kind(w, args.variant, args.prepared)
    n_sets = N_ROUTING_SETS if kind in ("gemv", "gemvp") else 4
    cpu_s = 0.0 if args.no_cpu_baseline else args.cpu_seconds
    rec = measure(args, w, kind, args.steps, args.warmup, cpu_s, n_sets)
    out = {
        "metric": METRIC, "value": rec["value"], "unit": rec["unit"], "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": rec["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": rec["dtype"], "data": "synthetic", "config": rec["config"],
        "roofline": rec["roofline"],
    }
    for key in ("packed_only_GBs", "whole_call_frac", "weight_GBs_whole_call", "cpu_baseline"):
        if key in rec:
            out[key] = rec[key]
    out["device"] = device_info()
    if suite:
        sub = {}
        sargs = argparse.Namespace(**{**vars(args), "prepared": False, "variant": None})
        for name in SUITE:
            sw = workloads.WORKLOADS[name]
            skind = _kind(sw)
            s_sets = N_ROUTING_SETS if skind == "gemv" else 4
            sub[name] = measure(sargs, sw, skind, args.steps, args.warmup,
                                0.0 if args.no_cpu_baseline else args.suite_cpu_seconds, s_sets)
        sub["stream_ceiling"] = stream_ceiling(dec.K * dec.O * dec.G * 17, args.steps, args.warmup, args.settle_ms)
        sub["dense_gemm_ceiling"] = dense_gemm_ceiling(("prefill", "skewed"), args.steps, args.settle_ms)
        out["suite"] = sub
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
