#!/usr/bin/env python3
"""Bench of the W4A16 group-quantised linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--configs c3,c4,...]

A step is one call of w4a16_gemm on the headline layer: the 70B-class MLP
up-projection at decode batch one (M=1, K=8192, N=28672, group 128, asymmetric
int4), whose metric is HBM throughput.  The other layer configurations (the
1-4B decode layers, the batch sweep of the 70B layer, the M=2048 prefill GEMM and
the act-order layout) are timed the same way and reported alongside, each against
its own roofline.  Prints one JSON line.

Timing: all inputs are resident in device memory before the timed region; the
weights rotate over a pool of distinct copies larger than twice the 256 MB
Infinity Cache, so every step streams its weights from HBM.  HIP events recorded on
the launch stream bracket the whole timed region of back-to-back launches (the rate
and the per-launch mean) and, in a separate pass, every launch (event pairs, which
add the events' own overhead).  The headline layer is timed over exactly --steps
launches after --warmup; every other layer over a fixed 200 launches (or --steps if
larger) after 20 warm-up launches.  Before each timed region the layer runs back to
back while amd-smi reads the gfx and memory clocks (SCLK averaged over the XCDs, MCLK);
the line reports them with the device's name and compute-unit count.

Throughput figures use algorithmic bytes (packed codes, binary16 scales, packed
zero points, the act-order permutation, x and y) and algorithmic flops 2*M*N*K.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak, published
POOL_BYTES = 640 << 20         # > 2 x 256 MB Infinity Cache
MAX_COPIES = 64
METRIC = "W4A16 GEMV HBM GB/s (% of peak) at M=1; prefill GEMM TFLOP/s (% MFMA)"
HEADLINE = ("c3", 1)
SECONDARY_STEPS = 200          # launches per timed region of every other layer (at least)
SECONDARY_WARMUP = 20
SECONDARY = [("c1", 1), ("c2up", 1), ("c2down", 1), ("c3", 2), ("c3", 4), ("c3", 8), ("c3", 16),
             ("c3s", 1), ("c3w8", 1), ("c3w8", 16), ("c4", 2048), ("c4w8", 2048), ("c5", 1), ("c5", 512)]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
KERNEL_SOURCES = ["w4a16_gemm_amd/csrc/kernels/nibbles.hpp", "w4a16_gemm_amd/csrc/kernels/gemv.hpp",
                  "w4a16_gemm_amd/csrc/kernels/gemm.hpp", "w4a16_gemm_amd/csrc/kernels/skinny.hpp",
                  "w4a16_gemm_amd/csrc/kernels/aux.hpp", "w4a16_gemm_amd/csrc/device.hip"]


def algo_bytes(cfg: wl.LayerConfig, M: int) -> int:
    N, K, G, b = cfg.N, cfg.K, cfg.G, cfg.bits
    zeros = 0 if cfg.sym else G * N * b // 8
    return N * K * b // 8 + 2 * G * N + zeros + (4 * K if cfg.act_order else 0) + 2 * M * K + 2 * M * N


def algo_flops(cfg: wl.LayerConfig, M: int) -> int:
    return 2 * M * cfg.N * cfg.K


def kernel_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(msg: str) -> None:
    sys.stderr.write(f"[bench] {msg}\n")
    sys.stderr.flush()


def _amd_smi_clocks():
    """Current clocks from `amd-smi metric -c --json`: (mean gfx clock over the XCDs,
    memory clock) in MHz, or None where the tool or the field is missing."""
    import subprocess
    try:
        out = subprocess.run(["amd-smi", "metric", "-c", "--json", "-g", "0"], capture_output=True, text=True,
                             timeout=20)
        data = json.loads(out.stdout)
    except (OSError, ValueError, subprocess.SubprocessError):
        return None
    gpu = data[0] if isinstance(data, list) else (data.get("gpu_data") or [data])[0]
    clk = gpu.get("clock", {}) if isinstance(gpu, dict) else {}

    def val(entry):
        try:
            v = entry["clk"]["value"]
            return float(v) if v not in (None, "N/A") else None
        except (KeyError, TypeError, ValueError):
            return None
    gfx = [val(v) for k, v in clk.items() if k.startswith("gfx")]
    gfx = [g for g in gfx if g is not None]
    mem = [val(v) for k, v in clk.items() if k.startswith("mem")]
    mem = [m for m in mem if m is not None]
    return (round(sum(gfx) / len(gfx), 1) if gfx else None, mem[0] if mem else None)


def clocks_under_load(launch, sync, max_s: float = 20.0):
    """SCLK and MCLK while the timed work runs: the layer is launched back to back in
    batches of about 4 ms of device work (one synchronisation per batch, so the device
    is rarely idle), and after 1 s of that amd-smi queries run one after the other in a
    thread while the launches go on (not timed), until two consecutive readings agree."""
    import threading
    box = {}

    def query():
        # the tool's reading averages over a window that can still hold the idle time
        # before the launches (after seconds of host-side layer preparation the first
        # layer's readings came back at an idle-like 150-200 MHz): at least three readings,
        # then until two consecutive ones agree within 3% (at most six); the last is kept
        prev = None
        for i in range(6):
            clk = _amd_smi_clocks()
            box["clk"] = clk
            if not clk or clk[0] is None:
                return
            if i >= 2 and abs(clk[0] - prev) <= 0.03 * max(clk[0], prev):
                return
            prev = clk[0]
    t0 = time.perf_counter()
    for _ in range(8):
        launch(0)
    sync()
    per = max(1e-6, (time.perf_counter() - t0) / 8)     # upper bound of one launch's time
    batch = int(min(4096, max(64, 4e-3 / per)))
    i = 0
    th = threading.Thread(target=query)
    t0 = time.perf_counter()
    while (th.ident is None or th.is_alive()) and time.perf_counter() - t0 < max_s:
        for _ in range(batch):
            launch(i)
            i += 1
        sync()
        if th.ident is None and time.perf_counter() - t0 > 1.0:
            th.start()
    if th.ident is not None:
        th.join()
    clk = box.get("clk")
    return {"sclk_mhz": clk[0] if clk else None, "mclk_mhz": clk[1] if clk else None, "launches": i}


def device_info():
    import torch
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", None), "cus": p.multi_processor_count,
            "hbm_gib": round(p.total_memory / 2**30, 1)}


# --- GPU leg (the library only) ---------------------------------------------------

def prepare_layer(cfg: wl.LayerConfig, M_max: int):
    """Quantise, pack and upload a layer with the library's own host entry points."""
    import torch
    import w4a16_gemm_amd as w4
    dev = torch.device("cuda:0")
    g = cfg.group_size
    g_idx = s = None
    if cfg.act_order or cfg.awq:
        X = wl.calibration(cfg)
        g_idx = w4.w4a16_act_order(X, g) if cfg.act_order else None
        s = w4.w4a16_awq_scales(X) if cfg.awq else None
    eight = cfg.bits == 8
    if cfg.sym:
        codes, S = (w4.w8a16_quantize_sym if eight else w4.w4a16_quantize_sym)(wl.weights(cfg), g, g_idx, s)
        Z = None
    else:
        codes, S, Z = (w4.w8a16_quantize if eight else w4.w4a16_quantize)(wl.weights(cfg), g, g_idx, s)
    x = wl.activations(cfg, M_max)
    if s is not None:
        x = w4.w4a16_awq_fold_activations(x, s)
    return {
        "x": torch.from_numpy(x).to(dev),
        "qweight": torch.from_numpy((w4.w8a16_pack if eight else w4.w4a16_pack)(codes, g_idx, g)).to(dev),
        "scales": torch.from_numpy(S).to(dev),
        "qzeros": None if Z is None else torch.from_numpy((w4.w8a16_pack_zeros if eight else w4.w4a16_pack_zeros)(Z)).to(dev),
        "g_idx": None if g_idx is None else torch.from_numpy(g_idx).to(dev),
    }


def time_layer(cfg: wl.LayerConfig, M: int, layer, steps: int, warmup: int, sample_clocks: bool = True):
    if layer["x"].shape[0] < M or layer["x"].shape[1] != cfg.K:
        # the library takes raw pointers: a batch larger than the prepared activations
        # would read past their end
        raise ValueError(f"{cfg.name}: activations prepared for {tuple(layer['x'].shape)}, asked for M={M}, "
                         f"K={cfg.K}")
    import torch
    import w4a16_gemm_amd as w4
    lib = w4.lib()
    dev = layer["x"].device
    per_copy = algo_bytes(cfg, M) - 2 * M * cfg.K - 2 * M * cfg.N
    copies = max(1, min(MAX_COPIES, -(-POOL_BYTES // per_copy)))
    pool = [(layer["qweight"], layer["scales"], layer["qzeros"])]
    for _ in range(copies - 1):
        z = layer["qzeros"]
        pool.append((layer["qweight"].clone(), layer["scales"].clone(), None if z is None else z.clone()))
    x = layer["x"][:M].contiguous()
    y = torch.empty((M, cfg.N), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)
    gptr = None if layer["g_idx"] is None else layer["g_idx"].data_ptr()
    args = [(x.data_ptr(), q.data_ptr(), s.data_ptr(), None if z is None else z.data_ptr(), gptr, cfg.group_size,
             M, cfg.N, cfg.K, y.data_ptr(), stream.cuda_stream) for q, s, z in pool]

    gemm = lib.w8a16_gemm if cfg.bits == 8 else lib.w4a16_gemm

    def launch(i):
        rc = gemm(*args[i % len(args)])
        if rc != 0:
            raise RuntimeError(f"w4a16_gemm failed ({rc}): {lib.w4a16_last_error().decode()}")

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    clocks = clocks_under_load(launch, torch.cuda.synchronize) if sample_clocks else None
    # per-launch events (kernel time) ...
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        launch(warmup + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_launch_ms = [a.elapsed_time(b) for a, b in ev]
    # ... and the whole timed region without per-launch events (whole-job time)
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for i in range(steps):
        launch(i)
    r1.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    region_ms = r0.elapsed_time(r1)
    del pool
    return {
        "copies": copies,
        "event_pair_us_mean": 1e3 * statistics.fmean(per_launch_ms),
        "event_pair_us_median": 1e3 * statistics.median(per_launch_ms),
        "region_us_per_step": 1e3 * region_ms / steps,
        "wall_us_per_step": 1e6 * wall_s / steps,
        "launches_timed": steps,
        "clocks": clocks,
    }


def summarize(cfg, M, t):
    """Rates use the region events (back-to-back launches, no event between them);
    the per-launch event pairs add the events' own overhead and are reported aside."""
    us = t["event_pair_us_mean"]
    ur = t["region_us_per_step"]
    b = algo_bytes(cfg, M)
    f = algo_flops(cfg, M)
    out = {
        "workload": f"{cfg.name}: {cfg.note}", "M": M, "N": cfg.N, "K": cfg.K, "group": cfg.group_size,
        "act_order": cfg.act_order, "awq": cfg.awq, "sym": cfg.sym, "bits": cfg.bits,
        "us_per_layer": round(ur, 3),
        "event_pair_us_mean": round(us, 3), "event_pair_us_median": round(t["event_pair_us_median"], 3),
        "region_us_per_step": round(ur, 3), "launches_timed": t["launches_timed"],
        "algo_bytes": b, "algo_flops": f,
        "GBps": round(b / ur / 1e3, 1), "hbm_frac": round(b / ur / 1e3 / HBM_PEAK_GBS, 4),
        "TFLOPs": round(f / ur / 1e6, 2), "mfma_frac": round(f / ur / 1e6 / MFMA_F16_PEAK_TFLOPS, 4),
        "weight_copies": t["copies"],
    }
    if t.get("clocks"):
        out["sclk_mhz_under_load"] = t["clocks"]["sclk_mhz"]
        out["mclk_mhz_under_load"] = t["clocks"]["mclk_mhz"]
    return out


# --- CPU baseline (the oracle, as it stands) ----------------------------------------

def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_layer_legs(cfg: wl.LayerConfig, rows, repeats: int):
    """Times the oracle on one layer (or the first `rows` output rows of it): the
    offline quantiser once, the forward (binary64 dequant + numpy matmul) as the median
    of `repeats` runs on every allowed BLAS thread and once on one thread."""
    import oracle
    from threadpoolctl import threadpool_limits
    sel = np.arange(cfg.N if rows is None else rows)
    w = wl.weights(cfg, sel)
    s = oracle.awq_scales(wl.calibration(cfg)) if cfg.awq else None
    t0 = time.perf_counter()
    codes, S, Z = oracle.rtn_quantize(w, cfg.group_size, None, s)
    t_quant = time.perf_counter() - t0
    x = wl.activations(cfg, 1)
    if s is not None:
        x = oracle.awq_fold_activations(x, s)
    times = []
    for _ in range(repeats):
        t0 = time.perf_counter()
        oracle.linear(x, codes, S, Z, cfg.group_size)
        times.append(time.perf_counter() - t0)
    with threadpool_limits(limits=1, user_api="blas"):
        t0 = time.perf_counter()
        oracle.linear(x, codes, S, Z, cfg.group_size)
        t_one = time.perf_counter() - t0
    n = len(sel)
    nbytes = n * cfg.K // 2 + 2 * cfg.G * n + cfg.G * n // 2 + 2 * cfg.K + 2 * n
    return {"rows": n, "of_rows": cfg.N, "quantize_rtn_s": round(t_quant, 3),
            "forward_s_median": round(statistics.median(times), 3), "forward_s_1thread": round(t_one, 3),
            "forward_GBps": round(nbytes / statistics.median(times) / 1e9, 4), "algo_bytes_sample": nbytes}


def cpu_baseline(head: wl.LayerConfig, rows: int, repeats: int = 3):
    """The oracle as it stands, on the host cores of this machine: the headline layer on
    a bounded sample of its output rows, and the small decode layers whole."""
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        blas = 1
    cores = len(os.sched_getaffinity(0))
    legs = {head.name: _oracle_layer_legs(head, rows, repeats)}
    for name in ("c1", "c2up", "c2down"):
        legs[name] = _oracle_layer_legs(wl.CONFIGS[name], None, repeats)
    h = legs[head.name]
    return {
        "value": h["forward_GBps"], "unit": "GB/s", "cores": cores, "kind": "oracle",
        "sample": (f"oracle forward (binary64 dequant + numpy matmul) of the first {h['rows']} of {head.N} output "
                   f"rows of the {head.name} layer at M=1, median of {repeats}: {h['forward_s_median']:.2f} s; "
                   f"algorithmic bytes of the sample / time. The elementwise dequant runs on one thread, the "
                   f"matmul on {blas} BLAS threads"),
        "blas_threads": blas, "cpu_model": _cpu_model(),
        "seconds_per_layer_extrapolated": round(h["forward_s_median"] * head.N / h["rows"], 2),
        "legs": legs,
    }


def copy_probe(mib: int) -> None:
    """Three launches of a plain streaming kernel (binary16 negation) that read and
    write mib MiB each: the reference for scaling the FETCH_SIZE / WRITE_SIZE counters
    of a counter run to bytes."""
    import torch
    n = (mib << 20) // 2
    a = torch.ones(n, dtype=torch.float16, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.neg(a, out=b)
    torch.cuda.synchronize()
    log(f"copy probe: 3 launches of a binary16 negation over {mib} MiB in, {mib} MiB out")
    del a, b
    torch.cuda.empty_cache()


def dense_reference_us(cfg: wl.LayerConfig, M: int, iters: int = 30) -> float:
    """Kernel time of the same layer with dense binary16 weights through the vendor
    library (torch.matmul, hipBLASLt), x @ W^T with W [N][K] as stored: context for
    the W4A16 numbers (decode reads 4x the bytes; prefill is the same contraction
    without dequantisation).  Random operands; nothing of the W4A16 path is used."""
    import torch
    g = torch.Generator(device="cuda:0").manual_seed(0)
    w = torch.randn(cfg.N, cfg.K, generator=g, device="cuda:0", dtype=torch.float16)
    x = torch.randn(M, cfg.K, generator=g, device="cuda:0", dtype=torch.float16)
    for _ in range(5):
        torch.matmul(x, w.t())
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        torch.matmul(x, w.t())
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1000.0 / iters
    del w, x
    torch.cuda.empty_cache()
    return round(us, 3)


def decode_step_bench(step: wl.DecodeStep, steps: int = 100, warmup: int = 10):
    """One decode token at batch one of a whole model's quantised linear layers:
    step.layers x the step's linears, each layer with its own weights (distinct device
    copies, more than twice the Infinity Cache in all), launched back to back.  Timed
    eagerly (one library call per layer) and as one HIP graph replay per step; each
    linear shape also alone.  The unquantised head is timed through the vendor library
    as context.  Values of the weights do not change the work: they are uniform random
    packed words and scales (the parity of these shapes is a test)."""
    import torch
    import w4a16_gemm_amd as w4
    lib = w4.lib()
    dev = torch.device("cuda:0")
    g = step.group_size
    shapes = []
    for i, (name, K, N) in enumerate(step.linears):
        G = K // g
        qw = torch.from_numpy(wl.random_words(N, K // 8, seed=900 + i)).to(dev)
        sc = torch.from_numpy(wl.random_scales(G, N, seed=900 + i)).to(dev)
        qz = torch.from_numpy(wl.random_words(G, N // 8, seed=950 + i)).to(dev)
        copies = [(qw, sc, qz)] + [(qw.clone(), sc.clone(), qz.clone()) for _ in range(step.layers - 1)]
        x = torch.from_numpy(wl.random_activations(1, K, seed=i)).to(dev)
        y = torch.empty((1, N), dtype=torch.float16, device=dev)
        nbytes = N * K // 2 + 2 * G * N + G * N // 2 + 2 * K + 2 * N
        shapes.append({"name": name, "K": K, "N": N, "copies": copies, "x": x, "y": y, "bytes": nbytes})

    def call(sh, layer, stream):
        q, sc, z = sh["copies"][layer]
        rc = lib.w4a16_gemm(sh["x"].data_ptr(), q.data_ptr(), sc.data_ptr(), z.data_ptr(), None, g, 1,
                            sh["N"], sh["K"], sh["y"].data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"w4a16_gemm failed ({rc}): {lib.w4a16_last_error().decode()}")

    def one_step():
        st = torch.cuda.current_stream(dev).cuda_stream
        for layer in range(step.layers):
            for sh in shapes:
                call(sh, layer, st)

    def region(fn, n):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return 1e3 * a.elapsed_time(b) / n

    eager_us = region(one_step, steps)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one_step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        one_step()
    graph_us = region(graph.replay, steps)
    # each shape alone: its launches over the layers' distinct weights as one graph, so
    # that the host's launch rate does not enter the per-launch time
    per_linear = {}
    for sh in shapes:
        def shape_layers(sh=sh):
            st = torch.cuda.current_stream(dev).cuda_stream
            for layer in range(step.layers):
                call(sh, layer, st)
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            shape_layers()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g1):
            shape_layers()
        us = region(g1.replay, max(4, steps // 4)) / step.layers
        del g1
        per_linear[sh["name"]] = {"K": sh["K"], "N": sh["N"], "us": round(us, 3),
                                  "GBps": round(sh["bytes"] / us / 1e3, 1)}
    step_bytes = step.layers * sum(sh["bytes"] for sh in shapes)
    del graph, shapes
    torch.cuda.empty_cache()
    # the unquantised head (bfloat16, as the recipe keeps it), vendor library
    hk, hn = step.head
    gen = torch.Generator(device=dev).manual_seed(0)
    wh = torch.randn(hn, hk, generator=gen, device=dev, dtype=torch.bfloat16)
    xh = torch.randn(1, hk, generator=gen, device=dev, dtype=torch.bfloat16)
    head_us = region(lambda: torch.matmul(xh, wh.t()), 50)
    del wh, xh
    torch.cuda.empty_cache()
    return {
        "workload": step.note, "layers": step.layers,
        "linears": [f"{n} {k}->{m}" for n, k, m in step.linears], "group_size": g,
        "launches_per_step": step.layers * len(step.linears),
        "algo_bytes_per_step": step_bytes,
        "eager_us_per_step": round(eager_us, 2),
        "graph_us_per_step": round(graph_us, 2),
        "tokens_per_s_graph": round(1e6 / graph_us, 1),
        "GBps_graph": round(step_bytes / graph_us / 1e3, 1),
        "hbm_frac_graph": round(step_bytes / graph_us / 1e3 / HBM_PEAK_GBS, 4),
        "roofline_us_per_step": round(step_bytes / HBM_PEAK_GBS / 1e3, 2),
        "per_linear_alone": per_linear,
        "head_bf16_library_us": round(head_us, 2),
        "tokens_per_s_graph_with_head": round(1e6 / (graph_us + head_us), 1),
        "head_note": (f"unquantised {hk}->{hn} head in bfloat16 through torch.matmul (vendor library), "
                      "timed alone as context; not part of the W4A16 path"),
    }


def shards_bench(head_us: float, prefill_us):
    """One GPU's share of the layers under tensor parallelism, at its real shape (the
    layer shards without any exchange when split by output rows; the down projection of
    the same MLP splits by input channels, whole groups per GPU, and its partial outputs
    would be summed by one all-reduce, which is not run here).  Each share is timed like
    a secondary layer; `ideal_us` is the full layer's time divided by the degree."""
    import torch
    c3, c4 = wl.CONFIGS["c3"], wl.CONFIGS["c4"]
    cases = [("c3 up, column-parallel", c3, 1, c3.K, c3.N // p, p, head_us) for p in (2, 4, 8)]
    if prefill_us:
        cases.append(("c4 prefill, column-parallel", c4, 2048, c4.K, c4.N // 8, 8, prefill_us))
    cases += [("70B-class down (K=28672, N=8192), row-parallel", c3, 1, 28672 // p, 8192, p, None) for p in (8,)]
    out = []
    for i, (what, base, M, K, N, p, full_us) in enumerate(cases):
        cfg = wl.custom_config(f"shard{i}", 500 + i, K=K, N=N, group_size=base.group_size, M_list=(M,))
        layer = prepare_layer(cfg, M)
        t = time_layer(cfg, M, layer, SECONDARY_STEPS, SECONDARY_WARMUP, sample_clocks=False)
        r = summarize(cfg, M, t)
        out.append({"shard": what, "degree": p, "M": M, "K": K, "N": N, "us": r["us_per_layer"],
                    "GBps": r["GBps"], "TFLOPs": r["TFLOPs"],
                    "ideal_us": round(full_us / p, 3) if full_us else None})
        del layer
        torch.cuda.empty_cache()
    return out


def awq_search_bench(cfg: wl.LayerConfig, n_alpha: int = 11):
    """The AWQ alpha search on one layer with its calibration activations: wall time of
    the whole search and the device time of one candidate's W4A16 GEMM at M = T (the
    hot path inside it)."""
    import torch
    import w4a16_gemm_amd as w4
    w = wl.weights(cfg)
    X = wl.calibration(cfg)
    alphas = np.linspace(0.0, 1.0, n_alpha)
    w4.w4a16_awq_search(w, X[:8], cfg.group_size, alphas[:1])      # load, first-touch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    losses, best = w4.w4a16_awq_search(w, X, cfg.group_size, alphas)
    wall = time.perf_counter() - t0
    T = X.shape[0]
    layer = prepare_layer(wl.custom_config(cfg.name + "_cal", cfg.cfg_id, K=cfg.K, N=cfg.N,
                                           group_size=cfg.group_size, M_list=(T,)), T)
    t = time_layer(wl.custom_config(cfg.name + "_cal", cfg.cfg_id, K=cfg.K, N=cfg.N, group_size=cfg.group_size,
                                    M_list=(T,)), T, layer, 20, 5, sample_clocks=False)
    return {
        "workload": f"AWQ alpha search on the {cfg.name} layer (N={cfg.N}, K={cfg.K}, group {cfg.group_size}) "
                    f"with its {T} calibration tokens, {n_alpha} alphas on [0, 1]",
        "best_alpha": float(alphas[best]), "loss_best": float(losses[best]), "loss_alpha0": float(losses[0]),
        "wall_s": round(wall, 3), "wall_ms_per_alpha": round(1e3 * wall / n_alpha, 2),
        "gemm_us_per_alpha_M_T": round(t["region_us_per_step"], 2),
        "note": "per candidate: the scale on the host (exact mean over the calibration tokens), then "
                "quantisation and packing, the activation fold, one W4A16 GEMM at M = T and the reduction "
                "on the device",
    }


def gptq_bench(cfg: wl.LayerConfig):
    """GPTQ of one layer with its calibration activations in act order: wall time of the
    whole call (host inputs, device work, host outputs) and the layer's output error on
    the calibration rows against round-to-nearest, both measured on the host."""
    import torch
    import w4a16_gemm_amd as w4
    w = wl.weights(cfg)
    X = wl.calibration(cfg)
    w4.w4a16_gptq(w[:64, :256], X[:8, :256], 32, True)      # load, first-touch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    codes, S, Z, g_idx = w4.w4a16_gptq(w, X, cfg.group_size, True)
    wall = time.perf_counter() - t0
    rc, rs, rz = w4.w4a16_quantize(w, cfg.group_size, g_idx)
    Wd = w.astype(np.float32)
    Xd = X.astype(np.float32).T
    ref = Wd @ Xd

    def out_err(c, s_, z_):
        gid = g_idx.astype(np.int64)
        What = (c.astype(np.float32) - z_.astype(np.float32)[gid, :].T) * s_.astype(np.float32)[gid, :].T
        return float(np.linalg.norm(ref - What @ Xd) / np.linalg.norm(ref))
    T = X.shape[0]
    return {
        "workload": f"GPTQ of the {cfg.name} layer (N={cfg.N}, K={cfg.K}, group {cfg.group_size}, act order, "
                    f"damp 0.01) with its {T} calibration tokens",
        "wall_s": round(wall, 3),
        "output_error_gptq": round(out_err(codes, S, Z), 5),
        "output_error_rtn": round(out_err(rc, rs, rz), 5),
        "note": "whole call: uploads, H = 2XX^T, factorisation and triangular inverse (pivots in blocks of 64), "
                "the blocked rounding with error feedback, downloads; output error ||(W - W^) X|| / ||W X|| "
                "on the calibration rows (float32 on the host)",
    }


def measure_peaks(read_bytes: int = 1 << 30, steps: int = 20) -> dict:
    """What the part sustains on plain work (libw4a16_peaks.so): a non-temporal streaming
    read of a 1 GiB buffer (four times the Infinity Cache), best of a few grid sizes, and
    an MFMA loop of independent v_mfma_f32_32x32x16_f16 chains, two wavefronts per SIMD.
    Region events around `steps` back-to-back launches."""
    import ctypes
    import torch
    from w4a16_gemm_amd import build as _build
    lib = ctypes.CDLL(_build.PEAKS_LIB)
    lib.w4a16_peak_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_void_p]
    lib.w4a16_peak_mfma_f16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.w4a16_peaks_last_error.restype = ctypes.c_char_p
    stream = torch.cuda.current_stream()
    cus = torch.cuda.get_device_properties(0).multi_processor_count

    def region_us(launch) -> float:
        for _ in range(3):
            launch()
        torch.cuda.synchronize()
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0.record(stream)
        for _ in range(steps):
            launch()
        r1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * r0.elapsed_time(r1) / steps

    def check(rc):
        if rc != 0:
            raise RuntimeError(f"peak probe failed ({rc}): {lib.w4a16_peaks_last_error().decode()}")

    buf = torch.ones(read_bytes // 2, dtype=torch.float16, device="cuda:0")
    best = None
    for blocks in (cus, 2 * cus, 4 * cus, 8 * cus):
        out = torch.empty(blocks * 512, dtype=torch.int32, device="cuda:0")
        us = region_us(lambda: check(lib.w4a16_peak_stream_read(buf.data_ptr(), read_bytes, out.data_ptr(), blocks,
                                                                 stream.cuda_stream)))
        if best is None or us < best[0]:
            best = (us, blocks)
    del buf
    iters = 20000
    out = torch.empty(cus * 512, dtype=torch.float32, device="cuda:0")
    mus = region_us(lambda: check(lib.w4a16_peak_mfma_f16(out.data_ptr(), iters, cus, stream.cuda_stream)))
    flops = cus * 8 * iters * 4 * 32768
    return {
        "hbm_read_GBps": round(read_bytes / best[0] / 1e3, 1),
        "hbm_read_note": f"non-temporal 16-byte streaming read of {read_bytes >> 20} MiB, {best[1]} workgroups "
                         f"of 512 threads: {best[0]:.1f} us per launch",
        "mfma_f16_TFLOPs": round(flops / mus / 1e6, 1),
        "mfma_note": f"{cus} workgroups x 8 wavefronts x {iters} rounds of four independent 32x32x16 f16 MFMA "
                     f"chains: {mus:.1f} us per launch",
    }


def traffic_for(hash_now: str, key: str):
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    if data.get("kernel_hash") != hash_now:
        return None
    entry = data.get("entries", {}).get(key)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


# --- counter post-processing (rocprofv3 --pmc output; no GPU needed) ---------------

HEADLINE_KERNELS = {"c3:M1": "gemv_m1_kernelILi64ELi4ELi8ELi2ELb1ELb0ELi8ELi1ELi4ELb1E",
                    "c4:M2048": "gemm_big_kernelILi3ELi8ELi4ELb0E"}


def _counter_rows(d: str):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    per = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = (r["Kernel_Name"], int(r["Dispatch_Id"]))
            per.setdefault(key, {})
            per[key][r["Counter_Name"]] = per[key].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return per


def _means(per, match: str, skip: int = 5):
    """Mean of every counter over the dispatches of the kernel whose name contains
    `match` (the first `skip` warm-up dispatches left out)."""
    keys = sorted(k for k in per if match in k[0])
    if len(keys) > skip + 2:
        keys = keys[skip:]
    if not keys:
        return None, 0
    names = set().union(*(per[k].keys() for k in keys))
    return {c: statistics.fmean(per[k].get(c, 0.0) for k in keys) for c in names}, len(keys)


def summarize_pmc(dirs) -> None:
    """Per headline kernel: counters per dispatch and derived ratios (SIMD counters are
    summed over the device: 256 CUs x 4 SIMDs; GRBM_GUI_ACTIVE over the 8 XCDs)."""
    merged = {}
    for d in dirs:
        for k, v in _counter_rows(d).items():
            merged.setdefault(k, {}).update(v)
    for label, match in HEADLINE_KERNELS.items():
        m, n = _means(merged, match)
        if m is None:
            continue
        print(f"## {label}: {match}  ({n} dispatches)")
        for c in sorted(m):
            print(f"  {c:30s} {m[c]:.6g}")
        g = m.get("GRBM_GUI_ACTIVE")
        simd_cycles = g / 8 * 1024 if g else None
        if simd_cycles and "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            print(f"  => MFMA busy / SIMD cycles          {m['SQ_VALU_MFMA_BUSY_CYCLES'] / simd_cycles:.3f}")
        if m.get("SQ_VALU_MFMA_BUSY_CYCLES") and "SQ_VALU_MFMA_COEXEC_CYCLES" in m:
            print(f"  => VALU co-issue / MFMA busy        {m['SQ_VALU_MFMA_COEXEC_CYCLES'] / m['SQ_VALU_MFMA_BUSY_CYCLES']:.3f}")
        if m.get("SQ_INSTS_MFMA") and "SQ_INSTS_VALU" in m:
            print(f"  => non-MFMA VALU per MFMA           {(m['SQ_INSTS_VALU'] - m['SQ_INSTS_MFMA']) / m['SQ_INSTS_MFMA']:.3f}")
        if simd_cycles and "SQ_ACTIVE_INST_VALU" in m:
            print(f"  => VALU issue (x4 cycles) / SIMD cycles {4 * m['SQ_ACTIVE_INST_VALU'] / simd_cycles:.3f}")
        if m.get("SQ_WAVE_CYCLES"):
            for c in ("SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_LDS"):
                if c in m:
                    print(f"  => {c} / SQ_WAVE_CYCLES   {m[c] / m['SQ_WAVE_CYCLES']:.3f}")
        if m.get("SQ_LDS_IDX_ACTIVE") and "SQ_LDS_BANK_CONFLICT" in m:
            print(f"  => LDS bank-conflict / LDS active   {m['SQ_LDS_BANK_CONFLICT'] / m['SQ_LDS_IDX_ACTIVE']:.3f}")


def summarize_trace(trace_dir: str, steps: int) -> None:
    """Per headline kernel, from a `rocprofv3 --kernel-trace` of bench.py: the launches of
    the headline layer are the first run of at least 2 `steps` consecutive dispatches of
    that kernel with one grid; its last `steps` are the back-to-back timed region, the
    `steps` before them the launches with an event pair around each."""
    import csv
    import glob
    files = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    rows = []
    for f in files:
        for r in csv.DictReader(open(f)):
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size_X"]),
                         int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort()
    for label, match in HEADLINE_KERNELS.items():
        runs, cur = [], []
        for d in rows:
            if cur and (d[1] != cur[-1][1] or d[2] != cur[-1][2]):
                runs.append(cur)
                cur = []
            cur.append(d)
        runs.append(cur)
        run = next((r for r in runs if match in r[0][1] and len(r) >= 2 * steps), None)
        if run is None:
            print(f"## {label}: no run of {2 * steps} launches of {match}")
            continue
        b2b, pairs = run[-steps:], run[-2 * steps:-steps]
        print(f"## {label}: {run[0][1]} (grid {run[0][2]}, {len(run)} launches in the run)")
        print("| pass | launches | mean us | median us |\n|---|---|---|---|")
        for name, part in (("event pairs", pairs), ("back-to-back (timed region)", b2b)):
            us = [(e - s) / 1e3 for _, _, _, s, e in part]
            print(f"| {name} | {len(us)} | {statistics.fmean(us):.2f} | {statistics.median(us):.2f} |")
        print(f"\nfirst start to last end of the back-to-back launches / {steps}: "
              f"{(b2b[-1][4] - b2b[0][3]) / 1e3 / steps:.2f} us")
    probes = {}
    for _, name, grid, s, e in rows:
        if "stream_read_kernel" in name or "mfma_loop_kernel" in name:
            label = "stream_read_kernel" if "stream_read_kernel" in name else "mfma_loop_kernel"
            probes.setdefault((label, grid), []).append((e - s) / 1e3)
    if probes:
        print("## achievable-peak probes\n| kernel | grid (threads) | launches | mean us | min us |\n|---|---|---|---|---|")
        for (name, grid), us in sorted(probes.items()):
            print(f"| {name} | {grid} | {len(us)} | {statistics.fmean(us):.2f} | {min(us):.2f} |")


def write_traffic(fetch_dir: str, write_dir: str) -> None:
    """profiles/traffic_counters.json from a FETCH_SIZE and a WRITE_SIZE run of
    `bench.py --configs c3:1,c4:2048 --copy-probe-mib 512`: the counters of the plain
    streaming copy (binary16 negation, 512 MiB in and out) give the scale to bytes."""
    fetch, write = _counter_rows(fetch_dir), _counter_rows(write_dir)
    mib = 512
    cf, _ = _means(fetch, "neg", skip=0)
    cw, _ = _means(write, "neg", skip=0)
    if cf is None or cw is None:
        raise SystemExit("the calibration copy (a kernel named ...neg...) is missing from the runs")
    fetch_scale = (mib << 20) / (cf["FETCH_SIZE"] * 1024)
    write_scale = (mib << 20) / (cw["WRITE_SIZE"] * 1024)
    entries = {}
    for label, match in HEADLINE_KERNELS.items():
        mf, n = _means(fetch, match)
        mw, _ = _means(write, match)
        if mf is None or mw is None:
            continue
        name, M = label.split(":M")
        algo = algo_bytes(wl.config(name), int(M))
        hbm = mf["FETCH_SIZE"] * 1024 * fetch_scale + mw["WRITE_SIZE"] * 1024 * write_scale
        entries[label] = {"kernel_match": match, "dispatches": n, "fetch_kib": round(mf["FETCH_SIZE"], 1),
                          "write_kib": round(mw["WRITE_SIZE"], 1), "hbm_bytes_per_launch": int(round(hbm)),
                          "algo_bytes_per_launch": algo, "traffic_over_algo": round(hbm / algo, 4)}
    out = {"kernel_hash": kernel_hash(),
           "kernel_hash_note": "hash of the kernel sources listed in bench.KERNEL_SOURCES when the counters were taken",
           "fetch_scale": round(fetch_scale, 6), "write_scale": round(write_scale, 6),
           "calibration": f"binary16 negation kernel, {mib} MiB read + {mib} MiB written per launch",
           "entries": entries}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--configs", default="all", help="'all', 'headline' or a comma list like c3:1,c4:2048")
    ap.add_argument("--cpu-rows", type=int, default=4096, help="oracle sample size (rows of the headline layer)")
    ap.add_argument("--no-clocks", action="store_true", help="skip sampling SCLK/MCLK under load (amd-smi)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense-ref", action="store_true",
                    help="skip timing the dense binary16 library GEMM of the same shapes")
    ap.add_argument("--no-shards", action="store_true",
                    help="skip timing one GPU's share of the layers under tensor parallelism")
    ap.add_argument("--no-awq-search", action="store_true", help="skip timing the AWQ alpha search")
    ap.add_argument("--no-gptq", action="store_true", help="skip timing the GPTQ quantiser")
    ap.add_argument("--no-decode-step", action="store_true",
                    help="skip the whole-decode-step workload of the 1.5B example")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip measuring the achievable streaming-read and MFMA rates")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="first run a plain streaming kernel over this many MiB (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs="+", metavar="DIR",
                    help="print counter summaries of rocprofv3 --pmc output directories and exit (no GPU)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_counters.json from FETCH_SIZE / WRITE_SIZE runs and exit")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print the headline layers' launch times from a rocprofv3 --kernel-trace output "
                         "directory of a bench run with --steps as given, and exit (no GPU)")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, max(args.steps, SECONDARY_STEPS))
        return 0
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return 0
    if args.write_traffic:
        write_traffic(*args.write_traffic)
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (see the sharding notes); "
              "run it with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import w4a16_gemm_amd as w4
    w4.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if not args.no_clocks:
        _amd_smi_clocks()   # the tool's first reading can be stale: discard it
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)

    if args.configs == "all":
        todo = [HEADLINE] + SECONDARY
    elif args.configs == "headline":
        todo = [HEADLINE]
    else:
        todo = []
        for item in args.configs.split(","):
            name, m = item.split(":")
            todo.append((name, int(m)))

    results = {}
    layers = {}
    rows_needed = {}
    for name, M in todo:
        rows_needed[name] = max(rows_needed.get(name, 1), M, max(wl.config(name).M_list))
    for name, M in todo:
        cfg = wl.config(name)
        if name not in layers:
            layers.clear()
            torch.cuda.empty_cache()
            log(f"preparing {name} (N={cfg.N} K={cfg.K} g={cfg.group_size}, {rows_needed[name]} activation rows)")
            layers[name] = prepare_layer(cfg, rows_needed[name])
        if (name, M) == HEADLINE:
            steps, warm = args.steps, args.warmup
        else:   # fixed counts: the other layers do not shrink with --steps
            steps, warm = max(SECONDARY_STEPS, args.steps), max(SECONDARY_WARMUP, args.warmup)
        log(f"timing {name} M={M}: {warm} warmup + {steps} launches")
        t = time_layer(cfg, M, layers[name], steps, warm, sample_clocks=not args.no_clocks)
        results[f"{name}:M{M}"] = summarize(cfg, M, t)
        results[f"{name}:M{M}"]["_t"] = t
        log(f"  {results[f'{name}:M{M}']['us_per_layer']} us")
    layers.clear()

    hname = f"{HEADLINE[0]}:M{HEADLINE[1]}"
    if hname not in results:
        print(json.dumps({"configs": {k: {kk: vv for kk, vv in v.items() if kk != "_t"} for k, v in results.items()}}))
        return 0
    head = results[hname]
    hcfg = wl.CONFIGS[HEADLINE[0]]
    t = head.pop("_t")
    for v in results.values():
        v.pop("_t", None)
    khash = kernel_hash()

    line = {
        "metric": METRIC,
        "value": round(head["algo_bytes"] / t["region_us_per_step"] / 1e3, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t["region_us_per_step"] / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded; shapes and distributions of the layer configurations)",
        "config": {
            "workload": ("70B-class MLP up-projection decode layer: M=1, K=8192, N=28672, group 128, asymmetric "
                         "int4 weights (fp16 scale, 4-bit zero), fp16 activations, fp32 accumulation"),
            "M": 1, "K": hcfg.K, "N": hcfg.N, "group_size": hcfg.group_size,
            "weight_copies_rotated": head["weight_copies"],
            "accumulate": "f32",
        },
        "device": device_info(),
        "roofline": {
            "bound": "hbm",
            "achieved": round(head["algo_bytes"] / head["region_us_per_step"] / 1e3, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(head["algo_bytes"] / head["region_us_per_step"] / 1e3 / HBM_PEAK_GBS, 4),
            "traffic": traffic_for(khash, hname),
            "kernel": "gemv_m1_kernel",
            "launch_us_region_mean": head["region_us_per_step"],
            "launch_us_note": ("HIP events on the launch stream around the timed region of back-to-back "
                               "launches (one kernel per launch), divided by the launches"),
            "event_pair_us_per_launch": head["event_pair_us_mean"],
            "algo_bytes_per_launch": head["algo_bytes"],
            "sclk_mhz_under_load": head.get("sclk_mhz_under_load"),
            "mclk_mhz_under_load": head.get("mclk_mhz_under_load"),
        },
        "kernel_hash": khash,
        "configs": results,
    }
    pre = results.get("c4:M2048")
    if pre:
        line["prefill"] = {
            "bound": "mfma", "achieved": pre["TFLOPs"], "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": pre["mfma_frac"], "us_per_layer": pre["us_per_layer"], "kernel": "gemm_big_kernel",
            "launches_timed": pre["launches_timed"],
            "traffic": traffic_for(khash, "c4:M2048"),
            "sclk_mhz_under_load": pre.get("sclk_mhz_under_load"),
            "mclk_mhz_under_load": pre.get("mclk_mhz_under_load"),
        }
    if not args.no_peaks:
        log("measuring the achievable streaming-read and MFMA rates")
        peaks = measure_peaks()
        line["achievable"] = peaks
        line["roofline"]["achievable"] = peaks["hbm_read_GBps"]
        line["roofline"]["frac_of_achievable"] = round(line["roofline"]["achieved"] / peaks["hbm_read_GBps"], 4)
        if pre:
            line["prefill"]["achievable"] = peaks["mfma_f16_TFLOPs"]
            line["prefill"]["frac_of_achievable"] = round(pre["TFLOPs"] / peaks["mfma_f16_TFLOPs"], 4)
    if not args.no_dense_ref:
        log("timing the dense binary16 library GEMM of the decode and prefill shapes")
        ref = {"library": "torch.matmul (hipBLASLt), binary16 weights [N][K], x @ W^T",
               "c3:M1_us": dense_reference_us(hcfg, 1, iters=100)}
        ref["c3:M1_w4a16_speedup"] = round(ref["c3:M1_us"] / head["region_us_per_step"], 2)
        if pre:
            ref["c4:M2048_us"] = dense_reference_us(wl.CONFIGS["c4"], 2048, iters=20)
            ref["c4:M2048_w4a16_speedup"] = round(ref["c4:M2048_us"] / pre["us_per_layer"], 3)
        line["dense_fp16_reference"] = ref
    if not args.no_decode_step and args.configs in ("all", "headline"):
        log("timing the decode step of the 1.5B example (eager and graph replay)")
        line["decode_step"] = decode_step_bench(wl.DECODE_1P5B)
    if not args.no_shards and args.configs in ("all", "headline"):
        log("timing one GPU's share of the up-projection and the prefill under tensor parallelism")
        line["shards"] = shards_bench(head["region_us_per_step"], pre["us_per_layer"] if pre else None)
    if not args.no_awq_search and args.configs in ("all", "headline"):
        log("timing the AWQ alpha search on the c2 up-projection layer")
        line["awq_search"] = awq_search_bench(wl.CONFIGS["c2up"])
    if not args.no_gptq and args.configs in ("all", "headline"):
        log("timing GPTQ on the c4 prefill layer")
        line["gptq"] = gptq_bench(wl.CONFIGS["c4"])
    if not args.no_cpu_baseline:
        log("timing the oracle on the host (cpu_baseline)")
        line["cpu_baseline"] = cpu_baseline(hcfg, args.cpu_rows)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
