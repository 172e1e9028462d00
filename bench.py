#!/usr/bin/env python3
"""Decode-step benchmark: weight-stream GB/s and microseconds per layer-stack step.

Default workload: the 70B-class decode stack (80 layers x q, k, v, o, gate, up,
down; hidden 8192, GQA 8 KV heads of 128, FFN 28672) with W4A16-g128 weights,
M = 1 activation row, in the fused layout a decode engine uses: q/k/v and
gate/up each concatenated along N into one matrix (the same weights, bytes and
results; 4 launches per layer instead of 7).  One step = every
y = x . dequant(W)^T call of the stack, replayed from one HIP graph; the packed
weights (~35.6 GB) are resident in HBM before timing starts, and the stack is
far larger than the 256 MB last-level cache, so every step streams the
weights from HBM.

The same run also reports, each from its own graph replays:
  * "separate_layout": the same stack with 7 launches per layer;
  * "targets": the rows the >= 80%-of-measured-bandwidth target names, the
    W4A16 stack at M = 4 and 8 (the headline's packed weights, new x) and the
    FP8-E4M3 stack at M = 1 and 8 (fused layout);
  * "swiglu_layout": the fused stack with gate/up packed for the SwiGLU
    epilogue (down reads silu(gate) * up);
  * "chain": the fused stack at M <= 2 as one persistent launch
    (wqd_chain_run: every matrix of the step, each waiting for the output it
    reads);
  * "config_rows": the remaining measured configurations: the W4A16 stack
    at M = 16 and 32 and the FP8 stack at M = 32 (with matrix-core
    utilisation), the 7B BF16 stack at M = 1, the 4096 x 4096 W4A16 GEMV
    (cold), and the gate matrix at 1024 verify rows in BF16, FP8 and W4A16
    (the product's TFLOP/s against the 2.5 PFLOP/s bf16 peak);
  * "next_rows": W8A8-FP8 on the gate matrix at 1024 rows, and the stack's
    decode attention at batch 32 over 2,048 positions, over a bf16 and an FP8
    cache;
  * "roofline": the dominant kernel (the launches of the step's costliest
    kernel family, replayed on their own) against the 8 TB/s HBM peak;
  * "cpu_baseline": the oracle on one full layer of the same workload on the
    host cores, extrapolated to the stack.

Prints ONE JSON line.  Options: --workload w4a16_70b | fp8_70b | bf16_7b |
w4a16_70b_swiglu | fp8_70b_swiglu | gemv4096 | verify:<fmt>:<mat> |
w8a8:<mat> | attn_70b | attn_fp8kv_70b | spec_accept; --m (activation rows); --separate (time the separate
layout as the headline); --no-alt; --no-targets; --chain (time only the
chain launch; --chain-workgroups sets its grid); --pmc-probe (a short fixed
launch sequence for hardware-counter runs).  A single-matrix workload
(gemv4096, verify:...) is packed into identical copies making 1.2 GB and each
call uses the next one, so that it too reads its weights from HBM; its step is
one call.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor peak
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
FP8_MFMA_PEAK_TFLOPS = 5000.0   # MI355X dense FP8 matrix peak
MAT_INDEX = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6, "w": 0}
TARGET_ROWS = (("w4a16", 4), ("w4a16", 8), ("fp8", 1), ("fp8", 8))
WIDE_ROWS = (("w4a16", 16), ("w4a16", 32), ("fp8", 32))  # stack rows past the target's M <= 8


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="w4a16_70b")
    ap.add_argument("--m", type=int, default=1)
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--separate", action="store_true", help="q, k, v, gate, up as separate matrices")
    ap.add_argument("--no-alt", action="store_true", help="do not also time the other layout")
    ap.add_argument("--no-targets", action="store_true", help="skip the target-row sub-records")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the measured HBM (and, for M >= 16, matrix-core) ceilings")
    ap.add_argument("--no-shapes", action="store_true", help="skip the per-shape timing breakdown")
    ap.add_argument("--spec", action="store_true",
                    help="also time the speculative accept / reject step (64 sequences x 4 drafts, 128256-token vocabulary)")
    ap.add_argument("--chain", action="store_true",
                    help="time the stack as one persistent chain launch (wqd_chain_run) as the headline")
    ap.add_argument("--chain-workgroups", type=int, default=0,
                    help="grid of the chain launch (0: the library's choice)")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run 8 x 1 GiB copies and 16 launches of the dominant kernel, then exit")
    return ap.parse_args()


def make_workload(name, fmt_m, layers, fused):
    from weight_only_quantized_decode_amd import workloads as WL

    m = fmt_m
    if name == "w4a16_70b":
        return WL.stack_70b("w4a16", m, layers or 80, fused)
    if name == "fp8_70b":
        return WL.stack_70b("fp8", m, layers or 80, fused)
    if name in ("w4a16_70b_swiglu", "fp8_70b_swiglu"):
        return WL_stack(name.replace("_swiglu", ""), m, layers)
    if name == "bf16_7b":
        return WL.stack_7b_bf16(m, layers or 32, fused)
    if name == "gemv4096":
        return WL.gemv_4096_w4a16()
    if name.startswith("verify:"):
        _, fmt, mat = name.split(":")
        return WL.verify_matrix(fmt, mat, m)
    if name.startswith("w8a8:"):
        return WL.verify_w8a8(name.split(":")[1], m)
    raise SystemExit(f"unknown workload {name!r}")


def WL_stack(name, M, layers):
    """The fused stack with gate/up packed for the SwiGLU epilogue."""
    from weight_only_quantized_decode_amd import workloads as WL

    return WL.stack_70b("w4a16" if name == "w4a16_70b" else "fp8", M, layers or 80, fused=True, swiglu=True)


def with_m(wl, M):
    """The same stack (same weights) driven by M activation rows."""
    import dataclasses

    return dataclasses.replace(wl, M=M, name=wl.name.replace(f"_m{wl.M}", f"_m{M}"))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def weight_for(wl, layer, name, N, K, dev):
    """The float32 weights of one matrix; fused matrices concatenate their parts'
    draws, so fused and separate stacks hold identical weights."""
    import torch

    import wqd_inputs as I
    from weight_only_quantized_decode_amd import workloads as WL

    if name in WL.FUSED_PARTS:
        shapes = {n: (Nn, Kn) for n, Nn, Kn in (I.LAYER_70B if K == 8192 else I.LAYER_7B)}
        parts = [I.w_device(I.stack_seed(wl.cfg, layer, MAT_INDEX[p]), shapes[p][0], K, device=dev)
                 for p in WL.FUSED_PARTS[name]]
        W = torch.cat(parts, dim=0)
        assert W.shape == (N, K)
        return W
    return I.w_device(I.stack_seed(wl.cfg, layer, MAT_INDEX[name]), N, K, device=dev)


COLD_BYTES = 1.2e9  # a single matrix is timed over this many bytes of packed copies


def copies_for(wl):
    """Packed copies of a single-matrix workload (1 for a stack)."""
    import math

    return max(2, math.ceil(COLD_BYTES / wl.weight_stream_bytes())) if wl.layers == 1 else 1


def pack_stack(wl):
    """Pack every weight matrix of the workload on the device (untimed setup).

    A single-matrix workload (one layer) is packed into as many identical
    copies as make COLD_BYTES, several times the 256 MB last-level cache, and
    each timed call uses the next copy: otherwise every call after the first
    would find its weights in cache.  Returns one row of packed matrices per
    layer (per copy)."""
    import torch

    import weight_only_quantized_decode_amd as wqd

    dev = torch.device("cuda", 0)
    t0 = time.time()
    packed = []
    for layer in range(wl.layers):
        row = []
        for name, N, K in wl.mats:
            W = weight_for(wl, layer, name, N, K, dev)
            swi = wl.swiglu and name == "gate_up"  # gate rows then up rows, packed interleaved
            row.append(wqd.pack_gate_up(wl.fmt, W) if swi else wqd.pack_weights(wl.fmt, W))
            del W
        packed.append(row)
        if layer % 20 == 19:
            torch.cuda.synchronize()
            log(f"[bench] packed layer {layer + 1}/{wl.layers} ({time.time() - t0:.1f}s)")
    for _ in range(copies_for(wl) - 1):
        packed.append([wqd.pack_weights(wl.fmt, weight_for(wl, 0, name, N, K, dev)) for name, N, K in wl.mats])
    torch.cuda.synchronize()
    return packed


def stack_io(wl):
    """x rows per input width, y per output width, and the largest workspace."""
    import torch

    import weight_only_quantized_decode_amd as wqd
    import wqd_inputs as I

    dev = torch.device("cuda", 0)
    xs, ys = {}, {}
    for name, N, K in wl.mats:
        if K not in xs:
            xs[K] = I.x_bf16(I.x_seed(wl.cfg, wl.M, K), wl.M, K, outliers=wl.outliers).to(dev)
        if N not in ys:
            ys[N] = torch.empty((wl.M, N), dtype=torch.bfloat16, device=dev)
    if wl.act == "fp8":
        need = max(max(wqd.w8a8_workspace_bytes(wl.M, N, K) for _, N, K in wl.mats), wqd.ACT_QUANT_WORKSPACE_BYTES)
    else:
        need = max(wqd.workspace_bytes(wl.fmt, wl.M, N, K) for _, N, K in wl.mats)
    return xs, ys, wqd.get_workspace(need, dev)


def replay_timing(launch_all, stream, steps, warmup, use_graph=True):
    """Capture launch_all() in one HIP graph (after an eager warm-up), replay it
    `warmup` times untimed, then `steps` times between HIP events recorded on
    the launch stream, one event before each replay and one after the last.
    Returns (mean ms per replay over the steps, per-replay ms samples)."""
    import torch

    with torch.cuda.stream(stream):
        launch_all()
        torch.cuda.synchronize()
        graph = None
        if use_graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                launch_all()
        run = graph.replay if graph is not None else launch_all
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(stream)
        for i in range(steps):
            run()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
    samples = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    total = ev[0].elapsed_time(ev[steps])
    del graph
    return total / steps, samples


def kernel_group(wl, N, K):
    import weight_only_quantized_decode_amd as wqd

    if wl.act == "fp8":
        return "w8a8 fp8 matrix cores"
    return "%s(%d waves)" % wqd.kernel_path(wl.fmt, wl.M, N, K)


def time_step(wl, packed, args, stream, dominant=False, shapes=False):
    """Time the step of `wl` on its packed weights; optionally also the
    dominant kernel family on its own and a per-matrix breakdown."""
    import weight_only_quantized_decode_amd as wqd
    from weight_only_quantized_decode_amd import workloads as WL

    import torch

    xs, ys, ws = stack_io(wl)
    rows = len(packed) // wl.layers  # copies of a single matrix: one replay calls each once
    # W8A8: a call is the activation quantisation, then the product (the
    # kernel-family replays time the product alone, on codes made once)
    codes = {K: wqd.act_quant_fp8(x, workspace=ws) for K, x in xs.items()} if wl.act == "fp8" else None
    hbuf = None
    if wl.swiglu:
        F = dict((name, N) for name, N, _ in wl.mats)["gate_up"] // 2
        hbuf = torch.empty((wl.M, F), dtype=torch.bfloat16, device=ys[next(iter(ys))].device)

    def launches(only=None):
        def go():
            for row in packed:
                for j, ((name, N, K), pw) in enumerate(zip(wl.mats, row)):
                    if only is not None and j not in only:
                        continue
                    if wl.swiglu and name == "gate_up":  # h = silu(gate) * up, read by down
                        wqd.qgemm_swiglu(xs[K], pw, h=hbuf, workspace=ws)
                        continue
                    if wl.swiglu and name == "down":
                        wqd.qgemm(hbuf, pw, y=ys[N], workspace=ws)
                        continue
                    if codes is None:
                        wqd.qgemm(xs[K], pw, y=ys[N], workspace=ws)
                        continue
                    if only is None:
                        wqd.act_quant_fp8(xs[K], *codes[K], workspace=ws)
                    wqd.qgemm_w8a8(*codes[K], pw, y=ys[N], workspace=ws)
        return go

    log(f"[bench] {wl.name}: {wl.launches} launches/step, {wl.step_bytes() / 1e9:.3f} GB/step; "
        f"timing {args.steps} steps")
    ms, samples = replay_timing(launches(), stream, args.steps, args.warmup, not args.no_graph)
    ms, samples = ms / rows, [s / rows for s in samples]
    gbps = wl.step_bytes() / (ms / 1e3) / 1e9
    res = {"workload": wl.name, "fmt": wl.fmt, "M": wl.M, "layers": wl.layers, "launches_per_step": wl.launches,
           "ms_per_step": round(ms, 4), "GBps": round(gbps, 2),
           "step_samples_ms": {"n": len(samples), "median": round(statistics.median(samples), 4),
                               "min": round(min(samples), 4), "max": round(max(samples), 4)},
           "kernels": sorted({kernel_group(wl, N, K) for _, N, K in wl.mats})}
    if dominant:
        groups = {}
        for j, (_, N, K) in enumerate(wl.mats):
            groups.setdefault(kernel_group(wl, N, K), []).append(j)
        per = {}
        for label, js in groups.items():
            g_ms, _ = replay_timing(launches(set(js)), stream, args.steps, args.warmup, not args.no_graph)
            n_launch = len(js) * len(packed)
            g_bytes = len(packed) * sum(wl.call_bytes(wl.mats[j][1], wl.mats[j][2], wl.mats[j][0]) for j in js)
            g_flops = len(packed) * sum(WL.call_flops(wl.M, wl.mats[j][1], wl.mats[j][2]) for j in js)
            # per step: a replay calls every copy of a single matrix once (rows steps)
            per[label] = {"matrices": [wl.mats[j][0] for j in js], "launches": n_launch // rows, "ms": g_ms / rows,
                          "avg_launch_us": g_ms * 1e3 / n_launch, "bytes": g_bytes / rows, "flops": g_flops / rows}
        res["groups"] = per
    if shapes and wl.layers > 1:
        out = {}
        for j, (name, N, K) in enumerate(wl.mats):
            s_ms, _ = replay_timing(launches({j}), stream, max(3, args.steps // 4), 1, not args.no_graph)
            us = s_ms * 1e3 / wl.layers
            b = wl.call_bytes(N, K, name)
            out[name] = {"N": N, "K": K, "us": round(us, 2), "GBps": round(b / (us * 1e-6) / 1e9, 1),
                         "kernel": kernel_group(wl, N, K)}
        res["shapes"] = out
    del xs, ys, ws
    return res


def chain_steps(wl, packed):
    """The stack as a dependent chain for one persistent launch: qkv reads the
    previous layer's down output, o the first M x 8192 of qkv's output (in
    place of attention's), gate/up o's output, down the SwiGLU output (or, in
    the plain fused layout, the first M x 28672 of gate/up's output in place
    of it).  One set of buffers serves every layer: each buffer's readers are
    ancestors of its next writer through the waits."""
    import torch

    import weight_only_quantized_decode_amd as wqd
    import wqd_inputs as I

    dev = torch.device("cuda", 0)
    K0 = wl.mats[0][2]
    x0 = I.x_bf16(I.x_seed(wl.cfg, wl.M, K0), wl.M, K0, outliers=wl.outliers).to(dev)
    bufs = {}
    steps = []
    prev = x0
    for layer, row in enumerate(packed):
        for (name, N, K), pw in zip(wl.mats, row):
            swi = wl.swiglu and name == "gate_up"
            cols = N // 2 if swi else N
            if name not in bufs:
                bufs[name] = torch.empty((wl.M, cols), dtype=torch.bfloat16, device=dev)
            x = prev if prev.shape[1] == K else prev.reshape(-1)[: wl.M * K].view(wl.M, K)
            steps.append(wqd.ChainStep(x, pw, bufs[name], len(steps) - 1, swi))
            prev = bufs[name]
    return steps, x0


def chain_timing(wl, packed, args, stream):
    """The step as one chain launch (plus its clearing launch), replayed from a graph."""
    import weight_only_quantized_decode_amd as wqd

    steps, _ = chain_steps(wl, packed)
    chain = wqd.chain_prepare(steps, workgroups=args.chain_workgroups)
    log(f"[bench] chain {wl.name}: {len(steps)} calls, {chain.plan.total_items} items, "
        f"{chain.plan.workgroups} workgroups")
    ms, samples = replay_timing(lambda: wqd.chain_run(chain), stream, args.steps, args.warmup, not args.no_graph)
    st = wqd.chain_status(chain, stream)
    if st != 0:
        raise RuntimeError(f"chain run reported status {st}")
    gbps = wl.step_bytes() / (ms / 1e3) / 1e9
    res = {"workload": wl.name, "fmt": wl.fmt, "M": wl.M, "layers": wl.layers, "calls": len(steps),
           "launches_per_step": 2, "workgroups": chain.plan.workgroups, "items": chain.plan.total_items,
           "ms_per_step": round(ms, 4), "GBps": round(gbps, 2),
           "step_samples_ms": {"n": len(samples), "median": round(statistics.median(samples), 4),
                               "min": round(min(samples), 4), "max": round(max(samples), 4)},
           "kernel": "chain_kernel: every matrix of the step in one persistent launch, each waiting for "
                     "the output it reads"}
    del chain, steps
    return res


def free_cache():
    import torch

    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def mfma_ceiling(iters=20000):
    """Measured matrix-core throughput (TFLOP/s): back-to-back bf16 multiplies
    from registers on every SIMD (the library's ceiling kernel)."""
    import torch

    import weight_only_quantized_decode_amd as wqd

    sink = torch.empty(wqd.mfma_peak_sink_words(), dtype=torch.float32, device="cuda")
    wqd.mfma_peak(100, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    flops = wqd.mfma_peak(iters, sink)
    e1.record()
    torch.cuda.synchronize()
    return flops / (e0.elapsed_time(e1) / 1e3) / 1e12


def hbm_ceiling(gib=4, reps=10):
    """Measured HBM read and copy bandwidth (GB/s) with the library's stream
    kernels: each the best of three timed runs of `reps` back-to-back launches."""
    import torch

    import weight_only_quantized_decode_amd as wqd

    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    dst = torch.empty(n // 2, dtype=torch.uint8, device="cuda")
    sink = wqd.stream_read(buf)
    wqd.stream_copy(dst, buf[: n // 2])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    read = copy = 0.0
    for _ in range(3):
        e0.record()
        for _ in range(reps):
            wqd.stream_read(buf, sink)
        e1.record()
        torch.cuda.synchronize()
        read = max(read, n * reps / (e0.elapsed_time(e1) / 1e3) / 1e9)
        e0.record()
        for _ in range(reps):
            wqd.stream_copy(dst, buf[: n // 2])
        e1.record()
        torch.cuda.synchronize()
        copy = max(copy, 2 * (n // 2) * reps / (e0.elapsed_time(e1) / 1e3) / 1e9)
    del buf, dst
    free_cache()
    return read, copy


# The sources the broadcast kernel (the headline's dominant kernel) and its
# kernel choice are built from: counters taken before a change to any of them
# no longer describe the kernel.
TRAFFIC_SOURCES = ("wqd_gemv_bcast.hip", "wqd_bcast_tile.h", "wqd_device.h", "wqd_internal.h", "wqd_plan.h",
                   "wqd_plan.cpp")


def profiled_traffic(wl):
    """HBM bytes per launch from the committed counter summary of this workload
    (profiles/traffic_<workload>.json: FETCH_SIZE and WRITE_SIZE runs scaled by
    a copy kernel of known size), or None when there is none or the kernel's
    sources (TRAFFIC_SOURCES) changed since the counters were taken."""
    import hashlib

    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"traffic_{wl.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    csrc = os.path.join(root, "weight_only_quantized_decode_amd", "csrc")
    recorded = d.get("kernel_sources_sha256_16", {})
    if sorted(recorded) != sorted(TRAFFIC_SOURCES):  # the dominant kernel's sources, no more, no fewer
        return None
    for fn, digest in recorded.items():
        with open(os.path.join(csrc, fn), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest()[:16] != digest:
                return None
    return d["traffic_bytes_per_launch"]


def host_description():
    try:
        from threadpoolctl import threadpool_info

        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    desc = (f"host {model} ({platform.machine()}), {os.cpu_count()} logical CPUs, {affinity} in this "
            f"process's affinity mask, BLAS threads {threads}")
    return int(threads), desc


def cpu_baseline(wl, budget_s=12.0):
    """The oracle as it stands (exact dequantisation, float64 matmul, bf16
    rounding: oracle.qgemm_ref) timed on the host cores on a bounded sample of
    the same workload.  A stack is sampled as one full layer (every matrix of
    the timed step, layer 0's weights) and extrapolated to all layers; a single
    matrix is timed whole."""
    import oracle
    import wqd_inputs as I
    from weight_only_quantized_decode_amd import workloads as WL

    import numpy as np

    t_setup = time.perf_counter()
    mats = []
    for name, N, K in wl.mats:
        if name in WL.FUSED_PARTS:
            shapes = {n: Nn for n, Nn, _ in (I.LAYER_70B if K == 8192 else I.LAYER_7B)}
            W = np.concatenate([I.w_host(I.stack_seed(wl.cfg, 0, MAT_INDEX[p]), shapes[p], K)
                                for p in WL.FUSED_PARTS[name]], axis=0)
        else:
            W = I.w_host(I.stack_seed(wl.cfg, 0, MAT_INDEX.get(name, 0)), N, K)
        mats.append((oracle.quantize(wl.fmt, W), K))
        del W
    xs = {K: I.x_bf16_bits(I.x_seed(wl.cfg, wl.M, K), wl.M, K, outliers=wl.outliers) for _, K in mats}
    setup_s = time.perf_counter() - t_setup
    reps, t_total = 0, 0.0
    ref = oracle.qgemm_w8a8_ref if wl.act == "fp8" else oracle.qgemm_ref
    while reps < 1 or (t_total < budget_s and reps < 50):
        t0 = time.perf_counter()
        for qw, K in mats:
            ref(xs[K], qw)
        t_total += time.perf_counter() - t0
        reps += 1
    per_layer = t_total / reps
    step_s = per_layer * wl.layers
    gbps = wl.step_bytes() / step_s / 1e9
    threads, host = host_description()
    what = (f"one full layer ({len(mats)} matrices, layer 0) x {reps} passes, extrapolated x {wl.layers} layers"
            if wl.layers > 1 else f"{reps} calls on one matrix")
    return {
        "value": round(gbps, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "ms_per_step": round(step_s * 1e3, 1),
        "extrapolated": wl.layers > 1,
        "sample": f"the float64 oracle ({'activation quantisation, exact code product' if wl.act == 'fp8' else 'exact dequant, matmul'}, bf16 rounding) on {wl.name}: {what}; "
                  f"{per_layer * 1e3:.1f} ms per layer ({t_total:.1f} s timed, {setup_s:.1f} s untimed "
                  f"quantisation); {host}",
    }


def pmc_probe():
    """Fixed sequence for counter runs: 8 copies of 1 GiB (known traffic: 1 GiB
    read + 1 GiB written each), then 16 launches of the W4A16 M=1 kernel on
    16 different 28672 x 8192 matrices (HBM-cold)."""
    import torch

    import weight_only_quantized_decode_amd as wqd
    import wqd_inputs as I

    dev = torch.device("cuda", 0)
    src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(8):
        wqd.stream_copy(dst, src)
    torch.cuda.synchronize()
    del src, dst
    N, K = 28672, 8192
    pws = []
    for i in range(16):
        W = I.w_device(900 + i, N, K, device=dev)
        pws.append(wqd.pack_weights("w4a16", W))
        del W
    x = I.x_bf16(1, 1, K).to(dev)
    y = torch.empty((1, N), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    for pw in pws:
        wqd.qgemm(x, pw, y=y)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_probe": "done", "copy_bytes_each": 2 << 30, "gemv_launches": 16, "N": N, "K": K}))


def spec_accept_timing(B=64, k=4, V=128256, reps=50):
    """The accept / reject step after a verify pass of k + 1 positions: time per
    call (its tile-sum and draw launches) from reps calls replayed in one HIP
    graph on one stream, and its algorithmic bytes (the accept tests' few
    values, then one target row per sequence, plus its draft row where a draft
    was rejected, read once)."""
    import numpy as np
    import torch

    import weight_only_quantized_decode_amd as wqd
    import wqd_inputs as I

    log(f"[bench] speculative accept / reject: B={B} k={k} V={V}")
    dev = [torch.from_numpy(np.ascontiguousarray(a)).to("cuda") for a in I.spec_inputs(5, B, k, V)]
    n, _ = wqd.spec_accept(*dev)
    torch.cuda.synchronize()
    n = n.cpu().numpy()
    rows = int(np.sum(np.where(n < k, 2, 1)))
    algo = rows * V * 4 + B * k * 16 + B * 4 + B * (k + 2) * 4
    stream = torch.cuda.Stream()
    ws = wqd.get_workspace(wqd.spec_workspace_bytes(B, V), dev[0].device)

    def go():
        for _ in range(reps):
            wqd.spec_accept(*dev, workspace=ws)

    ms, _ = replay_timing(go, stream, 5, 2, True)
    us = ms * 1e3 / reps
    gbps = algo / (us * 1e-6) / 1e9
    return {"B": B, "k": k, "V": V, "mean_kept": round(float(n.mean()), 3), "us_per_call": round(us, 2),
            "launches_per_call": 2, "algorithmic_bytes": algo, "GBps": round(gbps, 1),
            "roofline_frac_hbm": round(gbps / 8000.0, 4)}


ATTN_HQ, ATTN_HKV, ATTN_D = 64, 8, 128  # the 70B layer's grouped-query attention


def attn_stack_timing(args, stream, B=32, ctx=2048, layers=80, kv="bf16"):
    """Decode attention of every layer of the 70B-class stack for B sequences
    of ctx positions (the pages' batch-32 snapshot: 80 layers x 8 KV heads x
    128 x 2 bytes x 2 for keys and values = 671,088,640 bytes per sequence).
    Each layer has its own caches, so a step reads 21.5 GB of KV from HBM
    (half that from an FP8 cache, kv="fp8": one byte per element, the
    one-byte-KV case of the hands-on lab's exercise 5).  One step = 80
    wqd_decode_attention(_fp8kv) calls (split kernel and merge each),
    replayed from a HIP graph."""
    import math

    import torch

    import weight_only_quantized_decode_amd as wqd

    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev)
    g.manual_seed(2048 + B)
    fp8 = kv == "fp8"
    log(f"[bench] decode attention ({kv} cache): {layers} layers, B={B}, {ctx} positions, {ATTN_HQ}/{ATTN_HKV} heads")
    caches = []
    if fp8:
        k_scale = v_scale = 4.0 / 448  # N(0, 1) entries, saturating past 4 sigma
        tmp_k = torch.empty((B, ATTN_HKV, ctx, ATTN_D), dtype=torch.bfloat16, device=dev)
        tmp_v = torch.empty_like(tmp_k)
    for _ in range(layers):
        if fp8:
            c = wqd.alloc_kv_cache_fp8(B, ATTN_HKV, ctx, k_scale, v_scale, ATTN_D, device=dev)
            tmp_k.normal_(generator=g)
            tmp_v.normal_(generator=g)
            wqd.kv_pack_fp8(tmp_k, tmp_v, c)
        else:
            c = wqd.alloc_kv_cache(B, ATTN_HKV, ctx, ATTN_D, device=dev)
            c.k.normal_(generator=g)  # random entries: the tile order of the layout does not matter
            c.v.normal_(generator=g)
        caches.append(c)
    if fp8:
        del tmp_k, tmp_v
    q = torch.randn((B, ATTN_HQ, ATTN_D), generator=g, device=dev, dtype=torch.bfloat16)
    out = torch.empty_like(q)
    lens = torch.full((B,), ctx, dtype=torch.int32, device=dev)
    wsb = (wqd.attn_fp8kv_workspace_bytes if fp8 else wqd.attn_workspace_bytes)(B, ATTN_HQ, ATTN_HKV, ctx)
    ws = wqd.get_workspace(wsb, dev)  # None when 0 bytes
    scale = 1.0 / math.sqrt(ATTN_D)

    def go():
        for c in caches:
            if fp8:
                wqd.decode_attention_fp8kv(q, c, lens, scale, out=out, workspace=ws)
            else:
                wqd.decode_attention(q, c, lens, scale, out=out, workspace=ws)

    ms, samples = replay_timing(go, stream, args.steps, args.warmup, not args.no_graph)
    kv_bytes = B * ATTN_HKV * ctx * ATTN_D * (1 if fp8 else 2) * 2
    per_layer = kv_bytes + 2 * (B * ATTN_HQ * ATTN_D * 2) + 4 * B
    gbps = layers * per_layer / (ms / 1e3) / 1e9
    name = "70b_decode_attention_fp8kv" if fp8 else "70b_decode_attention"
    res = {"workload": f"{name}_{layers}l_b{B}_ctx{ctx}", "B": B, "context": ctx, "layers": layers, "kv": kv,
           "q_heads": ATTN_HQ, "kv_heads": ATTN_HKV, "head_dim": ATTN_D, "ms_per_step": round(ms, 4),
           "us_per_layer": round(ms * 1e3 / layers, 2), "kv_bytes_per_step": layers * kv_bytes,
           "algorithmic_bytes_per_step": layers * per_layer, "GBps": round(gbps, 2),
           "step_samples_ms": {"n": len(samples), "median": round(statistics.median(samples), 4),
                               "min": round(min(samples), 4), "max": round(max(samples), 4)},
           "splits": (wqd.attn_fp8kv_splits if fp8 else wqd.attn_splits)(B, ATTN_HQ, ATTN_HKV, ctx),
           "kernel": f"attn_split_kernel<{'true' if fp8 else 'false'}> (+ attn_combine_kernel when the context is "
                     "split) per layer"}
    del caches
    free_cache()
    return res


def pct(v, ceil):
    return None if not ceil else round(100 * v / ceil, 2)


def roofline_of(wl, res):
    """The dominant kernel: the kernel family whose launches, replayed on their
    own, take the most time per step.  achieved = its algorithmic bytes (or
    FLOPs) per launch / its average launch duration."""
    label, g = max(res["groups"].items(), key=lambda kv: kv[1]["ms"])
    per_launch_bytes = g["bytes"] / g["launches"]
    per_launch_flops = g["flops"] / g["launches"]
    avg_us = g["avg_launch_us"]
    peak_tf = FP8_MFMA_PEAK_TFLOPS if wl.act == "fp8" else BF16_MFMA_PEAK_TFLOPS
    if per_launch_flops / (peak_tf * 1e12) > per_launch_bytes / (HBM_PEAK_GBPS * 1e9):
        tf = per_launch_flops / (avg_us / 1e6) / 1e12
        r = {"bound": "mfma", "achieved": round(tf, 2), "peak": peak_tf, "unit": "TFLOP/s",
             "frac": round(tf / peak_tf, 4)}
    else:
        a = per_launch_bytes / (avg_us / 1e6) / 1e9
        r = {"bound": "hbm", "achieved": round(a, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
             "frac": round(a / HBM_PEAK_GBPS, 4)}
    r.update({"traffic": profiled_traffic(wl) if label.startswith("bcast") else None,
              "kernel": f"{label} {wl.fmt} M={wl.M}: the {'/'.join(g['matrices'])} launches of every layer, "
                        f"replayed on their own",
              "avg_launch_us": round(avg_us, 3), "launches": g["launches"],
              "bytes_per_launch": round(per_launch_bytes), "flops_per_launch": round(per_launch_flops),
              "share_of_step": round(g["ms"] / res["ms_per_step"], 4)})
    return r


def wide_row(wl, packed, args, stream, ceiling, mpeak):
    """A stack row past the M <= 8 target: GB/s against the ceilings and the
    matrix-core utilisation of its 2MNK FLOPs (against the vendor peak and,
    when measured, the back-to-back multiply ceiling)."""
    r = time_step(wl, packed, args, stream)
    r["pct_measured_read_ceiling"] = pct(r["GBps"], ceiling[0])
    r["pct_measured_copy_ceiling"] = pct(r["GBps"], ceiling[1])
    r["pct_hbm_peak"] = round(100 * r["GBps"] / HBM_PEAK_GBPS, 2)
    tflops = wl.step_flops() / (r["ms_per_step"] / 1e3) / 1e12
    r["mfma_util_pct"] = round(100 * tflops / BF16_MFMA_PEAK_TFLOPS, 2)
    if mpeak:
        r["mfma_util_pct_measured_ceiling"] = round(100 * tflops / mpeak, 2)
    return r


def other_configs(args, stream, ceiling, mpeak):
    """The 7B BF16 stack at M = 1, the 4096^2 W4A16 GEMV read cold, and the gate
    matrix at 1024 verify rows in each weight format (its product alone
    against the bf16 matrix peak), each from its own replays."""
    rows = []
    for name, M in (("bf16_7b", 1), ("gemv4096", 1)):
        wl = make_workload(name, M, None, True)
        packed = pack_stack(wl)
        r = time_step(wl, packed, args, stream)
        del packed
        free_cache()
        r["pct_measured_read_ceiling"] = pct(r["GBps"], ceiling[0])
        r["weight_copies"] = copies_for(wl)
        if wl.layers == 1:
            r["us_per_call"] = round(wl.step_bytes() / (r["GBps"] * 1e9) * 1e6, 2)
        rows.append(r)
    for fmt in ("bf16", "fp8", "w4a16"):
        wl = make_workload(f"verify:{fmt}:gate", 1024, None, True)
        packed = pack_stack(wl)
        r = time_step(wl, packed, args, stream, dominant=True)
        del packed
        free_cache()
        rr = roofline_of(wl, r)
        rows.append({"workload": wl.name, "fmt": fmt, "M": wl.M, "ms_per_call": r["ms_per_step"],
                     "product_us": rr["avg_launch_us"], "product_TFLOPs": rr["achieved"],
                     "frac_bf16_peak": rr["frac"], "kernel": kernel_group(wl, wl.mats[0][1], wl.mats[0][2]),
                     "frac_measured_mfma_ceiling": round(rr["achieved"] / mpeak, 4) if mpeak else None,
                     "weight_copies": copies_for(wl)})
    return rows


def attn_main(args, stream, ceiling):
    """--workload attn_70b / attn_fp8kv_70b: the stack's decode attention over
    a bf16 / FP8 cache as the headline."""
    B = args.m if args.m > 1 else 32
    a = attn_stack_timing(args, stream, B=B, layers=args.layers or 80,
                          kv="fp8" if args.workload == "attn_fp8kv_70b" else "bf16")
    per_layer_bytes = a["algorithmic_bytes_per_step"] / a["layers"]
    achieved = per_layer_bytes / (a["us_per_layer"] * 1e-6) / 1e9
    out = {
        "metric": "weight-stream GB/s (% of HBM peak) & us per layer-stack step, 70B W4A16/FP8/BF16",
        "value": a["GBps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": a["ms_per_step"], "us_per_step": round(a["ms_per_step"] * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": a["workload"], "B": B, "context": a["context"], "layers": a["layers"],
                   "graph": not args.no_graph},
        "pct_hbm_peak": round(100 * a["GBps"] / HBM_PEAK_GBPS, 2),
        "hbm_read_ceiling_GBps": None if ceiling[0] is None else round(ceiling[0], 1),
        "pct_measured_read_ceiling": pct(a["GBps"], ceiling[0]),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None, "kernel": a["kernel"],
                     "avg_launch_us": a["us_per_layer"], "bytes_per_launch": round(per_layer_bytes)},
        "attention": a,
    }
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this decode layer is measured on a single MI355X "
              "(sharding the layer across GPUs is not implemented).", file=sys.stderr)
        sys.exit(2)
    import torch

    import weight_only_quantized_decode_amd as wqd

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    wqd.lib()
    if args.pmc_probe:
        pmc_probe()
        return
    fused = not args.separate
    ceiling = (None, None) if args.no_ceiling else hbm_ceiling()
    if ceiling[0]:
        log(f"[bench] HBM ceiling: read {ceiling[0]:.0f} GB/s, copy {ceiling[1]:.0f} GB/s")
    stream = torch.cuda.Stream()
    if args.workload in ("attn_70b", "attn_fp8kv_70b"):
        attn_main(args, stream, ceiling)
        return
    if args.workload == "spec_accept":
        r = spec_accept_timing()
        print(json.dumps({"metric": "speculative accept / reject GB/s (% of HBM peak)", "value": r["GBps"],
                          "unit": "GB/s", "n_gpus": 1, "higher_is_better": True, "dtype": "f32", "data": "synthetic",
                          "config": {"workload": "spec_accept_b64_k4_v128256"},
                          "roofline": {"bound": "hbm", "achieved": r["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                       "frac": r["roofline_frac_hbm"], "traffic": None},
                          "spec_accept": r}), flush=True)
        return
    wl = make_workload(args.workload, args.m, args.layers, fused)

    packed = pack_stack(wl)
    if args.chain:
        r = chain_timing(wl, packed, args, stream)
        r["pct_measured_read_ceiling"] = pct(r["GBps"], ceiling[0])
        print(json.dumps({"chain": r}), flush=True)
        return
    head = time_step(wl, packed, args, stream, dominant=True, shapes=not args.no_shapes)
    targets = []
    is_stack = wl.layers > 1 and args.workload in ("w4a16_70b", "fp8_70b", "bf16_7b")
    chain_rec = None
    if is_stack and fused and wl.M <= 2 and not args.no_alt:
        chain_rec = chain_timing(wl, packed, args, stream)
    config_rows = []
    default_run = is_stack and not args.no_targets and args.workload == "w4a16_70b" and fused
    mpeak = mfma_ceiling() if default_run and not args.no_ceiling else None
    if mpeak:
        log(f"[bench] matrix-core ceiling: {mpeak:.0f} TFLOP/s")
    if default_run:
        for fmt, M in TARGET_ROWS:
            if fmt == wl.fmt and M != wl.M:
                targets.append(time_step(with_m(wl, M), packed, args, stream))
        for fmt, M in WIDE_ROWS:
            if fmt == wl.fmt and M != wl.M:
                config_rows.append(wide_row(with_m(wl, M), packed, args, stream, ceiling, mpeak))
    del packed
    free_cache()

    swiglu_rec = None
    if is_stack and not args.no_alt and args.workload in ("w4a16_70b", "fp8_70b") and fused:
        sw_wl = WL_stack(args.workload, args.m, args.layers)
        sw_packed = pack_stack(sw_wl)
        swiglu_rec = time_step(sw_wl, sw_packed, args, stream)
        del sw_packed
        free_cache()
    alt = None
    if is_stack and not args.no_alt:
        alt_wl = make_workload(args.workload, args.m, args.layers, not fused)
        alt_packed = pack_stack(alt_wl)
        alt = time_step(alt_wl, alt_packed, args, stream)
        del alt_packed
        free_cache()
    if is_stack and not args.no_targets and args.workload == "w4a16_70b" and fused:
        fp8_wl = make_workload("fp8_70b", 1, args.layers, True)
        fp8_packed = pack_stack(fp8_wl)
        for fmt, M in TARGET_ROWS:
            if fmt == "fp8":
                targets.append(time_step(with_m(fp8_wl, M), fp8_packed, args, stream))
        for fmt, M in WIDE_ROWS:
            if fmt == "fp8":
                config_rows.append(wide_row(with_m(fp8_wl, M), fp8_packed, args, stream, ceiling, mpeak))
        del fp8_packed
        free_cache()
        config_rows.extend(other_configs(args, stream, ceiling, mpeak))

    # the adjacent parts of the step, each from its own replays: W8A8-FP8 at the widest
    # verify width, and the stack's decode attention at the batch-32 snapshot
    next_rows = {}
    if is_stack and not args.no_targets and args.workload == "w4a16_70b" and fused:
        w8 = make_workload("w8a8:gate", 1024, None, True)
        w8_packed = pack_stack(w8)
        r = time_step(w8, w8_packed, args, stream, dominant=True)
        del w8_packed
        free_cache()
        rr = roofline_of(w8, r)
        next_rows["w8a8_gate_m1024"] = {"ms_per_call": r["ms_per_step"], "product_us": rr["avg_launch_us"],
                                        "product_TFLOPs": rr["achieved"], "frac_fp8_peak": rr["frac"],
                                        "workload": w8.name, "weight_copies": copies_for(w8)}
        for kv, key in (("bf16", "decode_attention"), ("fp8", "decode_attention_fp8kv")):
            a = attn_stack_timing(args, stream, kv=kv)
            a["pct_measured_read_ceiling"] = pct(a["GBps"], ceiling[0])
            a["frac_hbm_peak"] = round(a["GBps"] / HBM_PEAK_GBPS, 4)
            next_rows[key] = a

    ms = head["ms_per_step"]
    gbps = head["GBps"]
    roofline = roofline_of(wl, head)
    out = {
        "metric": "weight-stream GB/s (% of HBM peak) & us per layer-stack step, 70B W4A16/FP8/BF16",
        "value": gbps,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "us_per_step": round(ms * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3" if wl.act == "fp8" else {"w4a16": "u4+bf16", "fp8": "e4m3+bf16", "bf16": "bf16"}[wl.fmt],
        "data": "synthetic",
        "config": {"workload": wl.name, "fmt": wl.fmt, "M": wl.M, "layers": wl.layers,
                   "launches_per_step": wl.launches, "graph": not args.no_graph, "fused": fused,
                   "weight_copies": copies_for(wl), "algorithmic_bytes_per_step": wl.step_bytes()},
        "step_samples_ms": head["step_samples_ms"],
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "hbm_read_ceiling_GBps": None if ceiling[0] is None else round(ceiling[0], 1),
        "hbm_copy_ceiling_GBps": None if ceiling[1] is None else round(ceiling[1], 1),
        "pct_measured_read_ceiling": pct(gbps, ceiling[0]),
        "pct_measured_copy_ceiling": pct(gbps, ceiling[1]),
        "roofline": roofline,
        "kernel_groups": {k: {"matrices": v["matrices"], "launches": v["launches"],
                              "avg_launch_us": round(v["avg_launch_us"], 3),
                              "ms_per_step_replayed_alone": round(v["ms"], 4)}
                          for k, v in head["groups"].items()},
    }
    if alt is not None:
        alt["pct_measured_read_ceiling"] = pct(alt["GBps"], ceiling[0])
        out["separate_layout" if fused else "fused_layout"] = alt
    if swiglu_rec is not None:
        swiglu_rec["pct_measured_read_ceiling"] = pct(swiglu_rec["GBps"], ceiling[0])
        out["swiglu_layout"] = swiglu_rec
    if chain_rec is not None:
        chain_rec["pct_measured_read_ceiling"] = pct(chain_rec["GBps"], ceiling[0])
        out["chain"] = chain_rec
    if targets:
        for t in targets:
            t["pct_measured_read_ceiling"] = pct(t["GBps"], ceiling[0])
            t["pct_measured_copy_ceiling"] = pct(t["GBps"], ceiling[1])
            t["pct_hbm_peak"] = round(100 * t["GBps"] / HBM_PEAK_GBPS, 2)
        out["targets"] = targets
    if "shapes" in head:
        out["shapes"] = head["shapes"]
    if config_rows:
        out["config_rows"] = config_rows
    if mpeak:
        out["mfma_ceiling_TFLOPs"] = round(mpeak, 1)
    if next_rows:
        out["next_rows"] = next_rows
    if wl.M >= 16:
        tflops = wl.step_flops() / (ms / 1e3) / 1e12
        out["mfma_util_pct"] = round(100 * tflops / (FP8_MFMA_PEAK_TFLOPS if wl.act == "fp8" else
                                                     BF16_MFMA_PEAK_TFLOPS), 2)
        if not args.no_ceiling and wl.act != "fp8":  # the ceiling kernel runs bf16 multiplies
            peak = mfma_ceiling()
            log(f"[bench] matrix-core ceiling: {peak:.0f} TFLOP/s")
            out["mfma_ceiling_TFLOPs"] = round(peak, 1)
            out["mfma_util_pct_measured_ceiling"] = round(100 * tflops / peak, 2)
    if args.spec:
        out["spec_accept"] = spec_accept_timing()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(wl)
        out["cpu_baseline"]["gpu_ms_per_step"] = ms
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
