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
weights from HBM.  The same stack in the separate layout (7 launches per
layer) is timed in the same run and reported as "separate_layout".

Prints ONE JSON line.  Options: --workload w4a16_70b | fp8_70b | bf16_7b |
gemv4096 | verify:<fmt>:<mat>; --m (activation rows); --separate (time the
separate layout as the headline); --no-alt (skip the other layout);
--pmc-probe (a short fixed launch sequence for hardware-counter runs).  A
single-matrix workload (gemv4096, verify:...) is packed into identical copies
making 1.2 GB and each call uses the next one, so that it too reads its
weights from HBM; its step is one call.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, vendor peak
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
MAT_INDEX = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6, "w": 0}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="w4a16_70b")
    ap.add_argument("--m", type=int, default=1)
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--fused", action="store_true", help="q/k/v and gate/up as one matrix each (the default)")
    ap.add_argument("--separate", action="store_true", help="q, k, v, gate, up as separate matrices")
    ap.add_argument("--no-alt", action="store_true", help="do not also time the other layout")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying a HIP graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the measured HBM (and, for M >= 16, matrix-core) ceilings")
    ap.add_argument("--no-shapes", action="store_true", help="skip the per-shape timing breakdown")
    ap.add_argument("--spec", action="store_true",
                    help="also time the speculative accept / reject step (64 sequences x 4 drafts, 128256-token vocabulary)")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run 8 x 1 GiB copies and 16 launches of the dominant kernel, then exit")
    return ap.parse_args()


def make_workload(args):
    from weight_only_quantized_decode_amd import workloads as WL

    w = args.workload
    if w == "w4a16_70b":
        return WL.stack_70b("w4a16", args.m, args.layers or 80, args.fused)
    if w == "fp8_70b":
        return WL.stack_70b("fp8", args.m, args.layers or 80, args.fused)
    if w == "bf16_7b":
        return WL.stack_7b_bf16(args.m, args.layers or 32, args.fused)
    if w == "gemv4096":
        return WL.gemv_4096_w4a16()
    if w.startswith("verify:"):
        _, fmt, mat = w.split(":")
        return WL.verify_matrix(fmt, mat, args.m)
    raise SystemExit(f"unknown workload {w!r}")


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


def build_stack(wl):
    """Pack every weight matrix of the workload on the device (untimed setup).

    A single-matrix workload (one layer) is packed into as many identical
    copies as make COLD_BYTES, several times the 256 MB last-level cache, and
    each timed call uses the next copy: otherwise every call after the first
    would find its weights in cache.  Returns one row of packed matrices per
    layer (per copy)."""
    import torch

    import weight_only_quantized_decode_amd as wqd
    import wqd_inputs as I

    dev = torch.device("cuda", 0)
    packed = []
    t0 = time.time()
    copies = copies_for(wl)
    for layer in range(wl.layers):
        row = []
        for name, N, K in wl.mats:
            W = weight_for(wl, layer, name, N, K, dev)
            row.append(wqd.pack_weights(wl.fmt, W))
            del W
        packed.append(row)
    for _ in range(copies - 1):
        packed.append([wqd.pack_weights(wl.fmt, weight_for(wl, 0, name, N, K, dev)) for name, N, K in wl.mats])
        if layer % 10 == 0:
            torch.cuda.synchronize()
            log(f"[bench] packed layer {layer}/{wl.layers} ({time.time() - t0:.1f}s)")
    torch.cuda.synchronize()
    xs, ys = {}, {}
    for name, N, K in wl.mats:
        if K not in xs:
            xb = I.x_bf16(I.x_seed(wl.cfg, wl.M, K), wl.M, K, outliers=wl.outliers)
            xs[K] = xb.to(dev)
        if N not in ys:
            ys[N] = torch.empty((wl.M, N), dtype=torch.bfloat16, device=dev)
    need = max(wqd.workspace_bytes(wl.fmt, wl.M, N, K) for _, N, K in wl.mats)
    ws = wqd.get_workspace(need, dev)
    return packed, xs, ys, ws


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
    """Measured HBM read and copy bandwidth (GB/s) with the library's stream kernels."""
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
    e0.record()
    for _ in range(reps):
        wqd.stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    read = n * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    e0.record()
    for _ in range(reps):
        wqd.stream_copy(dst, buf[: n // 2])
    e1.record()
    torch.cuda.synchronize()
    copy = 2 * (n // 2) * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del buf, dst
    torch.cuda.empty_cache()
    return read, copy


def shape_breakdown(wl, packed, xs, ys, ws, stream):
    """Per-matrix timing: each matrix type launched once per layer (every launch
    on a different layer's weights, so HBM-cold), timed with events on the
    launch stream."""
    import torch

    import weight_only_quantized_decode_amd as wqd
    from weight_only_quantized_decode_amd import workloads as WL

    out = {}
    with torch.cuda.stream(stream):
        for j, (name, N, K) in enumerate(wl.mats):
            for layer in range(wl.layers):
                wqd.qgemm(xs[K], packed[layer][j], y=ys[N], workspace=ws)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for layer in range(wl.layers):
                wqd.qgemm(xs[K], packed[layer][j], y=ys[N], workspace=ws)
            e1.record(stream)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / wl.layers
            b = WL.call_bytes(wl.fmt, wl.M, N, K)
            out[name] = {"N": N, "K": K, "us": round(us, 2), "GBps": round(b / (us * 1e-6) / 1e9, 1)}
    return out


def kernel_label(wl):
    """Kernel family and waves per workgroup of every launch in the step."""
    import weight_only_quantized_decode_amd as wqd

    fams = sorted({"%s(%d waves)" % wqd.kernel_path(wl.fmt, wl.M, N, K) for _, N, K in wl.mats})
    return f"{'+'.join(fams)} {wl.fmt} M={wl.M} (every launch of the timed step)"


def profiled_traffic(wl):
    """HBM bytes per launch from the committed counter summary of this workload
    (profiles/traffic_<workload>.json: FETCH_SIZE and WRITE_SIZE runs scaled by
    a copy kernel of known size), or None when there is none or the kernel
    sources changed since the counters were taken."""
    import hashlib

    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"traffic_{wl.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    csrc = os.path.join(root, "weight_only_quantized_decode_amd", "csrc")
    recorded = d.get("kernel_sources_sha256_16", {})
    if sorted(recorded) != sorted(os.listdir(csrc)):  # every source file, no more, no fewer
        return None
    for fn, digest in recorded.items():
        with open(os.path.join(csrc, fn), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest()[:16] != digest:
                return None
    return d["traffic_bytes_per_launch"]


def cpu_baseline(wl):
    """The oracle (as it stands) on a bounded sample of the same workload, on the host cores."""
    import oracle
    import wqd_inputs as I
    from weight_only_quantized_decode_amd import workloads as WL

    name, N, K = max(wl.mats, key=lambda m: m[1] * m[2]) if wl.layers == 1 else wl.mats[0]
    if name in WL.FUSED_PARTS:  # time the first part of a fused matrix (the q matrix)
        name = WL.FUSED_PARTS[name][0]
        N = {n: Nn for n, Nn, _ in (I.LAYER_70B if K == 8192 else I.LAYER_7B)}[name]
    W = I.w_host(I.stack_seed(wl.cfg, 0, MAT_INDEX.get(name, 0)), N, K)
    qw = oracle.quantize(wl.fmt, W)
    x = I.x_bf16_bits(I.x_seed(wl.cfg, wl.M, K), wl.M, K, outliers=wl.outliers)
    reps, t_total = 0, 0.0
    while t_total < 10.0 and reps < 50:
        t0 = time.perf_counter()
        oracle.qgemm_exact(x, qw)
        t_total += time.perf_counter() - t0
        reps += 1
    per_call = t_total / reps
    gbps = WL.call_bytes(wl.fmt, wl.M, N, K) / per_call / 1e9
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
    return {
        "value": round(gbps, 3),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{reps} calls of the float64 oracle (exact dequant, matmul, bf16 rounding) on one "
                  f"{name} matrix {N}x{K} {wl.fmt}, M={wl.M}: {per_call * 1e3:.1f} ms per call; "
                  f"host {model} ({platform.machine()}), {os.cpu_count()} logical CPUs, {affinity} in this "
                  f"process's affinity mask, BLAS threads {threads}",
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


def time_stack(wl, args, with_shapes):
    """Build the packed stack of `wl`, replay its step args.steps times after
    args.warmup untimed steps (HIP events on the launch stream) and free it.
    Returns (ms per step, whether a graph was replayed, per-shape breakdown)."""
    import torch

    import weight_only_quantized_decode_amd as wqd

    log(f"[bench] workload {wl.name}: {wl.launches} launches/step, {wl.step_bytes() / 1e9:.3f} GB/step")
    packed, xs, ys, ws = build_stack(wl)
    stream = torch.cuda.Stream()

    # one graph replay runs every row of packed: the stack once, or each copy
    # of a single matrix once (then the step time is the replay time / copies)
    rows = len(packed) // wl.layers

    def step():
        for row in packed:
            for (name, N, K), pw in zip(wl.mats, row):
                wqd.qgemm(xs[K], pw, y=ys[N], workspace=ws)

    with torch.cuda.stream(stream):
        step()  # eager warm-up (also loads the kernels)
        torch.cuda.synchronize()
        graph = None
        if not args.no_graph:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=stream):
                step()
        run = graph.replay if graph is not None else step
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        log(f"[bench] timing {args.steps} steps")
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps / rows
    shapes = shape_breakdown(wl, packed, xs, ys, ws, stream) if with_shapes and wl.layers > 1 else None
    del graph, packed, xs, ys, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return ms, not args.no_graph, shapes


def spec_accept_timing(B=64, k=4, V=128256, reps=50):
    """The accept / reject step after a verify pass of k + 1 positions: HIP-event
    time per launch and its algorithmic bytes (the accept tests' few values,
    then one target row per sequence, plus its draft row where a draft was
    rejected, read once)."""
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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        wqd.spec_accept(*dev)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    gbps = algo / (us * 1e-6) / 1e9
    return {"B": B, "k": k, "V": V, "mean_kept": round(float(n.mean()), 3), "us_per_launch": round(us, 2),
            "algorithmic_bytes": algo, "GBps": round(gbps, 1), "roofline_frac_hbm": round(gbps / 8000.0, 4)}


def main():
    args = parse()
    args.fused = not args.separate
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this decode layer is measured on a single MI355X "
              "(multi-GPU sharding is a design note, not part of this build).", file=sys.stderr)
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
    wl = make_workload(args)
    ceiling = (None, None) if args.no_ceiling else hbm_ceiling()
    if ceiling[0]:
        log(f"[bench] HBM ceiling: read {ceiling[0]:.0f} GB/s, copy {ceiling[1]:.0f} GB/s")
    ms, graph_used, shapes = time_stack(wl, args, with_shapes=not args.no_shapes)
    alt = None
    if not args.no_alt and wl.layers > 1 and args.workload in ("w4a16_70b", "fp8_70b", "bf16_7b"):
        alt_args = argparse.Namespace(**vars(args))
        alt_args.fused = not args.fused
        alt_wl = make_workload(alt_args)
        alt_ms, _, _ = time_stack(alt_wl, alt_args, with_shapes=False)
        alt_gbps = alt_wl.step_bytes() / (alt_ms / 1e3) / 1e9
        alt = {"workload": alt_wl.name, "launches_per_step": alt_wl.launches, "value": round(alt_gbps, 2),
               "ms_per_step": round(alt_ms, 4), "kernel": kernel_label(alt_wl),
               "pct_measured_read_ceiling": None if ceiling[0] is None else round(100 * alt_gbps / ceiling[0], 2)}
    step_bytes = wl.step_bytes()
    gbps = step_bytes / (ms / 1e3) / 1e9
    per_launch_bytes = step_bytes / wl.launches
    avg_launch_us = ms * 1e3 / wl.launches
    achieved = per_launch_bytes / (avg_launch_us / 1e6) / 1e9
    # the bound of the step: HBM bytes at the vendor bandwidth, or bf16
    # matrix-core FLOPs at the vendor dense peak, whichever takes longer
    flops_per_launch = wl.step_flops() / wl.launches
    if flops_per_launch / (BF16_MFMA_PEAK_TFLOPS * 1e12) > per_launch_bytes / (HBM_PEAK_GBPS * 1e9):
        tf = flops_per_launch / (avg_launch_us / 1e6) / 1e12
        roofline = {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": profiled_traffic(wl)}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": profiled_traffic(wl)}
    roofline.update({"kernel": kernel_label(wl), "avg_launch_us": round(avg_launch_us, 3),
                     "bytes_per_launch": round(per_launch_bytes), "flops_per_launch": round(flops_per_launch)})
    graph = graph_used
    out = {
        "metric": "weight-stream GB/s (% of HBM peak) & us per layer-stack step, 70B W4A16/FP8/BF16",
        "value": round(gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "us_per_step": round(ms * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"w4a16": "u4+bf16", "fp8": "e4m3+bf16", "bf16": "bf16"}[wl.fmt],
        "data": "synthetic",
        "config": {"workload": wl.name, "fmt": wl.fmt, "M": wl.M, "layers": wl.layers,
                   "launches_per_step": wl.launches, "graph": graph, "fused": args.fused,
                   "weight_copies": copies_for(wl),
                   "algorithmic_bytes_per_step": step_bytes},
        "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "hbm_read_ceiling_GBps": None if ceiling[0] is None else round(ceiling[0], 1),
        "hbm_copy_ceiling_GBps": None if ceiling[1] is None else round(ceiling[1], 1),
        "pct_measured_read_ceiling": None if ceiling[0] is None else round(100 * gbps / ceiling[0], 2),
        "pct_measured_copy_ceiling": None if ceiling[1] is None else round(100 * gbps / ceiling[1], 2),
        "roofline": roofline,
    }
    if alt is not None:
        out["separate_layout" if args.fused else "fused_layout"] = alt
    if shapes is not None:
        out["shapes"] = shapes
    if wl.M >= 16:
        tflops = wl.step_flops() / (ms / 1e3) / 1e12
        out["mfma_util_pct"] = round(100 * tflops / BF16_MFMA_PEAK_TFLOPS, 2)
        if not args.no_ceiling:
            peak = mfma_ceiling()
            log(f"[bench] matrix-core ceiling: {peak:.0f} TFLOP/s")
            out["mfma_ceiling_TFLOPs"] = round(peak, 1)
            out["mfma_util_pct_measured_ceiling"] = round(100 * tflops / peak, 2)
    if args.spec:
        out["spec_accept"] = spec_accept_timing()
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
