#!/usr/bin/env python3
"""Benchmark of the DCNv4 spatial aggregation on one MI355X.

A step is one pass of the whole hot path -- forward (dcnv4_forward) and
backward (dcnv4_backward: grad_value and grad_offset_mask) -- over one
batch of the N=64, 56x56, C=64, G=4 (C'=16), 3x3 (K=9), fp32 workload (a
FlashInternImage-T-like first stage; synthetic inputs: value ~ N(0,1),
offsets ~ N(0,2) px, mask ~ N(0,0.5), grad_output ~ N(0,1)).

`value` is sampled points per second, N*Ho*Wo*G*K*C' per step divided by the
step time; every point is sampled by the forward and differentiated by the
backward in the same step.  Inputs are resident in HBM before timing starts;
several buffer sets are rotated so each step reads data that is not in the
256 MB Infinity Cache.

Per-call durations come from HIP events recorded on the stream the library
launches on; the roofline object reports the dominant call.  The CPU oracle
is timed on the host on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DCNv4 fwd/bwd sampled points/s (N·H·W·G·K·C') + achieved HBM GB/s % of peak"
HBM_PEAK_GBPS = 8000.0
KERNEL_SRCS = {op: [os.path.join(ROOT, "dynamic_sparse_vision_amd", "csrc", n) for n in names]
               for op, names in (("dcnv4", ("dcnv4_device.h", "dcnv4_kernels.hip", "dcnv4_tiled.h",
                                            "dcnv4_tiled_fwd.hip", "dcnv4_tiled_bwd_offsets.hip",
                                            "dcnv4_tiled_bwd_values.hip", "dcnv4_tiled_launch.hip",
                                            "dcnv4_api.cpp")),
                                 ("fdattn", ("dcnv4_device.h", "dcnv4_kernels.hip", "fdattn_kernels.hip",
                                             "fdattn_api.cpp")))}
FDA_METRIC = "flash deformable attention fwd/bwd sampled points/s (N·Q·M·L·K·D) + achieved HBM GB/s % of peak"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash(op: str = "dcnv4") -> str:
    """sha256 of the kernel sources and the tile planner of one operator
    (dcnv4 or fdattn): what decides the kernels' memory traffic."""
    h = hashlib.sha256()
    for path in KERNEL_SRCS[op]:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, call: str, op: str = "dcnv4"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    the operator's kernel sources have not changed since the counters were
    taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    wl = t.get("workloads", {}).get(workload, {})
    if wl.get("kernel_source_sha256") != kernel_source_hash(op):
        return None
    entry = wl.get(call)
    return None if entry is None else entry.get("hbm_bytes_per_launch")


def make_sets(w, nsets, dev):
    import torch

    from dynamic_sparse_vision_amd import synth

    v32, om32, g32 = w.make_inputs(pad_fill=0.0, with_grad=True)
    v_st, _ = synth.to_storage(v32, w.dtype)
    om_st, _ = synth.to_storage(om32, w.dtype)
    g_st, _ = synth.to_storage(g32, w.dtype)
    base = dict(v=v_st.to(dev), om=om_st.to(dev), g=g_st.to(dev))
    sets = []
    for i in range(nsets):
        s = {k: (t if i == 0 else t.clone()) for k, t in base.items()}
        s["out"] = torch.empty((w.N, w.Ho, w.Wo, w.C), dtype=s["v"].dtype, device=dev)
        s["gv"] = torch.empty(s["v"].shape, dtype=torch.float32, device=dev)   # fp32 for every dtype
        s["gom"] = torch.empty_like(s["om"])
        sets.append(s)
    return sets, (v32, om32, g32)


def set_bytes_of(w):
    """Bytes of one buffer set: value, offset_mask, grad_output, output,
    grad_offset_mask in the storage dtype, grad_value in fp32."""
    es = w.elem_bytes
    nv = w.N * w.H * w.W * w.C
    nom = w.N * w.Ho * w.Wo * w.P
    no = w.N * w.Ho * w.Wo * w.C
    return es * (nv + 2 * nom + 2 * no) + 4 * nv


def cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, arrays, seconds):
    """The oracle as it stands, forward + backward, on a bounded sample of
    the same workload: batches of images (the forward threads over output
    rows, the backward over images, so a batch of ``nthreads`` images keeps
    every thread busy in both).  Runs are repeated until about ``seconds``
    have passed (at least 3), and the median run is reported; a single-thread
    figure on one image is reported beside it."""
    import oracle

    v32, om32, g32 = arrays
    nthreads = min(int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)), os.cpu_count() or 1)
    lib = oracle.load()
    pts_per_image = w.Ho * w.Wo * w.G * w.K * w.Cg

    def runs(batch, threads, budget, min_runs=3):
        rates, n0 = [], 0
        t_start = time.perf_counter()
        while len(rates) < min_runs or time.perf_counter() - t_start < budget:
            idx = [(n0 + i) % w.N for i in range(batch)]
            n0 += batch
            v, om, g = v32[idx], om32[idx], g32[idx]
            t0 = time.perf_counter()
            oracle.forward(v, om, nthreads=threads, lib=lib, **w.kwargs())
            oracle.backward(v, om, g, nthreads=threads, lib=lib, **w.kwargs())
            rates.append(batch * pts_per_image / (time.perf_counter() - t0))
            if len(rates) >= 50:
                break
        return rates

    all_rates = runs(nthreads, nthreads, 0.75 * seconds)
    one_rates = runs(1, 1, 0.25 * seconds)
    return {"value": statistics.median(all_rates), "unit": "sampled points/s", "cores": nthreads,
            "kind": "oracle",
            "sample": f"median of {len(all_rates)} runs, each forward + backward over a batch of {nthreads} images "
                      f"of the same workload ({nthreads * pts_per_image} points; forward threaded over output "
                      f"rows, backward over images, {nthreads} threads each)",
            "single_thread": {"value": statistics.median(one_rates), "runs": len(one_rates),
                              "sample": "forward + backward of one image, 1 thread"},
            "cpu_model": cpu_model(), "hardware_threads": os.cpu_count()}


def time_configs(path, steps, warmup):
    """One informational JSON line per workload (forward or backward alone),
    with a 512 MB cache flush between calls; written to ``path``."""
    import torch

    from dynamic_sparse_vision_amd import dcnv4
    from dynamic_sparse_vision_amd.workloads import WORKLOADS

    dev = torch.device("cuda")
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    lines = []
    # (label, workload, direction, softmax): every workload in its own
    # direction, plus the DCNv3 softmax mode on the fp32 benchmark shape and
    # the 16-bit backward
    cases = [(name, w, w.direction, False) for name, w in WORKLOADS.items()]
    c2 = WORKLOADS["c2_fwd_fp32_56x56_b64"]
    cases += [("c2_softmax_fwd_fp32_56x56_b64", c2, "fwd", True),
              ("c2_softmax_bwd_fp32_56x56_b64", c2, "bwd", True),
              ("c3a_bwd_fp16_56x56x64_g4", WORKLOADS["c3a_fwd_fp16_56x56x64_g4"], "bwd", False),
              ("c4_bwd_bf16_270x480_k9", WORKLOADS["c4_fwd_bf16_270x480_k9"], "bwd", False)]
    for name, w, direction, softmax in cases:
        sets, _ = make_sets(w, 1, dev)
        s = sets[0]
        kw = dict(w.kwargs(), softmax=softmax)
        if direction == "fwd":
            call = lambda: dcnv4.dcnv4_forward_ex(s["v"], s["om"], s["out"], **kw)  # noqa: E731
            nbytes = w.fwd_bytes()
        else:
            call = lambda: dcnv4.dcnv4_backward_ex(s["v"], s["om"], s["g"], s["gv"], s["gom"], **kw)  # noqa: E731
            nbytes = w.bwd_bytes()
        times = []
        for i in range(warmup + steps):
            flush.fill_(float(i))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            call()
            e1.record()
            e1.synchronize()
            if i >= warmup:
                times.append(e0.elapsed_time(e1))
        ms = statistics.median(times)
        line = {"workload": name, "direction": direction, "softmax": softmax, "dtype": w.dtype, "ms": ms,
                "points_per_s": w.points / (ms * 1e-3), "compulsory_bytes": nbytes,
                "gbps": nbytes / (ms * 1e-3) / 1e9,
                "frac_of_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}
        lines.append(line)
        print(json.dumps(line), file=sys.stderr, flush=True)
        del sets, s
        torch.cuda.empty_cache()
    lines.append(time_layer(flush, steps, warmup))
    print(json.dumps(lines[-1]), file=sys.stderr, flush=True)
    for line in time_fdattn_configs(flush, steps, warmup):
        lines.append(line)
        print(json.dumps(line), file=sys.stderr, flush=True)
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        for line in lines:
            f.write(json.dumps(line) + "\n")


def time_fdattn_configs(flush, steps, warmup):
    """Flash deformable attention, forward and backward alone, on each of
    its full-size workloads (512 MB cache flush between calls)."""
    import torch

    from dynamic_sparse_vision_amd import flash_deform_attn as fda
    from dynamic_sparse_vision_amd import synth
    from dynamic_sparse_vision_amd.workloads import FDA_WORKLOADS

    dev = torch.device("cuda")
    out_lines = []
    for name in ("fda_enc_800x1280_b4_fp32", "fda_enc_800x1280_b4_fp16"):
        w = FDA_WORKLOADS[name]
        v32, la32, g32 = w.make_inputs(pad_fill=0.0)
        v, la, g = (synth.to_storage(a, w.dtype)[0].to(dev) for a in (v32, la32, g32))
        out = torch.empty((w.N, w.queries, w.M, w.D), dtype=v.dtype, device=dev)
        gv = torch.empty(v.shape, dtype=torch.float32, device=dev)
        gla = torch.empty_like(la)
        ws = fda.workspace_for(v, w.shapes, la, w.K)
        for direction in ("fwd", "bwd"):
            if direction == "fwd":
                call = lambda: fda.flash_deform_attn_forward(v, w.shapes, la, out, num_points=w.K)  # noqa: E731
                nbytes = w.fwd_bytes()
            else:
                call = lambda: fda.flash_deform_attn_backward(v, w.shapes, la, g, gv, gla,  # noqa: E731
                                                              num_points=w.K, workspace=ws)
                nbytes = w.bwd_bytes()
            times = []
            for i in range(warmup + steps):
                flush.fill_(float(i))
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                call()
                e1.record()
                e1.synchronize()
                if i >= warmup:
                    times.append(e0.elapsed_time(e1))
            ms = statistics.median(times)
            out_lines.append({"workload": name.replace("fda_", f"fda_{direction}_"), "direction": direction,
                              "softmax": True, "dtype": w.dtype, "ms": ms,
                              "points_per_s": w.points / (ms * 1e-3), "compulsory_bytes": nbytes,
                              "gbps": nbytes / (ms * 1e-3) / 1e9,
                              "frac_of_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS})
        del v, la, g, out, gv, gla, ws
        torch.cuda.empty_cache()
    return out_lines


def time_layer(flush, steps, warmup):
    """The DCNv4 layer (projections through the vendor BLAS, the operator in
    this library) forward + backward on the benchmark shape, random weights."""
    import torch

    from dynamic_sparse_vision_amd import layer
    from dynamic_sparse_vision_amd.workloads import WORKLOADS

    w = WORKLOADS["c2_fwd_fp32_56x56_b64"]
    dev = torch.device("cuda")
    cfg = layer.LayerConfig(channels=w.C, group=w.G)
    weights = {k: v.requires_grad_(True) for k, v in layer.init_weights(cfg, dev, seed=1).items()}
    x = torch.randn(w.N, w.H, w.W, w.C, device=dev, requires_grad=True)
    d_out = torch.randn(w.N, w.Ho, w.Wo, w.C, device=dev)
    times = []
    for i in range(warmup + steps):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        out = layer.layer_forward(x, weights, cfg)
        out.backward(d_out)
        e1.record()
        e1.synchronize()
        if i >= warmup:
            times.append(e0.elapsed_time(e1))
    ms = statistics.median(times)
    return {"workload": "c2_layer_fwd_bwd_fp32_56x56_b64", "direction": "fwd+bwd", "softmax": False,
            "dtype": "fp32", "ms": ms, "points_per_s": w.points / (ms * 1e-3),
            "note": "DCNv4 layer: value / offset-mask / output projections (vendor BLAS) + operator"}


def copy_probe(dev):
    """A copy kernel of known size (256 MiB read + 256 MiB written per
    launch, 3 launches): the calibration of the HBM byte counters."""
    import torch

    src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def fdattn_cpu_baseline(w, arrays, seconds):
    """The oracle as it stands, forward + backward, on blocks of 2048
    queries of one image at a time (cycling over the images and query
    blocks) until the time budget is spent: a bounded sample of the same
    workload."""
    import oracle

    v32, la32, g32 = arrays
    nthreads = min(int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)), os.cpu_count() or 1)
    lib = oracle.load_fdattn()
    qb = 2048
    nblk = -(-w.queries // qb)
    passes, units = 0, 0
    t0 = time.perf_counter()
    elapsed = 0.0
    while elapsed < seconds:
        n, b = divmod(passes, nblk)
        n %= w.N
        sl = slice(b * qb, min(w.queries, (b + 1) * qb))
        la = la32[n:n + 1, sl]
        oracle.fdattn_forward(v32[n:n + 1], w.shapes, la, w.K, nthreads=nthreads, lib=lib)
        oracle.fdattn_backward(v32[n:n + 1], w.shapes, la, g32[n:n + 1, sl], w.K, nthreads=nthreads, lib=lib)
        units += la.shape[1] * w.M
        passes += 1
        elapsed = time.perf_counter() - t0
    pts = units * w.L * w.K * w.D
    return {"value": pts / elapsed, "unit": "sampled points/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{passes} forward + backward passes over blocks of up to {qb} queries of one image "
                      f"of the same workload (the oracle's backward is serial per image), {elapsed:.1f} s"}


def run_fdattn(args):
    """The flash deformable attention step (forward + backward) of
    ``args.workload`` (a FDA_WORKLOADS name); prints one JSON line."""
    import torch

    from dynamic_sparse_vision_amd import dcnv4, synth
    from dynamic_sparse_vision_amd import flash_deform_attn as fda
    from dynamic_sparse_vision_amd.workloads import FDA_WORKLOADS

    dcnv4.load()
    w = FDA_WORKLOADS[args.workload]
    dev = torch.device("cuda")
    print(f"bench: generating {w.name}", file=sys.stderr, flush=True)
    v32, la32, g32 = w.make_inputs(pad_fill=0.0)
    base = {k: synth.to_storage(a, w.dtype)[0].to(dev) for k, a in (("v", v32), ("la", la32), ("g", g32))}
    es = w.elem_bytes
    per_set = es * w.N * (w.S * w.M * w.D + w.queries * w.M * (2 * w.P + 2 * w.D)) + 4 * w.N * w.S * w.M * w.D
    nsets = max(2, -(-(768 * 1024 * 1024) // per_set))
    sets = []
    for i in range(nsets):
        st = {k: (t if i == 0 else t.clone()) for k, t in base.items()}
        st["out"] = torch.empty((w.N, w.queries, w.M, w.D), dtype=st["v"].dtype, device=dev)
        st["gv"] = torch.empty(st["v"].shape, dtype=torch.float32, device=dev)
        st["gla"] = torch.empty_like(st["la"])
        sets.append(st)
    stream = torch.cuda.current_stream()
    # the sorted grad_value path: one workspace, reused by every step
    ws = fda.workspace_for(sets[0]["v"], w.shapes, sets[0]["la"], w.K)

    def step(i, ev=None):
        st = sets[i % nsets]
        if ev is not None:
            ev[0].record(stream)
        fda.flash_deform_attn_forward(st["v"], w.shapes, st["la"], st["out"], num_points=w.K)
        if ev is not None:
            ev[1].record(stream)
        fda.flash_deform_attn_backward(st["v"], w.shapes, st["la"], st["g"], st["gv"], st["gla"], num_points=w.K,
                                       workspace=ws)
        if ev is not None:
            ev[2].record(stream)

    print(f"bench: {nsets} buffer sets of {per_set / 1e6:.0f} MB; warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    fwd_ms = statistics.median(e[0].elapsed_time(e[1]) for e in events)
    bwd_ms = statistics.median(e[1].elapsed_time(e[2]) for e in events)
    print(f"bench: {ms_per_step:.4f} ms/step (forward {fwd_ms:.4f} ms, backward {bwd_ms:.4f} ms)",
          file=sys.stderr, flush=True)
    calls = {"flash_deform_attn_forward": (fwd_ms, w.fwd_bytes()),
             "flash_deform_attn_backward": (bwd_ms, w.bwd_bytes())}
    dom = max(calls, key=lambda c: calls[c][0])
    dom_ms, dom_bytes = calls[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = fdattn_cpu_baseline(w, (v32, la32, g32), args.cpu_seconds)
    line = {
        "metric": FDA_METRIC,
        "value": w.points / (ms_per_step * 1e-3),
        "unit": "sampled points/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32" if w.dtype == "fp32" else w.dtype,
        "data": "synthetic",
        "config": {"workload": f"flash deformable attention forward+backward, N={w.N}, levels "
                               + "/".join(f"{h}x{ww}" for h, ww in w.shapes)
                               + f", Q={w.queries}, M={w.M}, D={w.D}, K={w.K}, {w.dtype}",
                   "points_per_step": w.points},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(w.name, dom, "fdattn"),
                     "kernel": dom, "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_ms": round(dom_ms, 5)},
        "cpu_baseline": cpu,
        "detail": {"forward_ms": round(fwd_ms, 5), "backward_ms": round(bwd_ms, 5),
                   "forward_gbps": round(w.fwd_bytes() / (fwd_ms * 1e-3) / 1e9, 1),
                   "backward_gbps": round(w.bwd_bytes() / (bwd_ms * 1e-3) / 1e9, 1),
                   "forward_bytes": w.fwd_bytes(), "backward_bytes": w.bwd_bytes(),
                   "buffer_sets": nsets, "set_bytes": per_set},
    }
    if args.copy_probe:
        copy_probe(dev)
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--op", choices=("dcnv4", "fdattn"), default="dcnv4",
                    help="dcnv4 (the default step) or flash deformable attention")
    ap.add_argument("--workload", default=None,
                    help="workload name (default: c2_fwd_fp32_56x56_b64, or fda_enc_800x1280_b4_fp32 "
                         "with --op fdattn)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-detail", action="store_true",
                    help="skip the cold per-workload forward timings and the batch-share timings")
    ap.add_argument("--configs-out", default=None,
                    help="also time every workload alone and write JSON lines there")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: --gpus {args.gpus} (WORLD_SIZE {world}) requested, but this operator "
              "library is measured on one GPU only; the multi-GPU path (batch sharding, no "
              "communication inside the operator) is not built. Run with --gpus 1.",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.op == "fdattn":
        args.workload = args.workload or "fda_enc_800x1280_b4_fp32"
        run_fdattn(args)
        return
    args.workload = args.workload or "c2_fwd_fp32_56x56_b64"
    run_dcnv4(args)


def measured_kernel(workload: str, call: str):
    """The dominant single kernel of ``call`` on ``workload`` as the committed
    rocprofv3 kernel trace reports it (name, average duration), if the kernel
    sources have not changed since the trace was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    wl = t.get("workloads", {}).get(workload, {})
    if wl.get("kernel_source_sha256") != kernel_source_hash("dcnv4"):
        return None
    entry = wl.get(call) or {}
    return entry.get("dominant_kernel")


def cold_ms(call, flush, stream, calls=20, warmup=3):
    """Median duration (ms, HIP events on ``stream``) of ``calls`` calls, each
    after a 512 MB fill that evicts the L2 and Infinity Cache, so every call
    reads its inputs from HBM."""
    import torch

    times = []
    for i in range(warmup + calls):
        flush.fill_(float(i))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        e1.synchronize()
        if i >= warmup:
            times.append(e0.elapsed_time(e1))
    return statistics.median(times)


def forward_detail(flush, stream):
    """Every forward workload of the benchmark configurations other than the
    step's own, alone and cold (median of 20 calls): ms, compulsory GB/s and
    the fraction of 8 TB/s; plus the bytes-weighted aggregate of the four
    fp16 stage shapes."""
    import torch

    from dynamic_sparse_vision_amd import dcnv4, synth
    from dynamic_sparse_vision_amd.workloads import WORKLOADS

    dev = torch.device("cuda")
    out = {}
    agg_bytes, agg_ms = 0, 0.0
    for name in ("c3a_fwd_fp16_56x56x64_g4", "c3b_fwd_fp16_28x28x128_g8", "c3c_fwd_fp16_14x14x256_g16",
                 "c3d_fwd_fp16_7x7x512_g32", "c4_fwd_bf16_270x480_k9", "c4_fwd_bf16_270x480_k8",
                 "c1_fwd_fp32_14x14"):
        w = WORKLOADS[name]
        print(f"bench: forward {name}", file=sys.stderr, flush=True)
        v32, om32 = w.make_inputs(pad_fill=0.0)
        v = synth.to_storage(v32, w.dtype)[0].to(dev)
        om = synth.to_storage(om32, w.dtype)[0].to(dev)
        y = torch.empty((w.N, w.Ho, w.Wo, w.C), dtype=v.dtype, device=dev)
        ms = cold_ms(lambda: dcnv4.dcnv4_forward(v, om, y, **w.kwargs()), flush, stream)
        nbytes = w.fwd_bytes()
        gbps = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"dtype": w.dtype, "ms": round(ms, 5), "points_per_s": w.points / (ms * 1e-3),
                     "compulsory_bytes": nbytes, "gbps": round(gbps, 1),
                     "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4)}
        if name.startswith("c3"):
            agg_bytes += nbytes
            agg_ms += ms
        del v, om, y
    gbps = agg_bytes / (agg_ms * 1e-3) / 1e9
    out["c3_aggregate_fwd_fp16"] = {"ms": round(agg_ms, 5), "compulsory_bytes": agg_bytes, "gbps": round(gbps, 1),
                                    "frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
                                    "note": "the four fp16 stage shapes, sum of bytes / sum of times"}
    torch.cuda.empty_cache()
    return out


def share_detail(flush, stream):
    """The step's workload at the batch share one GPU of 8 (N=8) or 4 (N=16)
    would hold, cold: forward and backward ms and fractions of 8 TB/s."""
    import torch

    from dynamic_sparse_vision_amd import dcnv4
    from dynamic_sparse_vision_amd.workloads import WORKLOADS

    base = WORKLOADS["c2_fwd_fp32_56x56_b64"]
    out = {}
    for n in (8, 16, 64):
        w = dataclasses.replace(base, N=n)
        gen = torch.Generator(device="cuda").manual_seed(n)
        v = torch.randn((n, w.H, w.W, w.C), device="cuda", generator=gen)
        om = 2.0 * torch.randn((n, w.Ho, w.Wo, w.P), device="cuda", generator=gen)
        g = torch.randn((n, w.Ho, w.Wo, w.C), device="cuda", generator=gen)
        y = torch.empty_like(g)
        gv, gom = torch.empty_like(v), torch.empty_like(om)
        f_ms = cold_ms(lambda: dcnv4.dcnv4_forward(v, om, y, **w.kwargs()), flush, stream)
        b_ms = cold_ms(lambda: dcnv4.dcnv4_backward(v, om, g, gv, gom, **w.kwargs()), flush, stream)
        out[f"N={n}"] = {"forward_ms": round(f_ms, 5), "backward_ms": round(b_ms, 5),
                         "forward_frac_of_peak": round(w.fwd_bytes() / (f_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                         "backward_frac_of_peak": round(w.bwd_bytes() / (b_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
        del v, om, g, y, gv, gom
    torch.cuda.empty_cache()
    return out


def launch_floor(stream):
    """Launch-latency floor on the launch stream: a one-element fill kernel,
    median of 50 calls."""
    import torch

    x = torch.empty(1, device="cuda")
    times = []
    for i in range(60):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        x.fill_(float(i))
        e1.record(stream)
        e1.synchronize()
        if i >= 10:
            times.append(e0.elapsed_time(e1))
    return round(statistics.median(times), 5)


def first_call_parity(w, s, arrays):
    """The first step's forward and backward on the first and last image of
    the batch against the oracle (fp32 tolerance 1e-5 + 1e-5 |ref|)."""
    import numpy as np

    import oracle

    v32, om32, g32 = arrays
    worst = 0.0
    ok = True
    for n in (0, w.N - 1):
        sl = slice(n, n + 1)
        ref = oracle.forward(v32[sl], om32[sl], **w.kwargs())
        rgv, rgom = oracle.backward(v32[sl], om32[sl], g32[sl], **w.kwargs())
        for got, want in ((s["out"][sl], ref), (s["gv"][sl], rgv), (s["gom"][sl], rgom)):
            a = got.float().cpu().numpy().astype(np.float64)
            err = np.abs(a - want)
            worst = max(worst, float(err.max()))
            ok = ok and bool((err <= 1e-5 + 1e-5 * np.abs(want)).all())
    return {"images": [0, w.N - 1], "max_abs_err": worst, "ok": ok,
            "tolerance": "1e-5 + 1e-5*|ref| (forward, grad_value, grad_offset_mask)"}


def run_dcnv4(args):
    import torch

    from dynamic_sparse_vision_amd import dcnv4
    from dynamic_sparse_vision_amd.workloads import WORKLOADS

    dcnv4.load()  # fails loudly if the HIP library is missing
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda")
    print(f"bench: generating {w.name}", file=sys.stderr, flush=True)
    per_set = set_bytes_of(w)
    nsets = max(2, -(-(768 * 1024 * 1024) // per_set))
    sets, arrays = make_sets(w, nsets, dev)
    kw = w.kwargs()
    stream = torch.cuda.current_stream()

    def step(i, ev=None):
        s = sets[i % nsets]
        if ev is not None:
            ev[0].record(stream)
        dcnv4.dcnv4_forward(s["v"], s["om"], s["out"], **kw)
        if ev is not None:
            ev[1].record(stream)
        dcnv4.dcnv4_backward(s["v"], s["om"], s["g"], s["gv"], s["gom"], **kw)
        if ev is not None:
            ev[2].record(stream)

    # the first call of the run, checked against the oracle
    step(0)
    torch.cuda.synchronize()
    parity = first_call_parity(w, sets[0], arrays) if w.dtype == "fp32" else None
    print(f"bench: first-call parity {parity}", file=sys.stderr, flush=True)
    if parity is not None and not parity["ok"]:
        raise SystemExit("bench.py: the first call disagrees with the oracle")
    print(f"bench: {nsets} buffer sets of {per_set / 1e6:.0f} MB; warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    fwd_times = [e[0].elapsed_time(e[1]) for e in events]
    bwd_times = [e[1].elapsed_time(e[2]) for e in events]
    fwd_ms, bwd_ms = statistics.median(fwd_times), statistics.median(bwd_times)
    print(f"bench: {ms_per_step:.4f} ms/step (forward {fwd_ms:.4f} ms, backward {bwd_ms:.4f} ms, medians)",
          file=sys.stderr, flush=True)

    fwd_bytes = w.fwd_bytes()
    bwd_bytes = w.bwd_bytes()
    calls = {"dcnv4_forward": (fwd_ms, fwd_bytes), "dcnv4_backward": (bwd_ms, bwd_bytes)}
    dom = max(calls, key=lambda c: calls[c][0])
    dom_ms, dom_bytes = calls[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(w.name, dom),
                "kernel": dom,
                "algorithmic_bytes_per_launch": dom_bytes,
                "avg_launch_ms": round(dom_ms, 5),
                "launch_ms_stat": "median over the timed steps",
                "dominant_kernel": measured_kernel(w.name, dom)}

    del sets
    torch.cuda.empty_cache()
    flush = torch.empty(512 * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    detail = {
        "forward_ms": round(fwd_ms, 5), "backward_ms": round(bwd_ms, 5),
        "forward_gbps": round(fwd_bytes / (fwd_ms * 1e-3) / 1e9, 1),
        "backward_gbps": round(bwd_bytes / (bwd_ms * 1e-3) / 1e9, 1),
        "forward_bytes": fwd_bytes, "backward_bytes": bwd_bytes,
        "buffer_sets": nsets, "set_bytes": per_set,
        "first_call_parity": parity,
    }
    if not args.no_detail:
        detail["launch_floor_ms"] = launch_floor(stream)
        detail["forward_workloads_cold"] = forward_detail(flush, stream)
        detail["one_gpu_share_cold"] = share_detail(flush, stream)

    cpu = None
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, arrays, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": w.points / (ms_per_step * 1e-3),
        "unit": "sampled points/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == "fp32" else w.dtype,
        "data": "synthetic",
        "config": {"workload": f"DCNv4 forward+backward, N={w.N}, {w.H}x{w.W}, C={w.C}, G={w.G}, "
                               f"C'={w.Cg}, K={w.K}, {w.dtype}",
                   "N": w.N, "H": w.H, "W": w.W, "C": w.C, "G": w.G, "K": w.K,
                   "points_per_step": w.points},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": detail,
    }
    if args.configs_out:
        time_configs(args.configs_out, steps=max(20, args.steps), warmup=5)
    if args.copy_probe:
        copy_probe(dev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
