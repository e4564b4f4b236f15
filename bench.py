#!/usr/bin/env python3
"""Benchmark of the ConvRot W4A4 linear on one MI355X.

One step = one complete ``convrot_linear`` call (rotation, row absmax and
INT4 quantization of the activations, the integer product against the weight
image -- on the FP6 matrix cores, where the INT4 codes are exact e2m3 values,
or on the INT8 ones, as the library's plan picks -- and the scale + bias
epilogue to bf16) over one batch of seeded
synthetic input already resident in HBM.  The weight is prepared once before
timing (an offline step; its time is reported separately).  Steps cycle
through enough independent buffer sets (>= 512 MiB in total) that the 256 MiB
Infinity Cache cannot serve the weights from a previous step.

Prints one JSON line on stdout.  ``value`` is effective TOPS = 2*M*N*K per
step time (the K timed steps run as one HIP graph).  ``roofline`` rates the
dominant kernel -- the GEMM, or the whole linear where it is a single kernel
(M <= 4) -- from its average launch duration (a pair of HIP events on the
launch stream around each launch) against the dense peak of the matrix
cores it runs on (FP6 10.1 POP/s, INT8 5.0) or, for weight-streaming shapes,
the HBM peak;
``traffic`` comes from the committed rocprofv3 byte counters when they match
the current kernel source.  ``cpu_baseline`` is the CPU oracle timed on a
bounded sample of the same workload on this host's cores.
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

METRIC = "ConvRot W4A4 linear effective TOPS + GB/s and % of roofline, FLUX shapes"
DEFAULT_WORKLOAD = "flux_qkv_m1536_k3072_n9216"
PEAK_INT8_TOPS = 5000.0      # MI355X dense INT8 matrix-core peak, 5.0 POP/s
PEAK_FP6_TOPS = 10100.0      # MI355X dense FP6 / FP4 matrix-core peak, 10.1 POP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
KERNEL_SOURCE = os.path.join(ROOT, "w4a4_rotated_bit_amd", "csrc", "kernels.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(workload: str, gemm_ops_unit_launches: int):
    """HBM bytes per GEMM launch from the committed rocprofv3 counter summary,
    or None when there is none or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"gemm_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return int(float(vals["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, target_s: float, g: int, path: str = "w4a4"):
    """The oracle's linear on a bounded sample of the workload: as many rows of
    X as fit in about target_s seconds (the whole X, repeated, when one pass is
    shorter).  The weight is prepared by the oracle beforehand, untimed, like
    the GPU's offline weight step."""
    import oracle
    wl = inp["workload"]
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    qw, sw = oracle.prepare_weight(inp["w"], g, threads=threads)
    log(f"cpu baseline: oracle weight preparation {time.perf_counter() - t0:.1f} s (untimed)")
    probe = min(wl.M, 8)
    t0 = time.perf_counter()
    run = oracle.linear_w4a16 if path == "w4a16" else oracle.linear
    run(inp["x"][:probe], qw, sw, inp["bias"], g, threads=threads)
    dt = time.perf_counter() - t0
    rows = int(max(probe, min(wl.M, probe * target_s / max(dt, 1e-6))))
    reps = 1
    if rows == wl.M:
        reps = int(max(1, min(20, target_s / max(dt * wl.M / probe, 1e-6))))
    t0 = time.perf_counter()
    for _ in range(reps):
        run(inp["x"][:rows], qw, sw, inp["bias"], g, threads=threads)
    dt = time.perf_counter() - t0
    tops = 2.0 * rows * reps * wl.N * wl.K / dt / 1e12
    return {"value": tops, "unit": "TOPS", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {wl.M} rows of X x {reps} pass(es) against the full {wl.N}x{wl.K} weight "
                      + ("(W4A16 linear: rotation, bf16 rounding, binary64 dot products, epilogue)" if path == "w4a16"
                         else "(complete linear: rotation, quantization, int64 dot products, epilogue)")
                      + f", {dt:.2f} s"}


def copy_probe(nbytes: int, reps: int):
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": nbytes, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-bytes", type=float, default=512 * 2**20, help="total bytes of rotating buffer sets")
    ap.add_argument("--copy-probe", type=int, default=0, help="only run a device copy of this many bytes")
    ap.add_argument("--no-graph", action="store_true", help="launch the timed steps one by one instead of as a graph")
    ap.add_argument("--path", choices=("w4a4", "w4a16"), default="w4a4",
                    help="w4a16: weight-only INT4 with bf16 rotated activations (M <= 32)")
    ap.add_argument("--rotation", choices=("sylvester", "regular"), default="sylvester",
                    help="Hadamard matrix of the rotation (the regular one adds sign flips and a permutation)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from w4a4_rotated_bit_amd import binding, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args.copy_probe, 10)
        return

    binding.load()
    inp = synth.make(args.workload)
    wl = inp["workload"]
    M, N, K, g = wl.M, wl.N, wl.K, wl.g
    if args.rotation == "regular":
        g |= binding.CONVROT_REGULAR_HADAMARD
    log(f"workload {wl.name}: M={M} N={N} K={K} g={wl.g} rotation={args.rotation}")

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    X0, W0, B0 = dev_bf16(inp["x"]), dev_bf16(inp["w"]), dev_bf16(inp["bias"])
    # offline weight preparation (timed separately, informational)
    image0, sw0 = binding.convrot_prepare_weight(W0, g)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(3):
        binding.convrot_prepare_weight(W0, g, image=image0, sw=sw0)
    ev1.record()
    torch.cuda.synchronize()
    weight_prep_ms = ev0.elapsed_time(ev1) / 3

    w4a16 = args.path == "w4a16"
    if w4a16 and M > 32:
        log(f"--path w4a16 covers M <= 32 (the weight-bound regime); {wl.name} has M = {M}")
        sys.exit(2)
    ws_bytes = (binding.convrot_w4a16_workspace_bytes(M, K, g) if w4a16
                else binding.convrot_workspace_bytes(M, K, N, g))
    set_bytes = X0.numel() * 2 + image0.numel() + sw0.numel() * 4 + B0.numel() * 2 + M * N * 2 + ws_bytes
    n_sets = int(min(64, max(1, -(-args.cold_bytes // set_bytes))))
    sets = []
    for i in range(n_sets):
        sets.append(dict(X=X0.clone(), image=image0.clone(), sw=sw0.clone(), bias=B0.clone(),
                         Y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                         ws=torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")))
    del W0
    torch.cuda.synchronize()
    log(f"{n_sets} buffer sets of {set_bytes / 2**20:.1f} MiB each")

    linear = binding.convrot_linear_w4a16 if w4a16 else binding.convrot_linear

    def step(i):
        s = sets[i % n_sets]
        linear(s["X"], s["image"], s["sw"], s["bias"], N, g, Y=s["Y"], workspace=s["ws"])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # The K timed steps are captured once into a HIP graph and replayed, so the
    # GPU-side throughput is measured rather than the host's launch rate (a
    # small linear runs faster than Python can enqueue it).
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(args.steps):
                step(i)
        graph.replay()  # untimed replay: first-touch costs of the graph
        torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # Launch durations of the two kernels, timed with a pair of HIP events
    # around every launch on the launch stream, in the same prep -> GEMM order
    # and over the same buffer rotation as the timed steps.  A bounded spin
    # kernel holds the stream while the host enqueues, so that no event
    # measures the host's launch latency.
    # (the W4A16 path is timed as one unit: its bf16 activation rows and their product)
    single = w4a16 or binding.convrot_linear_kernel_count(M, K, N, g) == 1

    def launch_avg_ms(n):
        """Average launch durations: (prep, gemm) for the two-kernel path,
        (None, whole linear) where the linear is a single kernel."""
        pairs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n)]
        hold = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        hold.record()
        torch.cuda._sleep(int(2.0e5 * n))  # ~80 us per launch pair at 2.4 GHz
        t0 = time.perf_counter()
        for i in range(n):
            s = sets[i % n_sets]
            e = pairs[i]
            e[0].record()
            if single:
                e[1].record()
                linear(s["X"], s["image"], s["sw"], s["bias"], N, g, Y=s["Y"], workspace=s["ws"])
            else:
                binding.convrot_prepare_activations(s["X"], g, s["ws"])
                e[1].record()
                binding.convrot_gemm(s["ws"], M, K, s["image"], s["sw"], s["bias"], N, g, Y=s["Y"])
            e[2].record()
        host_ms = (time.perf_counter() - t0) * 1e3
        torch.cuda.synchronize()
        held_ms = hold.elapsed_time(pairs[0][0])
        if held_ms < host_ms:
            log(f"warning: stream held {held_ms:.2f} ms < host enqueue {host_ms:.2f} ms; "
                "launch durations may include host latency")
        prep = None if single else float(np.mean([e[0].elapsed_time(e[1]) for e in pairs]))
        gemm = float(np.mean([e[1].elapsed_time(e[2]) for e in pairs]))
        return prep, gemm

    n_k = max(20, min(args.steps, 200))
    prep_ms, gemm_ms = launch_avg_ms(n_k)

    ops = 2.0 * M * N * K
    value = ops / (ms_per_step * 1e-3) / 1e12
    gbs = wl.bytes_alg / (ms_per_step * 1e-3) / 1e9
    traffic = None if w4a16 else read_traffic(wl.name, 1)
    # Roofline of the GEMM kernel: the matrix-core peak for compute-bound
    # shapes; for weight-streaming shapes (arithmetic intensity below the ridge
    # point) the HBM peak, with the kernel's algorithmic bytes: packed weight
    # and activation codes, weight/activation scales, bias and Y.
    # (a single-kernel linear moves the whole path's algorithmic bytes)
    gemm_bytes = wl.bytes_alg if single else N * K // 2 + M * K // 2 + 4 * M + 4 * N + 2 * N + 2 * M * N
    kind = 0 if w4a16 else binding.convrot_linear_plan(M, K, N, g)["mfma"]
    peak = PEAK_FP6_TOPS if kind == binding.CONVROT_MFMA_FP6 else PEAK_INT8_TOPS
    if ops / wl.bytes_alg >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        ach = ops / (gemm_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TOP/s",
                "frac": round(ach / peak, 4), "traffic": traffic}
    else:
        ach = gemm_bytes / (gemm_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seconds, g, args.path)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w4a16 else ("fp6" if kind == binding.CONVROT_MFMA_FP6 else "int8"),
        "data": "synthetic",
        "config": {"workload": wl.name, "M": M, "K": K, "N": N, "group": wl.g, "path": args.path,
                   "rotation": args.rotation,
                   "x_kind": wl.x_kind,
                   "outlier_channels": wl.outlier_count, "cold_buffer_sets": n_sets,
                   "timed_as": "hip_graph" if graph is not None else "stream_launches"},
        "gbps": round(gbs, 1),
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "mfma_peak_tops": peak,
        "mfma_frac": round(value / peak, 4),
        "kernel_us": ({"linear": round(gemm_ms * 1e3, 2)} if single else
                      {"prep": round(prep_ms * 1e3, 2), "gemm": round(gemm_ms * 1e3, 2)}),
        "weight_prep_ms": round(weight_prep_ms, 4),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
