#!/usr/bin/env python3
"""Benchmark of the ConvRot W4A4 linear on one MI355X.

One step = one complete ``convrot_linear`` call (rotation, row absmax and
INT4 quantization of the activations, the integer product against the weight
image -- on the FP6 matrix cores, where the INT4 codes are exact e2m3 values,
or on the INT8 ones, as the library's plan picks -- and the scale + bias
epilogue to bf16) over one batch of seeded synthetic input already resident
in HBM.  The weight is prepared once before timing (an offline step; its time
is reported separately).  Steps cycle through enough independent buffer sets
(>= 512 MiB in total) that the 256 MiB Infinity Cache cannot serve the
weights from a previous step.

Prints one JSON line on stdout.  The headline is the fused-QKV workload
(1536 x 3072 -> 9216): ``value`` is effective TOPS = 2*M*N*K per step, the K
timed steps replayed as one HIP graph between two events.  The same graph is
replayed five more times for the median and minimum step time.

``roofline`` rates the dominant kernel -- the GEMM, or the whole linear where
it is a single kernel (M <= 4) -- from its average launch duration, measured
as a graph of back-to-back launches of that kernel alone between two events
on the launch stream (per-launch event pairs add about 2 us to a short
kernel), against the dense peak of the matrix cores it runs on (FP6 10.1
POP/s, INT8 5.0) or, for weight-streaming shapes, against the HBM peak (8
TB/s) with the kernel's algorithmic bytes.  ``traffic`` comes from the
committed rocprofv3 byte counters when they match the current kernel source.

``per_config`` measures every other workload the same way (tiny, group-64,
MLP up and down, decode M = 1 / 4 / 16, the 4096-row stress point, the QKV
shape with an INT4-only weight image).  ``baselines`` holds the empty-dispatch
floor, a 256 MiB device copy and, at the QKV shape, the vendor INT8 GEMM and
the dense bf16 linear.  ``cpu_baseline`` is the CPU oracle timed on a bounded
sample of the headline workload on this host's cores; ``cpu_single_thread``
times it on one core for the small workloads.
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
PER_CONFIG = ["tiny_m64_k1024_n1024_g256", "g64_m128_k2048_n2048", "flux_mlp_up_m1536_k3072_n12288",
              "flux_mlp_down_m1536_k12288_n3072", "decode_m1_k3072_n12288", "decode_m4_k3072_n12288",
              "decode_m16_k3072_n12288", "stress_m4096_k3072_n3072", "flux_qkv_m1536_k3072_n9216+int4"]
SINGLE_THREAD = ["tiny_m64_k1024_n1024_g256", "g64_m128_k2048_n2048", "decode_m1_k3072_n12288",
                 "decode_m4_k3072_n12288", "decode_m16_k3072_n12288"]
PEAK_INT8_TOPS = 5000.0      # MI355X dense INT8 matrix-core peak, 5.0 POP/s
PEAK_FP6_TOPS = 10100.0      # MI355X dense FP6 / FP4 matrix-core peak, 10.1 POP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
KERNEL_SOURCE = os.path.join(ROOT, "w4a4_rotated_bit_amd", "csrc", "kernels.hip")
BATCHES = 5


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(workload: str):
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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
    return {"value": tops, "unit": "TOPS", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{rows} of {wl.M} rows of X x {reps} pass(es) against the full {wl.N}x{wl.K} weight "
                      + ("(W4A16 linear: rotation, bf16 rounding, binary64 dot products, epilogue)" if path == "w4a16"
                         else "(complete linear: rotation, quantization, int64 dot products, epilogue)")
                      + f", {dt:.2f} s"}


def cpu_single_thread(names):
    """The oracle's whole linear on one thread for small workloads (weight
    prepared beforehand on all cores, untimed)."""
    import oracle
    from w4a4_rotated_bit_amd import synth
    out = {}
    weights = {}  # the decode shapes share one weight
    for name in names:
        inp = synth.make(name)
        wl = inp["workload"]
        key = (wl.seed, wl.sub, wl.N, wl.K, wl.g)
        if key not in weights:
            weights[key] = oracle.prepare_weight(inp["w"], wl.g)
        qw, sw = weights[key]
        t0 = time.perf_counter()
        oracle.linear(inp["x"], qw, sw, inp["bias"], wl.g, threads=1)
        dt = time.perf_counter() - t0
        out[name] = {"ms": round(dt * 1e3, 2), "tops": round(wl.ops / dt / 1e12, 5)}
    return out


def summarize_profile(path: str) -> str:
    """Per-kernel launch statistics (and counter averages, when collected)
    from a rocprofv3 results database (rocpd SQLite).  Prep launches that no
    GEMM follows are the offline weight preparation and are reported apart
    from the activation launches (a profile of the prep kernel alone should
    therefore include the GEMM launches)."""
    import collections
    import re
    import sqlite3
    db = sqlite3.connect(path)
    rows = list(db.execute("select dispatch_id, name, duration, grid_x, workgroup_x from kernels "
                           "order by dispatch_id"))

    def short(n):
        m = re.match(r"(?:void )?convrot::(\w+)<(.*)>\(", n)
        return f"{m.group(1)}<{m.group(2)}>" if m else n.split("(")[0][:70]

    gemm_like = ("gemm", "skinny", "small_m", "w4a16_kernel")
    stats, label = collections.defaultdict(list), {}
    for i, (d, n, dur, gx, wx) in enumerate(rows):
        # an activation prep is always followed by the GEMM that reads it
        nxt = rows[i + 1][1] if i + 1 < len(rows) else ""
        weight = "prep" in n and not any(k in nxt for k in gemm_like)
        k = short(n) + (" [not followed by a GEMM: weight prep]" if weight else "")
        stats[k].append(dur / 1e3)
        label[d] = k
    out = [f"{'kernel':72s} {'calls':>5s} {'avg_us':>9s} {'median_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
    for k, v in sorted(stats.items(), key=lambda kv: -sum(kv[1])):
        v.sort()
        out.append(f"{k:72s} {len(v):5d} {sum(v) / len(v):9.2f} {v[len(v) // 2]:9.2f} {v[0]:9.2f} {v[-1]:9.2f}")
    pmc = list(db.execute("select dispatch_id, counter_name, counter_value from pmc_events"))
    if pmc:
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        for d, c, v in pmc:
            per[d][c] += v
        agg = collections.defaultdict(lambda: collections.defaultdict(list))
        for d, cs in per.items():
            for c, v in cs.items():
                agg[label.get(d, "?")][c].append(v)
        out.append("counters (average per dispatch, summed over the GPU):")
        for k, cs in agg.items():
            out.append(f"  {k}: " + ", ".join(f"{c}={sum(v) / len(v):.1f}" for c, v in sorted(cs.items())))
    return "\n".join(out)


def _pmc_per_kernel(path: str, counter: str):
    """{kernel name: (dispatches, mean counter value per dispatch)} of one
    counter in a rocprofv3 results database."""
    import collections
    import sqlite3
    db = sqlite3.connect(path)
    names = dict(db.execute("select dispatch_id, name from kernels"))
    per = collections.defaultdict(float)
    for d, c, v in db.execute("select dispatch_id, counter_name, counter_value from pmc_events"):
        if c == counter:
            per[d] += v
    agg = collections.defaultdict(list)
    for d, v in per.items():
        agg[names.get(d, "?")].append(v)
    return {k: (len(v), sum(v) / len(v)) for k, v in agg.items()}


def traffic_summary(workload: str, fetch_db: str, write_db: str, copy_fetch_db: str, copy_write_db: str) -> str:
    """HBM traffic of the dominant product kernel of one workload, from
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch, each in its own run), scaled
    by what the same counters read on a plain 256 MiB device copy."""
    product = ("gemm", "skinny", "small_m", "w4a16_kernel")
    fetch = {k: v for k, v in _pmc_per_kernel(fetch_db, "FETCH_SIZE").items() if any(p in k for p in product)}
    write = _pmc_per_kernel(write_db, "WRITE_SIZE")
    # the product kernel with the most dispatches is the timed one (the
    # weight-prep and baseline launches are few)
    kernel = max(fetch, key=lambda k: fetch[k][0])
    n, fkib = fetch[kernel]
    _, wkib = write[kernel]
    cf = max(_pmc_per_kernel(copy_fetch_db, "FETCH_SIZE").values(), key=lambda t: t[1])[1]
    cw = max(_pmc_per_kernel(copy_write_db, "WRITE_SIZE").values(), key=lambda t: t[1])[1]
    copied_kib = 256 * 1024
    fs, ws = copied_kib / cf, copied_kib / cw
    fb, wb = int(fkib * 1024 * fs), int(wkib * 1024 * ws)
    short = kernel.split("(")[0].replace("void ", "")
    cmd = ("rocprofv3 --pmc {c} --kernel-include-regex 'gemm|skinny|small_m|prep' -d <out> -o run -- "
           f"python3 bench.py --workload {workload} --no-per-config --no-cpu-baseline --no-baselines "
           "--steps 20 --warmup 5")
    lines = [
        f"# HBM-side traffic of {short} on {workload} (per dispatch)",
        "# counters, each in its own run:",
        "#   " + cmd.format(c="FETCH_SIZE"),
        "#   " + cmd.format(c="WRITE_SIZE"),
        "# calibration, the same counters on a plain 256 MiB device copy:",
        "#   rocprofv3 --pmc FETCH_SIZE -d <out> -o run -- python3 bench.py --copy-probe 268435456",
        "#   (same with WRITE_SIZE)",
        "# summary: python3 bench.py --workload " + workload +
        " --write-traffic <fetch db> <write db> <copy fetch db> <copy write db>",
        "# scale = copied KiB / counter KiB on the copy; traffic = counter * scale",
        "# (L2-miss bytes toward the fabric: part may be served by the Infinity Cache)",
        f"fetch_kib_per_dispatch = {fkib:.1f}",
        f"write_kib_per_dispatch = {wkib:.1f}",
        f"copy_fetch_kib = {cf:.1f}",
        f"copy_write_kib = {cw:.1f}",
        f"fetch_scale = {fs:.4f}",
        f"write_scale = {ws:.4f}",
        f"fetch_bytes_per_launch = {fb}",
        f"write_bytes_per_launch = {wb}",
        f"hbm_bytes_per_launch = {fb + wb}",
        f"dispatches_sampled = {n}",
        f"kernel_source_sha256_16 = {kernel_source_hash()}",
    ]
    return "\n".join(lines)


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


SPIN_CYCLES = 10_000_000  # GPU clock cycles of the spin kernel ahead of timed eager launches


def graph_times_ms(fn, n: int, warmup: int, batches: int):
    """fn(i) enqueues one unit of work.  Captures n units in a HIP graph,
    replays it once untimed, then once timed (the primary figure) and
    `batches` more times; returns (primary ms per unit, [ms per unit of each
    batch]).  The primary replay starts right after a synchronize, on a GPU
    that has just gone idle: on the compute-bound shapes its first
    milliseconds run at a lower clock, so it is several percent slower than
    the back-to-back batches that follow (both are reported)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n):
            fn(i)
    graph.replay()  # first-touch costs of the graph
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(batches + 2)]
    ev[0].record()
    graph.replay()
    ev[1].record()
    for b in range(batches):
        graph.replay()
        ev[b + 2].record()
    torch.cuda.synchronize()
    primary = ev[0].elapsed_time(ev[1]) / n
    per_batch = [ev[b + 1].elapsed_time(ev[b + 2]) / n for b in range(batches)]
    del graph
    return primary, per_batch


def eager_times_ms(fn, n: int, warmup: int):
    """Average ms per call of n eager launches of fn between two events.  A
    spin kernel ahead of the start event holds the stream while the host
    enqueues the n launches, so host launch latency is not timed."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(SPIN_CYCLES)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def measure(name: str, steps: int, warmup: int, cold_bytes: float, rotation: str = "sylvester",
            path: str = "w4a4", want_inputs: bool = False):
    """Times one workload.  name may carry "+int4" (INT4-only weight image)."""
    import torch
    from w4a4_rotated_bit_amd import binding, synth

    base, _, variant = name.partition("+")
    inp = synth.make(base)
    wl = inp["workload"]
    M, N, K = wl.M, wl.N, wl.K
    g = wl.g
    if rotation == "regular":
        g |= binding.CONVROT_REGULAR_HADAMARD
    if variant == "int4":
        g |= binding.CONVROT_INT4_IMAGE
    w4a16 = path == "w4a16"

    def dev_bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()

    X0, W0, B0 = dev_bf16(inp["x"]), dev_bf16(inp["w"]), dev_bf16(inp["bias"])
    image0, sw0 = binding.convrot_prepare_weight(W0, g)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(3):
        binding.convrot_prepare_weight(W0, g, image=image0, sw=sw0)
    ev1.record()
    torch.cuda.synchronize()
    weight_prep_ms = ev0.elapsed_time(ev1) / 3
    del W0

    ws_bytes = (binding.convrot_w4a16_workspace_bytes(M, K, g) if w4a16
                else binding.convrot_workspace_bytes(M, K, N, g))
    set_bytes = X0.numel() * 2 + image0.numel() + sw0.numel() * 4 + B0.numel() * 2 + M * N * 2 + ws_bytes
    n_sets = int(min(64, max(1, -(-cold_bytes // set_bytes))))
    sets = [dict(X=X0.clone(), image=image0.clone(), sw=sw0.clone(), bias=B0.clone(),
                 Y=torch.empty((M, N), dtype=torch.bfloat16, device="cuda"),
                 ws=torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")) for _ in range(n_sets)]
    torch.cuda.synchronize()
    linear = binding.convrot_linear_w4a16 if w4a16 else binding.convrot_linear

    def step(i):
        s = sets[i % n_sets]
        linear(s["X"], s["image"], s["sw"], s["bias"], N, g, Y=s["Y"], workspace=s["ws"])

    ms_step, batch_ms = graph_times_ms(step, steps, warmup, BATCHES)

    # The dominant kernel alone: the GEMM of the two-kernel path on
    # workspaces the linear has just prepared (they hold the activation copy
    # the plan reads), or the whole linear where it is one kernel.
    single = w4a16 or binding.convrot_linear_kernel_count(M, K, N, g) == 1
    if single:
        kernel_ms = float(np.median(batch_ms))
    else:
        for i in range(n_sets):
            step(i)

        def gemm_only(i):
            s = sets[i % n_sets]
            binding.convrot_gemm(s["ws"], M, K, s["image"], s["sw"], s["bias"], N, g, Y=s["Y"])

        _, gemm_batches = graph_times_ms(gemm_only, steps, 2, BATCHES)
        kernel_ms = float(np.median(gemm_batches))

    plan = binding.convrot_linear_plan(M, K, N, g)
    kind = 0 if w4a16 else plan["mfma"]
    peak = PEAK_FP6_TOPS if kind == binding.CONVROT_MFMA_FP6 else PEAK_INT8_TOPS
    ops = float(wl.ops)
    # algorithmic bytes of the dominant kernel: the whole path's for a single
    # kernel; the GEMM's otherwise (packed weight and activation codes, both
    # scales, bias, Y)
    kernel_bytes = wl.bytes_alg if single else N * K // 2 + M * K // 2 + 4 * M + 4 * N + 2 * N + 2 * M * N
    if ops / wl.bytes_alg >= peak * 1e12 / (PEAK_HBM_GBS * 1e9):
        ach = ops / (kernel_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 2), "peak": peak, "unit": "TOP/s",
                "frac": round(ach / peak, 4)}
    else:
        ach = kernel_bytes / (kernel_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
    # the counters of the GEMM this workload runs (the rotation changes only the
    # prep; the INT4-only image has its own summary)
    roof["traffic"] = None if w4a16 else read_traffic(name)
    med = float(np.median(batch_ms))
    rec = {
        "workload": name, "M": M, "K": K, "N": N, "group": wl.g, "rotation": rotation, "path": path,
        "ms_per_step": round(ms_step, 5),
        "median_ms": round(med, 5), "min_ms": round(float(np.min(batch_ms)), 5), "batches": BATCHES,
        "tops": round(ops / (med * 1e-3) / 1e12, 2),
        "gbs": round(wl.bytes_alg / (med * 1e-3) / 1e9, 1),
        "kernels": 1 if single else 2,
        "dominant_kernel": "linear" if single else "gemm",
        "dominant_kernel_us": round(kernel_ms * 1e3, 2),
        "prep_and_gaps_us": None if single else round((med - kernel_ms) * 1e3, 2),
        "plan": {"mfma": {0: "bf16", 1: "int8", 2: "fp6"}.get(kind, kind), "tile": list(plan["tile"]),
                 "splits": plan["splits"]},
        "weight_bytes_per_weight": round(image0.numel() / (N * K), 3),
        "weight_prep_ms": round(weight_prep_ms, 4),
        "cold_buffer_sets": n_sets,
        "roofline": roof,
        "dtype": "bf16" if w4a16 else ("fp6" if kind == binding.CONVROT_MFMA_FP6 else "int8"),
    }
    del sets, image0, sw0, X0, B0
    torch.cuda.empty_cache()
    return (rec, inp) if want_inputs else rec


def baselines(steps: int):
    """Empty-dispatch floor, a plain device copy, a plain streaming read of
    the decode weight size, the matrix-core rate of an MFMA-only loop (FP6
    and INT8), and at the QKV shape the vendor INT8 GEMM (int8 operands, int32
    out, no rotation, quantization or epilogue) and the dense bf16 linear."""
    import torch
    out = {}
    empty_ms, _ = graph_times_ms(lambda i: torch.cuda._sleep(0), steps, 5, 1)
    out["empty_dispatch_us"] = round(empty_ms * 1e3, 2)
    nbytes = 256 << 20
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    copy_ms, _ = graph_times_ms(lambda i: dst.copy_(src), 10, 2, 1)
    out["copy_256MiB_us"] = round(copy_ms * 1e3, 1)
    out["copy_gbs_read_plus_write"] = round(2 * nbytes / (copy_ms * 1e-3) / 1e9, 1)
    del src, dst
    # a plain streaming read of the decode weight stream's size (12288 x 3072
    # INT4 codes, 18.9 MB): a row-wise integer sum that writes 18 KB
    rd = torch.ones(12288 * 3072 // 8, dtype=torch.int32, device="cuda").view(4608, 1024)
    read_ms = eager_times_ms(lambda: rd.sum(dim=1, dtype=torch.int32), 50, 5)
    out["stream_read_18.9MB_us"] = round(read_ms * 1e3, 2)
    out["stream_read_gbs"] = round(rd.numel() * 4 / (read_ms * 1e-3) / 1e9, 1)
    del rd
    # the MFMA-only loop of the library's probe: the rate the matrix cores
    # sustain here (the practical denominator beside the published peak)
    from w4a4_rotated_bit_amd import binding
    for label, kind in (("fp6", binding.CONVROT_PROBE_FP6), ("int8", binding.CONVROT_PROBE_INT8)):
        count, buf = binding.convrot_matrix_core_probe(kind, 100)
        ms = eager_times_ms(lambda: binding.convrot_matrix_core_probe(kind, 4000, out=buf), 3, 1)
        count, _ = binding.convrot_matrix_core_probe(kind, 4000, out=buf)
        out[f"{label}_mfma_loop_tops"] = round(count * binding.PROBE_OPS_PER_MFMA[kind] / (ms * 1e-3) / 1e12, 1)
    torch.cuda.synchronize()
    M, K, N = 1536, 3072, 9216
    a = torch.randint(-7, 8, (M, K), dtype=torch.int8, device="cuda")
    b = torch.randint(-7, 8, (K, N), dtype=torch.int8, device="cuda")
    try:
        out["vendor_int8_gemm_qkv_us"] = round(eager_times_ms(lambda: torch._int_mm(a, b), 50, 5) * 1e3, 2)
    except Exception as e:  # the vendor kernel is context only
        out["vendor_int8_gemm_qkv_us"] = f"unavailable: {type(e).__name__}"
    x = torch.randn(M, K, device="cuda").to(torch.bfloat16)
    w = torch.randn(N, K, device="cuda").to(torch.bfloat16)
    bias = torch.randn(N, device="cuda").to(torch.bfloat16)
    dense_ms = eager_times_ms(lambda: torch.nn.functional.linear(x, w, bias), 50, 5)
    out["dense_bf16_linear_qkv_us"] = round(dense_ms * 1e3, 2)
    del a, b, x, w, bias
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    # 1000 steps: long enough that the primary replay's start, on a GPU that
    # has just idled, is a small part of it (at 200 steps it was 2-11% slower
    # than the back-to-back batches on the compute-bound shapes)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, help="headline workload (name, optionally +int4)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-config", action="store_true", help="time only the headline workload")
    ap.add_argument("--cold-bytes", type=float, default=512 * 2**20, help="total bytes of rotating buffer sets")
    ap.add_argument("--copy-probe", type=int, default=0, help="only run a device copy of this many bytes")
    ap.add_argument("--summarize-profile", metavar="DB", help="print per-kernel statistics of a rocprofv3 "
                    "results database and exit (no GPU needed)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB"),
                    help="print the HBM traffic summary of --workload's dominant kernel from four rocprofv3 "
                    "counter databases and exit (no GPU needed)")
    ap.add_argument("--no-baselines", action="store_true", help="skip the floor and vendor baselines")
    ap.add_argument("--path", choices=("w4a4", "w4a16"), default="w4a4",
                    help="w4a16: weight-only INT4 with bf16 rotated activations (M <= 32)")
    ap.add_argument("--rotation", choices=("sylvester", "regular"), default="sylvester",
                    help="Hadamard matrix of the rotation (the regular one adds sign flips and a permutation)")
    args = ap.parse_args()

    if args.summarize_profile:
        print(summarize_profile(args.summarize_profile))
        return
    if args.write_traffic:
        print(traffic_summary(args.workload, *args.write_traffic))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from w4a4_rotated_bit_amd import binding

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_probe:
        copy_probe(args.copy_probe, 10)
        return
    binding.load()
    if args.path == "w4a16" and args.workload.startswith(("flux", "stress", "tiny", "g64")):
        log(f"--path w4a16 covers M <= 32 (the weight-bound regime); {args.workload} is larger")
        sys.exit(2)

    head, inp = measure(args.workload, args.steps, args.warmup, args.cold_bytes, args.rotation, args.path,
                        want_inputs=True)
    log(f"headline {args.workload}: {head['ms_per_step'] * 1e3:.2f} us/step")
    per_config = {}
    if not args.no_per_config:
        for name in PER_CONFIG:
            if name == args.workload:
                continue
            per_config[name] = measure(name, min(args.steps, 500), args.warmup, args.cold_bytes)
            log(f"{name}: {per_config[name]['median_ms'] * 1e3:.2f} us/step (median)")
    base = None if args.no_baselines else baselines(min(args.steps, 100))
    cpu = None
    single = None
    if not args.no_cpu_baseline:
        wl = inp["workload"]
        g = wl.g | (binding.CONVROT_REGULAR_HADAMARD if args.rotation == "regular" else 0)
        cpu = cpu_baseline(inp, args.cpu_seconds, g, args.path)
        if not args.no_per_config:
            single = cpu_single_thread(SINGLE_THREAD)

    wl = inp["workload"]
    rec = {
        "metric": METRIC,
        "value": round(wl.ops / (head["ms_per_step"] * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": {"workload": head["workload"], "M": wl.M, "K": wl.K, "N": wl.N, "group": wl.g,
                   "path": args.path, "rotation": args.rotation, "x_kind": wl.x_kind,
                   "outlier_channels": wl.outlier_count, "cold_buffer_sets": head["cold_buffer_sets"],
                   "timed_as": "hip_graph"},
        "median_ms": head["median_ms"],
        "min_ms": head["min_ms"],
        "gbps": round(wl.bytes_alg / (head["ms_per_step"] * 1e-3) / 1e9, 1),
        "hbm_frac": round(wl.bytes_alg / (head["ms_per_step"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "plan": head["plan"],
        "dominant_kernel_us": head["dominant_kernel_us"],
        "prep_and_gaps_us": head["prep_and_gaps_us"],
        "weight_bytes_per_weight": head["weight_bytes_per_weight"],
        "weight_prep_ms": head["weight_prep_ms"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "cpu_single_thread": single,
        "baselines": base,
        "per_config": per_config,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
