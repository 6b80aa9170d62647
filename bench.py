"""Benchmark of the W4A16 hot path on one MI355X.

Headline (one JSON line on stdout): the decode GEMV, M=1 K=5120 N=13824
group 128 with asymmetric 4-bit zero-points and fp16 scales.  One step is one
fused call (w4a16_gemm) over one resident input set; input sets rotate so the
36.8 MB of packed weights per call come from HBM, not from the 256 MiB
Infinity Cache.  `value` is algorithmic bytes per call / time per call.

Also reported (stderr table and the JSON `m_sweep` / `extras` fields): the
same shape for M = 2..128, with µs, TFLOP/s (2MNK / t, croqtile tutorial
"TFLOPS"), GB/s and the fraction of the HBM and fp16-MFMA peaks; the group
sweep at M=16 K=N=4096 with the fused bias+ReLU epilogue and RMSNorm prologue
against their unfused chains (analytic bytes beside measured time); the fused
gate_up SwiGLU at M=32; the MLP block (gate_up, fp16 intermediate, down
projection) at the decode MLP shapes; a streaming-read probe of the achievable HBM rate; and
the CPU oracle timed on the host's cores.

Timing: exactly --steps calls are timed (HIP events and the wall clock);
200 further graph replays give the spread (median, p10, p90, min); a
cache-warm figure (one input set re-read) is reported apart, labelled; the
fused and unfused chains are sampled in alternation; the CPU oracle runs on
all host cores and on one, and its result checks the timed GPU output.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--profile-kernel M [--eager] [--gate-up]] [--profile-mlp M]
                       [--profile-fusion] [--probes]
                       [--traffic-summary FETCH_DIR WRITE_DIR]
                       [--fusion-summary FETCH_DIR WRITE_DIR]
                       [--counter-summary DIR [--kernel-filter S]]

--profile-kernel M launches only the GEMM at M (graph-replayed, or eagerly
with --eager, the form for rocprofv3 --pmc runs) and then a plain 256 MiB copy
whose FETCH_SIZE / WRITE_SIZE readings calibrate those counters.
--traffic-summary reads the counter CSVs of a FETCH_SIZE run and a WRITE_SIZE
run of that command and writes the per-launch HBM traffic to
profiles/traffic_gemv_m1.json (taken into `roofline.traffic` while the kernel
sources are unchanged).  --profile-fusion and --fusion-summary do the same for
the fused and unfused chains of the group sweep
(profiles/fusion_bytes_m16_k4096_n4096.json).  --counter-summary prints the
mean per dispatch of every counter in a rocprofv3 --pmc output directory.
--probes runs only the streaming-read HBM probe and the two compute-unit
probes (LDS read rate, L2 -> LDS copy rate) and prints them as JSON.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("W4A16 GEMM µs + TFLOP/s + HBM GB/s (% peak), K=5120 N=13824 g=128, M=1..128")
K, N, GROUP = 5120, 13824, 128
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published
INFINITY_CACHE = 256 << 20
PAGE_M1_US = 69.5  # the pages' M=1 time for this shape (H200, context only)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_m1.json")
FUSION_FILE = os.path.join(ROOT, "profiles", "fusion_bytes_m16_k4096_n4096.json")
CSRC = os.path.join(ROOT, "decode_w4a16_repack_amd", "csrc")
# every kernel source: counter figures are reported only while none has changed
KERNEL_SOURCES = sorted("decode_w4a16_repack_amd/csrc/" + f for f in os.listdir(CSRC)
                        if f.endswith((".hip", ".h")))
COPY_PROBE_BYTES = 256 << 20  # plain copy of known size, counter calibration


def algorithmic_bytes(M, K=K, N=N, group=GROUP, scale_bytes=2, has_zp=True, n_weights=1):
    """Bytes the method must move once: packed int4 weights, scales,
    zero-points, A read once, out written once."""
    G = K // group
    w = K * N // 2 + N * G * scale_bytes + (N * ((G + 1) // 2) if has_zp else 0)
    return n_weights * w + 2 * M * K + 2 * M * N


def flops(M, K=K, N=N, n_weights=1):
    return 2 * M * N * K * n_weights


def kernel_source_hash():
    """Hash of the kernel sources' code: comments and blank space removed,
    so that an edit of a comment does not retire the counter figures."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)   # block comments
        text = re.sub(r"//[^\n]*", " ", text)                  # line comments
        h.update(rel.encode() + b"\0" + " ".join(text.split()).encode())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class InputSets:
    """R rotating resident input sets of one shape (packed weights + A).
    Set 0 is the seeded host problem (synth.make_problem, the oracle's input
    in the CPU-baseline leg); the others are drawn on the device with the same
    distributions.  ``sdt``: fp16 or fp32 scales; ``asym``: 4-bit zero-points
    (else symmetric, zero-point 8)."""

    def __init__(self, M, R, seed=0, sdt=np.float16, asym=True):
        import torch
        import decode_w4a16_repack_amd as w4
        from decode_w4a16_repack_amd import synth
        self.M = M
        G = K // GROUP
        self.sets = []
        self.problem0 = synth.make_problem(M, K, N, GROUP, seed=seed, scale_dtype=sdt, asym=asym)
        p0 = self.problem0
        dev = lambda a: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()
        g = torch.Generator(device="cuda")
        g.manual_seed(seed + 1)
        tdt = torch.float16 if sdt == np.float16 else torch.float32
        for r in range(R):
            if r == 0:
                q, s, z, A = dev(p0.w.qweight), dev(p0.w.scales), dev(p0.w.zeros), dev(p0.A)
            else:
                q = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda", generator=g)
                s = (torch.rand((N, G), device="cuda", generator=g) * 0.019 + 0.001).to(tdt)
                z = (torch.randint(0, 256, (N, (G + 1) // 2), dtype=torch.uint8, device="cuda",
                                   generator=g) if asym else None)
                A = torch.randn((M, K), device="cuda", generator=g).half()
            pw = w4.repack(q, s, z, K, N, GROUP)
            out = torch.empty((M, N), dtype=torch.float16, device="cuda")
            self.sets.append((A, pw, out))
            del q, s, z
        torch.cuda.synchronize()

    def calls(self, ws):
        import decode_w4a16_repack_amd as w4
        return [(lambda A=A, pw=pw, out=out: w4.gemm(A, pw, out=out, workspace=ws))
                for A, pw, out in self.sets]


def rotations_needed(M):
    per = algorithmic_bytes(M)
    return max(2, math.ceil(2 * INFINITY_CACHE / per))


def stats(xs):
    """median, p10, p90, min, max and count of a list of samples."""
    a = np.asarray(xs, dtype=np.float64)
    return {"median": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "min": float(a.min()), "max": float(a.max()),
            "n": int(a.size)}


def capture(calls, stream):
    """One HIP graph of the given calls, captured on ``stream``."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for c in calls:
                c()
    return g


def time_calls(calls, steps, warmup, samples=200):
    """Device and wall time of exactly ``steps`` calls.

    ``calls`` are R zero-argument callables, one per rotating input set.
    The timed calls, ``calls[i % R]`` for i < steps, are captured in one HIP
    graph (no host launch cost between calls; one launch for the whole timed
    region up to 2048 calls, else replays of an R-call graph and one of the
    remainder).  Untimed first: R eager calls (they also set the kernel
    attributes), replays of the R-call graph until at least ``warmup``
    calls, and one replay of each timed graph (a graph's first replay also
    uploads it).  The timed region is bracketed by HIP events on the replay
    stream and by the wall clock, with a synchronize on both sides.  Then
    ``samples`` replays of the R-call graph, each bracketed by its own event
    pair, give the spread (a sample is the mean call time over one replay: a
    single call is shorter than an event pair's own cost).
    """
    import torch
    R = len(calls)
    for c in calls:
        c()
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g_full = capture(calls, stream)
    if steps <= 2048:
        timed = [(capture([calls[i % R] for i in range(steps)], stream), 1)]
    else:
        rem = steps % R
        timed = [(g_full, steps // R)]
        if rem:
            timed.append((capture(calls[:rem], stream), 1))
    with torch.cuda.stream(stream):
        for _ in range(max(0, math.ceil((warmup - R) / R))):
            g_full.replay()
        for g, _ in timed:
            g.replay()
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        for g, reps in timed:
            for _ in range(reps):
                g.replay()
        stop.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per = []
        if samples:
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(samples)]
            for a, b in evs:
                a.record(stream)
                g_full.replay()
                b.record(stream)
            torch.cuda.synchronize()
            per = [a.elapsed_time(b) * 1e3 / R for a, b in evs]
    us = start.elapsed_time(stop) * 1e3 / steps
    return {"us_per_call": us, "wall_s": wall, "calls": steps, "calls_per_replay": R,
            "samples_us": stats(per) if per else None}


class DevProblem:
    """R rotating device input sets of one W4A16 shape: packed weights (one or
    two streams), A, bias and gamma, all drawn on the device with the
    recipe's distributions (codes U{0..15}, scales U[0.001, 0.02], zero-points
    U{0..15}, A ~ N(0,1), bias ~ N(0, 0.1), gamma ~ N(1, 0.1))."""

    def __init__(self, M, K, N, group, R, n_weights=1, seed=100):
        import torch
        import decode_w4a16_repack_amd as w4
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        G = K // group
        self.M, self.K, self.N, self.group = M, K, N, group
        self.sets = []
        for _ in range(R):
            ws_ = []
            for _ in range(n_weights):
                q = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda", generator=g)
                sc = (torch.rand((N, G), device="cuda", generator=g) * 0.019 + 0.001).half()
                z = torch.randint(0, 256, (N, (G + 1) // 2), dtype=torch.uint8, device="cuda", generator=g)
                ws_.append(w4.repack(q, sc, z, K, N, group))
                del q, sc, z
            A = torch.randn((M, K), device="cuda", generator=g).half()
            bias = (torch.randn((N,), device="cuda", generator=g) * 0.1).half()
            gamma = (1.0 + 0.1 * torch.randn((K,), device="cuda", generator=g)).half()
            out = torch.empty((M, N), dtype=torch.float16, device="cuda")
            self.sets.append({"A": A, "w": ws_, "bias": bias, "gamma": gamma, "out": out})
        # scratch of the unfused chains (shared: rewritten by every call)
        self.tmp = torch.empty((M, N), dtype=torch.float16, device="cuda")
        self.tmp2 = torch.empty((M, N), dtype=torch.float16, device="cuda")
        self.an = torch.empty((M, K), dtype=torch.float16, device="cuda")
        torch.cuda.synchronize()


def time_graph(call, sets, steps=200, warmup=10):
    """us per call of call(set) over the rotating sets (time_calls, no
    samples)."""
    calls = [(lambda st=st: call(st)) for st in sets]
    return time_calls(calls, steps, warmup, samples=0)["us_per_call"]


AB_TIMING = ("medians of 24 interleaved replays of a graph of at least 192 calls per path "
             "over the rotating sets")


def ab_samples(paths, sets, rounds=24, warmup=2, min_calls=192):
    """Interleaved A/B samples ("Fusion benchmark" page, "Two paths on one
    rig"): each path is one HIP graph of at least ``min_calls`` calls
    cycling over the rotating sets (so one graph launch and one event pair
    are a small part of a sample); a round replays every path once in turn,
    each replay bracketed by its own event pair.  Returns {name: stats of
    us per call}."""
    import torch
    stream = torch.cuda.Stream()
    R = len(sets)
    n_calls = R * math.ceil(min_calls / R)
    graphs = {}
    for name, call in paths.items():
        calls = [(lambda st=st: call(st)) for st in sets]
        for c in calls:
            c()
        torch.cuda.synchronize()
        graphs[name] = capture([calls[i % R] for i in range(n_calls)], stream)
    per = {name: [] for name in paths}
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            for g in graphs.values():
                g.replay()
        torch.cuda.synchronize()
        evs = []
        for _ in range(rounds):
            for name, g in graphs.items():
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                g.replay()
                b.record(stream)
                evs.append((name, a, b))
        torch.cuda.synchronize()
    for name, a, b in evs:
        per[name].append(a.elapsed_time(b) * 1e3 / n_calls)
    return {name: stats(v) for name, v in per.items()}


# The "Fusion benchmark" comparison at config 4: M=16 K=N=4096, the fused
# bias+ReLU epilogue and RMSNorm prologue against their unfused chains.
FUSION_M, FUSION_K, FUSION_N = 16, 4096, 4096
FUSION_GROUPS = (16, 32, 64, 128)
# (path, kernels per call) in the order the counter pass runs them
FUSION_PATHS = (("bias_relu_fused", 1), ("bias_relu_unfused", 3), ("rmsnorm_fused", 1),
                ("rmsnorm_unfused", 2))


def fusion_paths(pr, ws):
    """The four paths of the fusion comparison on a DevProblem's sets: the
    fused kernels, and the chains of separate passes (GEMM -> bias pass ->
    ReLU pass; RMSNorm pass -> GEMM) through scratch tensors."""
    import decode_w4a16_repack_amd as w4

    def unfused_bias(st):
        w4.gemm(st["A"], st["w"][0], out=pr.tmp, workspace=ws)
        w4.add_bias(pr.tmp, st["bias"], out=pr.tmp2)
        w4.relu(pr.tmp2, out=st["out"])

    def unfused_rms(st):
        w4.rmsnorm(st["A"], st["gamma"], 1e-6, out=pr.an)
        w4.gemm(pr.an, st["w"][0], out=st["out"], workspace=ws)
    return {
        "bias_relu_fused": lambda st: w4.gemm(st["A"], st["w"][0], epilogue="bias_relu",
                                              bias=st["bias"], out=st["out"], workspace=ws),
        "bias_relu_unfused": unfused_bias,
        "rmsnorm_fused": lambda st: w4.gemm(st["A"], st["w"][0], gamma=st["gamma"], eps=1e-6,
                                            out=st["out"], workspace=ws),
        "rmsnorm_unfused": unfused_rms,
    }


def profile_fusion(iters=8):
    """Eager calls of the four fusion paths for every group (all inputs
    created first), then plain copies of COPY_PROBE_BYTES that calibrate
    the counters: the command of the FETCH_SIZE / WRITE_SIZE passes whose
    CSVs summarize_fusion() reads."""
    import torch
    import decode_w4a16_repack_amd as w4
    ws = w4.Workspace()
    probs = {g: DevProblem(FUSION_M, FUSION_K, FUSION_N, g, 2, seed=200 + g) for g in FUSION_GROUPS}
    torch.cuda.synchronize()
    for g in FUSION_GROUPS:
        paths = fusion_paths(probs[g], ws)
        for name, _ in FUSION_PATHS:
            for i in range(iters):
                paths[name](probs[g].sets[i % 2])
    torch.cuda.synchronize()
    copy_probe()
    log(f"profile fusion: {iters} eager calls per path and group, then 4 copies")


def copy_probe():
    """Four plain copies of COPY_PROBE_BYTES (the counter calibration)."""
    import torch
    import decode_w4a16_repack_amd as w4
    src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty_like(src)
    for _ in range(4):
        w4.probe_copy(src, dst)
    torch.cuda.synchronize()


def _dispatches(d, counter):
    """[(dispatch id, kernel name, value)] of one counter from the rocprofv3
    CSVs under d, in dispatch order (instances of a dispatch summed)."""
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                key = int(row.get("Dispatch_Id") or row.get("Correlation_Id"))
                name, v = row["Kernel_Name"], float(row["Counter_Value"])
                per[key] = (name, per.get(key, (name, 0.0))[1] + v)
    return [(k, n, v) for k, (n, v) in sorted(per.items())]


def summarize_fusion(fetch_dir, write_dir):
    """Measured HBM bytes per call of each fusion path and group, from the
    FETCH_SIZE and WRITE_SIZE passes of profile_fusion(): the library's
    dispatches other than the repacks, in order, are the paths' kernels
    (FUSION_PATHS counts) and then the copies; each counter is scaled by what
    it reads for a copy of known size."""
    res = {"kernel_source_hash": kernel_source_hash(), "copy_probe_bytes": COPY_PROBE_BYTES,
           "groups": {}}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        # (the library's kernels: demangled "w4a16::..." names, or mangled
        # "_ZN5w4a16..." ones where rocprofv3 leaves them so)
        ds = [(n, v) for _, n, v in _dispatches(d, counter)
              if "w4a16" in n and "repack" not in n]
        copies = [v for n, v in ds if "probe_copy_kernel" in n]
        ds = [(n, v) for n, v in ds if "probe_copy_kernel" not in n]
        if not copies:
            raise SystemExit(f"{counter}: no calibration copy in {d}")
        factor = COPY_PROBE_BYTES / (float(np.median(copies)) * 1024.0)
        iters = len(ds) // (len(FUSION_GROUPS) * sum(k for _, k in FUSION_PATHS))
        if iters * len(FUSION_GROUPS) * sum(k for _, k in FUSION_PATHS) != len(ds) or iters == 0:
            raise SystemExit(f"{counter}: {len(ds)} dispatches do not match the fusion sequence")
        pos = 0
        for g in FUSION_GROUPS:
            row = res["groups"].setdefault(str(g), {})
            for name, k in FUSION_PATHS:
                calls = [sum(v for _, v in ds[pos + i * k:pos + (i + 1) * k]) for i in range(iters)]
                pos += iters * k
                row[name] = row.get(name, 0.0) + float(np.median(calls)) * 1024.0 * factor
        res[counter + "_scale_factor"] = factor
    return res


def load_fusion():
    """The committed fusion byte counts, if taken on the current kernel sources."""
    try:
        with open(FUSION_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t if t.get("kernel_source_hash") == kernel_source_hash() else None


def extras(ws):
    """The pages' other workloads: the group sweep at M=16 K=N=4096 with the
    fused bias+ReLU epilogue and the fused RMSNorm prologue against their
    unfused chains (analytic bytes beside measured time, "Fusion benchmark"
    page), the fused gate_up SwiGLU at M=32 K=5120 N=13824, the split-K
    sweep at M=8, the MLP block, and the cost of the RMSNorm prologues."""
    import torch
    import decode_w4a16_repack_amd as w4
    res = {"group_sweep_m16_k4096_n4096": [], "gate_up_m32_k5120_n13824_g128": None}
    M, K_, N_ = FUSION_M, FUSION_K, FUSION_N
    measured = load_fusion()
    for g in FUSION_GROUPS:
        byt = algorithmic_bytes(M, K_, N_, g)
        R = max(2, math.ceil(2 * INFINITY_CACHE / byt))
        pr = DevProblem(M, K_, N_, g, R, seed=200 + g)
        sets = pr.sets
        # the plain GEMM and the fused and unfused chains sampled in
        # alternation on the same buffers
        ab = ab_samples({"gemm": lambda st: w4.gemm(st["A"], st["w"][0], out=st["out"], workspace=ws),
                         **fusion_paths(pr, ws)}, sets)
        med = {k: v["median"] for k, v in ab.items()}
        t_plain = med["gemm"]
        row = {
            "group": g, "rotating_sets": R, "level": "HBM (rotated inputs), graph replay",
            "gemm_us": t_plain, "gemm_GBps": byt / t_plain / 1e3,
            "gemm_pct_hbm_peak": 100 * byt / t_plain / 1e3 / HBM_PEAK_GBS,
            "ab_samples_us": ab,
            "bias_relu_fused_us": med["bias_relu_fused"],
            "bias_relu_unfused_us": med["bias_relu_unfused"],
            # output side, fp16: fused writes 2MN; the unfused chain writes the
            # GEMM output, reads+writes it in the bias pass and again in ReLU
            "bias_relu_analytic_output_bytes": {"fused": 2 * M * N_, "unfused": 10 * M * N_,
                                                "saved": 8 * M * N_},
            "rmsnorm_fused_us": med["rmsnorm_fused"], "rmsnorm_unfused_us": med["rmsnorm_unfused"],
            # activation side, fp16: fused reads A once; unfused reads A,
            # writes the normalized A and the GEMM reads it back
            "rmsnorm_analytic_a_side_bytes": {"fused": 2 * M * K_, "unfused": 6 * M * K_,
                                              "saved": 4 * M * K_},
        }
        if measured is not None and str(g) in measured["groups"]:
            mg = measured["groups"][str(g)]
            row["measured_bytes_per_call"] = {
                "level": "counter (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated; "
                         "cache-warm eager calls)", **mg,
                "bias_relu_saved": mg["bias_relu_unfused"] - mg["bias_relu_fused"],
                "rmsnorm_saved": mg["rmsnorm_unfused"] - mg["rmsnorm_fused"]}
        res["group_sweep_m16_k4096_n4096"].append(row)
        log(f"[bench] C4 g={g:3d}: gemm {t_plain:6.2f} us ({row['gemm_pct_hbm_peak']:4.1f}% HBM)  "
            f"bias+relu fused {med['bias_relu_fused']:6.2f} / unfused {med['bias_relu_unfused']:6.2f} us  "
            f"rmsnorm fused {med['rmsnorm_fused']:6.2f} / unfused {med['rmsnorm_unfused']:6.2f} us "
            f"(medians of {ab['bias_relu_fused']['n']} interleaved samples)")
        del pr, sets
        torch.cuda.empty_cache()
    # gate_up SwiGLU
    M, g = 32, 128
    byt = algorithmic_bytes(M, K, N, g, n_weights=2)
    R = max(2, math.ceil(2 * INFINITY_CACHE / byt))
    pr = DevProblem(M, K, N, g, R, n_weights=2, seed=300)
    ab = ab_samples({
        "gate_up": lambda st: w4.gemm_gate_up(st["A"], st["w"][0], st["w"][1], out=st["out"],
                                              workspace=ws),
        "two_gemms": lambda st: (w4.gemm(st["A"], st["w"][0], out=pr.tmp, workspace=ws),
                                 w4.gemm(st["A"], st["w"][1], out=pr.tmp2, workspace=ws))}, pr.sets)
    t_gu, t_two = ab["gate_up"]["median"], ab["two_gemms"]["median"]
    res["gate_up_m32_k5120_n13824_g128"] = {
        "rotating_sets": R, "level": "HBM (rotated inputs), graph replay",
        "us": t_gu, "GBps": byt / t_gu / 1e3, "pct_hbm_peak": 100 * byt / t_gu / 1e3 / HBM_PEAK_GBS,
        "TFLOPs": flops(M, n_weights=2) / t_gu / 1e6, "algorithmic_bytes": byt,
        "two_plain_gemms_us": t_two,
        "timing": AB_TIMING,
    }
    log(f"[bench] C5 gate_up M=32: {t_gu:.2f} us ({res['gate_up_m32_k5120_n13824_g128']['pct_hbm_peak']:.1f}% HBM); "
        f"two plain GEMMs {t_two:.2f} us")
    del pr
    torch.cuda.empty_cache()
    res["split_sweep_m8"] = split_sweep(ws)
    res["mlp_chain"] = mlp_chain(ws)
    res["rmsnorm_prologue_k5120_n13824"] = rmsnorm_prologue_cost(ws)
    return res


def rmsnorm_prologue_cost(ws, Ms=(1, 8, 16, 32, 64, 128), group=128):
    """The RMSNorm prologue's cost at K=5120 N=13824: the plain product, the
    product with the RMSNorm prologue and with the residual + RMSNorm
    prologue, for the GEMM and for gate_up, at each M (medians of
    interleaved replays, ``ab_samples``)."""
    import torch
    import decode_w4a16_repack_amd as w4
    rows = []
    for M in Ms:
        byt = algorithmic_bytes(M, K, N, group, n_weights=2)
        R = max(2, math.ceil(2 * INFINITY_CACHE / byt))
        pr = DevProblem(M, K, N, group, R, n_weights=2, seed=600 + M)
        g = torch.Generator(device="cuda")
        g.manual_seed(700 + M)
        for st in pr.sets:
            st["resid"] = torch.randn((M, K), device="cuda", generator=g).half()
            st["sum"] = torch.empty((M, K), dtype=torch.float16, device="cuda")
        paths = {
            "gemm_plain": lambda st: w4.gemm(st["A"], st["w"][0], out=st["out"], workspace=ws),
            "gemm_rms": lambda st: w4.gemm(st["A"], st["w"][0], gamma=st["gamma"], out=st["out"],
                                           workspace=ws),
            "gemm_skip_rms": lambda st: w4.gemm(st["A"], st["w"][0], gamma=st["gamma"],
                                                residual=st["resid"], residual_out=st["sum"],
                                                out=st["out"], workspace=ws),
            "gate_up_plain": lambda st: w4.gemm_gate_up(st["A"], st["w"][0], st["w"][1],
                                                        out=st["out"], workspace=ws),
            "gate_up_rms": lambda st: w4.gemm_gate_up(st["A"], st["w"][0], st["w"][1],
                                                      gamma=st["gamma"], out=st["out"], workspace=ws),
            "gate_up_skip_rms": lambda st: w4.gemm_gate_up(st["A"], st["w"][0], st["w"][1],
                                                           gamma=st["gamma"], residual=st["resid"],
                                                           residual_out=st["sum"], out=st["out"],
                                                           workspace=ws),
        }
        res = ab_samples(paths, pr.sets)
        row = {"M": M, "K": K, "N": N, "group": group, "rotating_sets": R, "timing": AB_TIMING,
               "us": {k: v["median"] for k, v in res.items()},
               "gemm_plan": w4.plan(M, K, N, group).kernel,
               "gate_up_plan": w4.plan(M, K, N, group, gate_up=True).kernel}
        rows.append(row)
        u = row["us"]
        log(f"[bench] RMSNorm prologue M={M:3d}: gemm {u['gemm_plain']:6.2f} / {u['gemm_rms']:6.2f} / "
            f"{u['gemm_skip_rms']:6.2f} us, gate_up {u['gate_up_plain']:6.2f} / {u['gate_up_rms']:6.2f} / "
            f"{u['gate_up_skip_rms']:6.2f} us (plain / RMSNorm / residual + RMSNorm)")
        del pr
        torch.cuda.empty_cache()
    return rows

# The M=8 decode shapes the "Small-M split-K retune" update tunes: (name, K,
# N per projection, gate_up).  The gate_up rows are paired projections of
# N each (4096 x 2*13696 and 5120 x 2*13824 in the update's table).
SPLIT_SWEEP_SHAPES = [("o_q_proj", 4096, 4096, False), ("down_proj", 13696, 4096, False),
                      ("gate_up_glm", 4096, 13696, True), ("gate_up_qwen", 5120, 13824, True)]


def split_sweep(ws, M=8, group=128):
    """Each shape at M=8: the automatic plan's time and %HBM, beside every
    forced split-K factor in {1, 2, 3, 4, 6, 8} the shape can run (medians of
    interleaved replays, ``ab_samples``)."""
    import torch
    import decode_w4a16_repack_amd as w4
    rows = []
    for name, K_, N_, gu in SPLIT_SWEEP_SHAPES:
        nw = 2 if gu else 1
        byt = algorithmic_bytes(M, K_, N_, group, n_weights=nw)
        R = max(2, math.ceil(2 * INFINITY_CACHE / byt))
        pr = DevProblem(M, K_, N_, group, R, n_weights=nw, seed=400)

        def call(st, split):
            if gu:
                w4.gemm_gate_up(st["A"], st["w"][0], st["w"][1], out=st["out"], workspace=ws,
                                split=split)
            else:
                w4.gemm(st["A"], st["w"][0], out=st["out"], workspace=ws, split=split)
        auto = w4.plan(M, K_, N_, group, gate_up=gu)
        paths = {"auto": lambda st: call(st, 0)}
        for sk in (1, 2, 3, 4, 6, 8):
            try:
                fp = w4.plan(M, K_, N_, group, gate_up=gu, split=sk)
            except w4.W4A16Error:
                continue
            if f"sk{fp.split}" not in paths:
                paths[f"sk{fp.split}"] = (lambda st, sk=sk: call(st, sk))
        # Interleaved: a path timed first after the inputs were made would
        # also pay for the clocks ramping back up.
        res = ab_samples(paths, pr.sets)
        t_auto = res["auto"]["median"]
        forced = {int(k[2:]): v["median"] for k, v in res.items() if k != "auto"}
        best = min(forced, key=forced.get) if forced else auto.split
        row = {"shape": name, "M": M, "K": K_, "N": N_, "gate_up": gu, "group": group,
               "rotating_sets": R, "algorithmic_bytes": byt,
               "auto_kernel": auto.kernel, "auto_split": auto.split, "auto_us": t_auto,
               "auto_pct_hbm_peak": 100 * byt / t_auto / 1e3 / HBM_PEAK_GBS,
               "forced_split_us": {str(k): v for k, v in sorted(forced.items())},
               "best_forced_split": best,
               "timing": AB_TIMING}
        rows.append(row)
        log(f"[bench] split sweep {name:12s} M={M} K={K_} N={N_}{' x2' if gu else ''}: auto sk{auto.split} "
            f"{t_auto:6.2f} us ({row['auto_pct_hbm_peak']:4.1f}% HBM); forced "
            + " ".join(f"sk{k}={v:.2f}" for k, v in sorted(forced.items())))
        del pr
        torch.cuda.empty_cache()
    return rows


# The decode MLP blocks of the "Small-M split-K retune" update's shapes:
# (name, hidden H, intermediate I).  gate_up is H x 2*I, down is I x H.
MLP_SHAPES = [("mlp_4096x13696", 4096, 13696), ("mlp_5120x13824", 5120, 13824)]


def mlp_weight_bytes(H, I, group):
    return 2 * algorithmic_bytes(0, H, I, group) + algorithmic_bytes(0, I, H, group)


def mlp_sets(gen, H, I, group):
    """Rotating resident sets of the three packed MLP weights (gate, up:
    K = H, N = I; down: K = I, N = H) and gamma, enough that a replay cycle
    streams twice the Infinity Cache from HBM."""
    import torch
    import decode_w4a16_repack_amd as w4

    def packed(K_, N_):
        G = K_ // group
        q = torch.randint(0, 256, (N_, K_ // 2), dtype=torch.uint8, device="cuda", generator=gen)
        sc = (torch.rand((N_, G), device="cuda", generator=gen) * 0.019 + 0.001).half()
        z = torch.randint(0, 256, (N_, (G + 1) // 2), dtype=torch.uint8, device="cuda", generator=gen)
        return w4.repack(q, sc, z, K_, N_, group)
    R = max(2, math.ceil(2 * INFINITY_CACHE / mlp_weight_bytes(H, I, group)))
    return [{"w": [packed(H, I), packed(H, I), packed(I, H)], "H": H, "I": I,
             "gamma": (1.0 + 0.1 * torch.randn((H,), device="cuda", generator=gen)).half()}
            for _ in range(R)]


def mlp_inputs(gen, sets, M):
    """Activations, intermediate and output buffers of M rows in every set."""
    import torch
    for st in sets:
        st["A"] = torch.randn((M, st["H"]), device="cuda", generator=gen).half()
        st["inter"] = torch.empty((M, st["I"]), dtype=torch.float16, device="cuda")
        st["out"] = torch.empty((M, st["H"]), dtype=torch.float16, device="cuda")


def mlp_chain(ws, Ms=(1, 8, 32), group=128):
    """w4a16_mlp (gate_up with the RMSNorm prologue, fp16 intermediate, down
    projection) at the decode MLP shapes, beside its two projections timed
    alone.  Bytes: the three packed weights, A, the intermediate written and
    read back, and the output."""
    import torch
    import decode_w4a16_repack_amd as w4
    rows = []
    gen = torch.Generator(device="cuda")
    gen.manual_seed(500)
    for name, H, I in MLP_SHAPES:
        wbytes = mlp_weight_bytes(H, I, group)
        sets = mlp_sets(gen, H, I, group)
        R = len(sets)
        for M in Ms:
            mlp_inputs(gen, sets, M)
            byt = wbytes + 2 * M * H + 2 * 2 * M * I + 2 * M * H
            res = ab_samples({
                "mlp": lambda st: w4.mlp(st["A"], *st["w"], gamma=st["gamma"], inter=st["inter"],
                                         out=st["out"], workspace=ws),
                "gate_up": lambda st: w4.gemm_gate_up(st["A"], st["w"][0], st["w"][1],
                                                      gamma=st["gamma"], out=st["inter"],
                                                      workspace=ws),
                "down": lambda st: w4.gemm(st["inter"], st["w"][2], out=st["out"], workspace=ws),
            }, sets)
            t_mlp, t_gu, t_dn = (res[k]["median"] for k in ("mlp", "gate_up", "down"))
            row = {"shape": name, "M": M, "H": H, "I": I, "group": group, "rotating_sets": R,
                   "algorithmic_bytes": byt, "mlp_us": t_mlp,
                   "mlp_GBps": byt / t_mlp / 1e3,
                   "mlp_pct_hbm_peak": 100 * byt / t_mlp / 1e3 / HBM_PEAK_GBS,
                   "gate_up_alone_us": t_gu, "down_alone_us": t_dn,
                   "gate_up_plan": w4.plan(M, H, I, group, gate_up=True).__dict__,
                   "down_plan": w4.plan(M, I, H, group).__dict__,
                   "timing": AB_TIMING}
            rows.append(row)
            log(f"[bench] {name} M={M:2d}: mlp {t_mlp:6.2f} us ({row['mlp_pct_hbm_peak']:4.1f}% HBM); "
                f"gate_up alone {t_gu:6.2f} + down alone {t_dn:6.2f} us")
        del sets
        torch.cuda.empty_cache()
    return rows


def self_check(sets, ws):
    """Checks of the timed launch configuration that need no oracle: every
    output finite, and a repeated call bit-identical (fixed-order split-K
    reduction).  Returns them with set 0's output, which the CPU-baseline
    leg compares with the oracle."""
    import torch
    import decode_w4a16_repack_amd as w4
    A, pw, out = sets.sets[0]
    y1 = w4.gemm(A, pw, workspace=ws).clone()
    y2 = w4.gemm(A, pw, workspace=ws)
    torch.cuda.synchronize()
    return ({"finite": bool(torch.isfinite(y1).all()), "repeat_bit_identical": bool(torch.equal(y1, y2))},
            y1.cpu().numpy())


def hbm_probe(nbytes=1 << 30, reps=20):
    import torch
    import decode_w4a16_repack_amd as w4
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    for _ in range(3):
        w4.probe_read(buf, sink)
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        w4.probe_read(buf, sink)
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) * 1e-3)
    del buf
    return nbytes / float(np.median(times)) / 1e9


def cu_probes():
    """One compute unit's data paths, the limits of the MFMA-tile kernel: the
    LDS read rate (1024 workgroups of 512 threads, 2000 x 16 KiB read per
    wavefront) and the global-to-LDS copy rate of a 64 x 5120 fp16 matrix
    held in L2 (216 workgroups, the tile kernel's grid at M=128, 160 steps
    of 32 KiB each), both per compute unit (256 CUs for the first: 1024
    workgroups spread over all of them; 216 for the second, one workgroup
    each).  And the issue probe: how far independent VALU work overlaps the
    matrix cores (``w4a16_probe_mfma_valu``).  Medians of 5 timed launches
    with HIP events."""
    import torch
    import decode_w4a16_repack_amd as w4
    sink = torch.zeros(1024 * 512, dtype=torch.int32, device="cuda")
    rows = torch.randn(64, 5120, device="cuda").half()

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return float(np.median(ts))

    t_read = timed(lambda: w4.probe_lds_read(1024, 2000, sink))
    read_bytes = 1024 * 512 * 2000 * 256
    t_copy = timed(lambda: w4.probe_lds_copy(rows, 216, 160, sink))
    copy_bytes = 216 * 161 * 32 * 1024
    # issue probe: ns per round of 8 MFMAs + X fp32 FMAs per wavefront, one
    # workgroup per compute unit, 1 or 2 wavefronts per SIMD
    fsink = torch.zeros(256 * 512, dtype=torch.float32, device="cuda")
    iters = 20000
    issue = {}
    for waves in (1, 2):
        issue[f"{waves}_wave_per_simd"] = {
            str(x): timed(lambda x=x: w4.probe_mfma_valu(x, waves, 256, iters, fsink)) / iters * 1e9
            for x in (0, 8, 16, 32, 48, 64)}
    return {"lds_read_GBps_per_cu": read_bytes / t_read / 1e9 / 256,
            "lds_read_seconds": t_read,
            "l2_to_lds_copy_GBps_per_cu": copy_bytes / t_copy / 1e9 / 216,
            "l2_to_lds_copy_seconds": t_copy,
            "mfma_valu_ns_per_round": issue,
            "what": "LDS read: 1024 workgroups x 512 threads, 2000 x 16 KiB per wavefront; "
                    "L2 -> LDS copy: 216 workgroups, 161 x 32 KiB each of a 640 KiB fp16 "
                    "matrix, two steps in flight, one barrier per step; issue: 256 workgroups "
                    "of 256 or 512 threads, 20000 rounds of 8 independent-accumulator "
                    "v_mfma_f32_16x16x32_f16 and X (key) independent fp32 FMAs per wavefront, "
                    "ns per round"}


def tile_read_probe(steps=480, warmup=2000):
    """Plain reads of the headline shape's packed weight tiles (K=5120,
    N=13824: 864 column tiles x 40 k tiles of 1 KiB, 35.4 MB) under two
    decompositions: the streaming kernel's (216 workgroups of 4 column tiles,
    8 k slices each) and the same tiles split evenly over all 256 compute
    units (256 workgroups of 135 tiles).  Rotating resident copies (twice
    the Infinity Cache), graph replay, HIP events, like the headline."""
    import torch
    import decode_w4a16_repack_amd as w4
    nbytes = K * N // 2
    R = max(2, math.ceil(2 * INFINITY_CACHE / nbytes))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(11)
    ws_ = [w4.PackedWeight(torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda",
                                         generator=gen), K, N, GROUP, 0, False) for _ in range(R)]
    sink = torch.zeros(256 * 512, dtype=torch.int32, device="cuda")
    res = {"bytes_per_call": nbytes, "rotating_sets": R, "level": "HBM (rotated inputs), graph replay"}
    for name, mode, wgs in (("stream_kernel_grid_216", 0, 0), ("even_256", 1, 256)):
        calls = [(lambda w=w, mode=mode, wgs=wgs: w4.probe_read_tiles(w, mode, wgs, sink)) for w in ws_]
        us = time_calls(calls, steps, warmup, samples=0)["us_per_call"]
        res[name] = {"us_per_call": us, "GBps": nbytes / us / 1e3}
    del ws_
    torch.cuda.empty_cache()
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


# The oracle is timed in child processes (no torch loaded), where
# OMP_NUM_THREADS takes effect before the oracle's OpenMP runtime starts;
# each reports the threads its OpenMP runtime actually used.
_ORACLE_TIMING = r"""
import os, sys, time, json
sys.path.insert(0, {root!r})
if {one_core}:
    os.sched_setaffinity(0, {{min(os.sched_getaffinity(0))}})
import oracle
from decode_w4a16_repack_amd import synth
oracle.build(force=False)
oracle.set_threads({threads})
p = synth.make_problem(1, {K}, {N}, {G}, seed=0)
ts = []
t_start = time.perf_counter()
while True:
    t0 = time.perf_counter()
    oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, {G}, {N})
    ts.append(time.perf_counter() - t0)
    if len(ts) >= {min_reps} and (time.perf_counter() - t_start > {budget} or len(ts) >= 400):
        break
print(json.dumps({{"times": ts, "threads": oracle.max_threads(),
                  "cores": len(os.sched_getaffinity(0))}}))
"""


def _time_oracle(threads, budget_s, min_reps):
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS=str(threads))
    code = _ORACLE_TIMING.format(root=ROOT, K=K, N=N, G=GROUP, budget=budget_s, min_reps=min_reps,
                                 threads=int(threads), one_core=threads == 1)
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=900, check=True)
    out = json.loads(r.stdout.strip().splitlines()[-1])
    ts = out["times"]
    t = float(np.median(ts))
    return {"value": algorithmic_bytes(1) / t / 1e9, "unit": "GB/s",
            "cores": min(out["threads"], out["cores"]), "threads": out["threads"],
            "us_per_call": t * 1e6, "calls": len(ts), "cpu_seconds": float(sum(ts))}


def cpu_baseline(gpu_out=None, budget_s=12.0):
    """The oracle as it stands (never tuned), over whole M=1 calls of the
    headline shape with the dequantization inside the timed region, median
    wall time: on all the host cores the process may use (OpenMP over output
    columns) and on one core, each in a child process.  One more oracle call
    here is the reference for the GPU output of the timed configuration (set
    0, the same seeded input): every output within the parity tolerance."""
    import oracle
    from decode_w4a16_repack_amd import synth
    oracle.build(force=False)
    allc = _time_oracle(int(os.environ.get("OMP_NUM_THREADS") or host_cores()), budget_s, 3)
    one = None
    try:
        one = _time_oracle(1, 0.0, 3)
        one["sample"] = f"median of {one['calls']} whole M=1 calls on one core"
    except Exception as e:  # the one-core figure is context; its failure is reported
        log(f"[bench] one-core oracle run failed: {e}")
    check = None
    if gpu_out is not None:
        p = synth.make_problem(1, K, N, GROUP, seed=0)
        ref = oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, GROUP, N)
        got = np.asarray(gpu_out, np.float64)
        err = float(np.abs(got - ref).max())
        tol = 2e-2 * float(np.abs(ref).max())
        check = {"what": "GPU output of the timed configuration (input set 0) against the "
                         "oracle, every one of the 13824 outputs",
                 "max_abs_err": err, "tol": tol, "pass": bool(err <= tol)}
    return {"value": allc["value"], "unit": "GB/s", "cores": allc["cores"], "kind": "oracle",
            "us_per_call": allc["us_per_call"],
            "sample": f"{allc['calls']} whole M=1 calls (K=5120 N=13824 g=128, all 13824 "
                      f"columns), f64, median; {allc['cpu_seconds']:.1f} s of CPU work",
            "cpu_model": cpu_model(), "host_cores": host_cores(),
            "one_core": one, "parity_check": check,
            "note": "a plain f64 oracle, not a tuned CPU kernel"}


def load_traffic():
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch")


def _counter_rows(d, counter):
    """{kernel name: [per-dispatch value]} from the rocprofv3 counter CSVs
    under directory d (values of one dispatch summed over their instances)."""
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                key = (row["Kernel_Name"], row.get("Dispatch_Id") or row.get("Correlation_Id"))
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    out = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def summarize_traffic(fetch_dir, write_dir):
    """HBM bytes per GEMM launch: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch, median over dispatches), each scaled by what the counter reads
    for the plain copy of COPY_PROBE_BYTES in the same run."""
    res = {"kernel_source_hash": kernel_source_hash(), "copy_probe_bytes": COPY_PROBE_BYTES}
    total = 0.0
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _counter_rows(d, counter)
        gemm = [n for n in rows if "stream_kernel" in n]
        copy = [n for n in rows if "probe_copy_kernel" in n]
        if len(gemm) != 1 or len(copy) != 1:
            raise SystemExit(f"{counter}: expected one GEMM and one copy kernel, got {sorted(rows)}")
        g, c = float(np.median(rows[gemm[0]])), float(np.median(rows[copy[0]]))
        factor = COPY_PROBE_BYTES / (c * 1024.0)
        byts = g * 1024.0 * factor
        total += byts
        res[counter] = {"gemm_kib_per_dispatch": g, "copy_kib_per_dispatch": c,
                        "scale_factor": factor, "bytes_per_launch": byts,
                        "dispatches": len(rows[gemm[0]]), "kernel": gemm[0]}
    res["bytes_per_launch"] = total
    res["algorithmic_bytes_per_launch"] = algorithmic_bytes(1)
    return res


def traffic_summary(fetch_dir, write_dir):
    """Write summarize_traffic(...) to the committed traffic file."""
    res = summarize_traffic(fetch_dir, write_dir)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))


def counter_summary(d, kernel_filter=""):
    """Per kernel: dispatches and the mean per dispatch (instances summed) of
    every counter in the rocprofv3 CSVs under d (the table of a profiles/
    summary)."""
    import csv
    import glob
    per = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                name = row["Kernel_Name"]
                if kernel_filter not in name:
                    continue
                key = (name, row["Counter_Name"])
                disp = row.get("Dispatch_Id") or row.get("Correlation_Id")
                per.setdefault(key, {})
                per[key][disp] = per[key].get(disp, 0.0) + float(row["Counter_Value"])
    out = {}
    for (name, counter), byd in sorted(per.items()):
        v = list(byd.values())
        out.setdefault(name, {})[counter] = {"dispatches": len(v), "mean": float(np.mean(v)),
                                             "median": float(np.median(v))}
    print(json.dumps(out, indent=1))
    return out


# The M sweep of the headline shape: (M, scale dtype, asymmetric), the
# symmetric and fp32-scale variants and the odd edge-tile sizes included.
SWEEP = ([(m, np.float16, True) for m in (1, 2, 4, 7, 8, 16, 32, 33, 64, 128)] +
         [(m, sdt, asym) for m in (1, 16, 128) for sdt, asym in ((np.float16, False),
                                                                 (np.float32, True))])


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=480)
    # (2000 untimed steps, about 20 ms of GPU work: enough for the clocks of a
    # freshly taken GPU to settle before the timed steps)
    ap.add_argument("--warmup", type=int, default=2000)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--profile-kernel", type=int, default=0,
                    help="only launch the GEMM at this M (for rocprofv3)")
    ap.add_argument("--eager", action="store_true",
                    help="with --profile-kernel: eager launches, no graph")
    ap.add_argument("--gate-up", action="store_true",
                    help="with --profile-kernel: the paired gate/up projection instead")
    ap.add_argument("--profile-mlp", type=int, default=0,
                    help="only run the MLP block (H=4096, I=13696, RMSNorm) at this M "
                         "(for rocprofv3)")
    ap.add_argument("--profile-fusion", action="store_true",
                    help="only run the fusion comparison's paths eagerly (for rocprofv3 --pmc)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--fusion-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--probes", action="store_true",
                    help="only the HBM and compute-unit probes (JSON on stdout)")
    ap.add_argument("--counter-summary", metavar="DIR")
    ap.add_argument("--kernel-filter", default="")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.fusion_summary:
        res = summarize_fusion(*args.fusion_summary)
        with open(FUSION_FILE, "w") as f:
            json.dump(res, f, indent=1)
        print(json.dumps(res, indent=1))
        return
    if args.counter_summary:
        counter_summary(args.counter_summary, args.kernel_filter)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_w4a16_repack_amd as w4
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    ws = w4.Workspace()

    if args.profile_fusion:
        profile_fusion()
        return
    if args.probes:
        print(json.dumps({"hbm_probe_GBps": hbm_probe(), "cu_probes": cu_probes(),
                          "tile_read_probe": tile_read_probe()}, indent=1))
        return
    if args.profile_mlp:
        M = args.profile_mlp
        gen = torch.Generator(device="cuda")
        gen.manual_seed(500)
        sets = mlp_sets(gen, 4096, 13696, GROUP)
        mlp_inputs(gen, sets, M)
        us = time_graph(lambda st: w4.mlp(st["A"], *st["w"], gamma=st["gamma"],
                                          inter=st["inter"], out=st["out"], workspace=ws),
                        sets, steps=args.steps, warmup=args.warmup)
        log(f"profile mlp M={M}: {us:.2f} us per block, graph-replayed")
        return
    if args.profile_kernel:
        M = args.profile_kernel
        if args.gate_up:
            byt = algorithmic_bytes(M, n_weights=2)
            pr = DevProblem(M, K, N, GROUP, max(2, math.ceil(2 * INFINITY_CACHE / byt)),
                            n_weights=2, seed=300)
            calls = [(lambda st=st: w4.gemm_gate_up(st["A"], st["w"][0], st["w"][1], out=st["out"],
                                                    workspace=ws)) for st in pr.sets]
        else:
            sets = InputSets(M, rotations_needed(M))
            calls = sets.calls(ws)
        if args.eager:
            for i in range(args.warmup + args.steps):
                calls[i % len(calls)]()
            torch.cuda.synchronize()
            log(f"profile M={M}: {args.warmup + args.steps} eager calls")
        else:
            r = time_calls(calls, args.steps, args.warmup, samples=0)
            log(f"profile M={M}: {r['us_per_call']:.2f} us per call over {r['calls']} "
                "graph-replayed calls")
        del calls
        torch.cuda.empty_cache()
        copy_probe()
        log(f"profile: 4 copies of {COPY_PROBE_BYTES} bytes")
        return

    # headline: M = 1, exactly args.steps timed calls
    M = 1
    R = rotations_needed(M)
    log(f"[bench] headline M=1 K={K} N={N} g={GROUP}: {R} rotating input sets")
    sets = InputSets(M, R)
    head = time_calls(sets.calls(ws), args.steps, args.warmup, samples=200)
    us_mean, wall, n_timed = head["us_per_call"], head["wall_s"], head["calls"]
    parity, gpu_out = self_check(sets, ws)
    log(f"[bench] self-check {parity}")
    b1 = algorithmic_bytes(M)
    ms_per_step = wall / n_timed * 1e3
    value = b1 / (ms_per_step * 1e-3) / 1e9
    achieved = b1 / (us_mean * 1e-6) / 1e9
    sm = head["samples_us"]
    log(f"[bench] M=1: {us_mean:.2f} us per call (events, {n_timed} calls), "
        f"{ms_per_step * 1e3:.2f} us per step (wall); samples median {sm['median']:.2f} "
        f"p10 {sm['p10']:.2f} p90 {sm['p90']:.2f} min {sm['min']:.2f} us")
    # the same calls on one input set: its 36.8 MB stay in the Infinity Cache
    warm = time_calls(sets.calls(ws)[:1] * R, 400, 100, samples=200)
    cache_warm = {"level": "cache-warm: one input set re-read by every call (its 36.8 MB stay in "
                           "the 256 MiB Infinity Cache); not an HBM figure",
                  "us_per_call": warm["us_per_call"], "samples_us": warm["samples_us"],
                  "apparent_GBps": b1 / warm["us_per_call"] / 1e3}
    log(f"[bench] M=1 cache-warm: {warm['us_per_call']:.2f} us per call")
    del sets
    torch.cuda.empty_cache()

    sweep = []
    if not args.no_sweep:
        for Ms, sdt, asym in SWEEP:
            s2 = InputSets(Ms, rotations_needed(Ms), seed=Ms, sdt=sdt, asym=asym)
            # the headline's call count and warmup: a short warmup leaves
            # the first rows paying for clocks that ramp back up
            r = time_calls(s2.calls(ws), args.steps, args.warmup, samples=40)
            t = r["us_per_call"]
            byt = algorithmic_bytes(Ms, scale_bytes=np.dtype(sdt).itemsize, has_zp=asym)
            fl = flops(Ms)
            pl = w4.plan(Ms, K, N, GROUP, 1 if sdt == np.float32 else 0)
            row = {"M": Ms, "scales": np.dtype(sdt).name, "zero_points": "asym" if asym else "sym",
                   "us": t, "samples_us": r["samples_us"], "GBps": byt / t / 1e3,
                   "TFLOPs": fl / t / 1e6, "algorithmic_bytes": byt,
                   "pct_hbm_peak": 100 * byt / t / 1e3 / HBM_PEAK_GBS,
                   "pct_mfma_peak": 100 * fl / t / 1e6 / MFMA_F16_PEAK_TFLOPS,
                   "kernel": pl.kernel, "level": "HBM (rotated inputs), graph replay"}
            sweep.append(row)
            log(f"[bench] M={Ms:4d} {row['scales']} {row['zero_points']:4s} {t:8.2f} us  "
                f"{row['GBps']:8.1f} GB/s ({row['pct_hbm_peak']:5.1f}% HBM)"
                f"  {row['TFLOPs']:7.2f} TFLOP/s ({row['pct_mfma_peak']:5.2f}% MFMA)")
            del s2
            torch.cuda.empty_cache()

    extra = None if args.no_extras else extras(ws)
    probe = hbm_probe()
    log(f"[bench] streaming-read probe: {probe:.1f} GB/s")
    cu = cu_probes()
    trp = tile_read_probe()
    log(f"[bench] tile-read probe (35.4 MB of weight tiles, no arithmetic): streaming kernel's grid "
        f"{trp['stream_kernel_grid_216']['us_per_call']:.2f} us, even over 256 workgroups "
        f"{trp['even_256']['us_per_call']:.2f} us")
    log(f"[bench] compute-unit probes: LDS read {cu['lds_read_GBps_per_cu']:.0f} GB/s per CU, "
        f"L2 -> LDS copy {cu['l2_to_lds_copy_GBps_per_cu']:.0f} GB/s per CU")
    for k, v in cu["mfma_valu_ns_per_round"].items():
        log(f"[bench] issue probe, {k.replace('_', ' ')}: ns per round of 8 MFMAs + X FMAs: "
            + " ".join(f"X={x}:{t:.1f}" for x, t in v.items()))
    cpu = None if args.no_cpu else cpu_baseline(gpu_out)
    if cpu:
        log(f"[bench] cpu oracle: {cpu['value']:.3f} GB/s on {cpu['cores']} threads"
            + (f", {cpu['one_core']['value']:.3f} GB/s on one" if cpu["one_core"] else "")
            + f"; parity of the timed output: {cpu['parity_check']}")

    line = {
        "metric": METRIC,
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": n_timed,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode GEMV M=1 K=5120 N=13824 group=128, asymmetric 4-bit zp, "
                               f"fp16 scales, fp16 A ~ N(0,1), {R} rotating resident input sets",
                   "M": 1, "K": K, "N": N, "group": GROUP},
        "us_per_call": us_mean,
        "samples_us": {**sm, "sample": f"one graph replay of the {R} rotating calls "
                                       "(mean call time), HIP events; level HBM"},
        "cache_warm": cache_warm,
        "tflops": flops(1) / us_mean / 1e6,
        "pct_hbm_peak": 100 * value / HBM_PEAK_GBS,
        "hbm_probe_GBps": probe,
        "cu_probes": cu,
        "tile_read_probe": trp,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic(),
                     "algorithmic_bytes_per_launch": b1, "avg_launch_us": us_mean},
        "cpu_baseline": cpu,
        "self_check": parity,
        "m_sweep": sweep,
        "extras": extra,
        "page_context": {"M1_us_H200": PAGE_M1_US, "note": "other hardware, context only"},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
