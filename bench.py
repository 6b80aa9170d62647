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

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
                       [--profile-kernel M [--eager]] [--profile-mlp M]
                       [--traffic-summary FETCH_DIR WRITE_DIR]

--profile-kernel M launches only the GEMM at M (graph-replayed, or eagerly
with --eager, the form for rocprofv3 --pmc runs) and then a plain 256 MiB copy
whose FETCH_SIZE / WRITE_SIZE readings calibrate those counters.
--traffic-summary reads the counter CSVs of a FETCH_SIZE run and a WRITE_SIZE
run of that command and writes the per-launch HBM traffic to
profiles/traffic_gemv_m1.json (taken into `roofline.traffic` while the kernel
sources are unchanged).
"""
from __future__ import annotations

import argparse
import hashlib
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
KERNEL_SOURCES = ["decode_w4a16_repack_amd/csrc/" + f for f in
                  ("stream.hip", "stream_kernel.h", "panel.hip", "tile.hip", "device.h", "gemm.hip",
                   "common.h")]
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
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class InputSets:
    """R rotating resident input sets of one shape (packed weights + A)."""

    def __init__(self, M, R, seed=0):
        import torch
        import decode_w4a16_repack_amd as w4
        from decode_w4a16_repack_amd import synth
        self.M = M
        G = K // GROUP
        self.sets = []
        p0 = synth.make_problem(M, K, N, GROUP, seed=seed)
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
        g = torch.Generator(device="cuda")
        g.manual_seed(seed + 1)
        for r in range(R):
            if r == 0:
                q, s, z, A = dev(p0.w.qweight), dev(p0.w.scales), dev(p0.w.zeros), dev(p0.A)
            else:
                q = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device="cuda", generator=g)
                s = (torch.rand((N, G), device="cuda", generator=g) * 0.019 + 0.001).half()
                z = torch.randint(0, 256, (N, (G + 1) // 2), dtype=torch.uint8, device="cuda", generator=g)
                A = torch.randn((M, K), device="cuda", generator=g).half()
            pw = w4.repack(q, s, z, K, N, GROUP)
            out = torch.empty((M, N), dtype=torch.float16, device="cuda")
            self.sets.append((A, pw, out))
            del q, s, z
        torch.cuda.synchronize()


def rotations_needed(M):
    per = algorithmic_bytes(M)
    return max(2, math.ceil(2 * INFINITY_CACHE / per))


def time_calls(sets, steps, warmup, ws):
    """Device time per call.  The R rotating calls are captured once in a HIP
    graph (no host launch cost between calls) and replayed; HIP events on the
    launch stream bracket the whole timed region, synchronized on both sides.
    Returns (us per call from events, wall seconds of the timed region,
    number of calls timed)."""
    import torch
    import decode_w4a16_repack_amd as w4
    R = len(sets.sets)
    for i in range(max(warmup, R)):       # eager warmup (also sets kernel attributes)
        A, pw, out = sets.sets[i % R]
        w4.gemm(A, pw, out=out, workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for A, pw, out in sets.sets:
                w4.gemm(A, pw, out=out, workspace=ws)
    reps = max(1, steps // R)
    with torch.cuda.stream(stream):
        for _ in range(max(1, warmup // R)):
            g.replay()
        torch.cuda.synchronize()
        start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record(stream)
        for _ in range(reps):
            g.replay()
        stop.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    n = reps * R
    us = start.elapsed_time(stop) * 1e3 / n
    return us, wall, n


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
    """us per call of call(set) over the rotating sets, graph-replayed, HIP
    events on the replay stream (as time_calls)."""
    import torch
    for i in range(max(warmup, len(sets))):
        call(sets[i % len(sets)])
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(gr, stream=stream):
            for st in sets:
                call(st)
    reps = max(1, steps // len(sets))
    with torch.cuda.stream(stream):
        gr.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            gr.replay()
        b.record(stream)
        torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * len(sets))


def extras(ws):
    """The pages' other workloads: the group sweep at M=16 K=N=4096 with the
    fused bias+ReLU epilogue and the fused RMSNorm prologue against their
    unfused chains (analytic bytes beside measured time, "Fusion benchmark"
    page), and the fused gate_up SwiGLU at M=32 K=5120 N=13824."""
    import torch
    import decode_w4a16_repack_amd as w4
    res = {"group_sweep_m16_k4096_n4096": [], "gate_up_m32_k5120_n13824_g128": None}
    M, K_, N_ = 16, 4096, 4096
    for g in (16, 32, 64, 128):
        byt = algorithmic_bytes(M, K_, N_, g)
        R = max(2, math.ceil(2 * INFINITY_CACHE / byt))
        pr = DevProblem(M, K_, N_, g, R, seed=200 + g)
        sets = pr.sets
        t_plain = time_graph(lambda st: w4.gemm(st["A"], st["w"][0], out=st["out"], workspace=ws), sets)
        t_bias_fused = time_graph(lambda st: w4.gemm(st["A"], st["w"][0], epilogue="bias_relu",
                                                     bias=st["bias"], out=st["out"], workspace=ws), sets)

        def unfused_bias(st):
            w4.gemm(st["A"], st["w"][0], out=pr.tmp, workspace=ws)
            w4.add_bias(pr.tmp, st["bias"], out=pr.tmp2)
            w4.relu(pr.tmp2, out=st["out"])
        t_bias_unfused = time_graph(unfused_bias, sets)
        t_rms_fused = time_graph(lambda st: w4.gemm(st["A"], st["w"][0], gamma=st["gamma"], eps=1e-6,
                                                    out=st["out"], workspace=ws), sets)

        def unfused_rms(st):
            w4.rmsnorm(st["A"], st["gamma"], 1e-6, out=pr.an)
            w4.gemm(pr.an, st["w"][0], out=st["out"], workspace=ws)
        t_rms_unfused = time_graph(unfused_rms, sets)
        row = {
            "group": g, "rotating_sets": R, "level": "HBM (rotated inputs), graph replay",
            "gemm_us": t_plain, "gemm_GBps": byt / t_plain / 1e3,
            "gemm_pct_hbm_peak": 100 * byt / t_plain / 1e3 / HBM_PEAK_GBS,
            "bias_relu_fused_us": t_bias_fused, "bias_relu_unfused_us": t_bias_unfused,
            # output side, fp16: fused writes 2MN; the unfused chain writes the
            # GEMM output, reads+writes it in the bias pass and again in ReLU
            "bias_relu_analytic_output_bytes": {"fused": 2 * M * N_, "unfused": 10 * M * N_,
                                                "saved": 8 * M * N_},
            "rmsnorm_fused_us": t_rms_fused, "rmsnorm_unfused_us": t_rms_unfused,
            # activation side, fp16: fused reads A once; unfused reads A,
            # writes the normalized A and the GEMM reads it back
            "rmsnorm_analytic_a_side_bytes": {"fused": 2 * M * K_, "unfused": 6 * M * K_,
                                              "saved": 4 * M * K_},
        }
        res["group_sweep_m16_k4096_n4096"].append(row)
        log(f"[bench] C4 g={g:3d}: gemm {t_plain:6.2f} us ({row['gemm_pct_hbm_peak']:4.1f}% HBM)  "
            f"bias+relu fused {t_bias_fused:6.2f} / unfused {t_bias_unfused:6.2f} us  "
            f"rmsnorm fused {t_rms_fused:6.2f} / unfused {t_rms_unfused:6.2f} us")
        del pr, sets
        torch.cuda.empty_cache()
    # gate_up SwiGLU
    M, g = 32, 128
    byt = algorithmic_bytes(M, K, N, g, n_weights=2)
    R = max(2, math.ceil(2 * INFINITY_CACHE / byt))
    pr = DevProblem(M, K, N, g, R, n_weights=2, seed=300)
    t_gu = time_graph(lambda st: w4.gemm_gate_up(st["A"], st["w"][0], st["w"][1], out=st["out"],
                                                 workspace=ws), pr.sets)
    t_two = time_graph(lambda st: (w4.gemm(st["A"], st["w"][0], out=pr.tmp, workspace=ws),
                                   w4.gemm(st["A"], st["w"][1], out=pr.tmp2, workspace=ws)), pr.sets)
    res["gate_up_m32_k5120_n13824_g128"] = {
        "rotating_sets": R, "level": "HBM (rotated inputs), graph replay",
        "us": t_gu, "GBps": byt / t_gu / 1e3, "pct_hbm_peak": 100 * byt / t_gu / 1e3 / HBM_PEAK_GBS,
        "TFLOPs": flops(M, n_weights=2) / t_gu / 1e6, "algorithmic_bytes": byt,
        "two_plain_gemms_us": t_two,
    }
    log(f"[bench] C5 gate_up M=32: {t_gu:.2f} us ({res['gate_up_m32_k5120_n13824_g128']['pct_hbm_peak']:.1f}% HBM); "
        f"two plain GEMMs {t_two:.2f} us")
    del pr
    torch.cuda.empty_cache()
    res["split_sweep_m8"] = split_sweep(ws)
    res["mlp_chain"] = mlp_chain(ws)
    return res


# The M=8 decode shapes the "Small-M split-K retune" update tunes: (name, K,
# N per projection, gate_up).  The gate_up rows are paired projections of
# N each (4096 x 2*13696 and 5120 x 2*13824 in the update's table).
SPLIT_SWEEP_SHAPES = [("o_q_proj", 4096, 4096, False), ("down_proj", 13696, 4096, False),
                      ("gate_up_glm", 4096, 13696, True), ("gate_up_qwen", 5120, 13824, True)]


def split_sweep(ws, M=8, group=128):
    """Each shape at M=8: the automatic plan's time and %HBM, beside every
    forced split-K factor in {1, 2, 3, 4, 6, 8} the shape can run."""
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
        t_auto = time_graph(lambda st: call(st, 0), pr.sets)
        forced = {}
        for sk in (1, 2, 3, 4, 6, 8):
            try:
                fp = w4.plan(M, K_, N_, group, gate_up=gu, split=sk)
            except w4.W4A16Error:
                continue
            if fp.split in forced:
                continue
            forced[fp.split] = time_graph(lambda st: call(st, sk), pr.sets)
        best = min(forced, key=forced.get) if forced else auto.split
        row = {"shape": name, "M": M, "K": K_, "N": N_, "gate_up": gu, "group": group,
               "rotating_sets": R, "algorithmic_bytes": byt,
               "auto_kernel": auto.kernel, "auto_split": auto.split, "auto_us": t_auto,
               "auto_pct_hbm_peak": 100 * byt / t_auto / 1e3 / HBM_PEAK_GBS,
               "forced_split_us": {str(k): v for k, v in sorted(forced.items())},
               "best_forced_split": best}
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
            t_mlp = time_graph(lambda st: w4.mlp(st["A"], *st["w"], gamma=st["gamma"],
                                                 inter=st["inter"], out=st["out"], workspace=ws),
                               sets)
            t_gu = time_graph(lambda st: w4.gemm_gate_up(st["A"], st["w"][0], st["w"][1],
                                                         gamma=st["gamma"], out=st["inter"],
                                                         workspace=ws), sets)
            t_dn = time_graph(lambda st: w4.gemm(st["inter"], st["w"][2], out=st["out"],
                                                 workspace=ws), sets)
            row = {"shape": name, "M": M, "H": H, "I": I, "group": group, "rotating_sets": R,
                   "algorithmic_bytes": byt, "mlp_us": t_mlp,
                   "mlp_GBps": byt / t_mlp / 1e3,
                   "mlp_pct_hbm_peak": 100 * byt / t_mlp / 1e3 / HBM_PEAK_GBS,
                   "gate_up_alone_us": t_gu, "down_alone_us": t_dn,
                   "gate_up_plan": w4.plan(M, H, I, group, gate_up=True).__dict__,
                   "down_plan": w4.plan(M, I, H, group).__dict__}
            rows.append(row)
            log(f"[bench] {name} M={M:2d}: mlp {t_mlp:6.2f} us ({row['mlp_pct_hbm_peak']:4.1f}% HBM); "
                f"gate_up alone {t_gu:6.2f} + down alone {t_dn:6.2f} us")
        del sets
        torch.cuda.empty_cache()
    return rows


def self_check(sets, ws):
    """Cheap checks of the timed launch configuration that need no oracle:
    every output finite, and a repeated call bit-identical (fixed-order
    split-K reduction).  Element parity of this configuration against the
    oracle is the GPU test suite's job."""
    import torch
    import decode_w4a16_repack_amd as w4
    A, pw, out = sets.sets[0]
    y1 = w4.gemm(A, pw, workspace=ws).clone()
    y2 = w4.gemm(A, pw, workspace=ws)
    torch.cuda.synchronize()
    return {"finite": bool(torch.isfinite(y1).all()), "repeat_bit_identical": bool(torch.equal(y1, y2))}


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


def cpu_baseline(budget_s=12.0):
    """The oracle as it stands, on the host's cores, over whole M=1 calls of
    the headline shape (dequantization inside the timed region)."""
    import oracle
    from decode_w4a16_repack_amd import synth
    oracle.build(force=False)
    p = synth.make_problem(1, K, N, GROUP, seed=0)
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        oracle.gemm(p.A, p.w.qweight, p.w.scales, p.w.zeros, GROUP, N)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 400:
            break
    t = float(np.median(times))
    cores = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    return {"value": algorithmic_bytes(1) / t / 1e9, "unit": "GB/s", "cores": cores,
            "kind": "oracle", "us_per_call": t * 1e6,
            "sample": f"{len(times)} whole M=1 calls (K=5120 N=13824 g=128, all 13824 columns), "
                      f"f64, median; {sum(times):.1f} s of CPU work"}


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
    ap.add_argument("--profile-mlp", type=int, default=0,
                    help="only run the MLP block (H=4096, I=13696, RMSNorm) at this M "
                         "(for rocprofv3)")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
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
        sets = InputSets(M, rotations_needed(M))
        if args.eager:
            R = len(sets.sets)
            for i in range(args.warmup + args.steps):
                A, pw, out = sets.sets[i % R]
                w4.gemm(A, pw, out=out, workspace=ws)
            torch.cuda.synchronize()
            log(f"profile M={M}: {args.warmup + args.steps} eager calls")
        else:
            us, _, n = time_calls(sets, args.steps, args.warmup, ws)
            log(f"profile M={M}: {us:.2f} us per call over {n} graph-replayed calls")
        del sets
        torch.cuda.empty_cache()
        src = torch.empty(COPY_PROBE_BYTES, dtype=torch.uint8, device="cuda").fill_(3)
        dst = torch.empty_like(src)
        for _ in range(4):
            w4.probe_copy(src, dst)
        torch.cuda.synchronize()
        log(f"profile: 4 copies of {COPY_PROBE_BYTES} bytes")
        return

    # headline: M = 1
    M = 1
    R = rotations_needed(M)
    log(f"[bench] headline M=1 K={K} N={N} g={GROUP}: {R} rotating input sets")
    sets = InputSets(M, R)
    us_mean, wall, n_timed = time_calls(sets, args.steps, args.warmup, ws)
    parity = self_check(sets, ws)
    log(f"[bench] self-check {parity}")
    b1 = algorithmic_bytes(M)
    ms_per_step = wall / n_timed * 1e3
    value = b1 / (ms_per_step * 1e-3) / 1e9
    achieved = b1 / (us_mean * 1e-6) / 1e9
    log(f"[bench] M=1: {us_mean:.2f} us per call (events), {ms_per_step * 1e3:.2f} us per step (wall)")
    del sets
    torch.cuda.empty_cache()

    sweep = []
    if not args.no_sweep:
        for Ms in (1, 2, 4, 8, 16, 32, 64, 128):
            s2 = InputSets(Ms, rotations_needed(Ms), seed=Ms)
            t, _, _ = time_calls(s2, 160, 16, ws)
            byt, fl = algorithmic_bytes(Ms), flops(Ms)
            row = {"M": Ms, "us": t, "GBps": byt / t / 1e3, "TFLOPs": fl / t / 1e6,
                   "pct_hbm_peak": 100 * byt / t / 1e3 / HBM_PEAK_GBS,
                   "pct_mfma_peak": 100 * fl / t / 1e6 / MFMA_F16_PEAK_TFLOPS,
                   "level": "HBM (rotated inputs), graph replay"}
            sweep.append(row)
            log(f"[bench] M={Ms:4d} {t:8.2f} us  {row['GBps']:8.1f} GB/s ({row['pct_hbm_peak']:5.1f}% HBM)"
                f"  {row['TFLOPs']:7.2f} TFLOP/s ({row['pct_mfma_peak']:5.2f}% MFMA)")
            del s2
            torch.cuda.empty_cache()

    extra = None if args.no_extras else extras(ws)
    probe = hbm_probe()
    log(f"[bench] streaming-read probe: {probe:.1f} GB/s")
    cpu = None if args.no_cpu else cpu_baseline()
    if cpu:
        log(f"[bench] cpu oracle: {cpu['value']:.3f} GB/s on {cpu['cores']} threads")

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
        "tflops": flops(1) / us_mean / 1e6,
        "pct_hbm_peak": 100 * value / HBM_PEAK_GBS,
        "hbm_probe_GBps": probe,
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
