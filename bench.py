#!/usr/bin/env python3
"""Benchmark of the MI355X Q4_K matmul path; prints ONE JSON line.

Headline (`value`): Q4_K GEMV HBM throughput of the batch-1 MLP block of
Qwen3.6-27B — gate 17408x5120, up 17408x5120, down 5120x17408, each its own
launch (the SwiGLU between them belongs to the caller and is computed once,
outside the timed region).  One step = those three GEMVs on synthetic random
Q4_K weights (d, dmin ~U(1e-4, 1e-3) in binary16, uniform scale/min bytes and
nibbles) and an N(0,1) f32 activation.  Weights are COLD: each matrix is held
in 12 distinct copies, so both the step rotation (36 x 50 MB = 1.8 GB) and the
per-matrix bursts (12 x 50 MB = 601 MB) cycle through more than the 256 MB
Infinity Cache, and every launch streams its bytes from HBM.  (With 4 copies
a per-matrix burst cycles through 200 MB, which the Infinity Cache partly
holds: it read about 6% faster.)

Also measured and reported in the same line:
  * decode_stack: the full 64-layer per-token matmul chain (48 GDN-shaped +
    16 attention-shaped layers, 64 MLP blocks, lm_head 248320x5120; 14.41 GB
    of Q4_K) replayed as one hipGraph per token: us/token vs the weight-read
    roofline 14,412,349,440 B / 8 TB/s;
  * prefill_gemm: bf16-MFMA GEMM for both MLP shapes at P = 256, 512, 1024
    (TFLOP/s vs the 2.5 PFLOP/s dense bf16 peak), and prefill_gemm_short
    for short prompts, P = 16, 22, 27, 64;
  * gemv_batch: N = 1, 2, 4, 8, 16 vectors on the 17408x5120 weight;
  * gemv_small: the 512x1024 and 1024x512 GEMVs (latency-bound): per call
    from an idle queue, and per call inside a replayed hipGraph next to a
    one-kernel fill (the launch floor);
  * mlp_block: the same MLP block through q4k_mlp (RMSNorm gain, gate|up
    fused with the SwiGLU on device, down with the residual add);
  * gemv_q8_0_lm_head: the lm_head matmul in Q8_0 (248320x5120, 1.35 GB);
  * gemv_q6_k_mlp: Q6_K GEMVs on the two MLP shapes (73 MB each, cold);
  * roofline: the dominant kernel (the MLP GEMV) — algorithmic bytes per
    launch over its HIP-event duration, against 8 TB/s;
  * cpu_baseline: the CPU oracle (double precision, all threads) on the
    same three GEMVs; cpu_baseline_detail: the oracle at one thread and at
    all threads on every workload (C1 small GEMV, C2 MLP GEMVs, C3 decode
    stack from a sampled layer pair, C4 batched N = 1..16, C5 GEMM from a
    row sample), with the host CPU model.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
QK, BB = 256, 144
METRIC = "Q4_K GEMV HBM GB/s (% peak); decode-stack µs/token; prefill GEMM TFLOP/s"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "gemv_mlp_17408x5120_traffic.json")
SHORT_P = (16, 22, 27, 64)
SETTLE_MS = 50  # untimed steady-state run before every timed region  # short-prompt prefill lengths timed next to the prefill configs
GEMV_SOURCES = ["bit_block_quantized_gguf_amd/csrc/q4k_gemv.hip",
                "bit_block_quantized_gguf_amd/csrc/q4k_device.hpp"]


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def wbytes(M, K):
    return M * (K // QK) * BB


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_leg(x, step_bytes):
    """The CPU oracle (oracle/, double precision) timed on this host: one
    thread and all threads the harness allows (OMP_NUM_THREADS, else every
    core), on bounded samples of each workload, scaled to each workload's
    unit.  A reported baseline only: the oracle is never tuned for speed.
    Bounded so that the whole leg takes about half a minute."""
    import numpy as np  # noqa: F401  (arrays from synth)
    import oracle
    import synth
    from synth import workloads as wl
    n_all = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or (os.cpu_count() or 1)
    modes = (("1_thread", 1), ("all_threads", n_all))

    def med3(fn, min_s):
        """median over 3 runs of (seconds per call), each run >= min_s"""
        res = []
        for _ in range(3):
            n, t0 = 0, time.perf_counter()
            while True:
                fn()
                n += 1
                if time.perf_counter() - t0 >= min_s:
                    break
            res.append((time.perf_counter() - t0) / n)
        return float(sorted(res)[1])

    def once(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    det = {"cpu_model": cpu_model(), "cores_visible": os.cpu_count(), "threads_all": n_all}
    # C2: the three MLP GEMVs (the headline workload), whole matrices
    ws = [synth.q4k_weight(synth.key(2, i), M, K) for i, (_, M, K) in enumerate(wl.MLP)]
    a_h = synth.activations(2, 1, wl.INTER, first=1)[0]

    def mlp_step():
        for wh, (_, M, K) in zip(ws, wl.MLP):
            oracle.gemv(wh, x if K == wl.HIDDEN else a_h, M, K)

    c2 = {}
    for name, n in modes:
        oracle.set_threads(n)
        t = med3(mlp_step, 1.0 if n > 1 else 0.5)
        c2[name] = {"GBps": step_bytes / t / 1e9, "ms_per_step": t * 1e3,
                    "threads": oracle.get_threads()}
    det["C2_mlp_gemvs"] = c2
    # C1: the 512x1024 GEMV, whole
    w1 = synth.q4k_weight(synth.key(1, 0), 512, 1024)
    x1 = synth.activations(1, 1, 1024)[0]
    c1 = {}
    for name, n in modes:
        oracle.set_threads(n)
        t = med3(lambda: oracle.gemv(w1, x1, 512, 1024), 0.2)
        c1[name] = {"us": t * 1e6, "GBps": wbytes(512, 1024) / t / 1e9}
    det["C1_gemv_512x1024"] = c1
    # C4: batched GEMV on 17408x5120, N = 1..16, whole matrix
    M4, K4 = wl.BATCH_SHAPE
    w4 = ws[0]
    c4 = {}
    for name, n in modes:
        oracle.set_threads(n)
        per = {}
        for N in (wl.BATCH_N if n > 1 else (1, 16)):
            X = synth.activations(4, N, K4)
            t = med3(lambda: oracle.gemv_batch(w4, X, M4, K4), 0.3) if n > 1 else \
                once(lambda: oracle.gemv_batch(w4, X, M4, K4))
            per[str(N)] = {"us": t * 1e6, "us_per_vector": t * 1e6 / N}
        c4[name] = per
    det["C4_batch_17408x5120"] = c4
    # C5: prefill GEMM 17408x5120 at P = 256 on a sample of 256 rows, as TFLOP/s
    rows = list(range(0, M4, M4 // 256))[:256]
    X5 = synth.activations(5, 256, K4)
    c5 = {}
    for name, n in modes:
        oracle.set_threads(n)
        t = once(lambda: oracle.gemm(w4, X5, M4, K4, rows=rows))
        c5[name] = {"TFLOPs": 2.0 * len(rows) * K4 * 256 / t / 1e12, "seconds": t}
    det["C5_gemm_17408x5120_P256"] = dict(c5, sample="256 evenly spaced rows x all 256 tokens "
                                                  "(0.67 GFLOP), one run")
    # C3: decode stack, sampled: one GDN layer, one attention layer and the
    # lm_head through the oracle chain, scaled to the 64-layer token by bytes
    del ws
    sample = [0, 3]
    mats, shp = [], []
    for l in sample:
        for name in wl.LAYER_MATS:
            M, K = wl.layer_shapes(l)[name]
            mats.append(synth.q4k_weight(wl.stack_tensor_key(l, name), M, K))
            shp.append((M, K))
    mats.append(synth.q4k_weight(wl.stack_tensor_key(None, "lm_head"), wl.VOCAB, wl.HIDDEN))
    shp.append((wl.VOCAB, wl.HIDDEN))
    sb = sum(wbytes(M, K) for M, K in shp)
    h0 = synth.activations(3, 1, wl.HIDDEN)[0]
    c3 = {}
    for name, n in modes:
        oracle.set_threads(n)
        t = once(lambda: oracle.stack(mats, shp, len(sample), wl.HIDDEN, h0))
        c3[name] = {"us_per_token": t * 1e6 * wl.stack_bytes() / sb, "sample_seconds": t}
    det["C3_decode_stack"] = dict(c3, sample="layers 0 (GDN-shaped) and 3 (attention-shaped) "
                                             "plus the lm_head (%.2f GB), scaled by bytes to "
                                             "the 14.41 GB token" % (sb / 1e9))
    oracle.set_threads(n_all)
    head = c2["all_threads"]
    return {"cpu_baseline": {"value": head["GBps"], "unit": "GB/s", "cores": head["threads"],
                             "kind": "oracle",
                             "sample": "median of 3 runs (>= 1 s each) of the three full MLP "
                                       "GEMVs (gate, up, down), double-precision oracle, rows "
                                       "over %d threads on %s" % (head["threads"], det["cpu_model"])},
            "cpu_baseline_detail": det}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--sections", default="gemv,batch,small,q8,q6,gemm,stack,mixers,cpu",
                    help="comma list of gemv,batch,small,gemm,stack,cpu (and copy: the "
                         "256 MiB device copy that calibrates the PMC traffic counters)")
    ap.add_argument("--copies", type=int, default=12, help="cold-rotation copies per MLP matrix")
    ap.add_argument("--stack-tokens", type=int, default=20)
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    sections = set(s.strip() for s in args.sections.split(",") if s.strip())

    import numpy as np
    import torch

    import bit_block_quantized_gguf_amd as q4k
    import synth
    from synth import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    q4k.load()
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()

    def upload(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def settle(fn, ms=SETTLE_MS):
        """Untimed: call fn(i) for i = 0, 1, ... until `ms` of wall time have
        passed (synchronising every few calls).  The weights of each section
        are generated on the host first, during which the GPU idles; the
        first milliseconds of work after that run slower than the steady
        state (clocks, first touches of fresh allocations)."""
        t_end = time.perf_counter() + ms / 1e3
        i = 0
        while True:
            for _ in range(4):
                fn(i)
                i += 1
            torch.cuda.synchronize()
            if time.perf_counter() >= t_end:
                break

    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "settle_ms_before_each_timed_region": SETTLE_MS,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
           "data": "synthetic (seeded SplitMix64 Q4_K blocks, N(0,1) f32 activations)"}
    props = torch.cuda.get_device_properties(0)
    out["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                     "cus": props.multi_processor_count}

    # ------------------------------------------------------------ MLP GEMVs
    M_in, K_in = wl.INTER, wl.HIDDEN
    mlp_bytes = {name: wbytes(M, K) for name, M, K in wl.MLP}
    step_bytes = sum(mlp_bytes.values())
    x = synth.activations(2, 1, wl.HIDDEN)[0]
    xd = upload(x)
    if "gemv" in sections:
        log("generating MLP weights (%d copies of each)" % args.copies)
        copies = {}
        for i, (name, M, K) in enumerate(wl.MLP):
            hw = synth.q4k_weight(synth.key(2, i), M, K)
            copies[name] = [upload(hw) for _ in range(args.copies)]
        y_gate = torch.empty(M_in, device=dev)
        y_up = torch.empty(M_in, device=dev)
        y_down = torch.empty(wl.HIDDEN, device=dev)
        q4k.gemv(copies["gate"][0], xd, y_gate)
        q4k.gemv(copies["up"][0], xd, y_up)
        a = (torch.nn.functional.silu(y_gate) * y_up).contiguous()   # caller's SwiGLU, untimed
        torch.cuda.synchronize()

        def step(i):
            c = i % args.copies
            for name, w, xin, y in (("gate", copies["gate"][c], xd, y_gate),
                                    ("up", copies["up"][c], xd, y_up),
                                    ("down", copies["down"][c], a, y_down)):
                q4k.gemv(w, xin, y)

        for i in range(args.warmup):
            step(i)
        settle(step)
        # wall-clock step timing (no per-kernel events inside)
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        wall = (time.perf_counter() - t0) / args.steps
        # Per-matrix launch duration from HIP events on the launch stream: one
        # event pair around a burst of `steps` back-to-back launches of that
        # matrix (cold copies in rotation), so the average is the kernel time
        # plus the inter-kernel gap, as in the step, without event overhead
        # between launches.  Repeated 3 times; mean and median of the bursts.
        per = {n: [] for n in ("gate", "up", "down")}
        ins = {"gate": (xd, y_gate), "up": (xd, y_up), "down": (a, y_down)}
        for rep in range(3):
            for n in ("gate", "up", "down"):
                xin, y = ins[n]
                e0, e1 = ev(), ev()
                e0.record(stream)
                for i in range(args.steps):
                    q4k.gemv(copies[n][i % args.copies], xin, y)
                e1.record(stream)
                torch.cuda.synchronize()
                per[n].append(e0.elapsed_time(e1) * 1e3 / args.steps)   # us per launch
        kern = {n: float(np.mean(v)) for n, v in per.items()}
        kern_med = {n: float(np.median(v)) for n, v in per.items()}
        gpu_us = sum(kern.values())
        out["ms_per_step"] = wall * 1e3
        out["value"] = step_bytes / wall / 1e9
        out["unit"] = "GB/s"
        out["config"] = {
            "workload": "Qwen3.6-27B MLP block at batch 1: Q4_K GEMVs gate 17408x5120, "
                        "up 17408x5120, down 5120x17408 (SwiGLU by the caller), cold weights",
            "bytes_per_step": step_bytes, "copies_in_rotation": 3 * args.copies,
            "launch_shape": {"17408x5120": q4k.gemv_config(17408, 5120),
                             "5120x17408": q4k.gemv_config(5120, 17408)}}
        out["gemv_mlp"] = {n: {"us_mean": kern[n], "us_median": kern_med[n],
                               "GBps": mlp_bytes[n] / kern[n] / 1e3,
                               "frac_hbm": mlp_bytes[n] / kern[n] / 1e3 / HBM_PEAK_GBS}
                           for n in kern}
        out["gemv_mlp"]["kernel_sum_us"] = gpu_us
        gate_alg = mlp_bytes["gate"] + 4 * (5120 + 17408)  # weights + x + y
        achieved = gate_alg / kern["gate"] / 1e3
        traffic = None
        if os.path.exists(PROFILE_TRAFFIC):
            with open(PROFILE_TRAFFIC) as f:
                tr = json.load(f)
            if tr.get("source_hash") == source_hash(GEMV_SOURCES):
                traffic = tr.get("hbm_bytes_per_launch")
        out["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                           "kernel": "q4k_gemv on gate 17408x5120 (gemv_kernel<1,1,PLAIN>, one "
                                     "workgroup per resident slot over contiguous unit ranges, cut "
                                     "tiles finished in-kernel)",
                           "timing": "HIP events around bursts of back-to-back launches (kernel + gap)",
                           "algorithmic_bytes_per_launch": gate_alg}
        log("MLP GEMVs: step %.2f us wall, kernels %s" % (wall * 1e6, kern))
        # The same block through q4k_mlp: RMSNorm gain prologue, gate|up in one
        # pass with the SwiGLU on device, down with the residual add (bursts
        # of back-to-back calls on the cold copies, as above).
        gain = upload((0.2 * synth.normal(synth.key(2, 50), wl.HIDDEN)).astype(np.float32))
        y_mlp = torch.empty(wl.HIDDEN, device=dev)
        for i in range(args.warmup):
            c = i % args.copies
            q4k.mlp(copies["gate"][c], copies["up"][c], copies["down"][c], xd, gain, 1e-6, xd, y_mlp)
        settle(lambda i: q4k.mlp(copies["gate"][i % args.copies], copies["up"][i % args.copies],
                                 copies["down"][i % args.copies], xd, gain, 1e-6, xd, y_mlp))
        mlp_us = []
        for rep in range(3):
            e0, e1 = ev(), ev()
            e0.record(stream)
            for i in range(args.steps):
                c = i % args.copies
                q4k.mlp(copies["gate"][c], copies["up"][c], copies["down"][c], xd, gain, 1e-6, xd,
                        y_mlp)
            e1.record(stream)
            torch.cuda.synchronize()
            mlp_us.append(e0.elapsed_time(e1) * 1e3 / args.steps)
        t_mlp = float(np.mean(mlp_us))
        out["mlp_block"] = {"us_mean": t_mlp, "us_median": float(np.median(mlp_us)),
                            "GBps": step_bytes / t_mlp / 1e3,
                            "frac_hbm": step_bytes / t_mlp / 1e3 / HBM_PEAK_GBS,
                            "three_gemvs_us": gpu_us,
                            "call": "q4k_mlp: (1+w) RMSNorm prologue, gate|up SwiGLU GEMV, down GEMV + residual"}
        log("q4k_mlp: %.2f us per block (three GEMVs: %.2f us)" % (t_mlp, gpu_us))
        del copies
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ batched
    if "batch" in sections:
        M, K = wl.BATCH_SHAPE
        hw = synth.q4k_weight(synth.key(4, 0), M, K)
        ncop = 12
        ws = [upload(hw) for _ in range(ncop)]
        res = []
        for N in wl.BATCH_N:
            X = upload(synth.activations(4, N, K))
            Y = torch.empty((N, M), device=dev)
            for i in range(3):
                q4k.gemv_batch(ws[i % ncop], X, Y)
            settle(lambda i: q4k.gemv_batch(ws[i % ncop], X, Y))
            # bursts of back-to-back launches on the cold copies, one event
            # pair per burst (as for the MLP GEMVs above)
            nrep = max(10, args.steps)
            ts = []
            for rep in range(3):
                e0, e1 = ev(), ev()
                e0.record(stream)
                for i in range(nrep):
                    q4k.gemv_batch(ws[i % ncop], X, Y)
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3 / nrep)
            t = float(np.mean(ts))
            # matrix-core bound of the products the kernel issues: f32 MFMA
            # for N <= 8; for N = 16 three bf16 products per weight and vector
            # (split operands), at the bf16 rate
            if N == 16:
                mm_us, mm = 3 * 2.0 * M * K * N / (BF16_PEAK_TFLOPS * 1e12) * 1e6, "bf16 x3"
            else:
                mm_us, mm = 2.0 * M * K * N / 157.3e12 * 1e6, "f32"
            roof_us = max(wbytes(M, K) / HBM_PEAK_GBS / 1e3, mm_us)
            res.append({"N": N, "us": t, "us_per_vector": t / N, "matrix_products": mm,
                        "effective_GBps": N * wbytes(M, K) / t / 1e3,
                        "weight_GBps": wbytes(M, K) / t / 1e3,
                        "roofline_us": roof_us, "frac_roofline": roof_us / t})
        out["gemv_batch"] = res
        log("batched: %s" % [(r["N"], round(r["us"], 2)) for r in res])
        del ws
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ small GEMVs
    if "small" in sections:
        res = []
        for (M, K) in wl.SINGLE:
            hw = synth.q4k_weight(synth.key(1, 0), M, K)
            wd = upload(hw)
            xs = upload(synth.activations(1, 1, K)[0])
            y = torch.empty(M, device=dev)
            for _ in range(5):
                q4k.gemv(wd, xs, y)
            settle(lambda i: q4k.gemv(wd, xs, y))
            ts = []
            for _ in range(50):
                e0, e1 = ev(), ev()
                e0.record(stream)
                q4k.gemv(wd, xs, y)
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            # The per-call figure above includes the launch from an idle
            # queue.  The kernel's own latency: NG back-to-back calls
            # captured in one hipGraph, replayed; next to it the same for a
            # one-kernel torch fill of y (the launch floor).
            NG, R = 50, 10
            s2 = torch.cuda.Stream()
            s2.wait_stream(stream)
            with torch.cuda.stream(s2):
                for _ in range(3):
                    q4k.gemv(wd, xs, y)
                    y.fill_(0.0)
            torch.cuda.synchronize()
            per_graph = {}
            for name, fn in (("gemv", lambda: q4k.gemv(wd, xs, y)), ("fill", lambda: y.fill_(0.0))):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s2):
                    for _ in range(NG):
                        fn()
                g.replay()
                torch.cuda.synchronize()
                e0, e1 = ev(), ev()
                e0.record(stream)
                for _ in range(R):
                    g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                per_graph[name] = e0.elapsed_time(e1) * 1e3 / (R * NG)
                del g
            res.append({"M": M, "K": K, "us_median": float(np.median(ts)),
                        "us_in_graph": per_graph["gemv"], "floor_fill_us_in_graph": per_graph["fill"],
                        "bytes": wbytes(M, K)})
        out["gemv_small"] = res

    # ------------------------------------------------------------ Q8_0 GEMV
    if "q8" in sections:
        # the lm_head matmul in Q8_0 (vocab x hidden, 1.35 GB: larger than the
        # Infinity Cache, so every launch streams from HBM)
        M, K = wl.VOCAB, wl.HIDDEN
        log("generating the %dx%d Q8_0 lm_head" % (M, K))
        wq = upload(synth.q8_0_weight(synth.key(7, 1), M, K))
        xq = upload(synth.activations(7, 1, K)[0])
        yq = torch.empty(M, device=dev)
        for _ in range(3):
            q4k.gemv_q8_0(wq, xq, yq)
        settle(lambda i: q4k.gemv_q8_0(wq, xq, yq))
        reps = []
        for rep in range(3):
            e0, e1 = ev(), ev()
            e0.record(stream)
            for _ in range(10):
                q4k.gemv_q8_0(wq, xq, yq)
            e1.record(stream)
            torch.cuda.synchronize()
            reps.append(e0.elapsed_time(e1) * 1e3 / 10)
        qb = M * (K // 32) * 34 + 4 * (M + K)
        t = float(np.mean(reps))
        out["gemv_q8_0_lm_head"] = {"M": M, "K": K, "us": t, "bytes": qb, "GBps": qb / t / 1e3,
                                    "frac_hbm": qb / t / 1e3 / HBM_PEAK_GBS}
        log("q8_0 lm_head: %.1f us, %.0f GB/s" % (t, qb / t / 1e3))
        del wq
        torch.cuda.empty_cache()

    if "q6" in sections:
        # Q6_K, the other k-quant of q4_k_m files, on the two MLP shapes (73 MB
        # each; 8 copies of each in rotation, 585 MB, above the Infinity Cache)
        res = []
        for si, (name, M, K) in enumerate((("17408x5120", wl.INTER, wl.HIDDEN),
                                           ("5120x17408", wl.HIDDEN, wl.INTER))):
            hw = synth.q6_k_weight(synth.key(8, 100 + si), M, K)
            wc = [upload(hw) for _ in range(8)]
            x6 = upload(synth.activations(8, 1, K)[0])
            y6 = torch.empty(M, device=dev)
            for i in range(3):
                q4k.gemv_q6_k(wc[i % 8], x6, y6)
            settle(lambda i: q4k.gemv_q6_k(wc[i % 8], x6, y6))
            reps = []
            for rep in range(3):
                e0, e1 = ev(), ev()
                e0.record(stream)
                for i in range(args.steps):
                    q4k.gemv_q6_k(wc[i % 8], x6, y6)
                e1.record(stream)
                torch.cuda.synchronize()
                reps.append(e0.elapsed_time(e1) * 1e3 / args.steps)
            qb = hw.size + 4 * (M + K)
            t = float(np.mean(reps))
            res.append({"shape": name, "M": M, "K": K, "us": t, "bytes": qb, "GBps": qb / t / 1e3,
                        "frac_hbm": qb / t / 1e3 / HBM_PEAK_GBS})
            log("q6_k %s: %.1f us, %.0f GB/s" % (name, t, qb / t / 1e3))
            del wc
            torch.cuda.empty_cache()
        out["gemv_q6_k_mlp"] = res

    # ------------------------------------------------------------ prefill GEMM
    if "gemm" in sections:
        res = []
        for si, (M, K) in enumerate(wl.PREFILL_SHAPES):
            wd = upload(synth.q4k_weight(synth.key(5, si), M, K))
            # the prefill configs, then short prompts (22 and 27 tokens among them)
            for P in tuple(wl.PREFILL_P) + SHORT_P:
                X = upload(synth.activations(5, P, K))
                Y = torch.empty((P, M), device=dev)
                for _ in range(3):
                    q4k.gemm(wd, X, Y)
                settle(lambda i: q4k.gemm(wd, X, Y))
                pairs = []
                for _ in range(max(10, args.steps // 2)):
                    e0, e1 = ev(), ev()
                    e0.record(stream)
                    q4k.gemm(wd, X, Y)
                    e1.record(stream)
                    pairs.append((e0, e1))
                torch.cuda.synchronize()
                ts = [a.elapsed_time(b) * 1e3 for a, b in pairs]
                t = float(np.mean(ts))
                tf = 2.0 * M * K * P / t / 1e6
                res.append({"M": M, "K": K, "P": P, "us": t, "TFLOPs": tf,
                            "frac_bf16_peak": tf / BF16_PEAK_TFLOPS,
                            "tile_tokens_workgroups": list(q4k.gemm_config(M, K, P)),
                            "roofline": {"bound": "mfma", "achieved": tf,
                                         "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                                         "frac": tf / BF16_PEAK_TFLOPS, "traffic": None,
                                         "flops_per_call": 2.0 * M * K * P,
                                         "timing": "HIP events around each call (prologue, "
                                                   "main kernel and fix-up)"}})
                del X, Y
        out["prefill_gemm"] = [r for r in res if r["P"] not in SHORT_P]
        out["prefill_gemm_short"] = [r for r in res if r["P"] in SHORT_P]
        log("gemm: %s" % [(r["M"], r["P"], round(r["TFLOPs"], 1)) for r in res])
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ decode stack
    if "stack" in sections:
        L = wl.N_LAYERS
        log("generating the %d-layer stack (%.2f GB)" % (L, wl.stack_bytes() / 1e9))
        buf = None
        layers = []
        for l in range(L):
            d = {}
            for name, (M, K) in wl.layer_shapes(l).items():
                n = wbytes(M, K)
                if buf is None or buf.size < n:
                    buf = np.empty(wbytes(wl.VOCAB, wl.HIDDEN), np.uint8)
                hw = synth.q4k_weight(wl.stack_tensor_key(l, name), M, K,
                                      out=buf[:n].reshape(M, -1))
                d[name] = upload(hw)
            layers.append(d)
        n = wbytes(wl.VOCAB, wl.HIDDEN)
        lm = upload(synth.q4k_weight(wl.stack_tensor_key(None, "lm_head"), wl.VOCAB, wl.HIDDEN,
                                     out=buf[:n].reshape(wl.VOCAB, -1)))
        del buf
        log("capturing the decode graph")
        stk = q4k.DecodeStack(layers, lm, hidden=wl.HIDDEN,
                              kinds=[1 if wl.is_attention(l) else 0 for l in range(L)])
        h0 = upload(synth.activations(3, 1, wl.HIDDEN)[0])
        logits = torch.empty(wl.VOCAB, device=dev)
        for _ in range(3):
            stk(h0, logits)
        settle(lambda i: stk(h0, logits))
        pairs = []
        t0 = time.perf_counter()
        for _ in range(args.stack_tokens):
            e0, e1 = ev(), ev()
            e0.record(stream)
            stk(h0, logits)
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        wall_tok = (time.perf_counter() - t0) / args.stack_tokens * 1e6
        ts = [a.elapsed_time(b) * 1e3 for a, b in pairs]
        tot = wl.stack_bytes()
        roof = tot / HBM_PEAK_GBS / 1e3
        med = float(np.median(ts))
        out["decode_stack"] = {"us_per_token_median": med, "us_per_token_mean": float(np.mean(ts)),
                               "us_per_token_wall": wall_tok, "tokens": args.stack_tokens,
                               "weight_bytes": tot, "roofline_us": roof, "frac_roofline": roof / med,
                               "GBps": tot / med / 1e3, "graph_nodes": stk.nodes(),
                               "roofline": {"bound": "hbm", "achieved": tot / med / 1e3,
                                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                            "frac": tot / med / 1e3 / HBM_PEAK_GBS,
                                            "traffic": None,
                                            "bytes_per_token": tot,
                                            "timing": "HIP events around each token (h copy "
                                                      "in, graph launch, logits copy out)"}}
        log("stack: %.1f us/token (roofline %.1f)" % (med, roof))
        ref_logits = logits.clone()
        stk.close()
        # the same chain as one cooperative kernel per token
        log("persistent decode plan")
        pst = q4k.DecodeStack(layers, lm, hidden=wl.HIDDEN, persistent=True)
        for _ in range(3):
            pst(h0, logits)
        settle(lambda i: pst(h0, logits))
        pairs = []
        for _ in range(args.stack_tokens):
            e0, e1 = ev(), ev()
            e0.record(stream)
            pst(h0, logits)
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) * 1e3 for a, b in pairs]
        pmed = float(np.median(ts))
        same = bool(torch.equal(logits, ref_logits))
        out["decode_stack_persistent"] = {
            "us_per_token_median": pmed, "us_per_token_mean": float(np.mean(ts)),
            "tokens": args.stack_tokens, "roofline_us": roof, "frac_roofline": roof / pmed,
            "GBps": tot / pmed / 1e3, "kernels_per_token": 1, "logits_equal_graph": same,
            "wait_timeouts": pst.status()}
        log("persistent stack: %.1f us/token, logits equal to the graph plan's: %s" % (pmed, same))
        pst.close()
        # the same weights with the real token mixers (GDN step / gated
        # attention), positions 0 .. tokens-1 from zero states
        kinds = [1 if wl.is_attention(l) else 0 for l in range(L)]
        mixers = []
        for l in range(L):
            if kinds[l] == 0:
                C = (2 * 16 + 48) * 128
                mixers.append({"conv_w": upload((0.5 * synth.normal(synth.key(6, 10 * l), 4 * C)).astype(np.float32)),
                               "a_log": upload((0.5 * synth.normal(synth.key(6, 10 * l + 1), 48)).astype(np.float32)),
                               "dt_bias": upload((0.5 * synth.normal(synth.key(6, 10 * l + 2), 48)).astype(np.float32)),
                               "norm_w": upload((1 + 0.1 * synth.normal(synth.key(6, 10 * l + 3), 128)).astype(np.float32))})
            else:
                mixers.append({"q_norm_w": upload((0.2 * synth.normal(synth.key(6, 10 * l + 4), 256)).astype(np.float32)),
                               "k_norm_w": upload((0.2 * synth.normal(synth.key(6, 10 * l + 5), 256)).astype(np.float32))})
        ntok = max(args.stack_tokens, 4)
        mst = q4k.DecodeStack(layers, lm, hidden=wl.HIDDEN, kinds=kinds, mixers=mixers,
                              attn_capacity=ntok + 8)
        for _ in range(3):
            mst(h0, logits)
        torch.cuda.synchronize()
        mst.reset()
        pairs = []
        for _ in range(ntok):
            e0, e1 = ev(), ev()
            e0.record(stream)
            mst(h0, logits)
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        ts = [a.elapsed_time(b) * 1e3 for a, b in pairs]
        mmed = float(np.median(ts))
        state_bytes = 48 * (2 * 48 * 128 * 128 * 4)  # every GDN layer reads and writes its state
        out["decode_stack_mixers"] = {
            "us_per_token_median": mmed, "us_per_token_mean": float(np.mean(ts)),
            "tokens": ntok, "positions": "0..%d" % (ntok - 1), "graph_nodes": mst.nodes(),
            "bytes_per_token": tot + state_bytes,
            "roofline_us": (tot + state_bytes) / HBM_PEAK_GBS / 1e3,
            "frac_roofline": (tot + state_bytes) / HBM_PEAK_GBS / 1e3 / mmed,
            "logits_finite": bool(torch.isfinite(logits).all())}
        log("stack with mixers: %.1f us/token" % mmed)
        mst.close()
        del layers, lm
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ token mixers
    if "mixers" in sections:
        # One decode step of each mixer at the model's sizes, timed as a
        # replayed graph of 20 calls (the form it takes inside the decode
        # graph); bytes are the state (GDN) or the K/V cache (attention) that
        # one call must read and write.
        def graph_time(fn, calls=20, reps=10):
            fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(calls):
                    fn()
            g.replay()
            torch.cuda.synchronize()
            res = []
            for _ in range(reps):
                e0, e1 = ev(), ev()
                e0.record(stream)
                g.replay()
                e1.record(stream)
                torch.cuda.synchronize()
                res.append(e0.elapsed_time(e1) * 1e3 / calls)
            del g
            return float(np.median(res))

        Hk, Hv, D = 16, 48, 128
        C = (2 * Hk + Hv) * D
        nrm = lambda k, n, sc: upload((sc * synth.normal(synth.key(6, k), n)).astype(np.float32))
        gu = nrm(100, C + Hv * D + 2 * Hv, 1.0)
        gp = dict(conv_w=nrm(101, 4 * C, 0.5), a_log=nrm(102, Hv, 0.5), dt_bias=nrm(103, Hv, 0.5),
                  norm_w=upload((1 + 0.1 * synth.normal(synth.key(6, 104), D)).astype(np.float32)))
        cs, S = nrm(105, 3 * C, 1.0), nrm(106, Hv * D * D, 0.05)
        gout = torch.empty(Hv * D, device=dev)
        gws = q4k.Workspace(q4k.workspace_size(q4k.OP_GDN_STEP, Hk, Hv, 0))
        t_gdn = graph_time(lambda: q4k.gdn_step(gu, gp["conv_w"], gp["a_log"], gp["dt_bias"],
                                                gp["norm_w"], cs, S, gout, ws=gws))
        gdn_bytes = 2 * Hv * D * D * 4 + 2 * 3 * C * 4 + (C + Hv * D + 2 * Hv) * 4 + Hv * D * 4
        res = {"gdn_step": {"us": t_gdn, "bytes": gdn_bytes, "GBps": gdn_bytes / t_gdn / 1e3,
                            "frac_hbm": gdn_bytes / t_gdn / 1e3 / HBM_PEAK_GBS,
                            "kernels": 2, "heads": [Hk, Hv, D]}}
        Hq, Hkv, AD, cap = 24, 4, 256, 4096
        au = nrm(110, Hq * 2 * AD + 2 * Hkv * AD, 1.0)
        qw, kw = nrm(111, AD, 0.2), nrm(112, AD, 0.2)
        kc = nrm(113, Hkv * cap * AD, 1.0).view(Hkv, cap, AD)
        vc = nrm(114, Hkv * cap * AD, 1.0).view(Hkv, cap, AD)
        aout = torch.empty(Hq * AD, device=dev)
        aws = q4k.Workspace(q4k.workspace_size(q4k.OP_ATTN_STEP, Hq, Hkv, cap))
        res["attn_step"] = []
        for pos in (1023, 4095):
            t_a = graph_time(lambda: q4k.attn_step(au, qw, kw, kc, vc, pos, aout, ws=aws))
            ab = 2 * Hkv * (pos + 1) * AD * 4 + (Hq * 2 * AD + 2 * Hkv * AD + Hq * AD) * 4
            res["attn_step"].append({"pos": pos, "us": t_a, "bytes": ab,
                                     "GBps": ab / t_a / 1e3, "frac_hbm": ab / t_a / 1e3 / HBM_PEAK_GBS})
        out["mixers"] = res
        log("mixers: gdn %.2f us, attn %s" % (t_gdn, [(r["pos"], round(r["us"], 2)) for r in res["attn_step"]]))
        del kc, vc, S

    # ------------------------------------------------------------ counter calibration
    if "copy" in sections:
        # A plain device copy of known size: its FETCH_SIZE / WRITE_SIZE
        # readings under rocprofv3 --pmc give the factors that turn those
        # counters into bytes for the GEMV dispatches profiled in the same run.
        n = 256 << 20
        src = torch.ones(n // 4, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration"] = {"bytes_each_way": n, "launches": 3}
        del src, dst

    # ------------------------------------------------------------ CPU baseline
    if "cpu" in sections:
        out.update(cpu_leg(x, step_bytes))
    if "value" not in out:
        out["value"] = None
        out["unit"] = "GB/s"
        out["ms_per_step"] = None
        out["config"] = {"workload": "sections: " + ",".join(sorted(sections))}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
