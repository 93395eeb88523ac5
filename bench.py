"""Benchmark: block-scaled decode GEMV (and prefill GEMM) on one MI355X.

Default workload (one step = one launch of the fused qgemv kernel: weight
stream, decode, block-scale fold and dot, A1-A4 of the hot path):
    nvfp4 decode GEMV, m=1, n=k=4096, W ~ N(0, 0.02) packed to E2M1 codes +
    E4M3 micro-scales per 16 + f32 global, x bf16 ~ N(0,1), out bf16.

`value` is the weight-stream rate (codes + scales + global bytes per launch
divided by the time per launch) with every input already resident in HBM.
Launches rotate over enough distinct copies of the packed weight (> 512 MB)
that each launch reads its weight from HBM, not from the 256 MB Infinity
Cache; launches are replayed from a HIP graph so host launch cost is not
measured.  The same line carries the prefill GEMM (mxfp4, m=2048, n=k=4096)
and the other decode/prefill workloads as `extra` entries, a `roofline` object
for the timed kernel, and the CPU oracle timed on a bounded sample as
`cpu_baseline`.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-extra] [--no-cpu] [--only-timed]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
MFMA_FP8_PEAK_TFLOPS = 5000.0   # dense fp8 (an fp8 operand on either side of the scaled MFMA)
MFMA_FP4_PEAK_TFLOPS = 10100.0  # dense fp4 (both operands fp4)
ROTATE_BYTES = 640 << 20        # distinct weight copies per rotation (> 2x the 256 MB MALL)

# sources each timed kernel is compiled from: traffic counters taken on an
# older version of any of them are not reported
KERNEL_SOURCES = {"qgemv": ["block_scaled_bit_e2m1_amd/csrc/rows.hip", "block_scaled_bit_e2m1_amd/csrc/codec.hpp"],
                  "qgemm": ["block_scaled_bit_e2m1_amd/csrc/mfma.hip", "block_scaled_bit_e2m1_amd/csrc/codec.hpp",
                            "block_scaled_bit_e2m1_amd/csrc/epilogue.hpp"],
                  "qgemm_mx": ["block_scaled_bit_e2m1_amd/csrc/mxmma.hip", "block_scaled_bit_e2m1_amd/csrc/codec.hpp",
                               "block_scaled_bit_e2m1_amd/csrc/epilogue.hpp"]}
MX_PAIRS = [("mxfp4", "mxfp4"), ("mxfp8_e4m3", "mxfp4"), ("mxfp8_e4m3", "mxfp8_e4m3")]
# The headline metric has two halves: the m = 1 decode GEMV's weight stream
# (the line's value) and the m = 2048 prefill GEMM's TFLOP/s (reported beside it).
HEADLINE_METRIC = "weight-stream GB/s (qgemv m=1) and TFLOP/s (qgemm m=2048) vs MI355X roofline"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha(kind):
    """Hash of the kernel's sources with // comments and blank lines dropped
    (a comment edit does not change the kernel the counters were taken on)."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        with open(os.path.join(ROOT, rel)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(workload, kind):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(workload)
    if not e or e.get("source_sha") != source_sha(kind):
        return None
    return e.get("bytes_per_launch")


def setup(wl, device, rotate=True):
    import torch

    from block_scaled_bit_e2m1_amd import bsq, workloads

    W, X = workloads.generate(wl)
    pw = bsq.pack(wl.fmt, W)
    wbytes = pw.weight_bytes + (4 if wl.fmt == "nvfp4" else 0)
    copies = max(1, ROTATE_BYTES // max(1, pw.weight_bytes)) if (rotate and wl.op == "qgemv") else 1
    dev = [bsq.to_device(pw, device) for _ in range(copies)]
    xdt = torch.bfloat16 if wl.act == "bf16" else torch.float32
    x = torch.from_numpy(X).to(xdt).to(device)
    if wl.op == "qgemv":
        x = x[0]
        out = torch.empty((wl.n,), dtype=xdt, device=device)
    else:
        out = torch.empty((wl.m, wl.n), dtype=xdt, device=device)
    return {"W": W, "X": X, "pw": pw, "dev": dev, "x": x, "out": out, "wbytes": wbytes, "copies": copies}


def launch(wl, d, i):
    from block_scaled_bit_e2m1_amd import bsq

    w = d["dev"][i % len(d["dev"])]
    if wl.op == "qgemv":
        bsq.qgemv(w, d["x"], out=d["out"])
    else:
        bsq.qgemm(w, d["x"], out=d["out"])


def time_workload(wl, steps, warmup, device, rotate=True, per_graph=None):
    """Per-launch time (ms) over `steps` launches replayed from HIP graphs,
    measured with events on the launch stream and with the host clock."""
    import torch

    d = setup(wl, device, rotate)
    if per_graph is None:
        per_graph = d["copies"] if wl.op == "qgemv" else (4 if wl.m > 8 else 64)
    per_graph = max(1, min(per_graph, steps))
    stream = torch.cuda.Stream(device)
    torch.cuda.synchronize(device)
    with torch.cuda.stream(stream):
        for i in range(per_graph):  # eager warm-up of every copy before capture
            launch(wl, d, i)
    torch.cuda.synchronize(device)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(per_graph):
            launch(wl, d, i)
    reps = max(1, steps // per_graph)
    wreps = max(1, warmup // per_graph) if warmup > 0 else 0
    with torch.cuda.stream(stream):
        for _ in range(wreps):
            g.replay()
    torch.cuda.synchronize(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize(device)
    t1 = time.perf_counter()
    launches = reps * per_graph
    ev_ms = e0.elapsed_time(e1) / launches
    wall_ms = (t1 - t0) * 1e3 / launches
    return {"launches": launches, "event_ms": ev_ms, "wall_ms": wall_ms, "wbytes": d["wbytes"], "copies": d["copies"],
            "data": d}


def hot_time(wl, device, iters=200):
    """Same launch on one resident copy (served partly from the Infinity Cache)."""
    r = time_workload(wl, iters * 10, 50, device, rotate=False, per_graph=64)
    return r["event_ms"]


def time_quantize(device, fmt="mxfp4", n=4096, k=4096, launches=200):
    """Device-side pack of an f32 weight already in HBM (bsq_quantize):
    bytes = f32 read + codes/scales written, per launch."""
    import torch

    from block_scaled_bit_e2m1_amd import bsq, workloads

    W = torch.from_numpy(workloads.random_weights(n, k, seed=1003, sigma=0.02)).to(device)
    q = bsq.quantize(fmt, W)
    status = torch.zeros(1, dtype=torch.int32, device=device)
    gdev = torch.ones(1, dtype=torch.float32, device=device)
    stream = torch.cuda.Stream(device)

    def one():
        st = bsq.bsq_quantize(q.fmt, 0, bsq._ptr(W), bsq.F32, n, k, bsq._ptr(q.codes), bsq._ptr(q.scales),
                              bsq._ptr(q.biases), bsq._ptr(gdev), bsq._ptr(status), bsq._stream(device))
        assert st == bsq.OK

    with torch.cuda.stream(stream):
        for _ in range(5):
            one()
    torch.cuda.synchronize(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(launches):
            one()
        e1.record(stream)
    torch.cuda.synchronize(device)
    us = e0.elapsed_time(e1) * 1e3 / launches
    nbytes = n * k * 4 + q.weight_bytes
    return {"workload": f"quantize_{fmt}_{n}x{k}", "note": "device pack of an f32 weight (bsq_quantize)",
            "value": round(nbytes / (us * 1e-6) / 1e9, 2), "unit": "GB/s", "us_per_launch": round(us, 3),
            "roofline_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def graph_event_ms(fn, per_graph, reps, device):
    """Average time (ms) of one fn() call: per_graph calls captured in a HIP
    graph, replayed reps times, timed by events on the capture stream."""
    import torch

    stream = torch.cuda.Stream(device)
    torch.cuda.synchronize(device)
    with torch.cuda.stream(stream):
        for _ in range(per_graph):
            fn()
    torch.cuda.synchronize(device)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for _ in range(per_graph):
            fn()
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize(device)
    return e0.elapsed_time(e1) / (reps * per_graph)


def time_qgemm_mx(device, xfmt, wfmt, m=2048, n=4096, k=4096, reps=100):
    """Both-operands MX GEMM on the scaled MFMA (bsq_qgemm_mx), bf16 out:
    the GEMM alone, and with the device quantize of the bf16 activations in
    front of it (the activation-quantized step as a caller runs it)."""
    import torch

    from block_scaled_bit_e2m1_amd import bsq, workloads

    w = bsq.to_device(bsq.pack(wfmt, workloads.random_weights(n, k, seed=1003, sigma=0.02)), device)
    x = torch.from_numpy(workloads.random_activations(m, k, seed=1004, act="bf16")).to(torch.bfloat16).to(device)
    xq = bsq.quantize(xfmt, x)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=device)
    gdev = torch.ones(1, dtype=torch.float32, device=device)
    status = torch.zeros(1, dtype=torch.int32, device=device)

    def gemm():
        bsq.qgemm_mx(xq, w, out=out)

    def step():
        st = bsq.bsq_quantize(xq.fmt, 0, bsq._ptr(x), bsq.BF16, m, k, bsq._ptr(xq.codes), bsq._ptr(xq.scales), None,
                              bsq._ptr(gdev), bsq._ptr(status), bsq._stream(device))
        assert st == bsq.OK
        gemm()

    flops = 2.0 * m * n * k
    peak = MFMA_FP4_PEAK_TFLOPS if xfmt == wfmt == "mxfp4" else MFMA_FP8_PEAK_TFLOPS
    g_ms = graph_event_ms(gemm, 4, reps, device)
    s_ms = graph_event_ms(step, 4, reps // 2, device)
    tf = flops / (g_ms * 1e-3) / 1e12
    name = f"qgemm_mx_{xfmt}_x_{wfmt}_{m}x{n}x{k}"
    return {"workload": name, "traffic": measured_traffic(name, "qgemm_mx"),
            "note": "scaled-MFMA GEMM, X and W both MX-packed (bsq_qgemm_mx), bf16 out; step = X quantize + GEMM",
            "value": round(tf, 2), "unit": "TFLOP/s", "us_per_launch": round(g_ms * 1e3, 3),
            "peak": peak, "roofline_frac": round(tf / peak, 4), "us_per_step_with_x_quantize": round(s_ms * 1e3, 3)}


def time_rmsnorm_qgemv(device, fmt="nvfp4", n=4096, k=4096, eps=1e-6):
    """Fused RMSNorm + decode GEMV (bsq_rmsnorm_qgemv), bf16 x and norm weight,
    weight copies rotated like the timed GEMV so every launch reads HBM."""
    import torch

    from block_scaled_bit_e2m1_amd import bsq, workloads

    pw = bsq.pack(fmt, workloads.random_weights(n, k, seed=1001, sigma=0.02))
    copies = max(1, ROTATE_BYTES // pw.weight_bytes)
    ws = [bsq.to_device(pw, device) for _ in range(copies)]
    x = torch.from_numpy(workloads.random_activations(1, k, seed=1002, act="bf16")[0]).to(torch.bfloat16).to(device)
    g = torch.linspace(0.5, 1.5, k, device=device).to(torch.bfloat16)
    out = torch.empty((n,), dtype=torch.bfloat16, device=device)
    it = iter(range(1 << 62))
    us = graph_event_ms(lambda: bsq.rmsnorm_qgemv(ws[next(it) % copies], x, g, eps, out=out), copies,
                        max(1, 3000 // copies), device) * 1e3
    wb = pw.weight_bytes + (4 if fmt == "nvfp4" else 0)
    return {"workload": f"rmsnorm_qgemv_{fmt}_{n}x{k}", "note": "fused RMSNorm + decode GEMV (bsq_rmsnorm_qgemv)",
            "value": round(wb / (us * 1e-6) / 1e9, 2), "unit": "GB/s", "us_per_launch": round(us, 3),
            "roofline_frac": round(wb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def time_gather_qmm(device, fmt="mxfp4", E=8, n=14336, k=4096, ids=(1, 6, 2, 5)):
    """Expert-routed decode (bsq_gather_qmm): two tokens, top-2 of E experts,
    bf16 x; three expert stacks rotated so launches read HBM.  Rate = weight
    bytes of the routed experts per launch / time."""
    import torch

    from block_scaled_bit_e2m1_amd import bsq, workloads

    pw = bsq.pack(fmt, workloads.random_weights(E * n, k, seed=1005, sigma=0.02))
    copies = max(1, min(3, ROTATE_BYTES // pw.weight_bytes + 1))
    stacks = [bsq.to_device(pw, device) for _ in range(copies)]
    x = torch.from_numpy(workloads.random_activations(len(ids), k, seed=1006, act="bf16")).to(torch.bfloat16).to(device)
    eids = torch.tensor(ids, dtype=torch.int32, device=device)
    out = torch.empty((len(ids), n), dtype=torch.bfloat16, device=device)
    it = iter(range(1 << 62))
    us = graph_event_ms(lambda: bsq.gather_qmm(stacks[next(it) % copies], E, eids, x, out=out), copies,
                        max(1, 600 // copies), device) * 1e3
    wb = len(ids) * pw.weight_bytes // E
    return {"workload": f"gather_qmm_{fmt}_{E}x{n}x{k}_rows{len(ids)}",
            "note": "expert-routed decode: each routed row streams its expert (bsq_gather_qmm)",
            "value": round(wb / (us * 1e-6) / 1e9, 2), "unit": "GB/s", "us_per_launch": round(us, 3),
            "roofline_frac": round(wb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def warm_up(device, seconds=0.5):
    """Keep the GPU busy for a moment before anything is timed, so the first
    measurement does not run on a cold clock (measured: the first timing of a
    process read ~10% slow otherwise)."""
    import torch

    a = torch.randn(4096, 4096, device=device, dtype=torch.bfloat16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(20):
            a = a @ a
            a = a / a.abs().amax().clamp_min(1.0)
        torch.cuda.synchronize(device)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s=10.0):
    """The oracle as it stands on the host cores: pack, dequant and the fp64
    matmul timed separately (the matmul single-threaded and on all threads),
    then full passes (dequant + all-thread matmul) for ~budget_s seconds."""
    import numpy as np

    import oracle

    threads = max(1, min(16, os.cpu_count() or 1))
    W, X = __import__("block_scaled_bit_e2m1_amd.workloads", fromlist=["generate"]).generate(wl)
    t0 = time.perf_counter()
    p = oracle.pack(wl.fmt, W)
    t_pack = time.perf_counter() - t0
    wb = p["codes"].size + p["scales"].size + (0 if p["biases"] is None else p["biases"].size)
    wb += 4 if wl.fmt == "nvfp4" else 0
    t0 = time.perf_counter()
    wd = oracle.dequant_packed(p)
    t_deq = time.perf_counter() - t0
    rows = np.arange(max(1, min(wl.m, 16 if wl.op == "qgemv" else 2)))
    t0 = time.perf_counter()
    oracle.matmul(X, wd, rows=rows, threads=1)
    t_mm1 = (time.perf_counter() - t0) / len(rows)
    t0 = time.perf_counter()
    oracle.matmul(X, wd, rows=rows, threads=threads)
    t_mmn = (time.perf_counter() - t0) / len(rows)
    stages = {"cpu_model": cpu_model(), "nproc": os.cpu_count(), "pack_s": round(t_pack, 4), "dequant_s": round(t_deq, 4),
              "matmul_s_per_row_1_thread": round(t_mm1, 6), "matmul_s_per_row_all_threads": round(t_mmn, 6)}
    reps, t_total = 0, 0.0
    if wl.op == "qgemv":
        while t_total < budget_s or reps < 2:
            t0 = time.perf_counter()
            wd = oracle.dequant_packed(p)
            oracle.matmul(X, wd, threads=threads)
            t_total += time.perf_counter() - t0
            reps += 1
        v = wb * reps / t_total / 1e9
        return {"value": round(v, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
                "sample": f"{reps} full passes of {wl.name} (dequant to f32 on 1 core, then fp64 dot on "
                          f"{threads} threads), {t_total:.1f} s", **stages}
    rows = max(1, min(wl.m, 16))
    t0 = time.perf_counter()
    wd = oracle.dequant_packed(p)
    oracle.matmul(X, wd, rows=np.arange(rows), threads=threads)
    t = time.perf_counter() - t0
    v = 2.0 * rows * wl.n * wl.k / t / 1e12
    return {"value": round(v, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"dequant + fp64 dot of {rows} of {wl.m} rows of {wl.name}, {t:.1f} s", **stages}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="nvfp4_qgemv_4096")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only-timed", action="store_true", help="timed workload only (for profiling)")
    ap.add_argument("--mx-only", action="store_true", help="only time the scaled-MFMA GEMMs and exit")
    ap.add_argument("--mx-pair", default="", help="with --mx-only: one pair XFMT,WFMT (e.g. mxfp4,mxfp4)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="only run torch's copy kernel on MIB MiB (counter calibration) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (this build has no multi-GPU "
              f"path; the decode/prefill kernels shard along n with no exchange step).", file=sys.stderr)
        sys.exit(2)

    import torch

    from block_scaled_bit_e2m1_amd import bsq, workloads

    device = torch.device("cuda:0")
    if args.calib_copy:
        # A plain device copy of known size: its FETCH_SIZE / WRITE_SIZE
        # counters calibrate the byte counters of the timed kernels.
        n = args.calib_copy << 20
        src = torch.ones(n // 4, dtype=torch.int32, device=device)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize(device)
        print(json.dumps({"calib_copy_bytes": n, "launches": max(1, args.steps)}), flush=True)
        return
    bsq.lib()
    warm_up(device)
    if args.mx_only:
        pairs = [tuple(args.mx_pair.split(","))] if args.mx_pair else MX_PAIRS
        for xf, wf in pairs:
            print(json.dumps(time_qgemm_mx(device, xf, wf, reps=max(1, args.steps // 8))), flush=True)
        return
    wl = workloads.WORKLOADS[args.workload]
    kind = "qgemv" if wl.op == "qgemv" else "qgemm"
    log(f"bench: {wl.name} steps={args.steps} warmup={args.warmup}")
    r = time_workload(wl, args.steps, args.warmup, device)
    ms = r["wall_ms"]
    if kind == "qgemv":
        metric, unit = HEADLINE_METRIC, "GB/s"  # value: the qgemv half of the metric
        value = r["wbytes"] / (ms * 1e-3) / 1e9
        io_bytes = 2 * (wl.k + wl.n) if wl.act == "bf16" else 4 * (wl.k + wl.n)
        alg = r["wbytes"] + io_bytes
        achieved = alg / (r["event_ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl.name, kind),
                "kernel": "rows_kernel (bsq_qgemv)", "alg_bytes_per_launch": alg,
                "event_ms_per_launch": round(r["event_ms"], 6)}
    else:
        metric, unit = "TFLOP/s (qgemm)", "TFLOP/s"
        value = wl.flops / (ms * 1e-3) / 1e12
        achieved = wl.flops / (r["event_ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic(wl.name, kind),
                "kernel": "mfma_kernel (bsq_qgemm)", "alg_flops_per_launch": wl.flops,
                "event_ms_per_launch": round(r["event_ms"], 6)}
    log(f"  {wl.name}: {value:.1f} {unit}  ({r['event_ms'] * 1e3:.2f} us/launch by events, "
        f"{ms * 1e3:.2f} us by host clock, {r['copies']} weight copies)")

    extra = []
    if not args.no_extra and not args.only_timed:
        hot = hot_time(wl, device)
        extra.append({"workload": wl.name, "note": "same launch on one resident weight copy (Infinity Cache hot)",
                      "us_per_launch": round(hot * 1e3, 3), "value": round(r["wbytes"] / (hot * 1e-3) / 1e9, 2)
                      if kind == "qgemv" else round(wl.flops / (hot * 1e-3) / 1e12, 2), "unit": unit})
        for name, w2 in workloads.WORKLOADS.items():
            if name == wl.name:
                continue
            steps = 400 if w2.op == "qgemm" and w2.m > 8 else 2000
            r2 = time_workload(w2, steps, steps // 10, device)
            if w2.op == "qgemv":
                v, u = r2["wbytes"] / (r2["event_ms"] * 1e-3) / 1e9, "GB/s"
                fr = v / HBM_PEAK_GBS
            else:
                v, u = w2.flops / (r2["event_ms"] * 1e-3) / 1e12, "TFLOP/s"
                fr = v / MFMA_BF16_PEAK_TFLOPS if w2.act == "bf16" and w2.m > 8 else None
            e = {"workload": name, "value": round(v, 3), "unit": u, "us_per_launch": round(r2["event_ms"] * 1e3, 3),
                 "roofline_frac": None if fr is None else round(fr, 4)}
            extra.append(e)
            log(f"  {name}: {v:.2f} {u} ({r2['event_ms'] * 1e3:.2f} us/launch)")
            del r2
            torch.cuda.empty_cache()

    if not args.no_extra and not args.only_timed:
        extra.append(time_quantize(device))
        for e in (time_rmsnorm_qgemv(device), time_gather_qmm(device)):
            extra.append(e)
            log(f"  {e['workload']}: {e['value']:.1f} GB/s ({e['us_per_launch']:.2f} us/launch)")
        for xf, wf in MX_PAIRS:
            e = time_qgemm_mx(device, xf, wf)
            extra.append(e)
            log(f"  {e['workload']}: {e['value']:.1f} TFLOP/s ({e['us_per_launch']:.2f} us/launch, "
                f"{e['us_per_step_with_x_quantize']:.2f} us with X quantize)")

    cpu = None
    if not args.no_cpu and not args.only_timed:
        log("  cpu baseline (oracle) ...")
        cpu = cpu_baseline(wl)

    line = {
        "metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": r["launches"],
        "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if wl.act == "bf16" else "f32",
        "data": "synthetic (seeded N(0,sigma) weights, N(0,1) activations)",
        "config": {"workload": wl.name, "format": wl.fmt, "m": wl.m, "n": wl.n, "k": wl.k,
                   "weight_copies_rotated": r["copies"], "graph_replay": True},
        "roofline": roof, "cpu_baseline": cpu, "extra": extra,
    }
    gemm = [e for e in extra if e.get("workload") == "mxfp4_qgemm_2048" and e.get("unit") == "TFLOP/s"]
    if gemm:
        line["qgemm_m2048"] = {"workload": "mxfp4_qgemm_2048", "value": gemm[0]["value"], "unit": "TFLOP/s",
                               "us_per_launch": gemm[0]["us_per_launch"], "roofline_frac": gemm[0]["roofline_frac"],
                               "peak": MFMA_BF16_PEAK_TFLOPS}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
