"""Benchmark: block-scaled decode GEMV (and prefill GEMM) on one MI355X.

Default workload (one step = one launch of the fused qgemv kernel: weight
stream, decode, block-scale fold and dot, A1-A4 of the hot path):
    nvfp4 decode GEMV, m=1, n=k=4096, W ~ N(0, 0.02) packed to E2M1 codes +
    E4M3 micro-scales per 16 + f32 global, x bf16 ~ N(0,1), out bf16.

`value` is the weight-stream rate (codes + scales + global bytes per launch
divided by the host-clock time per launch over exactly --steps launches)
with every input already resident in HBM.  Launches rotate over distinct
copies of the packed weight (640 MB in all) and 640 MB of other memory is
read and written just before the timed region, so every timed launch reads
its weight from HBM, not from the 256 MB Infinity Cache; launches are
replayed from HIP graphs captured before the clock starts.  The calibration
kernels give the measured ceilings (cold streaming read of the same bytes;
register-only bf16 MFMA loop) reported beside the vendor peaks.  The same line carries the prefill GEMM (mxfp4, m=2048, n=k=4096)
and the other decode/prefill workloads as `extra` entries, a `roofline` object
for the timed kernel, and the CPU oracle timed on a bounded sample as
`cpu_baseline`.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--no-extra] [--no-cpu] [--only-timed] [--mx-only] [--grouped-only] [--moe-decode-only]
                    [--small-m-only]
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
MALL_BYTES = 256 << 20          # MI355X Infinity Cache
FLUSH_BYTES = 640 << 20         # read + written before every timed region, evicting the MALL and L2s
STEADY_STEPS = 2000             # launches of the region that gives the roofline's launch duration

# sources each timed kernel is compiled from: traffic counters taken on an
# older version of any of them are not reported
KERNEL_SOURCES = {"qgemv": ["block_scaled_bit_e2m1_amd/csrc/gemv.hip", "block_scaled_bit_e2m1_amd/csrc/dot.hpp",
                            "block_scaled_bit_e2m1_amd/csrc/codec.hpp"],
                  "qgemm": ["block_scaled_bit_e2m1_amd/csrc/mfma.hip", "block_scaled_bit_e2m1_amd/csrc/codec.hpp",
                            "block_scaled_bit_e2m1_amd/csrc/epilogue.hpp"],
                  "qgemm_mx": ["block_scaled_bit_e2m1_amd/csrc/mxmma.hip", "block_scaled_bit_e2m1_amd/csrc/codec.hpp",
                               "block_scaled_bit_e2m1_amd/csrc/epilogue.hpp"]}
KERNEL_SOURCES["grouped"] = ["block_scaled_bit_e2m1_amd/csrc/grouped.hip"] + KERNEL_SOURCES["qgemm"]
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


_FLUSH = None


def flush_caches(device, stream):
    """Read and write FLUSH_BYTES of unrelated memory on the launch stream, so
    no weight copy is left in the 256 MB Infinity Cache or the L2s."""
    import torch

    global _FLUSH
    if _FLUSH is None:
        _FLUSH = torch.zeros(FLUSH_BYTES // 4, dtype=torch.int32, device=device)
    with torch.cuda.stream(stream):
        _FLUSH.add_(1)


def timed_calls(launch, n_items, steps, warmup, device, flush=True):
    """Time exactly `steps` calls of launch(i), i cycling over n_items distinct
    inputs.  The calls are replayed from HIP graphs captured before the clock
    starts: one graph of per = min(steps, max(n_items, 64)) calls replayed
    steps // per times, and one of the remaining calls.  W eager calls warm
    up first and the whole timed sequence (replays, flush, synchronize) is
    rehearsed twice untimed; then (flush=True) the caches are flushed, so
    the first pass over the inputs reads HBM, and later passes do too when the
    n_items inputs exceed the MALL.  Returns (event ms per call on the launch
    stream, host-clock ms per call), both over the whole timed region."""
    import torch

    stream = torch.cuda.Stream(device)
    per = max(1, min(steps, max(n_items, 64)))  # calls per graph, cycling the inputs
    full, rem = divmod(steps, per)
    torch.cuda.synchronize(device)
    with torch.cuda.stream(stream):
        for i in range(max(1, warmup)):
            launch(i % n_items)
    torch.cuda.synchronize(device)
    graphs = []
    for count, reps in ((per, full), (rem, 1)):
        if count and reps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(count):
                    launch(i % n_items)
            graphs.append((g, reps))
    # two untimed rehearsals of exactly the timed sequence: the first pass of
    # it pays one-time costs (measured: 181 vs 110 us for 20 launches)
    for _ in range(2):
        with torch.cuda.stream(stream):
            for g, reps in graphs:
                for _ in range(reps):
                    g.replay()
        if flush:
            flush_caches(device, stream)
        torch.cuda.synchronize(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        e0.record(stream)
        for g, reps in graphs:
            for _ in range(reps):
                g.replay()
        e1.record(stream)
    torch.cuda.synchronize(device)
    t1 = time.perf_counter()
    return e0.elapsed_time(e1) / steps, (t1 - t0) * 1e3 / steps


def time_workload(wl, steps, warmup, device, rotate=True):
    """Per-launch time (ms) of exactly `steps` launches of one workload, by
    events on the launch stream and by the host clock, with the weight copies
    rotated (qgemv) and the caches flushed before the timed region."""
    d = setup(wl, device, rotate)
    ev_ms, wall_ms = timed_calls(lambda i: launch(wl, d, i), d["copies"], steps, warmup, device, flush=rotate)
    timed = min(d["copies"], steps)
    cold = rotate and (steps <= d["copies"] or d["copies"] * d["wbytes"] >= 2 * MALL_BYTES)
    return {"launches": steps, "event_ms": ev_ms, "wall_ms": wall_ms, "wbytes": d["wbytes"], "copies": d["copies"],
            "copies_timed": timed, "footprint_bytes": timed * d["wbytes"], "cold": bool(cold), "data": d}


def calib_read(device, nbytes, steps=2000, warmup=50):
    """Measured streaming-read ceiling for a weight stream of nbytes: the
    library's calibration read kernel (bsq_calib_read, the decode kernel's
    16-byte nontemporal load form) over rotated buffers of that size, same
    graph replay and cache flush as the timed GEMV.  Returns GB/s and us."""
    import torch

    from block_scaled_bit_e2m1_amd import bsq

    nb = (nbytes + 15) // 16 * 16
    copies = max(1, ROTATE_BYTES // nb)
    bufs = [torch.randint(0, 1 << 30, (nb // 4,), dtype=torch.int32, device=device) for _ in range(copies)]
    sink = torch.zeros(1, dtype=torch.float32, device=device)

    def one(i):
        st = bsq.bsq_calib_read(bsq._ptr(bufs[i]), nb, bsq._ptr(sink), bsq._stream(device))
        assert st == bsq.OK, bsq.bsq_last_error()

    ev_ms, _ = timed_calls(one, copies, steps, warmup, device)
    del bufs
    return {"bytes": nb, "us": round(ev_ms * 1e3, 4), "GB/s": round(nb / (ev_ms * 1e-3) / 1e9, 2),
            "kernel": "read_kernel (bsq_calib_read)", "copies": copies}


def calib_mfma(device, iters=20000, workgroups=1024, reps=5):
    """Measured bf16 MFMA ceiling: the library's register-only MFMA loop
    (bsq_calib_mfma) at 4 waves per SIMD.  Returns TFLOP/s."""
    import torch

    from block_scaled_bit_e2m1_amd import bsq

    sink = torch.zeros(1, dtype=torch.float32, device=device)
    stream = torch.cuda.Stream(device)
    flops = float(workgroups) * 4 * iters * 4 * 32768

    def one():
        st = bsq.bsq_calib_mfma(iters, workgroups, bsq._ptr(sink), bsq._stream(device))
        assert st == bsq.OK, bsq.bsq_last_error()

    with torch.cuda.stream(stream):
        one()
    torch.cuda.synchronize(device)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            one()
        e1.record(stream)
    torch.cuda.synchronize(device)
    ms = e0.elapsed_time(e1) / reps
    return {"TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1), "kernel": "mfma_loop_kernel (bsq_calib_mfma)",
            "flops_per_launch": flops, "ms": round(ms, 4)}


def hot_time(wl, device, iters=2000):
    """Same launch on one resident copy (served partly from the Infinity Cache)."""
    r = time_workload(wl, iters, 50, device, rotate=False)
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


def time_moe_decode_shared(device, fmt="mxfp4", E=8, n=14336, k=4096, ids=(1, 6, 2, 5) * 4):
    """Decode-sized MoE where tokens share experts (8 tokens, top-2, all on 4
    of the 8 experts): the expert-grouped call (decode form: one pass over
    each routed expert for all its rows) against the per-row gather (one pass
    per routed row).  Rate = weight bytes of the distinct routed experts per
    launch / time; three expert stacks rotated so launches read HBM."""
    import torch

    from block_scaled_bit_e2m1_amd import bsq, workloads

    pw = bsq.pack(fmt, workloads.random_weights(E * n, k, seed=1005, sigma=0.02))
    copies = max(1, min(3, ROTATE_BYTES // pw.weight_bytes + 1))
    stacks = [bsq.to_device(pw, device) for _ in range(copies)]
    m = len(ids)
    x = torch.from_numpy(workloads.random_activations(m, k, seed=1006, act="bf16")).to(torch.bfloat16).to(device)
    eids = torch.tensor(ids, dtype=torch.int32, device=device)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=device)
    st, need = bsq.bsq_grouped_qgemm_workspace(m, E)
    assert st == bsq.OK
    ws = torch.empty(max(need, 4), dtype=torch.uint8, device=device)
    it, it2 = iter(range(1 << 62)), iter(range(1 << 62))
    reps = max(1, 600 // copies)
    us = graph_event_ms(lambda: bsq.grouped_qmm(stacks[next(it) % copies], E, eids, x, out=out, workspace=ws), copies,
                        reps, device) * 1e3
    us_gather = graph_event_ms(lambda: bsq.gather_qmm(stacks[next(it2) % copies], E, eids, x, out=out), copies,
                               reps, device) * 1e3
    wb = len(set(ids)) * pw.weight_bytes // E
    return {"workload": f"moe_decode_shared_{fmt}_{E}x{n}x{k}_rows{m}_experts{len(set(ids))}",
            "note": "decode MoE, tokens sharing experts: expert-grouped call (decode form: one pass per routed expert) "
                    "vs the per-row gather (one pass per routed row)",
            "value": round(wb / (us * 1e-6) / 1e9, 2), "unit": "GB/s", "us_per_launch": round(us, 3),
            "roofline_frac": round(wb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "us_per_launch_gather": round(us_gather, 3)}


def time_small_m(device, fmt="mxfp4", n=14336, k=4096, m=4):
    """Batched decode (a few bf16 rows, bsq_qgemm's default path: the decode
    GEMV kernel's multi-row form, one weight pass per 4 rows) against the
    MFMA path on the same call.  Rate = packed weight bytes per launch / time
    (ceil(m/4) passes stream it); the weight copies rotated span 640 MB."""
    import torch

    from block_scaled_bit_e2m1_amd import bsq, workloads

    pw = bsq.pack(fmt, workloads.random_weights(n, k, seed=1007, sigma=0.02))
    copies = max(2, min(32, ROTATE_BYTES // pw.weight_bytes + 1))
    ws = [bsq.to_device(pw, device) for _ in range(copies)]
    x = torch.from_numpy(workloads.random_activations(m, k, seed=1008, act="bf16")).to(torch.bfloat16).to(device)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=device)
    it, it2 = iter(range(1 << 62)), iter(range(1 << 62))
    reps = max(1, 400 // copies)
    us = graph_event_ms(lambda: bsq.qgemm(ws[next(it) % copies], x, out=out), copies, reps, device) * 1e3
    us_mfma = graph_event_ms(lambda: bsq.qgemm(ws[next(it2) % copies], x, out=out, path=bsq.PATH_MFMA), copies,
                             reps, device) * 1e3
    wb = pw.weight_bytes
    return {"workload": f"qgemm_small_m_{fmt}_{n}x{k}_m{m}",
            "note": "batched decode: default path (multi-row GEMV form) vs the MFMA path",
            "value": round(wb / (us * 1e-6) / 1e9, 2), "unit": "GB/s", "us_per_launch": round(us, 3),
            "roofline_frac": round(wb / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4), "us_per_launch_mfma": round(us_mfma, 3)}


def time_grouped_qmm(device, name="mxfp4_moe_prefill_8x4096", reps=200):
    """Prefill MoE step (bsq_grouped_qgemm): the routing kernel, then the
    grouped MFMA GEMM over 128-row tiles of each expert's rows, bf16 out.  One
    expert stack (its 71 MB stay in the Infinity Cache across launches; the
    step is bound by the matrix cores, not HBM).  Rate = 2*m*n*k / time."""
    import numpy as np
    import torch

    from block_scaled_bit_e2m1_amd import bsq, workloads

    wl = workloads.MOE_WORKLOADS[name]
    W, X, ids = workloads.generate_moe(wl)
    stack = bsq.to_device(bsq.pack(wl.fmt, W), device)
    del W
    x = torch.from_numpy(X).to(torch.bfloat16).to(device)
    eids = torch.from_numpy(ids).to(device)
    st, need = bsq.bsq_grouped_qgemm_workspace(wl.m, wl.experts)
    assert st == bsq.OK
    ws = torch.empty(need, dtype=torch.uint8, device=device)
    out = torch.empty((wl.m, wl.n), dtype=torch.bfloat16, device=device)
    ms = graph_event_ms(lambda: bsq.grouped_qmm(stack, wl.experts, eids, x, out=out, workspace=ws), 4,
                        max(1, reps // 4), device)
    tf = wl.flops / (ms * 1e-3) / 1e12
    rows = np.bincount(ids, minlength=wl.experts)
    roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic(name, "grouped"),
            "kernel": "route_kernel + mfma_kernel (bsq_grouped_qgemm)", "alg_flops_per_launch": wl.flops,
            "event_ms_per_launch": round(ms, 6)}
    return {"workload": name, "note": f"prefill MoE: {wl.tokens} tokens top-{wl.topk} of {wl.experts} {wl.fmt} "
            f"experts of {wl.n}x{wl.k}, rows grouped by expert on the device (bsq_grouped_qgemm)",
            "value": round(tf, 2), "unit": "TFLOP/s", "us_per_launch": round(ms * 1e3, 3),
            "roofline_frac": roof["frac"], "roofline": roof, "expert_rows": rows.tolist(),
            "tiles": int(sum((c + 127) // 128 for c in rows))}


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
        used = min(threads, wl.m)  # the oracle splits its dot by activation rows: one row, one thread
        return {"value": round(v, 4), "unit": "GB/s", "cores": used, "kind": "oracle",
                "sample": f"{reps} full passes of {wl.name} (dequant to f32 and the fp64 dot of its one "
                          f"activation row, {used} thread), {t_total:.1f} s", **stages}
    rows = max(1, min(wl.m, 16))
    t0 = time.perf_counter()
    wd = oracle.dequant_packed(p)
    oracle.matmul(X, wd, rows=np.arange(rows), threads=threads)
    t = time.perf_counter() - t0
    v = 2.0 * rows * wl.n * wl.k / t / 1e12
    return {"value": round(v, 6), "unit": "TFLOP/s", "cores": min(threads, rows), "kind": "oracle",
            "sample": f"dequant (1 thread) + fp64 dot of {rows} of {wl.m} rows of {wl.name} "
                      f"({min(threads, rows)} threads), {t:.1f} s", **stages}


def kernel_name(wl):
    """The kernel a workload's launch runs (as the library dispatches it)."""
    four = wl.fmt in ("mxfp4", "nvfp4", "int4_affine")
    if wl.op == "qgemv" and wl.act == "bf16" and wl.k % (32 if four else 16) == 0:
        one = wl.k == 64 * (2 if four else 4) * (32 if four else 16)
        return ("gemv1_kernel" if one else "gemv_kernel") + " (bsq_qgemv)"
    if wl.op == "qgemm" and wl.act == "bf16" and wl.m > 8:
        return "mfma_kernel (bsq_qgemm)"
    return "rows_kernel (bsq_qgemv / bsq_qgemm)"


def roofline_obj(wl, r, read_calib=None, mfma_calib=None):
    """Roofline object of one timed workload: achieved = algorithmic bytes (or
    flops) per launch / event-timed launch duration, against the vendor peak
    and, where taken, the peak measured on this device by the calibration
    kernels (same byte count / register-only MFMA loop)."""
    kind = "qgemv" if wl.op == "qgemv" else "qgemm"
    ev_s = r["event_ms"] * 1e-3
    if wl.op == "qgemv":
        io = (2 if wl.act == "bf16" else 4) * (wl.k + wl.n)
        alg = r["wbytes"] + io
        a = alg / ev_s / 1e9
        o = {"bound": "hbm", "achieved": round(a, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
             "frac": round(a / HBM_PEAK_GBS, 4), "traffic": measured_traffic(wl.name, kind),
             "kernel": kernel_name(wl), "alg_bytes_per_launch": alg, "event_ms_per_launch": round(r["event_ms"], 6),
             "event_ms_launches": r.get("steady_launches", r["launches"])}
        if "region_event_ms" in r:
            o["event_ms_per_step_timed_region"] = round(r["region_event_ms"], 6)
        if read_calib:
            w = r["wbytes"] / ev_s / 1e9  # weight stream rate, like for like with the read of the same bytes
            o.update({"measured_peak": read_calib["GB/s"], "frac_measured": round(w / read_calib["GB/s"], 4),
                      "measured_peak_kernel": read_calib["kernel"]})
        return o
    if not (wl.act == "bf16" and wl.m > 8):
        return None  # the small f32 case is launch-latency bound: no roofline
    a = wl.flops / ev_s / 1e12
    o = {"bound": "mfma", "achieved": round(a, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
         "frac": round(a / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": measured_traffic(wl.name, kind),
         "kernel": kernel_name(wl), "alg_flops_per_launch": wl.flops, "event_ms_per_launch": round(r["event_ms"], 6)}
    if mfma_calib:
        o.update({"measured_peak": mfma_calib["TFLOP/s"], "frac_measured": round(a / mfma_calib["TFLOP/s"], 4),
                  "measured_peak_kernel": mfma_calib["kernel"]})
    return o


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
    ap.add_argument("--grouped-only", action="store_true", help="only time the prefill MoE grouped GEMM and exit")
    ap.add_argument("--moe-decode-only", action="store_true",
                    help="only time the decode MoE with shared experts (grouped call vs gather) and exit")
    ap.add_argument("--small-m-only", action="store_true",
                    help="only time the batched-decode qgemm (a few bf16 rows: default path vs MFMA) and exit")
    ap.add_argument("--mx-pair", default="", help="with --mx-only: one pair XFMT,WFMT (e.g. mxfp4,mxfp4)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MIB",
                    help="only run torch's copy kernel on MIB MiB (counter calibration) and exit")
    ap.add_argument("--calib-stream", action="store_true",
                    help="only run the calibration kernels (cold streaming read of each decode workload's weight "
                         "bytes; register-only bf16 MFMA loop) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (the library has no multi-GPU "
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
    decode = [w for w in workloads.WORKLOADS.values() if w.op == "qgemv"]

    def read_calibs(steps):
        out = {}
        for w in decode:
            wb = bsq.packed_bytes(w.fmt, w.n, w.k)
            nb = sum(wb) + (4 if w.fmt == "nvfp4" else 0)
            if nb not in out:
                out[nb] = calib_read(device, nb, steps=steps)
        return out

    if args.calib_stream:
        for nb, c in read_calibs(max(20, args.steps)).items():
            print(json.dumps({"calib": "stream_read", **c}), flush=True)
        print(json.dumps({"calib": "mfma_bf16", **calib_mfma(device)}), flush=True)
        return
    if args.mx_only:
        pairs = [tuple(args.mx_pair.split(","))] if args.mx_pair else MX_PAIRS
        for xf, wf in pairs:
            print(json.dumps(time_qgemm_mx(device, xf, wf, reps=max(1, args.steps // 8))), flush=True)
        return
    if args.moe_decode_only:
        print(json.dumps(time_moe_decode_shared(device)), flush=True)
        return
    if args.small_m_only:
        print(json.dumps(time_small_m(device)), flush=True)
        return
    if args.grouped_only:
        print(json.dumps(time_grouped_qmm(device, reps=max(4, args.steps))), flush=True)
        return
    wl = workloads.WORKLOADS[args.workload]
    kind = "qgemv" if wl.op == "qgemv" else "qgemm"
    log(f"bench: {wl.name} steps={args.steps} warmup={args.warmup}")
    r = time_workload(wl, args.steps, args.warmup, device)
    ms = r["wall_ms"]
    if kind == "qgemv":
        metric, unit = HEADLINE_METRIC, "GB/s"  # value: the qgemv half of the metric
        value = r["wbytes"] / (ms * 1e-3) / 1e9
    else:
        metric, unit = "TFLOP/s (qgemm)", "TFLOP/s"
        value = wl.flops / (ms * 1e-3) / 1e12
    log(f"  {wl.name}: {value:.1f} {unit}  ({r['event_ms'] * 1e3:.2f} us/step by events, {ms * 1e3:.2f} us/step "
        f"by host clock over the {r['launches']} timed steps, {r['copies_timed']} weight copies timed, cold={r['cold']})")
    # The launch duration of the roofline: the same launches, rotation and cache
    # flush over a region long enough that the graph's start on the device
    # (tens of us, paid once per region) does not count as kernel time.
    rs = r if args.steps >= STEADY_STEPS else time_workload(wl, STEADY_STEPS, args.warmup, device)
    r["region_event_ms"] = r["event_ms"]
    r["event_ms"] = rs["event_ms"]
    r["steady_launches"] = rs["launches"]
    log(f"  {wl.name}: {r['event_ms'] * 1e3:.2f} us/launch by events over {rs['launches']} launches")

    calib = None
    if not args.only_timed:
        rc = read_calibs(2000)
        mc = calib_mfma(device)
        calib = {"stream_read": list(rc.values()), "mfma_bf16": mc}
        for c in rc.values():
            log(f"  calibration read {c['bytes']} B: {c['us']:.2f} us, {c['GB/s']:.0f} GB/s")
        log(f"  calibration bf16 MFMA loop: {mc['TFLOP/s']:.0f} TFLOP/s")

    def calib_for(w2):
        if calib is None:
            return None, None
        wb = sum(bsq.packed_bytes(w2.fmt, w2.n, w2.k)) + (4 if w2.fmt == "nvfp4" else 0)
        rd = next((c for c in calib["stream_read"] if c["bytes"] == (wb + 15) // 16 * 16), None)
        return rd, calib["mfma_bf16"]

    roof = roofline_obj(wl, r, *calib_for(wl))

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
            else:
                v, u = w2.flops / (r2["event_ms"] * 1e-3) / 1e12, "TFLOP/s"
            ro = roofline_obj(w2, r2, *calib_for(w2))
            e = {"workload": name, "value": round(v, 3), "unit": u, "us_per_launch": round(r2["event_ms"] * 1e3, 3),
                 "roofline_frac": None if ro is None else ro["frac"], "roofline": ro,
                 "weight_copies_timed": r2["copies_timed"], "cold": r2["cold"]}
            extra.append(e)
            log(f"  {name}: {v:.2f} {u} ({r2['event_ms'] * 1e3:.2f} us/launch)")
            del r2
            torch.cuda.empty_cache()

    if not args.no_extra and not args.only_timed:
        extra.append(time_quantize(device))
        for e in (time_rmsnorm_qgemv(device), time_gather_qmm(device), time_moe_decode_shared(device),
                  time_small_m(device)):
            extra.append(e)
            log(f"  {e['workload']}: {e['value']:.1f} GB/s ({e['us_per_launch']:.2f} us/launch)"
                + (f", per-row gather {e['us_per_launch_gather']:.2f} us" if 'us_per_launch_gather' in e else "")
                + (f", MFMA path {e['us_per_launch_mfma']:.2f} us" if 'us_per_launch_mfma' in e else ""))
        torch.cuda.empty_cache()
        e = time_grouped_qmm(device)
        extra.append(e)
        log(f"  {e['workload']}: {e['value']:.1f} TFLOP/s ({e['us_per_launch']:.2f} us/launch)")
        torch.cuda.empty_cache()
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
                   "weight_copies": r["copies"], "weight_copies_timed": r["copies_timed"],
                   "timed_footprint_bytes": r["footprint_bytes"], "caches_flushed_before_timing": True,
                   "cold_hbm_reads": r["cold"], "graph_replay": True},
        "roofline": roof, "cpu_baseline": cpu, "calibration": calib, "extra": extra,
    }
    gemm = [e for e in extra if e.get("workload") == "mxfp4_qgemm_2048" and e.get("unit") == "TFLOP/s"]
    if gemm:
        line["qgemm_m2048"] = {"workload": "mxfp4_qgemm_2048", "value": gemm[0]["value"], "unit": "TFLOP/s",
                               "us_per_launch": gemm[0]["us_per_launch"], "roofline_frac": gemm[0]["roofline_frac"],
                               "peak": MFMA_BF16_PEAK_TFLOPS, "roofline": gemm[0]["roofline"]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
