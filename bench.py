"""Benchmark of the ROCmFP4 hot path on one MI355X.

A step is one decode GEMV over the up-projection workload: dual-scale ROCmFP4 weight
17408 x 5120 (50,135,040 packed bytes), fp16 activations, batch 1, fp32 output.
`value` is whole-job GB/s over the timed steps (algorithmic bytes: packed weights +
activations + outputs) with every input resident in HBM before timing starts. The
steps rotate over enough distinct weight copies (>= 600 MB) that no step is served
from the 256 MB Infinity Cache. The K steps are captured once in a HIP graph and
replayed inside the timed region, bracketed by device synchronizations.

Also measured in the same run (reported under "gemm" and "extra"): the prefill GEMM
(2048 x 17408 x 5120, bf16, TFLOP/s), the up-projection GEMV at batch 2/4/8 (matrix
cores), the fast-layout down-projection GEMV at batch 1/2/4/8 (bf16), dequantization,
encoding, and the 64-layer decode sweep (448 GEMVs, 12.3 GB).
The GEMV extras (batched, down-projection, fused) are timed as HIP graphs of 100
launches replayed back to back (event time of a replay / 100), so that the GPU never
waits for the host between these short kernels; the longer kernels (GEMM, dequant,
encoder) by HIP events around every launch on the stream they run on. A plain
streaming read of the same weight copies (librfp4_bench.so) gives the HBM read rate a
kernel of this size reaches, and a dense bf16 MFMA loop of the same library the matrix-core
rate the chip sustains (the GEMM's practical ceiling). The CPU baseline times the fp64 oracle on the host on every
workload (tiny, up-projection, down-projection at each batch, the full prefill GEMM).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-sweep] [--no-gemm]
       [--guard REFERENCE_JSON]   (exit 3 on a slowdown of more than 10 % against a saved line)
       [--pmc-mode | --pmc-gemm | --pmc-down | --sweep-only]   (short runs for rocprofv3)
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "ROCmFP4 GEMV GB/s (% of HBM peak) at 5120×17408 b=1; prefill GEMM TFLOP/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
ROTATE_MIN_BYTES = 600 * 2**20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemv_up.json")
GEMV_SOURCES = ["gemm_rfp4_block_amd/csrc/gemv_impl.h", "gemm_rfp4_block_amd/csrc/gemv_mfma.h",
                "gemm_rfp4_block_amd/csrc/gemv_f16.hip", "gemm_rfp4_block_amd/csrc/gemv.hip",
                "gemm_rfp4_block_amd/csrc/rfp4_decode.h", "gemm_rfp4_block_amd/csrc/gemv_tall.h"]
GEMM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_prefill.json")
GEMM_SOURCES = ["gemm_rfp4_block_amd/csrc/gemm.hip", "gemm_rfp4_block_amd/csrc/rfp4_decode.h",
                "gemm_rfp4_block_amd/csrc/rfp4_internal.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(paths):
    """Hash of the code in `paths` with comments and blank space taken out, so that the
    counters recorded against it stay valid across edits of comments only."""
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        # C/C++ comments (these sources hold no string literal with // or /*)
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def stats_us(samples_ms):
    a = np.asarray(samples_ms) * 1e3
    return dict(mean_us=float(a.mean()), median_us=float(np.median(a)),
                p10_us=float(np.percentile(a, 10)), p90_us=float(np.percentile(a, 90)))


def timed_launches(torch, fn, count):
    """Run fn(i) count times, each bracketed by events on the current stream.
    Returns per-launch durations in ms."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(count)]
    torch.cuda.synchronize()
    for i in range(count):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return [s.elapsed_time(e) for s, e in ev]


def graph_us(torch, fn, launches, replays=5):
    """Mean device time per call of fn(i), i < launches, with the GPU never waiting for
    the host: the calls are captured in one HIP graph on a stream that one eager call
    has set up first (per-stream workspaces exist before the capture, so the graph runs
    the eager plan), then replayed back to back; the mean over replays of
    (event time of one replay) / launches."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(launches):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    settle_graph(torch, g, 0.2)
    stream = torch.cuda.current_stream()
    per = []
    for _ in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        per.append(e0.elapsed_time(e1) * 1e3 / launches)
    del g
    return float(np.mean(per))


def settle_graph(torch, g, seconds):
    """Replay g untimed until `seconds` of wall time have passed: capturing a graph leaves
    the GPU idle long enough for its clocks to drop below their loaded level."""
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        g.replay()
        torch.cuda.synchronize()


def warm_up(torch, fn, seconds=0.3):
    """Call fn until `seconds` of wall time have passed (synchronizing every few calls),
    so that the timed region starts with the GPU clocks at their steady level (they
    take a few hundred milliseconds of load to settle)."""
    t_end = time.perf_counter() + seconds
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    return i


def rotation_copies(torch, R, layout, n, k, base_w, dev, seed0):
    import synth

    rb = synth.row_bytes(layout, k)
    count = max(2, -(-ROTATE_MIN_BYTES // (n * rb)))
    copies = [torch.from_numpy(base_w).to(dev)]
    for i in range(1, count):
        copies.append(synth.weights_device(layout, n, k, seed0 + i, dev))
    return copies


def bench_gemv_graph(torch, R, copies, layout, n, k, x, y, steps, warmup):
    """Headline: K GEMV launches captured in one graph, replayed in the timed region."""
    nc = len(copies)
    for i in range(warmup):
        R.rfp4_gemv(copies[i % nc], layout, n, k, x, y)
    warm_up(torch, lambda i: R.rfp4_gemv(copies[i % nc], layout, n, k, x, y))
    torch.cuda.synchronize()
    eager_ref = R.rfp4_gemv(copies[(steps - 1) % nc], layout, n, k, x).clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        R.rfp4_gemv(copies[0], layout, n, k, x, y)  # warm the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        for i in range(steps):
            R.rfp4_gemv(copies[i % nc], layout, n, k, x, y)
    g.replay()  # untimed replay, checked below against the eager result
    torch.cuda.synchronize()
    replay_ok = bool(torch.equal(y, eager_ref))
    settle_graph(torch, g, 0.3)
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    torch.cuda.synchronize()
    ev0.record(stream)
    g.replay()
    ev1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    replay_ok = replay_ok and bool(torch.equal(y, eager_ref))
    return (t1 - t0) * 1e3, ev0.elapsed_time(ev1), replay_ok


READ_UNROLL, READ_WGS_PER_CU = 1, 8  # the fastest launch shape of a sweep on MI355X


def bench_reader(torch, dev):
    """read(t, nbytes): one launch of the plain streaming read kernel (librfp4_bench.so)
    over the first nbytes of device tensor t, on the current stream."""
    import ctypes

    lib_path = os.path.join(ROOT, "gemm_rfp4_block_amd", "_lib", "librfp4_bench.so")
    B = ctypes.CDLL(lib_path)
    B.rfp4bench_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                 ctypes.c_void_p]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)

    def read(t, nbytes):
        st = B.rfp4bench_read(ctypes.c_void_p(t.data_ptr()), nbytes, READ_UNROLL, READ_WGS_PER_CU,
                              ctypes.c_void_p(sink.data_ptr()),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st != 0:
            raise RuntimeError(f"rfp4bench_read failed: {st}")

    return read


def read_ceiling(torch, copies, w_bytes, dev):
    """Plain streaming read (librfp4_bench.so) of the rotated weight copies (the bytes the
    headline GEMV reads, one 50 MB copy per launch) and of one 800 MiB buffer: the HBM
    read rate a kernel of that size reaches, for comparison with the GEMV."""
    read = bench_reader(torch, dev)
    nc = len(copies)
    fn = lambda i: read(copies[i % nc], w_bytes)
    warm_up(torch, fn, 0.1)
    us = graph_us(torch, fn, 100)
    big = torch.empty(800 * 2**20, dtype=torch.uint8, device=dev).fill_(3)
    fnb = lambda i: read(big, big.numel())
    warm_up(torch, fnb, 0.1)
    usb = graph_us(torch, fnb, 20)
    del big
    return {"rotated_50MB": {"us": round(us, 3), "GB/s": round(w_bytes / (us * 1e-6) / 1e9, 1),
                             "bytes": w_bytes, "copies": nc},
            "single_800MiB": {"us": round(usb, 2), "GB/s": round(800 * 2**20 / (usb * 1e-6) / 1e9, 1)},
            "kernel": f"rfp4bench_read (16-byte loads, {READ_UNROLL} per lane in flight, "
                      f"{READ_WGS_PER_CU} 256-thread workgroups per CU)"}


def mfma_ceiling(torch, dev):
    """Sustained dense bf16 matrix-core rate on this part (librfp4_bench.so's MFMA loop:
    v_mfma_f32_32x32x16_bf16 into independent accumulators, operands changing from one
    instruction to the next, no memory traffic), with one issuing wavefront per SIMD (what
    each phase of the GEMM's ping-pong schedule has) and with four. The published 2.5
    PFLOP/s stays the roofline peak; this is the rate the chip holds in practice."""
    import ctypes

    B = ctypes.CDLL(os.path.join(ROOT, "gemm_rfp4_block_amd", "_lib", "librfp4_bench.so"))
    B.rfp4bench_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    out = {}
    for key, wgs, threads, iters in (("one_wave_per_simd", 1, 256, 2048), ("four_waves_per_simd", 2, 512, 512)):
        def fn(i, wgs=wgs, threads=threads, iters=iters):
            st = B.rfp4bench_mfma(wgs, threads, iters, ctypes.c_void_p(sink.data_ptr()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
            if st != 0:
                raise RuntimeError(f"rfp4bench_mfma failed: {st}")
        warm_up(torch, fn, 0.3)
        d = stats_us(timed_launches(torch, fn, 10))
        flops = cus * wgs * (threads // 64) * iters * 8 * 32 * 32 * 16 * 2
        out[key] = {"TFLOP/s": round(flops / (d["mean_us"] * 1e-6) / 1e12, 1), "us": round(d["mean_us"], 1)}
    out["kernel"] = "rfp4bench_mfma (8 independent v_mfma_f32_32x32x16_bf16 chains per wavefront, hashed operands)"
    return out


GUARD_KEYS = [  # (path in the JSON line, True if lower is better)
    (("roofline", "avg_launch_us"), True),
    (("gemm", "mean_us"), True),
    (("extra", "gemv_down_fast_bf16", "b1", "mean_us"), True),
    (("extra", "gemv_down_fast_bf16", "b2", "mean_us"), True),
    (("extra", "gemv_down_fast_bf16", "b4", "mean_us"), True),
    (("extra", "gemv_down_fast_bf16", "b8", "mean_us"), True),
    (("extra", "gemv_up_dual_f16_batched", "b8", "mean_us"), True),
    (("extra", "gemv_multi", "gate_up", "fused_mean_us"), True),
    (("extra", "gemv_multi", "qkv", "fused_mean_us"), True),
    (("extra", "sweep_64_layers_fused", "ms_per_sweep"), True),
    (("extra", "dequant_up", "mean_us"), True),
]


def guard(result, ref_path, tol=0.10):
    """Regression guard: every GUARD_KEYS entry of `result` against the same entry of a
    committed reference line; a time more than `tol` above the reference is a
    regression. Returns (ok, report)."""
    with open(ref_path) as f:
        ref = json.loads(f.read().strip().splitlines()[-1])

    def get(d, path):
        for p in path:
            if not isinstance(d, dict) or p not in d:
                return None
            d = d[p]
        return d

    report, ok = {}, True
    for path, lower_better in GUARD_KEYS:
        a, b = get(result, path), get(ref, path)
        if a is None or b is None:
            continue
        ratio = a / b if lower_better else b / a
        bad = ratio > 1.0 + tol
        ok = ok and not bad
        report[".".join(path)] = {"now": a, "reference": b, "slowdown": round(ratio, 4), "regression": bad}
    return ok, report


def cpu_baseline(synth, w_host, x_host, layout, n, k, alg_bytes):
    """The fp64 oracle (dequantization, fp64 contraction and the |w||x| denominator) timed
    on the host: the tiny GEMV, the up-projection GEMV (the headline unit, GB/s), the
    down-projection GEMV at batch 1/2/4/8 and the full prefill GEMM once, each with its
    own wall time. `cores` is the number of BLAS threads the oracle's matrix products
    ran on; `host_cores` the CPUs this process may use."""
    import oracle.rfp4_oracle as O

    try:
        from threadpoolctl import threadpool_info

        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1

    def timed(fn, min_s, max_reps):
        reps, t = 0, 0.0
        while (t < min_s or reps == 0) and reps < max_reps:
            t0 = time.perf_counter()
            fn()
            t += time.perf_counter() - t0
            reps += 1
        return reps, t

    per = {}
    tw, tx, tcfg = synth.gemv_inputs("tiny")
    txh = tx.double().numpy()
    reps, t = timed(lambda: O.gemv(tw, tcfg["layout"], tcfg["n"], tcfg["k"], txh), 1.0, 4000)
    tb = tw.size + tcfg["k"] * 2 + tcfg["n"] * 4
    per["tiny_gemv"] = {"value": round(tb * reps / t / 1e9, 4), "unit": "GB/s", "reps": reps, "s": round(t, 2)}
    xh = x_host.double().numpy()
    reps, t = timed(lambda: O.gemv(w_host, layout, n, k, xh), 8.0, 40)
    up = {"value": round(alg_bytes * reps / t / 1e9, 4), "unit": "GB/s", "reps": reps, "s": round(t, 2)}
    per["up_gemv"] = up
    dw, dx, dcfg = synth.gemv_inputs("down")
    for b in (1, 2, 4, 8):
        xb = dx[:b].double().numpy()
        reps, t = timed(lambda: O.gemv(dw, dcfg["layout"], dcfg["n"], dcfg["k"], xb), 1.0, 8)
        bts = dw.size + b * dcfg["k"] * 2 + b * dcfg["n"] * 4
        per[f"down_gemv_b{b}"] = {"value": round(bts * reps / t / 1e9, 4), "unit": "GB/s", "reps": reps,
                                  "s": round(t, 2)}
    gw, ga, gcfg = synth.gemm_inputs("prefill")
    gah = ga.double().numpy()
    reps, t = timed(lambda: O.gemm(gw, gcfg["layout"], gcfg["n"], gcfg["k"], gah), 0.0, 1)
    flops = 2.0 * gcfg["m"] * gcfg["n"] * gcfg["k"]
    per["prefill_gemm"] = {"value": round(flops * reps / t / 1e12, 4), "unit": "TFLOP/s", "reps": reps,
                           "s": round(t, 2)}
    total_s = sum(v["s"] for v in per.values())
    return {"value": up["value"], "unit": "GB/s", "cores": int(blas_threads), "kind": "oracle",
            "host_cores": len(os.sched_getaffinity(0)),
            "sample": f"up-projection GEMV (17408 x 5120 dual, fp16 x, batch 1) x {up['reps']} in {up['s']} s; "
                      f"per_workload: the tiny GEMV repeated, the down-projection GEMV (5120 x 17408 fast, bf16 x) for about a second per batch, "
                      f"the full 2048 x 17408 x 5120 prefill GEMM once; {total_s:.1f} s of oracle work in all",
            "per_workload": per}


def run_sweeps(torch, R, synth, dev, reps=5):
    """The 64-layer decode sweep (448 dual GEMVs, 12.3 GB of weights, a fresh fp16 x per
    GEMV) as one captured graph, and the same layers with fused launches (q+k+v and
    gate+up share their x); wall time per sweep over `reps` replays after an untimed
    settling replay."""
    out = {}
    mats, xs, ys, total = [], [], [], 0
    for layer in range(synth.SWEEP_LAYERS):
        for pi, (name, sn, sk) in enumerate(synth.SWEEP_SHAPES):
            seed = 10_000 + layer * 16 + pi
            mats.append((synth.weights_device(0, sn, sk, seed, dev), sn, sk))
            xs.append(synth.activations_device(1, sk, "f16", seed, dev))
            ys.append(torch.empty((1, sn), dtype=torch.float32, device=dev))
            total += sn * synth.row_bytes(0, sk) + sk * 2 + sn * 4
    torch.cuda.synchronize()

    def sweep():
        for (wm, sn, sk), xx, yy in zip(mats, xs, ys):
            R.rfp4_gemv(wm, 0, sn, sk, xx, yy)

    sweep()
    g = torch.cuda.CUDAGraph()
    s2 = torch.cuda.Stream()
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s2):
        sweep()
    torch.cuda.current_stream().wait_stream(s2)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s2):
        sweep()
    g.replay()
    torch.cuda.synchronize()
    settle_graph(torch, g, 0.3)
    t0 = time.perf_counter()
    for _ in range(reps):
        g.replay()
    torch.cuda.synchronize()
    sweep_ms = (time.perf_counter() - t0) * 1e3 / reps
    out["sweep_64_layers"] = {"GB/s": round(total / (sweep_ms * 1e-3) / 1e9, 1), "bytes": total,
                                "ms_per_sweep": round(sweep_ms, 3), "launches": len(mats),
                                "tokens_per_s_equivalent": round(1e3 / sweep_ms, 1)}
    log(f"sweep: {sweep_ms:.3f} ms -> {out['sweep_64_layers']['GB/s']:.0f} GB/s")

    # fused: per layer one launch for q+k+v (shared x), o, gate+up (shared x), down
    nsh = len(synth.SWEEP_SHAPES)
    groups = [[0, 1, 2], [3], [4, 5], [6]]
    fcalls, ftotal = [], 0
    for layer in range(synth.SWEEP_LAYERS):
        for gidx in groups:
            ws_ = [mats[layer * nsh + j][0] for j in gidx]
            ns_ = [mats[layer * nsh + j][1] for j in gidx]
            kk = mats[layer * nsh + gidx[0]][2]
            xx = xs[layer * nsh + gidx[0]]
            yy = [ys[layer * nsh + j] for j in gidx]
            fcalls.append((ws_, ns_, kk, xx, yy))
            ftotal += sum(n * synth.row_bytes(0, kk) for n in ns_) + kk * 2 + sum(ns_) * 4

    def fsweep():
        for ws_, ns_, kk, xx, yy in fcalls:
            R.rfp4_gemv_multi(ws_, 0, ns_, kk, xx, yy)

    fsweep()
    g2 = torch.cuda.CUDAGraph()
    s3 = torch.cuda.Stream()
    s3.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s3):
        fsweep()
    torch.cuda.current_stream().wait_stream(s3)
    torch.cuda.synchronize()
    with torch.cuda.graph(g2, stream=s3):
        fsweep()
    g2.replay()
    torch.cuda.synchronize()
    settle_graph(torch, g2, 0.3)
    t0 = time.perf_counter()
    for _ in range(reps):
        g2.replay()
    torch.cuda.synchronize()
    fsweep_ms = (time.perf_counter() - t0) * 1e3 / reps
    out["sweep_64_layers_fused"] = {"GB/s": round(ftotal / (fsweep_ms * 1e-3) / 1e9, 1), "bytes": ftotal,
                                      "ms_per_sweep": round(fsweep_ms, 3), "launches": len(fcalls),
                                      "tokens_per_s_equivalent": round(1e3 / fsweep_ms, 1)}
    log(f"sweep fused: {fsweep_ms:.3f} ms -> {out['sweep_64_layers_fused']['GB/s']:.0f} GB/s")
    del mats, xs, ys, fcalls, g, g2
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--pmc-mode", action="store_true",
                    help="for rocprofv3 --pmc: a few headline GEMV launches and one plain "
                         "512 MiB device copy (the byte-count calibration), then exit")
    ap.add_argument("--pmc-gemm", action="store_true",
                    help="for rocprofv3 --pmc: a few prefill GEMM launches, then exit")
    ap.add_argument("--pmc-down", action="store_true",
                    help="for rocprofv3 --pmc: a few down-projection GEMV launches at batch 1 and 8, then exit")
    ap.add_argument("--sweep-only", action="store_true",
                    help="for rocprofv3 --kernel-trace: only the two 64-layer decode sweeps (a few replays each)")
    ap.add_argument("--guard", metavar="REFERENCE_JSON",
                    help="compare the run with a committed reference line; exit 3 if any guarded time "
                         "is more than 10 %% above (throughput more than 10 %% below) the reference")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the ROCmFP4 "
                          "contraction is measured per GPU; multi-GPU sharding is not built"}))
        sys.exit(2)

    import torch

    import gemm_rfp4_block_amd as R
    import synth

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    R.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    props = torch.cuda.get_device_properties(dev)
    log(f"device: {props.name} CUs={props.multi_processor_count} lib={R.library_path()}")

    if args.pmc_gemm:
        wg_host, a_host, gcfg = synth.gemm_inputs("prefill")
        wg = torch.from_numpy(wg_host).to(dev)
        a = a_host.to(dev)
        c = torch.empty((gcfg["m"], gcfg["n"]), dtype=torch.bfloat16, device=dev)
        for _ in range(8):
            R.rfp4_gemm(wg, gcfg["layout"], gcfg["n"], gcfg["k"], a, c)
        # a plain device copy of known size calibrates the HBM byte counters
        src = torch.empty(512 * 2**20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"pmc gemm mode done: 8 prefill GEMM launches, one copy of {src.numel()} bytes")
        return

    if args.pmc_down:
        wd_host, xd_host, dcfg = synth.gemv_inputs("down")
        dn, dk, dl = dcfg["n"], dcfg["k"], dcfg["layout"]
        dcopies = rotation_copies(torch, R, dl, dn, dk, wd_host, dev, 200)
        for b in (1, 8):
            xb = xd_host[:b].contiguous().to(dev)
            yb = torch.empty((b, dn), dtype=torch.float32, device=dev)
            for i in range(12):
                R.rfp4_gemv(dcopies[i % len(dcopies)], dl, dn, dk, xb, yb)
        src = torch.empty(512 * 2**20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log("pmc down mode done: 12 down-projection GEMVs at batch 1 and 8, one copy of 512 MiB")
        return

    if args.sweep_only:
        sw = run_sweeps(torch, R, synth, dev, reps=3)
        log(json.dumps(sw))
        return

    # ---------------- headline: up-projection GEMV, dual, fp16, batch 1
    w_host, x_host, cfg = synth.gemv_inputs("up")
    n, k, layout = cfg["n"], cfg["k"], cfg["layout"]
    copies = rotation_copies(torch, R, layout, n, k, w_host, dev, 100)
    x = x_host.to(dev)
    y = torch.empty((1, n), dtype=torch.float32, device=dev)
    w_bytes = n * synth.row_bytes(layout, k)
    alg_bytes = w_bytes + k * 2 + n * 4
    log(f"gemv up: {len(copies)} rotation copies ({len(copies) * w_bytes / 2**20:.0f} MiB)")

    if args.pmc_mode:
        nc = len(copies)
        for i in range(max(args.steps, 24)):
            R.rfp4_gemv(copies[i % nc], layout, n, k, x, y)
        # the read-ceiling kernel over the same copies (its own rows in the counter output)
        read = bench_reader(torch, dev)
        for i in range(max(args.steps, 24)):
            read(copies[i % nc], w_bytes)
        src = torch.empty(512 * 2**20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"pmc mode done: {max(args.steps, 24)} gemv launches of {alg_bytes} algorithmic bytes and as "
            f"many streaming reads of {w_bytes} bytes, "
            f"one copy of {src.numel()} bytes")
        return

    graph_ms, event_ms, replay_ok = bench_gemv_graph(torch, R, copies, layout, n, k, x, y, args.steps,
                                                     args.warmup)
    ms_per_step = graph_ms / args.steps
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    # Average launch duration: HIP events recorded on the launch stream around the timed
    # region (K back-to-back launches, so launch overheads overlap the previous kernel).
    launch_us = event_ms * 1e3 / args.steps
    achieved = alg_bytes / (launch_us * 1e-6) / 1e9

    nc = len(copies)
    # Per-launch distribution (each launch bracketed by its own events; includes the
    # dispatch gap, so these are upper bounds).
    durs = timed_launches(torch, lambda i: R.rfp4_gemv(copies[i % nc], layout, n, k, x, y), args.steps)
    st = stats_us(durs)
    # back-to-back launches without a graph, one event pair around all of them
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(args.steps):
        R.rfp4_gemv(copies[i % nc], layout, n, k, x, y)
    e1.record()
    torch.cuda.synchronize()
    direct_us = e0.elapsed_time(e1) * 1e3 / args.steps
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("source_hash") == source_hash(GEMV_SOURCES):
            traffic = tr.get("bytes_per_launch")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "gemv_kernel<dual, f16, batch 1, activations in LDS, block pairs>",
                "per_launch_bytes": alg_bytes, "avg_launch_us": round(launch_us, 3),
                "single_launch_event_us": {kk: round(v, 2) for kk, v in st.items()}}
    log(f"gemv up: wall {ms_per_step * 1e3:.2f} us/step -> {value:.0f} GB/s; "
        f"events over timed region {launch_us:.2f} us/launch -> {achieved:.0f} GB/s "
        f"({achieved / HBM_PEAK_GBS:.1%}); single-launch events mean {st['mean_us']:.2f} us")

    extra = {"gemv_up_graph_replay_matches_eager": replay_ok,
             "gemv_up_direct_launches": {"us_per_launch": round(direct_us, 3),
                                         "GB/s": round(alg_bytes / (direct_us * 1e-6) / 1e9, 1)}}
    # ---------------- HBM read ceiling: a plain streaming read of the same rotated 50 MB
    # weight copies, and of one 800 MiB buffer (graph-replayed like the GEMV extras)
    extra["hbm_read_ceiling"] = read_ceiling(torch, copies, w_bytes, dev)
    extra["hbm_read_ceiling"]["gemv_up_fraction_of_50MB_read"] = round(
        extra["hbm_read_ceiling"]["rotated_50MB"]["us"] / launch_us, 4)
    log(f"hbm read ceiling: 50 MB {extra['hbm_read_ceiling']['rotated_50MB']['us']:.2f} us "
        f"({extra['hbm_read_ceiling']['rotated_50MB']['GB/s']:.0f} GB/s), 800 MiB "
        f"{extra['hbm_read_ceiling']['single_800MiB']['GB/s']:.0f} GB/s; the GEMV runs at "
        f"{extra['hbm_read_ceiling']['gemv_up_fraction_of_50MB_read']:.1%} of the 50 MB read rate")
    # ---------------- up-projection GEMV at batch 2/4/8 (the matrix-core kernel)
    xs_host = synth.activations(np.random.default_rng(11), 8, k, "f16")
    up_batched = {}
    for b in (2, 4, 8):
        xb = xs_host[:b].contiguous().to(dev)
        yb = torch.empty((b, n), dtype=torch.float32, device=dev)
        fn = lambda i: R.rfp4_gemv(copies[i % nc], layout, n, k, xb, yb)
        warm_up(torch, fn, 0.1)
        us = graph_us(torch, fn, 100)
        bts = w_bytes + b * k * 2 + b * n * 4
        up_batched[f"b{b}"] = {"GB/s": round(bts / (us * 1e-6) / 1e9, 1), "bytes": bts, "mean_us": round(us, 2)}
        log(f"gemv up b={b}: {us:.2f} us/launch (graph) -> {up_batched[f'b{b}']['GB/s']:.0f} GB/s")
    extra["gemv_up_dual_f16_batched"] = up_batched
    del copies
    torch.cuda.empty_cache()

    # ---------------- down-projection GEMV, fast layout, bf16, batch 1/2/4/8 (1% stress blocks)
    wd_host, xd_host, dcfg = synth.gemv_inputs("down")
    dn, dk, dl = dcfg["n"], dcfg["k"], dcfg["layout"]
    dcopies = rotation_copies(torch, R, dl, dn, dk, wd_host, dev, 200)
    dw_bytes = dn * synth.row_bytes(dl, dk)
    down = {}
    for b in (1, 2, 4, 8):
        xb = xd_host[:b].contiguous().to(dev)
        yb = torch.empty((b, dn), dtype=torch.float32, device=dev)
        fn = lambda i: R.rfp4_gemv(dcopies[i % len(dcopies)], dl, dn, dk, xb, yb)
        warm_up(torch, fn, 0.1)
        us = graph_us(torch, fn, 100)
        bts = dw_bytes + b * dk * 2 + b * dn * 4
        down[f"b{b}"] = {"GB/s": round(bts / (us * 1e-6) / 1e9, 1), "bytes": bts, "mean_us": round(us, 2)}
        log(f"gemv down b={b}: {us:.2f} us/launch (graph) -> {down[f'b{b}']['GB/s']:.0f} GB/s")
    extra["gemv_down_fast_bf16"] = down
    del dcopies
    torch.cuda.empty_cache()

    # ---------------- dequant (write-bound)
    out = torch.empty((n, k), dtype=torch.float32, device=dev)
    wq = torch.from_numpy(w_host).to(dev)
    for _ in range(3):
        R.rfp4_dequant(wq, layout, n, k, out)
    d = stats_us(timed_launches(torch, lambda i: R.rfp4_dequant(wq, layout, n, k, out), 20))
    dq_bytes = w_bytes + n * k * 4
    extra["dequant_up"] = {"GB/s": round(dq_bytes / (d["mean_us"] * 1e-6) / 1e9, 1), "bytes": dq_bytes,
                           "mean_us": round(d["mean_us"], 2)}
    log(f"dequant: {d['mean_us']:.1f} us -> {extra['dequant_up']['GB/s']:.0f} GB/s")
    outb = torch.empty((n, k), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        R.rfp4_dequant_bf16(wq, layout, n, k, outb)
    d = stats_us(timed_launches(torch, lambda i: R.rfp4_dequant_bf16(wq, layout, n, k, outb), 20))
    dqb_bytes = w_bytes + n * k * 2
    extra["dequant_bf16_up"] = {"GB/s": round(dqb_bytes / (d["mean_us"] * 1e-6) / 1e9, 1), "bytes": dqb_bytes,
                                "mean_us": round(d["mean_us"], 2)}
    log(f"dequant bf16: {d['mean_us']:.1f} us -> {extra['dequant_bf16_up']['GB/s']:.0f} GB/s")
    # encoder (rfp4_quantize) on the same shape, bf16 source: reads 2 bytes, writes
    # 18/32 bytes per weight
    src = synth.real_weights(np.random.default_rng(3), n, k, "bf16").to(dev)
    wq2 = torch.empty_like(wq)
    call_q = lambda i: R.rfp4_quantize(src, layout, wq2)
    for _ in range(3):
        call_q(0)
    d = stats_us(timed_launches(torch, call_q, 20))
    q_bytes = n * k * 2 + w_bytes
    extra["quantize_bf16_up"] = {"GB/s": round(q_bytes / (d["mean_us"] * 1e-6) / 1e9, 1), "bytes": q_bytes,
                                 "mean_us": round(d["mean_us"], 2)}
    log(f"quantize bf16: {d['mean_us']:.1f} us -> {extra['quantize_bf16_up']['GB/s']:.0f} GB/s")
    del out, outb, src, wq2
    torch.cuda.empty_cache()

    # ---------------- prefill GEMM
    gemm = None
    if not args.no_gemm:
        wg_host, a_host, gcfg = synth.gemm_inputs("prefill")
        gn, gk, gm = gcfg["n"], gcfg["k"], gcfg["m"]
        # rotating weight copies (>= 600 MiB in all), as for the GEMVs: every call reads its
        # W from HBM rather than from the Infinity Cache
        gcopies = rotation_copies(torch, R, gcfg["layout"], gn, gk, wg_host, dev, 300)
        ngc = len(gcopies)
        a = a_host.to(dev)
        c = torch.empty((gm, gn), dtype=torch.bfloat16, device=dev)
        gfn = lambda i: R.rfp4_gemm(gcopies[i % ngc], gcfg["layout"], gn, gk, a, c)
        warm_up(torch, gfn)
        d = stats_us(timed_launches(torch, gfn, 50))
        flops = 2.0 * gm * gn * gk
        tf = flops / (d["mean_us"] * 1e-6) / 1e12
        # L2 <-> fabric bytes of one call (its three launches), from the FETCH_SIZE and
        # WRITE_SIZE counters scaled by a plain copy's readings; only while the GEMM
        # sources are the ones the counters were taken on
        gtraffic = None
        if os.path.exists(GEMM_TRAFFIC_FILE):
            with open(GEMM_TRAFFIC_FILE) as f:
                tr = json.load(f)
            if tr.get("source_hash") == source_hash(GEMM_SOURCES):
                gtraffic = tr.get("bytes_per_call")
        gemm = {"TFLOP/s": round(tf, 1), "flop": flops, "m": gm, "n": gn, "k": gk, "rotation_copies": ngc,
                "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": gtraffic},
                **{kk: round(v, 2) for kk, v in d.items()}}
        log(f"gemm: mean {d['mean_us']:.1f} us -> {tf:.1f} TFLOP/s ({tf / BF16_PEAK_TFLOPS:.1%} of bf16 peak)")
        mc = mfma_ceiling(torch, dev)
        gemm["mfma_ceiling"] = mc
        gemm["roofline"]["frac_of_sustained_mfma"] = round(tf / mc["four_waves_per_simd"]["TFLOP/s"], 4)
        log(f"sustained bf16 MFMA rate: {mc['four_waves_per_simd']['TFLOP/s']:.0f} TFLOP/s (four waves per SIMD), "
            f"{mc['one_wave_per_simd']['TFLOP/s']:.0f} (one); the GEMM runs at "
            f"{gemm['roofline']['frac_of_sustained_mfma']:.1%} of the former")
        # the dequantize-then-multiply baseline (bf16 expansion + rocBLAS dense GEMM)
        wbuf = torch.empty((gn, gk), dtype=torch.bfloat16, device=dev)
        call_fb = lambda i: R.rfp4_gemm_dequant(gcopies[i % ngc], gcfg["layout"], gn, gk, a, wbuf, c)
        warm_up(torch, call_fb)
        dfb = stats_us(timed_launches(torch, call_fb, 30))
        gemm["dequant_then_dense_baseline"] = {
            "TFLOP/s": round(flops / (dfb["mean_us"] * 1e-6) / 1e12, 1), "mean_us": round(dfb["mean_us"], 2),
            "what": "rfp4_gemm_dequant: bf16 expansion of W (178 MB written) + rocBLAS dense bf16 GEMM"}
        log(f"gemm dequant+dense baseline: mean {dfb['mean_us']:.1f} us -> "
            f"{gemm['dequant_then_dense_baseline']['TFLOP/s']:.1f} TFLOP/s")
        del gcopies, a, c, wbuf
        torch.cuda.empty_cache()

    # ---------------- fused multi-matrix GEMVs (gate + up, q + k + v), one launch each
    fused = {}
    for fname, parts in (("gate_up", [17408, 17408]), ("qkv", [6144, 1024, 1024])):
        fk = 5120
        sets = []
        total_w = sum(n * synth.row_bytes(0, fk) for n in parts)
        for ci in range(max(2, -(-ROTATE_MIN_BYTES // total_w))):
            sets.append([synth.weights_device(0, n, fk, 300 + 10 * ci + j, dev) for j, n in enumerate(parts)])
        xf = synth.activations_device(1, fk, "f16", 301, dev)
        yfs = [torch.empty((1, n), dtype=torch.float32, device=dev) for n in parts]
        call_f = lambda i: R.rfp4_gemv_multi(sets[i % len(sets)], 0, parts, fk, xf, yfs)
        call_s = lambda i: [R.rfp4_gemv(w, 0, n, fk, xf, y) for w, n, y in zip(sets[i % len(sets)], parts, yfs)]
        warm_up(torch, call_f, 0.1)
        warm_up(torch, call_s, 0.1)
        uf = graph_us(torch, call_f, 100)
        us_ = graph_us(torch, call_s, 100)
        bts = total_w + fk * 2 + sum(parts) * 4
        fused[fname] = {"parts": parts, "bytes": bts,
                        "fused_GB/s": round(bts / (uf * 1e-6) / 1e9, 1), "fused_mean_us": round(uf, 2),
                        "separate_GB/s": round(bts / (us_ * 1e-6) / 1e9, 1), "separate_mean_us": round(us_, 2)}
        log(f"gemv {fname}: fused {uf:.2f} us (graph) -> {fused[fname]['fused_GB/s']:.0f} GB/s; "
            f"separate {us_:.2f} us -> {fused[fname]['separate_GB/s']:.0f} GB/s")
        del sets
        torch.cuda.empty_cache()
    extra["gemv_multi"] = fused

    # ---------------- 64-layer decode sweep (448 dual GEMVs), separate and fused launches
    if not args.no_sweep:
        extra.update(run_sweeps(torch, R, synth, dev))

    # ---------------- CPU baseline: the fp64 oracle on the host, per workload
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(synth, w_host, x_host, layout, n, k, alg_bytes)
        log(f"cpu oracle: {cpu['value']} GB/s (up-projection); per workload: "
            + ", ".join(f"{kk} {v['value']} {v['unit']}" for kk, v in cpu["per_workload"].items()))

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded ROCmFP4 bytes: uniform indices, E4M3 scale exponents 4..9; fp16 x ~ N(0,1))",
        "config": {"workload": "ROCmFP4 dual-scale up-projection GEMV, weight 17408 x 5120, fp16 x, batch 1, fp32 y",
                   "rotation_copies": nc, "timing": "HIP graph of K launches, wall clock"},
        "roofline": roofline, "cpu_baseline": cpu, "gemm": gemm, "extra": extra,
    }
    status = 0
    if args.guard:
        ok, report = guard(result, args.guard)
        result["guard"] = {"reference": os.path.relpath(args.guard, ROOT), "ok": ok, "tolerance": 0.10,
                           "entries": report}
        if not ok:
            log("guard: regression of more than 10 % against " + args.guard + ": "
                + ", ".join(kk for kk, v in report.items() if v["regression"]))
            status = 3
    print(json.dumps(result), flush=True)
    if status:
        sys.exit(status)


if __name__ == "__main__":
    main()
