#!/usr/bin/env python3
"""Benchmark of libmgemm on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one mgemm_run over the workload (host normalisation and dispatch,
tile rasterisation, LDS staging, the MFMA/FMA contraction and the epilogue,
all in one kernel launch) with every operand already resident in HBM.  The
default workload is FP32 SGEMM 4096^3 row-major (uniform [-1,1] inputs).

Prints ONE JSON line.  `roofline` is measured live with HIP events around
each launch on the stream the kernel runs on; `cpu_baseline` times the CPU
oracle on a bounded sample of the same workload (and checks that sample
against the GPU result).  Other workloads are measured briefly and reported
under `workloads` (skip with --only-headline).
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

METRIC = "TFLOP/s and % of MFMA/FP32 peak (HBM GB/s for M≤64) vs CPU oracle, 1 GPU"
# Pages' number for this exact workload and metric: cuBLAS pure-FP32 SGEMM
# 4096^3 on an RTX 4090 (SGEMM report, cuBLAS denominator section): context only.
PAGES_SGEMM_4096_TFLOPS = 57.2424


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# Source file of each kernel variant; the counter summary of a kernel is valid
# while this file and the shared header are unchanged.
KERNEL_SOURCE = {
    "general": "k_general.hip", "f32_mfma": "k_f32_mfma.hip", "f32_fast": "k_f32_mfma.hip",
    "f32_fast_128": "k_f32_mfma.hip", "h_mfma_256x256": "k_h_mfma.hip",
    "h_mfma_256x192": "k_h_mfma.hip", "h_mfma_128x128": "k_h_mfma.hip",
    "h_pp_256x256": "k_h_pp.hip", "h_dma_256x256": "k_h_dma.hip", "skinny": "k_skinny.hip",
    "skinny_sk": "k_skinny_sk.hip", "h_dma_256x192": "k_h_dma.hip", "f32_fast_u": "k_f32_mfma.hip",
    "h_dma_gated": "k_h_dma.hip", "fp8_quant+fp8_gemm": "k_f8.hip", "f32_sk": "k_f32_mfma.hip", "h_dma_128x192": "k_h_dma.hip",
}


def src_hash(kernel: str | None = None) -> str:
    """Hash of the kernel's source and the shared header (all sources if None)."""
    d = os.path.join(ROOT, "dense_gemm_mgemm_amd", "csrc")
    if kernel is None:
        files = [f for f in sorted(os.listdir(d)) if f.endswith((".hip", ".h", ".cpp"))]
    else:
        files = ["common.h", KERNEL_SOURCE[kernel.split("/")[0]]]
    h = hashlib.sha256()
    for f in files:
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def workload_table():
    import workloads as W
    t = {"sgemm_4096": W.sgemm_4096(), "sgemm_256": W.sgemm_256(), "ragged_f32": W.ragged_f32(),
         "ffn_bf16": W.ffn_bf16(), "ffn_bf16_silu": W.ffn_bf16_silu(),
         "ffn_gated_bf16": W.ffn_gated_bf16(), "ffn_share_bf16": W.ffn_share_bf16(),
         "ffn_gated_share_bf16": W.ffn_gated_share_bf16(), "fp8_ffn": W.fp8_ffn_bf16(),
         "fp8_4096x1536x4096": W.fp8_quant_example()}
    for s in W.HGEMM_SHAPES:
        c = W.hgemm_colmajor(*s)
        t[c.name] = c
    for m in W.SKINNY_M:
        c = W.ffn_bf16(m)
        t["skinny_bf16_m%d" % m] = c
    return t


def algorithmic(case):
    from dense_gemm_mgemm_amd import costmodel as cm
    es = 4 if case.dtype == "f32" else 2
    if case.extra.get("gated"):     # two products sharing X; one output
        flops = 2 * cm.gemm_flops(case.M, case.N, case.K)
        return flops, es * (case.M * case.K + 2 * case.K * case.N + case.M * case.N)
    if case.extra.get("fp8"):       # quantise X (read X, write codes), then the FP8 product
        M, N, K = case.M, case.N, case.K
        return cm.gemm_flops(M, N, K), es * M * K + 2 * M * K + N * K + es * M * N
    flops = cm.gemm_flops(case.M, case.N, case.K)
    nbytes = cm.min_bytes(case.M, case.N, case.K, es) + (es * case.M * case.N if case.beta else 0)
    return flops, nbytes


def peak_key(case) -> str:
    return "fp8" if case.extra.get("fp8") else case.dtype


def is_hbm_bound(case) -> bool:
    return case.dtype != "f32" and case.M <= 64


_SLEEP_CYCLES_PER_S = None


def hold_stream(stream, seconds):
    """Keep `stream` busy for about `seconds` (at most 50 ms) with torch's
    bounded spin kernel, so that launches enqueued behind it reach the GPU
    back to back instead of at the host's enqueue pace.  The spin's rate is
    measured once."""
    import torch
    global _SLEEP_CYCLES_PER_S
    if not hasattr(torch.cuda, "_sleep"):
        return
    with torch.cuda.stream(stream):
        if _SLEEP_CYCLES_PER_S is None:
            torch.cuda._sleep(100_000)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            torch.cuda._sleep(2_000_000)
            e1.record(stream)
            torch.cuda.synchronize()
            _SLEEP_CYCLES_PER_S = 2_000_000 / max(e0.elapsed_time(e1) * 1e-3, 1e-6)
        torch.cuda._sleep(int(min(seconds, 0.05) * _SLEEP_CYCLES_PER_S))


def measure(h, case, steps, warmup, rotate=1, warm_s=0.0):
    """Time `steps` launches after `warmup` untimed ones (continued until
    `warm_s` seconds have passed, so short kernels run at a settled clock);
    returns timings, the kernel name and device buffers."""
    import torch
    import dense_gemm_mgemm_amd as mg
    from tests.parity import c_initial

    stream = torch.cuda.current_stream()
    epilogue = case.extra.get("epilogue", "none")
    if case.extra.get("fp8"):
        # One step: quantise X per row, then the FP8 product with the weights
        # (quantised once, before timing).
        A, B, C0 = case.make()
        M, N, K = case.M, case.N, case.K
        dX, dW = A.cuda(), B.cuda()
        qx = torch.empty(M * K, dtype=torch.uint8, device="cuda")
        qw = torch.empty(N * K, dtype=torch.uint8, device="cuda")
        sx = torch.empty(M, dtype=torch.float32, device="cuda")
        sw = torch.empty(N, dtype=torch.float32, device="cuda")
        mg.mgemm_quantize_fp8(h, N, K, dW, case.ldb, case.dtype, qw, K, sw, stream=stream)
        dC = [c_initial(case, None).cuda()]
        kname = "fp8_quant+fp8_gemm"

        def launch(i):
            mg.mgemm_quantize_fp8(h, M, K, dX, case.lda, case.dtype, qx, K, sx, stream=stream)
            mg.mgemm_run_fp8(h, "auto", M, N, K, case.alpha, qx, K, sx, qw, K, sw, 0.0, dC[0],
                             case.ldc, case.dtype, stream=stream)
    elif case.extra.get("gated"):
        import workloads as W
        X, Wg, Wu = W.gated_inputs(case)
        A, B, C0 = X, (Wg, Wu), None
        dX, dWg, dWu = X.cuda(), Wg.cuda(), Wu.cuda()
        dC = [c_initial(case, None).cuda()]
        kname = "h_dma_gated"

        def launch(i):
            mg.mgemm_run_gated(h, case.M, case.N, case.K, dX, case.lda, dWg, dWu, case.ldb,
                               dC[0], case.ldc, case.dtype, stream=stream)
    else:
        A, B, C0 = case.make()
        dA = [A.cuda() for _ in range(rotate)]
        dB = [B.cuda() for _ in range(rotate)]
        dC = [c_initial(case, C0).cuda() for _ in range(rotate)]
        kname, ks = mg.mgemm_select_variant(h, case.layoutA, case.layoutB, case.M, case.N,
                                            case.K, case.alpha, dA[0], case.lda, dB[0], case.ldb,
                                            case.beta, dC[0], case.ldc, case.dtype)
        if ks > 1:
            kname += "/k%d" % ks

        def launch(i):
            j = i % rotate
            if epilogue != "none":
                mg.mgemm_run_ex(h, "auto", case.layoutA, case.layoutB, case.M, case.N, case.K,
                                case.alpha, dA[j], case.lda, dB[j], case.ldb, case.beta, dC[j],
                                case.ldc, case.dtype, epilogue=epilogue, stream=stream)
                return
            mg.mgemm_run(h, case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha,
                         dA[j], case.lda, dB[j], case.ldb, case.beta, dC[j], case.ldc,
                         case.dtype, stream=stream)

    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < warm_s:
        for i in range(8):
            launch(i)
        torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t_all0, t_all1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # Host time to enqueue one step, from 16 steps.
    torch.cuda.synchronize()
    t_host = time.perf_counter()
    for i in range(16):
        launch(i)
    host_s = (time.perf_counter() - t_host) / 16
    torch.cuda.synchronize()
    # The timed region: `steps` launches back to back between two events.  A
    # kernel shorter than the host's enqueue time would otherwise be timed
    # with the GPU waiting for the host between steps, so the stream is held
    # until all of them are enqueued.  Average launch duration = region / steps.
    hold_stream(stream, 1.25 * host_s * steps + 1e-4)
    wall0 = time.perf_counter()
    t_all0.record(stream)
    for i in range(steps):
        launch(i)
    t_all1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_all0.elapsed_time(t_all1)
    # Spread of single launches, from a second pass with an event pair around
    # each (each pair adds a few microseconds of its own).
    hold_stream(stream, 1.5 * host_s * steps + 1e-4)
    for i in range(steps):
        ev[i][0].record(stream)
        launch(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in ev)
    return {
        "kernel": kname, "ms_per_step": total_ms / steps, "wall_ms_per_step": wall * 1e3 / steps,
        "host_ms_per_step": host_s * 1e3, "launch_ms_mean": total_ms / steps,
        "launch_ms_single_median": per[len(per) // 2],
        "launch_ms_p10": per[len(per) // 10], "launch_ms_p90": per[(len(per) * 9) // 10],
        "inputs": (A, B, C0), "out": dC[(steps - 1) % len(dC)],
    }


def measure_mix(h, steps=20):
    """The FFN projection X[M x 4096] W[4096 x 12288] (BF16) over the row mix
    of one group of ten calls: eight of 256 rows, one of 1536, one of 2048
    ("Chapter 5: Operators and Runtime", section 5.5.3, Example 5-12).  Times
    a group with the built-in model's choices, then with a dispatch table
    tuned on the three shapes weighted 8:1:1 (a second handle)."""
    import torch
    import dense_gemm_mgemm_amd as mg
    from workloads import operand
    K, N = 4096, 12288
    rows = [256] * 8 + [1536, 2048]
    X = operand("normal", 4201, max(rows), K, "row", K, "bf16").cuda()
    Wt = operand("normal", 4202, K, N, "row", N, "bf16", 0.02).cuda()
    C = torch.empty(max(rows) * N, dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()

    def group(hh):
        for m in rows:
            mg.mgemm_run(hh, "row", "row", m, N, K, 1.0, X, K, Wt, N, 0.0, C, N, "bf16",
                         stream=stream)

    def timed(hh):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < 0.25:
            group(hh)
            torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t1 = time.perf_counter()
        group(hh)
        host_s = time.perf_counter() - t1
        torch.cuda.synchronize()
        hold_stream(stream, 1.25 * host_s * steps + 1e-4)
        e0.record(stream)
        for _ in range(steps):
            group(hh)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    flops = sum(2.0 * m * N * K for m in rows)
    choice = lambda hh, m: "%s/k%d" % mg.mgemm_select_variant(hh, "row", "row", m, N, K, 1.0, X, K,
                                                              Wt, N, 0.0, C, N, "bf16")
    model_ms = timed(h)
    ht = mg.mgemm_create()
    try:
        t0 = time.perf_counter()
        mg.mgemm_tune(ht, "bf16", "row", "row", [(256, N, K), (1536, N, K), (2048, N, K)], [8, 1, 1])
        tune_s = time.perf_counter() - t0
        tuned_ms = timed(ht)
        picks = {m: (choice(h, m), choice(ht, m)) for m in (256, 1536, 2048)}
    finally:
        mg.mgemm_destroy(ht)
    return {"rows_per_group": rows, "model_ms_per_group": round(model_ms, 5),
            "tuned_ms_per_group": round(tuned_ms, 5), "tune_s": round(tune_s, 2),
            "model_TFLOPs": round(flops / model_ms / 1e9, 1),
            "tuned_TFLOPs": round(flops / tuned_ms / 1e9, 1),
            "choices_model_vs_tuned": {str(k): v for k, v in picks.items()}}


def cpu_baseline(case, out_dev, budget_s):
    """Time the oracle on a bounded row sample of the workload and check that
    sample against the GPU output."""
    import numpy as np
    import oracle
    from tests import parity as P
    from workloads import storage_view

    A, B, C0 = case.inputs
    if case.extra.get("fp8"):
        return cpu_baseline_fp8(case, out_dev, budget_s)
    gated = bool(case.extra.get("gated"))
    a = storage_view(A)
    bs = [storage_view(x) for x in (B if gated else (B,))]
    c0 = None if C0 is None else storage_view(C0)
    threads = oracle.max_threads()
    nrows = max(1, min(case.M, 16))
    rng = np.random.default_rng(0)
    rows_done, t_total, results = [], 0.0, []
    while True:
        rows = np.sort(rng.choice(case.M, size=nrows, replace=False)) if nrows < case.M \
            else np.arange(case.M)
        t0 = time.perf_counter()
        exact = [oracle.gemm(case.layoutA, case.layoutB, case.M, case.N, case.K, case.alpha, a,
                             case.lda, b, case.ldb, case.beta, c0, None, case.ldc, case.dtype,
                             rows=rows, nthreads=threads) for b in bs]
        if gated:
            exact.append(oracle.swiglu(case.dtype, exact[0], exact[1]))
        dt = time.perf_counter() - t0
        t_total, rows_done, results = dt, rows, exact
        if nrows >= case.M or dt * 2 > budget_s:
            break
        nrows = int(min(case.M, max(nrows * 2, nrows * budget_s / max(dt, 1e-3) * 0.8)))
    flops = 2.0 * len(rows_done) * case.N * case.K * len(bs)
    if gated:
        try:
            err = P.check_gated(case, A, B[0], B[1], out_dev.cpu(), rows=rows_done)
            rep = {"ok": True, "max_err": err, "tol": None}
        except AssertionError as e:
            rep = {"ok": False, "max_err": None, "tol": None, "what": str(e)[:200]}
    else:
        got = P.logical(case, oracle.decode(case.dtype, storage_view(out_dev.cpu())))[rows_done]
        if case.extra.get("epilogue") == "silu":
            y, bound = P.silu_reference(case, results[0])
            err = np.abs(got - y)
            rep = {"ok": bool(np.all(err <= bound)), "max_err": float(np.max(err)),
                   "tol": float(np.max(bound))}
        else:
            rep = P.compare(case, got, results[0])
    return ({"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": threads,
             "kind": "oracle", "sample": "%d of %d rows of C (%.1f GFLOP in %.1f s, FP64)" % (
                 len(rows_done), case.M, flops / 1e9, t_total)},
            {"rows": len(rows_done), "max_err": rep["max_err"], "tol": rep["tol"],
             "ok": rep["ok"]})


def cpu_baseline_fp8(case, out_dev, budget_s):
    """The FP8 oracle on a row sample: quantise the sampled rows of X, multiply
    by the weight codes (quantised once, not timed, like the GPU's), and check
    the sample against the GPU output within the FP32-accumulation bound."""
    import numpy as np
    import oracle
    from oracle import fp8 as f8
    from tests import parity as P
    from workloads import storage_view

    A, B, _ = case.inputs
    M, N, K = case.M, case.N, case.K
    X = oracle.decode(case.dtype, storage_view(A)).reshape(M, case.lda)[:, :K]
    Wv = oracle.decode(case.dtype, storage_view(B)).reshape(N, case.ldb)[:, :K]
    qw, sw = f8.quantize_rows(Wv)
    rng = np.random.default_rng(0)
    nrows = max(1, min(M, 8))
    while True:
        rows = np.sort(rng.choice(M, size=nrows, replace=False)) if nrows < M else np.arange(M)
        t0 = time.perf_counter()
        qx, sx = f8.quantize_rows(X[rows])
        exact = f8.fp8_gemm(len(rows), N, K, case.alpha, qx.ravel(), K, sx, qw.ravel(), K, sw)
        dt = time.perf_counter() - t0
        if nrows >= M or dt * 2 > budget_s:
            break
        nrows = int(min(M, max(nrows * 2, nrows * budget_s / max(dt, 1e-3) * 0.8)))
    got = oracle.decode(case.dtype, storage_view(out_dev.cpu())).reshape(-1, case.ldc)[rows, :N]
    tol = P.tol_f32_rel(K) * float(np.max(np.abs(exact))) + \
        P._ulp(case.dtype, oracle.round_to(case.dtype, exact)) / 2
    err = np.abs(got - exact)
    flops = 2.0 * len(rows) * N * K
    try:                                  # threads of numpy's BLAS (the matmul step)
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:                     # threadpoolctl missing or unreadable
        cores = 1
    return ({"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
             "sample": "%d of %d rows of C: FP8 quantisation + product (%.1f GFLOP in %.1f s, "
                       "numpy FP64)" % (len(rows), M, flops / 1e9, dt)},
            {"rows": len(rows), "max_err": float(np.max(err)), "tol": float(np.max(tol)),
             "ok": bool(np.all(err <= tol))})


def counters_for(kernel, workload):
    """The committed rocprofv3 counter summary of this kernel and workload, if
    it was taken on the current kernel sources, else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        e = json.load(open(p)).get("%s/%s" % (kernel, workload))
        if e and e.get("src_hash") == src_hash(kernel):
            return e
    except ValueError:
        pass
    return None


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed counter summary (or None)."""
    e = counters_for(kernel, workload)
    return e.get("bytes_per_launch") if e else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="sgemm_4096")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-headline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_gemm_mgemm_amd as mg
    from dense_gemm_mgemm_amd import costmodel as cm

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    h = mg.mgemm_create()
    table = workload_table()
    case = table[args.workload]
    flops, nbytes = algorithmic(case)
    hbm = is_hbm_bound(case)
    log("headline:", case.name)
    r = measure(h, case, args.steps, args.warmup, rotate=4 if hbm else 1)
    case.inputs = r["inputs"]

    if args.copy_probe:
        n = args.copy_probe * 2 ** 20 // 4
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copy probe: %d MiB x3" % args.copy_probe)

    per_launch_s = r["launch_ms_mean"] * 1e-3
    if hbm:
        achieved, peak, unit, bound = nbytes / per_launch_s / 1e9, cm.PEAK_HBM_GBS, "GB/s", "hbm"
        value, vunit = nbytes / (r["ms_per_step"] * 1e-3) / 1e9, "GB/s"
    else:
        achieved, peak = flops / per_launch_s / 1e12, cm.PEAK_TFLOPS[peak_key(case)]
        unit, bound = "TFLOP/s", "mfma"
        value, vunit = flops / (r["ms_per_step"] * 1e-3) / 1e12, "TFLOP/s"
    traffic = traffic_for(r["kernel"], case.name)
    line = {
        "metric": METRIC, "value": round(value, 3), "unit": vunit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak",
        "vs_baseline": (round(value / PAGES_SGEMM_4096_TFLOPS, 3)
                        if case.name == "sgemm_4096" else None),
        "dtype": case.dtype, "data": "synthetic",
        "config": {"workload": case.name, "M": case.M, "N": case.N, "K": case.K,
                   "layoutA": case.layoutA, "layoutB": case.layoutB, "lda": case.lda,
                   "ldb": case.ldb, "ldc": case.ldc, "alpha": case.alpha, "beta": case.beta,
                   "kernel": r["kernel"], "inputs": "%s/%s seeds %s" % (case.kindA, case.kindB,
                                                                        list(case.seeds[:2])),
                   "vs_baseline_ref": "cuBLAS pure-FP32 4096^3 on RTX 4090 from the pages, "
                                      "57.24 TFLOP/s (another machine: context only)"
                   if case.name == "sgemm_4096" else None},
        "roofline": {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "mfma_busy": (counters_for(r["kernel"], case.name) or {}).get("mfma_busy"),
                     "algorithmic_per_launch": flops if not hbm else nbytes,
                     "launch_ms_mean": round(r["launch_ms_mean"], 5),
                     "single_launch_ms_p10": round(r["launch_ms_p10"], 5),
                     "single_launch_ms_p90": round(r["launch_ms_p90"], 5)},
        "cpu_baseline": None,
        "src_hash": src_hash(),
    }
    if not args.no_cpu_baseline:
        cb, chk = cpu_baseline(case, r["out"], args.cpu_budget)
        line["cpu_baseline"] = cb
        line["parity_sample"] = chk
        if not chk["ok"]:
            log("PARITY FAILURE on the sampled rows:", chk)
    if not args.only_headline:
        others = {}
        for name, c in table.items():
            if name == case.name:
                continue
            f2, b2 = algorithmic(c)
            hb = is_hbm_bound(c)
            log("workload:", name)
            rr = measure(h, c, 20, 5, rotate=4 if hb else 1, warm_s=0.25)
            s = rr["launch_ms_mean"] * 1e-3
            ent = {"kernel": rr["kernel"], "launch_ms_mean": round(rr["launch_ms_mean"], 5),
                   "dtype": c.dtype}
            if hb:
                ent.update(GBs=round(b2 / s / 1e9, 1), frac_hbm=round(b2 / s / 1e9 / cm.PEAK_HBM_GBS, 4))
            else:
                tf = f2 / s / 1e12
                ent.update(TFLOPs=round(tf, 2), frac_peak=round(tf / cm.PEAK_TFLOPS[peak_key(c)], 4))
            cnt = counters_for(rr["kernel"], name)
            if cnt:
                ent.update(traffic=cnt.get("bytes_per_launch"), mfma_busy=cnt.get("mfma_busy"))
            others[name] = ent
            del rr
            torch.cuda.empty_cache()
        log("workload: ffn_mix_bf16 (model vs tuned table)")
        others["ffn_mix_bf16"] = measure_mix(h)
        line["workloads"] = others
    mg.mgemm_destroy(h)
    print(json.dumps(line), flush=True)
    if line.get("parity_sample") and not line["parity_sample"]["ok"]:
        sys.exit(1)


if __name__ == "__main__":
    main()
