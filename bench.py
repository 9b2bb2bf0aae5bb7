#!/usr/bin/env python3
"""Benchmark of the tiled mixed-precision GEMM / W8A8 GEMV library on one
MI355X.

A step is one call of the headline workload, the BF16 GEMM D = A . B + C at
M = N = K = 4096 (row-major, FP32 C and D), on inputs already resident in
HBM.  The other workloads of the suite (W8A8 batch-1 GEMV 1 x 4096 . 4096 x
14336 with a cold cache, FP8 block-scaled 4096 x 7168 x 7168, ragged FP16
8191 x 8193 x 4099, FP16 64^3, INT8 4096^3) are timed the same way and
reported under "extra", each with its own roofline figure, as are the next
steps around them: BF16 4096^3 with a BF16 D, the W8A8 layer for 4 and 16
tokens, and the INT8 / FP8 quantisers.

Prints ONE JSON line.  Kernel durations come from HIP events recorded on the
stream the kernels run on (torch's current stream).
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2500.0      # TFLOP/s, dense
PEAK_FP16 = 2500.0
PEAK_FP8 = 5000.0
PEAK_INT8 = 5000.0      # TOP/s
PEAK_HBM = 8000.0       # GB/s

METRIC = "TFLOP/s & % MFMA peak (BF16 4096³); GB/s & % HBM peak (W8A8 GEMV)"
GEMM_SOURCES = ("gemm.hip", "gemm_kernel.hpp", "gemm_common.hpp", "device_common.hpp")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # The part needs about 40 ms of sustained load after idle before its
    # clocks settle: the first ~300 launches of the BF16 GEMM run up to 15 %
    # slower than the rest.  The default warm-up covers that.
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--only", default="all",
                   choices=["all", "bf16", "bf16out", "epi", "gemv", "w8a8_tokens", "quant", "fp8",
                            "f16_ragged", "f16_64", "i8", "copy", "ceiling", "bf16+gemv"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--procs", type=int, default=3,
                   help="independent processes that repeat the headline BF16 GEMM and the cold "
                        "GEMV, for the median [min, max] across processes (1: none)")
    p.add_argument("--child", action="store_true", help=argparse.SUPPRESS)
    p.add_argument("--no-clock", action="store_true",
                   help="skip the clock-stamped run of the headline GEMM")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the bounded oracle sample")
    return p.parse_args()


def source_digest(*names) -> str:
    """Digest of the listed kernel sources with comments and blank lines
    removed (counters describe the code, so comment edits keep them valid)."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "mixed_precision_dense_tiled_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
        h.update("\n".join(lines).encode())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, digest: str, per_launch_units: float = 1.0):
    """Counter-measured HBM bytes per launch from profiles/traffic.json, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(kernel)
    if not e or e.get("source_digest") != digest:
        return None
    return e.get("bytes_per_launch")


def timed(fn, steps, warmup, stream):
    """warmup untimed calls, then `steps` back-to-back calls bracketed by HIP
    events on the stream the kernels run on.  Returns (region_ms, per_launch_ms):
    the average launch duration is region_ms / steps; per_launch_ms comes
    from a separate, untimed pass with an event pair around each launch (its
    spread only: the extra events there slow the launches down)."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for i in range(steps):
        fn(warmup + i)
    r1.record(stream)
    torch.cuda.synchronize()
    region = r0.elapsed_time(r1)
    n = min(steps, 20)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    for i in range(n):
        ev[i][0].record(stream)
        fn(warmup + steps + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return region, [a.elapsed_time(b) for a, b in ev]


def timed_graph(fn, period, reps, warmup, stream, before_replay=None):
    """The calls fn(0) .. fn(period - 1) (one rotation over the rotating
    inputs) captured once into a HIP graph, which is replayed `warmup` times
    untimed and then `reps` times between two HIP events: the kernels run
    back to back at the GPU's own pace, with no host launch cost between
    them (a short kernel launched one call at a time from Python waits on
    the host).  Returns (region_ms, steps = reps * period)."""
    import torch
    for i in range(period):                 # eager calls first (lazy set-up outside the capture)
        fn(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(period):
            fn(i)
    if before_replay is not None:           # (e.g. clear the outputs, so a check after
        before_replay()                     #  the replays sees only what they wrote)
        torch.cuda.synchronize()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    r0.record(stream)
    for _ in range(reps):
        g.replay()
    r1.record(stream)
    torch.cuda.synchronize()
    return r0.elapsed_time(r1), reps * period


def stats(per, region_ms=None, steps=None):
    s = sorted(per)
    n = len(s)
    out = {"median_us_eventpair": 1e3 * s[n // 2], "min_us_eventpair": 1e3 * s[0],
           "max_us_eventpair": 1e3 * s[-1]}
    if region_ms is not None:
        out = {"mean_us": 1e3 * region_ms / steps, **out}
    return out


def note(msg):
    """One progress line on stderr per finished section (stdout keeps the
    single JSON line)."""
    print(f"# bench: section {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import numpy as np

    def want(name):
        return args.only == "all" or args.only == name or (args.only == "bf16+gemv" and name in ("bf16", "gemv"))

    # Independent processes first, before this one touches the GPU: each
    # repeats the headline GEMM and the cold GEMV in a fresh process (own
    # context, own clock ramp); their spread is reported with the median.
    spread = None
    if not args.child and args.procs > 1 and want("bf16"):
        spread = process_spread(args)

    import torch

    import mixed_precision_dense_tiled_amd as mp
    from mixed_precision_dense_tiled_amd import inputs

    if not os.path.exists(mp.lib_path()):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def to_dev(x):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            x = x.view(np.int16)
        return torch.from_numpy(x).to(dev)

    extra = {}
    result = None

    note("headline: BF16 4096^3")
    # ---------------- headline: BF16 4096^3 -----------------------------------
    if want("bf16"):
        M = N = K = 4096
        A, B, C = inputs.gemm16_operands(M, N, K, dist="normal", fmt="bf16")
        tA, tB, tC = to_dev(A), to_dev(B), to_dev(C)
        tD = torch.empty((M, N), dtype=torch.float32, device=dev)
        region, per = timed(lambda i: mp.gemm_bf16(tA, tB, tC, out=tD), args.steps, args.warmup,
                            stream)
        st = stats(per, region, args.steps)
        flop = 2.0 * M * N * K
        avg_s = st["mean_us"] * 1e-6
        achieved = flop / avg_s / 1e12
        traffic = traffic_for("gemm_bf16_4096", source_digest(*GEMM_SOURCES))
        clock = None if (args.no_clock or args.child) else gemm_clock(tA, tB, tC, tD, stream, M, N, K)
        smi = None if args.child else smi_clocks(lambda: mp.gemm_bf16(tA, tB, tC, out=tD), stream)
        result = {
            "metric": METRIC,
            "value": flop * args.steps / (region * 1e-3) / 1e12,
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": args.warmup,
            "ms_per_step": region / args.steps,
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": "bf16",
            "data": "synthetic",
            "config": {"workload": "gemm_bf16 D=A*B+C, M=N=K=4096, row-major, A,B~N(0,1) as BF16, "
                                   "C~N(0,1) FP32, FP32 accumulate and output",
                       "M": M, "N": N, "K": K, "parallelism": "single GPU"},
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16,
                         "unit": "TFLOP/s", "frac": achieved / PEAK_BF16, "traffic": traffic,
                         "kernel": "gemm_kernel<BF16,256x256,one wave per SIMD>", "launch_us": st,
                         "clock": clock},
        }
        if smi is not None:
            result["smi_clocks_under_load"] = smi
        if not args.child:
            ceil = optional(mfma_ceiling, args, stream, inputs, "bf16")
            result["roofline"]["mfma_ceiling"] = ceil
            if "TFLOP_s" in ceil:
                result["roofline"]["frac_of_mfma_ceiling"] = achieved / ceil["TFLOP_s"]
        if spread is not None:
            result["process_spread"] = spread["bf16"]
        if not args.no_cpu_baseline and not args.child:
            result["cpu_baseline"] = cpu_baseline_gemm16(A, B, C, "bf16", args.cpu_seconds)
        del tA, tB, tC, tD

    note("BF16 4096^3 with a BF16 D (16-bit-output variant)")
    # ---------------- BF16 4096^3 with a BF16 D (16-bit-output variant) -------
    if want("bf16out"):
        M = N = K = 4096
        A, B, C = inputs.gemm16_operands(M, N, K, dist="normal", fmt="bf16")
        tA, tB, tC = to_dev(A), to_dev(B), to_dev(C)
        tD = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        region, per = timed(lambda i: mp.gemm_bf16_bf16out(tA, tB, tC, out=tD), args.steps,
                            args.warmup, stream)
        st = stats(per, region, args.steps)
        tf = 2.0 * M * N * K / (st["mean_us"] * 1e-6) / 1e12
        extra["gemm_bf16_bf16out"] = {
            "workload": "gemm_bf16_bf16out D=bf16(A*B+C), M=N=K=4096, FP32 C, BF16 D",
            "TFLOP_s": tf, "launch_us": st,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16, "unit": "TFLOP/s",
                         "frac": tf / PEAK_BF16}}
        del tA, tB, tC, tD

    note("BF16 4096^3 + bias + GELU into BF16 (fused epilogue)")
    # ---------------- BF16 4096^3 + bias + GELU into BF16 (fused epilogue) ------
    if want("epi"):
        M = N = K = 4096
        A, B, C = inputs.gemm16_operands(M, N, K, dist="normal", fmt="bf16")
        bias = inputs.normal_f32((N,), inputs.SEED_BIAS)
        tA, tB, tC, tb = to_dev(A), to_dev(B), to_dev(C), to_dev(bias)
        tD = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        region, per = timed(lambda i: mp.gemm_bf16_bias_act(tA, tB, tC, tb, mp.ACT_GELU, out=tD),
                            args.steps, args.warmup, stream)
        st = stats(per, region, args.steps)
        tf = 2.0 * M * N * K / (st["mean_us"] * 1e-6) / 1e12
        extra["gemm_bf16_bias_gelu_bf16out"] = {
            "workload": "gemm_bf16_bias_act D=bf16(GELU(A*B+C+bias)), M=N=K=4096, FP32 C and "
                        "bias, BF16 D",
            "TFLOP_s": tf, "launch_us": st,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_BF16, "unit": "TFLOP/s",
                         "frac": tf / PEAK_BF16}}
        del tA, tB, tC, tb, tD

    note("practical HBM read ceiling")
    # ---------------- practical HBM read ceiling ------------------------------
    ceiling = None
    if (want("gemv") or want("ceiling")) and not args.child:
        ceiling = optional(read_ceiling, args, stream)
        extra["hbm_read_ceiling"] = ceiling

    note("W8A8 GEMV, cold cache")
    # ---------------- W8A8 GEMV, cold cache ------------------------------------
    if want("gemv"):
        N, K = 14336, 4096
        x, s_x, W, s_w = inputs.w8a8_operands(N, K)
        copies = 8  # 8 x 58.7 MB rotated: larger than the 256 MB Infinity Cache
        tWs = [to_dev(W) for _ in range(copies)]
        tx, tsw = to_dev(x), to_dev(s_w)
        ty = torch.empty(N, dtype=torch.bfloat16, device=dev)
        region, per = timed(lambda i: mp.gemv_w8a8(tx, float(s_x), tWs[i % copies], tsw, out=ty),
                            args.steps, args.warmup, stream)
        y_eager = ty.clone()
        st = stats(per, region, args.steps)
        nbytes = N * K + K + 4 * N + 4 + 2 * N      # W + x + s_w + s_x + y (algorithmic)
        gbs = nbytes / (st["mean_us"] * 1e-6) / 1e9
        # the same rotation replayed from a HIP graph (no host cost between
        # launches; checked against the eager result)
        reps = max(args.steps // copies, 4)
        region_g, gsteps = timed_graph(lambda i: mp.gemv_w8a8(tx, float(s_x), tWs[i % copies], tsw, out=ty),
                                       copies, reps, max(args.warmup // copies, 8), stream,
                                       before_replay=lambda: ty.fill_(-1.0))
        assert torch.equal(ty, y_eager), "graph replays must give the eager result"
        graph_us = 1e3 * region_g / gsteps
        region_w, per_w = timed(lambda i: mp.gemv_w8a8(tx, float(s_x), tWs[0], tsw, out=ty),
                                args.steps, args.warmup, stream)
        stw = stats(per_w, region_w, args.steps)
        digest = source_digest("gemv_w8a8.hip", "device_common.hpp")
        extra["gemv_w8a8"] = {
            "workload": "batch-1 W8A8 linear, x int8 [4096], W int8 [14336 x 4096] (stored N x K), "
                        "BF16 out; cold: 8 rotating W copies",
            "GB_s": gbs, "algorithmic_bytes": nbytes, "launch_us": st,
            "timing": f"{args.steps} back-to-back launches over {copies} rotating weight copies, "
                      "between HIP events",
            "graph_replay": {"mean_us": graph_us, "GB_s": nbytes / (graph_us * 1e-6) / 1e9,
                             "launches": gsteps},
            "warm_same_W_GB_s": nbytes / (stw["mean_us"] * 1e-6) / 1e9,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM,
                         "traffic": traffic_for("gemv_w8a8_14336x4096", digest)},
        }
        if ceiling is not None and "error" not in ceiling:
            c = max(v["GB_s"] for k, v in ceiling.items() if k.startswith("same_bytes_cold"))
            extra["gemv_w8a8"]["roofline"]["calibrated_ceiling_GB_s"] = c
            extra["gemv_w8a8"]["roofline"]["frac_of_calibrated_ceiling"] = gbs / c
        if spread is not None:
            extra["gemv_w8a8"]["process_spread"] = spread["gemv"]
        if not args.no_cpu_baseline and not args.child:
            extra["gemv_w8a8"]["cpu_baseline"] = cpu_baseline_gemv(x, s_x, W, s_w, nbytes)
        del tWs

    note("W8A8 layer for a few tokens, cold cache")
    # ---------------- W8A8 layer for a few tokens, cold cache --------------------
    if want("w8a8_tokens"):
        N, K = 14336, 4096
        r = np.random.default_rng(12)
        copies = 8
        W = r.integers(-127, 128, (N, K)).astype(np.int8)
        tWs = [to_dev(W) for _ in range(copies)]
        tsw = to_dev(r.uniform(0.001, 0.01, N).astype(np.float32))
        tb = to_dev(r.standard_normal(N).astype(np.float32))
        for M in (4, 16):
            tX = to_dev(r.integers(-127, 128, (M, K)).astype(np.int8))
            tsx = to_dev(r.uniform(0.01, 0.1, M).astype(np.float32))
            ty = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            region, per = timed(lambda i: mp.gemm_w8a8(tX, tsx, tWs[i % copies], tsw, tb, out=ty),
                                args.steps, args.warmup, stream)
            st = stats(per, region, args.steps)
            nbytes = N * K + M * K + 4 * M + 8 * N + 2 * M * N
            gbs = nbytes / (st["mean_us"] * 1e-6) / 1e9
            extra[f"gemm_w8a8_m{M}"] = {
                "workload": f"W8A8 layer, {M} tokens x 4096 . W int8 [14336 x 4096], bias, BF16 out; "
                            "cold: 8 rotating W copies",
                "GB_s": gbs, "algorithmic_bytes": nbytes, "launch_us": st,
                "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM, "unit": "GB/s",
                             "frac": gbs / PEAK_HBM,
                             "traffic": traffic_for("gemm_w8a8_stream_16x14336x4096",
                                                    source_digest("gemv_w8a8.hip", "device_common.hpp"))
                             if M == 16 else None}}
            if M == 16:
                # the same layer with the weights stored K x N
                tWkn = [tW.t().contiguous() for tW in tWs[:4]]
                region, per = timed(lambda i: mp.gemm_w8a8_kn(tX, tsx, tWkn[i % 4], tsw, tb, out=ty),
                                    args.steps, args.warmup, stream)
                st = stats(per, region, args.steps)
                gbs = nbytes / (st["mean_us"] * 1e-6) / 1e9
                extra["gemm_w8a8_kn_m16"] = {
                    "workload": "W8A8 layer, 16 tokens x 4096 . W int8 stored K x N [4096 x 14336], bias, "
                                "BF16 out; cold: 4 rotating W copies",
                    "GB_s": gbs, "algorithmic_bytes": nbytes, "launch_us": st,
                    "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM, "unit": "GB/s",
                                 "frac": gbs / PEAK_HBM}}
                del tWkn
                # the same layer requantised to INT8 for a next INT8 layer
                tq = torch.empty((M, N), dtype=torch.int8, device=dev)
                region, per = timed(lambda i: mp.gemm_w8a8_requant(tX, tsx, tWs[i % copies], tsw, tb,
                                                                   0.05, out=tq),
                                    args.steps, args.warmup, stream)
                st = stats(per, region, args.steps)
                nbytes = N * K + M * K + 4 * M + 8 * N + M * N
                gbs = nbytes / (st["mean_us"] * 1e-6) / 1e9
                extra["gemm_w8a8_requant_m16"] = {
                    "workload": "W8A8 layer, 16 tokens x 4096 . W int8 [14336 x 4096], bias, "
                                "requantised INT8 out; cold: 8 rotating W copies",
                    "GB_s": gbs, "algorithmic_bytes": nbytes, "launch_us": st,
                    "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM, "unit": "GB/s",
                                 "frac": gbs / PEAK_HBM}}
        del tWs

    note("quantisers")
    # ---------------- quantisers -----------------------------------------------
    if want("quant"):
        r = np.random.default_rng(13)
        X = r.standard_normal((16, 4096)).astype(np.float32)
        tX = to_dev((X.view(np.uint32) >> 16).astype(np.uint16))
        region, per = timed(lambda i: mp.quantize_i8_rows(tX), args.steps, args.warmup, stream)
        extra["quantize_i8_rows_16x4096"] = {
            "workload": "per-token INT8 quantisation of 16 BF16 tokens x 4096 (latency bound)",
            "launch_us": stats(per, region, args.steps)}
        for name, (R, Cc, br) in (("a", (4096, 7168, 1)), ("b", (7168, 7168, 128))):
            tA = torch.randn((R, Cc), device=dev)
            region, per = timed(lambda i: mp.quantize_fp8_blocks(tA, br), max(args.steps // 2, 5),
                                args.warmup, stream)
            st = stats(per, region, max(args.steps // 2, 5))
            nbytes = R * Cc * 5 + 4 * (-(-R // br)) * (-(-Cc // 128))
            gbs = nbytes / (st["mean_us"] * 1e-6) / 1e9
            extra[f"quantize_fp8_blocks_{name}"] = {
                "workload": f"FP8 E4M3 block quantisation of FP32 {R} x {Cc} in {br} x 128 blocks "
                            "(the FP8 GEMM workload's operand)",
                "GB_s": gbs, "algorithmic_bytes": nbytes, "launch_us": st,
                "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM, "unit": "GB/s",
                             "frac": gbs / PEAK_HBM}}
            del tA
        # per-tensor E5M2 (three launches: maximum, quantisation, scale)
        R, Cc = 7168, 7168
        tA = torch.randn((R, Cc), device=dev)
        tq = torch.empty((R, Cc), dtype=torch.uint8, device=dev)
        ts = torch.empty((1, 1), dtype=torch.float32, device=dev)
        region, per = timed(lambda i: mp.quantize_fp8(tA, mp.FP8_E5M2, R, Cc, q_out=tq, scales_out=ts),
                            max(args.steps // 2, 5), args.warmup, stream)
        st = stats(per, region, max(args.steps // 2, 5))
        nbytes = R * Cc * 9 + 4                          # X read twice, Q written
        gbs = nbytes / (st["mean_us"] * 1e-6) / 1e9
        extra["quantize_fp8_tensor_e5m2"] = {
            "workload": "FP8 E5M2 per-tensor quantisation of FP32 7168 x 7168 (maximum pass, then "
                        "quantisation pass)",
            "GB_s": gbs, "algorithmic_bytes": nbytes, "launch_us": st,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM}}
        del tA, tq

    note("FP8 block-scaled 4096 x 7168 x 7168")
    # ---------------- FP8 block-scaled 4096 x 7168 x 7168 ----------------------
    if want("fp8"):
        M, N, K = 4096, 7168, 7168
        qa, sa, qb, sb = inputs.fp8_operands(M, N, K)
        ta, tsa, tb, tsb = to_dev(qa), to_dev(sa), to_dev(qb), to_dev(sb)
        td = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        steps = max(args.steps // 2, 5)
        region, per = timed(lambda i: mp.gemm_fp8_blockscaled(ta, tsa, tb, tsb, out=td), steps,
                            args.warmup, stream)
        st = stats(per, region, steps)
        tf = 2.0 * M * N * K / (st["mean_us"] * 1e-6) / 1e12
        extra["gemm_fp8_blockscaled"] = {
            "workload": "FP8 E4M3 4096x7168x7168, 1x128 A / 128x128 B FP32 scales, BF16 out",
            "TFLOP_s": tf, "launch_us": st,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP8, "unit": "TFLOP/s",
                         "frac": tf / PEAK_FP8}}
        if not args.child:
            ceil = optional(mfma_ceiling, args, stream, inputs, "fp8")
            extra["gemm_fp8_blockscaled"]["roofline"]["mfma_ceiling"] = ceil
            if "TFLOP_s" in ceil:
                extra["gemm_fp8_blockscaled"]["roofline"]["frac_of_mfma_ceiling"] = tf / ceil["TFLOP_s"]
        if not args.no_cpu_baseline and not args.child:
            extra["gemm_fp8_blockscaled"]["cpu_baseline"] = cpu_baseline_fp8(qa, sa, qb, sb, args.cpu_seconds / 3)
        # the same operands with B read as E5M2 codes (the format of gradients)
        qb5 = qb.copy()
        qb5[(qb5 & 0x7C) == 0x7C] = 0x3C                   # no infinity / NaN codes
        tb5 = to_dev(qb5)
        region, per = timed(lambda i: mp.gemm_fp8_blockscaled_fmt(ta, mp.FP8_E4M3, tsa, tb5, mp.FP8_E5M2,
                                                                  tsb, out=td),
                            steps, args.warmup, stream)
        st = stats(per, region, steps)
        tf = 2.0 * M * N * K / (st["mean_us"] * 1e-6) / 1e12
        extra["gemm_fp8_blockscaled_e4m3_e5m2"] = {
            "workload": "FP8 E4M3 A x E5M2 B 4096x7168x7168, 1x128 A / 128x128 B FP32 scales, BF16 out",
            "TFLOP_s": tf, "launch_us": st,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP8, "unit": "TFLOP/s",
                         "frac": tf / PEAK_FP8}}
        # one scale per row of A and per column of B
        r = np.random.default_rng(14)
        tra = to_dev(r.uniform(0.5, 2, M).astype(np.float32))
        trb = to_dev(r.uniform(0.5, 2, N).astype(np.float32))
        region, per = timed(lambda i: mp.gemm_fp8_rowscaled(ta, mp.FP8_E4M3, tra, tb, mp.FP8_E4M3, trb,
                                                            out=td),
                            steps, args.warmup, stream)
        st = stats(per, region, steps)
        tf = 2.0 * M * N * K / (st["mean_us"] * 1e-6) / 1e12
        extra["gemm_fp8_rowscaled"] = {
            "workload": "FP8 E4M3 4096x7168x7168, per-row A and per-column B FP32 scales, BF16 out",
            "TFLOP_s": tf, "launch_us": st,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP8, "unit": "TFLOP/s",
                         "frac": tf / PEAK_FP8}}
        del ta, tb, td, tb5

    note("FP16 ragged 8191 x 8193 x 4099")
    # ---------------- FP16 ragged 8191 x 8193 x 4099 ---------------------------
    if want("f16_ragged"):
        M, N, K = 8191, 8193, 4099
        A, B, C = inputs.gemm16_operands(M, N, K, dist="uniform", fmt="f16", c_zero=True)
        tA, tB, tC = to_dev(A), to_dev(B), to_dev(C)
        tD = torch.empty((M, N), dtype=torch.float32, device=dev)
        steps = max(args.steps // 4, 5)
        region, per = timed(lambda i: mp.gemm_f16(tA, tB, tC, out=tD), steps, args.warmup, stream)
        st = stats(per, region, steps)
        tf = 2.0 * M * N * K / (st["mean_us"] * 1e-6) / 1e12
        extra["gemm_f16_ragged"] = {
            "workload": "FP16 8191x8193x4099 tight leading dims, C=0, FP32 out",
            "TFLOP_s": tf, "launch_us": st,
            "roofline": {"bound": "mfma", "achieved": tf, "peak": PEAK_FP16, "unit": "TFLOP/s",
                         "frac": tf / PEAK_FP16,
                         "traffic": traffic_for("gemm_f16_ragged", source_digest(*GEMM_SOURCES))}}
        if not args.no_cpu_baseline and not args.child:
            extra["gemm_f16_ragged"]["cpu_baseline"] = cpu_baseline_gemm16(A, B, C, "f16", args.cpu_seconds / 3)
        del tA, tB, tC, tD
        if not args.child:
            # the same tiles and rounds with aligned rows (8192 x 8192 x 4096):
            # what the tight, 2-byte-aligned leading dimensions cost
            Aa, Ba, Ca = inputs.gemm16_operands(8192, 8192, 4096, dist="uniform", fmt="f16", c_zero=True)
            tA, tB, tC = to_dev(Aa), to_dev(Ba), to_dev(Ca)
            tD = torch.empty((8192, 8192), dtype=torch.float32, device=dev)
            region, per = timed(lambda i: mp.gemm_f16(tA, tB, tC, out=tD), steps, args.warmup, stream)
            sta = stats(per, region, steps)
            extra["gemm_f16_ragged"]["aligned_8192x8192x4096_same_tiles"] = {
                "launch_us": sta, "TFLOP_s": 2.0 * 8192 * 8192 * 4096 / (sta["mean_us"] * 1e-6) / 1e12}
            del tA, tB, tC, tD

    note("FP16 64^3 (latency)")
    # ---------------- FP16 64^3 (latency) --------------------------------------
    if want("f16_64"):
        A, B, C = inputs.gemm16_operands(64, 64, 64, dist="uniform", fmt="f16")
        tA, tB, tC = to_dev(A), to_dev(B), to_dev(C)
        tD = torch.empty((64, 64), dtype=torch.float32, device=dev)
        region, per = timed(lambda i: mp.gemm_f16(tA, tB, tC, out=tD), args.steps, args.warmup,
                            stream)
        extra["gemm_f16_64"] = {"workload": "FP16 64^3 with FP32 C (latency bound)",
                                "launch_us": stats(per, region, args.steps)}
        if not args.no_cpu_baseline and not args.child:
            extra["gemm_f16_64"]["cpu_baseline"] = cpu_baseline_small(A, B, C)

    note("INT8 4096^3")
    # ---------------- INT8 4096^3 ----------------------------------------------
    if want("i8"):
        M = N = K = 4096
        A, B, C = inputs.i8_operands(M, N, K)
        tA, tB, tC = to_dev(A), to_dev(B), to_dev(C)
        tD = torch.empty((M, N), dtype=torch.int32, device=dev)
        region, per = timed(lambda i: mp.gemm_i8_i32(tA, tB, tC, out=tD), args.steps, args.warmup,
                            stream)
        st = stats(per, region, args.steps)
        tops = 2.0 * M * N * K / (st["mean_us"] * 1e-6) / 1e12
        extra["gemm_i8_i32"] = {"workload": "INT8 4096^3, INT32 C/D", "TOP_s": tops,
                                "launch_us": st,
                                "roofline": {"bound": "mfma", "achieved": tops, "peak": PEAK_INT8,
                                             "unit": "TOP/s", "frac": tops / PEAK_INT8,
                                             "traffic": traffic_for("gemm_i8_4096", source_digest(*GEMM_SOURCES))}}
        if not args.child:
            ceil = optional(mfma_ceiling, args, stream, inputs, "i8")
            extra["gemm_i8_i32"]["roofline"]["mfma_ceiling"] = ceil
            if "TOP_s" in ceil:
                extra["gemm_i8_i32"]["roofline"]["frac_of_mfma_ceiling"] = tops / ceil["TOP_s"]
        if not args.no_cpu_baseline and not args.child:
            extra["gemm_i8_i32"]["cpu_baseline"] = cpu_baseline_i8(A, B, C, args.cpu_seconds / 3)
        del tA, tB, tC, tD

    note("plain copy (counter calibration)")
    # ---------------- plain copy (counter calibration) -------------------------
    if args.only == "copy":
        n = 256 << 20
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        region, per = timed(lambda i: dst.copy_(src), args.steps, args.warmup, stream)
        extra["copy"] = {"bytes_read": n, "bytes_written": n,
                         "launch_us": stats(per, region, args.steps)}

    if result is None:
        result = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1,
                  "steps": args.steps, "warmup": args.warmup, "only": args.only}
    result["extra"] = extra
    print(json.dumps(result), flush=True)


def gemm_clock(tA, tB, tC, tD, stream, M, N, K, runs=6):
    """Where the BF16 GEMM's time goes, read from the instrumented build of the
    same kernels (libmpdt_clock.so: per-workgroup s_memtime and s_memrealtime
    stamps at entry, after the K loop and after the last store), run
    back-to-back right after the timed region.  The workgroups of the last
    launch are those whose entry stamps lie within a millisecond of the
    latest.  Reported (medians over the last runs): the shader clock, K-loop
    and epilogue cycles per workgroup (for each half of the grid when two
    workgroups share a CU: the first half issues ahead), and the exposed
    epilogue -- from the last K loop's end to the last store, the part of the
    kernel no MFMA work overlaps.  The clock-adjusted peak scales the 2.5
    PFLOP/s spec (quoted at 2.4 GHz) to the measured clock."""
    import ctypes
    import numpy as np
    import torch
    path = os.path.join(ROOT, "mixed_precision_dense_tiled_amd", "libmpdt_clock.so")
    if not os.path.exists(path):
        return None
    L = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    L.gemm_bf16.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, vp, i64, vp]
    L.gemm_bf16.restype = ctypes.c_int
    L.mpdt_clock_stamps.argtypes = [vp, ctypes.c_int]
    L.mpdt_clock_stamps.restype = ctypes.c_int
    cap = 4096
    buf = np.zeros(cap * 6, dtype=np.uint64)
    rec = {k: [] for k in ("clk", "loop", "epi", "loop_a", "epi_a", "loop_b", "epi_b", "span", "exposed", "wgs")}
    for r in range(runs):
        rc = L.gemm_bf16(M, N, K, tA.data_ptr(), K, tB.data_ptr(), N, tC.data_ptr(), N,
                         tD.data_ptr(), N, stream.cuda_stream)
        torch.cuda.synchronize()
        if rc != 0 or L.mpdt_clock_stamps(buf.ctypes.data, cap) != 0:
            return None
        if r < runs // 2:
            continue
        q = buf.reshape(cap, 6).astype(np.float64)
        live = q[:, 3] >= q[:, 3].max() - 100e3          # entry within 1 ms of the latest
        wgs = int(live.sum())
        q = q[:wgs] if live[:wgs].all() else q[live]
        real_s = (q[:, 5] - q[:, 3]) / 100e6
        ghz = np.median((q[:, 2] - q[:, 0]) / real_s) / 1e9
        rec["clk"].append(ghz)
        rec["loop"].append(np.median(q[:, 1] - q[:, 0]))
        rec["epi"].append(np.median(q[:, 2] - q[:, 1]))
        h = wgs // 2
        rec["loop_a"].append(np.median(q[:h, 1] - q[:h, 0]))
        rec["epi_a"].append(np.median(q[:h, 2] - q[:h, 1]))
        rec["loop_b"].append(np.median(q[h:, 1] - q[h:, 0]))
        rec["epi_b"].append(np.median(q[h:, 2] - q[h:, 1]))
        rec["span"].append((q[:, 5].max() - q[:, 3].min()) / 100e6 * 1e6)
        rec["exposed"].append((q[:, 5].max() - q[:, 4].max()) / 100e6 * ghz * 1e9)
        rec["wgs"].append(wgs)
    med = {k: float(np.median(v)) for k, v in rec.items()}
    wgs = int(med["wgs"])
    out = {"shader_clock_ghz": med["clk"], "workgroups": wgs,
           "k_loop_cycles": med["loop"], "epilogue_cycles": med["epi"],
           "kernel_span_us": med["span"], "exposed_epilogue_cycles": med["exposed"],
           # MFMA-bound work: 2MNK FLOP at 1024 FLOP per clock and SIMD
           "mfma_cycles_per_simd": 2.0 * M * N * K / 1024.0 / (256 * 4),
           "k_loop_cycles_mfma_bound_per_workgroup": 2.0 * M * N * K / 1024.0 / (wgs * 4),
           "clock_adjusted_peak_tflops": PEAK_BF16 * med["clk"] / 2.4,
           "source": "libmpdt_clock.so (same kernels + s_memtime/s_memrealtime stamps)"}
    if wgs > 256:
        out["first_half"] = {"k_loop_cycles": med["loop_a"], "epilogue_cycles": med["epi_a"]}
        out["second_half"] = {"k_loop_cycles": med["loop_b"], "epilogue_cycles": med["epi_b"]}
    return out


def cpu_info():
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return int(os.environ["OMP_NUM_THREADS"]), model


def _grow_rows(run, total_rows, target_s):
    """Time run(rows) on a growing leading block of rows until it takes
    about target_s (or covers every row); returns (rows, seconds)."""
    rows = 8
    while True:
        t0 = time.perf_counter()
        run(rows)
        t = time.perf_counter() - t0
        if t * 2 > target_s or rows >= total_rows:
            return rows, t
        rows = min(total_rows, max(rows * 2, int(rows * target_s / max(t, 1e-3) * 0.9)))


def cpu_baseline_gemm16(A, B, C, fmt, target_s):
    """The CPU oracle (FP64 GEMM + bound matrix, OpenMP) timed on a leading
    block of rows of a 16-bit workload; TFLOP/s of that block (2 FLOP per
    multiply-add)."""
    cores, model = cpu_info()
    import oracle
    fn = oracle.gemm_bf16 if fmt == "bf16" else oracle.gemm_f16
    M, K = A.shape
    N = B.shape[1]
    rows, t = _grow_rows(lambda r: fn(A[:r], B, C[:r]), M, target_s)
    return {"value": 2.0 * rows * N * K / t / 1e12, "unit": "TFLOP/s", "cores": cores, "cpu": model,
            "kind": "oracle",
            "sample": f"oracle_gemm_{fmt} (FP64 sum and bound matrix) on the first {rows} of {M} rows of A "
                      f"(all {N} columns, K = {K}), {t:.2f} s wall"}


def cpu_baseline_i8(A, B, C, target_s):
    cores, model = cpu_info()
    import oracle
    M, K = A.shape
    N = B.shape[1]
    rows, t = _grow_rows(lambda r: oracle.gemm_i8_i32(A[:r], B, C[:r]), M, target_s)
    return {"value": 2.0 * rows * N * K / t / 1e12, "unit": "TOP/s", "cores": cores, "cpu": model,
            "kind": "oracle",
            "sample": f"oracle_gemm_i8_i32 (INT64 sums) on the first {rows} of {M} rows of A "
                      f"(all {N} columns, K = {K}), {t:.2f} s wall"}


def cpu_baseline_fp8(qa, sa, qb, sb, target_s):
    cores, model = cpu_info()
    import oracle
    M, K = qa.shape
    N = qb.shape[1]
    rows, t = _grow_rows(lambda r: oracle.gemm_fp8_blockscaled(qa[:r], sa[:r], qb, sb), M, target_s)
    return {"value": 2.0 * rows * N * K / t / 1e12, "unit": "TFLOP/s", "cores": cores, "cpu": model,
            "kind": "oracle",
            "sample": f"oracle_gemm_fp8_blockscaled (FP64 block sums and bound matrix) on the first {rows} "
                      f"of {M} rows of A (all {N} columns, K = {K}), {t:.2f} s wall"}


def cpu_baseline_small(A, B, C, runs=5):
    """The whole 64^3 problem, median of five runs (it is latency-bound)."""
    cores, model = cpu_info()
    import oracle
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle.gemm_f16(A, B, C)
        ts.append(time.perf_counter() - t0)
    t = sorted(ts)[runs // 2]
    M, K = A.shape
    N = B.shape[1]
    return {"value": t * 1e6, "unit": "us per call", "gflop_s": 2.0 * M * N * K / t / 1e9, "cores": cores,
            "cpu": model, "kind": "oracle",
            "sample": f"oracle_gemm_f16 on the whole {M}x{N}x{K} problem, median of {runs} runs "
                      f"[{min(ts) * 1e6:.0f}, {max(ts) * 1e6:.0f}] us"}


def cpu_baseline_gemv(x, s_x, W, s_w, nbytes, runs=5):
    """The whole layer, median of five runs; GB/s of the same algorithmic bytes."""
    cores, model = cpu_info()
    import oracle
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle.gemv_w8a8(x, s_x, W, s_w)
        ts.append(time.perf_counter() - t0)
    t = sorted(ts)[runs // 2]
    return {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": cores, "cpu": model, "kind": "oracle",
            "sample": f"oracle_gemv_w8a8 (INT64 sums, FP32 dequantisation) on the whole 14336 x 4096 layer, "
                      f"median of {runs} runs {t * 1e3:.1f} ms [{min(ts) * 1e3:.1f}, {max(ts) * 1e3:.1f}]"}


def process_spread(args):
    """Run the headline GEMM and the cold GEMV in args.procs fresh processes
    (this script with --child), one after the other; median and [min, max]
    of their figures."""
    import subprocess
    vals = {"bf16": [], "gemv": []}
    for _ in range(args.procs):
        cmd = [sys.executable, os.path.abspath(__file__), "--only", "bf16+gemv", "--child",
               "--no-cpu-baseline", "--steps", str(args.steps), "--warmup", str(args.warmup)]
        out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        if out.returncode != 0:
            sys.stderr.write(out.stdout[-2000:] + out.stderr[-2000:])
            raise SystemExit(f"child bench process failed ({out.returncode})")
        line = [ln for ln in out.stdout.splitlines() if ln.startswith("{")][-1]
        r = json.loads(line)
        vals["bf16"].append(r["value"])
        vals["gemv"].append(r["extra"]["gemv_w8a8"]["GB_s"])
        print(f"# child process {len(vals['bf16'])}: {r['value']:.1f} TFLOP/s, "
              f"{vals['gemv'][-1]:.1f} GB/s", file=sys.stderr, flush=True)

    def summary(v, unit):
        s = sorted(v)
        return {"processes": len(v), "unit": unit, "median": s[len(s) // 2], "min": s[0], "max": s[-1],
                "values": v}
    return {"bf16": summary(vals["bf16"], "TFLOP/s"), "gemv": summary(vals["gemv"], "GB/s")}


def smi_clocks(launch, stream, n=4000):
    """Clock levels rocm-smi reports while the GEMM runs: n launches are
    queued (about half a second of work), rocm-smi is read while they run."""
    import subprocess
    import torch
    for _ in range(n):
        launch()
    try:
        out = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                             timeout=30)
        data = json.loads(out.stdout) if out.returncode == 0 else None
    except (OSError, ValueError, subprocess.TimeoutExpired):
        data = None
    torch.cuda.synchronize()
    if not data:
        return None
    card = next(iter(data.values()))
    return {k.rstrip(":").strip(): v for k, v in card.items() if isinstance(v, str) and "clk" in k.lower()}


def optional(fn, *a):
    """A context measurement (probe ceilings): its failure to load or run is
    reported in the line instead of ending the benchmark."""
    try:
        return fn(*a)
    except (OSError, RuntimeError) as e:
        return {"error": f"{type(e).__name__}: {e}"}


def mfma_ceiling(args, stream, inputs, kind="bf16"):
    """Practical MFMA rate on this part under sustained load
    (libmpdt_probes.so, mpdt_probe_mfma_peak: one wavefront per SIMD on every
    CU, each issuing back-to-back MFMAs of one kind from registers and
    nothing else -- for BF16 the 4096 32x32x16 MFMAs of the 4096^3 GEMM, for
    FP8 and INT8 the same number of cycles of 32x32x64 / 32x32x32 MFMAs),
    with operands drawn like the workloads' (N(0,1) as BF16, N(0,1)
    block-quantised to E4M3, uniform INT8) and with all-zero operands; timed
    like the GEMMs (back-to-back launches after the same warm-up), shader
    clock from the probe's own s_memtime / s_memrealtime stamps."""
    import ctypes
    import numpy as np
    import torch
    L = ctypes.CDLL(os.path.join(ROOT, "mixed_precision_dense_tiled_amd", "libmpdt_probes.so"))
    L.mpdt_probe_mfma_peak.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p]
    L.mpdt_probe_mfma_peak.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    wgs = 256
    code, iters, per_mfma = {"bf16": (0, 32, 2.0 * 32 * 32 * 16), "fp8": (1, 16, 2.0 * 32 * 32 * 64),
                             "i8": (2, 32, 2.0 * 32 * 32 * 32)}[kind]
    flop = wgs * 4 * iters * 128 * per_mfma
    out = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    stamps = torch.zeros(wgs * 4, dtype=torch.int64, device=dev)
    if kind == "bf16":
        bits = inputs.to_bf16_bits(inputs.normal_f32((2048 * 8,), 11)).view(np.uint8)
    elif kind == "fp8":
        bits = inputs.fp8_quantize_rows(inputs.normal_f32((64, 512), 11))[0].reshape(-1)
    else:
        bits = inputs.int_uniform((2048 * 16,), 11, -128, 127, np.int8).view(np.uint8)
    res = {"note": "one wavefront per SIMD on every CU, back-to-back MFMAs from registers "
                   "(" + {"bf16": "4096 32x32x16 BF16 each, the 4096^3 GEMM's MFMA work",
                          "fp8": "2048 32x32x64 FP8 E4M3 each", "i8": "4096 32x32x32 INT8 each"}[kind]
                   + "), nothing else"}
    for name, b in (("data", bits), ("zero", np.zeros_like(bits))):
        data = torch.from_numpy(np.ascontiguousarray(b)).to(dev)

        def run(i):
            rc = L.mpdt_probe_mfma_peak(code, data.data_ptr(), iters, out.data_ptr(), stamps.data_ptr(),
                                        torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"mpdt_probe_mfma_peak failed: {rc}")
        region, per = timed(run, args.steps, args.warmup, stream)
        st = stats(per, region, args.steps)
        q = stamps.cpu().numpy().reshape(wgs, 4).astype(np.float64)
        ghz = float(np.median((q[:, 1] - q[:, 0]) / ((q[:, 3] - q[:, 2]) / 100e6)) / 1e9)
        key = "" if name == "data" else "zero_data_"
        unit = "TOP_s" if kind == "i8" else "TFLOP_s"
        res[key + unit] = flop / (st["mean_us"] * 1e-6) / 1e12
        res[key + "mean_us"] = st["mean_us"]
        res[key + "shader_clock_ghz"] = ghz
    return res


def read_ceiling(args, stream):
    """Practical HBM read rates on this part (libmpdt_probes.so,
    mpdt_probe_stream_read: non-temporal 16-byte loads, all of a wave's
    loads in flight before use): the GEMV's own byte count with 8 rotating
    copies (cold, like the GEMV timing) at the GEMV's 8 KiB per wave and at
    16 KiB per wave, and a long 1 GiB stream."""
    import ctypes
    import torch
    L = ctypes.CDLL(os.path.join(ROOT, "mixed_precision_dense_tiled_amd", "libmpdt_probes.so"))
    L.mpdt_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
    L.mpdt_probe_stream_read.restype = ctypes.c_int
    dev = torch.device("cuda:0")
    sink = torch.zeros(16, dtype=torch.int32, device=dev)
    out = {}
    nbytes = 58_720_256
    copies = [torch.ones(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(8)]

    def run(buf, n, per, waves):
        # torch's current stream: the capture stream while a graph is recorded
        rc = L.mpdt_probe_stream_read(buf.data_ptr(), n, per, waves, sink.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)
        if rc != 0:
            raise RuntimeError(f"mpdt_probe_stream_read failed: {rc}")
    for per, waves, name in ((8, 4, "same_bytes_cold_8KiB_per_wave"), (16, 4, "same_bytes_cold_16KiB_per_wave"),
                             (4, 1, "same_bytes_cold_4KiB_per_wave_1_wave_groups")):
        region, _ = timed(lambda i: run(copies[i % 8], nbytes, per, waves), args.steps, args.warmup, stream)
        us = 1e3 * region / args.steps
        out[name] = {"bytes": nbytes, "GB_s": nbytes / (us * 1e-6) / 1e9, "mean_us": us}
    del copies
    big = 1 << 30
    buf = torch.ones(big // 4, dtype=torch.int32, device=dev)
    steps = max(args.steps // 5, 5)
    region, per_l = timed(lambda i: run(buf, big, 16, 4), steps, 20, stream)
    st = stats(per_l, region, steps)
    out["long_stream_1GiB"] = {"bytes": big, "GB_s": big / (st["mean_us"] * 1e-6) / 1e9, "launch_us": st}
    out["note"] = ("back-to-back launches between HIP events, timed like the GEMV (each launch's start "
                   "and drain included); short reads rotate 8 copies")
    return out


if __name__ == "__main__":
    main()
