"""Benchmark of the group-quantized linear layer on one MI355X.

Headline workload (one step): Llama-shaped W4A16 decode, M = 1 token,
K = 4096, g = 128 asymmetric INT4, packed ahead of time; a step runs the
N = 11008 layer and the N = 4096 layer on the same X, as one
w4a16_linear_multi launch. The metric is HBM throughput: the algorithmic
bytes of a step (packed codes + fp16 scales + 4-bit zero-points + X + Y of
both layers) over its time. Inputs are resident in HBM before the timed
region; every step reads a different copy of the packed weights (copies
totalling more than 512 MB), so the 256 MB Infinity Cache cannot serve
repeats. Launches are captured in a HIP graph (one graph holds one pass over
the weight copies) and replayed.

The JSON line also carries:
  roofline      the dominant kernel (the two-layer decode GEMV launch) timed
                with HIP events on its stream, against 8 TB/s;
  cpu_baseline  the CPU oracle (fp64 reference over the dequantized weights)
                timed on this host's cores on the same step;
  extra         (every figure the median of 5 timed repeats) the same step as
                two w4a16_linear launches, each layer alone, the harness's
                floors (a one-element launch, device copies of the codes),
                prefill (M = 2048, sym) TFLOP/s against the fp16 MFMA peak,
                W8A8 (M = 2048, K = N = 8192) TOP/s against the int8 peak,
                its FP8 E4M3 variant TFLOP/s against the fp8 peak, MXFP4
                weights x E4M3 activations on that layer and on the prefill
                shape, NF4 decode GB/s,
                quantize + pack GB/s, batched decode M = 16 / 64 (N = 11008) and
                M = 8 / 16 (N = 4096).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-cpu]
                       [--only decode|prefill|w8a8|fp8|mxfp4|nf4|nvfp4|quant|batched] [--eager]
                       [--copy-calibration]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
FP16_MFMA_PEAK_TFLOPS = 2500.0  # dense fp16
INT8_MFMA_PEAK_TOPS = 5000.0    # dense int8
FP8_MFMA_PEAK_TFLOPS = 5000.0   # dense fp8
METRIC = "W4A16 g128 GEMM: GB/s at M=1, TFLOP/s at M=2048 (% of roofline)"
MALL_BYTES = 512 * 2 ** 20
COPY_BYTES = 2 ** 30
# The kernel the dispatcher picks for the decode step: both layers (N = 11008
# and 4096, M = 1, K = 4096, g = 128 asym) in one launch of 688 + 256 blocks
# of 8 wavefronts, 4 k-blocks per wavefront.
DECODE_KERNEL = "w4a16_gemv_multi_kernel<8, 4, true, true>"
# the decode GEMV's source files: the committed traffic figures are valid only
# for the revision of these files they were taken on
DECODE_SOURCES = [os.path.join(ROOT, "quantized_gemm_q4_amd", "csrc", f)
                  for f in ("w4a16_gemv.hip", "w4a16_dequant.hpp", "q4_internal.hpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "w4a16_gemv_decode_step_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def w4a16_bytes(M: int, N: int, K: int, g: int = 128, sym: bool = False) -> int:
    """Algorithmic HBM bytes of one W4A16 call: packed codes, fp16 scales,
    4-bit zero-points (asym), fp16 X read once, fp16 Y written once."""
    G = K // g
    return N * K // 2 + N * G * 2 + (0 if sym else N * ((G + 1) // 2)) + M * K * 2 + M * N * 2


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--only", default=None, choices=["decode", "prefill", "w8a8", "fp8", "mxfp4", "nf4", "nvfp4",
                                                     "quant", "batched"])
    ap.add_argument("--eager", action="store_true", help="launch eagerly instead of replaying a graph")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (reference for the HBM byte counters)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "this layer has no multi-GPU path to time.", file=sys.stderr)
        sys.exit(2)

    import torch
    import quantized_gemm_q4_amd as q4
    import workloads

    if not os.path.exists(q4.LIB_PATH):
        from quantized_gemm_q4_amd import build
        build.build()
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def gpu(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.float16:
            return torch.from_numpy(a.view(np.int16)).view(torch.float16).to(dev)
        return torch.from_numpy(a).to(dev)

    def timed_once(fn, n):
        """Run fn(i) for i < n between two HIP events on the current stream."""
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3  # seconds

    def timed(fn, n, repeats=5):
        """Median over `repeats` timings of fn(0..n-1) (seconds for the n calls)."""
        return float(np.median([timed_once(fn, n) for _ in range(repeats)]))

    def graph_of(fn, n):
        """Capture fn(0..n-1) into one HIP graph (eager fallback with --eager)."""
        if args.eager:
            return lambda: [fn(i) for i in range(n)]
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream(dev)
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            fn(0)
        stream.wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(i)
        torch.cuda.synchronize()
        return g.replay

    out = {"metric": METRIC, "n_gpus": 1, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f16", "data": "synthetic"}
    extra = {}
    only = args.only

    # ---- headline: decode step (N = 11008 and N = 4096 on one X, M = 1) ----
    if only in (None, "decode"):
        layers = []
        X = None
        for N in (11008, 4096):
            w = workloads.decode(N)
            X = gpu(w["X"])    # the same X for both layers
            packed = q4.q4_quantize_pack(gpu(w["W"]), g=128, sym=False)
            layers.append(dict(N=N, packed=packed,
                               Y=torch.empty((1, N), dtype=torch.float16, device=dev)))
        step_bytes = sum(w4a16_bytes(1, L["N"], 4096) for L in layers) - 4096 * 2   # X read once
        # enough copies that even the N = 11008 layer alone cycles > 512 MB
        copies = max(2, math.ceil(MALL_BYTES / w4a16_bytes(1, 11008, 4096)) + 1)
        for L in layers:
            L["copies"] = [tuple(t.clone() for t in L["packed"]) for _ in range(copies)]
        Ys = [L["Y"] for L in layers]

        def step(i):
            c = i % copies
            q4.w4a16_linear_multi(X, [L["copies"][c] for L in layers], out=Ys)

        for i in range(args.warmup):
            step(i)
        K = args.steps
        # each graph holds whole cycles over the weight copies, about 240 steps,
        # so the K timed steps take few graph launches
        per_graph = copies * max(1, 240 // copies)
        full = graph_of(step, per_graph)
        rem = K % per_graph
        tail = graph_of(step, rem) if rem else None
        full()
        torch.cuda.synchronize()
        t = timed_once(lambda i: full() if i < K // per_graph else tail(), K // per_graph + (1 if rem else 0))
        out.update(value=step_bytes * K / t / 1e9, unit="GB/s", steps=K, warmup=args.warmup,
                   ms_per_step=t / K * 1e3)
        out["config"] = {"workload": "W4A16 decode: M=1, K=4096, N=11008 and N=4096 on the same X "
                                     "(one w4a16_linear_multi launch), asym INT4 g=128 pre-packed; "
                                     "X ~ N(0,1), W ~ N(0,0.02) with 1% of K-channels x10",
                         "bytes_per_step": step_bytes, "weight_copies": copies,
                         "launch": "eager" if args.eager else "hip-graph",
                         "seeds": {"W": 1002, "X": 2002, "outliers": 4002}}

        # dominant kernel: the two-layer launch, on its own graph
        reps = max(1, 2 * K // copies)
        gm = graph_of(step, copies)
        gm()
        tm = timed(lambda i: gm(), reps) / (reps * copies)
        out["roofline"] = {"kernel": DECODE_KERNEL + " (M=1, N=11008 + 4096, K=4096)",
                           "bound": "hbm", "achieved": step_bytes / tm / 1e9, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": step_bytes / tm / 1e9 / HBM_PEAK_GBS,
                           "traffic": measured_traffic(), "avg_launch_us": tm * 1e6,
                           "algorithmic_bytes_per_launch": step_bytes, "launches": reps * copies}

        # the same step as two single-layer launches, and each layer alone
        # (the per-call figures go into the roofline block beside the fused launch)
        def step2(i):
            c = i % copies
            for L in layers:
                q4.w4a16_linear(X, *L["copies"][c], out=L["Y"])
        g2 = graph_of(step2, copies)
        g2()
        t2 = timed(lambda i: g2(), reps) / (reps * copies)
        extra["decode_two_launches"] = {"us": t2 * 1e6, "GB/s": (step_bytes + 4096 * 2) / t2 / 1e9}
        for L in layers:
            gl = graph_of(lambda i, L=L: q4.w4a16_linear(X, *L["copies"][i % copies], out=L["Y"]), copies)
            gl()
            tl = timed(lambda i: gl(), reps) / (reps * copies)
            bl = w4a16_bytes(1, L["N"], 4096)
            extra[f"decode_n{L['N']}"] = {"us": tl * 1e6, "GB/s": bl / tl / 1e9,
                                          "frac_hbm": bl / tl / 1e9 / HBM_PEAK_GBS}
            out["roofline"].setdefault("per_call", {})[f"w4a16_linear M=1 N={L['N']} K=4096"] = {
                "avg_launch_us": tl * 1e6, "algorithmic_bytes_per_launch": bl,
                "achieved": bl / tl / 1e9, "frac": bl / tl / 1e9 / HBM_PEAK_GBS}
        # the N = 11008 layer in its AWQ form: x / s fused into the GEMV's X loads
        L = next(L for L in layers if L["N"] == 11008)
        s_awq = torch.from_numpy(np.exp(np.random.default_rng(5002).uniform(-0.5, 0.5, 4096))
                                 .astype(np.float32)).to(dev)
        ws = torch.empty((q4.w4a16_awq_workspace_bytes(1, 4096),), dtype=torch.uint8, device=dev)
        ga = graph_of(lambda i: q4.w4a16_linear_awq(X, *L["copies"][i % copies], s_awq,
                                                   workspace=ws, out=L["Y"]), copies)
        ga()
        ta = timed(lambda i: ga(), reps) / (reps * copies)
        ba = w4a16_bytes(1, 11008, 4096) + 4096 * 4
        extra["awq_decode_n11008"] = {"us": ta * 1e6, "GB/s": ba / ta / 1e9,
                                      "frac_hbm": ba / ta / 1e9 / HBM_PEAK_GBS}
        # floors in the same harness (graph replays over the same number of
        # copies), from library kernels: a one-element add per launch and
        # device copies of the step's packed codes (read + write)
        extra["floors"] = floors(graph_of, timed, reps, copies, dev,
                                 [[L["copies"][c][0] for L in layers] for c in range(copies)])
        del layers
        torch.cuda.empty_cache()

        if not args.skip_cpu:
            out["cpu_baseline"] = cpu_baseline(step_bytes)
            extra["cpu_oracle"] = cpu_oracle_samples()

    # ---- batched decode M = 16, 64 ---------------------------------------------
    if only in (None, "batched"):
        w = workloads.quant()
        packed = q4.q4_quantize_pack(gpu(w["W"]), g=128, sym=False)
        bytes1 = w4a16_bytes(16, 11008, 4096)
        copies = max(2, math.ceil(MALL_BYTES / bytes1) + 1)
        cps = [tuple(t.clone() for t in packed) for _ in range(copies)]
        for M in (16, 64):
            X = gpu(workloads.quant(M)["X"])
            Y = torch.empty((M, 11008), dtype=torch.float16, device=dev)
            gr = graph_of(lambda i: q4.w4a16_linear(X, *cps[i % copies], out=Y), copies)
            gr()
            reps = max(1, 1000 // copies)
            tt = timed(lambda i: gr(), reps) / (reps * copies)
            nb = w4a16_bytes(M, 11008, 4096)
            extra[f"batched_m{M}"] = {"us": tt * 1e6, "GB/s": nb / tt / 1e9,
                                      "frac_hbm": nb / tt / 1e9 / HBM_PEAK_GBS,
                                      "TFLOP/s": 2 * M * 11008 * 4096 / tt / 1e12}
        del cps, packed
        # the second decode layer's shape (N = 4096): 8 <= M <= 16 runs the
        # X-in-registers batched kernel
        w4 = workloads.decode(4096)
        packed = q4.q4_quantize_pack(gpu(w4["W"]), g=128, sym=False)
        bytes1 = w4a16_bytes(16, 4096, 4096)
        copies = max(2, math.ceil(MALL_BYTES / bytes1) + 1)
        cps = [tuple(t.clone() for t in packed) for _ in range(copies)]
        X16 = workloads.quant(16)["X"]
        for M in (8, 16):
            X = gpu(X16[:M])
            Y = torch.empty((M, 4096), dtype=torch.float16, device=dev)
            gr = graph_of(lambda i: q4.w4a16_linear(X, *cps[i % copies], out=Y), copies)
            gr()
            reps = max(1, 1000 // copies)
            tt = timed(lambda i: gr(), reps) / (reps * copies)
            nb = w4a16_bytes(M, 4096, 4096)
            extra[f"batched_m{M}_n4096"] = {"us": tt * 1e6, "GB/s": nb / tt / 1e9,
                                            "frac_hbm": nb / tt / 1e9 / HBM_PEAK_GBS,
                                            "TFLOP/s": 2 * M * 4096 * 4096 / tt / 1e12}
        del cps, packed
        torch.cuda.empty_cache()

    # ---- quantize + pack -----------------------------------------------------
    if only in (None, "quant"):
        w = workloads.quant()
        W = gpu(w["W"])
        nW = max(2, math.ceil(MALL_BYTES / W.numel() / 2) + 1)
        Ws = [W.clone() for _ in range(nW)]
        res = q4.q4_quantize_pack(W)
        for i in range(5):
            q4.q4_quantize_pack(Ws[i % nW], out=res)
        # graph replays (an eager Python loop is host-bound at this kernel time)
        nq = 4 * nW
        gq = graph_of(lambda i: q4.q4_quantize_pack(Ws[i % nW], out=res), nq)
        gq()
        reps = 15
        tq = timed(lambda i: gq(), reps) / (reps * nq)
        qbytes = 11008 * 4096 * 2 + 11008 * 2048 + 11008 * 32 * 2 + 11008 * 16
        extra["quantize_pack"] = {"shape": [11008, 4096], "us": tq * 1e6, "GB/s": qbytes / tq / 1e9,
                                  "frac_hbm": qbytes / tq / 1e9 / HBM_PEAK_GBS, "bytes": qbytes}
        del Ws, W, res
        torch.cuda.empty_cache()

    # ---- prefill M = 2048 --------------------------------------------------------
    if only in (None, "prefill"):
        w = workloads.prefill()
        packed = q4.q4_quantize_pack(gpu(w["W"]), g=128, sym=True)
        X = gpu(w["X"])
        Y = torch.empty((2048, 11008), dtype=torch.float16, device=dev)
        for _ in range(3):
            q4.w4a16_linear(X, *packed, out=Y)
        reps = 30
        tp = timed(lambda i: q4.w4a16_linear(X, *packed, out=Y), reps) / reps
        flops = 2 * 2048 * 11008 * 4096
        extra["prefill"] = {"shape": [2048, 11008, 4096], "us": tp * 1e6,
                            "TFLOP/s": flops / tp / 1e12,
                            "frac_mfma_fp16": flops / tp / 1e12 / FP16_MFMA_PEAK_TFLOPS}
        del packed, X, Y
        torch.cuda.empty_cache()

    # ---- W8A8 M = 2048, K = N = 8192 ------------------------------------------
    if only in (None, "w8a8"):
        w = workloads.w8a8()
        s = q4.smoothquant_scales(gpu(w["Xcal"]), gpu(w["W"]), 0.5)
        Wq, sw = q4.q8_quantize_weight(gpu(w["W"]), s)
        X = gpu(w["X"])
        M, K = X.shape
        N = Wq.shape[0]
        ws = q4.w8a8_workspace(M, K, dev)
        Y = torch.empty((M, N), dtype=torch.float16, device=dev)
        Xq, sx = q4.q8_quantize_act(X, s)
        for _ in range(3):
            q4.w8a8_linear(X, Wq, sw, s, workspace=ws, out=Y)
        reps = 30
        tl = timed(lambda i: q4.w8a8_linear(X, Wq, sw, s, workspace=ws, out=Y), reps) / reps
        tg = timed(lambda i: q4.w8a8_gemm(Xq, sx, Wq, sw, out=Y), reps) / reps
        ga = graph_of(lambda i: q4.q8_quantize_act(X, s, out=(Xq, sx)), 8)
        ga()
        ta = timed(lambda i: ga(), reps) / (reps * 8)
        ops = 2 * M * N * K
        abytes = M * K * 2 + K * 4 + M * K + M * 4
        extra["w8a8"] = {"shape": [M, N, K], "linear_us": tl * 1e6, "linear_TOP/s": ops / tl / 1e12,
                         "gemm_us": tg * 1e6, "gemm_TOP/s": ops / tg / 1e12,
                         "gemm_frac_mfma_int8": ops / tg / 1e12 / INT8_MFMA_PEAK_TOPS,
                         "act_quant_us": ta * 1e6, "act_quant_GB/s": abytes / ta / 1e9}
        # the LayerNorm in front of the layer with the divide by s and the
        # per-token quantizer fused in (X read as the hidden state before the
        # norm), against the unfused pair: torch's fp16 layer_norm writing the
        # normalised X, then q8_quantize_act on it
        p = workloads.layernorm_params(K)
        gam, bet, sln = gpu(p["gamma"]), gpu(p["beta"]), gpu(p["s"])
        gn = graph_of(lambda i: q4.layernorm_quant_smooth(X, gam, bet, sln, 1e-5, out=(Xq, sx)), 8)
        gn()
        tn = timed(lambda i: gn(), reps) / (reps * 8)
        g16, b16 = gam.half(), bet.half()
        gu = graph_of(lambda i: q4.q8_quantize_act(torch.nn.functional.layer_norm(X, (K,), g16, b16, 1e-5), sln,
                                                   out=(Xq, sx)), 8)
        gu()
        tu = timed(lambda i: gu(), reps) / (reps * 8)
        nbytes = M * K * 2 + 3 * K * 4 + M * K + M * 4
        extra["w8a8"]["norm_quant_fused"] = {
            "us": tn * 1e6, "GB/s": nbytes / tn / 1e9, "frac_hbm": nbytes / tn / 1e9 / HBM_PEAK_GBS,
            "bytes": nbytes, "unfused_layer_norm_then_act_quant_us": tu * 1e6,
            "layer_with_fused_norm_us": (tn + tg) * 1e6, "over_gemm_alone": (tn + tg) / tg}
        del gu, gn
        del Wq, Xq
        # the decode workload's N = 11008 layer (M = 1) with INT8 weights: the decode GEMV
        w = workloads.decode(11008)
        N, K = w["W"].shape
        Wq, sw = q4.q8_quantize_weight(gpu(w["W"]))
        Xq, sx = q4.q8_quantize_act(gpu(w["X"]))
        nb = N * K + N * 4 + K + 4 + N * 2
        copies = max(2, math.ceil(MALL_BYTES / nb) + 1)
        cps = [(Wq.clone(), sw.clone()) for _ in range(copies)]
        Y = torch.empty((1, N), dtype=torch.float16, device=dev)
        reps = max(1, 2000 // copies)
        gg = graph_of(lambda i: q4.w8a8_gemm(Xq, sx, *cps[i % copies], out=Y), copies)
        gg()
        tg = timed(lambda i: gg(), reps) / (reps * copies)
        # the whole layer from fp16 X: one launch, the per-token quantizer fused in
        X1 = gpu(w["X"])
        ws1 = q4.w8a8_workspace(1, K, dev)
        gl = graph_of(lambda i: q4.w8a8_linear(X1, *cps[i % copies], None, workspace=ws1, out=Y), copies)
        gl()
        tl = timed(lambda i: gl(), reps) / (reps * copies)
        extra["w8a8"]["decode_n11008"] = {"gemv_us": tg * 1e6, "GB/s": nb / tg / 1e9,
                                          "frac_hbm": nb / tg / 1e9 / HBM_PEAK_GBS, "bytes": nb,
                                          "linear_fused_us": tl * 1e6}
        del cps, Wq, Xq, Y

    # ---- FP8 E4M3 variant of the same layer ------------------------------------
    if only in (None, "w8a8", "fp8"):
        w = workloads.w8a8()
        s = q4.smoothquant_scales(gpu(w["Xcal"]), gpu(w["W"]), 0.5)
        Wq, sw = q4.fp8_quantize_weight(gpu(w["W"]), s)
        X = gpu(w["X"])
        M, K = X.shape
        N = Wq.shape[0]
        ws = q4.w8a8_workspace(M, K, dev)
        Y = torch.empty((M, N), dtype=torch.float16, device=dev)
        Xq, sx = q4.fp8_quantize_act(X, s)
        for _ in range(3):
            q4.fp8_linear(X, Wq, sw, s, workspace=ws, out=Y)
        reps = 30
        tl = timed(lambda i: q4.fp8_linear(X, Wq, sw, s, workspace=ws, out=Y), reps) / reps
        tg = timed(lambda i: q4.fp8_gemm(Xq, sx, Wq, sw, out=Y), reps) / reps
        ga = graph_of(lambda i: q4.fp8_quantize_act(X, s, out=(Xq, sx)), 8)
        ga()
        ta = timed(lambda i: ga(), reps) / (reps * 8)
        ops = 2 * M * N * K
        abytes = M * K * 2 + K * 4 + M * K + M * 4
        extra["fp8"] = {"shape": [M, N, K], "linear_us": tl * 1e6, "linear_TFLOP/s": ops / tl / 1e12,
                        "gemm_us": tg * 1e6, "gemm_TFLOP/s": ops / tg / 1e12,
                        "gemm_frac_mfma_fp8": ops / tg / 1e12 / FP8_MFMA_PEAK_TFLOPS,
                        "act_quant_us": ta * 1e6, "act_quant_GB/s": abytes / ta / 1e9}
        del Wq, Xq
        # the decode workload's N = 11008 layer (M = 1) with E4M3 weights: the decode GEMV
        w = workloads.decode(11008)
        N, K = w["W"].shape
        Wq, sw = q4.fp8_quantize_weight(gpu(w["W"]))
        Xq, sx = q4.fp8_quantize_act(gpu(w["X"]))
        nb = N * K + N * 4 + K + 4 + N * 2
        copies = max(2, math.ceil(MALL_BYTES / nb) + 1)
        cps = [(Wq.clone(), sw.clone()) for _ in range(copies)]
        Y = torch.empty((1, N), dtype=torch.float16, device=dev)
        reps = max(1, 2000 // copies)
        gg = graph_of(lambda i: q4.fp8_gemm(Xq, sx, *cps[i % copies], out=Y), copies)
        gg()
        tg = timed(lambda i: gg(), reps) / (reps * copies)
        X1 = gpu(w["X"])
        ws1 = q4.w8a8_workspace(1, K, dev)
        gl = graph_of(lambda i: q4.fp8_linear(X1, *cps[i % copies], None, workspace=ws1, out=Y), copies)
        gl()
        tl = timed(lambda i: gl(), reps) / (reps * copies)
        extra["fp8"]["decode_n11008"] = {"gemv_us": tg * 1e6, "GB/s": nb / tg / 1e9,
                                         "frac_hbm": nb / tg / 1e9 / HBM_PEAK_GBS, "bytes": nb,
                                         "linear_fused_us": tl * 1e6}
        del cps, Wq, Xq, Y

    # ---- MXFP4 weights x E4M3 activations (W4A8) ------------------------------
    if only in (None, "w8a8", "mxfp4"):
        res = {}
        # the W8A8 workload's layer, and the prefill workload's shape
        for name in ("w8a8", "prefill"):
            w = workloads.w8a8() if name == "w8a8" else workloads.prefill()
            X = gpu(w["X"])
            s = q4.smoothquant_scales(gpu(w["Xcal"]), gpu(w["W"]), 0.5) if name == "w8a8" else None
            codes, sc = q4.mxfp4_quantize_weight(gpu(w["W"]), s)
            M, K = X.shape
            N = codes.shape[0]
            ws = q4.w8a8_workspace(M, K, dev)
            Y = torch.empty((M, N), dtype=torch.float16, device=dev)
            Xq, sx = q4.fp8_quantize_act(X, s)
            for _ in range(3):
                q4.mxfp4_linear(X, codes, sc, s, workspace=ws, out=Y)
            reps = 30
            tl = timed(lambda i: q4.mxfp4_linear(X, codes, sc, s, workspace=ws, out=Y), reps) / reps
            tg = timed(lambda i: q4.mxfp4_gemm(Xq, sx, codes, sc, out=Y), reps) / reps
            ops = 2 * M * N * K
            res[name] = {"shape": [M, N, K], "linear_us": tl * 1e6, "linear_TFLOP/s": ops / tl / 1e12,
                         "gemm_us": tg * 1e6, "gemm_TFLOP/s": ops / tg / 1e12,
                         "gemm_frac_mfma_fp8": ops / tg / 1e12 / FP8_MFMA_PEAK_TFLOPS}
            del codes, sc, Xq, X, Y, ws
        # the decode workload's N = 11008 layer (M = 1): the decode GEMV
        w = workloads.decode(11008)
        N, K = w["W"].shape
        X = gpu(w["X"])
        codes, sc = q4.mxfp4_quantize_weight(gpu(w["W"]))
        Xq, sx = q4.fp8_quantize_act(X)
        nb = N * K // 2 + N * K // 32 + K + 4 + N * 2
        copies = max(2, math.ceil(MALL_BYTES / nb) + 1)
        cps = [(codes.clone(), sc.clone()) for _ in range(copies)]
        Y = torch.empty((1, N), dtype=torch.float16, device=dev)
        ws = q4.w8a8_workspace(1, K, dev)
        reps = max(1, 2000 // copies)
        gg = graph_of(lambda i: q4.mxfp4_gemm(Xq, sx, *cps[i % copies], out=Y), copies)
        gg()
        tg = timed(lambda i: gg(), reps) / (reps * copies)
        gl = graph_of(lambda i: q4.mxfp4_linear(X, *cps[i % copies], None, workspace=ws, out=Y), copies)
        gl()
        tl = timed(lambda i: gl(), reps) / (reps * copies)
        res["decode_n11008"] = {"gemv_us": tg * 1e6, "GB/s": nb / tg / 1e9,
                                "frac_hbm": nb / tg / 1e9 / HBM_PEAK_GBS, "bytes": nb,
                                "linear_us": tl * 1e6}
        del cps, codes, sc, Xq, X, Y, ws
        extra["mxfp4_w4a8"] = res
        torch.cuda.empty_cache()

    # ---- NF4 and NVFP4: decode (M = 1, K = 4096, N = 11008 and 4096) and the
    # prefill shape (M = 2048) on the large-M GEMM ------------------------------------
    lut_formats = {
        # name: (quantize, linear, scale bytes per weight)
        "nf4": (q4.nf4_quantize, q4.nf4_linear, 4 / 64),
        "nvfp4": (q4.nvfp4_quantize, q4.nvfp4_linear, 1 / 16),
    }
    for fmt, (quant, linear, sbpw) in lut_formats.items():
        if only not in (None, fmt):
            continue
        res = {}
        for N in (11008, 4096):
            w = workloads.decode(N)
            X = gpu(w["X"])
            codes, sc = quant(gpu(w["W"]))
            nb = int(N * 4096 // 2 + N * 4096 * sbpw + 4096 * 2 + N * 2)
            copies = max(2, math.ceil(MALL_BYTES / nb) + 1)
            cps = [(codes.clone(), sc.clone()) for _ in range(copies)]
            Y = torch.empty((1, N), dtype=torch.float16, device=dev)
            gr = graph_of(lambda i: linear(X, *cps[i % copies], out=Y), copies)
            gr()
            reps = max(1, 2000 // copies)
            tt = timed(lambda i: gr(), reps) / (reps * copies)
            res[f"n{N}"] = {"us": tt * 1e6, "GB/s": nb / tt / 1e9, "frac_hbm": nb / tt / 1e9 / HBM_PEAK_GBS,
                            "bytes": nb}
            del cps, codes, sc
        extra[f"{fmt}_decode"] = res
        w = workloads.prefill()
        codes, sc = quant(gpu(w["W"]))
        X = gpu(w["X"])
        Y = torch.empty((2048, 11008), dtype=torch.float16, device=dev)
        for _ in range(3):
            linear(X, codes, sc, out=Y)
        tp = timed(lambda i: linear(X, codes, sc, out=Y), 30) / 30
        flops = 2 * 2048 * 11008 * 4096
        extra[f"{fmt}_prefill"] = {"shape": [2048, 11008, 4096], "us": tp * 1e6, "TFLOP/s": flops / tp / 1e12,
                                   "frac_mfma_fp16": flops / tp / 1e12 / FP16_MFMA_PEAK_TFLOPS}
        del codes, sc, X, Y
        torch.cuda.empty_cache()

    # ---- known-size copy: scales the HBM byte counters (profiling runs only) -
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).uniform_()
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        extra["copy_calibration"] = {"bytes_read": COPY_BYTES, "bytes_written": COPY_BYTES,
                                     "launches": 4}
        del src, dst

    if extra:
        out["extra"] = extra
    if "value" not in out:
        out.update(value=None, unit="GB/s", steps=0, warmup=args.warmup, ms_per_step=None,
                   config={"workload": f"partial run: {only}"})
    print(json.dumps(out), flush=True)


def floors(graph_of, timed, reps, copies, dev, codes):
    """Per-launch floors of the decode harness (graph replays over the weight
    copies, as the GEMV figures): a one-element add, and device copies of the
    packed codes of both layers and of the N = 11008 layer (codes[c] holds the
    codes of the step's layers for weight copy c, N = 11008 first)."""
    import torch
    res = {}

    def per_launch(fn):
        g = graph_of(fn, copies)
        g()
        return timed(lambda i: g(), reps) / (reps * copies)

    tiny = torch.zeros(1, device=dev)
    res["launch_us"] = per_launch(lambda i: tiny.add_(1.0)) * 1e6
    for name, sel in (("copy_step_codes", None), ("copy_n11008_codes", 0)):
        src = [torch.cat([c.view(-1) for c in cs]) if sel is None else cs[sel].view(-1).clone() for cs in codes]
        dst = torch.empty_like(src[0])
        t = per_launch(lambda i: dst.copy_(src[i % copies]))
        res[name] = {"bytes_moved": 2 * src[0].numel(), "us": t * 1e6, "GB/s": 2 * src[0].numel() / t / 1e9}
        del src, dst
    return res


def measured_traffic():
    """HBM bytes per launch of the decode GEMV from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by what the counter reads
    for a copy of known size). None when that summary is missing or was
    taken on a different revision of the kernel source."""
    import hashlib
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        h = hashlib.sha256()
        for path in DECODE_SOURCES:
            with open(path, "rb") as f:
                h.update(f.read())
        sha = h.hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != sha or rec.get("kernel") != DECODE_KERNEL:
        return None
    return rec.get("traffic_bytes_per_launch")


def _wall(fn, min_s: float = 1.0):
    """Median wall time of fn() over at least three runs and about min_s seconds."""
    t0 = time.perf_counter()
    fn()
    first = time.perf_counter() - t0
    n = max(3, min(20, int(min_s / max(first, 1e-4))))
    ts = []
    for _ in range(n):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def cpu_oracle_samples() -> dict:
    """The oracle on bounded samples of the other workloads (same inputs as
    the GPU sections; a few seconds each): quantize + pack of the full
    [11008, 4096] weight, the fp64 W4A16 product on 256 of the prefill
    workload's 2048 rows, and the W8A8 chain (per-token INT8 of the rows,
    exact integer GEMM, fp32 epilogue) on 128 of its 2048 rows."""
    import oracle
    import workloads

    res = {"cores": oracle.num_threads()}
    w = workloads.quant()
    qbytes = 11008 * 4096 * 2 + 11008 * 2048 + 11008 * 32 * 2 + 11008 * 16
    t = _wall(lambda: oracle.q4_quantize_pack(w["W"], g=128, sym=False))
    res["quantize_pack"] = {"GB/s": qbytes / t / 1e9, "s": t, "sample": "full [11008, 4096] asym g=128"}
    w = workloads.prefill()
    c, sc, z = oracle.q4_quantize_pack(w["W"], g=128, sym=True)
    rows = np.arange(256)
    t = _wall(lambda: oracle.w4a16_ref(w["X"], c, sc, z, rows=rows))
    res["prefill_fp64"] = {"GFLOP/s": 2 * 256 * 11008 * 4096 / t / 1e9, "s": t,
                           "sample": "256 of 2048 rows, N=11008, K=4096, sym g=128"}
    w = workloads.w8a8()
    s_ref = oracle.smooth_scales(w["Xcal"], w["W"], 0.5)
    Wq, sw = oracle.q8_quantize_weight(w["W"], s_ref)
    Xs = w["X"][:128]

    def chain():
        Xq, sx = oracle.q8_quantize_act(Xs, s_ref)
        acc, aacc, _ = oracle.int8_gemm(Xq, Wq)
        oracle.w8a8_epilogue(acc, aacc, sx, sw)
    t = _wall(chain)
    res["w8a8_int"] = {"GOP/s": 2 * 128 * 8192 * 8192 / t / 1e9, "s": t,
                       "sample": "128 of 2048 rows, N=K=8192: per-token INT8, int64 GEMM, epilogue"}
    return res


def cpu_baseline(step_bytes: int) -> dict:
    """The CPU oracle on the decode step: the exact fp64 product over the
    dequantized weights for N = 11008 and N = 4096 at M = 1, repeated for
    about 12 s of work."""
    import oracle
    import workloads

    layers = []
    for N in (11008, 4096):
        w = workloads.decode(N)
        c, s, z = oracle.q4_quantize_pack(w["W"], g=128, sym=False)
        layers.append((w["X"], c, s, z))

    def one():
        for X, c, s, z in layers:
            oracle.w4a16_ref(X, c, s, z)

    one()   # warm-up (first-touch of the arrays, thread start)
    t0 = time.perf_counter()
    one()
    t1 = time.perf_counter() - t0
    reps = max(1, min(5000, int(12.0 / max(t1, 1e-3))))
    t0 = time.perf_counter()
    for _ in range(reps):
        one()
    t = time.perf_counter() - t0
    return {"value": step_bytes * reps / t / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle", "seconds": t,
            "sample": f"the full decode step (M=1, K=4096, N=11008 then N=4096) x {reps}; "
                      "fp64 reference product over the dequantized weights"}


if __name__ == "__main__":
    main()
