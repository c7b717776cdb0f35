"""Benchmark of the block-scaled GEMM library on one MI355X.

A step = the six MXFP8 NT GEMMs of the LLM-shaped workload (M in {4096,
16384} x (N, K) in {(4096, 4096), (14336, 4096), (4096, 14336)}; E4M3 codes
with one E8M0 scale per 32 K values, FP32 accumulation, BF16 output), each
one mxgemm_run call on weights preshuffled once before timing.  Inputs are
seeded synthetic data resident in HBM before the timed region.

Also measured (reported beside the headline, not part of `value`): the
grouped groupwise FP8 GEMM (G=8) in microseconds per call, tensor-wise FP8
GEMMs of a 4096 -> 11008 linear layer at 8192 tokens (forward NT, data
gradient NN, weight gradient TN), the MXFP8 data and weight gradients of the
same layer (NN, TN), the on-device quantizers (GB/s), the MXFP4 8192^3 GEMM,
and the CPU oracle on a bounded sample of the MXFP8 workload.

`roofline` describes the dominant kernel (the MXFP8 NT kernel with
preshuffled B): algorithmic FLOPs per launch (2MNK) over its mean launch
duration from HIP events on the launch stream.  Its `traffic` (HBM bytes per
launch) is read from the committed rocprofv3 counter summary when that
summary was taken from the current kernel sources, else null.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-grouped]
       [--no-cpu] [--no-extra] [--only-step] [--copy-probe]
"""
import hashlib
import re
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MXFP8_TFLOPS = 5033.2     # 256 CU x 2.4 GHz x 8192 FLOP/clk/CU (dense)
PEAK_FP8_TFLOPS = 5033.2
PEAK_MXFP4_TFLOPS = 10066.3
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 FLOP/clk/CU (dense)
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "dense_mxfp8_nt_psb_llm_shapes_counters.txt")
CSRC = os.path.join(ROOT, "block_scaled_precision_03_amd", "csrc")
KERNEL_SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hpp", ".hip")))
C3_CASES = [("fwd", 0, 8192, 11008, 4096), ("dgrad", 1, 8192, 4096, 11008),
            ("wgrad", 2, 11008, 4096, 8192)]
C2_SHAPES = [(4096, 4096, 4096), (4096, 14336, 4096), (4096, 4096, 14336),
             (16384, 4096, 4096), (16384, 14336, 4096), (16384, 4096, 14336)]
C4_SHAPES = [(128, 2048, 7168), (1024, 2048, 7168), (16384, 2048, 7168),
             (128, 7168, 2304), (1024, 7168, 2304), (16384, 7168, 2304)]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-grouped", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--only-step", action="store_true",
                    help="time the MXFP8 step only (for profiler runs)")
    ap.add_argument("--plain-b", action="store_true", help="time with plain (not preshuffled) B")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the tensor-wise FP8 and MXFP4 measurements")
    ap.add_argument("--profile-leg", choices=("grouped", "grouped_bf16", "mxfp4", "mx_backward", "tensorwise"),
                    help="only launch one leg's kernels, three times per shape (no graphs, no "
                         "cold rotation): the short program a profiler's counter passes run")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 256 MiB read + 256 MiB write elementwise kernel "
                         "(the calibration of the HBM byte counters)")
    return ap.parse_args()


def kernel_source_hash():
    """SHA-256 of the kernel sources' code: comments and blank lines are
    dropped, so that editing a comment does not void a measurement but any
    change to the code does."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, encoding="utf-8") as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            line = line.split("//", 1)[0].rstrip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()


def committed_traffic():
    """HBM bytes per launch of the MXFP8 kernel from the committed counter
    summary, if it was taken from the current kernel sources."""
    try:
        kv = {}
        with open(TRAFFIC_SUMMARY) as fh:
            for line in fh:
                if ":" in line:
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_probe(torch):
    """A plain elementwise kernel of known traffic: y = -x over 256 MiB of
    FP32 reads 256 MiB and writes 256 MiB per launch."""
    n = 64 << 20
    x = torch.randn(n, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(5):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe": True, "read_bytes": 4 * n, "write_bytes": 4 * n,
                      "launches": 5}), flush=True)


def c2_inputs(torch, synth, mxgemm, dev, preshuffle):
    """Quantized operands of the six GEMMs (X shared by the two M values)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    xs = {}
    for ki, K in enumerate((4096, 14336)):
        x = synth.normal(synth.seed_for(2, 1, ki), (16384, K))
        q, s = synth.quant_mx(x, "e4m3")
        xs[K] = (t(q), t(s))
        del x
    ws = {}
    for wi, (N, K) in enumerate(((4096, 4096), (14336, 4096), (4096, 14336))):
        w = synth.normal(synth.seed_for(2, 2, wi), (N, K), 0.02)
        q, s = synth.quant_mx(w, "e4m3")
        qd, sd = t(q), t(s)
        if preshuffle:
            qp = torch.empty(mxgemm.preshuffle_b_bytes(mxgemm.MXFP8_E4M3, N, K), dtype=torch.uint8, device=dev)
            sp = torch.empty(mxgemm.preshuffle_scales_bytes(N, K), dtype=torch.uint8, device=dev)
            mxgemm.preshuffle_b(mxgemm.MXFP8_E4M3, mxgemm.NT, qd, qp, N, K)
            mxgemm.preshuffle_scales(sd, sp, N, K)
            qd, sd = qp, sp
        ws[(N, K)] = (qd, sd, q, s)
        del w
    torch.cuda.synchronize()
    return xs, ws


def time_step(torch, mxgemm, calls, steps, warmup):
    """Run `calls` (list of closures) per step; per-launch HIP events on the
    launch stream.  Returns (ms_per_step, per-call mean ms, wall seconds,
    [steps, calls] per-launch ms)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        for c in calls:
            c()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in calls] for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for s in range(steps):
        for i, c in enumerate(calls):
            ev[s][i][0].record(stream)
            c()
            ev[s][i][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)
    per = np.array([[a.elapsed_time(b) for a, b in row] for row in ev])
    return total_ms / steps, per.mean(axis=0), wall, per


def grouped_bench(torch, synth, mxgemm, dev, reps=50):
    """µs per call for the six grouped G=8 shapes (preshuffled weights):
    warm (back-to-back calls) and cold (weights rotated through > 256 MB)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    out = []
    G = 8
    for si, (totM, N, K) in enumerate(C4_SHAPES):
        m_sizes = synth.m_sizes_for(totM, G, synth.seed_for(4, 4, si))
        x = synth.normal(synth.seed_for(4, 1, si), (totM, K))
        xq, xsc = synth.quant_group_act(x, m_sizes)
        w = synth.normal(synth.seed_for(4, 2, si), (G, N, K), 0.02)
        wq, wsc = synth.quant_group_weight(w)
        del x, w
        dm, dx, dxs, dws = t(m_sizes), t(xq), t(xsc), t(wsc)
        wplain = t(wq)
        copies = max(1, int(np.ceil(300e6 / wq.nbytes)) + 1)
        wps = []
        for _ in range(copies):
            wp = torch.empty_like(wplain)
            mxgemm.grouped_preshuffle_b(G, wplain, wp, N, K)
            wps.append(wp)
        D = torch.empty((totM, N), dtype=torch.bfloat16, device=dev)
        res = {"totM": totM, "N": N, "K": K, "m_sizes": [int(v) for v in m_sizes]}
        for name, W, pre in (("plain", wplain, False), ("preshuffled", wps[0], True)):
            call = lambda: mxgemm.grouped_run(G, dm, dx, dxs, W, dws, D, totM, N, K, b_preshuffled=pre)
            for _ in range(5):
                call()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                call()
            b.record()
            torch.cuda.synchronize()
            res[name + "_us"] = a.elapsed_time(b) * 1000.0 / reps
        # graph replay (the pages quote replay latency): one captured call,
        # replayed with per-replay events; its output must equal the eager one
        call_pre = lambda: mxgemm.grouped_run(G, dm, dx, dxs, wps[0], dws, D, totM, N, K,
                                              b_preshuffled=True)
        call_pre()
        torch.cuda.synchronize()
        eager = D.clone()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                call_pre()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call_pre()
        D.zero_()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(100)]
        for _ in range(10):
            graph.replay()
        for ea, eb in evs:
            ea.record()
            graph.replay()
            eb.record()
        torch.cuda.synchronize()
        rep_us = np.array([ea.elapsed_time(eb) * 1000.0 for ea, eb in evs])
        res["graph_replay_us"] = {"median": float(np.median(rep_us)), "p10": float(np.percentile(rep_us, 10)),
                                  "p90": float(np.percentile(rep_us, 90))}
        res["graph_replay_matches_eager"] = bool(torch.equal(D.view(torch.int16), eager.view(torch.int16)))
        # ten calls per graph: the per-call time with the graph launch amortized
        graph10 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph10):
            for _ in range(10):
                call_pre()
        for _ in range(3):
            graph10.replay()
        torch.cuda.synchronize()
        ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ea.record()
        for _ in range(20):
            graph10.replay()
        eb.record()
        torch.cuda.synchronize()
        res["graph_replay_x10_us_per_call"] = ea.elapsed_time(eb) * 1000.0 / 200
        del graph, graph10, eager
        # cold: rotate through weight copies totalling > 256 MB
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        n = 0
        for r in range(reps):
            W = wps[r % copies]
            mxgemm.grouped_run(G, dm, dx, dxs, W, dws, D, totM, N, K, b_preshuffled=True)
            n += 1
        b.record()
        torch.cuda.synchronize()
        res["preshuffled_cold_us"] = a.elapsed_time(b) * 1000.0 / n
        flops = 2.0 * totM * N * K
        nonempty = int(np.count_nonzero(m_sizes))
        hbm = totM * K + nonempty * N * K + 4 * totM * K / 128 + 4 * G * (N / 128) * (K / 128) + 2 * totM * N + 8 * G
        best = min(res["plain_us"], res["preshuffled_us"])
        res["tflops_best_warm"] = flops / (best * 1e-6) / 1e12
        res["algo_bytes"] = hbm
        res["gbs_cold"] = hbm / (res["preshuffled_cold_us"] * 1e-6) / 1e9
        out.append(res)
        res["kernel"] = ["persistent 64x64", "persistent 256x256 (dense pipeline)", "persistent 128x128"][mxgemm.grouped_variant(G, totM, N, K)]
        log("grouped %s: plain %.1f us, preshuffled %.1f us, graph replay median %.1f us (p10 %.1f, p90 %.1f%s), "
            "10-call graph %.1f us/call, cold %.1f us (%.0f GB/s) [%s]" % (
                (totM, N, K), res["plain_us"], res["preshuffled_us"], res["graph_replay_us"]["median"],
                res["graph_replay_us"]["p10"], res["graph_replay_us"]["p90"],
                "" if res["graph_replay_matches_eager"] else ", REPLAY OUTPUT DIFFERS",
                res["graph_replay_x10_us_per_call"], res["preshuffled_cold_us"], res["gbs_cold"], res["kernel"]))
        del wps, wplain, dx, D
        torch.cuda.empty_cache()
    return out


def time_calls(torch, call, reps=20, warmup=3):
    """Mean µs per launch of `call` over `reps` launches (HIP events on the
    launch stream)."""
    for _ in range(warmup):
        call()
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1000.0 / reps


def grouped_bf16_bench(torch, synth, mxgemm, dev, reps=30):
    """BF16 grouped GEMM at the six grouped shapes (G = 8, the grouped
    benchmark's m_sizes): us per call warm, plain and preshuffled weights,
    and cold (weights rotated over > 256 MB), with TFLOP/s against the
    published dense BF16 peak and the algorithmic bytes' rate."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    out = []
    G = 8
    for si, (totM, N, K) in enumerate(C4_SHAPES):
        m_sizes = synth.m_sizes_for(totM, G, synth.seed_for(4, 4, si))
        X = t(synth.bf16_bits(synth.normal(synth.seed_for(8, 1, si), (totM, K))).view(np.int16))
        Wplain = t(synth.bf16_bits(synth.normal(synth.seed_for(8, 2, si), (G, N, K), 0.02)).view(np.int16))
        dm = t(m_sizes)
        copies = max(1, int(np.ceil(300e6 / (Wplain.numel() * 2))) + 1)
        wps = []
        for _ in range(copies):
            wp = torch.empty_like(Wplain)
            mxgemm.grouped_bf16_preshuffle_b(G, Wplain, wp, N, K)
            wps.append(wp)
        D = torch.empty((totM, N), dtype=torch.bfloat16, device=dev)
        res = {"totM": totM, "N": N, "K": K}
        for name, W, pre in (("plain", Wplain, False), ("preshuffled", wps[0], True)):
            res[name + "_us"] = time_calls(torch, lambda: mxgemm.grouped_bf16_run(G, dm, X, W, D, totM, N, K,
                                                                                 b_preshuffled=pre), reps=reps)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for r in range(reps):
            mxgemm.grouped_bf16_run(G, dm, X, wps[r % copies], D, totM, N, K, b_preshuffled=True)
        b.record()
        torch.cuda.synchronize()
        res["preshuffled_cold_us"] = a.elapsed_time(b) * 1000.0 / reps
        nonempty = int(np.count_nonzero(m_sizes))
        algo = 2 * totM * K + 2 * nonempty * N * K + 2 * totM * N
        best = min(res["plain_us"], res["preshuffled_us"])
        res["tflops_best_warm"] = 2.0 * totM * N * K / (best * 1e-6) / 1e12
        res["pct_bf16_peak"] = 100.0 * res["tflops_best_warm"] / PEAK_BF16_TFLOPS
        res["algo_bytes"] = algo
        res["gbs_cold"] = algo / (res["preshuffled_cold_us"] * 1e-6) / 1e9
        out.append(res)
        log("grouped bf16 %s: plain %.1f us, preshuffled %.1f us (%.0f TFLOP/s, %.1f%% of BF16 peak), cold %.1f us "
            "(%.0f GB/s)" % ((totM, N, K), res["plain_us"], res["preshuffled_us"], res["tflops_best_warm"],
                             res["pct_bf16_peak"], res["preshuffled_cold_us"], res["gbs_cold"]))
        del wps, Wplain, X, D
        torch.cuda.empty_cache()
    return out


def small_bench(torch, synth, mxgemm, dev):
    """MXFP8 NT 256 x 256 x 256: launch- and latency-bound, so µs per call,
    not a fraction of peak.  Two figures: back-to-back launches from the
    host (each call's host-side launch included), and 20 calls captured in
    one HIP graph and replayed (the device-side cost per call, as the pages
    quote their grouped GEMMs); the graph's output is checked against the
    eager call's."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    M = N = K = 256
    qa, sa = synth.quant_mx(synth.normal(synth.seed_for(1, 1), (M, K)), "e4m3")
    qb, sb = synth.quant_mx(synth.normal(synth.seed_for(1, 2), (N, K)), "e4m3")
    A, SA, B, SB = t(qa), t(sa), t(qb), t(sb)
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    call = lambda: mxgemm.run(mxgemm.MXFP8_E4M3, mxgemm.MXFP8_E4M3, mxgemm.NT, A, SA, B, SB, D, M, N, K)
    us = time_calls(torch, call, reps=200, warmup=20)
    call()
    torch.cuda.synchronize()
    eager = D.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    calls = 20
    with torch.cuda.graph(graph):
        for _ in range(calls):
            call()
    D.zero_()
    torch.cuda.synchronize()
    g_us = time_calls(torch, graph.replay, reps=20, warmup=3) / calls
    same = bool(torch.equal(D.view(torch.int16), eager.view(torch.int16)))
    kernel = ["persistent 256x256", "64x64 tiles"][mxgemm.dense_variant(mxgemm.MXFP8_E4M3, mxgemm.MXFP8_E4M3,
                                                                        mxgemm.NT, M, N, K)]
    log("mxfp8 256^3: %.2f us per call (back-to-back launches), %.2f us per call in a %d-call graph "
        "(output %s the eager call's) [%s]" % (us, g_us, calls, "equals" if same else "DIFFERS FROM", kernel))
    return {"M": M, "N": N, "K": K, "us": us, "graph_us_per_call": g_us, "graph_output_equal": same,
            "kernel": kernel, "tflops": 2.0 * M * N * K / (g_us * 1e-6) / 1e12}


def tensorwise_bench(torch, synth, mxgemm, dev):
    """Tensor-wise FP8 (FP32 per-tensor scales) GEMMs of a 4096 -> 11008
    linear layer at 8192 tokens in its three layouts, each with both format
    assignments: E4M3 A x E5M2 B, and E5M2 A x E4M3 B (for the data and
    weight gradients A is the gradient, E5M2 in hybrid FP8 training)."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    out = []
    fmt = {"e4m3": mxgemm.FP8_E4M3_TENSOR, "e5m2": mxgemm.FP8_E5M2_TENSOR}
    for idx, (name, layout, M, N, K) in enumerate(C3_CASES):
        a = synth.normal(synth.seed_for(3, 1, idx), (M, K))
        b = synth.normal(synth.seed_for(3, 2, idx), (N, K), 0.02)
        for ea, eb in (("e4m3", "e5m2"), ("e5m2", "e4m3")):
            qa, sa = synth.quant_tensor(a, ea)
            qb, sb = synth.quant_tensor(b, eb)
            if layout == mxgemm.TN:
                qa = qa.T
            if layout in (mxgemm.NN, mxgemm.TN):
                qb = qb.T
            A, B = t(qa), t(qb)
            SA, SB = t(np.array([sa], np.float32)), t(np.array([sb], np.float32))
            D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            us = time_calls(torch, lambda: mxgemm.run(fmt[ea], fmt[eb], layout, A, SA, B, SB, D, M, N, K))
            tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
            out.append({"name": name, "layout": ["NT", "NN", "TN"][layout], "A": ea, "B": eb,
                        "M": M, "N": N, "K": K, "us": us, "tflops": tf,
                        "pct_peak": 100.0 * tf / PEAK_FP8_TFLOPS})
            log("tensor-wise %s %s %s x %s (%d,%d,%d): %.1f us, %.0f TFLOP/s (%.1f%% of FP8 peak)" % (
                name, out[-1]["layout"], ea, eb, M, N, K, us, tf, 100.0 * tf / PEAK_FP8_TFLOPS))
            del A, B, D
        del a, b
    torch.cuda.empty_cache()
    return out


def mx_backward_bench(torch, synth, mxgemm, dev):
    """MXFP8 data and weight gradients of the same 4096 -> 11008 linear layer
    (E8M0 per 32 values along each GEMM's K): dgrad NN 8192 x 4096 x 11008
    and wgrad TN 11008 x 4096 x 8192, the gradient dY in E5M2, weights and
    activations in E4M3."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    out = []
    for idx, (name, layout, M, N, K) in enumerate(C3_CASES):
        if layout == mxgemm.NT:
            continue
        a = synth.normal(synth.seed_for(6, 1, idx), (M, K))
        b = synth.normal(synth.seed_for(6, 2, idx), (N, K), 0.02 if name == "dgrad" else 1.0)
        qa, sa = synth.quant_mx(a, "e5m2")
        qb, sb = synth.quant_mx(b, "e4m3")
        if layout == mxgemm.TN:
            qa = qa.T
        qb = qb.T
        A, SA, B, SB = t(qa), t(sa), t(qb), t(sb)
        D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        us = time_calls(torch, lambda: mxgemm.run(mxgemm.MXFP8_E5M2, mxgemm.MXFP8_E4M3, layout, A, SA, B, SB,
                                                  D, M, N, K))
        tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
        out.append({"name": name, "layout": ["NT", "NN", "TN"][layout], "A": "e5m2", "B": "e4m3",
                    "M": M, "N": N, "K": K, "us": us, "tflops": tf, "pct_peak": 100.0 * tf / PEAK_MXFP8_TFLOPS})
        log("mxfp8 %s %s (%d,%d,%d): %.1f us, %.0f TFLOP/s (%.1f%% of MXFP8 peak)" % (
            name, out[-1]["layout"], M, N, K, us, tf, out[-1]["pct_peak"]))
        del A, B, D, a, b
    torch.cuda.empty_cache()
    return out


def quant_bench(torch, synth, mxgemm, dev):
    """The on-device quantizers at the workloads' shapes: MX E4M3 and
    tensor-wise E4M3 of the [16384, 4096] activation, groupwise E4M3 of the grouped
    GEMM's [16384, 7168] activation (G = 8, per-group block scales) and of its
    [8, 2048, 7168] weights (128 x 128 blocks).
    HBM-bound: algorithmic bytes = 4 per value read + 1 per code + scales."""
    out = []
    x = torch.from_numpy(synth.normal(synth.seed_for(2, 1, 0), (16384, 4096))).to(dev)
    codes = torch.empty((16384, 4096), dtype=torch.uint8, device=dev)
    scales = torch.empty((16384, 128), dtype=torch.uint8, device=dev)
    us = time_calls(torch, lambda: mxgemm.quantize_mx(mxgemm.MXFP8_E4M3, x, codes, scales, 16384, 4096))
    nbytes = 16384 * 4096 * 5 + 16384 * 128
    out.append({"name": "quantize_mx e4m3", "rows": 16384, "K": 4096, "us": us, "bytes": nbytes,
                "gbs": nbytes / us / 1e3, "pct_hbm": 100.0 * nbytes / us / 1e3 / PEAK_HBM_GBS})
    # tensor-wise E4M3 of the same activation: the data is read twice (amax,
    # then encode), but the algorithmic bytes count it once
    tscale = torch.empty((1,), dtype=torch.float32, device=dev)
    us = time_calls(torch, lambda: mxgemm.quantize_tensor(mxgemm.FP8_E4M3_TENSOR, x, codes, tscale, 16384 * 4096))
    nbytes = 16384 * 4096 * 5 + 4
    out.append({"name": "quantize_tensor e4m3", "rows": 16384, "K": 4096, "us": us, "bytes": nbytes,
                "gbs": nbytes / us / 1e3, "pct_hbm": 100.0 * nbytes / us / 1e3 / PEAK_HBM_GBS})
    del x, codes, scales, tscale
    totM, K = 16384, 7168
    ms = torch.from_numpy(synth.m_sizes_for(totM, 8, synth.seed_for(4, 4, 2))).to(dev)
    x = torch.from_numpy(synth.normal(synth.seed_for(4, 1, 2), (totM, K))).to(dev)
    codes = torch.empty((totM, K), dtype=torch.uint8, device=dev)
    xs = torch.empty((totM * K // 128,), dtype=torch.float32, device=dev)
    us = time_calls(torch, lambda: mxgemm.grouped_quantize_act(8, ms, x, codes, xs, totM, K))
    nbytes = totM * K * 5 + totM * K // 128 * 4 + 8 * 8
    out.append({"name": "grouped_quantize_act e4m3 G=8", "rows": totM, "K": K, "us": us, "bytes": nbytes,
                "gbs": nbytes / us / 1e3, "pct_hbm": 100.0 * nbytes / us / 1e3 / PEAK_HBM_GBS})
    del x, codes, xs
    G, N = 8, 2048
    w = torch.from_numpy(synth.normal(synth.seed_for(4, 2, 2), (G, N, K), 0.02)).to(dev)
    codes = torch.empty((G, N, K), dtype=torch.uint8, device=dev)
    xs = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device=dev)
    us = time_calls(torch, lambda: mxgemm.grouped_quantize_weight(G, w, codes, xs, N, K))
    nbytes = G * N * K * 5 + G * (N // 128) * (K // 128) * 4
    out.append({"name": "grouped_quantize_weight e4m3 G=8", "rows": G * N, "K": K, "us": us, "bytes": nbytes,
                "gbs": nbytes / us / 1e3, "pct_hbm": 100.0 * nbytes / us / 1e3 / PEAK_HBM_GBS})
    del w
    for r in out:
        log("%s [%d, %d]: %.1f us, %.0f GB/s (%.1f%% of HBM)" % (r["name"], r["rows"], r["K"], r["us"], r["gbs"],
                                                                r["pct_hbm"]))
    del codes, xs
    torch.cuda.empty_cache()
    return out


def preshuffle_bench(torch, synth, mxgemm, dev):
    """The one-time weight shuffles, outside every timed GEMM: MXFP8 B codes
    and E8M0 scales of the 14336 x 4096 weight of the LLM shapes, MXFP4 B of
    8192^3, and the grouped [8, 2048, 7168] E4M3 weights.  Byte permutations:
    algorithmic bytes = bytes read + bytes written."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    out = []

    def one(name, call, nbytes):
        us = time_calls(torch, call)
        out.append({"name": name, "us": us, "bytes": nbytes, "gbs": nbytes / us / 1e3,
                    "pct_hbm": 100.0 * nbytes / us / 1e3 / PEAK_HBM_GBS})
        log("%s: %.1f us, %.0f GB/s" % (name, us, nbytes / us / 1e3))

    N, K = 14336, 4096
    q, s = synth.quant_mx(synth.normal(synth.seed_for(2, 2, 1), (N, K), 0.02), "e4m3")
    qd, sd = t(q), t(s)
    qp = torch.empty(mxgemm.preshuffle_b_bytes(mxgemm.MXFP8_E4M3, N, K), dtype=torch.uint8, device=dev)
    sp = torch.empty(mxgemm.preshuffle_scales_bytes(N, K), dtype=torch.uint8, device=dev)
    one("preshuffle_b e4m3 [14336, 4096]", lambda: mxgemm.preshuffle_b(mxgemm.MXFP8_E4M3, mxgemm.NT, qd, qp, N, K),
        N * K + qp.numel())
    one("preshuffle_scales [14336, 4096/32]", lambda: mxgemm.preshuffle_scales(sd, sp, N, K), N * K // 32 + sp.numel())
    del qd, sd, qp, sp
    N = K = 8192
    q, s = synth.quant_mx(synth.normal(synth.seed_for(5, 2), (N, K)), "e2m1")
    qd = t(q)
    qp = torch.empty(mxgemm.preshuffle_b_bytes(mxgemm.MXFP4_E2M1, N, K), dtype=torch.uint8, device=dev)
    one("preshuffle_b e2m1 [8192, 8192]", lambda: mxgemm.preshuffle_b(mxgemm.MXFP4_E2M1, mxgemm.NT, qd, qp, N, K),
        N * K // 2 + qp.numel())
    del qd, qp
    G, N, K = 8, 2048, 7168
    wq, _ = synth.quant_group_weight(synth.normal(synth.seed_for(4, 2, 0), (G, N, K), 0.02))
    wd = t(wq)
    wp = torch.empty_like(wd)
    one("grouped_preshuffle_b e4m3 [8, 2048, 7168]", lambda: mxgemm.grouped_preshuffle_b(G, wd, wp, N, K),
        2 * G * N * K)
    del wd, wp
    torch.cuda.empty_cache()
    return out


def mfma_ceiling(torch, mxgemm, dev):
    """What the scaled matrix-core instruction sustains with nothing else
    running (FP8 and FP4 operands), and the shader clock meanwhile."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {}
    for name, fmt, iters in (("fp8", mxgemm.MXFP8_E4M3, 20000), ("fp4", mxgemm.MXFP4_E2M1, 40000)):
        clk = torch.zeros(3, dtype=torch.int64, device=dev)
        mxgemm.mfma_ceiling(fmt, 200, clk)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        mxgemm.mfma_ceiling(fmt, iters, clk)
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1000.0
        flops = float(cus) * 8 * iters * 32 * 2 * 16 * 16 * 128
        ticks, ref = [int(v) for v in clk[:2].cpu()]
        mhz = 100.0 * ticks / ref if ref else None
        peak = PEAK_MXFP4_TFLOPS if name == "fp4" else PEAK_MXFP8_TFLOPS
        out[name] = {"tflops": flops / (us * 1e-6) / 1e12, "shader_clock_mhz": mhz,
                     "pct_of_published_peak": 100.0 * flops / (us * 1e-6) / 1e12 / peak}
        log("MFMA ceiling %s: %.0f TFLOP/s (%.1f%% of the published peak), shader clock %s MHz" % (
            name, out[name]["tflops"], out[name]["pct_of_published_peak"],
            "%.0f" % mhz if mhz else "n/a"))
    return out


def mxfp4_bench(torch, synth, mxgemm, dev):
    """MXFP4 NT GEMM, M = N = K = 8192, preshuffled B."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    M = N = K = 8192
    qa, sa = synth.quant_mx(synth.normal(synth.seed_for(5, 1), (M, K)), "e2m1")
    qb, sb = synth.quant_mx(synth.normal(synth.seed_for(5, 2), (N, K)), "e2m1")
    A, SA, Bp, SBp = t(qa), t(sa), t(qb), t(sb)
    B = torch.empty(mxgemm.preshuffle_b_bytes(mxgemm.MXFP4_E2M1, N, K), dtype=torch.uint8, device=dev)
    SB = torch.empty(mxgemm.preshuffle_scales_bytes(N, K), dtype=torch.uint8, device=dev)
    mxgemm.preshuffle_b(mxgemm.MXFP4_E2M1, mxgemm.NT, Bp, B, N, K)
    mxgemm.preshuffle_scales(SBp, SB, N, K)
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    us = time_calls(torch, lambda: mxgemm.run(mxgemm.MXFP4_E2M1, mxgemm.MXFP4_E2M1 | mxgemm.PRESHUFFLED,
                                              mxgemm.NT, A, SA, B, SB, D, M, N, K))
    tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
    log("mxfp4 8192^3: %.1f us, %.0f TFLOP/s (%.1f%% of FP4 peak)" % (us, tf, 100.0 * tf / PEAK_MXFP4_TFLOPS))
    del B
    # the backward layouts on the same logical operands: B stored [K, N]
    # (NN), and A stored [K, M] too (TN), packed along the rows
    layouts = []
    BT = t(synth.transpose_e2m1(qb))
    AT = t(synth.transpose_e2m1(qa))
    for layout, a_op in ((mxgemm.NN, A), (mxgemm.TN, AT)):
        ul = time_calls(torch, lambda: mxgemm.run(mxgemm.MXFP4_E2M1, mxgemm.MXFP4_E2M1, layout, a_op, SA, BT, SBp,
                                                  D, M, N, K))
        tl = 2.0 * M * N * K / (ul * 1e-6) / 1e12
        name = ["NT", "NN", "TN"][layout]
        layouts.append({"layout": name, "us": ul, "tflops": tl, "pct_peak": 100.0 * tl / PEAK_MXFP4_TFLOPS})
        log("mxfp4 %s 8192^3: %.1f us, %.0f TFLOP/s (%.1f%% of FP4 peak)" % (name, ul, tl, 100.0 * tl / PEAK_MXFP4_TFLOPS))
    del A, AT, BT, D
    torch.cuda.empty_cache()
    return {"M": M, "N": N, "K": K, "us": us, "tflops": tf, "pct_peak": 100.0 * tf / PEAK_MXFP4_TFLOPS,
            "backward_layouts": layouts}


def fused_bench(torch, synth, mxgemm, dev):
    """The forward GEMM of a linear layer with its epilogue: MXFP8 NT
    16384 x 14336 x 4096, preshuffled B, + bias and GELU (tanh form) or
    SiLU, fused into the kernel (mxgemm_run_fused) against the plain GEMM
    followed by torch's bias add and activation on the BF16 output."""
    import torch.nn.functional as F
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    M, N, K = 16384, 14336, 4096
    qa, sa = synth.quant_mx(synth.normal(synth.seed_for(2, 1, 0), (M, K)), "e4m3")
    qb, sb = synth.quant_mx(synth.normal(synth.seed_for(2, 2, 1), (N, K), 0.02), "e4m3")
    A, SA = t(qa), t(sa)
    fB = mxgemm.MXFP8_E4M3 | mxgemm.PRESHUFFLED
    B = torch.empty(mxgemm.preshuffle_b_bytes(mxgemm.MXFP8_E4M3, N, K), dtype=torch.uint8, device=dev)
    SB = torch.empty(mxgemm.preshuffle_scales_bytes(N, K), dtype=torch.uint8, device=dev)
    mxgemm.preshuffle_b(mxgemm.MXFP8_E4M3, mxgemm.NT, t(qb), B, N, K)
    mxgemm.preshuffle_scales(t(sb), SB, N, K)
    bias = (torch.randn(N, device=dev, generator=torch.Generator(device=dev).manual_seed(7)) * 0.5).to(torch.bfloat16)
    D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    plain = lambda: mxgemm.run(mxgemm.MXFP8_E4M3, fB, mxgemm.NT, A, SA, B, SB, D, M, N, K)
    res = {"M": M, "N": N, "K": K, "gemm_us": time_calls(torch, plain)}
    for name, act, tf in (("gelu_tanh", mxgemm.ACT_GELU_TANH, lambda y: F.gelu(y, approximate="tanh")),
                          ("silu", mxgemm.ACT_SILU, F.silu)):
        fused = lambda: mxgemm.run_fused(mxgemm.MXFP8_E4M3, fB, mxgemm.NT, A, SA, B, SB, D, M, N, K,
                                         bias=bias, activation=act)

        def unfused():
            plain()
            tf(D + bias)
        res[name] = {"fused_us": time_calls(torch, fused), "unfused_us": time_calls(torch, unfused)}
        log("fused epilogue bias + %s (16384,14336,4096): fused %.1f us, GEMM alone %.1f us, "
            "GEMM + torch bias and activation %.1f us"
            % (name, res[name]["fused_us"], res["gemm_us"], res[name]["unfused_us"]))
    del A, B, D
    torch.cuda.empty_cache()
    return res


def profile_leg(torch, synth, mxgemm, dev, leg, launches=3):
    """Launch one leg's kernels `launches` times per shape, in a fixed order
    (for counter collection: the dispatches of each kernel and shape are
    consecutive), and print the order as one JSON line."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    order = []
    if leg == "grouped":
        G = 8
        for si, (totM, N, K) in enumerate(C4_SHAPES):
            m_sizes = synth.m_sizes_for(totM, G, synth.seed_for(4, 4, si))
            xq, xsc = synth.quant_group_act(synth.normal(synth.seed_for(4, 1, si), (totM, K)), m_sizes)
            wq, wsc = synth.quant_group_weight(synth.normal(synth.seed_for(4, 2, si), (G, N, K), 0.02))
            W = t(wq)
            Wp = torch.empty_like(W)
            mxgemm.grouped_preshuffle_b(G, W, Wp, N, K)
            torch.cuda.synchronize()
            dm, dx, dxs, dws = t(m_sizes), t(xq), t(xsc), t(wsc)
            D = torch.empty((totM, N), dtype=torch.bfloat16, device=dev)
            for _ in range(launches):
                mxgemm.grouped_run(G, dm, dx, dxs, Wp, dws, D, totM, N, K, b_preshuffled=True)
            torch.cuda.synchronize()
            order.append({"totM": totM, "N": N, "K": K, "G": G,
                          "nonempty_groups": int((m_sizes > 0).sum()),
                          "variant": mxgemm.grouped_variant(G, totM, N, K, True)})
    elif leg == "grouped_bf16":
        G = 8
        for si, (totM, N, K) in enumerate(C4_SHAPES):
            m_sizes = synth.m_sizes_for(totM, G, synth.seed_for(4, 4, si))
            X = t(synth.bf16_bits(synth.normal(synth.seed_for(8, 1, si), (totM, K))).view(np.int16))
            W = t(synth.bf16_bits(synth.normal(synth.seed_for(8, 2, si), (G, N, K), 0.02)).view(np.int16))
            Wp = torch.empty_like(W)
            mxgemm.grouped_bf16_preshuffle_b(G, W, Wp, N, K)
            dm = t(m_sizes)
            D = torch.empty((totM, N), dtype=torch.bfloat16, device=dev)
            torch.cuda.synchronize()
            for _ in range(launches):
                mxgemm.grouped_bf16_run(G, dm, X, Wp, D, totM, N, K, b_preshuffled=True)
            torch.cuda.synchronize()
            order.append({"totM": totM, "N": N, "K": K, "G": G, "nonempty_groups": int((m_sizes > 0).sum())})
    elif leg == "mxfp4":
        M = N = K = 8192
        qa, sa = synth.quant_mx(synth.normal(synth.seed_for(5, 1), (M, K)), "e2m1")
        qb, sb = synth.quant_mx(synth.normal(synth.seed_for(5, 2), (N, K)), "e2m1")
        B = torch.empty(mxgemm.preshuffle_b_bytes(mxgemm.MXFP4_E2M1, N, K), dtype=torch.uint8, device=dev)
        SB = torch.empty(mxgemm.preshuffle_scales_bytes(N, K), dtype=torch.uint8, device=dev)
        mxgemm.preshuffle_b(mxgemm.MXFP4_E2M1, mxgemm.NT, t(qb), B, N, K)
        mxgemm.preshuffle_scales(t(sb), SB, N, K)
        A, SA = t(qa), t(sa)
        D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        torch.cuda.synchronize()
        for _ in range(launches):
            mxgemm.run(mxgemm.MXFP4_E2M1, mxgemm.MXFP4_E2M1 | mxgemm.PRESHUFFLED, mxgemm.NT, A, SA, B, SB, D, M, N, K)
        torch.cuda.synchronize()
        order.append({"M": M, "N": N, "K": K, "fmt": "e2m1", "layout": "NT"})
        del B
        AT, BT, SBp = t(synth.transpose_e2m1(qa)), t(synth.transpose_e2m1(qb)), t(sb)
        for layout, a_op in ((mxgemm.NN, A), (mxgemm.TN, AT)):
            for _ in range(launches):
                mxgemm.run(mxgemm.MXFP4_E2M1, mxgemm.MXFP4_E2M1, layout, a_op, SA, BT, SBp, D, M, N, K)
            torch.cuda.synchronize()
            order.append({"M": M, "N": N, "K": K, "fmt": "e2m1", "layout": ["NT", "NN", "TN"][layout]})
    elif leg == "mx_backward":
        for idx, (name, layout, M, N, K) in enumerate(C3_CASES):
            if layout == mxgemm.NT:
                continue
            qa, sa = synth.quant_mx(synth.normal(synth.seed_for(6, 1, idx), (M, K)), "e5m2")
            qb, sb = synth.quant_mx(synth.normal(synth.seed_for(6, 2, idx), (N, K),
                                                 0.02 if name == "dgrad" else 1.0), "e4m3")
            if layout == mxgemm.TN:
                qa = qa.T
            A, SA, B, SB = t(qa), t(sa), t(qb.T), t(sb)
            D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            torch.cuda.synchronize()
            for _ in range(launches):
                mxgemm.run(mxgemm.MXFP8_E5M2, mxgemm.MXFP8_E4M3, layout, A, SA, B, SB, D, M, N, K)
            torch.cuda.synchronize()
            order.append({"name": name, "layout": ["NT", "NN", "TN"][layout], "M": M, "N": N, "K": K})
    elif leg == "tensorwise":
        for idx, (name, layout, M, N, K) in enumerate(C3_CASES):
            x = synth.normal(synth.seed_for(3, 1, idx), (M, K))
            w = synth.normal(synth.seed_for(3, 2, idx), (N, K), 0.02 if name != "wgrad" else 1.0)
            qa, sa = synth.quant_tensor(x, "e5m2")
            qb, sb = synth.quant_tensor(w, "e4m3")
            if layout == mxgemm.TN:
                qa = qa.T
            if layout != mxgemm.NT:
                qb = qb.T
            A, B = t(qa), t(qb)
            SA, SB = t(np.array([sa], np.float32)), t(np.array([sb], np.float32))
            D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
            torch.cuda.synchronize()
            for _ in range(launches):
                mxgemm.run(mxgemm.FP8_E5M2_TENSOR, mxgemm.FP8_E4M3_TENSOR, layout, A, SA, B, SB, D, M, N, K)
            torch.cuda.synchronize()
            order.append({"name": name, "layout": ["NT", "NN", "TN"][layout], "M": M, "N": N, "K": K})
    print(json.dumps({"profile_leg": leg, "launches_per_shape": launches, "order": order}), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def bf16_bits_to_f64(u16):
    return (u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def cpu_baseline(synth, gpu_bits=None, target_s=12.0):
    """The FP64 oracle, as it stands, on rows [0, R) of the M=16384,
    N=4096, K=4096 MXFP8 GEMM (dequantize + plain FP64 dot products).
    gpu_bits: the BF16 bits of the timed step's result for that GEMM (same
    seeded inputs); its rows [0, R) are checked against the oracle's."""
    import oracle
    N = K = 4096
    x = synth.normal(synth.seed_for(2, 1, 0), (16384, K))
    w = synth.normal(synth.seed_for(2, 2, 0), (N, K), 0.02)
    qb, sb = synth.quant_mx(w, "e4m3")
    opB = (oracle.E4M3, oracle.SCALE_MX, 0, qb, sb)
    def run(rows):
        qa, sa = synth.quant_mx(x[:rows], "e4m3")
        t0 = time.perf_counter()
        D = oracle.gemm((oracle.E4M3, oracle.SCALE_MX, 0, qa, sa), opB, rows, N, K)
        return time.perf_counter() - t0, D
    # size the sample from a probe, and once more from the first sample if
    # the probe (thread start-up included) misjudged it by more than 2x
    probe_rows = 128
    tp, _ = run(probe_rows)
    rows = int(max(probe_rows, min(16384, probe_rows * target_s / max(tp, 1e-3))))
    rows = max(16, rows // 16 * 16)
    dt, D = run(rows)
    if dt < 0.5 * target_s and rows < 16384:
        rows = max(16, int(min(16384, rows * target_s / max(dt, 1e-3))) // 16 * 16)
        dt, D = run(rows)
    flops = 2.0 * rows * N * K
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    res = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "sample": "rows 0..%d of the M=16384 N=4096 K=4096 MXFP8 NT GEMM (FP64 dequant + "
                     "dot products), %.1f s" % (rows, dt),
           "seconds": dt, "cpu_model": cpu_model()}
    if gpu_bits is not None:
        ok, worst = oracle.within_tolerance(bf16_bits_to_f64(gpu_bits[:rows]), D)
        res["parity"] = {"rows": rows, "worst_ratio": worst, "pass": ok,
                         "bound": "|d-ref| <= 2^-7|ref| + 1e-3 max|ref| (max over the sampled rows)"}
    return res


_SINGLE_THREAD = r'''
import json, sys, time
sys.path.insert(0, sys.argv[1])
import oracle
from block_scaled_precision_03_amd import synth
x = synth.normal(synth.seed_for(1, 1), (256, 256))
w = synth.normal(synth.seed_for(1, 2), (256, 256))
qa, sa = synth.quant_mx(x, "e4m3")
qb, sb = synth.quant_mx(w, "e4m3")
t0 = time.perf_counter()
oracle.gemm((oracle.E4M3, oracle.SCALE_MX, 0, qa, sa), (oracle.E4M3, oracle.SCALE_MX, 0, qb, sb), 256, 256, 256)
t1 = time.perf_counter() - t0
G, totM, N, K = 8, 128, 2048, 7168
ms = synth.m_sizes_for(totM, G, synth.seed_for(4, 4, 0))
xq, xs = synth.quant_group_act(synth.normal(synth.seed_for(4, 1, 0), (totM, K)), ms)
wq, ws = synth.quant_group_weight(synth.normal(synth.seed_for(4, 2, 0), (G, N, K), 0.02))
t0 = time.perf_counter()
oracle.grouped_gemm(ms, xq, xs, wq, ws, totM, N, K)
t4 = time.perf_counter() - t0
print(json.dumps({"mxfp8_256_cube_s": t1, "grouped_totM128_2048x7168_s": t4}))
'''


def cpu_single_thread_start():
    """Starts the oracle on one thread (OMP_NUM_THREADS=1) in a child process
    that never touches the GPU: the MXFP8 256^3 GEMM and the grouped G=8,
    totM=128, N=2048, K=7168 GEMM, contraction time only.  It runs beside the
    GPU legs (one host core) and is collected before the all-core sample."""
    import subprocess
    env = dict(os.environ, OMP_NUM_THREADS="1")
    return subprocess.Popen([sys.executable, "-c", _SINGLE_THREAD, ROOT], env=env,
                            stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def cpu_single_thread_collect(proc):
    import subprocess
    try:
        out, err = proc.communicate(timeout=300)
        if proc.returncode != 0:
            return {"error": err.strip()[-200:]}
        return json.loads(out.strip().splitlines()[-1])
    except (subprocess.SubprocessError, ValueError, IndexError) as exc:
        proc.kill()
        proc.communicate()
        return {"error": str(exc)[:200]}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_probe:
        copy_probe(torch)
        return
    from block_scaled_precision_03_amd import mxgemm, synth
    dev = "cuda:0"
    torch.cuda.set_device(0)
    mxgemm.init()
    if args.profile_leg:
        profile_leg(torch, synth, mxgemm, dev, args.profile_leg)
        return
    pre = not args.plain_b
    log("generating MXFP8 inputs ...")
    t0 = time.perf_counter()
    xs, ws = c2_inputs(torch, synth, mxgemm, dev, pre)
    log("inputs ready in %.1f s" % (time.perf_counter() - t0))
    fmtB = mxgemm.MXFP8_E4M3 | (mxgemm.PRESHUFFLED if pre else 0)
    outs = {}
    calls = []
    flops = []
    for (M, N, K) in C2_SHAPES:
        qa, sa = xs[K]
        qa, sa = qa[:M], sa[:M]
        qb, sb = ws[(N, K)][:2]
        D = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        outs[(M, N, K)] = D
        calls.append((lambda qa=qa, sa=sa, qb=qb, sb=sb, D=D, M=M, N=N, K=K:
                      mxgemm.run(mxgemm.MXFP8_E4M3, fmtB, mxgemm.NT, qa, sa, qb, sb, D, M, N, K)))
        flops.append(2.0 * M * N * K)
    log("timing %d steps (+%d warmup) ..." % (args.steps, args.warmup))
    ms, per_ms, wall, per_all = time_step(torch, mxgemm, calls, args.steps, args.warmup)
    step_flops = sum(flops)
    value = step_flops / (ms * 1e-3) / 1e12
    kernel_ms = float(per_ms.sum())
    achieved = step_flops / (kernel_ms * 1e-3) / 1e12
    per_gemm = []
    for i, (shape, f, pm) in enumerate(zip(C2_SHAPES, flops, per_ms)):
        tf = f / (pm * 1e-3) / 1e12
        col = per_all[:, i] * 1000.0
        per_gemm.append({"M": shape[0], "N": shape[1], "K": shape[2], "us": pm * 1000.0,
                         "us_median": float(np.median(col)), "us_p10": float(np.percentile(col, 10)),
                         "us_p90": float(np.percentile(col, 90)),
                         "tflops": tf, "pct_peak": 100.0 * tf / PEAK_MXFP8_TFLOPS})
        log("  %s: %.1f us, %.0f TFLOP/s (%.1f%% of peak)" % (shape, pm * 1000, tf, 100 * tf / PEAK_MXFP8_TFLOPS))
    log("step: %.3f ms -> %.0f TFLOP/s" % (ms, value))
    result = {
        "metric": "MXFP8 NT GEMM TFLOP/s + % MFMA peak; grouped FP8 GEMM us/call (G=8)",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3 x fp8_e4m3 (E8M0/32 scales), fp32 acc, bf16 out",
        "data": "synthetic (seeded N(0,1) activations, 0.02*N(0,1) weights, quantized on the host)",
        "config": {"workload": "MXFP8 NT GEMM, LLM shapes: M in {4096,16384} x (N,K) in "
                               "{(4096,4096),(14336,4096),(4096,14336)}; one step = the 6 GEMMs",
                   "b_preshuffled": pre, "layout": "NT"},
        "pct_mfma_peak": 100.0 * value / PEAK_MXFP8_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_MXFP8_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_MXFP8_TFLOPS,
                     "traffic": committed_traffic() if pre else None,
                     "kernel": "dense_kernel<E4M3,E4M3,MX,NT,preshuffled B>" if pre else
                               "dense_kernel<E4M3,E4M3,MX,NT>",
                     "launches_per_step": len(C2_SHAPES),
                     "mean_launch_us": kernel_ms * 1000.0 / len(C2_SHAPES),
                     "flops_per_launch": step_flops / len(C2_SHAPES),
                     "kernel_ms_per_step": kernel_ms},
        "per_gemm": per_gemm,
    }
    # the timed step's result of the M=16384 N=K=4096 GEMM, for the check in
    # the CPU leg (the oracle runs on the same seeded inputs)
    check_bits = None
    if not args.only_step and not args.no_cpu:
        check_bits = outs[(16384, 4096, 4096)].view(torch.int16).cpu().numpy().view(np.uint16)
    del outs, calls, xs, ws
    torch.cuda.empty_cache()
    single = None
    if not args.only_step and not args.no_cpu:
        single = cpu_single_thread_start()
    if not args.only_step and not args.no_grouped:
        log("grouped G=8 ...")
        result["grouped"] = grouped_bench(torch, synth, mxgemm, dev)
    if not args.only_step and not args.no_extra:
        result["mxfp8_256"] = small_bench(torch, synth, mxgemm, dev)
        log("tensor-wise FP8 ...")
        result["tensorwise_fp8"] = tensorwise_bench(torch, synth, mxgemm, dev)
        log("MXFP8 backward layouts ...")
        result["mxfp8_backward"] = mx_backward_bench(torch, synth, mxgemm, dev)
        log("quantizers ...")
        result["quantizers"] = quant_bench(torch, synth, mxgemm, dev)
        log("MXFP4 ...")
        result["mxfp4"] = mxfp4_bench(torch, synth, mxgemm, dev)
        log("fused epilogue ...")
        result["fused_epilogue"] = fused_bench(torch, synth, mxgemm, dev)
        log("BF16 grouped ...")
        result["grouped_bf16"] = grouped_bf16_bench(torch, synth, mxgemm, dev)
        log("weight preshuffles ...")
        result["preshuffle"] = preshuffle_bench(torch, synth, mxgemm, dev)
        result["mfma_ceiling"] = mfma_ceiling(torch, mxgemm, dev)
        result["roofline"]["frac_of_mfma_ceiling"] = (
            result["roofline"]["achieved"] / result["mfma_ceiling"]["fp8"]["tflops"])
    if not args.only_step and not args.no_cpu:
        log("CPU oracle, one thread (C1 256^3, grouped totM=128) ...")
        single = cpu_single_thread_collect(single)
        log("CPU oracle sample ...")
        result["cpu_baseline"] = cpu_baseline(synth, check_bits)
        del check_bits
        result["cpu_baseline"]["single_thread"] = single
        log("cpu baseline: %.4g TFLOP/s on %d threads" % (result["cpu_baseline"]["value"],
                                                          result["cpu_baseline"]["cores"]))
        par = result["cpu_baseline"].get("parity")
        if par is not None:
            log("step result vs oracle, rows 0..%d: worst ratio %.3g, %s"
                % (par["rows"], par["worst_ratio"], "pass" if par["pass"] else "FAIL"))
            if not par["pass"]:
                # a wrong result has no throughput: the line says so and the
                # process fails
                result["parity_failed"] = True
                result["value_if_valid"] = result["value"]
                result["value"] = None
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)
    if result.get("parity_failed"):
        sys.exit(3)


if __name__ == "__main__":
    main()
