#!/usr/bin/env python3
"""Benchmark of the weight-only-quantized SwiGLU MLP on one MI355X.

Headline (the JSON line's value): FP8 E4M3 per-channel W8A16 SwiGLU MLP decode
at hidden 5120 / intermediate 17408, M=1, bf16 activations -- effective weight
GB/s (weight + scale bytes per step / step time).  A step is one full MLP
forward (gate+up projection with SwiGLU, then the down projection).

Method (the routed-expert pull request's "Operator results" protocol, adapted):
all inputs are resident in HBM before timing; K steps are captured into one
hipGraph, each step reading the next of R weight copies so that the working set
(R x 267.5 MB) exceeds the 256 MB Infinity Cache; the replay is bracketed by a
device synchronisation and HIP events on the launch stream.  Per-kernel times
come from each stage captured alone into a graph of K launches over the same
rotating weights, timed the same way.

Extras measured the same way: NVFP4 decode, NVFP4 prefill at M=512 and 8192
(MFMA utilisation), both formats at a short batch (M=8) and FP8 at M=512 on the
MFMA path, and the AWQ routed-expert step (hot and rotating experts).
Opt-in extra "dense_f16": torch's own float16 matmul on the same prefill shapes
(unquantized weights; context for the MFMA fraction, not part of the path).
The CPU oracle is timed on the host on a bounded sample as a baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--extras all|none|a,b]
"""
import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective weight GB/s + tok/s, quantized SwiGLU MLP, M=1 decode & M=512 prefill"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
H, I = 5120, 17408


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--extras", default="all")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle baseline sample")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--counters", type=int, default=0,
                    help="only run this many plain (non-graph) headline steps, for rocprofv3 --pmc passes")
    ap.add_argument("--prefill-counters", type=int, default=0,
                    help="only run this many plain NVFP4 M=512 prefill steps, for rocprofv3 --pmc passes")
    ap.add_argument("--decode-counters", type=int, default=0,
                    help="only run this many plain NVFP4 M=1 decode steps (8 rotating weight copies), for rocprofv3")
    ap.add_argument("--fp8-prefill-counters", type=int, default=0,
                    help="only run this many plain FP8 M=512 prefill steps (bf16 x, 2 weight copies), for rocprofv3")
    ap.add_argument("--awq-counters", type=int, default=0,
                    help="only run this many plain routed-expert steps over rotating experts, for rocprofv3")
    ap.add_argument("--json-out", default=None)
    return ap.parse_args()


# ---- timing helpers ------------------------------------------------------------------------------
class GraphBench:
    """Capture fn(i) for i in range(K) into one graph on a side stream and time replays."""

    def __init__(self, torch, fn, K):
        self.torch = torch
        self.K = K
        self.stream = torch.cuda.Stream()
        s = self.stream
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn(0)                             # allocator/attribute warm-up outside capture
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph, stream=s):
            for i in range(K):
                fn(i)
        torch.cuda.synchronize()

    def replay_timed(self):
        """One replay on the graph's own stream, bracketed by synchronisation and two HIP
        events on that stream; returns seconds."""
        t = self.torch
        e0 = t.cuda.Event(enable_timing=True)
        e1 = t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        with t.cuda.stream(self.stream):
            e0.record(self.stream)
            self.graph.replay()
            e1.record(self.stream)
        t.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3


def fp8_batch(torch, wq, synth, d, M, K, copies):
    """FP8 MLP on M rows of the decode config's weights (path AUTO), R rotating weight copies."""
    dev = torch.device("cuda:0")
    names = ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down")
    base = [torch.from_numpy(d[n]).to(dev) for n in names]
    sets = [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
    import numpy as np
    xb = synth.to_bf16_bits(synth.rng(2, synth.T_X, (M,)).standard_normal((M, H), dtype=np.float32))
    x = torch.from_numpy(xb.view("int16")).to(dev).view(torch.bfloat16)
    out = torch.empty((M, H), dtype=torch.float32, device=dev)
    ws = torch.empty(wq.mlp_workspace_bytes(wq.WQ_FMT_FP8W, M, H, I), dtype=torch.uint8, device=dev)

    def step(i, stage=None):
        wq.mlp_fp8w_run(x, *sets[i % copies], out=out, workspace=ws, stage=stage)

    step(0)
    torch.cuda.synchronize()
    g = GraphBench(torch, step, K)
    g.replay_timed()
    t = g.replay_timed()
    gu_ms, dn_ms = stage_times(torch, step, K)
    return dict(t=t, K=K, M=M, gu_ms=gu_ms, dn_ms=dn_ms, copies=copies)


def stage_times(torch, step, K):
    """Mean per-launch durations (ms) of the gate/up and the down kernels.

    Each stage is captured on its own into a graph of K launches (same rotating
    weights as the full steps) and timed by HIP events around its replay on the
    launch stream.  (Events recorded inside a captured graph do not give usable
    durations on this runtime.)
    """
    res = []
    for which in ("gateup", "down"):
        g = GraphBench(torch, lambda i, w=which: step(i, w), K)
        g.replay_timed()
        res.append(g.replay_timed() / K * 1e3)
    return res[0], res[1]


def sha256_file(p):
    h = hashlib.sha256()
    with open(p, "rb") as f:
        for chunk in iter(lambda: f.read(1 << 20), b""):
            h.update(chunk)
    return h.hexdigest()


def read_traffic(name, src_files):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, or None if stale/missing."""
    p = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(p):
        return None
    kv = {}
    for line in open(p):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    want = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in src_files)).hexdigest()
    if kv.get("source_sha256") != want or "traffic_bytes_per_launch" not in kv:
        return None
    return float(kv["traffic_bytes_per_launch"])


# ---- workloads -------------------------------------------------------------------------------------
def fp8_decode(torch, wq, synth, K, W, copies=4):
    dev = torch.device("cuda:0")
    d = synth.fp8_mlp(M=1)
    names = ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down")
    base = [torch.from_numpy(d[n]).to(dev) for n in names]
    sets = [base] + [[t.clone() for t in base] for _ in range(copies - 1)]
    x = torch.from_numpy(d["x_bits"].view("int16")).to(dev).view(torch.bfloat16)
    out = torch.empty((1, H), dtype=torch.float32, device=dev)
    ws = torch.empty(wq.mlp_workspace_bytes(wq.WQ_FMT_FP8W, 1, H, I), dtype=torch.uint8, device=dev)

    def step(i, stage=None):
        wq.mlp_fp8w_run(x, *sets[i % copies], out=out, workspace=ws, stage=stage)

    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    g = GraphBench(torch, step, K)
    g.replay_timed()                                  # untimed warm replay
    t = g.replay_timed()
    gu_ms, dn_ms = stage_times(torch, step, K)
    wbytes = 3 * H * I + 4 * (2 * I + H)
    gu_alg = 2 * H * I + 4 * 2 * I + 2 * H + 4 * I      # gate+up codes+scales, x read, act write
    dn_alg = H * I + 4 * H + 4 * I + 4 * H              # down codes+scales, act read, out write
    return dict(t=t, K=K, M=1, gu_ms=gu_ms, dn_ms=dn_ms, wbytes=wbytes, gu_alg=gu_alg,
                dn_alg=dn_alg, copies=copies, data=d)


def nvfp4_weights(torch, wq, synth, dev):
    """Config-3 weights packed into Block64 records by the library's own packer on the device."""
    w = synth.nvfp4_mlp_weights()
    blk = {n: wq.nvfp4_pack_block64(torch.from_numpy(w["wp_" + n]).to(dev), torch.from_numpy(w["ws_" + n]).to(dev))
           for n in ("gate", "up", "down")}
    gs = {n: float(w["gs_" + n]) for n in ("gate", "up", "down")}
    torch.cuda.synchronize()
    return blk, gs


def nvfp4_run(torch, wq, synth, blk, gs, M, K, copies, outlier):
    dev = torch.device("cuda:0")
    sets = [blk] + [{n: t.clone() for n, t in blk.items()} for _ in range(copies - 1)]
    xb, _ = synth.nvfp4_x(M, outlier_frac=outlier)
    x = torch.from_numpy(xb.view("int16")).to(dev).view(torch.bfloat16)
    out = torch.empty((M, H), dtype=torch.float32, device=dev)
    ws = torch.empty(wq.mlp_workspace_bytes(wq.WQ_FMT_NVFP4, M, H, I), dtype=torch.uint8, device=dev)

    def step(i, stage=None):
        b = sets[i % copies]
        wq.mlp_nvfp4_run(x, b["gate"], gs["gate"], b["up"], gs["up"], b["down"], gs["down"], out=out, workspace=ws,
                         stage=stage)

    step(0)
    torch.cuda.synchronize()
    g = GraphBench(torch, step, K)
    g.replay_timed()
    t = g.replay_timed()
    gu_ms, dn_ms = stage_times(torch, step, K)
    return dict(t=t, K=K, M=M, gu_ms=gu_ms, dn_ms=dn_ms, copies=copies)


def awq_run(torch, wq, synth, K, calls=0, layout=3):
    """Routed-expert step, hot and rotating experts, timed as graphs of K steps; with calls > 0 only that
    many plain rotating-expert steps are run (for rocprofv3)."""
    dev = torch.device("cuda:0")
    d = synth.awq_moe()
    E, topk, HH, II = 512, 10, 2560, 160
    def bank(codes, scales, zeros):   # the library's packer, on the device
        return wq.awq_pack_bank(torch.from_numpy(codes).to(dev), torch.from_numpy(scales.view("int16")).to(dev),
                                torch.from_numpy(zeros).to(dev), layout)
    b13 = bank(*d["w13"])
    b2 = bank(*d["w2"])
    torch.cuda.synchronize()
    x = torch.from_numpy(d["x_bits"].view("int16")).to(dev).view(torch.float16)
    rw = torch.from_numpy(d["router_w"]).to(dev)
    hot = torch.from_numpy(d["ids"]).to(dev)
    rot = [torch.from_numpy(r).to(dev) for r in synth.awq_rotating_ids(48, topk, E)]
    act = torch.empty((topk, II), dtype=torch.float16, device=dev)
    out = torch.empty((HH,), dtype=torch.float16, device=dev)
    if calls:
        for i in range(calls):
            wq.moe_awq_m1_run(x, rot[i % len(rot)], rw, b13, b2, E, II, layout, act=act, out=out)
        torch.cuda.synchronize()
        return dict(calls=calls)
    res = {}
    for mode in ("hot", "rotating"):
        def step(i, mode=mode):
            ids = hot if mode == "hot" else rot[i % len(rot)]
            wq.moe_awq_m1_run(x, ids, rw, b13, b2, E, II, layout, act=act, out=out)
        step(0)
        torch.cuda.synchronize()
        g = GraphBench(torch, step, K)
        g.replay_timed()
        res[mode] = g.replay_timed() / K
    step_bytes = topk * (2 * II * HH // 2 + layout * 2 * II * HH // 32 + HH * II // 2 + layout * HH * II // 32)
    return dict(hot_s=res["hot"], rot_s=res["rotating"], step_bytes=step_bytes, K=K)


def dense_f16_ref(torch, M, K):
    """torch float16 matmuls of the prefill shapes with unquantized weights: [M,H] x [2I,H]^T (gate and up
    as one matrix) and [M,I] x [H,I]^T; context for the MFMA fraction of the quantized GEMMs."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(7)
    x = torch.randn(M, H, device=dev, dtype=torch.float16, generator=g)
    wgu = torch.randn(2 * I, H, device=dev, dtype=torch.float16, generator=g) * 0.02
    wd = torch.randn(H, I, device=dev, dtype=torch.float16, generator=g) * 0.02
    a = torch.randn(M, I, device=dev, dtype=torch.float16, generator=g)
    y1 = torch.empty(M, 2 * I, device=dev, dtype=torch.float16)
    y2 = torch.empty(M, H, device=dev, dtype=torch.float16)

    def step():
        torch.matmul(x, wgu.t(), out=y1)
        torch.matmul(a, wd.t(), out=y2)
    for _ in range(3):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(K):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    del x, wgu, wd, a, y1, y2
    return ms


def cpu_baseline(oracle, d, budget_s):
    """The oracle as it stands, on this host, on the headline workload (full calls)."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:
        blas = 1
    names = ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down")
    x64 = oracle.bf16_bits_to_f64(d["x_bits"])
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.mlp_fp8w_ref(x64, *(d[k] for k in names))
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el / n * (n + 1) > budget_s * 1.5:
            break
    per = el / n
    wbytes = 3 * H * I + 4 * (2 * I + H)
    return dict(value=round(wbytes / per / 1e9, 4), unit="GB/s", cores=int(blas), kind="oracle",
                sample=f"{n} full oracle calls (E4M3 decode + float64 SwiGLU MLP) of the 5120x17408 M=1 "
                       f"FP8 workload, {per:.2f} s per call = {1.0 / per:.3f} tok/s; "
                       f"{len(os.sched_getaffinity(0))} host cores visible")


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU; runs over several GPUs are not supported (each MI355X would run "
              "the same kernels on its own shard of the intermediate dimension). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    import synth
    import weight_quantized_mlp_amd as wq

    wq.lib()
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')} CUs {props.multi_processor_count}")

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy done: 3 x 1 GiB device-to-device")
        return

    if args.counters:
        d = synth.fp8_mlp(M=1)
        names = ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down")
        base = [torch.from_numpy(d[n]).to(dev) for n in names]
        sets = [base] + [[t.clone() for t in base] for _ in range(3)]
        x = torch.from_numpy(d["x_bits"].view("int16")).to(dev).view(torch.bfloat16)
        out = torch.empty((1, H), dtype=torch.float32, device=dev)
        ws = torch.empty(wq.mlp_workspace_bytes(wq.WQ_FMT_FP8W, 1, H, I), dtype=torch.uint8, device=dev)
        for i in range(args.counters):
            wq.mlp_fp8w_run(x, *sets[i % 4], out=out, workspace=ws)
        torch.cuda.synchronize()
        log(f"counter steps done: {args.counters}")
        return

    if args.prefill_counters:
        blk, gs = nvfp4_weights(torch, wq, synth, dev)
        M = 512
        xb, _ = synth.nvfp4_x(M, outlier_frac=0.01)
        x = torch.from_numpy(xb.view("int16")).to(dev).view(torch.bfloat16)
        out = torch.empty((M, H), dtype=torch.float32, device=dev)
        ws = torch.empty(wq.mlp_workspace_bytes(wq.WQ_FMT_NVFP4, M, H, I), dtype=torch.uint8, device=dev)
        for _ in range(args.prefill_counters):
            wq.mlp_nvfp4_run(x, blk["gate"], gs["gate"], blk["up"], gs["up"], blk["down"], gs["down"], out=out,
                             workspace=ws)
        torch.cuda.synchronize()
        log(f"prefill counter steps done: {args.prefill_counters}")
        return

    if args.decode_counters:
        blk, gs = nvfp4_weights(torch, wq, synth, dev)
        sets = [blk] + [{n: t.clone() for n, t in blk.items()} for _ in range(7)]
        xb, _ = synth.nvfp4_x(1)
        x = torch.from_numpy(xb.view("int16")).to(dev).view(torch.bfloat16)
        out = torch.empty((1, H), dtype=torch.float32, device=dev)
        ws = torch.empty(wq.mlp_workspace_bytes(wq.WQ_FMT_NVFP4, 1, H, I), dtype=torch.uint8, device=dev)
        for i in range(args.decode_counters):
            b = sets[i % 8]
            wq.mlp_nvfp4_run(x, b["gate"], gs["gate"], b["up"], gs["up"], b["down"], gs["down"], out=out, workspace=ws)
        torch.cuda.synchronize()
        log(f"nvfp4 decode counter steps done: {args.decode_counters}")
        return

    if args.fp8_prefill_counters:
        import numpy as np
        d = synth.fp8_mlp(M=1)
        names = ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down")
        base = [torch.from_numpy(d[n]).to(dev) for n in names]
        sets = [base, [t.clone() for t in base]]
        M = 512
        xb = synth.to_bf16_bits(synth.rng(2, synth.T_X, (M,)).standard_normal((M, H), dtype=np.float32))
        x = torch.from_numpy(xb.view("int16")).to(dev).view(torch.bfloat16)
        out = torch.empty((M, H), dtype=torch.float32, device=dev)
        ws = torch.empty(wq.mlp_workspace_bytes(wq.WQ_FMT_FP8W, M, H, I), dtype=torch.uint8, device=dev)
        for i in range(args.fp8_prefill_counters):
            wq.mlp_fp8w_run(x, *sets[i % 2], out=out, workspace=ws)
        torch.cuda.synchronize()
        log(f"fp8 prefill counter steps done: {args.fp8_prefill_counters}")
        return

    if args.awq_counters:
        a = awq_run(torch, wq, synth, 48, calls=args.awq_counters)
        log(f"routed-expert counter steps done: {a['calls']}")
        return

    K, W = args.steps, args.warmup
    log(f"fp8 decode: K={K} W={W}")
    r = fp8_decode(torch, wq, synth, K, W)
    t = r["t"]
    gbs = r["wbytes"] * K / t / 1e9
    gu_gbs = r["gu_alg"] / (r["gu_ms"] / 1e3) / 1e9
    dn_gbs = r["dn_alg"] / (r["dn_ms"] / 1e3) / 1e9
    log(f"fp8 decode: {t / K * 1e6:.2f} us/step, {gbs:.1f} GB/s; gate/up {r['gu_ms'] * 1e3:.2f} us "
        f"({gu_gbs:.0f} GB/s), down {r['dn_ms'] * 1e3:.2f} us ({dn_gbs:.0f} GB/s)")
    traffic = read_traffic("fp8w_gateup_row_5120x17408_counters.txt",
                           ["weight_quantized_mlp_amd/csrc/gemv_fast.hip", "weight_quantized_mlp_amd/csrc/dev_common.h"])

    extras = {}
    want = set() if args.extras == "none" else (
        {"nvfp4_decode", "nvfp4_prefill_512", "nvfp4_prefill_8192", "nvfp4_batch8", "fp8_batch8", "fp8_prefill_512",
         "awq", "awq4"} if args.extras == "all"
        else set(args.extras.split(",")))
    if want & {"fp8_batch8", "fp8_prefill_512"}:
        fp8_bytes = 3 * H * I + 4 * (2 * I + H)
        for M, key, steps, copies in ((8, "fp8_batch8", 200, 4), (512, "fp8_prefill_512", 60, 2)):
            if key not in want:
                continue
            n = fp8_batch(torch, wq, synth, r["data"], M, steps, copies)
            tfl = 2.0 * M * 3 * H * I * n["K"] / n["t"] / 1e12
            extras[key] = dict(
                us_per_step=round(n["t"] / n["K"] * 1e6, 2), tok_per_s=round(M * n["K"] / n["t"], 1),
                weight_GBps=round(fp8_bytes * n["K"] / n["t"] / 1e9, 1), TFLOPs=round(tfl, 1),
                mfma_frac_f16_peak=round(tfl / MFMA_F16_PEAK_TFLOPS, 4), gateup_us=round(n["gu_ms"] * 1e3, 2),
                down_us=round(n["dn_ms"] * 1e3, 2), path="mfma", weight_copies=copies)
            log(key, extras[key])
    if want & {"nvfp4_decode", "nvfp4_prefill_512", "nvfp4_prefill_8192", "nvfp4_batch8"}:
        blk, gs = nvfp4_weights(torch, wq, synth, dev)
        nv_bytes = 3 * (H * I // 64 * 36)
        if "nvfp4_decode" in want:
            n = nvfp4_run(torch, wq, synth, blk, gs, 1, K, 8, 0.0)
            extras["nvfp4_decode_M1"] = dict(
                us_per_step=round(n["t"] / n["K"] * 1e6, 3), GBps=round(nv_bytes * n["K"] / n["t"] / 1e9, 1),
                tok_per_s=round(n["K"] / n["t"], 1), hbm_frac=round(nv_bytes * n["K"] / n["t"] / 1e9 / HBM_PEAK_GBS, 4),
                gateup_us=round(n["gu_ms"] * 1e3, 3), down_us=round(n["dn_ms"] * 1e3, 3), weight_copies=n["copies"])
            log("nvfp4 decode", extras["nvfp4_decode_M1"])
        if "nvfp4_batch8" in want:
            n = nvfp4_run(torch, wq, synth, blk, gs, 8, 200, 8, 0.0)
            extras["nvfp4_batch8"] = dict(
                us_per_step=round(n["t"] / n["K"] * 1e6, 2), tok_per_s=round(8 * n["K"] / n["t"], 1),
                weight_GBps=round(nv_bytes * n["K"] / n["t"] / 1e9, 1), gateup_us=round(n["gu_ms"] * 1e3, 2),
                down_us=round(n["dn_ms"] * 1e3, 2), path="mfma", weight_copies=n["copies"])
            log("nvfp4_batch8", extras["nvfp4_batch8"])
        for M, key, steps in ((512, "nvfp4_prefill_512", 60), (8192, "nvfp4_prefill_8192", 12)):
            if key not in want:
                continue
            n = nvfp4_run(torch, wq, synth, blk, gs, M, steps, 2, 0.01)
            flops = 2.0 * M * 3 * H * I
            tfl = flops * n["K"] / n["t"] / 1e12
            extras[key] = dict(
                ms_per_step=round(n["t"] / n["K"] * 1e3, 4), tok_per_s=round(M * n["K"] / n["t"], 1),
                TFLOPs=round(tfl, 1), mfma_frac_f16_peak=round(tfl / MFMA_F16_PEAK_TFLOPS, 4),
                gateup_ms=round(n["gu_ms"], 4), down_ms=round(n["dn_ms"], 4),
                gateup_mfma_frac=round(2.0 * M * 2 * H * I / (n["gu_ms"] / 1e3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                down_mfma_frac=round(2.0 * M * H * I / (n["dn_ms"] / 1e3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4))
            log(key, extras[key])
        del blk
    if "dense_f16" in want:
        for M, steps in ((512, 100), (8192, 12)):
            ms = dense_f16_ref(torch, M, steps)
            tfl = 2.0 * M * 3 * H * I / (ms / 1e3) / 1e12
            extras[f"torch_f16_matmul_{M}"] = dict(ms_per_step=round(ms, 4), TFLOPs=round(tfl, 1),
                                                   mfma_frac_f16_peak=round(tfl / MFMA_F16_PEAK_TFLOPS, 4))
            log(f"torch f16 matmul M={M}", extras[f"torch_f16_matmul_{M}"])
    if "awq4" in want:
        a = awq_run(torch, wq, synth, 480, layout=4)
        extras["awq_moe_m1_layout4"] = dict(
            hot_us_per_step=round(a["hot_s"] * 1e6, 3), rotating_us_per_step=round(a["rot_s"] * 1e6, 3),
            rotating_GBps=round(a["step_bytes"] / a["rot_s"] / 1e9, 1),
            hot_ms_per_48=round(a["hot_s"] * 48e3, 4), rotating_ms_per_48=round(a["rot_s"] * 48e3, 4),
            step_bytes=a["step_bytes"])
        log("awq layout 4", extras["awq_moe_m1_layout4"])
    if "awq" in want:
        a = awq_run(torch, wq, synth, 480)
        extras["awq_moe_m1"] = dict(
            hot_us_per_step=round(a["hot_s"] * 1e6, 3), rotating_us_per_step=round(a["rot_s"] * 1e6, 3),
            rotating_GBps=round(a["step_bytes"] / a["rot_s"] / 1e9, 1),
            hot_ms_per_48=round(a["hot_s"] * 48e3, 4), rotating_ms_per_48=round(a["rot_s"] * 48e3, 4),
            step_bytes=a["step_bytes"])
        log("awq", extras["awq_moe_m1"])

    torch.cuda.synchronize()
    log(f"cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
    import oracle   # the CPU baseline leg is the only part of the benchmark that uses the oracle
    cpu = cpu_baseline(oracle, r["data"], args.cpu_seconds)
    log("cpu", cpu)

    roof = dict(bound="hbm", kernel="fp8_gu_row (gate+up+SwiGLU) 5120x17408 M=1", achieved=round(gu_gbs, 1),
                peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gu_gbs / HBM_PEAK_GBS, 4),
                traffic=traffic, algorithmic_bytes_per_launch=r["gu_alg"],
                avg_launch_us=round(r["gu_ms"] * 1e3, 3),
                down_kernel=dict(achieved=round(dn_gbs, 1), avg_launch_us=round(r["dn_ms"] * 1e3, 3),
                                 algorithmic_bytes_per_launch=r["dn_alg"]))
    res = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(t / K * 1e3, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "fp8_e4m3_per_channel_w8a16_swiglu_mlp_decode", "hidden": H, "intermediate": I,
                   "M": 1, "x_dtype": "bf16", "weight_copies_rotated": r["copies"],
                   "timing": "hipGraph of K steps, HIP events on the launch stream"},
        "tok_per_s": round(K / t, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": roof, "cpu_baseline": cpu, "extra": extras,
    }
    line = json.dumps(res)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
