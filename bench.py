#!/usr/bin/env python3
"""Benchmark of the weight-only-quantized SwiGLU MLP on one MI355X.

Headline (the JSON line's value): FP8 E4M3 per-channel W8A16 SwiGLU MLP decode at hidden 5120 /
intermediate 17408, M=1, bf16 activations -- effective weight GB/s (weight + scale bytes per step /
step time).  A step is one full MLP forward: the gate+up projection with SwiGLU, then the down
projection.

Method (the routed-expert pull request's "Operator results": graph replays, 7 samples, medians; the
NVFP4 page's "Reproduction": binary, input and settings recorded): all inputs are resident in HBM
before timing; K steps are captured into one hipGraph, each step reading the next of R weight copies so
that the working set exceeds the 256 MB Infinity Cache; each replay is one sample, bracketed by a device
synchronisation and HIP events on the launch stream, and at least 7 samples are taken (median, min,
max reported; the value is the median).  Per-kernel times come from each stage captured alone into a
graph of K launches over the same rotating weights, timed the same way.  The routed-expert step is timed
exactly as the pull request's operator: graphs of 48 calls, hot (the same 10 experts) and rotating
(48 x 10 = 480 experts per replay), medians in ms per 48 calls.

Extras measured the same way: the tiny FP8 MLP (M = 1 and 4), NVFP4 decode, NVFP4 prefill at M=512 and
8192 (MFMA utilisation), both formats at a short batch (M=8), FP8 at M=512 on the MFMA path, the
routed-expert step with both metadata layouts, and the HBM read ceiling of a plain streaming kernel of
the library (wq_read_probe) at the kernels' byte counts.  Opt-in extra "dense_f16": torch's own float16
matmul on the same prefill shapes (unquantized weights; context for the MFMA fraction, not the path).
The CPU oracle is timed on the host on bounded samples of all five workloads, as a baseline only.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--samples S] [--extras all|none|a,b]
"""
import argparse
import hashlib
import json
import os
import platform
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective weight GB/s + tok/s, quantized SwiGLU MLP, M=1 decode & M=512 prefill"
HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
H, I = 5120, 17408
FP8_BYTES = 3 * H * I + 4 * (2 * I + H)          # codes + per-channel scales of one MLP
NV_BYTES = 3 * (H * I // 64 * 36)                 # Block64 records of one MLP
SOURCE_DIRS = ("include", "weight_quantized_mlp_amd", "oracle", "synth")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--samples", type=int, default=11, help="timed graph replays per measurement (at least 7)")
    ap.add_argument("--extras", default="all")
    ap.add_argument("--cpu-seconds", type=float, default=30.0, help="budget of the oracle baseline leg")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--counters", type=int, default=0,
                    help="only run this many plain (non-graph) headline steps, for rocprofv3 --pmc passes")
    ap.add_argument("--prefill-counters", type=int, default=0,
                    help="only run this many plain NVFP4 prefill steps (M from --prefill-m), for rocprofv3 passes")
    ap.add_argument("--prefill-m", type=int, default=512, help="rows of the --prefill-counters steps (512 or 8192)")
    ap.add_argument("--decode-counters", type=int, default=0,
                    help="only run this many plain NVFP4 M=1 decode steps (8 rotating weight copies), for rocprofv3")
    ap.add_argument("--fp8-prefill-counters", type=int, default=0,
                    help="only run this many plain FP8 M=512 prefill steps (bf16 x, 2 weight copies), for rocprofv3")
    ap.add_argument("--awq-counters", type=int, default=0,
                    help="only run this many plain routed-expert steps over rotating experts, for rocprofv3")
    ap.add_argument("--w4a8-counters", type=int, default=0,
                    help="run N plain W4A8 prefill steps (M=512) and exit (for rocprofv3)")
    ap.add_argument("--json-out", default=None)
    a = ap.parse_args()
    a.samples = max(7, a.samples)
    return a


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
        """One replay on the graph's own stream, bracketed by synchronisation and two HIP events on that
        stream; returns seconds."""
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


class Samples:
    """Per-step seconds of S timed replays of a K-step graph (one untimed warm replay first)."""

    def __init__(self, torch, fn, K, S):
        g = GraphBench(torch, fn, K)
        g.replay_timed()
        self.K = K
        self.per_step = [g.replay_timed() / K for _ in range(S)]
        del g

    @property
    def med(self):
        return statistics.median(self.per_step)

    def summary(self, scale=1e6, unit="us"):
        v = [t * scale for t in self.per_step]
        return {f"median_{unit}": round(statistics.median(v), 4), f"min_{unit}": round(min(v), 4),
                f"max_{unit}": round(max(v), 4), "samples": len(v), "steps_per_sample": self.K}


def stage_samples(torch, step, K, S):
    """Per-launch samples of the gate/up and the down kernels: each stage captured on its own into a graph
    of K launches over the same rotating weights, timed by HIP events around its replays on the launch
    stream.  (Events recorded inside a captured graph do not give usable durations on this runtime.)"""
    return [Samples(torch, lambda i, w=which: step(i, w), K, S) for which in ("gateup", "down")]


# ---- provenance ------------------------------------------------------------------------------------
def sha256_file(p):
    h = hashlib.sha256()
    with open(p, "rb") as f:
        for chunk in iter(lambda: f.read(1 << 20), b""):
            h.update(chunk)
    return h.hexdigest()


def source_tree_sha256():
    """SHA-256 over the path and bytes of every source file of the library, oracle and inputs, and of this
    script (sorted paths), so a run names the exact sources even where no git history is present."""
    files = [os.path.join(ROOT, "bench.py")]
    for d in SOURCE_DIRS:
        for dp, _, fs in os.walk(os.path.join(ROOT, d)):
            files += [os.path.join(dp, f) for f in fs
                      if f.endswith((".py", ".h", ".hip", ".cpp")) and "__pycache__" not in dp]
    h = hashlib.sha256()
    for p in sorted(files):
        h.update(os.path.relpath(p, ROOT).encode())
        h.update(open(p, "rb").read())
    return h.hexdigest()


def _run(cmd, timeout=20):
    try:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout)
        return r.stdout.strip() if r.returncode == 0 else None
    except Exception:
        return None


def clocks():
    """Current and available shader / memory clocks from the amdgpu sysfs files of the visible cards."""
    out = {}
    base = "/sys/class/drm"
    try:
        cards = sorted(c for c in os.listdir(base) if c.startswith("card") and "-" not in c)
    except OSError:
        return None
    for c in cards:
        for name in ("pp_dpm_sclk", "pp_dpm_mclk", "pp_dpm_fclk"):
            p = os.path.join(base, c, "device", name)
            if os.path.exists(p):
                try:
                    out.setdefault(c, {})[name] = open(p).read().split("\n")[:16]
                except OSError:
                    pass
    return out or None


def provenance(torch, wq, props):
    rocm = None
    for p in ("/opt/rocm/.info/version", "/opt/rocm/.info/version-dev"):
        if os.path.exists(p):
            rocm = open(p).read().strip()
            break
    hipcc = _run(["/opt/rocm/bin/hipcc", "--version"])
    return {
        "git_sha": _run(["git", "-C", ROOT, "rev-parse", "HEAD"]),
        "source_tree_sha256": source_tree_sha256(),
        "library": os.path.relpath(wq.lib_path, ROOT),
        "library_sha256": sha256_file(wq.lib_path),
        "abi_version": wq.wq_abi_version(),
        "rocm": rocm,
        "hipcc": hipcc.splitlines()[0] if hipcc else None,
        "torch": torch.__version__, "hip_runtime": getattr(torch.version, "hip", None),
        "python": platform.python_version(),
        "device": props.name, "gcnArchName": getattr(props, "gcnArchName", None),
        "compute_units": props.multi_processor_count,
        "clock_mhz_reported": getattr(props, "clock_rate", None),
        "clocks_sysfs": clocks(),
        "host_cpu": next((l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if l.startswith("model name")),
                         None) if os.path.exists("/proc/cpuinfo") else None,
        "host_cores_visible": len(os.sched_getaffinity(0)),
    }


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
FP8_NAMES = ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down")


def fp8_sets(torch, d, copies):
    dev = torch.device("cuda:0")
    base = [torch.from_numpy(d[n]).to(dev) for n in FP8_NAMES]
    return [base] + [[t.clone() for t in base] for _ in range(copies - 1)]


def fp8_step_fn(torch, wq, sets, x, M, Hh=H, Ii=I):
    dev = torch.device("cuda:0")
    out = torch.empty((M, Hh), dtype=torch.float32, device=dev)
    ws = torch.empty(max(1, wq.mlp_workspace_bytes(wq.WQ_FMT_FP8W, M, Hh, Ii)), dtype=torch.uint8, device=dev)

    def step(i, stage=None):
        wq.mlp_fp8w_run(x, *sets[i % len(sets)], out=out, workspace=ws, stage=stage)
    return step


def fp8_decode(torch, wq, synth, d, K, W, S, copies=4):
    dev = torch.device("cuda:0")
    sets = fp8_sets(torch, d, copies)
    x = torch.from_numpy(d["x_bits"].view("int16")).to(dev).view(torch.bfloat16)
    step = fp8_step_fn(torch, wq, sets, x, 1)
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    full = Samples(torch, step, K, S)
    gu, dn = stage_samples(torch, step, K, S)
    gu_alg = 2 * H * I + 4 * 2 * I + 2 * H + 4 * I      # gate+up codes+scales, x read, act write
    dn_alg = H * I + 4 * H + 4 * I + 4 * H              # down codes+scales, act read, out write
    del sets
    return dict(full=full, gu=gu, dn=dn, gu_alg=gu_alg, dn_alg=dn_alg, copies=copies)


def fp8_batch(torch, wq, synth, d, M, K, S, copies):
    """FP8 MLP on M rows of the decode config's weights (path AUTO), R rotating weight copies."""
    import numpy as np
    dev = torch.device("cuda:0")
    sets = fp8_sets(torch, d, copies)
    xb = synth.to_bf16_bits(synth.rng(2, synth.T_X, (M,)).standard_normal((M, H), dtype=np.float32))
    x = torch.from_numpy(xb.view("int16")).to(dev).view(torch.bfloat16)
    step = fp8_step_fn(torch, wq, sets, x, M)
    step(0)
    torch.cuda.synchronize()
    full = Samples(torch, step, K, S)
    gu, dn = stage_samples(torch, step, K, S)
    del sets
    return dict(full=full, gu=gu, dn=dn, M=M, copies=copies)


def fp8_tiny(torch, wq, synth, K, S):
    """Config 1: H=256, I=512, x float32, M = 1 and 4 (one weight copy: 0.4 MB, cache-resident)."""
    dev = torch.device("cuda:0")
    res = {}
    for M in (1, 4):
        d = synth.fp8_tiny(M)
        sets = fp8_sets(torch, d, 1)
        x = torch.from_numpy(d["x"]).to(dev)
        step = fp8_step_fn(torch, wq, sets, x, M, 256, 512)
        step(0)
        torch.cuda.synchronize()
        s = Samples(torch, step, K, S)
        res[f"M{M}"] = dict(us_per_step=round(s.med * 1e6, 3), tok_per_s=round(M / s.med, 1), **s.summary())
    return res


def nvfp4_weights(torch, wq, w, dev):
    """Config-3 weights packed into Block64 records by the library's own packer on the device."""
    blk = {n: wq.nvfp4_pack_block64(torch.from_numpy(w["wp_" + n]).to(dev), torch.from_numpy(w["ws_" + n]).to(dev))
           for n in ("gate", "up", "down")}
    gs = {n: float(w["gs_" + n]) for n in ("gate", "up", "down")}
    torch.cuda.synchronize()
    return blk, gs


def nvfp4_run(torch, wq, synth, blk, gs, M, K, S, copies, outlier, act=None):
    dev = torch.device("cuda:0")
    sets = [blk] + [{n: t.clone() for n, t in blk.items()} for _ in range(copies - 1)]
    xb, _ = synth.nvfp4_x(M, outlier_frac=outlier)
    x = torch.from_numpy(xb.view("int16")).to(dev).view(torch.bfloat16)
    out = torch.empty((M, H), dtype=torch.float32, device=dev)
    ws = torch.empty(wq.mlp_workspace_bytes(wq.WQ_FMT_NVFP4, M, H, I, "auto", act), dtype=torch.uint8, device=dev)

    def step(i, stage=None):
        b = sets[i % copies]
        wq.mlp_nvfp4_run(x, b["gate"], gs["gate"], b["up"], gs["up"], b["down"], gs["down"], out=out, workspace=ws,
                         stage=stage, act=act)

    step(0)
    torch.cuda.synchronize()
    full = Samples(torch, step, K, S)
    gu, dn = stage_samples(torch, step, K, S)
    del sets
    return dict(full=full, gu=gu, dn=dn, M=M, copies=copies)


def awq_banks(torch, wq, d, layout):
    dev = torch.device("cuda:0")

    def bank(codes, scales, zeros):   # the library's packer, on the device
        return wq.awq_pack_bank(torch.from_numpy(codes).to(dev), torch.from_numpy(scales.view("int16")).to(dev),
                                torch.from_numpy(zeros).to(dev), layout)
    b = (bank(*d["w13"]), bank(*d["w2"]))
    torch.cuda.synchronize()
    return b


def awq_run(torch, wq, synth, d, S, calls=0, layout=3):
    """Routed-expert step, hot and rotating experts, as graphs of 48 calls (S timed replays each); with
    calls > 0 only that many plain rotating-expert steps are run (for rocprofv3)."""
    dev = torch.device("cuda:0")
    E, topk, HH, II = 512, 10, 2560, 160
    b13, b2 = awq_banks(torch, wq, d, layout)
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
        res[mode] = Samples(torch, step, 48, S)
    step_bytes = topk * (2 * II * HH // 2 + layout * 2 * II * HH // 32 + HH * II // 2 + layout * HH * II // 32)
    return dict(hot=res["hot"], rot=res["rotating"], step_bytes=step_bytes)


def awq_extra(a):
    return dict(hot_ms_per_48=round(a["hot"].med * 48e3, 4), rotating_ms_per_48=round(a["rot"].med * 48e3, 4),
                hot_us_per_step=round(a["hot"].med * 1e6, 3), rotating_us_per_step=round(a["rot"].med * 1e6, 3),
                rotating_GBps=round(a["step_bytes"] / a["rot"].med / 1e9, 1), step_bytes=a["step_bytes"],
                hot=a["hot"].summary(1e3, "ms_per_call"), rotating=a["rot"].summary(1e3, "ms_per_call"),
                timing="graphs of 48 calls; hot: the same 10 experts, rotating: 480 experts per replay")


def read_ceiling(torch, wq, S):
    """Streaming-read rate of wq_read_probe at the kernels' byte counts, reading consecutive windows of a
    2 GiB buffer (each window read from HBM, not from the Infinity Cache); the best of several grid sizes."""
    dev = torch.device("cuda:0")
    buf = torch.ones(1 << 31, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    res = {}
    for name, nbytes in (("nvfp4_down_50MB", H * I // 64 * 36), ("nvfp4_gateup_100MB", 2 * H * I // 64 * 36),
                         ("fp8_down_89MB", H * I), ("fp8_gateup_178MB", 2 * H * I), ("1GiB", 1 << 30)):
        nbytes = nbytes // 4096 * 4096
        nwin = (1 << 31) // nbytes
        best = None
        for grid in (1024, 2048, 4096, 8192, 16384):
            def step(i, nbytes=nbytes, nwin=nwin, grid=grid):
                off = (i % nwin) * nbytes
                wq.wq_read_probe(buf[off:off + nbytes], sink, nbytes, grid)
            step(0)
            torch.cuda.synchronize()
            s = Samples(torch, step, max(nwin, 8), S)
            if best is None or s.med < best[1].med:
                best = (grid, s)
        grid, s = best
        gbs = nbytes / s.med / 1e9
        res[name] = dict(bytes=nbytes, us_per_launch=round(s.med * 1e6, 3), GBps=round(gbs, 1),
                         frac_of_8TBps=round(gbs / HBM_PEAK_GBS, 4), grid=grid)
    del buf
    return res


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


# ---- CPU baseline (the oracle, as it stands) -------------------------------------------------------
def _timed_calls(fn, budget_s, min_calls=1):
    n = 0
    t0 = time.perf_counter()
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if n >= min_calls and (el >= budget_s or el / n * (n + 1) > budget_s * 1.5):
            return n, el / n


def cpu_baseline(oracle, synth, data, budget_s):
    """The oracle timed on this host on bounded samples of the five workloads (decode included in every
    call: the oracle has no packed-format kernels).  Returns the headline (config 2) entry with the
    per-workload entries under "configs"."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        blas = max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"), default=1)
    except Exception:
        blas = 1
    cfg = {}
    # 1: tiny FP8, M = 1 and 4
    for M in (1, 4):
        d = synth.fp8_tiny(M)
        n, per = _timed_calls(lambda: oracle.mlp_fp8w_ref(d["x"], *(d[k] for k in FP8_NAMES)), 0.05 * budget_s)
        cfg[f"1_fp8_tiny_M{M}"] = dict(value=round(M / per, 1), unit="tok/s", seconds_per_call=round(per, 6),
                                       calls=n, sample=f"{n} full oracle calls, H=256, I=512, M={M}")
    # 2: FP8 decode (the headline workload)
    d = data["fp8"]
    x64 = oracle.bf16_bits_to_f64(d["x_bits"])
    n, per = _timed_calls(lambda: oracle.mlp_fp8w_ref(x64, *(d[k] for k in FP8_NAMES)), 0.25 * budget_s)
    cfg["2_fp8_decode_M1"] = dict(value=round(FP8_BYTES / per / 1e9, 4), unit="GB/s", tok_per_s=round(1 / per, 3),
                                  seconds_per_call=round(per, 3), calls=n,
                                  sample=f"{n} full oracle calls (E4M3 decode + float64 SwiGLU MLP), 5120x17408, M=1")
    # 3 and 4: NVFP4 decode, prefill M=512 whole, M=8192 on a 512-row slice holding its outlier rows
    w = data["nvfp4_w"]
    blk = {n: oracle.block64_pack(w["wp_" + n], w["ws_" + n]) for n in ("gate", "up", "down")}
    nv = lambda x: oracle.mlp_nvfp4_ref(x, blk["gate"], w["gs_gate"], blk["up"], w["gs_up"], blk["down"],
                                        w["gs_down"])
    xb, _ = synth.nvfp4_x(1)
    x1 = oracle.bf16_bits_to_f64(xb)
    n, per = _timed_calls(lambda: nv(x1), 0.1 * budget_s)
    cfg["3_nvfp4_decode_M1"] = dict(value=round(NV_BYTES / per / 1e9, 4), unit="GB/s", tok_per_s=round(1 / per, 3),
                                    seconds_per_call=round(per, 3), calls=n,
                                    sample=f"{n} full oracle calls (Block64 decode + float64 MLP), M=1")
    xb, _ = synth.nvfp4_x(512, outlier_frac=0.01)
    x512 = oracle.bf16_bits_to_f64(xb)
    n, per = _timed_calls(lambda: nv(x512), 0.1 * budget_s)
    cfg["4_nvfp4_prefill_M512"] = dict(value=round(512 / per, 2), unit="tok/s", seconds_per_call=round(per, 3),
                                       calls=n, sample=f"{n} full oracle calls, M=512 (5 outlier rows)")
    xb, rows = synth.nvfp4_x(8192, outlier_frac=0.01)
    rest = np.setdiff1d(np.arange(8192), rows)[: 512 - len(rows)]
    sl = np.sort(np.concatenate([rows, rest]))
    xs = oracle.bf16_bits_to_f64(xb[sl])
    n, per = _timed_calls(lambda: nv(xs), 0.1 * budget_s)
    cfg["4_nvfp4_prefill_M8192_slice512"] = dict(
        value=round(512 / per, 2), unit="tok/s", seconds_per_call=round(per, 3), calls=n,
        sample=f"{n} oracle calls on a 512-row slice of the M=8192 batch (all {len(rows)} outlier rows + "
               f"the first other rows); tok/s of the slice")
    # 5: routed-expert step
    m = data["awq"]
    n, per = _timed_calls(lambda: oracle.moe_awq_m1_ref(m["x_bits"], m["ids"], m["router_w"], m["w13"], m["w2"],
                                                         160), 0.1 * budget_s, 3)
    cfg["5_awq_moe_m1"] = dict(value=round(per * 48e3, 2), unit="ms per 48 calls", seconds_per_call=round(per, 4),
                               calls=n, sample=f"{n} oracle steps (10 experts decoded per step)")
    head = cfg["2_fp8_decode_M1"]
    return dict(value=head["value"], unit="GB/s", cores=int(blas), kind="oracle",
                sample=head["sample"] + f"; {head['seconds_per_call']} s per call = {head['tok_per_s']} tok/s; "
                       f"numpy BLAS threads {blas}, {len(os.sched_getaffinity(0))} host cores visible",
                configs=cfg)


# ---- counter-pass modes (plain launches, for rocprofv3 --pmc) -----------------------------------------
def counter_modes(args, torch, wq, synth, dev):
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration copy done: 3 x 1 GiB device-to-device")
        return True
    if args.counters:
        d = synth.fp8_mlp(M=1)
        sets = fp8_sets(torch, d, 4)
        x = torch.from_numpy(d["x_bits"].view("int16")).to(dev).view(torch.bfloat16)
        step = fp8_step_fn(torch, wq, sets, x, 1)
        for i in range(args.counters):
            step(i)
        torch.cuda.synchronize()
        log(f"counter steps done: {args.counters}")
        return True
    if args.prefill_counters or args.decode_counters:
        blk, gs = nvfp4_weights(torch, wq, synth.nvfp4_mlp_weights(), dev)
        M, copies, n = (args.prefill_m, 1, args.prefill_counters) if args.prefill_counters else (1, 8, args.decode_counters)
        sets = [blk] + [{k: t.clone() for k, t in blk.items()} for _ in range(copies - 1)]
        xb, _ = synth.nvfp4_x(M, outlier_frac=0.01 if M > 1 else 0.0)
        x = torch.from_numpy(xb.view("int16")).to(dev).view(torch.bfloat16)
        out = torch.empty((M, H), dtype=torch.float32, device=dev)
        ws = torch.empty(wq.mlp_workspace_bytes(wq.WQ_FMT_NVFP4, M, H, I), dtype=torch.uint8, device=dev)
        for i in range(n):
            b = sets[i % copies]
            wq.mlp_nvfp4_run(x, b["gate"], gs["gate"], b["up"], gs["up"], b["down"], gs["down"], out=out, workspace=ws)
        torch.cuda.synchronize()
        log(f"nvfp4 M={M} counter steps done: {n}")
        return True
    if args.fp8_prefill_counters:
        import numpy as np
        d = synth.fp8_mlp(M=1)
        sets = fp8_sets(torch, d, 2)
        M = 512
        xb = synth.to_bf16_bits(synth.rng(2, synth.T_X, (M,)).standard_normal((M, H), dtype=np.float32))
        x = torch.from_numpy(xb.view("int16")).to(dev).view(torch.bfloat16)
        step = fp8_step_fn(torch, wq, sets, x, M)
        for i in range(args.fp8_prefill_counters):
            step(i)
        torch.cuda.synchronize()
        log(f"fp8 prefill counter steps done: {args.fp8_prefill_counters}")
        return True
    if args.w4a8_counters:
        blk, gs = nvfp4_weights(torch, wq, synth.nvfp4_mlp_weights(), dev)
        M = 512
        sets = [blk, {k: t.clone() for k, t in blk.items()}]
        xb, _ = synth.nvfp4_x(M, outlier_frac=0.01)
        x = torch.from_numpy(xb.view("int16")).to(dev).view(torch.bfloat16)
        out = torch.empty((M, H), dtype=torch.float32, device=dev)
        ws = torch.empty(wq.mlp_workspace_bytes(wq.WQ_FMT_NVFP4, M, H, I, "auto", "e4m3"), dtype=torch.uint8,
                         device=dev)
        for i in range(args.w4a8_counters):
            b = sets[i % 2]
            wq.mlp_nvfp4_run(x, b["gate"], gs["gate"], b["up"], gs["up"], b["down"], gs["down"], out=out,
                             workspace=ws, act="e4m3")
        torch.cuda.synchronize()
        log(f"w4a8 prefill counter steps done: {args.w4a8_counters}")
        return True
    if args.awq_counters:
        a = awq_run(torch, wq, synth, synth.awq_moe(), 7, calls=args.awq_counters)
        log(f"routed-expert counter steps done: {a['calls']}")
        return True
    return False


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
    if counter_modes(args, torch, wq, synth, dev):
        return

    K, W, S = args.steps, args.warmup, args.samples
    data = {"fp8": synth.fp8_mlp(M=1)}
    log(f"fp8 decode: K={K} W={W} samples={S}")
    r = fp8_decode(torch, wq, synth, data["fp8"], K, W, S)
    t = r["full"].med
    gbs = FP8_BYTES / t / 1e9
    gu_s, dn_s = r["gu"].med, r["dn"].med
    gu_gbs = r["gu_alg"] / gu_s / 1e9
    dn_gbs = r["dn_alg"] / dn_s / 1e9
    log(f"fp8 decode: {t * 1e6:.2f} us/step (median of {S}), {gbs:.1f} GB/s; gate/up {gu_s * 1e6:.2f} us "
        f"({gu_gbs:.0f} GB/s), down {dn_s * 1e6:.2f} us ({dn_gbs:.0f} GB/s)")
    traffic = read_traffic("fp8w_gateup_row_5120x17408_counters.txt",
                           ["weight_quantized_mlp_amd/csrc/gemv_fast.hip", "weight_quantized_mlp_amd/csrc/dev_common.h"])

    extras = {}
    want = set() if args.extras == "none" else (
        {"fp8_tiny", "nvfp4_decode", "nvfp4_prefill_512", "nvfp4_prefill_8192", "nvfp4_batch8", "fp8_batch8",
         "fp8_prefill_512", "nvfp4_w4a8_prefill_512", "nvfp4_w4a8_prefill_8192", "awq", "awq4", "read_ceiling"}
        if args.extras == "all"
        else set(args.extras.split(",")))
    if "fp8_tiny" in want:
        extras["fp8_tiny_256x512"] = fp8_tiny(torch, wq, synth, K, S)
        log("fp8 tiny", extras["fp8_tiny_256x512"])
    for M, key, steps, copies in ((8, "fp8_batch8", 200, 4), (512, "fp8_prefill_512", 60, 2)):
        if key not in want:
            continue
        n = fp8_batch(torch, wq, synth, data["fp8"], M, steps, S, copies)
        tm = n["full"].med
        tfl = 2.0 * M * 3 * H * I / tm / 1e12
        extras[key] = dict(
            us_per_step=round(tm * 1e6, 2), tok_per_s=round(M / tm, 1), weight_GBps=round(FP8_BYTES / tm / 1e9, 1),
            TFLOPs=round(tfl, 1), mfma_frac_f16_peak=round(tfl / MFMA_F16_PEAK_TFLOPS, 4),
            gateup_us=round(n["gu"].med * 1e6, 2), down_us=round(n["dn"].med * 1e6, 2), path="mfma",
            weight_copies=copies, step=n["full"].summary())
        log(key, extras[key])
    if want & {"nvfp4_decode", "nvfp4_prefill_512", "nvfp4_prefill_8192", "nvfp4_batch8", "nvfp4_w4a8_prefill_512",
               "nvfp4_w4a8_prefill_8192"}:
        data["nvfp4_w"] = synth.nvfp4_mlp_weights()
        blk, gs = nvfp4_weights(torch, wq, data["nvfp4_w"], dev)
        if "nvfp4_decode" in want:
            n = nvfp4_run(torch, wq, synth, blk, gs, 1, K, S, 8, 0.0)
            tm = n["full"].med
            extras["nvfp4_decode_M1"] = dict(
                us_per_step=round(tm * 1e6, 3), GBps=round(NV_BYTES / tm / 1e9, 1), tok_per_s=round(1 / tm, 1),
                hbm_frac=round(NV_BYTES / tm / 1e9 / HBM_PEAK_GBS, 4), gateup_us=round(n["gu"].med * 1e6, 3),
                down_us=round(n["dn"].med * 1e6, 3), weight_copies=n["copies"], step=n["full"].summary())
            log("nvfp4 decode", extras["nvfp4_decode_M1"])
        if "nvfp4_batch8" in want:
            n = nvfp4_run(torch, wq, synth, blk, gs, 8, 200, S, 8, 0.0)
            tm = n["full"].med
            extras["nvfp4_batch8"] = dict(
                us_per_step=round(tm * 1e6, 2), tok_per_s=round(8 / tm, 1), weight_GBps=round(NV_BYTES / tm / 1e9, 1),
                gateup_us=round(n["gu"].med * 1e6, 2), down_us=round(n["dn"].med * 1e6, 2), path="mfma",
                weight_copies=n["copies"], step=n["full"].summary())
            log("nvfp4_batch8", extras["nvfp4_batch8"])
        for M, key, steps, act in ((512, "nvfp4_prefill_512", 60, None), (8192, "nvfp4_prefill_8192", 12, None),
                                   (512, "nvfp4_w4a8_prefill_512", 60, "e4m3"),
                                   (8192, "nvfp4_w4a8_prefill_8192", 12, "e4m3")):
            if key not in want:
                continue
            n = nvfp4_run(torch, wq, synth, blk, gs, M, steps, S, 2, 0.01, act)
            tm = n["full"].med
            tfl = 2.0 * M * 3 * H * I / tm / 1e12
            gu_ms, dn_ms = n["gu"].med * 1e3, n["dn"].med * 1e3
            extras[key] = dict(
                ms_per_step=round(tm * 1e3, 4), tok_per_s=round(M / tm, 1), TFLOPs=round(tfl, 1),
                mfma_frac_f16_peak=round(tfl / MFMA_F16_PEAK_TFLOPS, 4), gateup_ms=round(gu_ms, 4),
                down_ms=round(dn_ms, 4),
                gateup_mfma_frac=round(2.0 * M * 2 * H * I / (gu_ms / 1e3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                down_mfma_frac=round(2.0 * M * H * I / (dn_ms / 1e3) / 1e12 / MFMA_F16_PEAK_TFLOPS, 4),
                step=n["full"].summary(1e3, "ms"))
            log(key, extras[key])
        del blk
    if "dense_f16" in want:
        for M, steps in ((512, 100), (8192, 12)):
            ms = dense_f16_ref(torch, M, steps)
            tfl = 2.0 * M * 3 * H * I / (ms / 1e3) / 1e12
            extras[f"torch_f16_matmul_{M}"] = dict(ms_per_step=round(ms, 4), TFLOPs=round(tfl, 1),
                                                   mfma_frac_f16_peak=round(tfl / MFMA_F16_PEAK_TFLOPS, 4))
            log(f"torch f16 matmul M={M}", extras[f"torch_f16_matmul_{M}"])
    if want & {"awq", "awq4"}:
        data["awq"] = synth.awq_moe()
        for layout, key in ((4, "awq_moe_m1_layout4"), (3, "awq_moe_m1")):
            if ("awq4" if layout == 4 else "awq") in want:
                extras[key] = awq_extra(awq_run(torch, wq, synth, data["awq"], max(S, 21), layout=layout))
                log(key, extras[key])
    if "read_ceiling" in want:
        extras["read_ceiling_wq_read_probe"] = read_ceiling(torch, wq, S)
        log("read ceiling", extras["read_ceiling_wq_read_probe"])

    torch.cuda.synchronize()
    prov = provenance(torch, wq, props)
    log(f"cpu baseline (oracle, ~{args.cpu_seconds:.0f} s)")
    import oracle   # the CPU baseline leg is the only part of the benchmark that uses the oracle
    if data.get("nvfp4_w") is None:
        data["nvfp4_w"] = synth.nvfp4_mlp_weights()
    if data.get("awq") is None:
        data["awq"] = synth.awq_moe()
    cpu = cpu_baseline(oracle, synth, data, args.cpu_seconds)
    log("cpu", json.dumps(cpu))

    roof = dict(bound="hbm", kernel="fp8_gu_row (gate+up+SwiGLU) 5120x17408 M=1", achieved=round(gu_gbs, 1),
                peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gu_gbs / HBM_PEAK_GBS, 4),
                traffic=traffic, algorithmic_bytes_per_launch=r["gu_alg"],
                avg_launch_us=round(gu_s * 1e6, 3), launch=r["gu"].summary(),
                down_kernel=dict(achieved=round(dn_gbs, 1), avg_launch_us=round(dn_s * 1e6, 3),
                                 algorithmic_bytes_per_launch=r["dn_alg"], launch=r["dn"].summary()))
    res = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(t * 1e3, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "fp8_e4m3_per_channel_w8a16_swiglu_mlp_decode", "hidden": H, "intermediate": I,
                   "M": 1, "x_dtype": "bf16", "weight_copies_rotated": r["copies"],
                   "timing": f"median of {S} replays of a hipGraph of K steps, HIP events on the launch stream"},
        "samples": r["full"].summary(),
        "tok_per_s": round(1 / t, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "roofline": roof, "cpu_baseline": cpu, "provenance": prov, "extra": extras,
    }
    line = json.dumps(res)
    print(line, flush=True)
    if args.json_out:
        with open(args.json_out, "w") as f:
            f.write(line + "\n")


if __name__ == "__main__":
    main()
