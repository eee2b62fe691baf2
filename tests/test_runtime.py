"""Runtime behaviour of the library: first use inside a hipGraph capture, and concurrent host threads.

* The library raises the LDS limit of its large-LDS kernels on their first launch on a device.  A fresh
  process whose very first calls happen under stream capture must still produce a graph whose replays
  equal eager calls (checked in a child process, so that no earlier test has made those first calls).
* Calls from several host threads on their own streams (ctypes releases the GIL) must give the same
  bits as the same calls made one after another.
"""
import os
import subprocess
import sys
import threading

import numpy as np
import pytest
import torch

import synth
import weight_quantized_mlp_amd as wq
from gpu_common import DEV, bf16_dev, host

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import synth, weight_quantized_mlp_amd as wq
dev = torch.device("cuda:0")
H, I = 512, 1024
W = {n: synth.nvfp4_tensor(*shp, 5, t) for n, t, shp in (("g", 1, (I, H)), ("u", 2, (I, H)), ("d", 3, (H, I)))}
import oracle
blk = {n: torch.from_numpy(oracle.block64_pack(W[n][0], W[n][1])).to(dev) for n in W}
res = []
for M, path in ((1, "gemv"), (8, "mfma"), (160, "mfma")):
    xb = synth.to_bf16_bits(np.random.default_rng(M).standard_normal((M, H)).astype(np.float32))
    x = torch.from_numpy(xb.view(np.int16)).to(dev).view(torch.bfloat16)
    out = torch.empty((M, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(wq.mlp_workspace_bytes(1, M, H, I, path), 1), dtype=torch.uint8, device=dev)
    run = lambda: wq.mlp_nvfp4_run(x, blk["g"], W["g"][2], blk["u"], W["u"][2], blk["d"], W["d"][2],
                                   out=out, workspace=ws, path=path)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):   # the first library call of this process for this path
            run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    replays = []
    for _ in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        replays.append(out.cpu().numpy().copy())
    run()
    torch.cuda.synchronize()
    eager = out.cpu().numpy()
    res.append(all(np.array_equal(r.view(np.uint32), eager.view(np.uint32)) for r in replays)
               and np.isfinite(eager).all())
print("RESULT", int(all(res)), flush=True)
"""


def test_first_use_inside_graph_capture():
    p = subprocess.run([sys.executable, "-c", CHILD, ROOT], capture_output=True, text=True, timeout=240,
                       cwd=ROOT)
    print(p.stdout[-2000:], p.stderr[-2000:], flush=True)
    assert p.returncode == 0
    assert "RESULT 1" in p.stdout


def test_concurrent_host_threads():
    d = synth.fp8_tiny(4)
    names = ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down")
    Wf = [torch.from_numpy(np.ascontiguousarray(d[n])).to(DEV) for n in names]
    H, I = 5120, 1024   # NVFP4 at hidden 5120, intermediate 1024 (AUTO: GEMV below 128 rows, 8.8 MB of weights)
    w = {n: synth.nvfp4_tensor(*shp, 6, t) for n, t, shp in (("g", 1, (I, H)), ("u", 2, (I, H)), ("d", 3, (H, I)))}
    import oracle
    blk = {n: torch.from_numpy(oracle.block64_pack(w[n][0], w[n][1])).to(DEV) for n in w}
    jobs = []
    for k in range(8):
        M = [1, 4, 130, 3][k % 4]
        xb = synth.to_bf16_bits(np.random.default_rng(100 + k).standard_normal((M, H)).astype(np.float32))
        jobs.append(("nv", bf16_dev(xb), "auto"))
        jobs.append(("fp8", torch.from_numpy(np.ascontiguousarray(d["x"])).to(DEV), ["gemv", "mfma"][k % 2]))

    def call(job, stream):
        kind, x, path = job
        with torch.cuda.stream(stream):
            if kind == "nv":
                y = wq.mlp_nvfp4_run(x, blk["g"], w["g"][2], blk["u"], w["u"][2], blk["d"], w["d"][2], path=path)
            else:
                y = wq.mlp_fp8w_run(x, *Wf, path=path)
            stream.synchronize()
        return host(y)

    serial = [call(j, torch.cuda.current_stream()) for j in jobs]
    results = [None] * len(jobs)
    errors = []

    def worker(t):
        s = torch.cuda.Stream()
        try:
            for i in range(t, len(jobs), 4):
                for _ in range(3):
                    results[i] = call(jobs[i], s)
        except Exception as e:   # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert not errors, errors
    for i, (a, b) in enumerate(zip(serial, results)):
        assert b is not None and np.array_equal(a.view(np.uint32), b.view(np.uint32)), i
