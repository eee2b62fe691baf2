"""mlp_fp8w_run_noalloc (the library's static scratch) against mlp_fp8w_run with a caller workspace.

Both run the same kernels with the same plan, so the outputs must agree bit for bit; two calls in a row,
the second on a smaller batch (the scratch keeps the first call's contents), on the GEMV and the MFMA
path and under AUTO at the FP8 decode shape (hidden 5120, intermediate 17408), where calls above the
scratch's size are rejected before anything is enqueued.
"""
import ctypes

import numpy as np
import pytest
import torch

import synth
import weight_quantized_mlp_amd as wq
from gpu_common import DEV, bf16_dev, dev, host

pytestmark = pytest.mark.gpu

NAMES = ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down")


def x_rows(M, H, seed):
    return bf16_dev(synth.to_bf16_bits(np.random.default_rng(seed).standard_normal((M, H), dtype=np.float32)))


def pair(W, x, path):
    """(noalloc output, workspace-call output) on fresh output buffers filled with NaN."""
    M, H = x.shape
    a = torch.full((M, H), float("nan"), dtype=torch.float32, device=DEV)
    b = torch.full((M, H), float("nan"), dtype=torch.float32, device=DEV)
    wq.mlp_fp8w_run_noalloc(x, *W, out=a, path=path)
    wq.mlp_fp8w_run(x, *W, out=b, path=path)
    torch.cuda.synchronize()
    return host(a), host(b)


@pytest.mark.parametrize("path,Ms", [("gemv", (4, 1)), ("mfma", (32, 8))])
def test_noalloc_equals_workspace_call_small(path, Ms):
    H, I = 1024, 2048
    d = synth.fp8_mlp(M=1, H=H, I=I, config_id=31)
    W = [dev(d[n]) for n in NAMES]
    for i, M in enumerate(Ms):
        print(f"[noalloc] path={path} M={M} shape {H}x{I}", flush=True)
        a, b = pair(W, x_rows(M, H, 40 + i), path)
        assert np.all(np.isfinite(b))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), (path, M)


def test_noalloc_at_the_decode_shape():
    d = synth.fp8_mlp(M=1)
    W = [dev(d[n]) for n in NAMES]
    H = 5120
    for i, M in enumerate((16, 1)):                       # MFMA (split K), then the GEMV
        print(f"[noalloc] auto M={M} shape 5120x17408", flush=True)
        a, b = pair(W, x_rows(M, H, 50 + i), "auto")
        assert np.all(np.isfinite(b))
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), M
    # beyond the scratch: rejected, nothing written
    M = 64
    x = x_rows(M, H, 60)
    out = torch.full((M, H), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(wq.WQError) as ei:
        wq.mlp_fp8w_run_noalloc(x, *W, out=out)
    assert ei.value.rc == -8
    torch.cuda.synchronize()
    assert bool(torch.all(out == 7.0))
