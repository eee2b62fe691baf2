"""Calls whose buffers pass 4 GiB: the copy-fed kernels address with 64-bit row or tile bases.

* MFMA GEMM (qlinear_run, both formats): 127,013 activation rows x K = 17,408 in bfloat16 and the
  row-scaled float16 copy in the workspace are 4.4 GB each, so the last ~3,600 rows start beyond 2^32
  bytes.
* NVFP4 GEMV (the single-row item kernel): a Block64 matrix of 262,144 rows x K = 29,184 is 4.3 GB, so its
  last ~500 rows start beyond 2^32 bytes.

Inputs this size are drawn on the device with seeded torch generators (the host generators would take
minutes); the rows that are checked are copied back and the oracle computes them from those bytes.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_mlp_amd as wq
from gpu_common import DEV, dev, gate, host

pytestmark = pytest.mark.gpu


def sampled_rows(M, cut):
    # rows at the start, around the 2^32-byte boundary and at the end
    return sorted({0, 1, 127, 128, cut - 1, cut, cut + 1, M - 129, M - 128, M - 2, M - 1})


@pytest.mark.parametrize("fmt", ["fp8", "nvfp4"])
def test_gemm_activations_past_4GiB(fmt):
    M, N, K = 127013, 128, 17408
    cut = (1 << 32) // (K * 2) + 1                     # first row whose bytes start past 2^32
    g = torch.Generator(device=DEV).manual_seed(91)
    x = torch.randn((M, K), generator=g, device=DEV, dtype=torch.bfloat16)
    if fmt == "fp8":
        r = np.random.default_rng(92)
        w = r.standard_normal((N, K)).astype(np.float32) * 0.02
        s = (np.abs(w).max(axis=1) / 448).astype(np.float32)
        codes = synth.to_e4m3_codes(w / s[:, None])
        dq = oracle.fp8w_dequant(codes, s)
        y = wq.qlinear_run(wq.WQ_FMT_FP8W, x, dev(codes), dev(s), path="mfma")
    else:
        wp, ws, gs = synth.nvfp4_tensor(N, K, 93, 1)
        blk = oracle.block64_pack(wp, ws)
        dq = oracle.nvfp4_dequant(blk, gs)
        y = wq.qlinear_run(wq.WQ_FMT_NVFP4, x, dev(blk), None, float(gs), path="mfma")
    rows = sampled_rows(M, cut)
    xs = host(x[rows].float()).astype(np.float64)      # bfloat16 values, exact in float64
    ys = host(y[rows])
    del x, y
    torch.cuda.empty_cache()
    gate(ys, xs @ dq.T, what=f"{fmt} linear M={M} rows past 4 GiB")


def test_gemv_weights_past_4GiB():
    N, K = 262144, 29184
    rb = K // 64 * 36
    cut = (1 << 32) // rb + 1
    g = torch.Generator(device=DEV).manual_seed(94)
    blk = torch.randint(0, 256, (N, K // 64, 36), generator=g, device=DEV, dtype=torch.uint8)
    blk[:, :, :4] = (blk[:, :, :4] & 0x3F) | 0x08      # E4M3 group scales: small, positive, never NaN
    gs = 37.0
    x = synth.to_bf16_bits(np.random.default_rng(95).standard_normal((1, K)).astype(np.float32))
    xt = dev(x.view(np.int16)).view(torch.bfloat16)
    y = host(wq.qlinear_run(wq.WQ_FMT_NVFP4, xt, blk, None, gs, path="gemv"))[0]
    rows = sampled_rows(N, cut)
    sub = host(blk[rows])
    del blk
    torch.cuda.empty_cache()
    ref = oracle.nvfp4_dequant(sub, np.float32(gs)) @ oracle.bf16_bits_to_f64(x)[0]
    gate(y[rows][None], ref[None], what=f"nvfp4 GEMV N={N} K={K} rows past 4 GiB")
