"""Single quantized linear (qlinear_run) against the oracle at the NVFP4 page's tail case.

Page "Qwen3.8-27B-NVFP4", section "Correctness and precision": the wide prefill tile masks
partial tiles instead of shrinking its launch, and its dedicated tail case is batch 129, 67 output
rows, 320 columns -- a multiple of neither tile side.  Here the same shape runs through both paths
of both formats (129 rows take the MFMA GEMM under AUTO: one full 128-row tile plus a 1-row tile;
67 output columns: one partial 128-column tile; K = 320: for NVFP4 five records, a short last
weight block), with bfloat16 and float32 activations, against y = x dq(W)^T in float64.  Shorter K
(FP8 K = 64, NVFP4 K = 192) takes the register-load GEMM, whose lanes past N must not read or store.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_mlp_amd as wq
from gpu_common import dev, gate, host

pytestmark = pytest.mark.gpu

M = 129
SHAPES = [(67, 320), (45, 64), (67, 192)]   # (N, K)


def x_rows(seed, K):
    # bf16-representable activations, so both dtypes carry the same values
    x = np.random.default_rng(seed).standard_normal((M, K)).astype(np.float32)
    xb = synth.to_bf16_bits(x)
    return oracle.bf16_bits_to_f64(xb).astype(np.float32)


@pytest.mark.parametrize("path", ["gemv", "mfma", "auto"])
@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N,K", SHAPES)
def test_fp8_tail_case(path, xdt, N, K):
    r = np.random.default_rng(11 + K)
    w = r.standard_normal((N, K)).astype(np.float32) * 0.05
    s = (np.abs(w).max(axis=1) / 448).astype(np.float32)
    codes = synth.to_e4m3_codes(w / s[:, None])
    x = x_rows(12, K)
    ref = x.astype(np.float64) @ oracle.fp8w_dequant(codes, s).T
    y = host(wq.qlinear_run(wq.WQ_FMT_FP8W, dev(x).to(xdt), dev(codes), dev(s), path=path))
    gate(y, ref, what=f"fp8 linear {M}x{N}x{K} {path} {xdt}")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("path", ["gemv", "mfma", "auto"])
@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("N,K", [(n, k) for n, k in SHAPES if k % 64 == 0])
def test_nvfp4_tail_case(path, xdt, N, K):
    wp, ws, gs = synth.nvfp4_tensor(N, K, 13, 1)
    blk = oracle.block64_pack(wp, ws)
    x = x_rows(14, K)
    ref = x.astype(np.float64) @ oracle.nvfp4_dequant(blk, gs).T
    y = host(wq.qlinear_run(wq.WQ_FMT_NVFP4, dev(x).to(xdt), dev(blk), None, float(gs), path=path))
    gate(y, ref, what=f"nvfp4 linear {M}x{N}x{K} {path} {xdt}")


def test_auto_tail_case_is_the_gemm():
    # 129 rows >= the MFMA threshold: AUTO and the forced GEMM give the same bits
    N, K = 67, 320
    wp, ws, gs = synth.nvfp4_tensor(N, K, 15, 1)
    blk = dev(oracle.block64_pack(wp, ws))
    x = dev(x_rows(16, K)).to(torch.bfloat16)
    a = host(wq.qlinear_run(wq.WQ_FMT_NVFP4, x, blk, None, float(gs), path="auto"))
    b = host(wq.qlinear_run(wq.WQ_FMT_NVFP4, x, blk, None, float(gs), path="mfma"))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("K", [320, 512])
@pytest.mark.parametrize("rows", [5, 37])
@pytest.mark.parametrize("fmt", ["fp8", "nvfp4"])
def test_short_batch_ragged_n_split_k(fmt, rows, K):
    # A batch inside one tile row (32- or 64-row tile) with N = 67: one column tile, so the K range is
    # split and the finish launches workgroups for the batch's rows only and stores column by column.
    # K = 512 (whole 128-byte FP8 rows, one row of 32-row tiles at 5 rows): the FP8 weight copies take
    # the non-temporal hint.
    N = 67
    x = x_rows(17 + rows, K)[:rows]
    if fmt == "fp8":
        r = np.random.default_rng(19)
        w = r.standard_normal((N, K)).astype(np.float32) * 0.05
        s = (np.abs(w).max(axis=1) / 448).astype(np.float32)
        codes = synth.to_e4m3_codes(w / s[:, None])
        ref = x.astype(np.float64) @ oracle.fp8w_dequant(codes, s).T
        y = host(wq.qlinear_run(wq.WQ_FMT_FP8W, dev(x).to(torch.bfloat16), dev(codes), dev(s), path="mfma"))
    else:
        wp, ws, gs = synth.nvfp4_tensor(N, K, 21, 1)
        blk = oracle.block64_pack(wp, ws)
        ref = x.astype(np.float64) @ oracle.nvfp4_dequant(blk, gs).T
        y = host(wq.qlinear_run(wq.WQ_FMT_NVFP4, dev(x).to(torch.bfloat16), dev(blk), None, float(gs), path="mfma"))
    assert y.shape == (rows, N)
    gate(y, ref, what=f"{fmt} linear {rows}x{N}x{K} mfma")
    assert np.all(np.isfinite(y))
