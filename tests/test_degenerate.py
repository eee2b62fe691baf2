"""Degenerate inputs through the C ABI: empty batches, zero activations and scales, NaN weight codes.

* M = 0 is a valid empty call (nothing enqueued), also through the binding, whose empty tensors have
  null data pointers.
* x = 0 gives act = silu(0) * 0 = 0 and an output of exact zeros on every path; a zero channel scale
  (FP8) or a zero group scale (NVFP4) zeroes its row the same way.
* A NaN weight code (E4M3 0x7F, as a FP8 code or as an NVFP4 group scale) turns its dot products into
  NaN: in gate it reaches every output (the down projection sums all of act), in down only its own output
  column.  The NaN positions must be the oracle's.
* The two-stage form (WQ_STAGE_GATEUP_ONLY, then WQ_STAGE_DOWN_ONLY on the same workspace) equals one call.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_mlp_amd as wq
from gpu_common import DEV, bf16_dev, dev, host

pytestmark = pytest.mark.gpu

H, I = 256, 512
FP8_NAMES = ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down")
PATHS = ["gemv", "mfma"]


def fp8_weights():
    r = np.random.default_rng(31)
    d = {}
    for n, shp in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        w = r.standard_normal(shp).astype(np.float32) * 0.05
        s = (np.abs(w).max(axis=1) / 448).astype(np.float32)
        d["w_" + n], d["s_" + n] = synth.to_e4m3_codes(w / s[:, None]), s
    return d


def nvfp4_weights():
    w = {n: synth.nvfp4_tensor(*shp, 32, t) for n, t, shp in (("gate", 1, (I, H)), ("up", 2, (I, H)),
                                                             ("down", 3, (H, I)))}
    return {n: oracle.block64_pack(w[n][0], w[n][1]) for n in w}, {n: w[n][2] for n in w}


def run_fp8(d, x, path):
    return host(wq.mlp_fp8w_run(x, *(dev(d[n]) for n in FP8_NAMES), path=path))


def run_nv(blk, gs, x, path):
    return host(wq.mlp_nvfp4_run(x, dev(blk["gate"]), gs["gate"], dev(blk["up"]), gs["up"], dev(blk["down"]),
                                 gs["down"], path=path))


@pytest.mark.parametrize("path", PATHS + ["auto"])
def test_empty_batch_through_the_binding(path):
    d = fp8_weights()
    x = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    assert run_fp8(d, x, path).shape == (0, H)
    blk, gs = nvfp4_weights()
    assert run_nv(blk, gs, x, path).shape == (0, H)
    y = wq.qlinear_run(wq.WQ_FMT_NVFP4, x, dev(blk["up"]), None, float(gs["up"]), path=path)
    assert tuple(y.shape) == (0, I)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M", [1, 130])
def test_zero_activations_give_exact_zeros(path, M):
    x = bf16_dev(np.zeros((M, H), dtype=np.uint16))
    y = run_fp8(fp8_weights(), x, path)
    assert np.all(y == 0), "fp8"
    blk, gs = nvfp4_weights()
    y = run_nv(blk, gs, x, path)
    assert np.all(y == 0), "nvfp4"


@pytest.mark.parametrize("path", PATHS)
def test_zero_scales_zero_their_rows(path):
    M = 130 if path == "mfma" else 3
    xb = synth.to_bf16_bits(np.random.default_rng(33).standard_normal((M, H)).astype(np.float32))
    d = fp8_weights()
    d["s_down"] = d["s_down"].copy()
    d["s_down"][[0, 77, H - 1]] = 0.0                    # FP8: zero channel scales of three down rows
    y = run_fp8(d, bf16_dev(xb), path)
    assert np.all(y[:, [0, 77, H - 1]] == 0) and np.all(y[:, 1] != 0)
    blk, gs = nvfp4_weights()
    blk = {n: b.copy() for n, b in blk.items()}
    blk["down"][5, :, :4] = 0                            # NVFP4: every group scale of down row 5
    y = run_nv(blk, gs, bf16_dev(xb), path)
    assert np.all(y[:, 5] == 0) and np.all(y[:, 4] != 0)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("where", ["gate", "down"])
def test_nan_codes_match_the_oracle(path, where):
    M = 130 if path == "mfma" else 2
    xb = synth.to_bf16_bits(np.random.default_rng(34).standard_normal((M, H)).astype(np.float32))
    x64 = oracle.bf16_bits_to_f64(xb)
    # FP8: a NaN code in one weight
    d = fp8_weights()
    d = {n: v.copy() for n, v in d.items()}
    if where == "gate":
        d["w_gate"][17, 40] = 0x7F
    else:
        d["w_down"][9, 300] = 0xFF
    ref = oracle.mlp_fp8w_ref(x64, *(d[n] for n in FP8_NAMES))
    y = run_fp8(d, bf16_dev(xb), path)
    assert np.array_equal(np.isnan(y), np.isnan(ref)) and np.isnan(ref).any(), "fp8"
    # NVFP4: a NaN group scale
    blk, gs = nvfp4_weights()
    blk = {n: b.copy() for n, b in blk.items()}
    if where == "gate":
        blk["gate"][17, 1, 2] = 0x7F
    else:
        blk["down"][9, 4, 0] = 0xFF
    ref = oracle.mlp_nvfp4_ref(x64, blk["gate"], gs["gate"], blk["up"], gs["up"], blk["down"], gs["down"])
    y = run_nv(blk, gs, bf16_dev(xb), path)
    assert np.array_equal(np.isnan(y), np.isnan(ref)) and np.isnan(ref).any(), "nvfp4"


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("M", [1, 130])
def test_split_stages_equal_one_call(path, M):
    # WQ_STAGE_GATEUP_ONLY leaves act in the workspace; WQ_STAGE_DOWN_ONLY on the same workspace finishes
    # the MLP: the two calls give the bits of one full call
    xb = synth.to_bf16_bits(np.random.default_rng(35 + M).standard_normal((M, H)).astype(np.float32))
    x = bf16_dev(xb)
    d = fp8_weights()
    W = [dev(d[n]) for n in FP8_NAMES]
    blk, gs = nvfp4_weights()
    B = {n: dev(b) for n, b in blk.items()}
    for fmt in ("fp8", "nvfp4"):
        f = wq.WQ_FMT_FP8W if fmt == "fp8" else wq.WQ_FMT_NVFP4
        ws = torch.empty(max(wq.mlp_workspace_bytes(f, M, H, I, path), 1), dtype=torch.uint8, device=DEV)
        full = torch.empty((M, H), dtype=torch.float32, device=DEV)
        split = torch.full((M, H), float("nan"), dtype=torch.float32, device=DEV)

        def run(out, stage):
            if fmt == "fp8":
                wq.mlp_fp8w_run(x, *W, out=out, workspace=ws, path=path, stage=stage)
            else:
                wq.mlp_nvfp4_run(x, B["gate"], gs["gate"], B["up"], gs["up"], B["down"], gs["down"], out=out,
                                 workspace=ws, path=path, stage=stage)
        run(full, None)
        run(split, "gateup")
        assert torch.isnan(split).all(), fmt        # the gate/up stage leaves the output alone
        run(split, "down")
        assert np.array_equal(host(full).view(np.uint32), host(split).view(np.uint32)), fmt
