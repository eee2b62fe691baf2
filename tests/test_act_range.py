"""FP8 act beyond float16's range, through both paths (GPU, through the C ABI).

The FP8 definition keeps act = silu(g) * u unrounded between the two projections (issue "tp>1 fp8w
tail-MLP shard host-dequantizes every layer", section "Proposed fix").  The GEMV path stores act as
float32; the MFMA path stores it as float32 and gives the down GEMM a float16 operand after an exact
power-of-two row scale, so act values far above 65504 must still give the oracle's result.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import bf16_dev, dev, gate, host
import weight_quantized_mlp_amd as wq

pytestmark = pytest.mark.gpu

H, I = 512, 1024
NAMES = ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down")


@pytest.fixture(scope="module")
def big_act():
    d = synth.fp8_mlp(M=1, H=H, I=I, config_id=21)
    return d


@pytest.mark.parametrize("path", ["gemv", "mfma"])
@pytest.mark.parametrize("M", [8, 130])
def test_fp8_act_above_f16_range(big_act, path, M):
    d = big_act
    x = synth.rng(21, synth.T_X, (M,)).standard_normal((M, H), dtype=np.float32) * np.float32(1024.0)
    xb = synth.to_bf16_bits(x)
    x64 = oracle.bf16_bits_to_f64(xb)
    ref, act = oracle.mlp_fp8w_ref(x64, *(d[n] for n in NAMES), return_act=True)
    amax = np.max(np.abs(act))
    print(f"[act-range] path={path} M={M} max|act|={amax:.3e}", flush=True)
    assert amax > 4 * 65504.0                     # the case really leaves float16's range
    y = host(wq.mlp_fp8w_run(bf16_dev(xb), *(dev(d[n]) for n in NAMES), path=path))
    assert np.all(np.isfinite(y))
    gate(y, ref, what=f"fp8 act beyond f16 range, {path}, M={M}")
