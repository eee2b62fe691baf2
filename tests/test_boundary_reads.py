"""One-hot linear read-outs: with x = e_k, every path must return exactly dq[:, k].

1.0 * w is exact, the zero terms add exactly and the final scale is one rounding,
so the read-out is bit-exact with the oracle's dequantised column (up to the sign
of a zero: the sums start from +0) -- through the
GEMV (bf16 and f32 activations) and the MFMA path alike.  This pins the K
indexing (record, nibble, group-scale and lane mappings) at every boundary.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_mlp_amd as wq
from gpu_common import DEV, dev, host, same_bits_f32

pytestmark = pytest.mark.gpu

KS = [0, 15, 16, 31, 32, 63, 64]


def fp8_weights(N, K, seed):
    r = np.random.default_rng(seed)
    valid = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    w = valid[r.integers(0, valid.size, size=(N, K))]
    s = (10.0 ** r.uniform(-3, -1, N)).astype(np.float32)
    return w, s


def one_hot_rows(M, K, ks):
    x = np.zeros((M, K), dtype=np.float32)
    for m in range(M):
        x[m, ks[m % len(ks)]] = 1.0
    return x


@pytest.mark.parametrize("path,M", [("gemv", 1), ("gemv", 4), ("mfma", 128)])
@pytest.mark.parametrize("xdt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("K", [256, 320, 5120])
def test_fp8_one_hot(path, M, xdt, K):
    N = 192
    w, s = fp8_weights(N, K, 5)
    dq = oracle.fp8w_dequant(w, s)
    r = np.random.default_rng(K + M)
    ks = KS + [K - 1] + list(r.integers(0, K, 8))
    x = one_hot_rows(M, K, ks)
    y = host(wq.qlinear_run(wq.WQ_FMT_FP8W, dev(x).to(xdt), dev(w), dev(s), path=path))
    for m in range(M):
        k = ks[m % len(ks)]
        assert same_bits_f32(y[m], dq[:, k], signed_zero=False), (path, m, k)


@pytest.mark.parametrize("path,M", [("gemv", 1), ("gemv", 4), ("mfma", 128)])
@pytest.mark.parametrize("xdt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("K", [256, 320, 5120])
def test_nvfp4_one_hot(path, M, xdt, K):
    N = 192
    wp, ws, gs = synth.nvfp4_tensor(N, K, 3, 21)
    blk = oracle.block64_pack(wp, ws)
    dq = oracle.nvfp4_dequant(blk, gs)
    r = np.random.default_rng(K + M + 1)
    ks = KS + [K - 1] + list(r.integers(0, K, 8))
    x = one_hot_rows(M, K, ks)
    y = host(wq.qlinear_run(wq.WQ_FMT_NVFP4, dev(x).to(xdt), dev(blk), None, float(gs), path=path))
    for m in range(M):
        k = ks[m % len(ks)]
        assert same_bits_f32(y[m], dq[:, k], signed_zero=False), (path, m, k)


def test_one_hot_through_the_mlp():
    # x = e_k: act = silu(dq_g[:,k]) * dq_u[:,k] exactly in the definition
    d = synth.fp8_tiny(1)
    for k in (0, 15, 16, 255):
        x = np.zeros((1, 256), dtype=np.float32)
        x[0, k] = 1.0
        ref = oracle.mlp_fp8w_ref(x, d["w_gate"], d["s_gate"], d["w_up"], d["s_up"], d["w_down"], d["s_down"])
        y = host(wq.mlp_fp8w_run(dev(x), *(dev(d[n]) for n in
                                          ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down"))))
        err, _ = oracle.normwise_rel_err(y, ref)
        assert err < 1e-5, (k, err)
