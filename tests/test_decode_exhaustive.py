"""Every E4M3 code, and every E2M1 code under every E4M3 group scale, through the kernels that compute.

The weight formats are FP8 E4M3 per output channel (issue "tp>1 fp8w tail-MLP shard host-dequantizes
every layer", section "Mechanism on the tp>1 path") and NVFP4: E2M1 codes, one E4M3 scale per 16 input
channels and a per-tensor global scale applied as 1/global_scale (page "Qwen3.8-27B-NVFP4", section
"NVFP4 numerics as implemented").  Each kernel decodes with its own conversion instructions (float32,
bfloat16 or float16 forms, chosen by the activation type and the path), so each one is read out here:

* single linear (``qlinear_run``): x rows are one-hot, so row m of y is column k_m of the dequantised
  matrix -- 1.0 * w is exact, the zero terms add exactly and the last scale is the one rounding of the
  definition, so y must equal the oracle's decode bit for bit (NaN as a class, and +0 for -0: the sums
  start from +0);
* gate/up projection (the MLP with its gate/up stage only): the gate's hot column decodes to 128, where
  silu is exactly 128 in float32, so act = 128 * dq(up) -- bitwise for the float32 act of FP8, and the
  single float16 rounding of it for NVFP4; with the two matrices swapped (up = 1.0) act = silu(dq(gate))
  up to the rounding of silu.

The weight matrices: at every hot column, rows 0..255 hold all 256 E4M3 codes (rows 0x7F and 0xFF the two
NaN codes, the other 254 rows the 254 finite codes, shifted from one hot column to the next); NVFP4 rows
0..255 carry all 256 E4M3 group scales (NaN in rows 0x7F and 0xFF), and the 16 positions of each hot group
see all 16 E2M1 codes in every row.  Other entries are random finite codes (x is zero there).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_mlp_amd as wq
from gpu_common import dev, host, same_bits_f32

pytestmark = pytest.mark.gpu

FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
FINITE_ROWS = np.array([n for n in range(256) if n not in (0x7F, 0xFF)])
NAN_ROWS = np.array([0x7F, 0xFF])
TORCH_X = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def a256(n):
    return -(-n // 256) * 256


def fp8_hot(K):
    """Hot columns: both sides of every 16-, 32-, 64- and 128-wide boundary up to K, and the last."""
    ks = sorted({k for k in (0, 1, 7, 8, 15, 16, 17, 31, 32, 63, 64, 65, 127, 128, 191, 255, 256, 383, 511)
                 if k < K} | {K - 2, K - 1})
    return ks


def fp8_matrix(N, K, hot, seed):
    r = np.random.default_rng(seed)
    w = FINITE[r.integers(0, FINITE.size, size=(N, K))]
    for j, k in enumerate(hot):
        w[FINITE_ROWS, k] = FINITE[(np.arange(FINITE.size) + 37 * j) % FINITE.size]
        w[NAN_ROWS, k] = NAN_ROWS
    s = (10.0 ** r.uniform(-3, -1, N)).astype(np.float32)
    return w, s


def nvfp4_hot(K):
    """Hot positions: all 16 of groups 0, 1, 3 (end of the first record), 4 (start of the second) and the
    last group."""
    G = K // 16
    return [16 * g + j for g in sorted({0, 1, 3, 4, G - 1}) for j in range(16)]


def nvfp4_matrix(N, K, seed, gs):
    r = np.random.default_rng(seed)
    G = K // 16
    nib = ((np.arange(N)[:, None] + np.arange(K)[None, :]) % 16).astype(np.uint8)   # all 16 codes per group
    ws = FINITE[r.integers(0, FINITE.size, size=(N, G))]
    for g in range(G):
        ws[FINITE_ROWS, g] = FINITE[(np.arange(FINITE.size) + 41 * g) % FINITE.size]
        ws[NAN_ROWS, g] = NAN_ROWS
    wp = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return oracle.block64_pack(wp, ws), np.float32(gs)


def one_hot(M, K, ks):
    x = np.zeros((M, K), dtype=np.float32)
    x[np.arange(M), ks[:M]] = 1.0
    return x


def check_columns(y, dq, ks, what):
    for m, k in enumerate(ks):
        ok = same_bits_f32(y[m], dq[:, k], signed_zero=False)
        if not ok:
            bad = np.flatnonzero(~((y[m] == dq[:, k]) | (np.isnan(y[m]) & np.isnan(dq[:, k]))))
            raise AssertionError(f"{what}: x row {m} (k={k}) differs at weight rows {bad[:8]}: "
                                 f"got {y[m][bad[:4]]}, want {dq[bad[:4], k]}")


# ---- single linear ---------------------------------------------------------------------------------------
# K = 4096 (a million weights at N = 256) reaches the GEMV item kernel (fp8_lin_items); the smaller K the
# general GEMV kernel (fp8w_gemv_kernel)
FP8_LINEAR = ([(p, x, K) for p in ("gemv", "mfma") for x in ("f32", "bf16") for K in (64, 192, 512)]
              + [("gemv", x, 4096) for x in ("f32", "bf16")])


@pytest.mark.parametrize("path,xdt,K", FP8_LINEAR)
def test_fp8_linear_reads_every_code(path, xdt, K):
    N = 256
    hot = fp8_hot(K)
    w, s = fp8_matrix(N, K, hot, 100 + K)
    dq = oracle.fp8w_dequant(w, s)
    x = one_hot(len(hot), K, hot)
    y = host(wq.qlinear_run(wq.WQ_FMT_FP8W, dev(x).to(TORCH_X[xdt]), dev(w), dev(s), path=path))
    check_columns(y, dq, hot, f"fp8 {path} {xdt} K={K}")
    for k in (hot[0], hot[len(hot) // 2], hot[-1]):            # the one-row kernels
        y1 = host(wq.qlinear_run(wq.WQ_FMT_FP8W, dev(one_hot(1, K, [k])).to(TORCH_X[xdt]), dev(w), dev(s),
                                 path=path))
        check_columns(y1, dq, [k], f"fp8 {path} {xdt} K={K} M=1")


# (path, x dtype, K, activation variant); the W4A8 variant (act "e4m3") quantizes the one-hot rows to E4M3
# (1.0 -> code 256 under the row scale 2^-8, exactly) and runs its E4M3 MFMAs on the decoded weights
NV_LINEAR = ([("gemv", x, K, None) for x in ("f32", "bf16", "f16") for K in (192, 512)]
             + [("mfma", x, K, None) for x in ("f32", "bf16") for K in (192, 512)]
             + [("mfma", x, K, "e4m3") for x in ("f32", "bf16") for K in (384, 512)])


@pytest.mark.parametrize("path,xdt,K,act", NV_LINEAR)
def test_nvfp4_linear_reads_every_code_under_every_scale(path, xdt, K, act):
    N = 256
    blk, gs = nvfp4_matrix(N, K, 200 + K, 448 * 6 / 0.3)
    dq = oracle.nvfp4_dequant(blk, gs)
    hot = nvfp4_hot(K)
    x = one_hot(len(hot), K, hot)
    y = host(wq.qlinear_run(wq.WQ_FMT_NVFP4, dev(x).to(TORCH_X[xdt]), dev(blk), None, float(gs), path=path, act=act))
    check_columns(y, dq, hot, f"nvfp4 {path} {xdt} K={K} act={act}")
    for k in (hot[0], hot[37], hot[-1]):
        y1 = host(wq.qlinear_run(wq.WQ_FMT_NVFP4, dev(one_hot(1, K, [k])).to(TORCH_X[xdt]), dev(blk), None,
                                 float(gs), path=path, act=act))
        check_columns(y1, dq, [k], f"nvfp4 {path} {xdt} K={K} act={act} M=1")


# ---- gate/up projection ------------------------------------------------------------------------------------
H, I = 512, 384          # gate/up [I, H]: rows 0..255 exhaustive, 256..383 random finite codes (both dimensions
                         # multiples of 128, as the W4A8 variant needs)


def act_view(ws, fmt, path, M):
    """act as the gate/up stage leaves it in the workspace (the header's layout)."""
    if fmt == "nvfp4w8":                            # W4A8: x's E4M3 values (float16), x scales, then act float32
        off, n, dt = a256(M * H * 2) + a256(M * 4), M * I * 4, np.float32
    elif path == "gemv":
        off, n, dt = 0, M * I * (4 if fmt == "fp8" else 2), (np.float32 if fmt == "fp8" else np.float16)
    elif fmt == "fp8":
        off, n, dt = a256(M * H * 2) + a256(M * 4) + a256(M * I * 2), M * I * 4, np.float32
    else:
        off, n, dt = a256(M * H * 2) + a256(M * 4), M * I * 2, np.float16
    return host(ws[off:off + n]).view(dt).reshape(M, I)


def gateup(fmt, path, xdt, x, gate, up, M):
    """Run the gate/up stage only and return act (float64)."""
    xt = dev(x).to(TORCH_X[xdt])
    if fmt == "fp8":
        (wg, sg), (wu, su) = gate, up
        wd, sd = np.zeros((H, I), np.uint8), np.ones(H, np.float32)
        nb = wq.mlp_workspace_bytes(wq.WQ_FMT_FP8W, M, H, I, path)
        ws = torch.zeros(nb, dtype=torch.uint8, device=xt.device)
        wq.mlp_fp8w_run(xt, dev(wg), dev(sg), dev(wu), dev(su), dev(wd), dev(sd), workspace=ws, path=path,
                        stage="gateup")
    else:
        (bg, gg), (bu, gu) = gate, up
        bd = np.zeros((H, I // 64, 36), np.uint8)
        act = "e4m3" if fmt == "nvfp4w8" else None
        nb = wq.mlp_workspace_bytes(wq.WQ_FMT_NVFP4, M, H, I, path, act)
        ws = torch.zeros(nb, dtype=torch.uint8, device=xt.device)
        wq.mlp_nvfp4_run(xt, dev(bg), float(gg), dev(bu), float(gu), dev(bd), 1.0, workspace=ws, path=path,
                         stage="gateup", act=act)
    torch.cuda.synchronize()
    return act_view(ws, fmt, path, M).astype(np.float64)


def const_fp8(value_code, hot, seed):
    """FP8 [I, H] whose hot columns all hold one code, scale 1."""
    w, _ = fp8_matrix(I, H, [], seed)
    w[:, hot] = value_code
    return w, np.ones(I, np.float32)


def const_nvfp4(nibble, scale_code, hot_groups, seed):
    """NVFP4 [I, H] whose hot groups hold one E2M1 code under one E4M3 scale, global scale 1."""
    r = np.random.default_rng(seed)
    nib = r.integers(0, 16, size=(I, H)).astype(np.uint8)
    ws = FINITE[r.integers(0, FINITE.size, size=(I, H // 16))]
    for g in hot_groups:
        nib[:, 16 * g:16 * g + 16] = nibble
        ws[:, g] = scale_code
    wp = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return oracle.block64_pack(wp, ws), np.float32(1.0)


def exhaustive_rows(w, s):
    """Pad a [256, H] exhaustive FP8 matrix to I rows with random finite codes."""
    r = np.random.default_rng(5)
    wf = FINITE[r.integers(0, FINITE.size, size=(I, H))]
    sf = (10.0 ** r.uniform(-3, -1, I)).astype(np.float32)
    wf[:256], sf[:256] = w, s
    return wf, sf


GATEUP = ([(f, p, x, M) for f in ("fp8", "nvfp4") for p in ("gemv", "mfma") for x in ("f32", "bf16")
           for M in (1, 20)]
          + [("nvfp4w8", "mfma", x, M) for x in ("f32", "bf16") for M in (1, 20)])


@pytest.mark.parametrize("fmt,path,xdt,M", GATEUP)
def test_gateup_reads_every_code(fmt, path, xdt, M):
    if fmt == "fp8":
        hot = fp8_hot(H)[:M] if M > 1 else [37]
        assert len(hot) == M
        w, s = fp8_matrix(256, H, hot, 300 + M)
        ex = exhaustive_rows(w, s)
        dq = oracle.fp8w_dequant(*ex).astype(np.float64)
        const128 = const_fp8(0x70, hot, 7)                      # E4M3 0x70 = 128, scale 1
        const1 = const_fp8(0x38, hot, 8)                        # E4M3 0x38 = 1
    else:
        hot = nvfp4_hot(H)[:M] if M > 1 else [37]
        assert len(hot) == M
        blk256, gs = nvfp4_matrix(256, H, 300 + M, 448 * 6 / 0.05)
        r = np.random.default_rng(9)
        wp_pad = r.integers(0, 256, size=(I - 256, H // 2)).astype(np.uint8)
        ws_pad = FINITE[r.integers(0, 0x70, size=(I - 256, H // 16))]
        ex = (np.concatenate([blk256, oracle.block64_pack(wp_pad, ws_pad)]), gs)
        dq = oracle.nvfp4_dequant(*ex).astype(np.float64)
        groups = sorted({k // 16 for k in hot})
        const128 = const_nvfp4(6, 0x60, groups, 7)              # E2M1 4.0 x E4M3 32 = 128
        const1 = const_nvfp4(2, 0x38, groups, 8)                # E2M1 1.0 x E4M3 1 = 1
    x = one_hot(M, H, hot)
    # up exhaustive, gate 128: act = 128 * dq(up) exactly (float16-rounded once for NVFP4)
    act = gateup(fmt, path, xdt, x, const128, ex, M)
    want = np.stack([128.0 * dq[:, k] for k in hot])
    if fmt == "nvfp4":                              # float16 act; W4A8 keeps act in float32
        want = want.astype(np.float16).astype(np.float64)
    ok = (act == want) | (np.isnan(act) & np.isnan(want))
    assert ok.all(), f"{fmt} {path} {xdt} M={M}: up read-out differs at {np.argwhere(~ok)[:6].tolist()}"
    # gate exhaustive, up 1: act = silu(dq(gate)) up to silu's own rounding
    act = gateup(fmt, path, xdt, x, ex, const1, M)
    g = np.stack([dq[:, k] for k in hot])
    want = oracle.silu(np.nan_to_num(g)) * np.where(np.isnan(g), np.nan, 1.0)
    if fmt in ("fp8", "nvfp4w8"):
        tol = 8 * np.spacing(np.abs(want).astype(np.float32)).astype(np.float64) + 1e-38
    else:
        w16 = want.astype(np.float16)
        tol = np.spacing(np.abs(w16)).astype(np.float64) + 1e-7
        want = w16.astype(np.float64)
    ok = (np.abs(act - want) <= tol) | (np.isnan(act) & np.isnan(want))
    assert ok.all(), f"{fmt} {path} {xdt} M={M}: gate read-out differs at {np.argwhere(~ok)[:6].tolist()}"
