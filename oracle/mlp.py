"""Dense SwiGLU MLP with dequantised weights (oracle; test infrastructure only).

The method computes, per activation row (issue "tp>1 fp8w tail-MLP shard
...", section "Proposed fix"):

    g[i]   = sum_k x[k] * dq(gate[i, k])
    u[i]   = sum_k x[k] * dq(up[i, k])
    act[i] = silu(g[i]) * u[i]                (float32-exact, no bf16 rounding)
    out[o] = sum_q act[q] * dq(down[o, q])

with silu(z) = z / (1 + exp(-z)).  The oracle evaluates this definition in
float64 on the exact dequantised values: for FP8 dq = e4m3(w) * s[n] and for
NVFP4 dq = e2m1(q) * e4m3(d) / gs, both taken in float64 (the float32-rounded
dq of the decoder definition differs from them by at most one float32
rounding, far inside the 1e-3 gate).
"""
import math
import numpy as np
from .codecs import e4m3_to_f64, e2m1_to_f64
from .pack import block64_unpack


def silu(z):
    """Textbook SiLU, z * sigmoid(z) = z / (1 + e^-z), evaluated in float64 without overflow."""
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = z[pos] / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = z[~pos] * ez / (1.0 + ez)
    return out


def swiglu_mlp(x, Wg, Wu, Wd):
    """out = (silu(x Wg^T) * (x Wu^T)) Wd^T in float64.  x [M, H]; Wg, Wu [I, H]; Wd [H, I]."""
    x = np.asarray(x, dtype=np.float64)
    g = x @ np.asarray(Wg, dtype=np.float64).T
    u = x @ np.asarray(Wu, dtype=np.float64).T
    act = silu(g) * u
    return act @ np.asarray(Wd, dtype=np.float64).T, act


def fp8w_weight_f64(w, s):
    """Exact float64 e4m3(w[n, k]) * s[n] (issue "tp>1 fp8w ...", section "Mechanism on the tp>1 path")."""
    return e4m3_to_f64(w) * np.asarray(s, dtype=np.float32).astype(np.float64)[:, None]


def nvfp4_weight_f64(blk, global_scale):
    """Exact float64 e2m1(q) * e4m3(d_group) * (1/gs) from Block64 records
    (page "Qwen3.8-27B-NVFP4", section "NVFP4 numerics as implemented"), with
    1/gs rounded once to float32 as the runtime factor."""
    wp, ws = block64_unpack(blk)
    n = wp.shape[0]
    nib = np.empty((n, wp.shape[1] * 2), dtype=np.uint8)
    nib[:, 0::2] = wp & 0x0F
    nib[:, 1::2] = wp >> 4
    d = np.repeat(e4m3_to_f64(ws), 16, axis=1)
    inv = np.float64(np.float32(1.0) / np.float32(global_scale))
    return e2m1_to_f64(nib) * d * inv


def mlp_fp8w_ref(x, wg, sg, wu, su, wd, sd, return_act=False):
    """FP8 E4M3 per-channel W8A16 SwiGLU MLP; x is float64-exact (from f32 or bf16)."""
    out, act = swiglu_mlp(x, fp8w_weight_f64(wg, sg), fp8w_weight_f64(wu, su), fp8w_weight_f64(wd, sd))
    return (out, act) if return_act else out


def mlp_nvfp4_ref(x, gblk, ggs, ublk, ugs, dblk, dgs, return_act=False, rows_block=None):
    """NVFP4 Block64 SwiGLU MLP in float64."""
    Wg = nvfp4_weight_f64(gblk, ggs)
    Wu = nvfp4_weight_f64(ublk, ugs)
    Wd = nvfp4_weight_f64(dblk, dgs)
    out, act = swiglu_mlp(x, Wg, Wu, Wd)
    return (out, act) if return_act else out


def mlp_nvfp4_w4a8_ref(x, gblk, ggs, ublk, ugs, dblk, dgs, stages=False):
    """The W4A8 variant of the NVFP4 MLP: the same definition with both linears' activations quantized per
    token to E4M3 (page "Qwen3.8-27B-NVFP4", section "Implemented execution path": per-token dynamic
    activation quantization, one quantization of x shared by gate and up; the down projection's input
    act is quantized the same way).

        xq, sx = quant(x);     xd = e4m3(xq) * sx                 (exact)
        act    = silu(xd Wg^T) * (xd Wu^T)                        (float64)
        act32  = RN_f32(act)   -- the quantization decision is taken on the float32 act, the precision in
                                  which the device holds act (reading: the page gives no precision for it)
        aq, sa = quant(act32); out = (e4m3(aq) * sa) Wd^T         (float64)

    With stages=True returns (out, dict(xq, sx, act32, aq, sa)).
    """
    from .actquant import quant_e4m3_per_token
    xq, sx = quant_e4m3_per_token(x)
    xd = e4m3_to_f64(xq) * sx[:, None]
    Wg = nvfp4_weight_f64(gblk, ggs)
    Wu = nvfp4_weight_f64(ublk, ugs)
    g = xd @ Wg.T
    u = xd @ Wu.T
    del Wg, Wu
    act32 = (silu(g) * u).astype(np.float32)
    aq, sa = quant_e4m3_per_token(act32.astype(np.float64))
    ad = e4m3_to_f64(aq) * sa[:, None]
    out = ad @ nvfp4_weight_f64(dblk, dgs).T
    if stages:
        return out, dict(xq=xq, sx=sx, act32=act32, aq=aq, sa=sa)
    return out


def mlp_bruteforce(x, Wg, Wu, Wd):
    """Pure-Python triple loop of the same definition, for tiny shapes only.

    x: list of rows; Wg, Wu: [I][H]; Wd: [H][I]; all Python floats.  Uses
    math.exp and left-to-right sums: an implementation that shares nothing
    with the NumPy path above.
    """
    out = []
    for row in x:
        act = []
        for i in range(len(Wg)):
            g = 0.0
            u = 0.0
            for k in range(len(row)):
                g += row[k] * Wg[i][k]
                u += row[k] * Wu[i][k]
            sig = 1.0 / (1.0 + math.exp(-g)) if g >= 0 else math.exp(g) / (1.0 + math.exp(g))
            act.append(g * sig * u)
        o_row = []
        for o in range(len(Wd)):
            acc = 0.0
            for q in range(len(act)):
                acc += act[q] * Wd[o][q]
            o_row.append(acc)
        out.append(o_row)
    return out
