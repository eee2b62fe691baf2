"""AWQ int4 group-32 routed-expert single-token step (oracle; test infrastructure only).

Page "[Kernel][SM70] Add native-g32 AWQ QPN M1 operator", section "What it
does": W13 runs over the selected experts in router order and materialises
gate and up in float16, SwiGLU is fused into a float16 intermediate of shape
(top-k, I); W2 forms one float16 result per route, and the router-weighted
sum is accumulated in float32, in route order, into a float16 output.
Invalid expert ids contribute zero and duplicate valid ids keep their own
router weights (same section, validation paragraph).

Readings where the page is silent: gate = W13 rows [0, I), up = rows [I, 2I);
silu in float64 on the float16-rounded gate; the router sum is taken in
float64 here (its float32 accumulation on the device is covered by the 1e-3
normwise gate, not compared bitwise).
"""
import math
import numpy as np
from .codecs import f16_bits_to_f64, f64_to_f16_bits
from .dequant import awq_dequant_parts
from .mlp import silu


def _valid(e, E):
    return 0 <= int(e) < E


def moe_w13_stage_ref(x_bits, ids, w13_codes, w13_scales, w13_zeros, I):
    """Stage 1: act[r, n] = RN_f16(silu(RN_f16(g)) * RN_f16(u)) with float64 sums.

    x_bits: f16 bits [H]; ids [topk]; w13_*: unpacked bank pieces [E, 2I, H] / [E, 2I, H/32].
    Returns act f16 bits [topk, I].  Invalid id -> zero row.
    """
    E = w13_codes.shape[0]
    x = f16_bits_to_f64(x_bits)
    topk = len(ids)
    act = np.zeros((topk, I), dtype=np.uint16)
    for r, e in enumerate(ids):
        if not _valid(e, E):
            continue
        dq = f16_bits_to_f64(awq_dequant_parts(w13_codes[e], w13_scales[e], w13_zeros[e]))  # [2I, H]
        gu = dq @ x
        g = f16_bits_to_f64(f64_to_f16_bits(gu[:I]))
        u = f16_bits_to_f64(f64_to_f16_bits(gu[I:]))
        act[r] = f64_to_f16_bits(silu(g) * u)
    return act


def moe_w2_stage_ref(act_bits, ids, router_w, w2_codes, w2_scales, w2_zeros):
    """Stage 2: y_r = RN_f16(act[r] . dq2[e_r]^T); out = RN_f16(sum_r w_r * y_r) over valid r, in order.

    act_bits: f16 bits [topk, I]; w2_*: [E, H, I] / [E, H, I/32].  Returns (out f16 bits [H], y f16 bits [topk, H]).
    """
    E, H, _ = w2_codes.shape
    topk = len(ids)
    y = np.zeros((topk, H), dtype=np.uint16)
    acc = np.zeros(H, dtype=np.float64)
    for r, e in enumerate(ids):
        if not _valid(e, E):
            continue
        dq = f16_bits_to_f64(awq_dequant_parts(w2_codes[e], w2_scales[e], w2_zeros[e]))  # [H, I]
        y[r] = f64_to_f16_bits(dq @ f16_bits_to_f64(act_bits[r]))
        acc += np.float64(np.float32(router_w[r])) * f16_bits_to_f64(y[r])
    return f64_to_f16_bits(acc), y


def moe_awq_m1_ref(x_bits, ids, router_w, w13, w2, I):
    """Whole step.  w13 = (codes, scales_bits, zeros) [E, 2I, H]; w2 = (codes, scales_bits, zeros) [E, H, I].

    Returns (out f16 bits [H], act f16 bits [topk, I]).
    """
    act = moe_w13_stage_ref(x_bits, ids, *w13, I)
    out, _ = moe_w2_stage_ref(act, ids, router_w, *w2)
    return out, act


def moe_bruteforce(x, ids, router_w, W13, W2, I):
    """Pure-Python loops over already-dequantised float weights (lists), tiny shapes only.

    x: [H] floats; W13[e]: [2I][H]; W2[e]: [H][I]; float16 rounding via
    numpy.float16 scalars at the materialisation points.  Returns out as floats [H].
    """
    E = len(W13)
    H = len(x)
    out = [0.0] * H
    for r, e in enumerate(ids):
        if not (0 <= e < E):
            continue
        act = []
        for n in range(I):
            g = sum(x[k] * W13[e][n][k] for k in range(H))
            u = sum(x[k] * W13[e][n + I][k] for k in range(H))
            g = float(np.float16(g))
            u = float(np.float16(u))
            sg = g / (1.0 + math.exp(-g)) if g >= 0 else g * math.exp(g) / (1.0 + math.exp(g))
            act.append(float(np.float16(sg * u)))
        for o in range(H):
            yv = float(np.float16(sum(act[q] * W2[e][o][q] for q in range(I))))
            out[o] += float(np.float32(router_w[r])) * yv
    return [float(np.float16(v)) for v in out]
