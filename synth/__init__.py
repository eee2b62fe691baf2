"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and writes them in the storage formats
a checkpoint would hold (E4M3 / E2M1 codes, float16 / bfloat16 bits, AWQ
codes with group scales and zeros).  It holds none of the method's arithmetic
(no dequantisation, no MLP) and imports neither the oracle nor the library.
Format encodings use library casts (torch float8_e4m3fn / bfloat16 /
numpy float16) except E2M1, which has no library cast on the CPU and is
encoded by nearest-value search over the format's published value set.

Every draw comes from numpy.random.default_rng(SeedSequence([config_id,
tensor_id])) in a fixed order; tensor ids: x=0, gate=1, up=2, down=3,
scales=4, ids=5, router=6.  Workload recipes (sizes and distributions follow
the three pages' shapes):

1. tiny FP8 W8A16 MLP, H=256, I=512, M in {1, 4}: x f32 N(0,1); codes uniform
   over the 254 non-NaN E4M3 bytes; per-row f32 scales 10^U(-3,-1).
2. FP8 E4M3 per-channel MLP, H=5120, I=17408, M=1: x = bf16(N(0,1));
   w ~ N(0, 0.02^2); s[n] = max|w[n,:]|/448; codes = E4M3(w/s).
3. NVFP4 MLP at the same shape, M=1: gs = 448*6/amax(W);
   d = E4M3(max|group16|/6 * gs) (at least the smallest subnormal);
   q = E2M1(w * gs / d).
4. the same NVFP4 weights with M in {512, 8192}; x = bf16(N(0,1)) with
   round(0.01*M) distinct rows scaled by 20 before rounding.
5. AWQ int4 g32 routed-expert step, E=512, top-k 10, W13 [2I=320, H=2560],
   W2 [H=2560, I=160]: w ~ N(0, 0.02^2); per group of 32 along K:
   s = f16((max-min)/15), z = clamp(round(-min/s), 0, 15),
   q = clamp(round(w/s) + z, 0, 15); x = f16(N(0,1)); ids uniform without
   replacement (int32); router weights = softmax of N(0,1) logits (f32).
"""
import numpy as np
import torch

T_X, T_GATE, T_UP, T_DOWN, T_SCALES, T_IDS, T_ROUTER = range(7)

E4M3_MAX = 448.0
E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)  # OCP MX E2M1 magnitudes, codes 0..7


def rng(config_id, tensor_id, extra=()):
    return np.random.default_rng(np.random.SeedSequence([int(config_id), int(tensor_id), *extra]))


# ---- storage encoders (library casts) ---------------------------------------------------------
def to_e4m3_codes(v):
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).clamp_(-E4M3_MAX, E4M3_MAX)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def e4m3_codes_as_f32(codes):
    """Library decode of E4M3 codes (torch), used only to build the next quantisation level."""
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def to_bf16_bits(v):
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_f16_bits(v):
    return np.asarray(v, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_e2m1_codes(v):
    """Nearest E2M1 code, ties to the even code, saturating at +-6; sign in bit 3.

    The value set {0, .5, 1, 1.5, 2, 3, 4, 6} has spacing 0.5 below 2, 1 in [2, 4)
    and 2 from 4: round-half-even at that spacing and offset into the code range
    (the even code is the even multiple at each tie).
    """
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    a = t.abs()
    c = torch.where(a < 2, torch.round(a * 2),
                    torch.where(a < 4, torch.round(a) + 2, torch.clamp(torch.round(a * 0.5) + 4, max=7)))
    sign = torch.signbit(t).to(torch.uint8) << 3
    return (c.to(torch.uint8) | sign).numpy()


# ---- workloads ---------------------------------------------------------------------------------
def fp8_tiny(M, H=256, I=512, config_id=1):
    """Recipe 1.  Returns dict of numpy arrays (x f32 [M,H]; w* uint8; s* f32)."""
    valid = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    out = {"x": rng(config_id, T_X, (M,)).standard_normal((M, H)).astype(np.float32)}
    shapes = {"gate": (I, H), "up": (I, H), "down": (H, I)}
    for name, tid in (("gate", T_GATE), ("up", T_UP), ("down", T_DOWN)):
        r = rng(config_id, tid)
        out["w_" + name] = valid[r.integers(0, valid.size, size=shapes[name])]
        out["s_" + name] = (10.0 ** r.uniform(-3.0, -1.0, size=shapes[name][0])).astype(np.float32)
    return out


def _fp8_channel_quant(w):
    s = (np.max(np.abs(w), axis=1) / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    return to_e4m3_codes(w / s[:, None]), s


def fp8_mlp(M=1, H=5120, I=17408, config_id=2, std=0.02):
    """Recipe 2: x bf16 bits [M,H]; per-channel FP8 gate/up [I,H], down [H,I]."""
    out = {"x_bits": to_bf16_bits(rng(config_id, T_X, (M,)).standard_normal((M, H), dtype=np.float32))}
    shapes = {"gate": (I, H), "up": (I, H), "down": (H, I)}
    for name, tid in (("gate", T_GATE), ("up", T_UP), ("down", T_DOWN)):
        w = rng(config_id, tid).standard_normal(shapes[name], dtype=np.float32) * np.float32(std)
        out["w_" + name], out["s_" + name] = _fp8_channel_quant(w)
        del w
    return out


def nvfp4_tensor(N, K, config_id, tensor_id, std=0.02):
    """Recipe 3 for one tensor -> (weight_packed [N,K/2] u8, weight_scale [N,K/16] u8, global_scale f32)."""
    w = torch.from_numpy(rng(config_id, tensor_id).standard_normal((N, K), dtype=np.float32))
    w.mul_(std)
    amax = np.float32(w.abs().max().item())
    gs = np.float32(E4M3_MAX * 6.0) / amax
    g = w.view(N, K // 16, 16)
    gmax = g.abs().amax(dim=2)
    d_codes = to_e4m3_codes((gmax / 6.0 * float(gs)).numpy())
    d_codes = np.where(d_codes == 0, np.uint8(1), d_codes).astype(np.uint8)   # keep the group scale positive
    d_val = torch.from_numpy(e4m3_codes_as_f32(d_codes))
    q = torch.from_numpy(to_e2m1_codes((g * (float(gs) / d_val)[:, :, None]).numpy())).view(N, K)
    del g, w
    packed = (q[:, 0::2] | (q[:, 1::2] << 4)).contiguous().numpy()
    return packed, d_codes, gs


def nvfp4_mlp_weights(H=5120, I=17408, config_id=3):
    out = {}
    for name, tid, shp in (("gate", T_GATE, (I, H)), ("up", T_UP, (I, H)), ("down", T_DOWN, (H, I))):
        out["wp_" + name], out["ws_" + name], out["gs_" + name] = nvfp4_tensor(*shp, config_id, tid)
    return out


def nvfp4_x(M, H=5120, config_id=3, outlier_frac=0.0, outlier_scale=20.0):
    """bf16 bits [M,H] from N(0,1); round(outlier_frac*M) distinct rows scaled before rounding."""
    r = rng(config_id, T_X, (M,))
    x = r.standard_normal((M, H), dtype=np.float32)
    n_out = int(round(outlier_frac * M))
    rows = np.sort(r.choice(M, size=n_out, replace=False)) if n_out else np.zeros(0, dtype=np.int64)
    x[rows] *= np.float32(outlier_scale)
    return to_bf16_bits(x), rows


def awq_quant(w):
    """Asymmetric min-max int4 quantisation per group of 32 along the last axis.

    w float32 [..., N, K] -> (codes u8 [..., N, K], scales f16 bits [..., N, K/32], zeros u8 [..., N, K/32]).
    """
    shp = w.shape
    g = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).view(*shp[:-1], shp[-1] // 32, 32)
    mn = g.amin(dim=-1)
    mx = g.amax(dim=-1)
    s16 = ((mx - mn) / 15.0).to(torch.float16)
    s16 = torch.where(s16 > 0, s16, torch.tensor(1e-3, dtype=torch.float16))
    s = s16.float()
    z = torch.clamp(torch.round(-mn / s), 0, 15)
    q = torch.clamp(torch.round(g / s[..., None]) + z[..., None], 0, 15).to(torch.uint8)
    return (q.view(shp).numpy(), s16.numpy().view(np.uint16), z.to(torch.uint8).numpy())


def awq_moe(E=512, topk=10, H=2560, I=160, config_id=5, std=0.02, expert_chunk=64):
    """Recipe 5: per-expert W13 [2I,H] and W2 [H,I] quantised weights plus x, ids, router weights."""
    out = {}
    for name, tid, shp in (("w13", T_GATE, (2 * I, H)), ("w2", T_DOWN, (H, I))):
        codes = np.empty((E, *shp), dtype=np.uint8)
        scales = np.empty((E, shp[0], shp[1] // 32), dtype=np.uint16)
        zeros = np.empty((E, shp[0], shp[1] // 32), dtype=np.uint8)
        r = rng(config_id, tid)
        for e0 in range(0, E, expert_chunk):
            e1 = min(E, e0 + expert_chunk)
            w = r.standard_normal((e1 - e0, *shp), dtype=np.float32) * np.float32(std)
            codes[e0:e1], scales[e0:e1], zeros[e0:e1] = awq_quant(w)
        out[name] = (codes, scales, zeros)
    out["x_bits"] = to_f16_bits(rng(config_id, T_X).standard_normal(H, dtype=np.float32))
    out["ids"] = rng(config_id, T_IDS).choice(E, size=topk, replace=False).astype(np.int32)
    logits = rng(config_id, T_ROUTER).standard_normal(topk).astype(np.float64)
    p = np.exp(logits - logits.max())
    out["router_w"] = (p / p.sum()).astype(np.float32)
    return out


def awq_rotating_ids(n_calls, topk, E, pool=480, config_id=5):
    """ids for n_calls consecutive calls cycling through `pool` distinct experts (topk per call)."""
    perm = rng(config_id, T_IDS, (pool,)).permutation(E)[:pool].astype(np.int32)
    return np.stack([perm[(c * topk + np.arange(topk)) % pool] for c in range(n_calls)])
