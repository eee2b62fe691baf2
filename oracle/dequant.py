"""Dequantised-weight definitions (oracle; test infrastructure only).

These are the bit-exact targets of the library's debug decoders.
"""
import numpy as np
from .codecs import e4m3_to_f64, e2m1_to_f64, f16_bits_to_f64, f64_to_f16_bits
from .pack import block64_unpack, awq_unpack_bank


def fp8w_dequant(w, scale):
    """FP8 E4M3 per-output-channel weights -> float32.

    dq[n, k] = F8E4M3ToF32(w[n, k]) * scale[n]  (issue "tp>1 fp8w tail-MLP
    shard ...", sections "Mechanism on the tp>1 path" and "Logic anchor").
    w: uint8 [N, K]; scale: float32 [N].  The float64 product of a 4-bit and a
    24-bit significand is exact, so one rounding to float32 reproduces the
    float32 multiply.
    """
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return (e4m3_to_f64(w) * s[:, None]).astype(np.float32)


def nvfp4_inv_global(global_scale):
    """The runtime dequantisation factor 1/weight_global_scale, rounded once to float32
    (page "Qwen3.8-27B-NVFP4", section "NVFP4 numerics as implemented")."""
    return np.float32(1.0) / np.float32(global_scale)      # IEEE float32 division: one rounding


def nvfp4_dequant_parts(weight_packed, weight_scale, global_scale):
    """Three-level NVFP4 tensor -> float32, from the checkpoint tensors.

    weight_packed: uint8 [N, K/2], two E2M1 per byte, low nibble = earlier weight;
    weight_scale: uint8 E4M3 [N, K/16], one per 16 consecutive input channels;
    global_scale: float32, applied as 1/global_scale (page "Qwen3.8-27B-NVFP4",
    section "NVFP4 numerics as implemented").
    dq = RN_f32(e2m1(q) * e4m3(d) * RN_f32(1/gs)); the float64 product is exact.
    """
    wp = np.asarray(weight_packed, dtype=np.uint8)
    n, khalf = wp.shape
    k = khalf * 2
    nib = np.empty((n, k), dtype=np.uint8)
    nib[:, 0::2] = wp & 0x0F
    nib[:, 1::2] = wp >> 4
    d = e4m3_to_f64(np.asarray(weight_scale, dtype=np.uint8))          # [N, K/16]
    dk = np.repeat(d, 16, axis=1)                                       # [N, K]
    inv = np.float64(nvfp4_inv_global(global_scale))
    return (e2m1_to_f64(nib) * dk * inv).astype(np.float32)


def nvfp4_dequant(blk, global_scale):
    """Block64 records [N, K/64, 36] -> float32 [N, K] (same definition as above)."""
    wp, ws = block64_unpack(blk)
    return nvfp4_dequant_parts(wp, ws, global_scale)


def awq_dequant_bias(codes, scales_bits, bias_bits):
    """AWQ int4 group-32 from a stored per-group bias -> float16 bits.

    dq = RN_f16(q * s + b) with b the float16 group bias: one fused multiply-add
    in half precision (page "[Kernel][SM70] Add native-g32 AWQ QPN M1 operator",
    section "What it does": the half_fma(q, scale, half(-zero*scale)) boundary;
    the 4-byte {scale, bias} metadata stores that half bias directly).
    codes: uint8 [..., N, K] in 0..15; scales_bits, bias_bits: uint16 (f16 bits)
    [..., N, K/32].  Returns uint16 f16 bits [..., N, K].  q * s + b is exact in
    float64 (q < 16 and two half operands span far fewer than 53 bits), so the
    cast to float16 is the single rounding of the fused operation.
    """
    q = np.asarray(codes).astype(np.float64)
    sk = np.repeat(f16_bits_to_f64(scales_bits), 32, axis=-1)
    bk = np.repeat(f16_bits_to_f64(bias_bits), 32, axis=-1)
    return f64_to_f16_bits(q * sk + bk)


def awq_bias_bits(scales_bits, zeros):
    """The group bias RN_f16(-z * s) as float16 bits (the exact float64 product, rounded once)."""
    s = f16_bits_to_f64(scales_bits)
    z = np.asarray(zeros).astype(np.float64)
    return f64_to_f16_bits(-z * s)


def awq_dequant_parts(codes, scales_bits, zeros):
    """AWQ int4 group-32 from (codes, scales, uint8 zeros) -> float16 bits.

    dq = RN_f16(q * s + RN_f16(-z * s)) (same section as above: the bias is the
    zero times the scale, negated and rounded to half, then one half fma; not
    half((q-zero)*scale)).  zeros: uint8 [..., N, K/32].
    """
    return awq_dequant_bias(codes, scales_bits, awq_bias_bits(scales_bits, zeros))


def awq_dequant(bank, E, N, K, meta_layout=3):
    """Prepared bank -> f16 bits [E, N, K] (unpacks the documented bank layout).

    meta_layout 3 stores uint8 zeros and the bias is formed from them;
    meta_layout 4 stores the float16 bias itself, which is used as read.
    """
    codes, scales, meta = awq_unpack_bank(bank, E, N, K, meta_layout)
    if meta_layout == 3:
        return awq_dequant_parts(codes, scales, meta)
    return awq_dequant_bias(codes, scales, meta)
