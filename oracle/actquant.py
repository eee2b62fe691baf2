"""Per-token 8-bit activation quantization of the W4A8 variant (oracle; test infrastructure only).

Page "Qwen3.8-27B-NVFP4", section "Implemented execution path": the activations of the NVFP4 linears
are quantized per token, dynamically, into a small reusable workspace, and gate and up share one
quantization per token; section "Correctness and precision" reports that quantization as the dominant
error (1.458e-2).  The page's kernels use INT8 because SM75 has integer matrix units only.

Reading (the page leaves the 8-bit format to the hardware): on gfx950 the 8-bit matrix type that carries
a floating-point value is E4M3 ("fn", the same element format as the FP8 weights), so each token row is
quantized to E4M3 codes with one float scale per row.  The scale is the power of two 2^e for which the
row's largest magnitude lands in (224, 448] (448 being E4M3's largest finite value): scaling by 2^-e is
exact, so the only rounding is the encode itself, round to nearest with ties to the even code, and a
row of zeros keeps the scale 1.  The dequantized activation is code * 2^e, exactly.
"""
import math

import numpy as np

from .codecs import e4m3_fields_to_f64

E4M3_MAX = 448.0
# the 127 non-negative finite E4M3 values, increasing with the code (codes 0x00..0x7E)
_POS_VALUES = e4m3_fields_to_f64(np.arange(0x7F))


def token_exponent(amax):
    """Smallest integer e with amax <= 448 * 2^e (so amax * 2^-e lies in (224, 448]); 0 for amax == 0.

    Found from a first estimate and corrected by exact comparisons (448 * 2^e is exact in float64).
    """
    a = float(amax)
    if not (a > 0.0) or not math.isfinite(a):
        return 0
    e = math.ceil(math.log2(a / E4M3_MAX))
    while a > E4M3_MAX * 2.0 ** e:
        e += 1
    while a <= E4M3_MAX * 2.0 ** (e - 1):
        e -= 1
    return e


def e4m3_encode_rne(v):
    """float64 values with |v| <= 448 -> E4M3 codes: the nearest finite E4M3 value, ties to the even code.

    The sign is kept as the code's top bit (so -0.0, and negatives that round to zero, give 0x80).
    Values above 448 in magnitude saturate to 0x7E / 0xFE; NaN gives 0x7F.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_POS_VALUES, a, side="left")                  # first value >= a
    hi = np.minimum(hi, _POS_VALUES.size - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))          # ties: the even code
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(v), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(v), np.uint8(0x7F), code).astype(np.uint8)


def quant_e4m3_per_token(x):
    """x float64 [M, K] (exact values) -> (codes uint8 [M, K], scale float64 [M] = 2^e per row)."""
    x = np.atleast_2d(np.asarray(x, dtype=np.float64))
    scale = np.empty(x.shape[0], dtype=np.float64)
    codes = np.empty(x.shape, dtype=np.uint8)
    for m in range(x.shape[0]):
        e = token_exponent(np.max(np.abs(x[m])) if x.shape[1] else 0.0)
        scale[m] = 2.0 ** e
        codes[m] = e4m3_encode_rne(np.ldexp(x[m], -e))
    return codes, scale
