"""Element decoders written from the bit-field definitions (oracle; test infrastructure only).

* E4M3 "fn" (OCP 8-bit float, bias 7, no infinities, NaN only at S.1111.111):
  named as the checkpoint's weight and scale element type -- issue "tp>1 fp8w
  tail-MLP shard ...", section "Claim" (e4m3fn bytes), and page
  "Qwen3.8-27B-NVFP4", section "Checkpoint specification" (scale dtype
  float8_e4m3fn).
* E2M1 (OCP 4-bit float, bias 1, no inf/NaN): page "Qwen3.8-27B-NVFP4",
  section "NVFP4 numerics as implemented" (two E2M1 values per byte).
* bfloat16 / float16 activations: exact widening of the stored bits.
"""
import numpy as np


def e4m3_fields_to_f64(codes):
    """Decode E4M3fn bytes to float64 exactly from the bit fields.

    value = (-1)^s * 2^(e-7) * (1 + m/8) for e > 0, (-1)^s * m * 2^-9 for e == 0,
    NaN for e == 15 and m == 7.  0x80 decodes to -0.0.
    """
    c = np.asarray(codes).astype(np.int64)
    s = c >> 7
    e = (c >> 3) & 15
    m = c & 7
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))
    sub = m * 2.0 ** -9
    mag = np.where(e == 0, sub, normal)
    val = np.where(s == 1, -mag, mag)
    return np.where((e == 15) & (m == 7), np.nan, val)


def e2m1_fields_to_f64(nibbles):
    """Decode E2M1 nibbles (0..15) to float64 exactly from the bit fields.

    value = (-1)^s * 2^(e-1) * (1 + m/2) for e > 0, (-1)^s * m * 0.5 for e == 0.
    Magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6}; code 8 decodes to -0.0.
    """
    c = np.asarray(nibbles).astype(np.int64) & 15
    s = c >> 3
    e = (c >> 1) & 3
    m = c & 1
    normal = np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int32))
    mag = np.where(e == 0, m * 0.5, normal)
    return np.where(s == 1, -mag, mag)


# Large tensors are decoded through the 256 / 16 values the field decoders give for
# every code (same definition, evaluated once per code instead of once per element).
_E4M3_ALL = e4m3_fields_to_f64(np.arange(256))
_E2M1_ALL = e2m1_fields_to_f64(np.arange(16))


def e4m3_to_f64(codes):
    """E4M3fn codes (uint8 array) -> float64, by the bit-field definition above."""
    return _E4M3_ALL[np.asarray(codes, dtype=np.uint8)]


def e2m1_to_f64(nibbles):
    """E2M1 codes (0..15) -> float64, by the bit-field definition above."""
    return _E2M1_ALL[np.asarray(nibbles).astype(np.uint8) & 15]


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns (uint16) -> float64: the bits are the top half of a float32."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


def f16_bits_to_f64(bits):
    """IEEE binary16 bit patterns (uint16) -> float64 (exact)."""
    return np.asarray(bits).astype(np.uint16).view(np.float16).astype(np.float64)


def f64_to_f16_bits(v):
    """Round float64 to the nearest binary16 (ties to even) and return the bits."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)
