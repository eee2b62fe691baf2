"""Weight packers, written independently of the library (oracle; test infrastructure only)."""
import numpy as np

BLOCK64_BYTES = 36


def block64_pack(weight_packed, weight_scale):
    """Checkpoint NVFP4 tensors -> 36-byte records [N, K/64, 36].

    Page "Qwen3.8-27B-NVFP4", section "NVFP4 numerics as implemented": a
    record covers 64 consecutive logical weights of one output row and holds
    d[4] (the four E4M3 group-16 scales, in K order) followed by qs[32] (the
    64 E2M1 values, two per byte, low nibble = earlier weight).  Records are
    row-major over [N, K/64].
    weight_packed: uint8 [N, K/2]; weight_scale: uint8 [N, K/16].
    """
    wp = np.asarray(weight_packed, dtype=np.uint8)
    ws = np.asarray(weight_scale, dtype=np.uint8)
    n, khalf = wp.shape
    k = khalf * 2
    if k % 64 or ws.shape != (n, k // 16):
        raise ValueError("NVFP4 Block64 needs K % 64 == 0 and scales [N, K/16]")
    nb = k // 64
    blk = np.empty((n, nb, BLOCK64_BYTES), dtype=np.uint8)
    blk[:, :, 0:4] = ws.reshape(n, nb, 4)
    blk[:, :, 4:36] = wp.reshape(n, nb, 32)
    return blk


def block64_unpack(blk):
    """Inverse of block64_pack: records [N, K/64, 36] -> (weight_packed [N, K/2], weight_scale [N, K/16])."""
    b = np.asarray(blk, dtype=np.uint8)
    n, nb, rb = b.shape
    if rb != BLOCK64_BYTES:
        raise ValueError("record size must be 36 bytes")
    ws = np.ascontiguousarray(b[:, :, 0:4]).reshape(n, nb * 4)
    wp = np.ascontiguousarray(b[:, :, 4:36]).reshape(n, nb * 32)
    return wp, ws


def _round16(v):
    return (v + 15) // 16 * 16


def awq_bank_layout(N, K, meta_layout=3):
    """Byte offsets inside one expert's slice of a prepared AWQ bank.

    The pages name the metadata sizes (3 bytes {f16 scale, u8 zero} or 4 bytes
    {f16 scale, f16 bias} per group of 32 -- page "[Kernel][SM70] Add
    native-g32 AWQ QPN M1 operator", section "What it does") but not the byte
    order, so this layout is this project's own, documented choice:

      codes  : [N][K/2] uint8, row-major; byte j of row n holds k = 2j (low
               nibble) and k = 2j+1 (high nibble)
      scales : [N][K/32] float16, row-major               (at scale_off)
      zeros  : [N][K/32] uint8     (meta_layout 3)        (at meta2_off)
      bias   : [N][K/32] float16 = RN_f16(-z*s) (layout 4) (at meta2_off)

    each plane starting on a 16-byte boundary; experts are stacked with
    stride ``expert_bytes``.
    """
    if K % 32:
        raise ValueError("AWQ group size is 32: K % 32 == 0")
    G = K // 32
    codes = N * K // 2
    scale_off = _round16(codes)
    meta2_off = scale_off + _round16(2 * N * G)
    meta2 = N * G if meta_layout == 3 else 2 * N * G
    if meta_layout not in (3, 4):
        raise ValueError("meta_layout must be 3 or 4")
    return dict(G=G, scale_off=scale_off, meta2_off=meta2_off,
                expert_bytes=meta2_off + _round16(meta2))


def awq_pack_bank(codes, scales_bits, zeros, meta_layout=3):
    """(codes [E,N,K] in 0..15, scales f16 bits [E,N,K/32], zeros u8 [E,N,K/32]) -> bank bytes."""
    c = np.asarray(codes, dtype=np.uint8)
    E, N, K = c.shape
    L = awq_bank_layout(N, K, meta_layout)
    G = L["G"]
    sb = np.asarray(scales_bits, dtype=np.uint16).reshape(E, N, G)
    z = np.asarray(zeros, dtype=np.uint8).reshape(E, N, G)
    bank = np.zeros((E, L["expert_bytes"]), dtype=np.uint8)
    packed = (c[:, :, 0::2] & 0x0F) | ((c[:, :, 1::2] & 0x0F) << 4)
    bank[:, : N * K // 2] = packed.reshape(E, -1)
    bank[:, L["scale_off"]: L["scale_off"] + 2 * N * G] = sb.reshape(E, -1).view(np.uint8).reshape(E, -1)
    if meta_layout == 3:
        bank[:, L["meta2_off"]: L["meta2_off"] + N * G] = z.reshape(E, -1)
    else:
        # bias = RN_f16(-z * s): exact product in float64, one rounding to half.
        s64 = sb.view(np.float16).astype(np.float64)
        bias = (-z.astype(np.float64) * s64).astype(np.float16).view(np.uint16)
        bank[:, L["meta2_off"]: L["meta2_off"] + 2 * N * G] = bias.reshape(E, -1).view(np.uint8).reshape(E, -1)
    return bank.reshape(-1)


def awq_unpack_bank(bank, E, N, K, meta_layout=3):
    """Inverse of awq_pack_bank -> (codes [E,N,K], scales f16 bits [E,N,G], zeros u8 [E,N,G]).

    For meta_layout 4 the zero is not stored; the third value returned is
    then the f16 bias bits [E,N,G] (decode them with dequant.awq_dequant_bias).
    """
    L = awq_bank_layout(N, K, meta_layout)
    G = L["G"]
    b = np.asarray(bank, dtype=np.uint8).reshape(E, L["expert_bytes"])
    packed = b[:, : N * K // 2].reshape(E, N, K // 2)
    codes = np.empty((E, N, K), dtype=np.uint8)
    codes[:, :, 0::2] = packed & 0x0F
    codes[:, :, 1::2] = packed >> 4
    sb = np.ascontiguousarray(b[:, L["scale_off"]: L["scale_off"] + 2 * N * G]).view(np.uint16).reshape(E, N, G)
    if meta_layout == 3:
        z = np.ascontiguousarray(b[:, L["meta2_off"]: L["meta2_off"] + N * G]).reshape(E, N, G)
    else:
        z = np.ascontiguousarray(b[:, L["meta2_off"]: L["meta2_off"] + 2 * N * G]).view(np.uint16).reshape(E, N, G)
    return codes, sb, z
