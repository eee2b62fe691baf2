"""Device decoders and packers are bit-exact with the oracle (exhaustive code tables)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_mlp_amd as wq
from golden import hex_bytes, load as golden
from gpu_common import DEV, dev, host, same_bits_f32

pytestmark = pytest.mark.gpu


def test_fp8_decoder_all_256_codes():
    r = np.random.default_rng(11)
    codes = np.stack([r.permutation(256) for _ in range(24)]).astype(np.uint8)     # every code in every row
    s = r.uniform(1e-3, 1e-1, 24).astype(np.float32)
    s[0] = 1.0
    got = host(wq.fp8w_dequant_f32(dev(codes), dev(s)))
    assert same_bits_f32(got, oracle.fp8w_dequant(codes, s))


def test_nvfp4_decoder_16_codes_x_256_scales():
    N, K = 256, 64
    ws = np.repeat(np.arange(256, dtype=np.uint8)[:, None], K // 16, axis=1)      # row n: every group scale = n
    nib = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))                      # all 16 codes in every group
    wp = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    blk = oracle.block64_pack(wp, ws)
    for gs in (1.0, 3.7e3, 0.37):
        got = host(wq.nvfp4_dequant_f32(dev(blk), gs))
        assert same_bits_f32(got, oracle.nvfp4_dequant(blk, np.float32(gs))), gs


@pytest.mark.parametrize("ml", [3, 4])
def test_awq_decoder_codes_x_zeros_x_scales(ml):
    E, N, K = 2, 256, 64
    r = np.random.default_rng(3)
    codes = np.tile(np.arange(16, dtype=np.uint8), (E, N, K // 16))
    zeros = r.integers(0, 16, size=(E, N, K // 32)).astype(np.uint8)
    zeros[0, :16, 0] = np.arange(16)
    scales = r.uniform(1e-4, 0.05, size=(E, N, K // 32)).astype(np.float16)
    scales[1, :8, :] = np.float16(6e-5)                                             # half subnormal scales
    bank = oracle.awq_pack_bank(codes, scales.view(np.uint16), zeros, ml)
    got = host(wq.awq_dequant_f16(dev(bank), E, N, K, ml)).view(np.uint16)
    want = oracle.awq_dequant_parts(codes, scales.view(np.uint16), zeros)
    bad = np.argwhere(got != want)
    detail = [(tuple(int(v) for v in b), int(codes[tuple(b)]), int(zeros[b[0], b[1], b[2] // 32]),
               float(scales[b[0], b[1], b[2] // 32]), hex(got[tuple(b)]), hex(want[tuple(b)])) for b in bad[:6]]
    assert bad.size == 0, f"{len(bad)} mismatches, e.g. (idx, q, z, s, got, want): {detail}"


def test_nvfp4_packer_bytes():
    wp, ws, gs = synth.nvfp4_tensor(96, 640, 3, 7)
    got = host(wq.nvfp4_pack_block64(dev(wp), dev(ws)))
    assert np.array_equal(got, oracle.block64_pack(wp, ws))


def test_nvfp4_packer_worked_example():
    # the page's 36-byte record, written out by hand (tests/golden/nvfp4_block64_record.txt)
    g = golden("nvfp4_block64_record.txt")
    codes = (np.arange(64) % 16).astype(np.uint8)[None, :]
    wp = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    ws = np.frombuffer(hex_bytes(g["example_scales"]), dtype=np.uint8)[None, :].copy()
    got = host(wq.nvfp4_pack_block64(dev(wp), dev(ws)))
    assert got.tobytes() == hex_bytes(g["example_record"])


@pytest.mark.parametrize("ml", [3, 4])
def test_awq_packer_bytes(ml):
    d = synth.awq_moe(E=5, topk=2, H=256, I=96)
    for c, s, z in (d["w13"], d["w2"]):
        got = host(wq.awq_pack_bank(dev(c), dev(s.view(np.int16)), dev(z), ml))
        assert np.array_equal(got, oracle.awq_pack_bank(c, s, z, ml))
