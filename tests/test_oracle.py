"""Pins of the CPU oracle against facts outside itself (no GPU needed).

Each test ties an oracle function to a library routine, a published table, a
closed form, an invariant or a brute-force evaluation, so that a dropped term,
a wrong sign or index, or a transposed operand fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from golden import hex_bytes, load as golden
from oracle import codecs, dequant, pack, mlp, moe

pytestmark = pytest.mark.cpu


def torch_e4m3(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).float().numpy()


def same_bits(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_nan = np.isnan(a) & np.isnan(b)
    eq = (a == b) & (np.signbit(a) == np.signbit(b))
    return np.all(both_nan | eq)


# ---- E4M3 ---------------------------------------------------------------------------------------
def test_e4m3_all_256_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    assert same_bits(codecs.e4m3_to_f64(codes), torch_e4m3(codes).astype(np.float64))


def test_e4m3_special_values():
    v = codecs.e4m3_to_f64(np.array([0x7E, 0x01, 0x07, 0x08, 0x38, 0x80, 0x7F, 0xFF, 0xFE], dtype=np.uint8))
    assert v[0] == 448.0                       # largest finite (the /448 of the per-channel scale)
    assert v[1] == 2.0 ** -9                   # smallest subnormal
    assert v[2] == 7 * 2.0 ** -9               # largest subnormal
    assert v[3] == 2.0 ** -6                   # smallest normal
    assert v[4] == 1.0
    assert v[5] == 0.0 and math.copysign(1, v[5]) < 0
    assert np.isnan(v[6]) and np.isnan(v[7])
    assert v[8] == -448.0
    finite = codecs.e4m3_to_f64(np.arange(256, dtype=np.uint8))
    assert np.sum(np.isnan(finite)) == 2       # fn variant: NaN only at S.1111.111, no infinities
    assert not np.any(np.isinf(finite))


# ---- E2M1 ---------------------------------------------------------------------------------------
# The OCP Microscaling spec's E2M1 table: codes 0..7 (sign bit clear).
OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table():
    v = codecs.e2m1_to_f64(np.arange(16))
    assert list(v[:8]) == OCP_E2M1
    assert list(-v[8:]) == OCP_E2M1
    assert math.copysign(1, v[8]) < 0          # code 8 is -0.0
    assert v.max() == 6.0                      # the /6 of the group-scale recipe


def test_e2m1_values_are_exact_in_e4m3():
    # every E2M1 magnitude survives an E4M3 round trip through the library cast (4-bit significand)
    v = codecs.e2m1_to_f64(np.arange(16)).astype(np.float32)
    assert same_bits(torch_e4m3(synth.to_e4m3_codes(v)), v)


# ---- bf16 / f16 ---------------------------------------------------------------------------------
def test_bf16_and_f16_widening_match_torch():
    r = np.random.default_rng(0)
    bits = r.integers(0, 1 << 16, size=20000).astype(np.uint16)
    tb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    th = torch.from_numpy(bits.view(np.int16)).view(torch.float16).double().numpy()
    assert same_bits(codecs.bf16_bits_to_f64(bits), tb)
    assert same_bits(codecs.f16_bits_to_f64(bits), th)


# ---- dequantised weights --------------------------------------------------------------------------
def test_fp8w_dequant_matches_torch_f32_multiply():
    d = synth.fp8_tiny(1)
    got = dequant.fp8w_dequant(d["w_gate"], d["s_gate"])
    ref = (torch.from_numpy(torch_e4m3(d["w_gate"])) * torch.from_numpy(d["s_gate"])[:, None]).numpy()
    assert got.dtype == np.float32 and np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_nvfp4_dequant_matches_table_times_torch_scales():
    wp, ws, gs = synth.nvfp4_tensor(48, 192, 3, 9)
    got = dequant.nvfp4_dequant(pack.block64_pack(wp, ws), gs)
    nib = np.stack([wp & 15, wp >> 4], axis=-1).reshape(48, 192)
    table = np.array(OCP_E2M1 + [-v for v in OCP_E2M1], dtype=np.float32)
    q = torch.from_numpy(table[nib])
    d = torch.from_numpy(np.repeat(torch_e4m3(ws), 16, axis=1))
    inv = torch.tensor(np.float32(1.0) / np.float32(gs), dtype=torch.float32)  # f32 division rounds once
    ref = ((q * d) * inv).numpy()                                               # q*d exact in f32
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def _nearest_f16_exact(fr):
    """Round an exact Fraction to binary16 by searching neighbours (ties to even mantissa)."""
    approx = np.float16(float(fr))
    cands = {approx, np.nextafter(approx, np.float16(np.inf)), np.nextafter(approx, np.float16(-np.inf))}
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        err = abs(Fraction(float(c)) - fr)
        key = (err, int(np.array(c).view(np.uint16)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_awq_dequant_single_rounding_fma():
    r = np.random.default_rng(5)
    q = r.integers(0, 16, size=(1, 2000)).astype(np.uint8)
    s = r.uniform(1e-4, 2e-2, size=(1, 2000)).astype(np.float16)
    z = r.integers(0, 16, size=(1, 2000)).astype(np.uint8)
    # one group per element: repeat codes 32x along K and take every 32nd result
    got = codecs.f16_bits_to_f64(dequant.awq_dequant_parts(
        np.repeat(q, 32, axis=1), s.view(np.uint16), z))[0, ::32]
    n_diff_naive = 0
    for i in range(2000):
        sf = Fraction(float(s[0, i]))
        bias = _nearest_f16_exact(-int(z[0, i]) * sf)
        want = _nearest_f16_exact(int(q[0, i]) * sf + Fraction(float(bias)))
        assert got[i] == float(want), i
        naive = _nearest_f16_exact((int(q[0, i]) - int(z[0, i])) * sf)
        n_diff_naive += float(naive) != float(want)
    assert n_diff_naive > 0      # the fma boundary is observably not half((q - z) * s)


# ---- packers --------------------------------------------------------------------------------------
def test_block64_record_worked_example():
    # the page's struct, written out by hand for one 64-weight row (tests/golden/nvfp4_block64_record.txt)
    g = golden("nvfp4_block64_record.txt")
    assert int(g["record_bytes"]) == int(g["d_count"]) + int(g["qs_bytes"]) == 36
    assert g["nibble_order"] == "low_first" and g["example_codes"] == "k mod 16"
    K = int(g["weights_per_record"])
    codes = (np.arange(K) % 16).astype(np.uint8)[None, :]
    wp = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    ws = np.frombuffer(hex_bytes(g["example_scales"]), dtype=np.uint8)[None, :]
    assert ws.shape[1] == K // int(g["group_size"])
    blk = pack.block64_pack(wp, ws)
    assert blk.tobytes() == hex_bytes(g["example_record"])
    rec = hex_bytes(g["example_record"])
    d0, q0 = int(g["d_offset"]), int(g["qs_offset"])
    assert rec[d0:d0 + 4] == hex_bytes(g["example_scales"]) and len(rec[q0:]) == int(g["qs_bytes"])


def test_block64_struct_layout():
    N, K = 3, 256
    ws = (np.arange(N * K // 16, dtype=np.uint8).reshape(N, K // 16) + 1)
    k = np.arange(K)
    codes = np.tile((k % 16).astype(np.uint8), (N, 1))          # weight k holds code k % 16
    wp = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    blk = pack.block64_pack(wp, ws)
    assert blk.shape == (N, K // 64, 36)
    for n in range(N):
        for b in range(K // 64):
            assert list(blk[n, b, :4]) == list(ws[n, 4 * b: 4 * b + 4])      # d[4] first, K order
            for j in range(32):
                assert blk[n, b, 4 + j] & 15 == (64 * b + 2 * j) % 16       # low nibble = earlier weight
                assert blk[n, b, 4 + j] >> 4 == (64 * b + 2 * j + 1) % 16
    wp2, ws2 = pack.block64_unpack(blk)
    assert np.array_equal(wp2, wp) and np.array_equal(ws2, ws)


@pytest.mark.parametrize("kk", [0, 15, 16, 31, 32, 63, 64, 127, 191, 255])
def test_nvfp4_one_hot_boundary_reads(kk):
    N, K = 4, 256
    ws = np.full((N, K // 16), 0x38, dtype=np.uint8)                 # 1.0 everywhere
    ws[:, kk // 16] = 0x40 + (kk // 16 % 8)                             # a distinct scale on the hot group
    codes = np.zeros((N, K), dtype=np.uint8)
    codes[:, kk] = 0x7                                                   # 6.0
    wp = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    dq = dequant.nvfp4_dequant(pack.block64_pack(wp, ws), np.float32(1.0))
    nz = np.argwhere(dq != 0)
    assert set(nz[:, 1]) == {kk} and len(nz) == N
    assert np.all(dq[:, kk] == np.float32(6.0) * torch_e4m3(ws[0, kk // 16]))


def test_awq_bank_round_trip_and_offsets():
    d = synth.awq_moe(E=3, topk=2, H=128, I=64)
    for name, (N, K) in (("w13", (128, 128)), ("w2", (128, 64))):
        c, s, z = d[name]
        for layout in (3, 4):
            bank = pack.awq_pack_bank(c, s, z, layout)
            L = pack.awq_bank_layout(N, K, layout)
            assert bank.size == 3 * L["expert_bytes"]
            c2, s2, m2 = pack.awq_unpack_bank(bank, 3, N, K, layout)
            assert np.array_equal(c2, c) and np.array_equal(s2, s)
            if layout == 3:
                assert np.array_equal(m2, z)
            else:   # bias = RN_f16(-z*s)
                want = (-(z.astype(np.float64)) * s.view(np.float16).astype(np.float64)).astype(np.float16)
                assert np.array_equal(m2, want.view(np.uint16))
    # sizes at the routed-expert shape: the metadata bytes per group of 32 that the pull request names
    # (tests/golden/awq_metadata_layouts.txt), on top of the packed codes
    g = golden("awq_metadata_layouts.txt")
    for layout in (3, 4):
        per_group = int(g[f"layout_{layout}"].split()[0].split("=")[1])
        assert per_group == layout
        L13 = pack.awq_bank_layout(320, 2560, layout)
        L2 = pack.awq_bank_layout(2560, 160, layout)
        assert L13["expert_bytes"] == 409600 + 320 * 80 * per_group
        assert L2["expert_bytes"] == 204800 + 2560 * 5 * per_group


@pytest.mark.parametrize("kk", [int(v) for v in golden("awq_one_hot_k.txt")["indices"].split()])
def test_awq_one_hot_boundary_reads(kk):
    # K and the indices the pull request's test plan reads (tests/golden/awq_one_hot_k.txt)
    E, N, K = 2, 8, int(golden("awq_one_hot_k.txt")["K"])
    codes = np.full((E, N, K), 8, dtype=np.uint8)
    zeros = np.full((E, N, K // 32), 8, dtype=np.uint8)                 # q == z -> exactly 0
    scales = np.full((E, N, K // 32), np.float16(0.25)).view(np.uint16)
    codes[:, :, kk] = 11
    bank = pack.awq_pack_bank(codes, scales, zeros, 3)
    dq = codecs.f16_bits_to_f64(dequant.awq_dequant(bank, E, N, K, 3))
    nz = np.argwhere(dq != 0)
    assert set(nz[:, 2]) == {kk} and np.all(dq[:, :, kk] == 0.75)


def test_awq_layout4_bank_decodes_like_the_parts():
    # the 4-byte layout stores RN_f16(-z*s) itself; decoding it must give the 3-byte layout's values bitwise
    d = synth.awq_moe(E=3, topk=2, H=128, I=64)
    for name, (E, N, K) in (("w13", (3, 128, 128)), ("w2", (3, 128, 64))):
        c, s, z = d[name]
        want = dequant.awq_dequant_parts(c, s, z)
        for layout in (3, 4):
            got = dequant.awq_dequant(pack.awq_pack_bank(c, s, z, layout), E, N, K, layout)
            assert np.array_equal(got, want), (name, layout)


@pytest.mark.parametrize("kk", [int(v) for v in golden("awq_one_hot_k.txt")["indices"].split()])
def test_awq_layout4_one_hot_boundary_reads(kk):
    # the same K indices as the 3-byte case, read through the stored-bias layout; a distinct non-zero
    # bias (z = 3) on every group makes a misplaced bias plane visible
    E, N, K = 2, 8, int(golden("awq_one_hot_k.txt")["K"])
    codes = np.full((E, N, K), 3, dtype=np.uint8)
    zeros = np.full((E, N, K // 32), 3, dtype=np.uint8)                 # q == z -> exactly 0
    scales = np.full((E, N, K // 32), np.float16(0.125)).view(np.uint16)
    scales[:, :, kk // 32] = np.float16(0.5).view(np.uint16)            # the hot group's own scale
    codes[:, :, kk] = 9
    dq = codecs.f16_bits_to_f64(dequant.awq_dequant(pack.awq_pack_bank(codes, scales, zeros, 4), E, N, K, 4))
    nz = np.argwhere(dq != 0)
    assert set(nz[:, 2]) == {kk} and np.all(dq[:, :, kk] == 3.0)        # (9 - 3) * 0.5


# ---- MLP ------------------------------------------------------------------------------------------
def test_silu_closed_forms():
    z = np.array([-800.0, -30.0, -1.0, 0.0, 1.0, 30.0, 800.0])
    s = mlp.silu(z)
    assert s[3] == 0.0 and s[-1] == 800.0 and abs(s[0]) < 1e-300
    assert abs(s[4] - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    zz = np.linspace(-40, 40, 801)
    assert np.allclose(mlp.silu(zz) - mlp.silu(-zz), zz, rtol=0, atol=1e-12)   # z*sig(z) + z*sig(-z) = z


@pytest.mark.parametrize("M", [1, 4])
def test_fp8_mlp_matches_pure_python_bruteforce(M):
    d = synth.fp8_tiny(M)
    ref = mlp.mlp_fp8w_ref(d["x"], d["w_gate"], d["s_gate"], d["w_up"], d["s_up"], d["w_down"], d["s_down"])

    def wt(w, s):   # independent dequantisation: library decode, float64 multiply
        return (torch_e4m3(w).astype(np.float64) * s.astype(np.float64)[:, None]).tolist()

    bf = mlp.mlp_bruteforce(d["x"].astype(np.float64).tolist(), wt(d["w_gate"], d["s_gate"]),
                            wt(d["w_up"], d["s_up"]), wt(d["w_down"], d["s_down"]))
    err, scale = oracle.normwise_rel_err(ref, np.array(bf))
    assert scale > 1e-3 and err < 1e-12


def test_nvfp4_mlp_matches_bruteforce_small():
    H, I = 128, 64
    W = {n: synth.nvfp4_tensor(*shp, 3, t) for n, t, shp in (("g", 1, (I, H)), ("u", 2, (I, H)), ("d", 3, (H, I)))}
    xb, _ = synth.nvfp4_x(2, H)
    x = codecs.bf16_bits_to_f64(xb)
    ref = mlp.mlp_nvfp4_ref(x, *(v for n in "gud" for v in (pack.block64_pack(*W[n][:2]), W[n][2])))
    table = np.array(OCP_E2M1 + [-v for v in OCP_E2M1])

    def wt(wp, ws, gs):
        nib = np.stack([wp & 15, wp >> 4], axis=-1).reshape(wp.shape[0], -1)
        inv = float(np.float32(1.0) / np.float32(gs))
        return (table[nib] * np.repeat(torch_e4m3(ws).astype(np.float64), 16, axis=1) * inv).tolist()

    bf = mlp.mlp_bruteforce(x.tolist(), wt(*W["g"]), wt(*W["u"]), wt(*W["d"]))
    err, scale = oracle.normwise_rel_err(ref, np.array(bf))
    assert scale > 1e-3 and err < 1e-12


# ---- the MLP at the decode workloads' full size (hidden 5120, intermediate 17408), sampled -------------
# The oracle's full-size act and out against pure-Python sums with weights decoded by other means (torch's
# float8 cast; the E2M1 table times that cast for NVFP4): act on sampled intermediate rows from x, out on
# sampled output rows from the oracle's own act (pinned by the first check).  Indices include both ends.
FULL_I_SAMPLES = [0, 1, 4095, 8704, 13001, 17406, 17407]
FULL_O_SAMPLES = [0, 1, 2047, 2560, 4099, 5119]


def _py_dot(a, b):
    acc = 0.0
    for u, v in zip(a, b):
        acc += u * v
    return acc


def _py_silu(z):
    return z / (1.0 + math.exp(-z)) if z >= 0 else z * math.exp(z) / (1.0 + math.exp(z))


def _check_full_size(x, act, out, dq_gate_row, dq_up_row, dq_down_row):
    xs = [float(v) for v in x]
    got, want = [], []
    for i in FULL_I_SAMPLES:
        g = _py_dot(xs, dq_gate_row(i))
        u = _py_dot(xs, dq_up_row(i))
        got.append(act[i])
        want.append(_py_silu(g) * u)
    err, scale = oracle.normwise_rel_err(np.array(got), np.array(want))
    assert scale > 1e-6 and err < 1e-12, err
    acts = [float(v) for v in act]
    got, want = [], []
    for o in FULL_O_SAMPLES:
        got.append(out[o])
        want.append(_py_dot(acts, dq_down_row(o)))
    err, scale = oracle.normwise_rel_err(np.array(got), np.array(want))
    assert scale > 1e-6 and err < 1e-12, err


def test_fp8_mlp_full_size_sampled():
    d = synth.fp8_mlp(M=1)
    x = codecs.bf16_bits_to_f64(d["x_bits"])
    out, act = mlp.mlp_fp8w_ref(x, d["w_gate"], d["s_gate"], d["w_up"], d["s_up"], d["w_down"], d["s_down"],
                                return_act=True)

    def row(w, sc):
        return lambda n: [float(v) * float(sc[n]) for v in torch_e4m3(w[n])]

    _check_full_size(x[0], act[0], out[0], row(d["w_gate"], d["s_gate"]), row(d["w_up"], d["s_up"]),
                     row(d["w_down"], d["s_down"]))


def test_nvfp4_mlp_full_size_sampled():
    w = synth.nvfp4_mlp_weights()
    xb, _ = synth.nvfp4_x(1)
    x = codecs.bf16_bits_to_f64(xb)
    blk = {n: pack.block64_pack(w["wp_" + n], w["ws_" + n]) for n in ("gate", "up", "down")}
    out, act = mlp.mlp_nvfp4_ref(x, blk["gate"], w["gs_gate"], blk["up"], w["gs_up"], blk["down"], w["gs_down"],
                                 return_act=True)
    table = OCP_E2M1 + [-v for v in OCP_E2M1]

    def row(n):   # from the checkpoint tensors, not the Block64 records
        wp, ws = w["wp_" + n], w["ws_" + n]
        inv = float(np.float32(1.0) / np.float32(w["gs_" + n]))

        def f(r):
            d = torch_e4m3(ws[r])
            vals = []
            for j, byte in enumerate(wp[r].tolist()):
                for nib in (byte & 15, byte >> 4):
                    vals.append(table[nib] * float(d[(2 * j) // 16]) * inv)
            return vals
        return f

    _check_full_size(x[0], act[0], out[0], row("gate"), row("up"), row("down"))


def test_mlp_invariants():
    d = synth.fp8_tiny(2)
    args = (d["w_gate"], d["s_gate"], d["w_up"], d["s_up"], d["w_down"], d["s_down"])
    assert np.all(mlp.mlp_fp8w_ref(np.zeros((1, 256)), *args) == 0.0)
    base = mlp.mlp_fp8w_ref(d["x"], *args)
    a = list(args)
    a[5] = (d["s_down"] * 2).astype(np.float32)                       # doubling the down scales doubles out
    assert np.array_equal(mlp.mlp_fp8w_ref(d["x"], *a), 2 * base)
    # one-hot x: g = dq(G)[:, k], u = dq(U)[:, k]
    k = 77
    x1 = np.zeros((1, 256)); x1[0, k] = 1.0
    _, act = mlp.mlp_fp8w_ref(x1, *args, return_act=True)
    g = mlp.fp8w_weight_f64(d["w_gate"], d["s_gate"])[:, k]
    u = mlp.fp8w_weight_f64(d["w_up"], d["s_up"])[:, k]
    assert np.allclose(act[0], g / (1 + np.exp(-g)) * u, rtol=1e-15, atol=0)


# ---- routed-expert step ----------------------------------------------------------------------------
def _moe_small(ids=None):
    d = synth.awq_moe(E=6, topk=3, H=64, I=32)
    if ids is not None:
        d["ids"] = np.array(ids, dtype=np.int32)
    return d


def _dq_lists(c, s, z):
    return codecs.f16_bits_to_f64(dequant.awq_dequant_parts(c, s, z)).tolist()


@pytest.mark.parametrize("ids", [None, [5, 5, 1], [-1, 2, 6]])
def test_moe_matches_bruteforce(ids):
    d = _moe_small(ids)
    out, act = moe.moe_awq_m1_ref(d["x_bits"], d["ids"], d["router_w"], d["w13"], d["w2"], 32)
    W13 = [_dq_lists(d["w13"][0][e], d["w13"][1][e], d["w13"][2][e]) for e in range(6)]
    W2 = [_dq_lists(d["w2"][0][e], d["w2"][1][e], d["w2"][2][e]) for e in range(6)]
    bf = moe.moe_bruteforce(codecs.f16_bits_to_f64(d["x_bits"]).tolist(), [int(i) for i in d["ids"]],
                            d["router_w"], W13, W2, 32)
    got = codecs.f16_bits_to_f64(out)
    assert np.max(np.abs(got - np.array(bf))) <= np.max(np.abs(bf)) * 2.0 ** -10
    assert np.max(np.abs(bf)) > 1e-6          # a zero result cannot pass


def test_moe_special_cases():
    d = _moe_small([-1, 6, 100])
    out, act = moe.moe_awq_m1_ref(d["x_bits"], d["ids"], d["router_w"], d["w13"], d["w2"], 32)
    assert np.all(out == 0) and np.all(act == 0)                        # all invalid -> exact zero
    d = _moe_small([4, -1, 7])
    d["router_w"] = np.array([1.0, 0.3, 0.2], dtype=np.float32)
    out, act = moe.moe_awq_m1_ref(d["x_bits"], d["ids"], d["router_w"], d["w13"], d["w2"], 32)
    _, y = moe.moe_w2_stage_ref(act, d["ids"], d["router_w"], *d["w2"])
    assert np.array_equal(out, y[0])                                    # one valid route, weight 1 -> y_r
    assert np.all(act[1] == 0) and np.all(act[2] == 0)
    # duplicate ids keep their own weights: (a + b) * y within one half rounding
    d = _moe_small([2, 2, -5])
    d["router_w"] = np.array([0.25, 0.5, 0.25], dtype=np.float32)
    out, act = moe.moe_awq_m1_ref(d["x_bits"], d["ids"], d["router_w"], d["w13"], d["w2"], 32)
    _, y = moe.moe_w2_stage_ref(act, d["ids"], d["router_w"], *d["w2"])
    assert np.array_equal(y[0], y[1])
    assert np.array_equal(out, (codecs.f16_bits_to_f64(y[0]) * 0.75).astype(np.float16).view(np.uint16))


# ---- per-token E4M3 activation quantization (W4A8 variant) --------------------------------------------
def torch_e4m3_encode(v32):
    """Library encode: float32 -> float8_e4m3fn (round to nearest even) -> code bytes."""
    return torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()


def e4m3_encode_cases():
    vals = codecs.e4m3_to_f64(np.arange(0x7F))                         # every non-negative finite value
    mids = (vals[:-1] + vals[1:]) / 2                                 # every exact tie between neighbours
    r = np.random.default_rng(17)
    rnd = np.concatenate([r.standard_normal(4000) * 10 ** r.uniform(-4, 2.6, 4000),
                          r.uniform(-448, 448, 2000), r.uniform(-2 ** -8, 2 ** -8, 2000)])
    v = np.concatenate([vals, -vals, mids, -mids, rnd, [0.0, -0.0, 448.0, -448.0, 2 ** -10, 3 * 2 ** -11]])
    v = v[np.abs(v) <= 448].astype(np.float32).astype(np.float64)     # float32-exact, within range
    return v


def test_e4m3_encode_matches_torch_cast():
    v = e4m3_encode_cases()
    assert np.array_equal(oracle.e4m3_encode_rne(v), torch_e4m3_encode(v))


def test_e4m3_encode_matches_pure_python_nearest_search():
    # independent of the value table and searchsorted: scan the 254 finite codes decoded from their fields
    table = [(float(codecs.e4m3_fields_to_f64(c)), c) for c in range(256) if c not in (0x7F, 0xFF)]
    r = np.random.default_rng(3)
    v = np.concatenate([e4m3_encode_cases()[::23], r.uniform(-448, 448, 300)])
    for x in v:
        best = None
        for val, c in table:
            if math.copysign(1.0, val) != math.copysign(1.0, x):   # same sign side (zero keeps x's sign)
                continue
            key = (abs(val - x), c & 1)                              # nearest, then the even code
            if best is None or key < best[0]:
                best = (key, c)
        assert oracle.e4m3_encode_rne(np.array([x]))[0] == best[1], x


def test_token_exponent_lands_the_row_max_in_224_448():
    assert oracle.token_exponent(448.0) == 0 and oracle.token_exponent(224.0) == -1
    assert oracle.token_exponent(np.nextafter(448.0, 1e9)) == 1
    assert oracle.token_exponent(np.nextafter(224.0, 1e9)) == 0
    assert oracle.token_exponent(0.0) == 0
    r = np.random.default_rng(8)
    for a in np.concatenate([10 ** r.uniform(-30, 30, 2000), 448.0 * 2.0 ** np.arange(-40, 40)]):
        e = oracle.token_exponent(a)
        assert 224.0 < a * 2.0 ** -e <= 448.0, a


def test_quant_per_token_rows():
    r = np.random.default_rng(4)
    x = r.standard_normal((5, 96)) * np.array([[1e-3], [1.0], [30.0], [1e5], [0.0]])
    codes, scale = oracle.quant_e4m3_per_token(x)
    assert scale[4] == 1.0 and np.all(codes[4] & 0x7F == 0)             # a row of (signed) zeros
    assert np.array_equal(codes[4] >> 7, np.signbit(x[4]).astype(np.uint8))
    for m in range(4):
        e = int(round(math.log2(scale[m])))
        assert scale[m] == 2.0 ** e and 224 < np.max(np.abs(x[m])) / scale[m] <= 448
        xs = np.ldexp(x[m], -e)
        x32 = xs.astype(np.float32)
        exact = x32.astype(np.float64) == xs                               # where float32 holds the value
        assert np.array_equal(codes[m][exact], torch_e4m3_encode(x32)[exact])
        # the row max maps onto the top binade's codes, and dequantisation stays within half a code step
        deq = codecs.e4m3_to_f64(codes[m]) * scale[m]
        assert np.all(np.abs(deq - x[m]) <= np.maximum(np.abs(x[m]) * 2.0 ** -4, 2.0 ** -10 * scale[m]))


def test_w4a8_mlp_matches_pure_python_bruteforce():
    # the whole W4A8 definition in plain Python: quantize x per row (nearest-code scan), dequantize, triple
    # loops, silu, act rounded to float32, quantize act per row, dequantize, down projection
    H, I = 64, 64
    W = {n: synth.nvfp4_tensor(*shp, 3, t) for n, t, shp in (("g", 1, (I, H)), ("u", 2, (I, H)), ("d", 3, (H, I)))}
    xb, _ = synth.nvfp4_x(3, H, outlier_frac=0.34)
    x = codecs.bf16_bits_to_f64(xb)
    blk = {n: pack.block64_pack(*W[n][:2]) for n in W}
    ref = mlp.mlp_nvfp4_w4a8_ref(x, blk["g"], W["g"][2], blk["u"], W["u"][2], blk["d"], W["d"][2])
    table = [(float(codecs.e4m3_fields_to_f64(c)), c) for c in range(256) if c not in (0x7F, 0xFF)]

    def q_row(row):
        amax = max(abs(v) for v in row)
        e = 0
        if amax > 0:
            while amax > 448.0 * 2.0 ** e:
                e += 1
            while amax <= 448.0 * 2.0 ** (e - 1):
                e -= 1
        out = []
        for v in row:
            t = v * 2.0 ** -e
            best = min((abs(val - t), c & 1, val) for val, c in table if math.copysign(1, val) == math.copysign(1, t))
            out.append(best[2] * 2.0 ** e)
        return out

    table16 = np.array(OCP_E2M1 + [-v for v in OCP_E2M1])

    def wt(wp, ws, gs):
        nib = np.stack([wp & 15, wp >> 4], axis=-1).reshape(wp.shape[0], -1)
        inv = float(np.float32(1.0) / np.float32(gs))
        return (table16[nib] * np.repeat(torch_e4m3(ws).astype(np.float64), 16, axis=1) * inv).tolist()

    Wg, Wu, Wd = wt(*W["g"]), wt(*W["u"]), wt(*W["d"])
    for m in range(3):
        xr = q_row(list(x[m]))
        act = []
        for i in range(I):
            g = sum(xr[k] * Wg[i][k] for k in range(H))
            u = sum(xr[k] * Wu[i][k] for k in range(H))
            sg = g / (1.0 + math.exp(-g)) if g >= 0 else g * math.exp(g) / (1.0 + math.exp(g))
            act.append(float(np.float32(sg * u)))
        ar = q_row(act)
        o = [sum(ar[q] * Wd[j][q] for q in range(I)) for j in range(H)]
        err, scale = oracle.normwise_rel_err(ref[m], np.array(o))
        assert scale > 1e-6 and err < 1e-12, (m, err)


def test_w4a8_pins_catch_planted_mistakes(monkeypatch):
    from oracle import actquant
    v = e4m3_encode_cases()
    good = torch_e4m3_encode(v)
    # ties away from zero instead of to the even code
    pos = actquant._POS_VALUES

    def away(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x)
        hi = np.minimum(np.searchsorted(pos, a), pos.size - 1)
        lo = np.maximum(hi - 1, 0)
        c = np.where(pos[hi] - a <= a - pos[lo], hi, lo).astype(np.uint8)
        return np.where(np.signbit(x), c | 0x80, c).astype(np.uint8)
    assert not np.array_equal(away(v), good)
    # truncation instead of rounding
    trunc = np.where(np.signbit(v), 0x80, 0) | (np.searchsorted(pos, np.abs(v), side="right") - 1)
    assert not np.array_equal(trunc.astype(np.uint8), good)
    # a scale that puts the row max at 448 exactly (amax / 448, not a power of two) changes the codes
    x = np.random.default_rng(5).standard_normal((1, 256)) * 3.0
    c_pow2, _ = oracle.quant_e4m3_per_token(x)
    c_div = torch_e4m3_encode((x[0] / (np.max(np.abs(x)) / 448.0)).astype(np.float32))
    assert not np.array_equal(c_pow2[0], c_div)


# ---- the parity metric ---------------------------------------------------------------------------------
# Hand-computed cases of the row-normwise error  max_m ( max_o |y - r| / max_o |r| ), with the row scale
# min_m max_o |r| returned beside it.  Each tuple: (y, ref, expected error, expected min row scale).
METRIC_CASES = [
    ([[1.0, 2.0]], [[1.0, 2.5]], 0.5 / 2.5, 2.5),                         # one row
    ([[1000.0, 0.0], [1.01, -1.0]], [[1000.0, 0.0], [1.0, -1.0]], 0.01, 1.0),   # each row on its own scale
    ([[4.0, 2e-6]], [[4.0, 1e-6]], 1e-6 / 4.0, 4.0),                       # a tiny element is not its own scale
    ([[-3.3, 1.0]], [[-3.0, 1.0]], 0.3 / 3.0, 3.0),                        # magnitudes, not signed values
    ([[1.0, 1.0], [1.0, 1.0], [1.3, 1.0]], [[1.0, 1.0]] * 3, 0.3, 1.0),    # the worst row, not the mean
    ([[2.0]], [[1.0]], 1.0, 1.0),                                          # the reference is the denominator
    ([[0.0, 0.0], [2.0, 0.0]], [[0.0, 0.0], [2.0, 0.5]], 0.25, 0.0),       # exact zero row: error 0, scale 0
    ([1.0, 3.0], [1.0, 4.0], 0.25, 4.0),                                   # 1-D input is one row
]


def _metric_failures(fn):
    """The METRIC_CASES (and the non-finite ones) that fn gets wrong."""
    bad = []
    for i, (y, r, want, want_scale) in enumerate(METRIC_CASES):
        err, scale = fn(np.array(y), np.array(r))
        if not (abs(err - want) <= 1e-12 * max(1.0, want) and abs(scale - want_scale) <= 1e-12):
            bad.append(i)
    err, _ = fn(np.array([[0.0, 1e-30]]), np.array([[0.0, 0.0]]))          # any error on a zero row fails
    if not np.isinf(err):
        bad.append("zero-row")
    return bad


def test_normwise_metric_hand_computed():
    assert _metric_failures(oracle.normwise_rel_err) == []


def test_normwise_metric_pins_catch_planted_metrics():
    def as_rows(y, r):
        return np.atleast_2d(np.asarray(y, float)), np.atleast_2d(np.asarray(r, float))

    def global_norm(y, r):          # one scale for the whole matrix: under-reports small rows
        y, r = as_rows(y, r)
        with np.errstate(divide="ignore", invalid="ignore"):
            return float(np.max(np.abs(y - r)) / np.max(np.abs(r))), float(np.min(np.max(np.abs(r), axis=1)))

    def mean_rows(y, r):            # mean over rows instead of the worst row
        y, r = as_rows(y, r)
        s = np.max(np.abs(r), axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            return float(np.mean(np.max(np.abs(y - r), axis=1) / s)), float(np.min(s))

    def y_denominator(y, r):        # scaled by the result under test
        return oracle.normwise_rel_err(r, y)

    def no_abs(y, r):               # signed difference
        y, r = as_rows(y, r)
        s = np.max(np.abs(r), axis=1)
        with np.errstate(divide="ignore", invalid="ignore"):
            return float(np.max(np.max(y - r, axis=1) / s)), float(np.min(s))

    def elementwise(y, r):          # per-element relative error
        y, r = as_rows(y, r)
        with np.errstate(divide="ignore", invalid="ignore"):
            e = np.where(r != 0, np.abs(y - r) / np.abs(r), np.where(y != r, np.inf, 0.0))
        return float(np.max(e)), float(np.min(np.max(np.abs(r), axis=1)))

    def zero_rows_pass(y, r):       # a zero reference row forgives any error
        err, s = oracle.normwise_rel_err(y, r)
        return (0.0 if np.isinf(err) else err), s

    for planted in (global_norm, mean_rows, y_denominator, no_abs, elementwise, zero_rows_pass):
        assert _metric_failures(planted), planted.__name__


# ---- planted mistakes: each must be caught by one of the pins above ---------------------------------
def test_pins_catch_planted_mistakes(monkeypatch):
    d = synth.fp8_tiny(1)
    args = (d["w_gate"], d["s_gate"], d["w_up"], d["s_up"], d["w_down"], d["s_down"])
    good = mlp.mlp_fp8w_ref(d["x"], *args)
    # (1) transposed down operand -> shape change / different values
    Wd = mlp.fp8w_weight_f64(d["w_down"], d["s_down"])
    _, act = mlp.mlp_fp8w_ref(d["x"], *args, return_act=True)
    bad = act @ Wd.reshape(Wd.shape[1], Wd.shape[0])
    assert bad.shape != good.shape or not np.allclose(bad, good)
    # (2) a dropped silu (act = g*u) breaks the closed form used by test_mlp_invariants
    monkeypatch.setattr(mlp, "silu", lambda z: np.asarray(z, dtype=np.float64))
    assert not np.allclose(mlp.mlp_fp8w_ref(d["x"], *args), good)
    monkeypatch.undo()
    # (3) swapped nibble order breaks the Block64 struct pin
    wp = np.array([[0x21] * 32], dtype=np.uint8)
    ws = np.array([[0x38] * 4], dtype=np.uint8)
    dq = dequant.nvfp4_dequant(pack.block64_pack(wp, ws), np.float32(1.0))
    assert dq[0, 0] == 0.5 and dq[0, 1] == 1.0            # low nibble (code 1 = 0.5) is the earlier weight
    # (4) e4m3 with a wrong bias is caught by the 256-code library pin
    wrong = np.ldexp(1.0, -8) * np.arange(8)
    assert not np.array_equal(codecs.e4m3_to_f64(np.arange(8)), wrong)
