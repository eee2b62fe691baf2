"""The W4A8 variant (NVFP4 weights, per-token E4M3 activations) against the oracle (GPU, through the C ABI).

Page "Qwen3.8-27B-NVFP4", section "Implemented execution path": per-token dynamic 8-bit activations,
one quantization of x shared by gate and up.  The oracle's definition (oracle.mlp_nvfp4_w4a8_ref) takes
every code decision the device takes, in the same precision, so:

* the x codes and row scales are bit-exact (the power-of-two scale is exact and both sides round to
  nearest even);
* the gate/up stage's float32 act matches the oracle's act within float32 accumulation;
* the act codes are bit-exact with the oracle's quantizer applied to the device's own act (the oracle's
  act differs from the device's in the last float32 bits, so a code can flip where an act value sits on a
  rounding midpoint: those flips are counted and bounded, not hidden);
* the down projection fed the device's codes matches the oracle's within float32 accumulation;
* end to end the outputs match the oracle's W4A8 within the 1e-3 gate, while the error against the
  exact (unquantized) MLP is the variant's own and is reported.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_mlp_amd as wq
from gpu_common import DEV, bf16_dev, dev, gate, host

pytestmark = pytest.mark.gpu
H, I = 5120, 17408


def a256(n):
    return -(-n // 256) * 256


def codes_of(q16):
    """The device's quantized rows (float16 bits, each an E4M3 value) -> their E4M3 codes.  Asserts that every
    value is exactly an E4M3 value (sign of zero included), so comparing codes compares the values."""
    v = np.asarray(q16).view(np.float16).astype(np.float64)
    codes = oracle.e4m3_encode_rne(v)
    back = oracle.codecs.e4m3_to_f64(codes)
    nan = np.isnan(v)
    assert np.array_equal(np.isnan(back), nan), "a NaN does not round-trip"
    same = (back == v) & (np.signbit(back) == np.signbit(v))
    assert np.all(same | nan), "a quantized value is not an E4M3 value"
    return codes


def ws_regions(M, Hh, Ii):
    xq = 0
    sx = a256(M * Hh * 2)
    act = sx + a256(M * 4)
    aq = act + a256(M * Ii * 4)
    sa = aq + a256(M * Ii * 2)
    return dict(xq=xq, sx=sx, act=act, aq=aq, sa=sa)


def view(ws, off, n, dt, shape):
    return host(ws[off:off + n * np.dtype(dt).itemsize]).view(dt).reshape(shape)


def check_w4a8(y, ws, x64, blk_args, rows, Hh, Ii, M, what):
    """The device's output against the oracle's W4A8, stage by stage.

    ws: the workspace of the call that produced y (it holds the codes the call used); rows: which of the
    call's M rows x64 holds.  Checks: act codes = the oracle's quantizer on the device's float32 act
    (bitwise); y = the oracle's down projection of those codes (the 1e-3 gate); y against the
    oracle's own end-to-end result within what its act-code differences explain: an act value on a
    rounding midpoint may take the neighbouring code when its last float32 bits differ, which moves
    out[o] by |delta act_q| |Wd[o, q]| -- the bound is that sum plus the gate's 1e-3 of the row.
    """
    R = ws_regions(M, Hh, Ii)
    act = view(ws, R["act"], M * Ii, np.float32, (M, Ii))[rows]
    aq = codes_of(view(ws, R["aq"], M * Ii, np.uint16, (M, Ii)))[rows]
    sa = view(ws, R["sa"], M, np.float32, (M,))[rows].astype(np.float64)
    own_q, own_s = oracle.quant_e4m3_per_token(act.astype(np.float64))
    assert np.array_equal(sa, own_s) and np.array_equal(aq, own_q), f"{what}: act codes"
    ref, st = oracle.mlp_nvfp4_w4a8_ref(x64, *blk_args, stages=True)
    gate(act, st["act32"], what=f"{what}: gate/up act (float32)")
    Wd = oracle.mlp.nvfp4_weight_f64(blk_args[4], blk_args[5])
    ad = oracle.codecs.e4m3_to_f64(aq) * sa[:, None]
    gate(y, ad @ Wd.T, what=f"{what}: down stage on the device's act codes")
    ad_ref = oracle.codecs.e4m3_to_f64(st["aq"]) * st["sa"][:, None]
    flips = int(np.sum(ad != ad_ref))
    bound = np.abs(ad - ad_ref) @ np.abs(Wd).T + 1e-3 * np.max(np.abs(ref), axis=1, keepdims=True)
    err, _ = oracle.normwise_rel_err(y, ref)
    print(f"[parity] {what}: {flips} act codes of {ad.size} differ from the oracle's; end-to-end normwise "
          f"error {err:.3e}", flush=True)
    assert flips <= 1e-3 * ad.size
    assert np.all(np.abs(y - ref) <= bound), f"{what}: an output differs from the oracle by more than its flips explain"
    return ref


@pytest.fixture(scope="module")
def nv_small():
    Hh, Ii = 512, 1024
    W = {n: synth.nvfp4_tensor(*shp, 41, t) for n, t, shp in (("g", 1, (Ii, Hh)), ("u", 2, (Ii, Hh)), ("d", 3, (Hh, Ii)))}
    blk = {n: oracle.block64_pack(W[n][0], W[n][1]) for n in W}
    return Hh, Ii, W, blk


def nv_args(blk, W, on_dev=True):
    f = dev if on_dev else (lambda a: a)
    return (f(blk["g"]), float(W["g"][2]), f(blk["u"]), float(W["u"][2]), f(blk["d"]), float(W["d"][2]))


def special_rows(Hh):
    """Rows that exercise the encoder: exact E4M3 midpoints (ties) scaled so that the row max maps to 448,
    values in E4M3's subnormal range, signed zeros, and plain normal draws in bf16 and float32."""
    vals = oracle.codecs.e4m3_to_f64(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    rows = []
    for e in (-3, 0, 5):
        r = np.resize(np.concatenate([[448.0], mids, -mids, vals[:16] / 2, [-0.0, 0.0]]), Hh) * 2.0 ** e
        rows.append(r)
    g = np.random.default_rng(9)
    rows.append(g.standard_normal(Hh) * 37.0)
    rows.append(g.standard_normal(Hh) * 1e-4)
    return np.array(rows, dtype=np.float32)


@pytest.mark.parametrize("xdt", [torch.float32, torch.bfloat16])
def test_x_codes_and_scales_bit_exact(nv_small, xdt):
    Hh, Ii, W, blk = nv_small
    x = special_rows(Hh)
    if xdt == torch.bfloat16:
        xb = synth.to_bf16_bits(x)
        xt = bf16_dev(xb)
        x64 = oracle.bf16_bits_to_f64(xb)
    else:
        xt = dev(x)
        x64 = x.astype(np.float64)
    M = x.shape[0]
    ws = torch.zeros(wq.mlp_workspace_bytes(wq.WQ_FMT_NVFP4, M, Hh, Ii, "mfma", "e4m3"), dtype=torch.uint8, device=DEV)
    wq.mlp_nvfp4_run(xt, *nv_args(blk, W), workspace=ws, stage="gateup", act="e4m3")
    torch.cuda.synchronize()
    R = ws_regions(M, Hh, Ii)
    q = codes_of(view(ws, R["xq"], M * Hh, np.uint16, (M, Hh)))
    s = view(ws, R["sx"], M, np.float32, (M,))
    wq_codes, wq_scale = oracle.quant_e4m3_per_token(x64)
    assert np.array_equal(s.astype(np.float64), wq_scale)
    bad = np.argwhere(q != wq_codes)
    assert bad.size == 0, f"{len(bad)} codes differ, e.g. {[(tuple(b), hex(q[tuple(b)]), hex(wq_codes[tuple(b)])) for b in bad[:5]]}"


def test_stages_against_the_oracle(nv_small):
    Hh, Ii, W, blk = nv_small
    M = 96
    xb, _ = synth.nvfp4_x(M, Hh, config_id=41, outlier_frac=0.05)
    x64 = oracle.bf16_bits_to_f64(xb)
    ws = torch.zeros(wq.mlp_workspace_bytes(wq.WQ_FMT_NVFP4, M, Hh, Ii, "mfma", "e4m3"), dtype=torch.uint8, device=DEV)
    xt = bf16_dev(xb)
    wq.mlp_nvfp4_run(xt, *nv_args(blk, W), workspace=ws, stage="gateup", act="e4m3")
    out = host(wq.mlp_nvfp4_run(xt, *nv_args(blk, W), workspace=ws, stage="down", act="e4m3"))
    check_w4a8(out, ws, x64, nv_args(blk, W, False), np.arange(M), Hh, Ii, M, "w4a8 two-stage 512x1024 M=96")
    # one call gives the same bits as the two stages
    one = host(wq.mlp_nvfp4_run(xt, *nv_args(blk, W), act="e4m3"))
    assert np.array_equal(one.view(np.uint32), out.view(np.uint32))


@pytest.fixture(scope="module")
def nv_big():
    w = synth.nvfp4_mlp_weights()
    blk = {n: oracle.block64_pack(w["wp_" + n], w["ws_" + n]) for n in ("gate", "up", "down")}
    d = {n: dev(blk[n]) for n in blk}
    return w, blk, d


def run_big(nv_big, M, outlier):
    w, blk, d = nv_big
    xb, rows = synth.nvfp4_x(M, outlier_frac=outlier)
    ws = torch.empty(wq.mlp_workspace_bytes(wq.WQ_FMT_NVFP4, M, H, I, "auto", "e4m3"), dtype=torch.uint8, device=DEV)
    y = host(wq.mlp_nvfp4_run(bf16_dev(xb), d["gate"], w["gs_gate"], d["up"], w["gs_up"], d["down"], w["gs_down"],
                              workspace=ws, act="e4m3"))
    return xb, rows, y, ws


def big_args(nv_big):
    w, blk, _ = nv_big
    return (blk["gate"], w["gs_gate"], blk["up"], w["gs_up"], blk["down"], w["gs_down"])


def test_prefill_M512(nv_big):
    xb, _, y, ws = run_big(nv_big, 512, 0.01)
    x64 = oracle.bf16_bits_to_f64(xb)
    check_w4a8(y, ws, x64, big_args(nv_big), np.arange(512), H, I, 512, "w4a8 prefill M=512")
    err, _ = oracle.normwise_rel_err(y, oracle.mlp_nvfp4_ref(x64, *big_args(nv_big)))
    print(f"[w4a8] M=512 error against the exact NVFP4 MLP (the variant's own quantization error): {err:.3e}")
    assert err < 0.1


def test_prefill_M8192_sampled(nv_big):
    xb, rows, y, ws = run_big(nv_big, 8192, 0.01)
    pick = np.unique(np.concatenate([rows, np.random.default_rng(3).choice(8192, 160, replace=False)]))
    x64 = oracle.bf16_bits_to_f64(xb[pick])
    check_w4a8(y[pick], ws, x64, big_args(nv_big), pick, H, I, 8192,
               f"w4a8 prefill M=8192 ({len(pick)} rows incl. all outliers)")


@pytest.mark.parametrize("M", [1, 5, 40, 129])
def test_ragged_and_short(nv_small, M):
    Hh, Ii, W, blk = nv_small
    xb, _ = synth.nvfp4_x(M, Hh, config_id=43)
    ws = torch.empty(wq.mlp_workspace_bytes(wq.WQ_FMT_NVFP4, M, Hh, Ii, "auto", "e4m3"), dtype=torch.uint8, device=DEV)
    y = host(wq.mlp_nvfp4_run(bf16_dev(xb), *nv_args(blk, W), workspace=ws, act="e4m3"))
    check_w4a8(y, ws, oracle.bf16_bits_to_f64(xb), nv_args(blk, W, False), np.arange(M), Hh, Ii, M,
               f"w4a8 M={M} 512x1024")


@pytest.mark.parametrize("N,K", [(67, 384), (45, 256), (130, 640), (67, 320)])
def test_linear_tail_shapes(N, K):
    # the NVFP4 page's tail case has 129 rows and 67 output rows; K is a multiple of 64 (one record) and at
    # least 256 (one weight block of four records), with a short last weight block at 320, 384 and 640
    wp, ws, gs = synth.nvfp4_tensor(N, K, 3, 44)
    blk = oracle.block64_pack(wp, ws)
    x = np.random.default_rng(N + K).standard_normal((129, K)).astype(np.float32)
    y = host(wq.qlinear_run(wq.WQ_FMT_NVFP4, dev(x), dev(blk), None, float(gs), act="e4m3"))
    xq, sx = oracle.quant_e4m3_per_token(x.astype(np.float64))
    ref = (oracle.codecs.e4m3_to_f64(xq) * sx[:, None]) @ oracle.mlp.nvfp4_weight_f64(blk, gs).T
    gate(y, ref, what=f"w4a8 linear 129 x {N} x {K}")


def test_rejected_forms(nv_small):
    Hh, Ii, W, blk = nv_small
    x = bf16_dev(synth.nvfp4_x(4, Hh)[0])
    with pytest.raises(wq.WQError):
        wq.mlp_nvfp4_run(x, *nv_args(blk, W), path="gemv", act="e4m3")
    assert wq.mlp_workspace_bytes(wq.WQ_FMT_FP8W, 4, 256, 256, "auto", "e4m3") == 0
    xs = dev(np.zeros((4, 192), np.float32))
    wp, ws_, gs = synth.nvfp4_tensor(64, 192, 3, 46)
    with pytest.raises(wq.WQError):                       # K = 192 is below one weight block (256)
        wq.qlinear_run(wq.WQ_FMT_NVFP4, xs, dev(oracle.block64_pack(wp, ws_)), None, float(gs), act="e4m3")
