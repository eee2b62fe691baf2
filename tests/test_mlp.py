"""Dense SwiGLU MLP parity against the FP64 oracle (configs at the pages' shapes).

Gate: row-normwise max relative error <= 1e-3 with a non-trivial reference
magnitude.  Plus bitwise properties of the GEMV order (M-independence,
run-to-run determinism) and hipGraph replay with changing inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import weight_quantized_mlp_amd as wq
from gpu_common import DEV, bf16_dev, dev, gate, host

pytestmark = pytest.mark.gpu

FP8_NAMES = ("w_gate", "s_gate", "w_up", "s_up", "w_down", "s_down")


def fp8_dev(d):
    return [dev(d[n]) for n in FP8_NAMES]


# ---- tiny FP8 W8A16 (H=256, I=512) -------------------------------------------------------------
@pytest.mark.parametrize("M", [1, 4])
def test_fp8_tiny(M):
    d = synth.fp8_tiny(M)
    ref = oracle.mlp_fp8w_ref(d["x"], *(d[n] for n in FP8_NAMES))
    y = host(wq.mlp_fp8w_run(dev(d["x"]), *fp8_dev(d)))
    gate(y, ref, what=f"fp8 tiny M={M}")


def test_fp8_tiny_rows_independent_and_deterministic():
    d = synth.fp8_tiny(4)
    W = fp8_dev(d)
    x = dev(d["x"])
    y4 = host(wq.mlp_fp8w_run(x, *W))
    y4b = host(wq.mlp_fp8w_run(x, *W))
    assert np.array_equal(y4.view(np.uint32), y4b.view(np.uint32))
    for m in range(4):
        y1 = host(wq.mlp_fp8w_run(x[m:m + 1].contiguous(), *W))
        assert np.array_equal(y1[0].view(np.uint32), y4[m].view(np.uint32)), m


def test_fp8_tiny_exact_scale_invariants():
    d = synth.fp8_tiny(1)
    W = fp8_dev(d)
    x = dev(d["x"])
    y = host(wq.mlp_fp8w_run(x, *W))
    W2 = list(W)
    W2[5] = W[5] * 2                                         # doubling every down scale doubles out exactly
    y2 = host(wq.mlp_fp8w_run(x, *W2))
    assert np.array_equal(y2, 2 * y)
    assert np.all(host(wq.mlp_fp8w_run(torch.zeros_like(x), *W)) == 0)


# ---- FP8 at the 27B tail-layer shape (H=5120, I=17408, M=1, bf16 x) ------------------------------
@pytest.fixture(scope="module")
def fp8_big():
    return synth.fp8_mlp(M=1)


def test_fp8_decode_5120x17408(fp8_big):
    d = fp8_big
    x64 = oracle.bf16_bits_to_f64(d["x_bits"])
    ref = oracle.mlp_fp8w_ref(x64, *(d[n] for n in FP8_NAMES))
    y = host(wq.mlp_fp8w_run(bf16_dev(d["x_bits"]), *fp8_dev(d)))
    gate(y, ref, what="fp8 5120x17408 M=1")


def test_fp8_prefill_M512_reproducible_sampled_rows(fp8_big):
    # FP8 on the MFMA path at M=512: the split-K plan and its ordered finish give the same bits run to
    # run; sampled rows (both ends of every 128-row band) match the oracle.
    d = fp8_big
    xb = synth.to_bf16_bits(np.random.default_rng(512).standard_normal((512, 5120)).astype(np.float32))
    W = fp8_dev(d)
    x = bf16_dev(xb)
    y1 = host(wq.mlp_fp8w_run(x, *W))
    y2 = host(wq.mlp_fp8w_run(x, *W))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    rows = np.array([0, 1, 126, 127, 128, 255, 256, 383, 384, 510, 511])
    ref = oracle.mlp_fp8w_ref(oracle.bf16_bits_to_f64(xb[rows]), *(d[n] for n in FP8_NAMES))
    gate(y1[rows], ref, what="fp8 M=512 sampled rows (mfma)")


@pytest.mark.parametrize("M", [8, 200])
def test_fp8_mfma_bf16_x_same_bits_as_f32_x(fp8_big, M):
    # bf16 x takes bf16 MFMAs on x as given; float32 x holding the same values is row-scaled by a power of
    # two to float16 first.  Every product is exact in both forms and the scaling is exact, so the MLP and
    # the single linear give the same bits.
    d = fp8_big
    xb = synth.to_bf16_bits(np.random.default_rng(M + 77).standard_normal((M, 5120)).astype(np.float32))
    W = fp8_dev(d)
    yb = host(wq.mlp_fp8w_run(bf16_dev(xb), *W, path="mfma"))
    yf = host(wq.mlp_fp8w_run(dev(oracle.bf16_bits_to_f64(xb).astype(np.float32)), *W, path="mfma"))
    assert np.array_equal(yb.view(np.uint32), yf.view(np.uint32))
    lb = host(wq.qlinear_run(wq.WQ_FMT_FP8W, bf16_dev(xb), W[0], W[1], path="mfma"))
    lf = host(wq.qlinear_run(wq.WQ_FMT_FP8W, dev(oracle.bf16_bits_to_f64(xb).astype(np.float32)), W[0], W[1],
                             path="mfma"))
    assert np.array_equal(lb.view(np.uint32), lf.view(np.uint32))


# ---- NVFP4 (H=5120, I=17408) ----------------------------------------------------------------------
@pytest.fixture(scope="module")
def nv_big():
    w = synth.nvfp4_mlp_weights()
    blk = {n: oracle.block64_pack(w["wp_" + n], w["ws_" + n]) for n in ("gate", "up", "down")}
    gs = {n: w["gs_" + n] for n in ("gate", "up", "down")}
    W = {n: oracle.mlp.nvfp4_weight_f64(blk[n], gs[n]) for n in ("gate", "up", "down")}
    dblk = {n: dev(blk[n]) for n in blk}
    return blk, gs, W, dblk


def nv_run(dblk, gs, x, path="auto"):
    return wq.mlp_nvfp4_run(x, dblk["gate"], gs["gate"], dblk["up"], gs["up"], dblk["down"], gs["down"], path=path)


def nv_ref(W, x64):
    return oracle.swiglu_mlp(x64, W["gate"], W["up"], W["down"])[0]


def test_nvfp4_decode_M1(nv_big):
    blk, gs, W, dblk = nv_big
    xb, _ = synth.nvfp4_x(1)
    y = host(nv_run(dblk, gs, bf16_dev(xb)))
    gate(y, nv_ref(W, oracle.bf16_bits_to_f64(xb)), what="nvfp4 M=1")


def test_nvfp4_gemv_rows_independent_of_M(nv_big):
    # The GEMV path's fixed order: row m of a 5-row call (a 3-row and a 2-row pass over the weights in the
    # down projection) equals the 1-row call on row m, bit for bit; two runs agree.
    blk, gs, W, dblk = nv_big
    xb, _ = synth.nvfp4_x(5, config_id=11)
    x = bf16_dev(xb)
    y5 = host(nv_run(dblk, gs, x, path="gemv"))
    assert np.array_equal(y5.view(np.uint32), host(nv_run(dblk, gs, x, path="gemv")).view(np.uint32))
    for m in range(5):
        y1 = host(nv_run(dblk, gs, x[m:m + 1].contiguous(), path="gemv"))
        assert np.array_equal(y1[0].view(np.uint32), y5[m].view(np.uint32)), m
    gate(y5, nv_ref(W, oracle.bf16_bits_to_f64(xb)), what="nvfp4 M=5 gemv")


def test_nvfp4_gpu_packer_feeds_the_mlp(nv_big):
    blk, gs, W, dblk = nv_big
    w = synth.nvfp4_mlp_weights()
    packed = {n: wq.nvfp4_pack_block64(dev(w["wp_" + n]), dev(w["ws_" + n])) for n in ("gate", "up", "down")}
    for n in packed:
        assert torch.equal(packed[n], dblk[n])


def test_nvfp4_prefill_M512(nv_big):
    blk, gs, W, dblk = nv_big
    xb, rows = synth.nvfp4_x(512, outlier_frac=0.01)
    assert len(rows) == 5
    y = host(nv_run(dblk, gs, bf16_dev(xb)))
    gate(y, nv_ref(W, oracle.bf16_bits_to_f64(xb)), what="nvfp4 M=512 (mfma)")


def test_nvfp4_prefill_M512_split_k_reproducible(nv_big):
    # At M=512 the last round of gate/up tiles and every down tile are split along K and finished by
    # an ordered sum of the parts: two runs give the same bits, and the split rows (the last 128-row
    # band, whose upper column tiles form the split round of gate/up) match the oracle.
    blk, gs, W, dblk = nv_big
    xb, _ = synth.nvfp4_x(512, config_id=7, outlier_frac=0.01)
    x = bf16_dev(xb)
    y1 = host(nv_run(dblk, gs, x))
    y2 = host(nv_run(dblk, gs, x))
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))
    band = np.arange(384, 512)
    gate(y1[band], nv_ref(W, oracle.bf16_bits_to_f64(xb[band])), what="nvfp4 M=512 split band")


def test_nvfp4_prefill_M8192_sampled(nv_big):
    blk, gs, W, dblk = nv_big
    xb, rows = synth.nvfp4_x(8192, outlier_frac=0.01)
    assert len(rows) == 82
    y = host(nv_run(dblk, gs, bf16_dev(xb)))
    r = np.random.default_rng(8192)
    sample = np.union1d(rows, r.choice(8192, 512 - len(rows), replace=False))   # every outlier row + random rows
    ref = nv_ref(W, oracle.bf16_bits_to_f64(xb[sample]))
    gate(y[sample], ref, what="nvfp4 M=8192 sampled rows (mfma)")
    assert np.all(np.isfinite(y))


# M spans the short-batch tiles of the MFMA path: 32-row tiles with the block schedule (M <= 32 for
# gate/up, M <= 96 for down, 1..3 row tiles), 64-row stepped tiles (gate/up 33..64, down 97..128) and
# 128-row ones, split-K at every size.
@pytest.mark.parametrize("M", [2, 3, 8, 17, 32, 37, 64, 96, 97, 112, 127, 128, 200])
def test_nvfp4_paths_agree_with_oracle(nv_big, M):
    blk, gs, W, dblk = nv_big
    xb, _ = synth.nvfp4_x(M, outlier_frac=0.05)
    ref = nv_ref(W, oracle.bf16_bits_to_f64(xb))
    ys = {}
    for path in ("gemv", "mfma"):
        ys[path] = host(nv_run(dblk, gs, bf16_dev(xb), path=path))
        gate(ys[path], ref, what=f"nvfp4 M={M} {path}")
    # AUTO takes the GEMV below WQ_NARROW_MIN_ROWS_NVFP4 rows and the MFMA GEMM from there on
    want = "gemv" if M < 3 else "mfma"
    assert np.array_equal(host(nv_run(dblk, gs, bf16_dev(xb))).view(np.uint32), ys[want].view(np.uint32))


@pytest.mark.parametrize("M", [2, 12, 33, 128])
def test_fp8_short_batch_paths_agree_with_oracle(fp8_big, M):
    d = fp8_big
    xb = synth.to_bf16_bits(np.random.default_rng(500 + M).standard_normal((M, 5120)).astype(np.float32))
    ref = oracle.mlp_fp8w_ref(oracle.bf16_bits_to_f64(xb), *(d[n] for n in FP8_NAMES))
    W = fp8_dev(d)
    ys = {}
    for path in ("gemv", "mfma"):
        ys[path] = host(wq.mlp_fp8w_run(bf16_dev(xb), *W, path=path))
        gate(ys[path], ref, what=f"fp8 M={M} {path}")
    want = "gemv" if M < 2 else "mfma"                       # WQ_NARROW_MIN_ROWS_FP8
    assert np.array_equal(host(wq.mlp_fp8w_run(bf16_dev(xb), *W)).view(np.uint32), ys[want].view(np.uint32))


# ---- ragged tails: partial m and n tiles ----------------------------------------------------------------
@pytest.mark.parametrize("fmt", ["fp8", "nvfp4"])
# K = 64 takes the register-load GEMM for both formats; K = 128 / 192 / 320 / 448 the copy-fed one with
# short last blocks (FP8: odd K-step counts; NVFP4 K >= 256: record counts not a multiple of 4).
@pytest.mark.parametrize("M,H,I", [(129, 320, 192), (1, 320, 192), (130, 64, 64), (255, 576, 448), (40, 128, 256),
                                   (7, 192, 320)])
def test_tail_shapes(fmt, M, H, I):
    r = np.random.default_rng(M * 7 + H)
    x = r.standard_normal((M, H)).astype(np.float32)
    xb = synth.to_bf16_bits(x)
    x64 = oracle.bf16_bits_to_f64(xb)
    for path in ("gemv", "mfma"):
        if fmt == "fp8":
            d = {}
            for n, shp in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
                w = r.standard_normal(shp).astype(np.float32) * 0.05
                s = (np.abs(w).max(axis=1) / 448).astype(np.float32)
                d["w_" + n], d["s_" + n] = synth.to_e4m3_codes(w / s[:, None]), s
            ref = oracle.mlp_fp8w_ref(x64, *(d[n] for n in FP8_NAMES))
            y = host(wq.mlp_fp8w_run(bf16_dev(xb), *fp8_dev(d), path=path))
        else:
            ws = {n: synth.nvfp4_tensor(*shp, 40 + M, t) for n, t, shp in
                  (("gate", 1, (I, H)), ("up", 2, (I, H)), ("down", 3, (H, I)))}
            blk = {n: oracle.block64_pack(ws[n][0], ws[n][1]) for n in ws}
            gs = {n: ws[n][2] for n in ws}
            ref = oracle.mlp_nvfp4_ref(x64, blk["gate"], gs["gate"], blk["up"], gs["up"], blk["down"], gs["down"])
            y = host(nv_run({n: dev(blk[n]) for n in blk}, gs, bf16_dev(xb), path=path))
        gate(y, ref, what=f"{fmt} tail M={M} H={H} I={I} {path}")


# ---- hipGraph capture / replay with changing inputs ---------------------------------------------------------
def test_graph_replay_changing_inputs(nv_big):
    blk, gs, W, dblk = nv_big
    for M in (1, 8, 256):          # GEMV; 32-row tiles with the block schedule; 128-row tiles with split K
        xs = [synth.nvfp4_x(M, config_id=30 + i)[0] for i in range(3)]
        xin = bf16_dev(xs[0])
        out = torch.empty((M, 5120), dtype=torch.float32, device=DEV)
        ws = torch.empty(wq.mlp_workspace_bytes(1, M, 5120, 17408), dtype=torch.uint8, device=DEV)
        eager = [host(nv_run(dblk, gs, bf16_dev(x))) for x in xs]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            wq.mlp_nvfp4_run(xin, dblk["gate"], gs["gate"], dblk["up"], gs["up"], dblk["down"], gs["down"],
                             out=out, workspace=ws)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            wq.mlp_nvfp4_run(xin, dblk["gate"], gs["gate"], dblk["up"], gs["up"], dblk["down"], gs["down"],
                             out=out, workspace=ws)
        for rep in range(2):
            for i, x in enumerate(xs):
                xin.copy_(bf16_dev(x))
                g.replay()
                torch.cuda.synchronize()
                assert np.array_equal(host(out).view(np.uint32), eager[i].view(np.uint32)), (M, rep, i)


def test_fp8_graph_replay_changing_inputs(fp8_big):
    # FP8 on both paths inside a captured graph (M=1 GEMV, M=8 and M=256 MFMA with split-K partials in the
    # workspace): every replay equals the eager call on the same input.
    d = fp8_big
    W = fp8_dev(d)
    for M in (1, 8, 256):
        r = np.random.default_rng(900 + M)
        xs = [synth.to_bf16_bits(r.standard_normal((M, 5120)).astype(np.float32)) for _ in range(3)]
        xin = bf16_dev(xs[0])
        out = torch.empty((M, 5120), dtype=torch.float32, device=DEV)
        ws = torch.empty(wq.mlp_workspace_bytes(0, M, 5120, 17408), dtype=torch.uint8, device=DEV)
        eager = [host(wq.mlp_fp8w_run(bf16_dev(x), *W)) for x in xs]
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            wq.mlp_fp8w_run(xin, *W, out=out, workspace=ws)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            wq.mlp_fp8w_run(xin, *W, out=out, workspace=ws)
        for rep in range(2):
            for i, x in enumerate(xs):
                xin.copy_(bf16_dev(x))
                g.replay()
                torch.cuda.synchronize()
                assert np.array_equal(host(out).view(np.uint32), eager[i].view(np.uint32)), (M, rep, i)
