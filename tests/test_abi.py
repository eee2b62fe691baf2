"""Host-only checks of the C ABI: symbols, sizes and the argument-validation phase.

Every call here returns from the pure-arithmetic validation phase before any HIP
call, so these run on a machine without a GPU.  Pointers are fake addresses.
"""
import ctypes
import os
import re

import pytest

import oracle
import weight_quantized_mlp_amd as wq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wqmlp.h")

EINVAL, EALIGN, EOVERLAP, EWORKSPACE = -1, -2, -3, -6


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(wq.lib_path):
        pytest.fail("libwqmlp.so is not built (run __graft_entry__.build())")
    return wq.lib()


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(L):
    names = header_functions()
    assert set(names) == {
        "wq_abi_version", "wq_strerror", "wq_last_hip_error", "mlp_workspace_bytes", "mlp_fp8w_run",
        "mlp_nvfp4_run", "awq_bank_bytes", "moe_awq_m1_run", "nvfp4_pack_block64", "awq_pack_bank",
        "fp8w_dequant_f32", "nvfp4_dequant_f32", "awq_dequant_f16", "qlinear_workspace_bytes", "qlinear_run",
        "mlp_fp8w_run_noalloc", "wq_read_probe"}
    for n in names:
        assert hasattr(L, n), n
        assert n in wq.__all__ or n == "wq_last_hip_error", n


def test_version_and_messages(L):
    assert wq.wq_abi_version() == 1
    for rc in range(0, -9, -1):
        assert wq.wq_strerror(rc) != "unknown error"
    assert wq.wq_strerror(-99) == "unknown error"


def test_workspace_queries(L):
    assert wq.mlp_workspace_bytes(0, 1, 5120, 17408) == 17408 * 4
    n = wq.mlp_workspace_bytes(1, 512, 5120, 17408)
    assert n >= 512 * 5120 * 2 + 512 * 4 + 512 * 17408 * 2
    assert wq.mlp_workspace_bytes(1, 4, 5120, 17408, "gemv") == 4 * 17408 * 2   # NVFP4 act: float16
    # MFMA path: x16, row scales, act16, then split-K partial tiles of at most 64 MiB
    base = 4 * 5120 * 2 + 256 + 4 * 17408 * 2
    for fmt in (0, 1):                                   # + the split-K partial tiles
        assert base < wq.mlp_workspace_bytes(fmt, 4, 5120, 17408, "mfma") <= base + (64 << 20)
    # AUTO on short batches: the MFMA GEMM from the format's row threshold, for large weights only
    gemv = lambda fmt, M, I: M * I * (2 if fmt == 1 else 4)    # act: float16 (NVFP4) / float32 (FP8)
    assert wq.mlp_workspace_bytes(1, 2, 5120, 17408) == gemv(1, 2, 17408)
    assert wq.mlp_workspace_bytes(1, 3, 5120, 17408) == wq.mlp_workspace_bytes(1, 3, 5120, 17408, "mfma")
    assert wq.mlp_workspace_bytes(0, 1, 5120, 17408) == gemv(0, 1, 17408)
    assert wq.mlp_workspace_bytes(0, 2, 5120, 17408) == wq.mlp_workspace_bytes(0, 2, 5120, 17408, "mfma")
    assert wq.mlp_workspace_bytes(1, 64, 256, 512) == gemv(1, 64, 512)           # 0.2 MB of weights
    assert wq.mlp_workspace_bytes(0, 64, 5120 + 16, 17408) == gemv(0, 64, 17408)   # H not a multiple of 64
    assert wq.qlinear_workspace_bytes(1, 2, 5120, 17408) == 0
    assert wq.qlinear_workspace_bytes(1, 3, 5120, 17408) > 0
    assert wq.mlp_workspace_bytes(7, 1, 64, 64) == 0
    assert wq.mlp_workspace_bytes(0, 0, 64, 64) == 0
    assert wq.qlinear_workspace_bytes(1, 4, 64, 64) == 0
    assert wq.qlinear_workspace_bytes(1, 128, 64, 64) > 0
    # every dimension is capped at WQ_MAX_DIM = 2^23
    assert wq.mlp_workspace_bytes(1, 1 << 23, 64, 64) > 0
    assert wq.mlp_workspace_bytes(1, (1 << 23) + 1, 64, 64) == 0
    assert wq.mlp_workspace_bytes(0, 1, 64, (1 << 23) + 64) == 0
    assert wq.qlinear_workspace_bytes(1, (1 << 23) + 1, 64, 64) == 0
    # ... and every activation or output matrix at 2^36 elements
    assert wq.mlp_workspace_bytes(1, 1 << 23, 1 << 13, 64) > 0
    assert wq.mlp_workspace_bytes(1, 1 << 23, 64, (1 << 13) + 64) == 0
    assert wq.qlinear_workspace_bytes(1, 1 << 23, (1 << 13) + 1, 64) == 0


@pytest.mark.parametrize("E,N,K", [(512, 320, 2560), (512, 2560, 160), (3, 64, 96)])
@pytest.mark.parametrize("ml", [3, 4])
def test_awq_bank_bytes_match_oracle_layout(L, E, N, K, ml):
    assert wq.awq_bank_bytes(E, N, K, ml) == E * oracle.awq_bank_layout(N, K, ml)["expert_bytes"]
    assert wq.awq_bank_bytes(E, N, K + 1, ml) == 0
    assert wq.awq_bank_bytes(E, N, K, 5) == 0


A = 1 << 32   # fake, 16-byte aligned device-looking addresses (never dereferenced)


def fp8_args(**kw):
    a = dict(M=1, H=64, I=128, x=A, dt=1, wg=A + 0x100000, sg=A + 0x200000, wu=A + 0x300000, su=A + 0x400000,
             wd=A + 0x500000, sd=A + 0x600000, ws=A + 0x700000, wsb=1 << 20, out=A + 0x800000, flags=0, st=None)
    a.update(kw)
    return [a[k] for k in ("M", "H", "I", "x", "dt", "wg", "sg", "wu", "su", "wd", "sd", "ws", "wsb", "out", "flags",
                           "st")]


@pytest.mark.parametrize("kw,rc", [
    (dict(x=None), EINVAL), (dict(wd=None), EINVAL), (dict(sg=None), EINVAL), (dict(out=None), EINVAL),
    (dict(dt=2), EINVAL), (dict(dt=9), EINVAL), (dict(flags=3), EINVAL), (dict(M=-1), EINVAL),
    (dict(H=0), EINVAL), (dict(H=72), EINVAL), (dict(I=40), EINVAL),
    (dict(M=200, H=80), EINVAL),                        # MFMA path needs multiples of 64
    (dict(x=A + 8), EALIGN), (dict(wg=A + 0x100004), EALIGN), (dict(sd=A + 0x600002), EALIGN),
    (dict(out=A + 0x800008), EALIGN), (dict(ws=A + 0x700001), EALIGN),
    (dict(ws=None), EWORKSPACE), (dict(wsb=128 * 4 - 1), EWORKSPACE),
    (dict(out=A), EOVERLAP), (dict(out=A + 0x100000), EOVERLAP), (dict(ws=A + 0x600000), EOVERLAP),
    (dict(ws=A + 0x800000), EOVERLAP),
])
def test_fp8_validation(L, kw, rc):
    assert L.mlp_fp8w_run(*fp8_args(**kw)) == rc


def test_flag_combinations(L):
    # path bits 3 (both paths) and both stage bits together are invalid, as are unknown bits
    assert L.mlp_fp8w_run(*fp8_args(flags=3)) == EINVAL
    assert L.mlp_fp8w_run(*fp8_args(flags=4 | 8)) == EINVAL
    assert L.mlp_fp8w_run(*fp8_args(flags=16)) == EINVAL


def test_empty_batch_is_ok(L):
    assert L.mlp_fp8w_run(*fp8_args(M=0)) == 0
    # an empty batch may pass NULL activations, output and workspace; the weights are still checked
    assert L.mlp_fp8w_run(*fp8_args(M=0, x=None, out=None, ws=None, wsb=0)) == 0
    assert L.mlp_fp8w_run(*fp8_args(M=0, wg=None)) == EINVAL
    assert L.qlinear_run(1, 0, 64, 64, None, 1, A + 4096, None, 1.0, None, 0, None, 0, None) == 0
    assert L.qlinear_run(1, 0, 64, 64, None, 1, None, None, 1.0, None, 0, None, 0, None) == EINVAL


def nv_args(**kw):
    a = dict(M=1, H=64, I=128, x=A, dt=1, gb=A + 0x100000, gg=1.0, ub=A + 0x300000, ug=1.0,
             db=A + 0x500000, dg=1.0, ws=A + 0x700000, wsb=1 << 20, out=A + 0x800000, flags=0, st=None)
    a.update(kw)
    return [a[k] for k in ("M", "H", "I", "x", "dt", "gb", "gg", "ub", "ug", "db", "dg", "ws", "wsb", "out",
                           "flags", "st")]


@pytest.mark.parametrize("kw,rc", [
    (dict(H=96), EINVAL), (dict(I=32), EINVAL), (dict(gg=0.0), EINVAL), (dict(dg=-1.0), EINVAL),
    (dict(ug=float("inf")), EINVAL), (dict(ug=float("nan")), EINVAL), (dict(db=None), EINVAL),
    (dict(gb=A + 0x100004), EALIGN), (dict(ws=None), EWORKSPACE),
    (dict(out=A + 0x500000), EOVERLAP),
])
def test_nvfp4_validation(L, kw, rc):
    assert L.mlp_nvfp4_run(*nv_args(**kw)) == rc


def moe_args(**kw):
    a = dict(E=512, topk=10, H=2560, I=160, x=A, ids=A + 0x1000, rw=A + 0x2000, w13=A + 0x10000000,
             w2=A + 0x40000000, ml=3, act=A + 0x3000, out=A + 0x4000, st=None)
    a.update(kw)
    return [a[k] for k in ("E", "topk", "H", "I", "x", "ids", "rw", "w13", "w2", "ml", "act", "out", "st")]


@pytest.mark.parametrize("kw,rc", [
    (dict(E=0), EINVAL), (dict(topk=0), EINVAL), (dict(topk=17), EINVAL), (dict(H=2561), EINVAL),
    (dict(I=100), EINVAL), (dict(ml=5), EINVAL), (dict(ids=None), EINVAL), (dict(out=None), EINVAL),
    (dict(x=A + 2), EALIGN), (dict(rw=A + 0x2004), EALIGN), (dict(w2=A + 0x40000008), EALIGN),
    (dict(act=A + 0x10), EOVERLAP), (dict(out=A + 0x3000 + 64), EOVERLAP), (dict(out=A + 0x10000000 + 4096), EOVERLAP),
])
def test_moe_validation(L, kw, rc):
    assert L.moe_awq_m1_run(*moe_args(**kw)) == rc


def test_packer_and_decoder_validation(L):
    assert L.nvfp4_pack_block64(4, 96, A, A + 4096, A + 8192, None) == EINVAL
    assert L.nvfp4_pack_block64(4, 128, A, A + 4096, A + 128, None) == EOVERLAP
    assert L.awq_pack_bank(2, 8, 33, A, A + 4096, A + 8192, 3, A + 16384, None) == EINVAL
    assert L.awq_pack_bank(2, 8, 64, A, A + 4096, A + 8192, 3, A + 16388, None) == EALIGN
    assert L.fp8w_dequant_f32(4, 16, A, None, A + 4096, None) == EINVAL
    assert L.nvfp4_dequant_f32(4, 64, A, 0.0, A + 4096, None) == EINVAL
    assert L.awq_dequant_f16(1, 8, 64, A, 4, A + 16, None) == EOVERLAP
    assert L.qlinear_run(2, 1, 64, 64, A, 1, A + 4096, A + 8192, 1.0, None, 0, A + 12288, 0, None) == EINVAL
    assert L.qlinear_run(0, 1, 64, 64, A, 1, A + 4096, None, 1.0, None, 0, A + 12288, 0, None) == EINVAL
    assert L.qlinear_run(1, 128, 64, 64, A, 1, A + 4096, None, 1.0, None, 0, A + 1 << 20, 0, None) == EWORKSPACE


def test_qlinear_shape_rules(L):
    # K carries the alignment (NVFP4 records, MFMA K steps, FP8 16-byte chunks); any N passes the shape
    # checks (the workspace check after them is what rejects these calls: none is given)
    assert L.qlinear_run(1, 1, 64, 96, A, 1, A + 4096, None, 1.0, None, 0, A + 12288, 0, None) == EINVAL
    assert L.qlinear_run(0, 1, 64, 24, A, 1, A + 4096, A + 8192, 1.0, None, 0, A + 12288, 1, None) == EINVAL
    assert L.qlinear_run(0, 128, 64, 96, A, 1, A + 4096, A + 8192, 1.0, None, 0, A + 12288, 2, None) == EINVAL
    for fmt, scale in ((1, None), (0, A + 0x100000)):
        assert L.qlinear_run(fmt, 129, 67, 320, A, 1, A + 0x200000, scale, 1.0, None, 0, A + 0x400000, 0,
                             None) == EWORKSPACE
        assert wq.qlinear_workspace_bytes(fmt, 129, 67, 320) > 0
    # float16 x: NVFP4 on the GEMV path only
    assert L.qlinear_run(0, 1, 64, 64, A, 2, A + 4096, A + 8192, 1.0, None, 0, A + 12288, 0, None) == EINVAL
    assert L.qlinear_run(1, 1, 64, 64, A, 2, A + 4096, None, 1.0, None, 0, A + 12288, 2, None) == EINVAL
    assert L.qlinear_run(1, 1, 64, 64, A, 3, A + 4096, None, 1.0, None, 0, A + 12288, 0, None) == EINVAL
    assert L.qlinear_run(1, 1, 64, 64, A + 2, 2, A + 4096, None, 1.0, None, 0, A + 12288, 0, None) == EALIGN


def test_header_and_library_from_c(tmp_path):
    # the boundary needs no Python: the header compiles as C99 and a C program links the library and calls it
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.join(root, "weight_quantized_mlp_amd")
    src = tmp_path / "use.c"
    src.write_text('#include "wqmlp.h"\n#include <stdio.h>\n'
                   "int main(void) {\n"
                   "  size_t ws = mlp_workspace_bytes(WQ_FMT_NVFP4, 1, 5120, 17408, WQ_PATH_AUTO);\n"
                   '  printf("%d %zu %s\\n", wq_abi_version(), ws, wq_strerror(WQ_EINVAL));\n'
                   "  return ws == 17408 * 2 ? 0 : 1;\n}\n")
    exe = tmp_path / "use"
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(root, "include"),
                    str(src), "-o", str(exe), "-L", libdir, "-lwqmlp", "-Wl,-rpath," + libdir], check=True)
    p = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert p.returncode == 0, p.stdout + p.stderr
    assert p.stdout.split()[0] == str(wq.lib().wq_abi_version())


def test_mfma_workspace_holds_the_documented_regions(L):
    # The header's MFMA workspace: x16 [M,H] f16, row scales [M], act16 [M,I] f16, for FP8 also act [M,I]
    # f32 and its row scales [M], each 256-byte aligned, then split-K partial tiles of at most 64 MiB.  At
    # M = 8192 both GEMMs run whole rounds of tiles (no split), so the workspace is exactly the regions.
    H, I = 5120, 17408
    a = lambda n: -(-n // 256) * 256
    for fmt in (0, 1):
        for M in (2, 3, 8, 32, 33, 64, 65, 96, 97, 128, 129, 512, 8192):
            regions = a(M * H * 2) + a(M * 4) + a(M * I * 2)
            if fmt == 0:
                regions += a(M * I * 4) + a(M * 4)
            n = wq.mlp_workspace_bytes(fmt, M, H, I, "mfma")
            assert regions <= n <= regions + (64 << 20), (fmt, M)
            assert n % 256 == 0
            if M == 8192:
                assert n == regions, fmt
            if M <= 128:
                assert n > regions, (fmt, M)    # short batches split every tile along K


def test_w4a8_workspace_holds_the_documented_regions(L):
    # The header's W4A8 workspace (NVFP4 with WQ_ACT_E4M3): x's E4M3 values as float16 [M,H], x row scales
    # [M], act f32 [M,I], act's E4M3 values as float16 [M,I], act row scales [M], each 256-byte aligned, then
    # the split-K partial tiles (at most 64 MiB; none at M = 8192); 0 for FP8 or the GEMV path, and for a
    # K that is not a multiple of 64 or is below 256.
    H, I = 5120, 17408
    a = lambda n: -(-n // 256) * 256
    for M in (1, 8, 32, 64, 129, 512, 8192):
        regions = a(M * H * 2) + a(M * 4) + a(M * I * 4) + a(M * I * 2) + a(M * 4)
        n = wq.mlp_workspace_bytes(1, M, H, I, "auto", "e4m3")
        assert regions <= n <= regions + (64 << 20) and n % 256 == 0, M
        if M == 8192:
            assert n == regions
    assert wq.mlp_workspace_bytes(0, 8, H, I, "auto", "e4m3") == 0
    assert wq.mlp_workspace_bytes(1, 8, H, I, "gemv", "e4m3") == 0
    assert wq.mlp_workspace_bytes(1, 8, 320, 512, "auto", "e4m3") > 0      # K = 320: a multiple of 64
    assert wq.mlp_workspace_bytes(1, 8, 192, 512, "auto", "e4m3") == 0     # K = 192: below 256
    assert wq.mlp_workspace_bytes(1, 8, 288, 512, "auto", "e4m3") == 0     # K = 288: not a multiple of 64


def test_binding_stage_calls_need_a_workspace():
    # a one-stage call hands act to the other stage through the caller's workspace; without one the
    # binding raises before touching the device (CPU tensors here never reach the library)
    x = __import__("torch").zeros((1, 64))
    for run in (wq.mlp_fp8w_run, wq.mlp_nvfp4_run):
        for stage in ("gateup", "down"):
            with pytest.raises(ValueError, match="workspace"):
                run(x, *([None] * 6), stage=stage)
        with pytest.raises(ValueError, match="stage"):
            run(x, *([None] * 6), stage="both")


def test_noalloc_validation(L):
    # mlp_fp8w_run_noalloc: pure checks first; a call needing more than the static scratch is WQ_ESCRATCH
    ESCRATCH = -8
    H, I = 5120, 17408
    args = lambda M, flags: (M, H, I, A, 1, A + 0x10000000, A + 0x20000000, A + 0x30000000, A + 0x40000000,
                             A + 0x50000000, A + 0x60000000, A + 0x70000000, flags, None)
    assert wq.mlp_workspace_bytes(0, 64, H, I) > wq.WQ_STATIC_SCRATCH_BYTES >= wq.mlp_workspace_bytes(0, 32, H, I)
    assert L.mlp_fp8w_run_noalloc(*args(64, 0)) == ESCRATCH
    assert L.mlp_fp8w_run_noalloc(*args(512, 0)) == ESCRATCH
    assert L.mlp_fp8w_run_noalloc(*args(1, 4)) == EINVAL            # stage bits: whole calls only
    assert L.mlp_fp8w_run_noalloc(*args(1, 16)) == EINVAL
    assert L.mlp_fp8w_run_noalloc(*args(0, 0)) == 0                 # empty batch
    a = list(args(1, 0))
    a[3] = None
    assert L.mlp_fp8w_run_noalloc(*a) == EINVAL                     # null x
    a = list(args(1, 0))
    a[11] = A + 4                                                   # misaligned out
    assert L.mlp_fp8w_run_noalloc(*a) == EALIGN
    a = list(args(1, 0))
    a[11] = A + 0x10000000                                          # out on the gate weights
    assert L.mlp_fp8w_run_noalloc(*a) == EOVERLAP


def test_read_probe_validation(L):
    assert L.wq_read_probe(None, 1 << 20, A, 8, None) == EINVAL
    assert L.wq_read_probe(A, 0, A + (1 << 30), 8, None) == EINVAL
    assert L.wq_read_probe(A, 100, A + (1 << 30), 8, None) == EINVAL          # not a multiple of 16
    assert L.wq_read_probe(A, 1 << 20, A + (1 << 30), 0, None) == EINVAL
    assert L.wq_read_probe(A + 8, 1 << 20, A + (1 << 30), 8, None) == EALIGN
    assert L.wq_read_probe(A, 1 << 20, A + 4096, 8, None) == EOVERLAP


def test_c_consumer_compiles_links_and_runs(L, tmp_path):
    # the header as strict C99 and the library linked by a C program (tests/c_consumer.c)
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    if os.environ.get("WQMLP_LIBRARY"):
        pytest.skip("another build of the library is loaded (the sanitizer build needs its runtime linked)")
    libdir = os.path.dirname(os.path.abspath(wq.lib_path))
    exe = str(tmp_path / "c_consumer")
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                        "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_consumer.c"),
                        "-L", libdir, "-l:" + os.path.basename(wq.lib_path), "-Wl,-rpath," + libdir, "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "c consumer ok", (r.returncode, r.stdout, r.stderr)
