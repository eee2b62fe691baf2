"""Python binding of libwqmlp (the C ABI declared in include/wqmlp.h).

Argument marshalling only: torch tensors provide device memory and the
current HIP stream; every step of the computation runs in the library's
gfx950 kernels.  Functions carry the C entry points' names.  A missing or
unloadable library raises at first use; nothing falls back to another path.

Outputs and workspaces that the caller does not pass are allocated with
torch on the input's device (the library itself never allocates).
"""
import ctypes
import os

import torch

__all__ = [
    "WQError", "lib", "lib_path", "WQ_F32", "WQ_BF16", "WQ_F16", "WQ_FMT_FP8W", "WQ_FMT_NVFP4",
    "WQ_PATH_AUTO", "WQ_PATH_GEMV", "WQ_PATH_MFMA", "WQ_STAGE_GATEUP_ONLY", "WQ_STAGE_DOWN_ONLY", "WQ_ACT_E4M3",
    "wq_abi_version", "wq_strerror",
    "WQ_STATIC_SCRATCH_BYTES", "mlp_workspace_bytes", "mlp_fp8w_run", "mlp_fp8w_run_noalloc", "mlp_nvfp4_run", "awq_bank_bytes", "moe_awq_m1_run",
    "nvfp4_pack_block64", "awq_pack_bank", "fp8w_dequant_f32", "nvfp4_dequant_f32", "awq_dequant_f16",
    "qlinear_workspace_bytes", "qlinear_run", "wq_read_probe",
]

WQ_F32, WQ_BF16, WQ_F16 = 0, 1, 2
WQ_FMT_FP8W, WQ_FMT_NVFP4 = 0, 1
WQ_PATH_AUTO, WQ_PATH_GEMV, WQ_PATH_MFMA = 0, 1, 2
WQ_STAGE_GATEUP_ONLY, WQ_STAGE_DOWN_ONLY = 4, 8
WQ_ACT_E4M3 = 16
WQ_STATIC_SCRATCH_BYTES = 32 << 20
_PATHS = {"auto": WQ_PATH_AUTO, "gemv": WQ_PATH_GEMV, "mfma": WQ_PATH_MFMA}
_STAGES = {None: 0, "gateup": WQ_STAGE_GATEUP_ONLY, "down": WQ_STAGE_DOWN_ONLY}
_ACTS = {None: 0, "e4m3": WQ_ACT_E4M3}

# The in-tree library; WQMLP_LIBRARY names another build of it (the host-sanitizer build of the CPU tests).
lib_path = os.environ.get("WQMLP_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libwqmlp.so")
_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_INT = ctypes.c_int
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_SIGS = {
    "wq_abi_version": (_INT, []),
    "wq_strerror": (ctypes.c_char_p, [_INT]),
    "wq_last_hip_error": (_INT, []),
    "mlp_workspace_bytes": (_SZ, [_INT, _I64, _I64, _I64, _INT]),
    "mlp_fp8w_run": (_INT, [_I64, _I64, _I64, _P, _INT, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _INT, _P]),
    "mlp_fp8w_run_noalloc": (_INT, [_I64, _I64, _I64, _P, _INT, _P, _P, _P, _P, _P, _P, _P, _INT, _P]),
    "mlp_nvfp4_run": (_INT, [_I64, _I64, _I64, _P, _INT, _P, _F, _P, _F, _P, _F, _P, _SZ, _P, _INT, _P]),
    "awq_bank_bytes": (_SZ, [_I64, _I64, _I64, _INT]),
    "moe_awq_m1_run": (_INT, [_I64, _I64, _I64, _I64, _P, _P, _P, _P, _P, _INT, _P, _P, _P]),
    "nvfp4_pack_block64": (_INT, [_I64, _I64, _P, _P, _P, _P]),
    "awq_pack_bank": (_INT, [_I64, _I64, _I64, _P, _P, _P, _INT, _P, _P]),
    "fp8w_dequant_f32": (_INT, [_I64, _I64, _P, _P, _P, _P]),
    "nvfp4_dequant_f32": (_INT, [_I64, _I64, _P, _F, _P, _P]),
    "awq_dequant_f16": (_INT, [_I64, _I64, _I64, _P, _INT, _P, _P]),
    "qlinear_workspace_bytes": (_SZ, [_INT, _I64, _I64, _I64, _INT]),
    "qlinear_run": (_INT, [_INT, _I64, _I64, _I64, _P, _INT, _P, _P, _F, _P, _SZ, _P, _INT, _P]),
    "wq_read_probe": (_INT, [_P, _SZ, _P, _INT, _P]),
}


class WQError(RuntimeError):
    def __init__(self, fn, rc):
        self.rc = rc
        msg = lib().wq_strerror(rc).decode()
        extra = ""
        if rc in (-4, -7):
            extra = f" (hipError {lib().wq_last_hip_error()})"
        super().__init__(f"{fn}: rc={rc}: {msg}{extra}")


def lib():
    """Load the in-tree libwqmlp.so once; raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(lib_path):
            raise RuntimeError(f"{lib_path} is not built: run __graft_entry__.build() first")
        so = ctypes.CDLL(lib_path)
        for name, (res, args) in _SIGS.items():
            f = getattr(so, name)
            f.restype = res
            f.argtypes = args
        _lib = so
    return _lib


def _check(fn, rc):
    if rc != 0:
        raise WQError(fn, rc)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t, name, dtype, dev=None, numel=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not t.is_cuda or (dev is not None and t.device != dev):
        raise ValueError(f"{name} must live on {dev or 'a GPU'}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, has {t.numel()}")
    return t


def _xdtype(x, allow_f16=False):
    if x.dtype == torch.float32:
        return WQ_F32
    if x.dtype == torch.bfloat16:
        return WQ_BF16
    if allow_f16 and x.dtype == torch.float16:
        return WQ_F16
    raise TypeError("x must be float32 or bfloat16" + (" (or float16 for NVFP4)" if allow_f16 else ""))


def wq_abi_version():
    return lib().wq_abi_version()


def wq_strerror(rc):
    return lib().wq_strerror(rc).decode()


def mlp_workspace_bytes(fmt, M, H, I, path="auto", act=None):
    return lib().mlp_workspace_bytes(fmt, M, H, I, _PATHS[path] | _ACTS[act])


def _workspace(nbytes, dev, workspace):
    if workspace is None:
        return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev)
    return workspace


def _stage_flags(stage, workspace):
    """Stage bits; a one-stage call must bring the workspace that carries act between the two stages."""
    if stage not in _STAGES:
        raise ValueError(f"stage must be one of {list(_STAGES)}")
    if stage is not None and workspace is None:
        raise ValueError("stage='gateup' or 'down' needs the caller's workspace: act is handed from the "
                         "gate/up stage to the down stage through it")
    return _STAGES[stage]


def mlp_fp8w_run(x, w_gate, s_gate, w_up, s_up, w_down, s_down, out=None, workspace=None, path="auto",
                 stage=None):
    """FP8 E4M3 per-channel SwiGLU MLP.  x [M,H] f32/bf16; w_gate/w_up [I,H] u8; w_down [H,I] u8; s_* f32."""
    sflags = _stage_flags(stage, workspace)
    dev = x.device
    M, H = x.shape
    I = w_gate.shape[0]
    _need(x, "x", x.dtype, dev)
    for n, t, k in (("w_gate", w_gate, I * H), ("w_up", w_up, I * H), ("w_down", w_down, H * I)):
        _need(t, n, torch.uint8, dev, k)
    for n, t, k in (("s_gate", s_gate, I), ("s_up", s_up, I), ("s_down", s_down, H)):
        _need(t, n, torch.float32, dev, k)
    if out is None:
        out = torch.empty((M, H), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, M * H)
    nb = mlp_workspace_bytes(WQ_FMT_FP8W, M, H, I, path)
    ws = _workspace(nb, dev, workspace)
    rc = lib().mlp_fp8w_run(M, H, I, _ptr(x), _xdtype(x), _ptr(w_gate), _ptr(s_gate), _ptr(w_up), _ptr(s_up),
                            _ptr(w_down), _ptr(s_down), _ptr(ws), ws.numel(), _ptr(out),
                            _PATHS[path] | sflags, _stream(dev))
    _check("mlp_fp8w_run", rc)
    return out


def mlp_fp8w_run_noalloc(x, w_gate, s_gate, w_up, s_up, w_down, s_down, out, path="auto"):
    """mlp_fp8w_run on the library's static scratch: no workspace, and the caller passes out (nothing is
    allocated, here or in the library).  Calls needing more than WQ_STATIC_SCRATCH_BYTES raise (WQ_ESCRATCH)."""
    dev = x.device
    M, H = x.shape
    I = w_gate.shape[0]
    _need(x, "x", x.dtype, dev)
    for n, t, k in (("w_gate", w_gate, I * H), ("w_up", w_up, I * H), ("w_down", w_down, H * I)):
        _need(t, n, torch.uint8, dev, k)
    for n, t, k in (("s_gate", s_gate, I), ("s_up", s_up, I), ("s_down", s_down, H)):
        _need(t, n, torch.float32, dev, k)
    _need(out, "out", torch.float32, dev, M * H)
    rc = lib().mlp_fp8w_run_noalloc(M, H, I, _ptr(x), _xdtype(x), _ptr(w_gate), _ptr(s_gate), _ptr(w_up),
                                    _ptr(s_up), _ptr(w_down), _ptr(s_down), _ptr(out), _PATHS[path], _stream(dev))
    _check("mlp_fp8w_run_noalloc", rc)
    return out


def mlp_nvfp4_run(x, gate_blk, gate_gs, up_blk, up_gs, down_blk, down_gs, out=None, workspace=None, path="auto",
                  stage=None, act=None):
    """NVFP4 Block64 SwiGLU MLP.  x [M,H]; gate/up_blk [I,H/64,36] u8; down_blk [H,I/64,36] u8; gs floats.
    act="e4m3": the W4A8 variant (activations quantized per row to E4M3; MFMA path)."""
    sflags = _stage_flags(stage, workspace)
    dev = x.device
    M, H = x.shape
    I = gate_blk.shape[0]
    _need(x, "x", x.dtype, dev)
    for n, t, k in (("gate_blk", gate_blk, I * H // 64 * 36), ("up_blk", up_blk, I * H // 64 * 36),
                    ("down_blk", down_blk, H * I // 64 * 36)):
        _need(t, n, torch.uint8, dev, k)
    if out is None:
        out = torch.empty((M, H), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, M * H)
    nb = mlp_workspace_bytes(WQ_FMT_NVFP4, M, H, I, path, act)
    ws = _workspace(nb, dev, workspace)
    rc = lib().mlp_nvfp4_run(M, H, I, _ptr(x), _xdtype(x), _ptr(gate_blk), float(gate_gs), _ptr(up_blk),
                             float(up_gs), _ptr(down_blk), float(down_gs), _ptr(ws), ws.numel(), _ptr(out),
                             _PATHS[path] | sflags | _ACTS[act], _stream(dev))
    _check("mlp_nvfp4_run", rc)
    return out


def awq_bank_bytes(E, N, K, meta_layout=3):
    return lib().awq_bank_bytes(E, N, K, meta_layout)


def moe_awq_m1_run(x, expert_ids, router_w, w13_bank, w2_bank, E, I, meta_layout=3, act=None, out=None):
    """AWQ routed-expert M=1 step.  x f16-bits [H] (int16/uint16 view or float16); ids int32; weights f32."""
    dev = x.device
    H = x.numel()
    topk = expert_ids.numel()
    xb = x.view(torch.int16) if x.dtype in (torch.float16, torch.int16) else None
    if xb is None:
        raise TypeError("x must be float16 (or its int16 bits)")
    _need(xb, "x", torch.int16, dev)
    _need(expert_ids, "expert_ids", torch.int32, dev)
    _need(router_w, "router_w", torch.float32, dev, topk)
    _need(w13_bank, "w13_bank", torch.uint8, dev, awq_bank_bytes(E, 2 * I, H, meta_layout))
    _need(w2_bank, "w2_bank", torch.uint8, dev, awq_bank_bytes(E, H, I, meta_layout))
    if act is None:
        act = torch.empty((topk, I), dtype=torch.float16, device=dev)
    if out is None:
        out = torch.empty((H,), dtype=torch.float16, device=dev)
    _need(act, "act", torch.float16, dev, topk * I)
    _need(out, "out", torch.float16, dev, H)
    rc = lib().moe_awq_m1_run(E, topk, H, I, _ptr(xb), _ptr(expert_ids), _ptr(router_w), _ptr(w13_bank),
                              _ptr(w2_bank), meta_layout, _ptr(act), _ptr(out), _stream(dev))
    _check("moe_awq_m1_run", rc)
    return out, act


def nvfp4_pack_block64(weight_packed, weight_scale, blk=None):
    """[N,K/2] u8 + [N,K/16] u8 (device) -> Block64 records [N,K/64,36] u8."""
    dev = weight_packed.device
    N, Kh = weight_packed.shape
    K = 2 * Kh
    _need(weight_packed, "weight_packed", torch.uint8, dev)
    _need(weight_scale, "weight_scale", torch.uint8, dev, N * K // 16)
    if blk is None:
        blk = torch.empty((N, K // 64, 36), dtype=torch.uint8, device=dev)
    _need(blk, "blk", torch.uint8, dev, N * K // 64 * 36)
    _check("nvfp4_pack_block64", lib().nvfp4_pack_block64(N, K, _ptr(weight_packed), _ptr(weight_scale),
                                                          _ptr(blk), _stream(dev)))
    return blk


def awq_pack_bank(codes, scales, zeros, meta_layout=3, bank=None):
    """codes [E,N,K] u8 (0..15), scales [E,N,K/32] f16 (or int16 bits), zeros [E,N,K/32] u8 -> bank u8."""
    dev = codes.device
    E, N, K = codes.shape
    _need(codes, "codes", torch.uint8, dev)
    sb = scales.view(torch.int16)
    _need(sb, "scales", torch.int16, dev, E * N * K // 32)
    _need(zeros, "zeros", torch.uint8, dev, E * N * K // 32)
    nb = awq_bank_bytes(E, N, K, meta_layout)
    if bank is None:
        bank = torch.empty(nb, dtype=torch.uint8, device=dev)
    _need(bank, "bank", torch.uint8, dev, nb)
    _check("awq_pack_bank", lib().awq_pack_bank(E, N, K, _ptr(codes), _ptr(sb), _ptr(zeros), meta_layout,
                                                _ptr(bank), _stream(dev)))
    return bank


def fp8w_dequant_f32(w, s):
    dev = w.device
    N, K = w.shape
    _need(w, "w", torch.uint8, dev)
    _need(s, "s", torch.float32, dev, N)
    out = torch.empty((N, K), dtype=torch.float32, device=dev)
    _check("fp8w_dequant_f32", lib().fp8w_dequant_f32(N, K, _ptr(w), _ptr(s), _ptr(out), _stream(dev)))
    return out


def nvfp4_dequant_f32(blk, global_scale):
    dev = blk.device
    N, nb, rb = blk.shape
    _need(blk, "blk", torch.uint8, dev)
    out = torch.empty((N, nb * 64), dtype=torch.float32, device=dev)
    _check("nvfp4_dequant_f32", lib().nvfp4_dequant_f32(N, nb * 64, _ptr(blk), float(global_scale), _ptr(out),
                                                        _stream(dev)))
    return out


def awq_dequant_f16(bank, E, N, K, meta_layout=3):
    dev = bank.device
    _need(bank, "bank", torch.uint8, dev)
    out = torch.empty((E, N, K), dtype=torch.float16, device=dev)
    _check("awq_dequant_f16", lib().awq_dequant_f16(E, N, K, _ptr(bank), meta_layout, _ptr(out), _stream(dev)))
    return out


def qlinear_workspace_bytes(fmt, M, N, K, path="auto", act=None):
    return lib().qlinear_workspace_bytes(fmt, M, N, K, _PATHS[path] | _ACTS[act])


def qlinear_run(fmt, x, w, scale=None, global_scale=1.0, N=None, path="auto", out=None, workspace=None, act=None):
    """y = x dq(W)^T.  FP8: w [N,K] u8 + scale [N] f32; NVFP4: w Block64 [N,K/64,36] + global_scale.
    act="e4m3" (NVFP4): x quantized per row to E4M3 first (the W4A8 variant; MFMA path)."""
    dev = x.device
    M, K = x.shape
    N = w.shape[0] if N is None else N
    _need(x, "x", x.dtype, dev)
    _need(w, "w", torch.uint8, dev)
    if scale is not None:
        _need(scale, "scale", torch.float32, dev, N)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=dev)
    _need(out, "out", torch.float32, dev, M * N)
    nb = 0 if x.dtype == torch.float16 else qlinear_workspace_bytes(fmt, M, N, K, path, act)
    ws = _workspace(nb, dev, workspace) if nb else None
    rc = lib().qlinear_run(fmt, M, N, K, _ptr(x), _xdtype(x, allow_f16=True), _ptr(w), _ptr(scale), float(global_scale), _ptr(ws),
                           0 if ws is None else ws.numel(), _ptr(out), _PATHS[path] | _ACTS[act], _stream(dev))
    _check("qlinear_run", rc)
    return out


def wq_read_probe(src, sink, nbytes=None, grid=None):
    """Streaming read of nbytes (default: all) of the device tensor src; sink: int32 tensor of >= grid words."""
    dev = src.device
    nbytes = src.numel() * src.element_size() if nbytes is None else nbytes
    grid = sink.numel() if grid is None else grid
    _need(sink, "sink", torch.int32, dev)
    if grid > sink.numel() or nbytes > src.numel() * src.element_size():
        raise ValueError("grid exceeds sink or nbytes exceeds src")
    _check("wq_read_probe", lib().wq_read_probe(_ptr(src), nbytes, _ptr(sink), grid, _stream(dev)))
