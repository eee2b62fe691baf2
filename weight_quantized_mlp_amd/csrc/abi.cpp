// C ABI of libwqmlp (declarations and contracts: include/wqmlp.h).
//
// Every entry point validates in two phases before anything is enqueued:
//   1. pure arithmetic on the arguments (nulls, enums, shapes, 16-byte alignment,
//      pairwise byte-range overlap of outputs/workspace against inputs, workspace
//      size) -- no HIP call, so a host without a GPU can exercise every such path;
//   2. device checks: the current device is gfx950 and every pointer is device
//      memory of that device.
// Then the kernels are enqueued on the caller's stream.  A failed launch is reported
// as WQ_ELAUNCH; there is no alternative or host path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>
#include <mutex>

#include "../../include/wqmlp.h"
#include "launch.h"

// Static scratch of mlp_fp8w_run_noalloc: one array per device, part of the library's code object; the
// loader places it in each device's memory when the library is first used there, and it stays until the
// process ends.  In host code `scratch` names a host-side stand-in, never the device array: its device
// address is taken once per device with hipGetSymbolAddress (that device current, static_scratch below)
// and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[WQ_STATIC_SCRATCH_BYTES];

namespace {

thread_local int g_last_hip = 0;

struct Rng {
  const void* p;
  size_t n;
};

bool overlaps(Rng a, Rng b) {
  if (a.n == 0 || b.n == 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + b.n && b0 < a0 + a.n;
}

bool any_overlap(std::initializer_list<Rng> outs, std::initializer_list<Rng> ins) {
  for (const Rng& o : outs)
    for (const Rng& i : ins)
      if (overlaps(o, i)) return true;
  // outputs must not overlap each other either
  for (auto a = outs.begin(); a != outs.end(); ++a)
    for (auto b = a + 1; b != outs.end(); ++b)
      if (overlaps(*a, *b)) return true;
  return false;
}

bool all_aligned(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (((uintptr_t)p & 15u) != 0) return false;
  return true;
}

bool any_null(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (p == nullptr) return true;
  return false;
}

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// ---- device checks (phase 2) ---------------------------------------------------------------------
constexpr int kMaxDev = 64;
std::once_flag g_arch_once[kMaxDev];
int g_arch_ok[kMaxDev];

int check_device(std::initializer_list<const void*> ptrs) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDev) {
    g_last_hip = (int)e;
    return WQ_EDEVICE;
  }
  std::call_once(g_arch_once[dev], [dev] {
    hipDeviceProp_t p;
    g_arch_ok[dev] = hipGetDeviceProperties(&p, dev) == hipSuccess && std::strncmp(p.gcnArchName, "gfx950", 6) == 0;
  });
  if (!g_arch_ok[dev]) return WQ_EARCH;
  for (const void* p : ptrs) {
    if (p == nullptr) continue;
    hipPointerAttribute_t a;
    e = hipPointerGetAttributes(&a, p);
    if (e != hipSuccess) {
      (void)hipGetLastError();  // clear the sticky error left by an unknown pointer
      g_last_hip = (int)e;
      return WQ_EDEVICE;
    }
    if (a.type != hipMemoryTypeDevice || a.device != dev) return WQ_EDEVICE;
  }
  return WQ_OK;
}

int launched(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip = (int)e;
    return WQ_ELAUNCH;
  }
  return WQ_OK;
}

size_t xsize(int dt) { return dt == WQ_F32 ? 4 : 2; }

// GEMV activation staging must fit one workgroup's LDS (160 KiB on gfx950).
bool gemv_fits(int fmt, int64_t K, int dt) {
  const size_t esz = xsize(dt);
  const size_t per_row = fmt == WQ_FMT_FP8W ? (size_t)(K / 16) * (16 * esz + 16) : (size_t)(K / 64) * (64 * esz + 16);
  return per_row <= 160 * 1024;
}

constexpr int64_t kMaxDim = WQ_MAX_DIM;
// rows x columns of any activation or output matrix (keeps tile and grid counts in int)
constexpr int64_t kMaxElems = WQ_MAX_ELEMS;
bool elems_ok(int64_t M, int64_t a, int64_t b) { return M * std::max(a, b) <= kMaxElems; }

size_t wbytes(int fmt, int64_t N, int64_t K) {
  return fmt == WQ_FMT_FP8W ? (size_t)N * (size_t)K : (size_t)N * (size_t)(K / 64) * 36;
}

// AUTO: the MFMA GEMM for M >= WQ_MFMA_MIN_ROWS, and for shorter batches of at least the format's
// WQ_NARROW_MIN_ROWS_* rows when the call's weights hold at least WQ_NARROW_MIN_WEIGHT_BYTES and both
// dimensions are multiples of 64 (the GEMV streams the weights once per row; the GEMM once per call).
// wb: weight bytes of the call (all matrices).
int pick_path(int fmt, int64_t M, int64_t D0, int64_t D1, size_t wb, int flags) {
  flags &= 3;
  if (flags == WQ_PATH_GEMV || flags == WQ_PATH_MFMA) return flags;
  if (M >= WQ_MFMA_MIN_ROWS) return WQ_PATH_MFMA;
  const int64_t narrow = fmt == WQ_FMT_NVFP4 ? WQ_NARROW_MIN_ROWS_NVFP4 : WQ_NARROW_MIN_ROWS_FP8;
  if (M >= narrow && wb >= (size_t)WQ_NARROW_MIN_WEIGHT_BYTES && D0 % 64 == 0 && D1 % 64 == 0) return WQ_PATH_MFMA;
  return WQ_PATH_GEMV;
}
// The W4A8 variant (WQ_ACT_E4M3) runs on the MFMA path only.
int mlp_path(int fmt, int64_t M, int64_t H, int64_t I, int flags) {
  if (flags & WQ_ACT_E4M3) return WQ_PATH_MFMA;
  return pick_path(fmt, M, H, I, 2 * wbytes(fmt, I, H) + wbytes(fmt, H, I), flags);
}
int linear_path(int fmt, int64_t M, int64_t N, int64_t K, int flags) {
  if (flags & WQ_ACT_E4M3) return WQ_PATH_MFMA;
  return pick_path(fmt, M, N, K, wbytes(fmt, N, K), flags);
}
// A dimension the W4A8 GEMMs take as K: whole 64-wide steps (Block64 records), at least four (one weight block).
bool w8_k_ok(int64_t K) { return K % 64 == 0 && K >= 256; }

// Split-K scratch of the MFMA path: gate+up and down run one after the other and share it.
size_t mlp_partials(int fmt, int64_t M, int64_t H, int64_t I) {
  const int f = fmt == WQ_FMT_NVFP4 ? 1 : 0;
  return std::max(wq::mfma_partial_bytes(f, (int)M, (int)H, (int)I, true),
                  wq::mfma_partial_bytes(f, (int)M, (int)I, (int)H, false));
}

// GEMV path act element: float32 for FP8 (no rounding between the GEMMs, as the FP8 definition asks),
// float16 for NVFP4.
size_t act_gemv_bytes(int fmt) { return fmt == WQ_FMT_NVFP4 ? 2 : 4; }

// Byte offsets of the MFMA path's workspace regions (each 256-byte aligned, in this order):
//   x16 [M,H] float16 (row-scaled x), rs [M] float32 (x row scales), act16 [M,I] float16 (the down
//   GEMM's operand); FP8 only: act32 [M,I] float32 (act as the gate/up stage produced it) and ars [M]
//   float32 (act row scales); then the split-K partial tiles.
struct MfmaWs {
  size_t x16, rs, act16, act32, ars, partials, total;
};
MfmaWs mfma_ws(int fmt, int64_t M, int64_t H, int64_t I) {
  MfmaWs w{};
  size_t o = 0;
  w.x16 = o;
  o += align256((size_t)M * H * 2);
  w.rs = o;
  o += align256((size_t)M * 4);
  w.act16 = o;
  o += align256((size_t)M * I * 2);
  if (fmt == WQ_FMT_FP8W) {
    w.act32 = o;
    o += align256((size_t)M * I * 4);
    w.ars = o;
    o += align256((size_t)M * 4);
  }
  w.partials = o;
  o += align256(mlp_partials(fmt, M, H, I));
  w.total = o;
  return w;
}

// Workspace regions of the W4A8 variant (each 256-byte aligned, in this order): xq [M,H] float16 holding
// the E4M3 values of x's rows (scaled by their row scale's inverse), sx [M] float32 (x row scales), act32
// [M,I] float32, aq [M,I] float16 holding the E4M3 values of act's rows, sa [M] float32 (act row scales),
// then the split-K partial tiles of the larger of the two GEMMs.
struct W8Ws {
  size_t xq, sx, act32, aq, sa, partials, total;
};
W8Ws w8_ws(int64_t M, int64_t H, int64_t I) {
  W8Ws w{};
  size_t o = 0;
  w.xq = o;
  o += align256((size_t)M * H * 2);
  w.sx = o;
  o += align256((size_t)M * 4);
  w.act32 = o;
  o += align256((size_t)M * I * 4);
  w.aq = o;
  o += align256((size_t)M * I * 2);
  w.sa = o;
  o += align256((size_t)M * 4);
  w.partials = o;
  o += align256(std::max(wq::w4a8_partial_bytes((int)M, (int)H, (int)I, true),
                         wq::w4a8_partial_bytes((int)M, (int)I, (int)H, false)));
  w.total = o;
  return w;
}

// Workspace of the two-layer MLP; 0 means "invalid".
size_t mlp_ws(int fmt, int64_t M, int64_t H, int64_t I, int flags) {
  if (M <= 0 || H <= 0 || I <= 0 || M > kMaxDim || H > kMaxDim || I > kMaxDim || !elems_ok(M, H, I)) return 0;
  if (flags & WQ_ACT_E4M3) return fmt == WQ_FMT_NVFP4 && w8_k_ok(H) && w8_k_ok(I) ? w8_ws(M, H, I).total : 0;
  if (mlp_path(fmt, M, H, I, flags) == WQ_PATH_GEMV) return align256((size_t)M * I * act_gemv_bytes(fmt));
  return mfma_ws(fmt, M, H, I).total;
}

bool shape_ok(int fmt, int path, int64_t H, int64_t I, int x_dtype) {
  if (H <= 0 || I <= 0 || H > kMaxDim || I > kMaxDim) return false;
  if (path == WQ_PATH_MFMA || fmt == WQ_FMT_NVFP4) {
    if (H % 64 || I % 64) return false;
  } else if (H % 16 || I % 16) {
    return false;
  }
  if (path == WQ_PATH_GEMV && (!gemv_fits(fmt, H, x_dtype) || !gemv_fits(fmt, I, fmt == WQ_FMT_NVFP4 ? WQ_F16 : WQ_F32)))
    return false;
  return true;
}

// ---- the static scratch of mlp_fp8w_run_noalloc (the array itself is declared at file scope above) ------
std::once_flag g_scratch_once[kMaxDev];
void* g_scratch_ptr[kMaxDev];
int g_scratch_err[kMaxDev];

// Device address of the current device's scratch (WQ_OK), or WQ_EDEVICE with the hipError_t recorded.
int static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDev) {
    g_last_hip = (int)e;
    return WQ_EDEVICE;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_err[dev] = (int)err;
    g_scratch_ptr[dev] = err == hipSuccess ? p : nullptr;
  });
  if (g_scratch_ptr[dev] == nullptr) {
    g_last_hip = g_scratch_err[dev] ? g_scratch_err[dev] : (int)hipErrorInvalidSymbol;
    return WQ_EDEVICE;
  }
  *out = g_scratch_ptr[dev];
  return WQ_OK;
}

// Shared body of the MLP entry points.
// use_static: the workspace is the library's static scratch (ws and ws_bytes are ignored): a call that
// needs more than WQ_STATIC_SCRATCH_BYTES is WQ_ESCRATCH, and the scratch's address is taken only after
// every other check has passed (it is not an allocation the pointer query knows, so it is not checked).
int mlp_run(int fmt, int64_t M, int64_t H, int64_t I, const void* x, int x_dtype, const uint8_t* wg,
            const float* sg, float gg, const uint8_t* wu, const float* su, float gu, const uint8_t* wd,
            const float* sd, float gd, void* ws, size_t ws_bytes, float* out, int flags, void* stream,
            bool use_static = false) {
  const int stage = flags & (WQ_STAGE_GATEUP_ONLY | WQ_STAGE_DOWN_ONLY);
  if ((flags & ~31) || (flags & 3) == 3 || stage == (WQ_STAGE_GATEUP_ONLY | WQ_STAGE_DOWN_ONLY)) return WQ_EINVAL;
  const bool w8 = (flags & WQ_ACT_E4M3) != 0;   // W4A8: NVFP4 only, MFMA path only
  if (w8 && (fmt != WQ_FMT_NVFP4 || (flags & 3) == WQ_PATH_GEMV)) return WQ_EINVAL;
  const bool do_gu = stage != WQ_STAGE_DOWN_ONLY, do_down = stage != WQ_STAGE_GATEUP_ONLY;
  if (x_dtype != WQ_F32 && x_dtype != WQ_BF16) return WQ_EINVAL;
  if (M < 0 || M > kMaxDim) return WQ_EINVAL;
  if (H <= 0 || I <= 0 || H > kMaxDim || I > kMaxDim || !elems_ok(M, H, I)) return WQ_EINVAL;
  const int path = mlp_path(fmt, M, H, I, flags);
  if (!shape_ok(fmt, path, H, I, x_dtype)) return WQ_EINVAL;
  if (w8 && (!w8_k_ok(H) || !w8_k_ok(I))) return WQ_EINVAL;
  if (any_null({wg, wu, wd})) return WQ_EINVAL;
  if (fmt == WQ_FMT_FP8W && any_null({sg, su, sd})) return WQ_EINVAL;
  if (fmt == WQ_FMT_NVFP4) {
    for (float g : {gg, gu, gd})
      if (!(g > 0.f) || !std::isfinite(g)) return WQ_EINVAL;
  }
  if (M == 0) return WQ_OK;   // nothing to do: x, out and the workspace may be null
  if (any_null({x, out})) return WQ_EINVAL;
  if (use_static) ws = nullptr;
  if (!all_aligned({x, wg, wu, wd, out, ws})) return WQ_EALIGN;
  if (fmt == WQ_FMT_FP8W && !all_aligned({sg, su, sd})) return WQ_EALIGN;
  const size_t need = mlp_ws(fmt, M, H, I, flags & (3 | WQ_ACT_E4M3));
  if (use_static) {
    if (need > WQ_STATIC_SCRATCH_BYTES) return WQ_ESCRATCH;
  } else if (ws == nullptr || ws_bytes < need) {
    return WQ_EWORKSPACE;
  }
  const size_t nx = (size_t)M * H * xsize(x_dtype);
  const size_t nw_gu = wbytes(fmt, I, H), nw_d = wbytes(fmt, H, I);
  const size_t ns_gu = fmt == WQ_FMT_FP8W ? (size_t)I * 4 : 0, ns_d = fmt == WQ_FMT_FP8W ? (size_t)H * 4 : 0;
  if (any_overlap({{out, (size_t)M * H * 4}, {ws, use_static ? 0 : need}},
                  {{x, nx}, {wg, nw_gu}, {wu, nw_gu}, {wd, nw_d}, {sg, ns_gu}, {su, ns_gu}, {sd, ns_d}}))
    return WQ_EOVERLAP;
  int rc = check_device({x, wg, wu, wd, sg, su, sd, ws, out});
  if (rc != WQ_OK) return rc;
  if (use_static && (rc = static_scratch(&ws)) != WQ_OK) return rc;

  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const wq::XType xt = x_dtype == WQ_BF16 ? wq::X_BF16 : wq::X_F32;
  const int m = (int)M, h = (int)H, i = (int)I;
  if (path == WQ_PATH_GEMV) {
    float* act = reinterpret_cast<float*>(ws);          // FP8: float32; NVFP4: float16 bits
    if (fmt == WQ_FMT_FP8W) {
      if (do_gu) rc = launched(wq::launch_fp8w_gemv(m, h, i, x, xt, wg, sg, wu, su, act, st));
      if (rc == WQ_OK && do_down)
        rc = launched(wq::launch_fp8w_gemv(m, i, h, act, wq::X_F32, wd, sd, nullptr, nullptr, out, st));
    } else {
      if (do_gu) rc = launched(wq::launch_nvfp4_gemv(m, h, i, x, xt, wg, 1.0f / gg, wu, 1.0f / gu, act, true, st));
      if (rc == WQ_OK && do_down)
        rc = launched(wq::launch_nvfp4_gemv(m, i, h, act, wq::X_F16, wd, 1.0f / gd, nullptr, 0.f, out, false, st));
    }
    return rc;
  }
  uint8_t* base = reinterpret_cast<uint8_t*>(ws);
  if (w8) {
    // W4A8: x quantized per token once for gate and up; act (float32) quantized the same way for down
    const W8Ws L = w8_ws(M, H, I);
    uint16_t* xq = reinterpret_cast<uint16_t*>(base + L.xq);
    float* sx = reinterpret_cast<float*>(base + L.sx);
    float* act32 = reinterpret_cast<float*>(base + L.act32);
    uint16_t* aq = reinterpret_cast<uint16_t*>(base + L.aq);
    float* sa = reinterpret_cast<float*>(base + L.sa);
    float* partials = L.total > L.partials ? reinterpret_cast<float*>(base + L.partials) : nullptr;
    if (do_gu) {
      rc = launched(wq::launch_quant_e4m3(m, h, x, xt, xq, sx, st));
      if (rc == WQ_OK)
        rc = launched(wq::launch_w4a8_gateup(m, h, i, xq, sx, wg, 1.0f / gg, wu, 1.0f / gu, act32, partials, st));
    }
    if (rc == WQ_OK && do_down) {
      rc = launched(wq::launch_quant_e4m3(m, i, act32, wq::X_F32, aq, sa, st));
      if (rc == WQ_OK) rc = launched(wq::launch_w4a8_linear(m, i, h, aq, sa, wd, 1.0f / gd, out, partials, st));
    }
    return rc;
  }
  const MfmaWs L = mfma_ws(fmt, M, H, I);
  uint16_t* x16 = reinterpret_cast<uint16_t*>(base + L.x16);
  float* rs = reinterpret_cast<float*>(base + L.rs);
  uint16_t* act16 = reinterpret_cast<uint16_t*>(base + L.act16);
  // FP8: the gate/up stage stores act as float32 (no rounding between the projections, as the FP8
  // definition asks); the down stage makes its float16 operand with an exact power-of-two row scale and
  // takes the scale back out in its epilogue, so no act value can overflow.  NVFP4: act16 directly.
  float* act32 = fmt == WQ_FMT_FP8W ? reinterpret_cast<float*>(base + L.act32) : nullptr;
  float* ars = fmt == WQ_FMT_FP8W ? reinterpret_cast<float*>(base + L.ars) : nullptr;
  void* act_out = fmt == WQ_FMT_FP8W ? static_cast<void*>(act32) : static_cast<void*>(act16);
  float* partials = mlp_partials(fmt, M, H, I) ? reinterpret_cast<float*>(base + L.partials) : nullptr;
  const int f = fmt == WQ_FMT_NVFP4 ? 1 : 0;
  if (do_gu) {
    // FP8 with bf16 x: bf16 MFMAs on x as given; otherwise x is row-scaled to float16 first
    if (xt == wq::X_BF16 && wq::mfma_bf16_ok(f, h)) {
      rc = launched(wq::launch_mfma_gateup(f, m, h, i, reinterpret_cast<const uint16_t*>(x), nullptr, wg, sg, 0.f,
                                           wu, su, 0.f, act_out, partials, true, st));
    } else {
      rc = launched(wq::launch_rowscale_f16(m, h, x, xt, x16, rs, st));
      if (rc == WQ_OK)
        rc = launched(wq::launch_mfma_gateup(f, m, h, i, x16, rs, wg, sg, f ? 1.0f / gg : 0.f, wu, su,
                                             f ? 1.0f / gu : 0.f, act_out, partials, false, st));
    }
  }
  if (rc == WQ_OK && do_down) {
    if (fmt == WQ_FMT_FP8W) rc = launched(wq::launch_rowscale_f16(m, i, act32, wq::X_F32, act16, ars, st));
    if (rc == WQ_OK)
      rc = launched(wq::launch_mfma_linear(f, m, i, h, act16, ars, wd, sd, f ? 1.0f / gd : 0.f, out, partials,
                                           false, st));
  }
  return rc;
}

}  // namespace

extern "C" {

int wq_abi_version(void) { return WQ_ABI_VERSION; }

const char* wq_strerror(int rc) {
  switch (rc) {
    case WQ_OK: return "ok";
    case WQ_EINVAL: return "invalid argument (null pointer, shape, dtype, format or flags)";
    case WQ_EALIGN: return "pointer not 16-byte aligned";
    case WQ_EOVERLAP: return "output or workspace overlaps an input or another output";
    case WQ_EDEVICE: return "pointer is not device memory of the current device";
    case WQ_EARCH: return "current device is not gfx950";
    case WQ_EWORKSPACE: return "workspace missing or too small";
    case WQ_ELAUNCH: return "kernel launch failed";
    case WQ_ESCRATCH: return "call needs more scratch than the library's static scratch holds (WQ_STATIC_SCRATCH_BYTES)";
    default: return "unknown error";
  }
}

int wq_last_hip_error(void) { return g_last_hip; }

size_t mlp_workspace_bytes(int fmt, int64_t M, int64_t H, int64_t I, int flags) {
  if ((fmt != WQ_FMT_FP8W && fmt != WQ_FMT_NVFP4) || (flags & ~31) || (flags & 3) == 3) return 0;
  if ((flags & WQ_ACT_E4M3) && (flags & 3) == WQ_PATH_GEMV) return 0;
  return mlp_ws(fmt, M, H, I, flags & (3 | WQ_ACT_E4M3));
}

int mlp_fp8w_run(int64_t M, int64_t H, int64_t I, const void* x, int x_dtype, const uint8_t* w_gate,
                 const float* s_gate, const uint8_t* w_up, const float* s_up, const uint8_t* w_down,
                 const float* s_down, void* workspace, size_t workspace_bytes, float* out, int flags,
                 void* stream) {
  return mlp_run(WQ_FMT_FP8W, M, H, I, x, x_dtype, w_gate, s_gate, 0.f, w_up, s_up, 0.f, w_down, s_down, 0.f,
                 workspace, workspace_bytes, out, flags, stream);
}

int mlp_fp8w_run_noalloc(int64_t M, int64_t H, int64_t I, const void* x, int x_dtype, const uint8_t* w_gate,
                         const float* s_gate, const uint8_t* w_up, const float* s_up, const uint8_t* w_down,
                         const float* s_down, float* out, int flags, void* stream) {
  if (flags & ~3) return WQ_EINVAL;   // whole calls only: a stage split would hand act over in shared scratch
  return mlp_run(WQ_FMT_FP8W, M, H, I, x, x_dtype, w_gate, s_gate, 0.f, w_up, s_up, 0.f, w_down, s_down, 0.f,
                 nullptr, 0, out, flags, stream, true);
}

int mlp_nvfp4_run(int64_t M, int64_t H, int64_t I, const void* x, int x_dtype, const uint8_t* gate_blk,
                  float gate_global_scale, const uint8_t* up_blk, float up_global_scale, const uint8_t* down_blk,
                  float down_global_scale, void* workspace, size_t workspace_bytes, float* out, int flags,
                  void* stream) {
  return mlp_run(WQ_FMT_NVFP4, M, H, I, x, x_dtype, gate_blk, nullptr, gate_global_scale, up_blk, nullptr,
                 up_global_scale, down_blk, nullptr, down_global_scale, workspace, workspace_bytes, out, flags,
                 stream);
}

size_t awq_bank_bytes(int64_t E, int64_t N, int64_t K, int meta_layout) {
  if (E <= 0 || N <= 0 || K <= 0 || K % 32 || (meta_layout != 3 && meta_layout != 4)) return 0;
  if (E > kMaxDim || N > kMaxDim || K > kMaxDim) return 0;
  return (size_t)E * (size_t)wq::awq_layout(N, K, meta_layout).expert_bytes;
}

int moe_awq_m1_run(int64_t E, int64_t topk, int64_t H, int64_t I, const uint16_t* x, const int32_t* expert_ids,
                   const float* router_w, const void* w13_bank, const void* w2_bank, int meta_layout,
                   uint16_t* act, uint16_t* out, void* stream) {
  if (E <= 0 || E > kMaxDim || topk < 1 || topk > WQ_MOE_MAX_TOPK) return WQ_EINVAL;
  if (H <= 0 || I <= 0 || H % 32 || I % 32 || H > 16384 || I > 16384) return WQ_EINVAL;
  if (meta_layout != 3 && meta_layout != 4) return WQ_EINVAL;
  // LDS of the two kernels: x groups (H/32 * 80 B); act groups + route results.
  if ((H / 32) * 80 > 65536 || topk * ((I / 32) * 80 + 128) > 65536) return WQ_EINVAL;
  if (any_null({x, expert_ids, router_w, w13_bank, w2_bank, act, out})) return WQ_EINVAL;
  if (!all_aligned({x, expert_ids, router_w, w13_bank, w2_bank, act, out})) return WQ_EALIGN;
  const size_t b13 = awq_bank_bytes(E, 2 * I, H, meta_layout), b2 = awq_bank_bytes(E, H, I, meta_layout);
  if (any_overlap({{act, (size_t)topk * I * 2}, {out, (size_t)H * 2}},
                  {{x, (size_t)H * 2}, {expert_ids, (size_t)topk * 4}, {router_w, (size_t)topk * 4},
                   {w13_bank, b13}, {w2_bank, b2}}))
    return WQ_EOVERLAP;
  int rc = check_device({x, expert_ids, router_w, w13_bank, w2_bank, act, out});
  if (rc != WQ_OK) return rc;
  return launched(wq::launch_moe_awq_m1((int)E, (int)topk, (int)H, (int)I, x, expert_ids, router_w,
                                        reinterpret_cast<const uint8_t*>(w13_bank),
                                        reinterpret_cast<const uint8_t*>(w2_bank), meta_layout, act, out,
                                        reinterpret_cast<hipStream_t>(stream)));
}

int nvfp4_pack_block64(int64_t N, int64_t K, const uint8_t* weight_packed, const uint8_t* weight_scale,
                       uint8_t* blk, void* stream) {
  if (N <= 0 || K <= 0 || K % 64 || N > kMaxDim || K > kMaxDim) return WQ_EINVAL;
  if (any_null({weight_packed, weight_scale, blk})) return WQ_EINVAL;
  if (any_overlap({{blk, wbytes(WQ_FMT_NVFP4, N, K)}},
                  {{weight_packed, (size_t)N * K / 2}, {weight_scale, (size_t)N * K / 16}}))
    return WQ_EOVERLAP;
  int rc = check_device({weight_packed, weight_scale, blk});
  if (rc != WQ_OK) return rc;
  return launched(wq::launch_nvfp4_pack(N, K, weight_packed, weight_scale, blk, reinterpret_cast<hipStream_t>(stream)));
}

int awq_pack_bank(int64_t E, int64_t N, int64_t K, const uint8_t* codes, const uint16_t* scales,
                  const uint8_t* zeros, int meta_layout, void* bank, void* stream) {
  const size_t nb = awq_bank_bytes(E, N, K, meta_layout);
  if (nb == 0) return WQ_EINVAL;
  if (any_null({codes, scales, zeros, bank})) return WQ_EINVAL;
  if (!all_aligned({bank})) return WQ_EALIGN;
  const size_t ng = (size_t)E * N * (K / 32);
  if (any_overlap({{bank, nb}}, {{codes, (size_t)E * N * K}, {scales, ng * 2}, {zeros, ng}})) return WQ_EOVERLAP;
  int rc = check_device({codes, scales, zeros, bank});
  if (rc != WQ_OK) return rc;
  return launched(wq::launch_awq_pack(E, N, K, codes, scales, zeros, meta_layout, reinterpret_cast<uint8_t*>(bank),
                                      reinterpret_cast<hipStream_t>(stream)));
}

int fp8w_dequant_f32(int64_t N, int64_t K, const uint8_t* w, const float* s, float* out, void* stream) {
  if (N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim) return WQ_EINVAL;
  if (any_null({w, s, out})) return WQ_EINVAL;
  if (any_overlap({{out, (size_t)N * K * 4}}, {{w, (size_t)N * K}, {s, (size_t)N * 4}})) return WQ_EOVERLAP;
  int rc = check_device({w, s, out});
  if (rc != WQ_OK) return rc;
  return launched(wq::launch_fp8w_dequant(N, K, w, s, out, reinterpret_cast<hipStream_t>(stream)));
}

int nvfp4_dequant_f32(int64_t N, int64_t K, const uint8_t* blk, float global_scale, float* out, void* stream) {
  if (N <= 0 || K <= 0 || K % 64 || N > kMaxDim || K > kMaxDim) return WQ_EINVAL;
  if (!(global_scale > 0.f) || !std::isfinite(global_scale)) return WQ_EINVAL;
  if (any_null({blk, out})) return WQ_EINVAL;
  if (any_overlap({{out, (size_t)N * K * 4}}, {{blk, wbytes(WQ_FMT_NVFP4, N, K)}})) return WQ_EOVERLAP;
  int rc = check_device({blk, out});
  if (rc != WQ_OK) return rc;
  return launched(wq::launch_nvfp4_dequant(N, K, blk, 1.0f / global_scale, out, reinterpret_cast<hipStream_t>(stream)));
}

int awq_dequant_f16(int64_t E, int64_t N, int64_t K, const void* bank, int meta_layout, uint16_t* out,
                    void* stream) {
  const size_t nb = awq_bank_bytes(E, N, K, meta_layout);
  if (nb == 0) return WQ_EINVAL;
  if (any_null({bank, out})) return WQ_EINVAL;
  if (!all_aligned({bank})) return WQ_EALIGN;
  if (any_overlap({{out, (size_t)E * N * K * 2}}, {{bank, nb}})) return WQ_EOVERLAP;
  int rc = check_device({bank, out});
  if (rc != WQ_OK) return rc;
  return launched(wq::launch_awq_dequant(E, N, K, reinterpret_cast<const uint8_t*>(bank), meta_layout, out,
                                         reinterpret_cast<hipStream_t>(stream)));
}

int wq_read_probe(const void* src, size_t bytes, uint32_t* sink, int grid, void* stream) {
  if (src == nullptr || sink == nullptr || bytes == 0 || bytes % 16 || grid < 1 || grid > (1 << 20)) return WQ_EINVAL;
  if (!all_aligned({src, sink})) return WQ_EALIGN;
  if (any_overlap({{sink, (size_t)grid * 4}}, {{src, bytes}})) return WQ_EOVERLAP;
  const int rc = check_device({src, sink});
  if (rc != WQ_OK) return rc;
  return launched(wq::launch_read_probe(src, bytes, sink, grid, reinterpret_cast<hipStream_t>(stream)));
}

size_t qlinear_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, int flags) {
  if ((fmt != WQ_FMT_FP8W && fmt != WQ_FMT_NVFP4) || (flags & ~(3 | WQ_ACT_E4M3)) || (flags & 3) == 3) return 0;
  if (M <= 0 || N <= 0 || K <= 0 || M > kMaxDim || N > kMaxDim || K > kMaxDim || !elems_ok(M, N, K)) return 0;
  if (flags & WQ_ACT_E4M3) {
    if (fmt != WQ_FMT_NVFP4 || (flags & 3) == WQ_PATH_GEMV || !w8_k_ok(K)) return 0;
    return align256((size_t)M * K * 2) + align256((size_t)M * 4) + align256(wq::w4a8_partial_bytes((int)M, (int)K, (int)N, false));
  }
  if (linear_path(fmt, M, N, K, flags) == WQ_PATH_GEMV) return 0;
  return align256((size_t)M * K * 2) + align256((size_t)M * 4) +
         align256(wq::mfma_partial_bytes(fmt == WQ_FMT_NVFP4 ? 1 : 0, (int)M, (int)K, (int)N, false));
}

int qlinear_run(int fmt, int64_t M, int64_t N, int64_t K, const void* x, int x_dtype, const uint8_t* w,
                const float* scale, float global_scale, void* workspace, size_t workspace_bytes, float* y, int flags,
                void* stream) {
  if (fmt != WQ_FMT_FP8W && fmt != WQ_FMT_NVFP4) return WQ_EINVAL;
  if ((flags & ~(3 | WQ_ACT_E4M3)) || (flags & 3) == 3) return WQ_EINVAL;
  const bool w8 = (flags & WQ_ACT_E4M3) != 0;   // W4A8: NVFP4 only, MFMA path only, float32 or bf16 x
  if (w8 && (fmt != WQ_FMT_NVFP4 || (flags & 3) == WQ_PATH_GEMV || x_dtype == WQ_F16)) return WQ_EINVAL;
  if (x_dtype != WQ_F32 && x_dtype != WQ_BF16 && x_dtype != WQ_F16) return WQ_EINVAL;
  // float16 x: the operand type of the NVFP4 MLP's GEMV down projection; NVFP4 on the GEMV path only
  if (x_dtype == WQ_F16 && (fmt != WQ_FMT_NVFP4 || (flags & 3) == WQ_PATH_MFMA)) return WQ_EINVAL;
  if (M < 0 || M > kMaxDim || N <= 0 || K <= 0 || N > kMaxDim || K > kMaxDim || !elems_ok(M, N, K)) return WQ_EINVAL;
  const int path = x_dtype == WQ_F16 ? WQ_PATH_GEMV : linear_path(fmt, M, N, K, flags);
  // K runs along the records (NVFP4), the 64-wide MFMA K steps and the 16-byte FP8 chunks; N (output
  // rows) is free: every kernel clamps its row loads to N-1 and guards its stores
  if (path == WQ_PATH_MFMA || fmt == WQ_FMT_NVFP4) {
    if (K % 64) return WQ_EINVAL;
  } else if (K % 16) {
    return WQ_EINVAL;
  }
  if (path == WQ_PATH_GEMV && !gemv_fits(fmt, K, x_dtype)) return WQ_EINVAL;
  if (w8 && !w8_k_ok(K)) return WQ_EINVAL;
  if (w == nullptr) return WQ_EINVAL;
  if (fmt == WQ_FMT_FP8W && scale == nullptr) return WQ_EINVAL;
  if (fmt == WQ_FMT_NVFP4 && (!(global_scale > 0.f) || !std::isfinite(global_scale))) return WQ_EINVAL;
  if (M == 0) return WQ_OK;   // nothing to do: x, y and the workspace may be null
  if (any_null({x, y})) return WQ_EINVAL;
  if (!all_aligned({x, w, y, scale, workspace})) return WQ_EALIGN;
  const size_t need = path == WQ_PATH_GEMV ? 0 : qlinear_workspace_bytes(fmt, M, N, K, flags);
  if (need && (workspace == nullptr || workspace_bytes < need)) return WQ_EWORKSPACE;
  const size_t ns = fmt == WQ_FMT_FP8W ? (size_t)N * 4 : 0;
  if (any_overlap({{y, (size_t)M * N * 4}, {workspace, need}},
                  {{x, (size_t)M * K * xsize(x_dtype)}, {w, wbytes(fmt, N, K)}, {scale, ns}}))
    return WQ_EOVERLAP;
  int rc = check_device({x, w, scale, need ? workspace : nullptr, y});
  if (rc != WQ_OK) return rc;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const wq::XType xt = x_dtype == WQ_BF16 ? wq::X_BF16 : (x_dtype == WQ_F16 ? wq::X_F16 : wq::X_F32);
  const float inv = fmt == WQ_FMT_NVFP4 ? 1.0f / global_scale : 0.f;
  if (path == WQ_PATH_GEMV) {
    if (fmt == WQ_FMT_FP8W)
      return launched(wq::launch_fp8w_gemv((int)M, (int)K, (int)N, x, xt, w, scale, nullptr, nullptr, y, st));
    return launched(wq::launch_nvfp4_gemv((int)M, (int)K, (int)N, x, xt, w, inv, nullptr, 0.f, y, false, st));
  }
  uint8_t* base = reinterpret_cast<uint8_t*>(workspace);
  if (w8) {   // workspace: xq [M,K] float16 (E4M3 values), sx [M], partials
    uint16_t* xq = reinterpret_cast<uint16_t*>(base);
    float* sx = reinterpret_cast<float*>(base + align256((size_t)M * K * 2));
    float* partials = wq::w4a8_partial_bytes((int)M, (int)K, (int)N, false)
                          ? reinterpret_cast<float*>(base + align256((size_t)M * K * 2) + align256((size_t)M * 4))
                          : nullptr;
    rc = launched(wq::launch_quant_e4m3((int)M, (int)K, x, xt, xq, sx, st));
    if (rc == WQ_OK) rc = launched(wq::launch_w4a8_linear((int)M, (int)K, (int)N, xq, sx, w, inv, y, partials, st));
    return rc;
  }
  uint16_t* x16 = reinterpret_cast<uint16_t*>(base);
  float* rs = reinterpret_cast<float*>(base + align256((size_t)M * K * 2));
  const int f = fmt == WQ_FMT_NVFP4 ? 1 : 0;
  float* partials = wq::mfma_partial_bytes(f, (int)M, (int)K, (int)N, false)
                        ? reinterpret_cast<float*>(base + align256((size_t)M * K * 2) + align256((size_t)M * 4))
                        : nullptr;
  if (xt == wq::X_BF16 && wq::mfma_bf16_ok(f, (int)K))   // FP8 with bf16 x: bf16 MFMAs on x as given
    return launched(wq::launch_mfma_linear(f, (int)M, (int)K, (int)N, reinterpret_cast<const uint16_t*>(x), nullptr,
                                           w, scale, inv, y, partials, true, st));
  rc = launched(wq::launch_rowscale_f16((int)M, (int)K, x, xt, x16, rs, st));
  if (rc == WQ_OK)
    rc = launched(wq::launch_mfma_linear(f, (int)M, (int)K, (int)N, x16, rs, w, scale, inv, y, partials, false, st));
  return rc;
}

}  // extern "C"
