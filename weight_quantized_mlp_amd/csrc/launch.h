// Host-side launchers of the gfx950 kernels (internal to the library).
// Argument checking happens in abi.cpp before any of these is called; the
// launchers only compute launch shapes and enqueue.  Each returns the
// hipError_t of the launch (hipGetLastError after the enqueue).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace wq {

// Raise kernel KERN's dynamic-LDS limit to what the 160 KB of a gfx950 CU leaves beside its static LDS
// (needed above 64 KB), once per device (the attribute is per kernel and device; devices are tracked as
// bits, 256 at most).
template <auto KERN>
inline bool raise_lds_limit() {
  static std::atomic<uint64_t> done[4];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 256) return false;
  const uint64_t bit = (uint64_t)1 << (dev & 63);
  std::atomic<uint64_t>& word = done[dev >> 6];
  if (word.load(std::memory_order_acquire) & bit) return true;
  hipFuncAttributes attr;
  if (hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(KERN)) != hipSuccess) return false;
  const int dyn = 160 * 1024 - (int)attr.sharedSizeBytes;   // static LDS of the kernel counts against the CU's
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(KERN), hipFuncAttributeMaxDynamicSharedMemorySize, dyn) !=
      hipSuccess)
    return false;
  word.fetch_or(bit, std::memory_order_release);
  return true;
}

enum XType { X_F32 = 0, X_BF16 = 1, X_F16 = 2 };

// ---- M < 128: split-K GEMV family -------------------------------------------------------------
// FP8: y[m,n] = s0[n] * sum_k x[m,k] e4m3(w0[n,k]); with w1/s1 (gate+up) y = silu(g)*u.
hipError_t launch_fp8w_gemv(int M, int K, int N, const void* x, XType xt,
                            const uint8_t* w0, const float* s0, const uint8_t* w1, const float* s1,
                            float* y, hipStream_t st);
// NVFP4 Block64: same with the per-tensor factors inv0 = 1/gs0, inv1 = 1/gs1.  x: X_F32, X_BF16, or
// (single matrix only) X_F16.  y16 (gate+up only): y is float16 [M, N] (the NVFP4 MLP's act), else
// float32.
hipError_t launch_nvfp4_gemv(int M, int K, int N, const void* x, XType xt,
                             const uint8_t* b0, float inv0, const uint8_t* b1, float inv1,
                             void* y, bool y16, hipStream_t st);

// Main M < 128 kernels (gemv_fast.hip); the *_ok predicates say whether a shape is covered.
// For a given shape the same family serves every M < 128, so row results do not depend on M.
bool fast_gemv_fp8_ok(int K, XType xt, bool gu);
bool fast_gemv_nvfp4_ok(int K, XType xt, bool gu);
hipError_t launch_fast_fp8(int M, int K, int N, const void* x, XType xt, const uint8_t* w0, const float* s0,
                           const uint8_t* w1, const float* s1, float* y, hipStream_t st);
hipError_t launch_fast_nvfp4(int M, int K, int N, const void* x, XType xt, const uint8_t* b0, float inv0,
                             const uint8_t* b1, float inv1, void* y, bool y16, hipStream_t st);

// ---- M >= 128: MFMA GEMM family ---------------------------------------------------------------
// x [M,K] (f32 or bf16) -> x16 [M,K] f16 scaled per row by 2^-e, rowscale[m] = 2^e, where max_k |x[m,k]| * 2^-e
// lies in [2^14, 2^15); every K that is a multiple of 64.
hipError_t launch_rowscale_f16(int M, int K, const void* x, XType xt, uint16_t* x16, float* rowscale,
                               hipStream_t st);
// fmt 0 FP8 (w = [N,K] codes, colscale[n]) / 1 NVFP4 (w = Block64, uniform inv).
// gate+up: act[m,n] = silu(g) * u with g = rowscale[m]*colscale(n)*acc, stored as float32 (FP8) or rounded to
// float16 (NVFP4).
// partials: float32 scratch of mfma_partial_bytes(fmt, M, K, N, gu) bytes (NULL allowed when that is 0);
// the NVFP4 GEMM splits the tiles of an underfilled last round along K and finishes them from there.
// abf: the activations are bfloat16 bits as given (rowscale must be null) and the GEMM runs bf16 MFMAs;
// only where mfma_bf16_ok(fmt, K) (FP8 weights, K >= 128), else hipErrorInvalidValue.
size_t mfma_partial_bytes(int fmt, int M, int K, int N, bool gu);
bool mfma_bf16_ok(int fmt, int K);
hipError_t launch_mfma_gateup(int fmt, int M, int K, int N, const uint16_t* x16, const float* rowscale,
                              const uint8_t* w0, const float* cs0, float inv0,
                              const uint8_t* w1, const float* cs1, float inv1,
                              void* act, float* partials, bool abf, hipStream_t st);
// single matrix: y[m,n] = rowscale[m] (1 if null) * colscale(n) * sum_k a16[m,k] dq(w[n,k]).
hipError_t launch_mfma_linear(int fmt, int M, int K, int N, const uint16_t* a16, const float* rowscale,
                              const uint8_t* w, const float* cs, float inv, float* y, float* partials, bool abf,
                              hipStream_t st);

// ---- W4A8: NVFP4 weights x per-token E4M3 activations (MFMA) --------------------------------------
// x [M,K] (f32 or bf16) -> q [M,K] float16 holding the E4M3 values of x[m,k] * 2^-e (round to nearest
// even), rowscale[m] = 2^e with max_k |x[m,k]| * 2^-e in (224, 448]; K a multiple of 8.
hipError_t launch_quant_e4m3(int M, int K, const void* x, XType xt, uint16_t* q, float* rowscale, hipStream_t st);
// GEMMs on those values and Block64 weights (the float16 path's GEMM; K a multiple of 64, at least 256):
// gate+up writes act = silu(g) * u as float32 [M,N] with g = rowscale[m] * inv0 * acc; the single matrix
// writes y [M,N].  partials: float32 scratch of w4a8_partial_bytes(M, K, N, gu) bytes (NULL allowed when
// that is 0).
size_t w4a8_partial_bytes(int M, int K, int N, bool gu);
hipError_t launch_w4a8_gateup(int M, int K, int N, const uint16_t* xq, const float* sx, const uint8_t* w0, float inv0,
                              const uint8_t* w1, float inv1, float* act, float* partials, hipStream_t st);
hipError_t launch_w4a8_linear(int M, int K, int N, const uint16_t* aq, const float* sa, const uint8_t* w, float inv,
                              float* y, float* partials, hipStream_t st);

// ---- AWQ routed-expert single-token step ------------------------------------------------------
hipError_t launch_moe_awq_m1(int E, int topk, int H, int I, const uint16_t* x, const int32_t* ids,
                             const float* router_w, const uint8_t* w13, const uint8_t* w2, int meta_layout,
                             uint16_t* act, uint16_t* out, hipStream_t st);

// ---- packers and debug decoders -------------------------------------------------------------
hipError_t launch_nvfp4_pack(int64_t N, int64_t K, const uint8_t* wp, const uint8_t* ws, uint8_t* blk,
                             hipStream_t st);
hipError_t launch_awq_pack(int64_t E, int64_t N, int64_t K, const uint8_t* codes, const uint16_t* scales,
                           const uint8_t* zeros, int meta_layout, uint8_t* bank, hipStream_t st);
hipError_t launch_fp8w_dequant(int64_t N, int64_t K, const uint8_t* w, const float* s, float* out,
                               hipStream_t st);
hipError_t launch_nvfp4_dequant(int64_t N, int64_t K, const uint8_t* blk, float inv, float* out,
                                hipStream_t st);
hipError_t launch_awq_dequant(int64_t E, int64_t N, int64_t K, const uint8_t* bank, int meta_layout,
                              uint16_t* out, hipStream_t st);

// ---- measurement helper ---------------------------------------------------------------------
// Streaming read of `bytes` (a multiple of 16) at src by `grid` workgroups of 256 threads; sink holds
// grid 32-bit words (written only when a lane's XOR fold equals one fixed value).
hipError_t launch_read_probe(const void* src, size_t bytes, uint32_t* sink, int grid, hipStream_t st);

// ---- AWQ bank geometry (shared by the packer, the decoder and the step) ------------------------
struct AwqLayout {
  int64_t G;           // groups of 32 per row
  int64_t scale_off;   // byte offset of the f16 scale plane inside an expert
  int64_t meta2_off;   // byte offset of the zero (u8) or bias (f16) plane
  int64_t expert_bytes;
};
inline AwqLayout awq_layout(int64_t N, int64_t K, int meta_layout) {
  auto r16 = [](int64_t v) { return (v + 15) / 16 * 16; };
  AwqLayout L;
  L.G = K / 32;
  L.scale_off = r16(N * K / 2);
  L.meta2_off = L.scale_off + r16(2 * N * L.G);
  L.expert_bytes = L.meta2_off + r16((meta_layout == 3 ? 1 : 2) * N * L.G);
  return L;
}

}  // namespace wq
