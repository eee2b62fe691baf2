// M >= 128 path: LDS-tiled MFMA GEMMs with in-kernel weight decode (gfx950).
//
// Method: issue "tp>1 fp8w tail-MLP shard host-dequantizes every layer", section
// "Proposed fix" (SwiGLU MLP); NVFP4 numerics and the 36-byte record from page
// "Qwen3.8-27B-NVFP4", section "NVFP4 numerics as implemented".  That page's
// prefill tile ("Implemented execution path", "Wide-N64 prefill tile") reuses one
// activation tile across many output rows and one decoded weight tile across many
// activation rows; the same reuse is built here around CDNA4 matrix cores.
//
// Numerics of this path (a dense contraction, run as float16 MFMA with float32
// accumulation):
//   * x rows are scaled by a power of two 2^-e_m (max |x| in [2^14, 2^15)) and
//     rounded to float16 once (exact for bf16 input above 2^-29 of the row max);
//   * weights are decoded exactly into float16: E2M1 * E4M3 group scale has at most
//     6 significant bits (the K=16 rescale is folded into every decoded weight), and
//     every E4M3 value is a float16;
//   * gate/up: acc * 2^e_m * (1/global_scale or channel scale), act = silu(g) * u in
//     float32, rounded once to float16 for the down GEMM (|act| < 65504 required);
//   * down: acc * (1/global_scale or channel scale), stored as float32.
//
// Tiling: a workgroup of 4 waves computes a (32*MB) x 128 output tile (of both gate
// and up for the fused kernel).  All waves share the activation tile, staged in LDS
// (rows padded to 144 bytes: conflict-free 16-byte fragment reads); each wave owns
// 32 output columns and decodes its own weight fragments straight from global memory
// into registers, so every decoded fragment feeds MB (x2 with gate+up) MFMAs.  K is
// walked in steps of 64 (one Block64 record) with the next step's loads in flight.
//
// MFMA v_mfma_f32_32x32x16_f16 operand layout (checked on gfx950): A lane l holds row
// l%32, k = 8*(l/32) + j; B lane l holds column l%32, same k; D register r of lane l
// is (row 8*(r/4) + 4*(l/32) + r%4, column l%32).  Within a 64-wide K step, step s
// (0..3) feeds the instruction k' = 8*(l/32) + j with the logical k = 32*(l/32) +
// 8*s + j, for both operands, so each lane's weight bytes for a whole record are one
// contiguous 16-byte (NVFP4) or 32-byte (FP8) load.
#include "dev_common.h"
#include "launch.h"

namespace wq {

namespace {

constexpr int kLdsRow = 144;  // 64 f16 + 16 bytes padding

__device__ __forceinline__ u32x4 ld16(const uint8_t* p) {
  u32x4 v;
  __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 16);
  return v;
}

// ---- x -> float16 with a per-row power-of-two scale -------------------------------------------
template <typename XT>
__device__ __forceinline__ float to_f32(XT v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<uint16_t>(uint16_t v) { return bf16_bits_to_f32(v); }

template <typename XT>
__global__ void __launch_bounds__(256) rowscale_f16_kernel(int K, const XT* __restrict__ x,
                                                           uint16_t* __restrict__ x16,
                                                           float* __restrict__ rowscale) {
  __shared__ float red[4];
  const size_t m = blockIdx.x;
  const XT* xr = x + m * K;
  float amax = 0.f;
  for (int k = threadIdx.x; k < K; k += 256) amax = fmaxf(amax, fabsf(to_f32<XT>(xr[k])));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int e = 0;
  if (amax > 0.f && amax <= 3.0e38f) {
    int ex;
    (void)frexpf(amax, &ex);   // amax = f * 2^ex, f in [0.5, 1)
    e = ex - 15;                // amax * 2^-e in [2^14, 2^15)
    e = e < -100 ? -100 : (e > 100 ? 100 : e);
  }
  if (threadIdx.x == 0) rowscale[m] = ldexpf(1.0f, e);
  uint16_t* o = x16 + m * K;
  for (int k = threadIdx.x; k < K; k += 256) {
    const _Float16 h = (_Float16)ldexpf(to_f32<XT>(xr[k]), -e);
    o[k] = __builtin_bit_cast(uint16_t, h);
  }
}

// ---- the GEMM ------------------------------------------------------------------------------------
// FMT 0: FP8 E4M3 codes [N][K], per-column scale cs[n].  FMT 1: NVFP4 Block64 [N][K/64], factor inv.
// GU: two weight matrices, out = f16 act [M][N]; else one matrix, out = f32 y [M][N].
template <int FMT, bool GU, int MB>
__global__ void __launch_bounds__(256, 2) mfma_gemm_kernel(int M, int K, int N, int ntm, int ntn,
                                                          const uint16_t* __restrict__ a16,
                                                          const float* __restrict__ rowscale,
                                                          const uint8_t* __restrict__ w0,
                                                          const float* __restrict__ cs0, float inv0,
                                                          const uint8_t* __restrict__ w1,
                                                          const float* __restrict__ cs1, float inv1,
                                                          void* __restrict__ out) {
  constexpr int NM = GU ? 2 : 1;
  constexpr int BM = 32 * MB;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][BM * kLdsRow];

  // XCD-aware tile order: workgroup b runs on XCD b % 8; give each XCD a contiguous
  // run of tiles (n fastest) so the activation band it works on stays in its L2.
  const int per = gridDim.x >> 3;
  const int tile = (int)(blockIdx.x & 7) * per + (int)(blockIdx.x >> 3);
  if (tile >= ntm * ntn) return;
  const int tm = tile / ntn;
  const int tn = tile - tm * ntn;
  const int m0 = tm * BM;
  const int n0 = tn * 128;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;
  const int h = lane >> 5;
  const int ncol = n0 + 32 * wave + li;  // this lane's output column / weight row
  const bool wave_on = n0 + 32 * wave < N;
  const int nk = K >> 6;

  const uint8_t* wrow[NM];
  {
    const size_t rb = FMT == 1 ? (size_t)(K >> 6) * 36 : (size_t)K;
    wrow[0] = w0 + (size_t)(wave_on ? ncol : 0) * rb;
    if constexpr (GU) wrow[1] = w1 + (size_t)(wave_on ? ncol : 0) * rb;
  }

  f32x16 acc[NM][MB];
#pragma unroll
  for (int t = 0; t < NM; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][mb][r] = 0.f;

  // Activation tile pieces: BM rows x 8 pieces of 16 bytes; MB pieces per thread.
  u32x4 apre[MB];
  auto load_a = [&](int kt) {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int p = tid + 256 * i;
      const int row = p >> 3;
      const int cp = p & 7;
      const int m = m0 + row;
      u32x4 v = {0u, 0u, 0u, 0u};
      if (m < M) v = *reinterpret_cast<const u32x4*>(a16 + (size_t)m * K + (size_t)kt * 64 + cp * 8);
      apre[i] = v;
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int i = 0; i < MB; ++i) {
      const int p = tid + 256 * i;
      *reinterpret_cast<u32x4*>(&lds[buf][(p >> 3) * kLdsRow + (p & 7) * 16]) = apre[i];
    }
  };

  // Weight bytes of this lane for one K step.
  struct WRegs {
    u32x4 q0, q1;  // NVFP4: q0 = 16 qs bytes (32 nibbles); FP8: q0, q1 = 32 codes
    uint32_t d;    // NVFP4 record scales d[0..3]
  };
  WRegs wcur[NM], wnxt[NM];
  auto load_w = [&](int kt, WRegs* wr) {
    if (!wave_on) return;
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      if constexpr (FMT == 1) {
        const uint8_t* rec = wrow[t] + (size_t)kt * 36;
        wr[t].d = *reinterpret_cast<const uint32_t*>(rec);
        wr[t].q0 = ld16(rec + 4 + 16 * h);
      } else {
        const uint8_t* p = wrow[t] + (size_t)kt * 64 + 32 * h;
        wr[t].q0 = *reinterpret_cast<const u32x4*>(p);
        wr[t].q1 = *reinterpret_cast<const u32x4*>(p + 16);
      }
    }
  };

  auto compute = [&](int buf, const WRegs* wr) {
    f16x2 dsc[NM];
    if constexpr (FMT == 1) {
#pragma unroll
      for (int t = 0; t < NM; ++t) dsc[t] = e4m3x2_f16<false>(wr[t].d >> (16 * h));  // groups 2h, 2h+1
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      f16x8 bfr[NM];
#pragma unroll
      for (int t = 0; t < NM; ++t) {
        f16x2 p0, p1, p2, p3;
        if constexpr (FMT == 1) {
          const uint32_t w = wr[t].q0[s];
          const _Float16 g = (s < 2) ? dsc[t].x : dsc[t].y;
          const f16x2 gg = {g, g};
          p0 = e2m1x2_f16<0>(w) * gg;
          p1 = e2m1x2_f16<1>(w) * gg;
          p2 = e2m1x2_f16<2>(w) * gg;
          p3 = e2m1x2_f16<3>(w) * gg;
        } else {
          const uint32_t wa = s < 2 ? wr[t].q0[2 * s] : wr[t].q1[2 * s - 4];
          const uint32_t wb = s < 2 ? wr[t].q0[2 * s + 1] : wr[t].q1[2 * s - 3];
          p0 = e4m3x2_f16<false>(wa);
          p1 = e4m3x2_f16<true>(wa);
          p2 = e4m3x2_f16<false>(wb);
          p3 = e4m3x2_f16<true>(wb);
        }
        bfr[t] = f16x8{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const f16x8 afr =
            *reinterpret_cast<const f16x8*>(&lds[buf][(32 * mb + li) * kLdsRow + (32 * h + 8 * s) * 2]);
#pragma unroll
        for (int t = 0; t < NM; ++t)
          acc[t][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(afr, bfr[t], acc[t][mb], 0, 0, 0);
      }
    }
  };

  load_a(0);
  load_w(0, wcur);
  store_a(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      load_a(kt + 1);
      load_w(kt + 1, wnxt);
    }
    if (wave_on) compute(cur, wcur);
    if (more) {
      store_a(cur ^ 1);
#pragma unroll
      for (int t = 0; t < NM; ++t) wcur[t] = wnxt[t];
    }
    __syncthreads();
  }

  if (!wave_on) return;
  float cf[NM];
#pragma unroll
  for (int t = 0; t < NM; ++t) {
    if constexpr (FMT == 1) cf[t] = t == 0 ? inv0 : inv1;
    else cf[t] = (t == 0 ? cs0 : cs1)[ncol];
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
      if (m < M) {
        const float rs = rowscale ? rowscale[m] : 1.0f;
        if constexpr (GU) {
          const float g = acc[0][mb][r] * rs * cf[0];
          const float u = acc[1][mb][r] * rs * cf[1];
          const _Float16 a = (_Float16)(silu_f32(g) * u);
          reinterpret_cast<uint16_t*>(out)[(size_t)m * N + ncol] = __builtin_bit_cast(uint16_t, a);
        } else {
          reinterpret_cast<float*>(out)[(size_t)m * N + ncol] = acc[0][mb][r] * rs * cf[0];
        }
      }
    }
  }
}

template <int FMT, bool GU>
hipError_t gemm_dispatch(int M, int K, int N, const uint16_t* a16, const float* rowscale, const uint8_t* w0,
                         const float* cs0, float inv0, const uint8_t* w1, const float* cs1, float inv1, void* out,
                         hipStream_t st) {
  const int ntn = (N + 127) / 128;
  // Fewer than ~2 tiles per CU with 128-row tiles: use 64-row tiles.
  const bool small = (long)((M + 127) / 128) * ntn < 512;
  const int BM = small ? 64 : 128;
  const int ntm = (M + BM - 1) / BM;
  const int ntiles = ntm * ntn;
  const int grid = (ntiles + 7) / 8 * 8;
  if (small)
    hipLaunchKernelGGL((mfma_gemm_kernel<FMT, GU, 2>), dim3(grid), dim3(256), 0, st, M, K, N, ntm, ntn, a16,
                       rowscale, w0, cs0, inv0, w1, cs1, inv1, out);
  else
    hipLaunchKernelGGL((mfma_gemm_kernel<FMT, GU, 4>), dim3(grid), dim3(256), 0, st, M, K, N, ntm, ntn, a16,
                       rowscale, w0, cs0, inv0, w1, cs1, inv1, out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rowscale_f16(int M, int K, const void* x, XType xt, uint16_t* x16, float* rowscale,
                               hipStream_t st) {
  if (xt == X_BF16)
    hipLaunchKernelGGL(rowscale_f16_kernel<uint16_t>, dim3(M), dim3(256), 0, st, K,
                       reinterpret_cast<const uint16_t*>(x), x16, rowscale);
  else
    hipLaunchKernelGGL(rowscale_f16_kernel<float>, dim3(M), dim3(256), 0, st, K,
                       reinterpret_cast<const float*>(x), x16, rowscale);
  return hipGetLastError();
}

hipError_t launch_mfma_gateup(int fmt, int M, int K, int N, const uint16_t* x16, const float* rowscale,
                              const uint8_t* w0, const float* cs0, float inv0, const uint8_t* w1,
                              const float* cs1, float inv1, uint16_t* act16, hipStream_t st) {
  if (fmt == 1)
    return gemm_dispatch<1, true>(M, K, N, x16, rowscale, w0, cs0, inv0, w1, cs1, inv1, act16, st);
  return gemm_dispatch<0, true>(M, K, N, x16, rowscale, w0, cs0, inv0, w1, cs1, inv1, act16, st);
}

hipError_t launch_mfma_linear(int fmt, int M, int K, int N, const uint16_t* a16, const float* rowscale,
                              const uint8_t* w, const float* cs, float inv, float* y, hipStream_t st) {
  if (fmt == 1) return gemm_dispatch<1, false>(M, K, N, a16, rowscale, w, cs, inv, nullptr, nullptr, 0.f, y, st);
  return gemm_dispatch<0, false>(M, K, N, a16, rowscale, w, cs, inv, nullptr, nullptr, 0.f, y, st);
}

}  // namespace wq
