// M < 128 path, general kernels: split-K GEMVs for FP8 E4M3 per-channel and NVFP4
// Block64 weights, with an optional fused SwiGLU epilogue (gate + up share one
// activation load).  They serve the shapes the main kernels in gemv_fast.hip do not
// cover (float32 activations into gate+up, very long rows).
//
// Method: issue "tp>1 fp8w tail-MLP shard host-dequantizes every layer", section
// "Proposed fix" (the MLP equation); FP8 decode from section "Mechanism on the tp>1
// path"; NVFP4 decode and the 36-byte record from page "Qwen3.8-27B-NVFP4", section
// "NVFP4 numerics as implemented" (group scale re-applied at every K=16 boundary,
// as that page's "Implemented execution path" describes for its decode kernel).
//
// Data flow per workgroup: the activation rows are staged once into LDS (padded
// chunks, conflict-free 16-byte reads); every wave then streams its own contiguous
// range of weight rows with coalesced 16-byte global loads, decodes them in
// registers and accumulates in float32.  Loads of the next step are issued before
// the current step is computed (register double buffering).
//
// Fixed accumulation order (independent of M, so row m of an M-row call is bitwise
// equal to a 1-row call):
//   FP8:   lane l owns 16-byte chunks c = l, l+64, ... of the row (ascending); each
//          chunk's 16 products go into two partial sums (even / odd 4-k quads,
//          ascending k); after the row, s = p_even + p_odd, then a butterfly over
//          the 64 lanes (xor 32, 16, 8, 4, 2, 1), then * channel scale.
//   NVFP4: 16 lanes per row; lane j owns records j, j+16, ... (ascending); inside a
//          record each K=16 group forms its own partial (ascending k), which is
//          multiplied by the group's E4M3 scale and added to the lane sum; then a
//          butterfly over the 16 lanes (xor 8, 4, 2, 1), then * (1/global_scale).
#include "dev_common.h"
#include "launch.h"

namespace wq {

namespace {

constexpr int kNumCU = 256;

__device__ __forceinline__ u32x4 ld16(const uint8_t* p) {
  u32x4 v;
  __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 16);
  return v;
}

// Stage rows m0 .. m0+MR-1 of x [M][K] (element type XT) into LDS as chunks of CK
// elements, each chunk padded to PAY+16 bytes.  Rows >= M are zero-filled.
template <typename XT, int CK>
__device__ __forceinline__ void stage_rows(uint8_t* lds, const XT* __restrict__ x, int m0, int MR, int M,
                                           int K) {
  constexpr int PAY = CK * (int)sizeof(XT);
  constexpr int STRIDE = PAY + 16;
  constexpr int PIECES = PAY / 16;
  const int C = K / CK;
  const int total = MR * C * PIECES;
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(x);
  for (int idx = threadIdx.x; idx < total; idx += blockDim.x) {
    const int p = idx % PIECES;
    const int rc = idx / PIECES;
    const int r = rc / C;
    const int c = rc - r * C;
    const int m = m0 + r;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (m < M) v = *reinterpret_cast<const u32x4*>(xb + ((size_t)m * K + (size_t)c * CK) * sizeof(XT) + p * 16);
    *reinterpret_cast<u32x4*>(lds + (size_t)rc * STRIDE + p * 16) = v;
  }
}

// ================================= FP8 E4M3 per-channel ========================================
template <typename XT, bool GU, int MR, int SEG>
__global__ void __launch_bounds__(256) fp8w_gemv_kernel(int M, int K, int N, int rpw,
                                                       const XT* __restrict__ x,
                                                       const uint8_t* __restrict__ w0,
                                                       const float* __restrict__ s0,
                                                       const uint8_t* __restrict__ w1,
                                                       const float* __restrict__ s1, float* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int NM = GU ? 2 : 1;
  constexpr int STRIDE = 16 * (int)sizeof(XT) + 16;
  const int C = K >> 4;
  const int CH = (C + 63) >> 6;
  const int nseg = (CH + SEG - 1) / SEG;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int r_begin = gw * rpw;
  const int r_end = min(N, r_begin + rpw);
  const uint8_t* wm[NM];
  wm[0] = w0;
  if constexpr (GU) wm[1] = w1;

  for (int m0 = 0; m0 < M; m0 += MR) {
    if (m0) __syncthreads();
    stage_rows<XT, 16>(lds, x, m0, MR, M, K);
    __syncthreads();
    if (r_begin >= r_end) continue;
    const int nsteps = (r_end - r_begin) * nseg;

    u32x4 buf[2][NM][SEG];
    float acc[MR][NM][2];
#pragma unroll
    for (int a = 0; a < MR; ++a)
#pragma unroll
      for (int b = 0; b < NM; ++b) acc[a][b][0] = acc[a][b][1] = 0.f;

    auto load_step = [&](int s, int bi) {
      const int row = r_begin + s / nseg;
      const int seg = s % nseg;
#pragma unroll
      for (int j = 0; j < SEG; ++j) {
        const int c = lane + 64 * (seg * SEG + j);
        if (c < C) {
#pragma unroll
          for (int mt = 0; mt < NM; ++mt) buf[bi][mt][j] = ld16(wm[mt] + (size_t)row * K + (size_t)c * 16);
        }
      }
    };

    auto compute_step = [&](int s, int bi) {
      const int row = r_begin + s / nseg;
      const int seg = s % nseg;
#pragma unroll
      for (int j = 0; j < SEG; ++j) {
        const int c = lane + 64 * (seg * SEG + j);
        if (c < C) {
#pragma unroll
          for (int mr = 0; mr < MR; ++mr) {
            const uint8_t* xl = lds + (size_t)(mr * C + c) * STRIDE;
            if constexpr (sizeof(XT) == 2) {  // bf16 activations: exact bf16 weights, dot2 into f32
              const u32x4 xa = *reinterpret_cast<const u32x4*>(xl);
              const u32x4 xb = *reinterpret_cast<const u32x4*>(xl + 16);
#pragma unroll
              for (int mt = 0; mt < NM; ++mt) {
                const u32x4 w = buf[bi][mt][j];
                float p0 = acc[mr][mt][0], p1 = acc[mr][mt][1];
                p0 = dot2_bf16(e4m3x2_bf16<false>(w.x), xa.x, p0);
                p0 = dot2_bf16(e4m3x2_bf16<true>(w.x), xa.y, p0);
                p1 = dot2_bf16(e4m3x2_bf16<false>(w.y), xa.z, p1);
                p1 = dot2_bf16(e4m3x2_bf16<true>(w.y), xa.w, p1);
                p0 = dot2_bf16(e4m3x2_bf16<false>(w.z), xb.x, p0);
                p0 = dot2_bf16(e4m3x2_bf16<true>(w.z), xb.y, p0);
                p1 = dot2_bf16(e4m3x2_bf16<false>(w.w), xb.z, p1);
                p1 = dot2_bf16(e4m3x2_bf16<true>(w.w), xb.w, p1);
                acc[mr][mt][0] = p0;
                acc[mr][mt][1] = p1;
              }
            } else {  // float32 activations: exact float32 weights, fma chain
              f32x4 xv[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) xv[q] = *reinterpret_cast<const f32x4*>(xl + 16 * q);
#pragma unroll
              for (int mt = 0; mt < NM; ++mt) {
                const u32x4 w = buf[bi][mt][j];
                float p[2] = {acc[mr][mt][0], acc[mr][mt][1]};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const f32x2 lo = e4m3x2_f32<false>(w[q]);
                  const f32x2 hi = e4m3x2_f32<true>(w[q]);
                  float& pp = p[q & 1];
                  pp = fmaf(xv[q].x, lo.x, pp);
                  pp = fmaf(xv[q].y, lo.y, pp);
                  pp = fmaf(xv[q].z, hi.x, pp);
                  pp = fmaf(xv[q].w, hi.y, pp);
                }
                acc[mr][mt][0] = p[0];
                acc[mr][mt][1] = p[1];
              }
            }
          }
        }
      }
      if (seg == nseg - 1) {  // row complete: reduce, epilogue, reset
#pragma unroll
        for (int mr = 0; mr < MR; ++mr) {
          float v[NM];
#pragma unroll
          for (int mt = 0; mt < NM; ++mt) {
            v[mt] = group_sum<64>(acc[mr][mt][0] + acc[mr][mt][1]);
            acc[mr][mt][0] = acc[mr][mt][1] = 0.f;
          }
          const int m = m0 + mr;
          if (lane == 0 && m < M) {
            float r;
            if constexpr (GU) {
              const float g = v[0] * s0[row];
              const float u = v[1] * s1[row];
              r = silu_f32(g) * u;
            } else {
              r = v[0] * s0[row];
            }
            y[(size_t)m * N + row] = r;
          }
        }
      }
    };

    load_step(0, 0);
    for (int s = 0; s < nsteps; s += 2) {
      if (s + 1 < nsteps) load_step(s + 1, 1);
      compute_step(s, 0);
      if (s + 1 >= nsteps) break;
      if (s + 2 < nsteps) load_step(s + 2, 0);
      compute_step(s + 1, 1);
    }
  }
}

// ===================================== NVFP4 Block64 ===========================================
// XF16 (16-bit XT only): x holds float16 bits, else bfloat16 bits.  Y16: y is stored as float16 bits
// (the NVFP4 MLP's act), else float32.
template <typename XT, bool GU, int MR, int SEG, bool XF16, bool Y16>
__global__ void __launch_bounds__(256) nvfp4_gemv_kernel(int M, int K, int N, int rpw,
                                                        const XT* __restrict__ x,
                                                        const uint8_t* __restrict__ b0, float inv0,
                                                        const uint8_t* __restrict__ b1, float inv1,
                                                        void* __restrict__ y) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  constexpr int NM = GU ? 2 : 1;
  constexpr int STRIDE = 64 * (int)sizeof(XT) + 16;
  const int nrec = K >> 6;
  const size_t rowbytes = (size_t)nrec * 36;
  const int T = (nrec + 15) >> 4;
  const int nseg = (T + SEG - 1) / SEG;
  const int lane = threadIdx.x & 63;
  const int j = lane & 15;
  const int q = lane >> 4;
  const int gw = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  const int r_begin = gw * rpw;
  const int r_end = min(N, r_begin + rpw);
  const uint8_t* bm[NM];
  bm[0] = b0;
  if constexpr (GU) bm[1] = b1;

  for (int m0 = 0; m0 < M; m0 += MR) {
    if (m0) __syncthreads();
    stage_rows<XT, 64>(lds, x, m0, MR, M, K);
    __syncthreads();
    if (r_begin >= r_end) continue;
    const int npass = (r_end - r_begin + 3) >> 2;
    const int nsteps = npass * nseg;

    u32x4 bufA[2][NM][SEG], bufB[2][NM][SEG];
    uint32_t bufC[2][NM][SEG];
    float acc[MR][NM];
#pragma unroll
    for (int a = 0; a < MR; ++a)
#pragma unroll
      for (int b = 0; b < NM; ++b) acc[a][b] = 0.f;

    auto load_step = [&](int s, int bi) {
      const int row = r_begin + 4 * (s / nseg) + q;
      const int seg = s % nseg;
      if (row < r_end) {
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
          const int rr = j + 16 * (seg * SEG + i);
          if (rr < nrec) {
#pragma unroll
            for (int mt = 0; mt < NM; ++mt) {
              const uint8_t* p = bm[mt] + (size_t)row * rowbytes + (size_t)rr * 36;
              bufA[bi][mt][i] = ld16(p);
              bufB[bi][mt][i] = ld16(p + 16);
              bufC[bi][mt][i] = *reinterpret_cast<const uint32_t*>(p + 32);
            }
          }
        }
      }
    };

    auto compute_step = [&](int s, int bi) {
      const int row = r_begin + 4 * (s / nseg) + q;
      const int seg = s % nseg;
      if (row < r_end) {
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
          const int rr = j + 16 * (seg * SEG + i);
          if (rr < nrec) {
#pragma unroll
            for (int mr = 0; mr < MR; ++mr) {
              const uint8_t* xl = lds + (size_t)(mr * nrec + rr) * STRIDE;
#pragma unroll
              for (int mt = 0; mt < NM; ++mt) {
                const u32x4 va = bufA[bi][mt][i], vb = bufB[bi][mt][i];
                const uint32_t d = va.x;
                const uint32_t qs[8] = {va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w, bufC[bi][mt][i]};
                float a = acc[mr][mt];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                  float part = 0.f;
                  if constexpr (sizeof(XT) == 2) {
                    const u32x4 x0 = *reinterpret_cast<const u32x4*>(xl + 32 * g);
                    const u32x4 x1 = *reinterpret_cast<const u32x4*>(xl + 32 * g + 16);
                    const uint32_t w0 = qs[2 * g], w1 = qs[2 * g + 1];
                    if constexpr (XF16) {
                      part = dot2_f16(e2m1x2_f16<0>(w0), as_f16x2(x0.x), part);
                      part = dot2_f16(e2m1x2_f16<1>(w0), as_f16x2(x0.y), part);
                      part = dot2_f16(e2m1x2_f16<2>(w0), as_f16x2(x0.z), part);
                      part = dot2_f16(e2m1x2_f16<3>(w0), as_f16x2(x0.w), part);
                      part = dot2_f16(e2m1x2_f16<0>(w1), as_f16x2(x1.x), part);
                      part = dot2_f16(e2m1x2_f16<1>(w1), as_f16x2(x1.y), part);
                      part = dot2_f16(e2m1x2_f16<2>(w1), as_f16x2(x1.z), part);
                      part = dot2_f16(e2m1x2_f16<3>(w1), as_f16x2(x1.w), part);
                    } else {
                    part = dot2_bf16(e2m1x2_bf16<0>(w0), x0.x, part);
                    part = dot2_bf16(e2m1x2_bf16<1>(w0), x0.y, part);
                    part = dot2_bf16(e2m1x2_bf16<2>(w0), x0.z, part);
                    part = dot2_bf16(e2m1x2_bf16<3>(w0), x0.w, part);
                    part = dot2_bf16(e2m1x2_bf16<0>(w1), x1.x, part);
                    part = dot2_bf16(e2m1x2_bf16<1>(w1), x1.y, part);
                    part = dot2_bf16(e2m1x2_bf16<2>(w1), x1.z, part);
                    part = dot2_bf16(e2m1x2_bf16<3>(w1), x1.w, part);
                    }
                  } else {
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                      const uint32_t w = qs[2 * g + h];
                      const f32x4 xa = *reinterpret_cast<const f32x4*>(xl + 64 * g + 32 * h);
                      const f32x4 xb = *reinterpret_cast<const f32x4*>(xl + 64 * g + 32 * h + 16);
                      f32x2 e;
                      e = e2m1x2_f32<0>(w);
                      part = fmaf(xa.x, e.x, part);
                      part = fmaf(xa.y, e.y, part);
                      e = e2m1x2_f32<1>(w);
                      part = fmaf(xa.z, e.x, part);
                      part = fmaf(xa.w, e.y, part);
                      e = e2m1x2_f32<2>(w);
                      part = fmaf(xb.x, e.x, part);
                      part = fmaf(xb.y, e.y, part);
                      e = e2m1x2_f32<3>(w);
                      part = fmaf(xb.z, e.x, part);
                      part = fmaf(xb.w, e.y, part);
                    }
                  }
                  float dg;
                  if (g == 0) dg = e4m3_byte_f32<0>(d);
                  else if (g == 1) dg = e4m3_byte_f32<1>(d);
                  else if (g == 2) dg = e4m3_byte_f32<2>(d);
                  else dg = e4m3_byte_f32<3>(d);
                  a = fmaf(part, dg, a);
                }
                acc[mr][mt] = a;
              }
            }
          }
        }
      }
      if (seg == nseg - 1) {  // pass complete: 16-lane reduce (all lanes take part), epilogue, reset
#pragma unroll
        for (int mr = 0; mr < MR; ++mr) {
          float v[NM];
#pragma unroll
          for (int mt = 0; mt < NM; ++mt) {
            v[mt] = group_sum<16>(acc[mr][mt]);
            acc[mr][mt] = 0.f;
          }
          const int m = m0 + mr;
          if (j == 0 && row < r_end && m < M) {
            float r;
            if constexpr (GU) {
              r = silu_f32(v[0] * inv0) * (v[1] * inv1);
            } else {
              r = v[0] * inv0;
            }
            if constexpr (Y16) reinterpret_cast<uint16_t*>(y)[(size_t)m * N + row] = __builtin_bit_cast(uint16_t, (_Float16)r);
            else reinterpret_cast<float*>(y)[(size_t)m * N + row] = r;
          }
        }
      }
    };

    load_step(0, 0);
    for (int s = 0; s < nsteps; s += 2) {
      if (s + 1 < nsteps) load_step(s + 1, 1);
      compute_step(s, 0);
      if (s + 1 >= nsteps) break;
      if (s + 2 < nsteps) load_step(s + 2, 0);
      compute_step(s + 1, 1);
    }
  }
}

// ---- launch shape ----------------------------------------------------------------------------
struct Shape {
  int grid, threads, rpw;
};

// Contiguous row ranges per wave, 4 waves per workgroup; choose the number of
// workgroups per CU (1 or 2, LDS permitting) that minimises the largest per-CU
// row count, preferring more occupancy on ties.  `gran` rounds rows per wave
// (4 for the 16-lane NVFP4 row groups).
Shape pick_shape(int N, size_t lds_bytes, int gran) {
  Shape best{0, 256, 0};
  long best_cost = -1;
  const int max_k = lds_bytes * 2 <= 160 * 1024 ? 2 : 1;
  for (int k = 1; k <= max_k; ++k) {
    const int waves = kNumCU * 4 * k;
    int rpw = (N + waves - 1) / waves;
    rpw = (rpw + gran - 1) / gran * gran;
    if (rpw < 1) rpw = 1;
    const int used_waves = (N + rpw - 1) / rpw;
    const int grid = (used_waves + 3) / 4;
    const int wg_per_cu = (grid + kNumCU - 1) / kNumCU;
    const long cost = (long)wg_per_cu * 4 * rpw;  // rows on the busiest CU
    if (best_cost < 0 || cost <= best_cost) {
      best_cost = cost;
      best = Shape{grid, 256, rpw};
    }
  }
  return best;
}

template <auto KERN>
bool lds_ok(size_t bytes) {
  return bytes <= 64 * 1024 || raise_lds_limit<KERN>();
}

constexpr size_t kLdsBudget = 96 * 1024;  // activation staging per workgroup for multi-row slabs

template <typename XT, bool GU>
hipError_t fp8_dispatch(int M, int K, int N, const void* x, const uint8_t* w0, const float* s0,
                        const uint8_t* w1, const float* s1, float* y, hipStream_t st) {
  constexpr int STRIDE = 16 * (int)sizeof(XT) + 16;
  const size_t per_row = (size_t)(K / 16) * STRIDE;
  const bool slab4 = M > 1 && 4 * per_row <= kLdsBudget;
  const size_t lds = (slab4 ? 4 : 1) * per_row;
  const Shape sh = pick_shape(N, lds, 1);
  constexpr int SEG = GU ? 5 : 6;
  if (slab4) {
    constexpr auto kern = &fp8w_gemv_kernel<XT, GU, 4, SEG>;
    if (!lds_ok<kern>(lds)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3(sh.grid), dim3(sh.threads), lds, st, M, K, N, sh.rpw,
                       reinterpret_cast<const XT*>(x), w0, s0, w1, s1, y);
  } else {
    constexpr auto kern = &fp8w_gemv_kernel<XT, GU, 1, SEG>;
    if (!lds_ok<kern>(lds)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3(sh.grid), dim3(sh.threads), lds, st, M, K, N, sh.rpw,
                       reinterpret_cast<const XT*>(x), w0, s0, w1, s1, y);
  }
  return hipGetLastError();
}

template <typename XT, bool GU, bool XF16, bool Y16>
hipError_t nvfp4_dispatch(int M, int K, int N, const void* x, const uint8_t* b0, float inv0,
                          const uint8_t* b1, float inv1, void* y, hipStream_t st) {
  constexpr int STRIDE = 64 * (int)sizeof(XT) + 16;
  const size_t per_row = (size_t)(K / 64) * STRIDE;
  const bool slab4 = M > 1 && 4 * per_row <= kLdsBudget;
  const size_t lds = (slab4 ? 4 : 1) * per_row;
  const Shape sh = pick_shape(N, lds, 4);
  constexpr int SEG = GU ? 1 : 2;
  if (slab4) {
    constexpr auto kern = &nvfp4_gemv_kernel<XT, GU, 4, SEG, XF16, Y16>;
    if (!lds_ok<kern>(lds)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3(sh.grid), dim3(sh.threads), lds, st, M, K, N, sh.rpw,
                       reinterpret_cast<const XT*>(x), b0, inv0, b1, inv1, y);
  } else {
    constexpr auto kern = &nvfp4_gemv_kernel<XT, GU, 1, SEG, XF16, Y16>;
    if (!lds_ok<kern>(lds)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(kern, dim3(sh.grid), dim3(sh.threads), lds, st, M, K, N, sh.rpw,
                       reinterpret_cast<const XT*>(x), b0, inv0, b1, inv1, y);
  }
  return hipGetLastError();
}

}  // namespace

// A single linear with fewer weights than this stays on the kernels above: the item kernel's activation
// staging, item loop and workgroup reduction are built for long, numerous rows and cost more than the
// whole product below about a million weights (hidden 256 x intermediate 512 down projection: 8.7 -> 2 us
// per launch at M = 1, the MLP step at M = 4 15.9 -> 8.5 us).
constexpr size_t kFp8ItemMinWeights = (size_t)1 << 20;

hipError_t launch_fp8w_gemv(int M, int K, int N, const void* x, XType xt, const uint8_t* w0, const float* s0,
                            const uint8_t* w1, const float* s1, float* y, hipStream_t st) {
  const bool gu = w1 != nullptr;
  if (fast_gemv_fp8_ok(K, xt, gu) && (gu || (size_t)N * K >= kFp8ItemMinWeights))
    return launch_fast_fp8(M, K, N, x, xt, w0, s0, w1, s1, y, st);
  if (xt == X_BF16)
    return gu ? fp8_dispatch<uint16_t, true>(M, K, N, x, w0, s0, w1, s1, y, st)
              : fp8_dispatch<uint16_t, false>(M, K, N, x, w0, s0, w1, s1, y, st);
  return gu ? fp8_dispatch<float, true>(M, K, N, x, w0, s0, w1, s1, y, st)
            : fp8_dispatch<float, false>(M, K, N, x, w0, s0, w1, s1, y, st);
}

hipError_t launch_nvfp4_gemv(int M, int K, int N, const void* x, XType xt, const uint8_t* b0, float inv0,
                             const uint8_t* b1, float inv1, void* y, bool y16, hipStream_t st) {
  const bool gu = b1 != nullptr;
  if (y16 && !gu) return hipErrorInvalidValue;
  if (fast_gemv_nvfp4_ok(K, xt, gu)) return launch_fast_nvfp4(M, K, N, x, xt, b0, inv0, b1, inv1, y, y16, st);
  if (gu) {
    if (xt == X_BF16)
      return y16 ? nvfp4_dispatch<uint16_t, true, false, true>(M, K, N, x, b0, inv0, b1, inv1, y, st)
                 : nvfp4_dispatch<uint16_t, true, false, false>(M, K, N, x, b0, inv0, b1, inv1, y, st);
    if (xt == X_F16) return hipErrorInvalidValue;
    return y16 ? nvfp4_dispatch<float, true, false, true>(M, K, N, x, b0, inv0, b1, inv1, y, st)
               : nvfp4_dispatch<float, true, false, false>(M, K, N, x, b0, inv0, b1, inv1, y, st);
  }
  if (xt == X_BF16) return nvfp4_dispatch<uint16_t, false, false, false>(M, K, N, x, b0, inv0, b1, inv1, y, st);
  if (xt == X_F16) return nvfp4_dispatch<uint16_t, false, true, false>(M, K, N, x, b0, inv0, b1, inv1, y, st);
  return nvfp4_dispatch<float, false, false, false>(M, K, N, x, b0, inv0, b1, inv1, y, st);
}

}  // namespace wq
