// M < 128 path, main kernels: HBM-streaming GEMVs tuned on MI355X for the decode shapes.
//
// Method: issue "tp>1 fp8w tail-MLP shard host-dequantizes every layer", section
// "Proposed fix" (SwiGLU MLP, float32 act); NVFP4 decode from page
// "Qwen3.8-27B-NVFP4", section "NVFP4 numerics as implemented" (the E4M3 group
// scale applied at every K=16 boundary).
//
// Two kernel shapes, chosen from measurements of the 5120 x 17408 decode:
//  * row kernels (gate+up): one wave per output row pair; every weight load of the
//    pair is issued at once (2 x 5 KB for FP8 at K=5120), the activation row sits in
//    registers (FP8) or LDS (NVFP4), occupancy 8 waves/SIMD.  The weights stay in
//    registers while the m rows of a multi-row call are processed one by one.
//  * item kernels (down projection / single linear): a 16-wave workgroup owns RB
//    output rows; the activation row is staged once into LDS; the (row pair, K slot)
//    work items -- a K slot is one 16-byte load per lane -- are dealt round-robin to the
//    waves, each wave streaming its items with the next D loads in flight; each wave
//    keeps one partial per row it touches and the workgroup adds the 16 partials of a
//    row in wave order.
// Fixed accumulation orders (bitwise reproducible; independent of M because m rows
// are processed one after another with the same schedule):
//  * FP8 row kernel: lane l owns 16-byte chunks l, l+64, ...; per chunk the 8 code pairs
//    go into two partials (even / odd 4-code quads), chunks ascending; s = p0 + p1;
//    butterfly over 64 lanes (xor 32..1); times the channel scale.
//  * NVFP4 row kernel: lane l owns records l, l+64, ...; per record each K=16 group's
//    partial (ascending k) is multiplied by its E4M3 scale and added in group order;
//    butterfly over 64 lanes; times 1/global_scale.
//  * item kernels: within a wave, items ascending, each item a chunk (FP8: 16 codes, two
//    partials as above; NVFP4: one record as above); per row a butterfly over 64 lanes
//    when the wave leaves the row; then the workgroup sums the per-wave partials in wave
//    order 0..15; times the channel scale or 1/global_scale.
#include "dev_common.h"
#include "launch.h"

namespace wq {

namespace {

constexpr int kItemWaves = 16;   // waves per item-kernel workgroup
constexpr int kItemRows = 20;    // output rows per item-kernel workgroup
constexpr int kItemDepth = 2;    // loads in flight per wave (items)

__device__ __forceinline__ u32x4 ld_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x4 ld16a4(const uint8_t* p) {
  u32x4 v;
  __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 16);
  return v;
}
template <int W>
__device__ __forceinline__ float gsum(float v) {
#pragma unroll
  for (int o = W / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float e4m3_group(uint32_t d, int g) {
  return g == 0 ? e4m3_byte_f32<0>(d) : g == 1 ? e4m3_byte_f32<1>(d) : g == 2 ? e4m3_byte_f32<2>(d)
                                                                             : e4m3_byte_f32<3>(d);
}

// ---- FP8 gate+up row kernel (bf16 x) -------------------------------------------------------------
// ONE: the call has a single activation row (compile-time loop bound).
template <int CH, bool ONE>
__global__ void __launch_bounds__(256) fp8_gu_row(int M, int K, int N, const uint16_t* __restrict__ x,
                                                 const uint8_t* __restrict__ wg, const float* __restrict__ sg,
                                                 const uint8_t* __restrict__ wu, const float* __restrict__ su,
                                                 float* __restrict__ act) {
  const int C = K >> 4;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= N) return;
  u32x4 w[2][CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = lane + 64 * c;
    if (ch < C) {
      w[0][c] = ld_stream(wg + (size_t)row * K + 16 * ch);
      w[1][c] = ld_stream(wu + (size_t)row * K + 16 * ch);
    }
  }
  const float gsc = sg[row], usc = su[row];
  const int Mloop = ONE ? 1 : M;
  for (int m = 0; m < Mloop; ++m) {
    const uint16_t* xm = x + (size_t)m * K;
    u32x4 xr[CH][2];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = lane + 64 * c;
      if (ch < C) {
        xr[c][0] = *reinterpret_cast<const u32x4*>(xm + 16 * ch);
        xr[c][1] = *reinterpret_cast<const u32x4*>(xm + 16 * ch + 8);
      }
    }
    float a[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (lane + 64 * c < C) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 v = w[t][c];
          float p0 = a[t][0], p1 = a[t][1];
          p0 = dot2_bf16(e4m3x2_bf16<false>(v.x), xr[c][0].x, p0);
          p0 = dot2_bf16(e4m3x2_bf16<true>(v.x), xr[c][0].y, p0);
          p1 = dot2_bf16(e4m3x2_bf16<false>(v.y), xr[c][0].z, p1);
          p1 = dot2_bf16(e4m3x2_bf16<true>(v.y), xr[c][0].w, p1);
          p0 = dot2_bf16(e4m3x2_bf16<false>(v.z), xr[c][1].x, p0);
          p0 = dot2_bf16(e4m3x2_bf16<true>(v.z), xr[c][1].y, p0);
          p1 = dot2_bf16(e4m3x2_bf16<false>(v.w), xr[c][1].z, p1);
          p1 = dot2_bf16(e4m3x2_bf16<true>(v.w), xr[c][1].w, p1);
          a[t][0] = p0;
          a[t][1] = p1;
        }
      }
    }
    const float g = gsum<64>(a[0][0] + a[0][1]) * gsc;
    const float u = gsum<64>(a[1][0] + a[1][1]) * usc;
    if (lane == 0) act[(size_t)m * N + row] = silu_f32(g) * u;
  }
}

// ---- NVFP4 gate+up row kernel (bf16 x in LDS, record r at r*144) -----------------------------------
template <int NR, bool ONE>
__global__ void __launch_bounds__(512) nv_gu_row(int M, int K, int N, const uint16_t* __restrict__ x,
                                                const uint8_t* __restrict__ bg, float inv_g,
                                                const uint8_t* __restrict__ bu, float inv_u, float* __restrict__ act) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int nrec = K >> 6;
  const size_t rb = (size_t)nrec * 36;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 8 + (threadIdx.x >> 6);
  const bool on = row < N;
  u32x4 A[2][NR], B[2][NR];
  uint32_t Cw[2][NR];
  if (on) {
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      const int r = lane + 64 * t;
      if (r < nrec) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const uint8_t* p = (mt ? bu : bg) + (size_t)row * rb + (size_t)r * 36;
          A[mt][t] = ld16a4(p);
          B[mt][t] = ld16a4(p + 16);
          Cw[mt][t] = *reinterpret_cast<const uint32_t*>(p + 32);
        }
      }
    }
  }
  const int Mloop = ONE ? 1 : M;
  for (int m = 0; m < Mloop; ++m) {
    if (m) __syncthreads();
    const u32x4* xm = reinterpret_cast<const u32x4*>(x + (size_t)m * K);
    for (int i = threadIdx.x; i < nrec * 8; i += blockDim.x)
      *reinterpret_cast<u32x4*>(lds + (i >> 3) * 144 + (i & 7) * 16) = xm[i];
    __syncthreads();
    if (!on) continue;
    float acc[2] = {0.f, 0.f};
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      const int r = lane + 64 * t;
      if (r < nrec) {
        const uint8_t* xl = lds + r * 144;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const uint32_t d = A[mt][t].x;
          const uint32_t qs[8] = {A[mt][t].y, A[mt][t].z, A[mt][t].w, B[mt][t].x,
                                  B[mt][t].y, B[mt][t].z, B[mt][t].w, Cw[mt][t]};
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const u32x4 x0 = *reinterpret_cast<const u32x4*>(xl + 32 * g);
            const u32x4 x1 = *reinterpret_cast<const u32x4*>(xl + 32 * g + 16);
            float part = 0.f;
            part = dot2_bf16(e2m1x2_bf16<0>(qs[2 * g]), x0.x, part);
            part = dot2_bf16(e2m1x2_bf16<1>(qs[2 * g]), x0.y, part);
            part = dot2_bf16(e2m1x2_bf16<2>(qs[2 * g]), x0.z, part);
            part = dot2_bf16(e2m1x2_bf16<3>(qs[2 * g]), x0.w, part);
            part = dot2_bf16(e2m1x2_bf16<0>(qs[2 * g + 1]), x1.x, part);
            part = dot2_bf16(e2m1x2_bf16<1>(qs[2 * g + 1]), x1.y, part);
            part = dot2_bf16(e2m1x2_bf16<2>(qs[2 * g + 1]), x1.z, part);
            part = dot2_bf16(e2m1x2_bf16<3>(qs[2 * g + 1]), x1.w, part);
            acc[mt] = fmaf(part, e4m3_group(d, g), acc[mt]);
          }
        }
      }
    }
    const float gv = gsum<64>(acc[0]) * inv_g;
    const float uv = gsum<64>(acc[1]) * inv_u;
    if (lane == 0) act[(size_t)m * N + row] = silu_f32(gv) * uv;
  }
}

// ---- item kernels ---------------------------------------------------------------------------------
// Activation row m staged into LDS piece-major: piece q (16 bytes) of unit u at (q * U + u) * 16, where a
// unit is an FP8 chunk (16 codes) or an NVFP4 record (64 codes) and PQ pieces make one unit.
template <typename XT, int UNIT>
__device__ __forceinline__ void stage_units(uint8_t* lds, const XT* __restrict__ xm, int U) {
  constexpr int PQ = UNIT * (int)sizeof(XT) / 16;
  const u32x4* src = reinterpret_cast<const u32x4*>(xm);
  for (int i = threadIdx.x; i < U * PQ; i += blockDim.x) {
    const int u = i / PQ, q = i - u * PQ;
    *reinterpret_cast<u32x4*>(lds + ((size_t)q * U + u) * 16) = src[i];
  }
}

// Item cursor: item it = g * T + t advanced by NW per step without divisions.
struct ItemCursor {
  int g, t;
  __device__ __forceinline__ void init(int it, int T) {
    g = it / T;
    t = it - g * T;
  }
  __device__ __forceinline__ void step(int nw, int T) {
    t += nw;
    while (t >= T) {
      t -= T;
      ++g;
    }
  }
};

// FP8 single linear: y[m, n] = s[n] * sum_k xa[m, k] e4m3(w[n, k]); XT float or bf16 bits.
template <typename XT, bool ONE>
__global__ void __launch_bounds__(64 * kItemWaves, 8) fp8_lin_items(int M, int K, int N, const XT* __restrict__ xa,
                                                                 const uint8_t* __restrict__ w,
                                                                 const float* __restrict__ s, float* __restrict__ y) {
  constexpr int R = 2, D = kItemDepth, NW = kItemWaves, RB = kItemRows;
  constexpr int PQ = 16 * (int)sizeof(XT) / 16;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ float part[NW][RB];
  const int C = K >> 4, T = (C + 63) >> 6;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rbase = blockIdx.x * RB;
  const int NI = (RB / R) * T;
  const int nk = NI > wv ? (NI - wv + NW - 1) / NW : 0;
  const int Mloop = ONE ? 1 : M;
  for (int m = 0; m < Mloop; ++m) {
    if (m) __syncthreads();
    for (int i = threadIdx.x; i < NW * RB; i += blockDim.x) (&part[0][0])[i] = 0.f;
    u32x4 buf[D][R];
    ItemCursor lc;  // next item to load
    lc.init(wv, T);
    int lk = 0;
    auto load = [&](int b) {
      if (lk < nk) {
        // Clamped to the last chunk / row: in bounds, and never accumulated or stored.
        const int c = min(lane + 64 * lc.t, C - 1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int n = min(rbase + lc.g * R + r, N - 1);
          buf[b][r] = ld_stream(w + (size_t)n * K + 16 * c);
        }
      }
      ++lk;
      lc.step(NW, T);
    };
#pragma unroll
    for (int b = 0; b < D; ++b) load(b);
    stage_units<XT, 16>(lds, xa + (size_t)m * K, C);
    __syncthreads();
    float acc[R][2];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r][0] = acc[r][1] = 0.f;
    int cur = -1;
    auto flush = [&]() {
      if (cur < 0) return;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v = gsum<64>(acc[r][0] + acc[r][1]);
        acc[r][0] = acc[r][1] = 0.f;
        if (lane == 0) part[wv][cur * R + r] = v;
      }
    };
    ItemCursor cc;  // item being computed
    cc.init(wv, T);
    for (int k0 = 0; k0 < nk; k0 += D) {
#pragma unroll
      for (int b = 0; b < D; ++b) {
        const int k = k0 + b;
        if (k < nk) {
          const int g = cc.g, c = lane + 64 * cc.t;
          cc.step(NW, T);
          if (g != cur) {
            flush();
            cur = g;
          }
          if (c < C) {
            if constexpr (sizeof(XT) == 4) {
              f32x4 xv[4];
#pragma unroll
              for (int q = 0; q < 4; ++q) xv[q] = *reinterpret_cast<const f32x4*>(lds + ((size_t)q * C + c) * 16);
#pragma unroll
              for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const f32x2 lo = e4m3x2_f32<false>(buf[b][r][q]), hi = e4m3x2_f32<true>(buf[b][r][q]);
                  float& sacc = acc[r][q & 1];
                  sacc = fmaf(xv[q].x, lo.x, sacc);
                  sacc = fmaf(xv[q].y, lo.y, sacc);
                  sacc = fmaf(xv[q].z, hi.x, sacc);
                  sacc = fmaf(xv[q].w, hi.y, sacc);
                }
              }
            } else {
              const u32x4 x0 = *reinterpret_cast<const u32x4*>(lds + ((size_t)0 * C + c) * 16);
              const u32x4 x1 = *reinterpret_cast<const u32x4*>(lds + ((size_t)1 * C + c) * 16);
#pragma unroll
              for (int r = 0; r < R; ++r) {
                const u32x4 v = buf[b][r];
                float p0 = acc[r][0], p1 = acc[r][1];
                p0 = dot2_bf16(e4m3x2_bf16<false>(v.x), x0.x, p0);
                p0 = dot2_bf16(e4m3x2_bf16<true>(v.x), x0.y, p0);
                p1 = dot2_bf16(e4m3x2_bf16<false>(v.y), x0.z, p1);
                p1 = dot2_bf16(e4m3x2_bf16<true>(v.y), x0.w, p1);
                p0 = dot2_bf16(e4m3x2_bf16<false>(v.z), x1.x, p0);
                p0 = dot2_bf16(e4m3x2_bf16<true>(v.z), x1.y, p0);
                p1 = dot2_bf16(e4m3x2_bf16<false>(v.w), x1.z, p1);
                p1 = dot2_bf16(e4m3x2_bf16<true>(v.w), x1.w, p1);
                acc[r][0] = p0;
                acc[r][1] = p1;
              }
            }
          }
          load(b);
        }
      }
    }
    flush();
    __syncthreads();
    if (threadIdx.x < RB) {
      const int n = rbase + threadIdx.x;
      if (n < N) {
        float v = 0.f;
        for (int ww = 0; ww < NW; ++ww) v += part[ww][threadIdx.x];
        y[(size_t)m * N + n] = v * s[n];
      }
    }
    (void)PQ;
  }
}

// NVFP4 single linear: y[m, n] = inv * sum_k xa[m, k] dq(blk[n, k]).
template <typename XT, bool ONE>
__global__ void __launch_bounds__(64 * kItemWaves, 8) nv_lin_items(int M, int K, int N, const XT* __restrict__ xa,
                                                                const uint8_t* __restrict__ blk, float inv,
                                                                float* __restrict__ y) {
  constexpr int D = kItemDepth, NW = kItemWaves, RB = kItemRows;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ float part[NW][RB];
  const int nrec = K >> 6, T = (nrec + 63) >> 6;
  const size_t rb = (size_t)nrec * 36;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rbase = blockIdx.x * RB;
  const int NI = RB * T;
  const int nk = NI > wv ? (NI - wv + NW - 1) / NW : 0;
  const int Mloop = ONE ? 1 : M;
  for (int m = 0; m < Mloop; ++m) {
    if (m) __syncthreads();
    for (int i = threadIdx.x; i < NW * RB; i += blockDim.x) (&part[0][0])[i] = 0.f;
    u32x4 A[D], B[D];
    uint32_t Cw[D];
    ItemCursor lc;
    lc.init(wv, T);
    int lk = 0;
    auto load = [&](int b) {
      if (lk < nk) {
        // Clamped to the last record / row: in bounds, and never accumulated or stored.
        const int r = min(lane + 64 * lc.t, nrec - 1), n = min(rbase + lc.g, N - 1);
        const uint8_t* p = blk + (size_t)n * rb + (size_t)r * 36;
        A[b] = ld16a4(p);
        B[b] = ld16a4(p + 16);
        Cw[b] = *reinterpret_cast<const uint32_t*>(p + 32);
      }
      ++lk;
      lc.step(NW, T);
    };
#pragma unroll
    for (int b = 0; b < D; ++b) load(b);
    stage_units<XT, 64>(lds, xa + (size_t)m * K, nrec);
    __syncthreads();
    float acc = 0.f;
    int cur = -1;
    auto flush = [&]() {
      if (cur < 0) return;
      const float v = gsum<64>(acc);
      acc = 0.f;
      if (lane == 0) part[wv][cur] = v;
    };
    ItemCursor cc;
    cc.init(wv, T);
    for (int k0 = 0; k0 < nk; k0 += D) {
#pragma unroll
      for (int b = 0; b < D; ++b) {
        const int k = k0 + b;
        if (k < nk) {
          const int g = cc.g, r = lane + 64 * cc.t;
          cc.step(NW, T);
          if (g != cur) {
            flush();
            cur = g;
          }
          if (r < nrec) {
            const uint32_t d = A[b].x;
            const uint32_t qs[8] = {A[b].y, A[b].z, A[b].w, B[b].x, B[b].y, B[b].z, B[b].w, Cw[b]};
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              float pt = 0.f;
              if constexpr (sizeof(XT) == 4) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                  const f32x4 xa0 = *reinterpret_cast<const f32x4*>(lds + ((size_t)(4 * gq + 2 * h) * nrec + r) * 16);
                  const f32x4 xa1 = *reinterpret_cast<const f32x4*>(lds + ((size_t)(4 * gq + 2 * h + 1) * nrec + r) * 16);
                  const uint32_t wq = qs[2 * gq + h];
                  f32x2 e = e2m1x2_f32<0>(wq);
                  pt = fmaf(xa0.x, e.x, pt);
                  pt = fmaf(xa0.y, e.y, pt);
                  e = e2m1x2_f32<1>(wq);
                  pt = fmaf(xa0.z, e.x, pt);
                  pt = fmaf(xa0.w, e.y, pt);
                  e = e2m1x2_f32<2>(wq);
                  pt = fmaf(xa1.x, e.x, pt);
                  pt = fmaf(xa1.y, e.y, pt);
                  e = e2m1x2_f32<3>(wq);
                  pt = fmaf(xa1.z, e.x, pt);
                  pt = fmaf(xa1.w, e.y, pt);
                }
              } else {
                const u32x4 x0 = *reinterpret_cast<const u32x4*>(lds + ((size_t)(2 * gq) * nrec + r) * 16);
                const u32x4 x1 = *reinterpret_cast<const u32x4*>(lds + ((size_t)(2 * gq + 1) * nrec + r) * 16);
                pt = dot2_bf16(e2m1x2_bf16<0>(qs[2 * gq]), x0.x, pt);
                pt = dot2_bf16(e2m1x2_bf16<1>(qs[2 * gq]), x0.y, pt);
                pt = dot2_bf16(e2m1x2_bf16<2>(qs[2 * gq]), x0.z, pt);
                pt = dot2_bf16(e2m1x2_bf16<3>(qs[2 * gq]), x0.w, pt);
                pt = dot2_bf16(e2m1x2_bf16<0>(qs[2 * gq + 1]), x1.x, pt);
                pt = dot2_bf16(e2m1x2_bf16<1>(qs[2 * gq + 1]), x1.y, pt);
                pt = dot2_bf16(e2m1x2_bf16<2>(qs[2 * gq + 1]), x1.z, pt);
                pt = dot2_bf16(e2m1x2_bf16<3>(qs[2 * gq + 1]), x1.w, pt);
              }
              acc = fmaf(pt, e4m3_group(d, gq), acc);
            }
          }
          load(b);
        }
      }
    }
    flush();
    __syncthreads();
    if (threadIdx.x < RB) {
      const int n = rbase + threadIdx.x;
      if (n < N) {
        float v = 0.f;
        for (int ww = 0; ww < NW; ++ww) v += part[ww][threadIdx.x];
        y[(size_t)m * N + n] = v * inv;
      }
    }
  }
}

template <typename KF>
bool lds_ok(KF kernel, size_t bytes) {
  if (bytes > 64 * 1024)
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes) == hipSuccess;
  return true;
}

constexpr size_t kMaxItemLds = 150 * 1024;

}  // namespace

bool fast_gemv_fp8_ok(int K, XType xt, bool gu) {
  if (K % 16) return false;
  if (gu) return xt == X_BF16 && (K / 16 + 63) / 64 <= 8;
  return (size_t)K * (xt == X_F32 ? 4 : 2) <= kMaxItemLds;
}

bool fast_gemv_nvfp4_ok(int K, XType xt, bool gu) {
  if (K % 64) return false;
  if (gu) return xt == X_BF16 && (K / 64 + 63) / 64 <= 4;
  return (size_t)K * (xt == X_F32 ? 4 : 2) <= kMaxItemLds;
}

hipError_t launch_fast_fp8(int M, int K, int N, const void* x, XType xt, const uint8_t* w0, const float* s0,
                           const uint8_t* w1, const float* s1, float* y, hipStream_t st) {
  if (w1 != nullptr) {
    const int CH = (K / 16 + 63) / 64;
    const dim3 grid((N + 3) / 4), block(256);
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    switch (CH) {
#define WQ_CASE(n)                                                                                       \
  case n:                                                                                                \
    if (M == 1) hipLaunchKernelGGL((fp8_gu_row<n, true>), grid, block, 0, st, M, K, N, xb, w0, s0, w1, s1, y); \
    else hipLaunchKernelGGL((fp8_gu_row<n, false>), grid, block, 0, st, M, K, N, xb, w0, s0, w1, s1, y);      \
    break;
      WQ_CASE(1) WQ_CASE(2) WQ_CASE(3) WQ_CASE(4) WQ_CASE(5) WQ_CASE(6) WQ_CASE(7) WQ_CASE(8)
#undef WQ_CASE
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const size_t lds = (size_t)K * (xt == X_F32 ? 4 : 2);
  const dim3 grid((N + kItemRows - 1) / kItemRows), block(64 * kItemWaves);
#define WQ_LAUNCH(T, O)                                                                                     \
  do {                                                                                                      \
    if (!lds_ok(fp8_lin_items<T, O>, lds)) return hipErrorInvalidValue;                                     \
    hipLaunchKernelGGL((fp8_lin_items<T, O>), grid, block, lds, st, M, K, N, reinterpret_cast<const T*>(x), w0, s0, y); \
  } while (0)
  if (xt == X_F32) {
    if (M == 1) WQ_LAUNCH(float, true);
    else WQ_LAUNCH(float, false);
  } else {
    if (M == 1) WQ_LAUNCH(uint16_t, true);
    else WQ_LAUNCH(uint16_t, false);
  }
#undef WQ_LAUNCH
  return hipGetLastError();
}

hipError_t launch_fast_nvfp4(int M, int K, int N, const void* x, XType xt, const uint8_t* b0, float inv0,
                             const uint8_t* b1, float inv1, float* y, hipStream_t st) {
  if (b1 != nullptr) {
    const int NR = (K / 64 + 63) / 64;
    const size_t lds = (size_t)(K / 64) * 144;
    const dim3 grid((N + 7) / 8), block(512);
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    switch (NR) {
#define WQ_CASE(n)                                                                                          \
  case n:                                                                                                   \
    if (M == 1) hipLaunchKernelGGL((nv_gu_row<n, true>), grid, block, lds, st, M, K, N, xb, b0, inv0, b1, inv1, y); \
    else hipLaunchKernelGGL((nv_gu_row<n, false>), grid, block, lds, st, M, K, N, xb, b0, inv0, b1, inv1, y);      \
    break;
      WQ_CASE(1) WQ_CASE(2) WQ_CASE(3) WQ_CASE(4)
#undef WQ_CASE
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const size_t lds = (size_t)K * (xt == X_F32 ? 4 : 2);
  const dim3 grid((N + kItemRows - 1) / kItemRows), block(64 * kItemWaves);
#define WQ_LAUNCH(T, O)                                                                                      \
  do {                                                                                                       \
    if (!lds_ok(nv_lin_items<T, O>, lds)) return hipErrorInvalidValue;                                       \
    hipLaunchKernelGGL((nv_lin_items<T, O>), grid, block, lds, st, M, K, N, reinterpret_cast<const T*>(x), b0, inv0, y); \
  } while (0)
  if (xt == X_F32) {
    if (M == 1) WQ_LAUNCH(float, true);
    else WQ_LAUNCH(float, false);
  } else {
    if (M == 1) WQ_LAUNCH(uint16_t, true);
    else WQ_LAUNCH(uint16_t, false);
  }
#undef WQ_LAUNCH
  return hipGetLastError();
}

}  // namespace wq
