// AWQ int4 group-32 routed-expert single-token (M=1) step on gfx950.
//
// Method: pull request "[Kernel][SM70] Add native-g32 AWQ QPN M1 operator", section
// "What it does": W13 over the selected experts in router order with float16 gate/up
// materialisation and a fused SwiGLU into a (top-k, I) float16 intermediate; W2 with
// one float16 result per route and an ordered float32 router-weighted sum into a
// float16 output, without atomics; the half-fma dequantisation boundary
// RN_f16(q*s + RN_f16(-z*s)); invalid ids contribute zero, duplicates keep their own
// weights.
//
// Kernel 1 (W13 + SwiGLU): one workgroup per (route, 8 consecutive n).  A wave holds
// four 16-lane row groups: (gate n, up n, gate n+1, up n+1); lane j of a group owns
// the groups of 32 k  g = j, j+16, ...: one coalesced 16-byte code load per group plus
// its scale and zero.  x sits in LDS, permuted so that each dword holds the pair
// (k, k+4) that matches the nibble extraction.  Order: per lane, groups ascending,
// inside a group 16 dot2 steps ascending; then a butterfly over the 16 lanes.
// Kernel 2 (W2 + ordered sum): one workgroup per 32 outputs; thread (r, o) computes
// y_r[o] over its row's 5 groups (lane-per-row, act[r] broadcast from LDS), rounds
// it to float16 into LDS; then 32 threads sum the routes in order with fmaf.
#include "dev_common.h"
#include "launch.h"

namespace wq {

namespace {

constexpr int kGrpStride = 80;  // 32 f16 (64 B) + 16 B padding per group of 32 in LDS

// Copy n16 halves from src into LDS groups of 32 in (k, k+4) pair order.
__device__ __forceinline__ void stage_pairs(uint8_t* lds, const uint16_t* __restrict__ src, int n16) {
  const int nblk = n16 >> 3;  // 8-k blocks
  for (int b = threadIdx.x; b < nblk; b += blockDim.x) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + 8 * b);
    const uint16_t e[8] = {(uint16_t)v.x, (uint16_t)(v.x >> 16), (uint16_t)v.y, (uint16_t)(v.y >> 16),
                           (uint16_t)v.z, (uint16_t)(v.z >> 16), (uint16_t)v.w, (uint16_t)(v.w >> 16)};
    uint4 o;
    o.x = (uint32_t)e[0] | ((uint32_t)e[4] << 16);
    o.y = (uint32_t)e[1] | ((uint32_t)e[5] << 16);
    o.z = (uint32_t)e[2] | ((uint32_t)e[6] << 16);
    o.w = (uint32_t)e[3] | ((uint32_t)e[7] << 16);
    const int g = b >> 2;
    *reinterpret_cast<uint4*>(lds + g * kGrpStride + (b & 3) * 16) = o;
  }
}

// Dot product of one group of 32 codes (16 bytes) with 32 LDS activations.
__device__ __forceinline__ float awq_group_dot(const u32x4 c, _Float16 s, _Float16 b, const uint8_t* xg,
                                               float acc) {
  const f16x2 s2 = {s, s};
  const f16x2 b2 = {b, b};
#pragma unroll
  for (int dw = 0; dw < 4; ++dw) {
    const u32x4 xv = *reinterpret_cast<const u32x4*>(xg + 16 * dw);
    const uint32_t w = c[dw];
    acc = dot2_f16(awq_pair<0>(w, s2, b2), as_f16x2(xv.x), acc);
    acc = dot2_f16(awq_pair<1>(w, s2, b2), as_f16x2(xv.y), acc);
    acc = dot2_f16(awq_pair<2>(w, s2, b2), as_f16x2(xv.z), acc);
    acc = dot2_f16(awq_pair<3>(w, s2, b2), as_f16x2(xv.w), acc);
  }
  return acc;
}

template <int ML>
__device__ __forceinline__ _Float16 group_bias(const uint8_t* expert, const AwqLayout& L, int64_t idx, _Float16 s) {
  if constexpr (ML == 3) return awq_bias(expert[L.meta2_off + idx], s);
  else return f16_from_bits(reinterpret_cast<const uint16_t*>(expert + L.meta2_off)[idx]);
}

template <int ML>
__global__ void __launch_bounds__(256) awq_w13_kernel(int E, int H, int I, const uint16_t* __restrict__ x,
                                                      const int32_t* __restrict__ ids,
                                                      const uint8_t* __restrict__ bank, AwqLayout L,
                                                      uint16_t* __restrict__ act) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int r = blockIdx.x;
  const int nb = blockIdx.y * 8;
  const int e = ids[r];
  const int tid = threadIdx.x;
  if (e < 0 || e >= E) {  // invalid id: zero act row, no contribution
    if (tid < 8 && nb + tid < I) act[(size_t)r * I + nb + tid] = 0;
    return;
  }
  stage_pairs(lds, x, H);
  __syncthreads();
  const int lane = tid & 63;
  const int j = lane & 15;
  const int rg = lane >> 4;
  const int n = nb + 2 * (tid >> 6) + (rg >> 1);
  const int row = (rg & 1) ? n + I : n;
  const int G = H >> 5;
  const uint8_t* expert = bank + (size_t)e * L.expert_bytes;
  const uint8_t* codes = expert + (size_t)row * (H >> 1);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(expert + L.scale_off);
  float acc = 0.f;
  if (n < I) {
    for (int g = j; g < G; g += 16) {
      const u32x4 c = *reinterpret_cast<const u32x4*>(codes + 16 * g);
      const int64_t mi = (int64_t)row * G + g;
      const _Float16 s = f16_from_bits(scales[mi]);
      const _Float16 b = group_bias<ML>(expert, L, mi, s);
      acc = awq_group_dot(c, s, b, lds + g * kGrpStride, acc);
    }
  }
  acc = group_sum<16>(acc);
  const float u = __shfl_down(acc, 16, 64);
  if (j == 0 && (rg & 1) == 0 && n < I) {
    const float gh = (float)(_Float16)acc;
    const float uh = (float)(_Float16)u;
    const _Float16 a = (_Float16)(silu_f32(gh) * uh);
    act[(size_t)r * I + n] = __builtin_bit_cast(uint16_t, a);
  }
}

template <int ML>
__global__ void __launch_bounds__(512) awq_w2_kernel(int E, int topk, int H, int I,
                                                     const int32_t* __restrict__ ids,
                                                     const float* __restrict__ router_w,
                                                     const uint8_t* __restrict__ bank, AwqLayout L,
                                                     const uint16_t* __restrict__ act, uint16_t* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int G = I >> 5;
  const int act_bytes = G * kGrpStride;  // per route
  float* ys = reinterpret_cast<float*>(lds + topk * act_bytes);  // [topk][32]
  const int tid = threadIdx.x;
  for (int r = 0; r < topk; ++r) stage_pairs(lds + r * act_bytes, act + (size_t)r * I, I);
  __syncthreads();
  const int r = tid >> 5;
  const int ol = tid & 31;
  const int o = blockIdx.x * 32 + ol;
  if (r < topk) {
    const int e = ids[r];
    float v = 0.f;
    if (e >= 0 && e < E && o < H) {
      const uint8_t* expert = bank + (size_t)e * L.expert_bytes;
      const uint8_t* codes = expert + (size_t)o * (I >> 1);
      const uint16_t* scales = reinterpret_cast<const uint16_t*>(expert + L.scale_off);
      float acc = 0.f;
      for (int g = 0; g < G; ++g) {
        const u32x4 c = *reinterpret_cast<const u32x4*>(codes + 16 * g);
        const int64_t mi = (int64_t)o * G + g;
        const _Float16 s = f16_from_bits(scales[mi]);
        const _Float16 b = group_bias<ML>(expert, L, mi, s);
        acc = awq_group_dot(c, s, b, lds + r * act_bytes + g * kGrpStride, acc);
      }
      v = (float)(_Float16)acc;  // per-route float16 materialisation
    }
    ys[r * 32 + ol] = v;
  }
  __syncthreads();
  if (tid < 32 && o < H) {
    float acc = 0.f;
    for (int rr = 0; rr < topk; ++rr) {
      const int e = ids[rr];
      if (e >= 0 && e < E) acc = fmaf(router_w[rr], ys[rr * 32 + tid], acc);
    }
    out[o] = __builtin_bit_cast(uint16_t, (_Float16)acc);
  }
}

}  // namespace

hipError_t launch_moe_awq_m1(int E, int topk, int H, int I, const uint16_t* x, const int32_t* ids,
                             const float* router_w, const uint8_t* w13, const uint8_t* w2, int meta_layout,
                             uint16_t* act, uint16_t* out, hipStream_t st) {
  const AwqLayout L13 = awq_layout(2 * (int64_t)I, H, meta_layout);
  const AwqLayout L2 = awq_layout(H, I, meta_layout);
  const size_t lds13 = (size_t)(H / 32) * kGrpStride;
  const dim3 g13(topk, (I + 7) / 8);
  if (meta_layout == 3)
    hipLaunchKernelGGL(awq_w13_kernel<3>, g13, dim3(256), lds13, st, E, H, I, x, ids, w13, L13, act);
  else
    hipLaunchKernelGGL(awq_w13_kernel<4>, g13, dim3(256), lds13, st, E, H, I, x, ids, w13, L13, act);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds2 = (size_t)topk * (I / 32) * kGrpStride + (size_t)topk * 32 * 4;
  const int threads = (topk * 32 + 63) / 64 * 64;
  const dim3 g2((H + 31) / 32);
  if (meta_layout == 3)
    hipLaunchKernelGGL(awq_w2_kernel<3>, g2, dim3(threads), lds2, st, E, topk, H, I, ids, router_w, w2, L2, act,
                       out);
  else
    hipLaunchKernelGGL(awq_w2_kernel<4>, g2, dim3(threads), lds2, st, E, topk, H, I, ids, router_w, w2, L2, act,
                       out);
  return hipGetLastError();
}

}  // namespace wq
