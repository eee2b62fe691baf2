// One-time weight packers and the debug decoders (gfx950).
//
// Block64: page "Qwen3.8-27B-NVFP4", section "NVFP4 numerics as implemented" -- a
// record {uint8 d[4]; uint8 qs[32]} per 64 consecutive weights of a row, d = the four
// E4M3 group-16 scales in K order, qs = the 64 E2M1 codes, low nibble first.
// AWQ bank: the layout documented in wqmlp.h (codes row-major, float16 scale plane,
// uint8 zero plane or float16 bias plane), metadata sizes from pull request
// "[Kernel][SM70] Add native-g32 AWQ QPN M1 operator", section "What it does".
// The decoders decode one element per thread with the float32 conversions (the ones the float32-activation
// GEMV kernels use) and the AWQ kernels' own half-fma pair decode.  Kernels with bfloat16 or float16
// operands decode with the packed bfloat16 / float16 conversions, which these decoders do not run.
#include "dev_common.h"
#include "launch.h"

namespace wq {

namespace {

__global__ void nvfp4_pack_kernel(int64_t N, int64_t nb, const uint8_t* __restrict__ wp,
                                  const uint8_t* __restrict__ ws, uint8_t* __restrict__ blk) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one record
  if (idx >= N * nb) return;
  const int64_t n = idx / nb, b = idx - n * nb;
  uint8_t* o = blk + idx * 36;
  const uint8_t* s = ws + n * nb * 4 + b * 4;
  const uint8_t* q = wp + n * nb * 32 + b * 32;
  for (int i = 0; i < 4; ++i) o[i] = s[i];
  for (int i = 0; i < 32; ++i) o[4 + i] = q[i];
}

__global__ void awq_pack_codes_kernel(int64_t total_bytes, const uint8_t* __restrict__ codes,
                                      uint8_t* __restrict__ bank, int64_t per_expert, int64_t stride) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one packed byte
  if (i >= total_bytes) return;
  const int64_t e = i / per_expert, j = i - e * per_expert;
  const uint8_t lo = codes[2 * i] & 15, hi = codes[2 * i + 1] & 15;
  bank[e * stride + j] = (uint8_t)(lo | (hi << 4));
}

__global__ void awq_pack_meta_kernel(int64_t total, int64_t per_expert, const uint16_t* __restrict__ scales,
                                     const uint8_t* __restrict__ zeros, int meta_layout, uint8_t* __restrict__ bank,
                                     AwqLayout L) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one group
  if (i >= total) return;
  const int64_t e = i / per_expert, j = i - e * per_expert;
  uint8_t* ex = bank + e * L.expert_bytes;
  reinterpret_cast<uint16_t*>(ex + L.scale_off)[j] = scales[i];
  if (meta_layout == 3) {
    ex[L.meta2_off + j] = zeros[i];
  } else {
    const _Float16 b = awq_bias(zeros[i], f16_from_bits(scales[i]));
    reinterpret_cast<uint16_t*>(ex + L.meta2_off)[j] = __builtin_bit_cast(uint16_t, b);
  }
}

__global__ void fp8w_dequant_kernel(int64_t N, int64_t K, const uint8_t* __restrict__ w,
                                    const float* __restrict__ s, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * K) return;
  const int64_t n = i / K;
  out[i] = e4m3_byte_f32<0>((uint32_t)w[i]) * s[n];
}

__global__ void nvfp4_dequant_kernel(int64_t N, int64_t K, const uint8_t* __restrict__ blk, float inv,
                                     float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one byte = two weights
  if (i >= N * K / 2) return;
  const int64_t n = (2 * i) / K, k = (2 * i) - n * K;
  const uint8_t* rec = blk + (n * (K / 64) + k / 64) * 36;
  const int kk = (int)(k & 63);
  const float d = e4m3_byte_f32<0>((uint32_t)rec[kk / 16]);
  const f32x2 v = e2m1x2_f32<0>((uint32_t)rec[4 + kk / 2]);
  out[n * K + k] = (v.x * d) * inv;      // e2m1 * e4m3 is exact; one rounding by inv
  out[n * K + k + 1] = (v.y * d) * inv;
}

template <int ML>
__global__ void awq_dequant_kernel(int64_t E, int64_t N, int64_t K, const uint8_t* __restrict__ bank,
                                   AwqLayout L, uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // one dword of codes = 8 weights
  const int64_t per_e = N * K / 8;
  if (i >= E * per_e) return;
  const int64_t e = i / per_e, rem = i - e * per_e;
  const int64_t n = rem / (K / 8), k8 = rem - n * (K / 8);
  const uint8_t* ex = bank + e * L.expert_bytes;
  const uint32_t w = reinterpret_cast<const uint32_t*>(ex)[(n * K) / 8 + k8];
  const int64_t mi = n * L.G + (k8 * 8) / 32;
  const _Float16 s = f16_from_bits(reinterpret_cast<const uint16_t*>(ex + L.scale_off)[mi]);
  _Float16 b;
  if constexpr (ML == 3) b = awq_bias(ex[L.meta2_off + mi], s);
  else b = f16_from_bits(reinterpret_cast<const uint16_t*>(ex + L.meta2_off)[mi]);
  const f16x2 s2 = {s, s}, b2 = {b, b};
  // pair t holds (local k = t, local k = t + 4); reorder to k = 0..7
  const uint32_t p0 = as_u32(awq_pair<0>(w, s2, b2));
  const uint32_t p1 = as_u32(awq_pair<1>(w, s2, b2));
  const uint32_t p2 = as_u32(awq_pair<2>(w, s2, b2));
  const uint32_t p3 = as_u32(awq_pair<3>(w, s2, b2));
  u32x4 o;
  o.x = (p0 & 0xFFFFu) | (p1 << 16);
  o.y = (p2 & 0xFFFFu) | (p3 << 16);
  o.z = (p0 >> 16) | (p1 & 0xFFFF0000u);
  o.w = (p2 >> 16) | (p3 & 0xFFFF0000u);
  *reinterpret_cast<u32x4*>(out + ((e * N + n) * K + k8 * 8)) = o;
}

inline unsigned blocks_for(int64_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

}  // namespace

hipError_t launch_nvfp4_pack(int64_t N, int64_t K, const uint8_t* wp, const uint8_t* ws, uint8_t* blk,
                             hipStream_t st) {
  const int64_t nb = K / 64;
  hipLaunchKernelGGL(nvfp4_pack_kernel, dim3(blocks_for(N * nb, 256)), dim3(256), 0, st, N, nb, wp, ws, blk);
  return hipGetLastError();
}

hipError_t launch_awq_pack(int64_t E, int64_t N, int64_t K, const uint8_t* codes, const uint16_t* scales,
                           const uint8_t* zeros, int meta_layout, uint8_t* bank, hipStream_t st) {
  const AwqLayout L = awq_layout(N, K, meta_layout);
  const int64_t per_e = N * K / 2;
  hipLaunchKernelGGL(awq_pack_codes_kernel, dim3(blocks_for(E * per_e, 256)), dim3(256), 0, st, E * per_e, codes,
                     bank, per_e, L.expert_bytes);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t per_g = N * L.G;
  hipLaunchKernelGGL(awq_pack_meta_kernel, dim3(blocks_for(E * per_g, 256)), dim3(256), 0, st, E * per_g, per_g,
                     scales, zeros, meta_layout, bank, L);
  return hipGetLastError();
}

hipError_t launch_fp8w_dequant(int64_t N, int64_t K, const uint8_t* w, const float* s, float* out,
                               hipStream_t st) {
  hipLaunchKernelGGL(fp8w_dequant_kernel, dim3(blocks_for(N * K, 256)), dim3(256), 0, st, N, K, w, s, out);
  return hipGetLastError();
}

hipError_t launch_nvfp4_dequant(int64_t N, int64_t K, const uint8_t* blk, float inv, float* out,
                                hipStream_t st) {
  hipLaunchKernelGGL(nvfp4_dequant_kernel, dim3(blocks_for(N * K / 2, 256)), dim3(256), 0, st, N, K, blk, inv,
                     out);
  return hipGetLastError();
}

hipError_t launch_awq_dequant(int64_t E, int64_t N, int64_t K, const uint8_t* bank, int meta_layout,
                              uint16_t* out, hipStream_t st) {
  const AwqLayout L = awq_layout(N, K, meta_layout);
  const int64_t n = E * N * K / 8;
  if (meta_layout == 3)
    hipLaunchKernelGGL(awq_dequant_kernel<3>, dim3(blocks_for(n, 256)), dim3(256), 0, st, E, N, K, bank, L, out);
  else
    hipLaunchKernelGGL(awq_dequant_kernel<4>, dim3(blocks_for(n, 256)), dim3(256), 0, st, E, N, K, bank, L, out);
  return hipGetLastError();
}

}  // namespace wq
