// MFMA path: LDS-tiled MFMA GEMMs with in-kernel weight decode (gfx950).
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
//     float32.  FP8: act is stored as float32 (the FP8 definition keeps act unrounded
//     between the two projections) and the down GEMM's operand is made from it by the
//     same exact power-of-two row scaling as x, so no act value can overflow float16.
//     NVFP4: act is rounded once to float16 (|act| < 65504 required);
//   * down: acc * (act row scale, FP8) * (1/global_scale or channel scale), stored as
//     float32.
//
// Tiling (both kernels): a workgroup of 4 waves computes a (32*MB) x 128 output tile (of both gate and
// up for the fused projection).  All waves share the activation tile, staged in LDS; each wave owns 32
// output columns and decodes its own weight fragments into registers, so every decoded fragment feeds
// MB (x2 with gate+up) MFMAs.  K is walked in steps of 64.
//
// Copy-fed GEMM (nv_gemm_kernel, both formats, K >= 256 for NVFP4 and K >= 128 for FP8): a lane-per-
// column load of weight bytes touches one cache line per lane, and that access pattern, not bandwidth,
// limited the register-load form (mfma_gemm_kernel, kept for shorter K).  Here both operands move by
// direct global->LDS copies (global_load_lds_dwordx4) in a coalesced order: the activation tile
// (128-byte rows, 16-byte chunk c of row r stored at chunk c ^ ((r >> 1) & 7): with 64 four-byte banks,
// rows two apart share banks, and this swizzle gives the 8 rows of each parity among 16 consecutive lanes
// 8 distinct chunks; c ^ (r & 7) gives them 4, and measured the same within 0.4%) in a 2-stage ring, and the weights in blocks per column (NVFP4: 4 records = 144
// contiguous bytes; FP8: 2 K steps = 128 code bytes, chunk-swizzled), one block buffer per wave.  At
// the start of a block each wave reads the whole block of its columns into registers and immediately
// refills the buffer with the next block, so the weight copy has the block's K steps to land.  Inside
// a K step the activation fragments of sub-step s+1 are read while the MFMAs of sub-step s run; the
// single barrier per K step sits after the third sub-step.  Two workgroups share a CU (at most 72 KB of
// LDS each).  Batches of at most 32 or 64 rows run 32- or 64-row tiles (MB = 1, 2), so a short batch
// streams the weights once with little padding; the split-K plan below then spreads the few tiles over
// the chip.  A 32-row tile's K step is too short to cover a memory round trip, so those tiles copy the
// activations of a whole block with its weights and wait once per block (block schedule).
//
// MFMA v_mfma_f32_32x32x16_f16 operand layout (checked on gfx950): A lane l holds row
// l%32, k = 8*(l/32) + j; B lane l holds column l%32, same k; D register r of lane l
// is (row 8*(r/4) + 4*(l/32) + r%4, column l%32).  Within a 64-wide K step, step s
// (0..3) feeds the instruction k' = 8*(l/32) + j with the logical k = 32*(l/32) +
// 8*s + j, for both operands, so each lane's weight bytes for a whole record are one
// contiguous 16-byte (NVFP4) or 32-byte (FP8) load.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "dev_common.h"
#include "launch.h"

namespace wq {

namespace {

constexpr int kLdsRow = 144;  // 64 f16 + 16 bytes padding
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

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

// One wave per row: the row is read once in 16-byte chunks (8 bf16 or 4 float32 per chunk) and kept in
// registers (up to RC chunks per lane; rows longer than 64*RC chunks re-read the rest from memory),
// reduced to max |x| across the wave, then scaled and written as float16 chunks.
// Power-of-two row scale e: max |x| * 2^-e lies in [2^14, 2^15).
template <typename XT>
struct RowChunk;
template <>
struct RowChunk<uint16_t> {   // 8 bf16
  static constexpr int E = 8;
  static __device__ __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(v[i] << 16);
      f[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct RowChunk<float> {      // 4 float32
  static constexpr int E = 4;
  static __device__ __forceinline__ void unpack(u32x4 v, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(v[i]);
  }
};

// Power-of-two row scale e: max |x| * 2^-e lies in [2^14, 2^15) (e = 0 for a zero or non-finite max).
__device__ __forceinline__ int row_pow2_exp(float amax) {
  int e = 0;
  if (amax > 0.f && amax <= 3.0e38f) {
    int ex;
    (void)frexpf(amax, &ex);   // amax = f * 2^ex, f in [0.5, 1)
    e = ex - 15;                // amax * 2^-e in [2^14, 2^15)
    e = e < -100 ? -100 : (e > 100 ? 100 : e);
  }
  return e;
}
template <typename XT>
__device__ __forceinline__ float chunk_absmax(u32x4 v, float amax) {
  constexpr int E = RowChunk<XT>::E;
  float f[E];
  RowChunk<XT>::unpack(v, f);
#pragma unroll
  for (int j = 0; j < E; ++j) amax = fmaxf(amax, fabsf(f[j]));
  return amax;
}
// Chunk c of a row, scaled by 2^-e and rounded to float16, stored at chunk c of the float16 row o.
template <typename XT>
__device__ __forceinline__ void put_scaled(uint16_t* o, int c, u32x4 v, int e) {
  constexpr int E = RowChunk<XT>::E;
  float f[E];
  RowChunk<XT>::unpack(v, f);
  uint32_t hh[E / 2];
#pragma unroll
  for (int j = 0; j < E / 2; ++j) {
    const _Float16 lo = (_Float16)ldexpf(f[2 * j], -e), hi = (_Float16)ldexpf(f[2 * j + 1], -e);
    hh[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
  }
  if constexpr (E == 8) reinterpret_cast<u32x4*>(o)[c] = u32x4{hh[0], hh[1], hh[2], hh[3]};
  else reinterpret_cast<u32x2*>(o)[c] = u32x2{hh[0], hh[1]};
}

template <typename XT, int RC>
__global__ void __launch_bounds__(256) rowscale_f16_kernel(int M, int K, const XT* __restrict__ x,
                                                           uint16_t* __restrict__ x16,
                                                           float* __restrict__ rowscale) {
  constexpr int E = RowChunk<XT>::E;
  const int m = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
  if (m >= M) return;
  const int lane = threadIdx.x & 63;
  const int nch = K / E;                               // K is a multiple of 64
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + (size_t)m * K);
  u32x4 cache[RC];
#pragma unroll
  for (int i = 0; i < RC; ++i) {
    const int c = lane + 64 * i;
    cache[i] = c < nch ? xr[c] : u32x4{0u, 0u, 0u, 0u};
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < RC; ++i) amax = chunk_absmax<XT>(cache[i], amax);
  for (int c = lane + 64 * RC; c < nch; c += 64) amax = chunk_absmax<XT>(xr[c], amax);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  const int e = row_pow2_exp(amax);
  if (lane == 0) rowscale[m] = ldexpf(1.0f, e);
  uint16_t* o = x16 + (size_t)m * K;
#pragma unroll
  for (int i = 0; i < RC; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) put_scaled<XT>(o, c, cache[i], e);
  }
  for (int c = lane + 64 * RC; c < nch; c += 64) put_scaled<XT>(o, c, xr[c], e);
}

// Long rows (the MLP's act, K = intermediate): one 256-thread workgroup per row, RC chunks per thread
// kept in registers (the rest re-read), the row max reduced across each wave and then across the four
// waves through LDS.  Same scale and rounding as rowscale_f16_kernel.
template <typename XT, int RC>
__global__ void __launch_bounds__(256) rowscale_f16_wg_kernel(int M, int K, const XT* __restrict__ x,
                                                              uint16_t* __restrict__ x16,
                                                              float* __restrict__ rowscale) {
  constexpr int E = RowChunk<XT>::E;
  __shared__ float wmax[4];
  const int m = (int)blockIdx.x;
  const int t = (int)threadIdx.x;
  const int nch = K / E;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + (size_t)m * K);
  u32x4 cache[RC];
#pragma unroll
  for (int i = 0; i < RC; ++i) {
    const int c = t + 256 * i;
    cache[i] = c < nch ? xr[c] : u32x4{0u, 0u, 0u, 0u};
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < RC; ++i) amax = chunk_absmax<XT>(cache[i], amax);
  for (int c = t + 256 * RC; c < nch; c += 256) amax = chunk_absmax<XT>(xr[c], amax);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((t & 63) == 0) wmax[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int e = row_pow2_exp(amax);
  if (t == 0) rowscale[m] = ldexpf(1.0f, e);
  uint16_t* o = x16 + (size_t)m * K;
#pragma unroll
  for (int i = 0; i < RC; ++i) {
    const int c = t + 256 * i;
    if (c < nch) put_scaled<XT>(o, c, cache[i], e);
  }
  for (int c = t + 256 * RC; c < nch; c += 256) put_scaled<XT>(o, c, xr[c], e);
}

// ---- the GEMM ------------------------------------------------------------------------------------
// lds_copy16_run with the non-temporal hint on every copy (runs of 4 in one M0 write, shorter runs copy by
// copy): for weight blocks that exactly one workgroup reads.
template <int N>
__device__ __forceinline__ void lds_copy16_run_nt(const uint32_t* v, const uint8_t* const* b, uint32_t lds_base) {
  static_assert(N >= 1 && N <= 4, "run length");
  if constexpr (N == 4) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
    asm volatile(
        "s_mov_b32 m0, %8\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %4 nt\n\t"
        "global_load_lds_dwordx4 %1, %5 offset:1024 nt\n\tglobal_load_lds_dwordx4 %2, %6 offset:2048 nt\n\t"
        "global_load_lds_dwordx4 %3, %7 offset:3072 nt" ::"v"(v[0]),
        "v"(v[1]), "v"(v[2]), "v"(v[3]), "s"(b[0]), "s"(b[1]), "s"(b[2]), "s"(b[3]), "s"(lds_base)
        : "memory", "m0");
#pragma clang diagnostic pop
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) lds_copy16_nt(v[k], b[k] + 1024 * k, lds_base + 1024 * k);
  }
}
// FMT 0: FP8 E4M3 codes [N][K], per-column scale cs[n].  FMT 1: NVFP4 Block64 [N][K/64], factor inv.
// GU: two weight matrices, out = act [M][N] (float32 for FP8, float16 for NVFP4); else one matrix,
// out = f32 y [M][N].
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
  // lanes past the last column (N not a multiple of 32) load row N-1 and store nothing
  const int wcol = min(ncol, N - 1);

  const uint8_t* wrow[NM];
  {
    const size_t rb = FMT == 1 ? (size_t)(K >> 6) * 36 : (size_t)K;
    wrow[0] = w0 + (size_t)(wave_on ? wcol : 0) * rb;
    if constexpr (GU) wrow[1] = w1 + (size_t)(wave_on ? wcol : 0) * rb;
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

  if (!wave_on || ncol >= N) return;
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
          const float a = silu_f32(g) * u;
          if constexpr (FMT == 0) reinterpret_cast<float*>(out)[(size_t)m * N + ncol] = a;   // FP8: float32 act
          else reinterpret_cast<uint16_t*>(out)[(size_t)m * N + ncol] = __builtin_bit_cast(uint16_t, (_Float16)a);
        } else {
          reinterpret_cast<float*>(out)[(size_t)m * N + ncol] = acc[0][mb][r] * rs * cf[0];
        }
      }
    }
  }
}

// ---- NVFP4: operands by global->LDS copy (lds_copy16 / wait_vmem / wait_lds in dev_common.h) -----

// Weight blocks of the copy-fed GEMM, by format: KSB K steps (64 k each) per block, CB bytes of one
// column per block, CPM copy instructions per matrix and wave (32 columns), MBYTES of LDS per matrix and
// wave.  NVFP4 (FMT 1): 4 Block64 records = 144 bytes = 9 chunks per column (288 slots, 32 pad slots).
// FP8 (FMT 0): 2 K steps = 128 code bytes = 8 chunks per column (256 slots).
template <int FMT> struct WGeo;
template <> struct WGeo<1> { static constexpr int KSB = 4, CB = 144, CPM = 5, MBYTES = 5120; };
template <> struct WGeo<0> { static constexpr int KSB = 2, CB = 128, CPM = 4, MBYTES = 4096; };
// MB = 1, 2, 4: 32-, 64- or 128-row tiles
constexpr int nv_astage(int mb) { return 32 * mb * 128; }   // bytes per activation stage
template <int FMT> constexpr int g_wave_wbytes(bool gu) { return (gu ? 2 : 1) * WGeo<FMT>::MBYTES; }
// Activation stages in the LDS ring: 2 (one per K step, stepped schedule) or two blocks' worth (block
// schedule)
template <int FMT> constexpr int g_astages(bool bs) { return bs ? 2 * WGeo<FMT>::KSB : 2; }
template <int FMT> constexpr int g_lds_bytes(bool gu, int mb, bool bs) {
  return g_astages<FMT>(bs) * nv_astage(mb) + 4 * g_wave_wbytes<FMT>(gu);
}
// Smallest K the copy-fed GEMM takes (the short last block is copied as the row's last CB bytes).
constexpr int g_min_k(int fmt) { return fmt == 1 ? 256 : 128; }
// Tile rows / 32 for an M-row launch.  The down projection (long K, short N) keeps 32-row tiles up to
// M = 96 (re-reading its weights once per 32 rows costs less than the stepped schedule's waits) and takes
// 64-row tiles up to 128 (at M=128: 38 us in 6 parts against 42 us for 32-row tiles in 3).
inline int nv_mb(int M, bool gu) {
  if (!gu && M <= 96) return 1;
  if (!gu && M <= 128) return 2;
  return M <= 32 ? 1 : (M <= 64 ? 2 : 4);
}

// Work plan of one launch, a pure function of the shape.  (32*MB)x128 tiles; with two workgroups on each
// of the 256 CUs there are 512 slots.  When the last round of tiles would leave most slots idle (or
// there are fewer tiles than slots at all) the tiles of that round are split along K into S parts of
// whole weight blocks: the parts run first, store raw float32 partial tiles, and a second
// kernel adds the S parts of every element in part order and applies the epilogue.  The sum order
// is fixed by the shape, so results are reproducible.
constexpr int kNvSlots = 512;
constexpr size_t kNvMaxPartials = (size_t)64 << 20;
struct NvPlan {
  int bm;                // tile rows: 32 * MB
  int ntm, ntn, tiles;   // tile grid
  int full;              // tiles [0, full) run whole
  int S, bps;            // split tiles [full, tiles) run as S parts of bps blocks (S = 1: none)
  int units, units_grid; // (tiles - full) * S parts; rounded up to a multiple of 8
};
// ksb: K steps per weight block; slots: concurrent workgroups; smax: most K parts per tile; mb: tile rows
// / 32 (0: nv_mb(M))
inline NvPlan nv_plan_ex(int M, int K, int N, bool gu, int ksb, int slots, int smax, int mb = 0) {
  NvPlan p{};
  p.bm = 32 * (mb > 0 ? mb : nv_mb(M, gu));
  p.ntm = (M + p.bm - 1) / p.bm;
  p.ntn = (N + 127) / 128;
  p.tiles = p.ntm * p.ntn;
  const int nblk = (K / 64 + ksb - 1) / ksb;
  int tail = 0;
  {
    if (p.tiles < slots) {
      tail = p.tiles;
    } else {
      const int rounds = (p.tiles + slots - 1) / slots;
      tail = p.tiles - (rounds - 1) * slots;
      if (tail * 10 >= slots * 9) tail = 0;   // a nearly full last round runs whole
    }
  }
  // S: when at least two parts of every tail tile fit one round of slots, the most that do (a second
  // round of parts measured slower: M=64 gate+up 65 us for 7 parts in two rounds against 48 us for 3 in
  // one); otherwise S minimises the rounds of parts per tile, ceil(tail * S / slots) / S (ties: fewer
  // parts).  The partial scratch stays within kNvMaxPartials either way.
  int S = 1;
  if (tail > 0) {
    const size_t per_part = (size_t)(gu ? 2 : 1) * p.bm * 128 * 4;
    const int one_round = std::min(std::min(smax, nblk), slots / tail);
    if (one_round >= 2) {
      S = one_round;
      while (S > 1 && (size_t)tail * S * per_part > kNvMaxPartials) --S;
    } else {
      double best = 1.0;
      for (int s = 2; s <= std::min(smax, nblk); ++s) {
        if ((size_t)tail * s * per_part > kNvMaxPartials) break;
        const double t = (double)((tail * s + slots - 1) / slots) / s;
        if (t < best - 1e-9) { best = t; S = s; }
      }
    }
  }
  if (S < 2) { tail = 0; S = 1; }
  p.bps = (nblk + S - 1) / S;
  p.S = S > 1 ? (nblk + p.bps - 1) / p.bps : 1;   // no empty parts
  p.full = p.tiles - tail;
  p.units = tail * p.S;
  p.units_grid = (p.units + 7) / 8 * 8;
  return p;
}
// At most 8 K parts per tile, 16 for the single projection's 32-row tiles: its few, long-K tiles (40 at
// N = 5120) run 12 parts in one round of slots (measured at K = 17408, M <= 32: 16.5 us against 20.7 us for
// 8 parts, finish included either way within 0.1 us).
inline NvPlan nv_plan(int fmt, int M, int K, int N, bool gu) {
  const int smax = (!gu && nv_mb(M, gu) == 1) ? 16 : 8;
  return nv_plan_ex(M, K, N, gu, fmt == 1 ? WGeo<1>::KSB : WGeo<0>::KSB, kNvSlots, smax);
}
inline size_t nv_partial_bytes(const NvPlan& p, bool gu) {
  return (size_t)p.units * (gu ? 2 : 1) * p.bm * 128 * 4;
}

// FMT 1: NVFP4 Block64 weights, column factor inv0 / inv1.  FMT 0: FP8 E4M3 codes [N][K], column scales
// cs0[n] / cs1[n].  ABF (FMT 0 only): a16 holds bfloat16 activations as given (no row scale) and the
// MFMAs run on bf16 operands (E4M3 codes decode to bf16 exactly); otherwise both operands are f16.
// A32 (gate+up): act is stored as float32 (FP8, whose definition keeps act unrounded, and the W4A8 variant,
// which quantizes it per token next), else as float16.
template <int FMT, bool GU, int MB, bool BS, bool ABF, bool A32>
__global__ void __launch_bounds__(256, 2) nv_gemm_kernel(int M, int K, int N, NvPlan plan,
                                                        const uint16_t* __restrict__ a16,
                                                        const float* __restrict__ rowscale,
                                                        const uint8_t* __restrict__ w0, const float* __restrict__ cs0,
                                                        float inv0, const uint8_t* __restrict__ w1,
                                                        const float* __restrict__ cs1, float inv1,
                                                        void* __restrict__ out, float* __restrict__ partials) {
  static_assert(!ABF || FMT == 0, "bf16 operands: FP8 weights only");
  using Geo = WGeo<FMT>;
  using AFrag = std::conditional_t<ABF, bf16x8, f16x8>;   // 8 activations (or weights) of one MFMA operand
  constexpr int KSB = Geo::KSB, CB = Geo::CB, CPM = Geo::CPM, MBYTES = Geo::MBYTES;
  constexpr int NM = GU ? 2 : 1;
  constexpr int kNvAStage = nv_astage(MB);
  constexpr int AS = g_astages<FMT>(BS);
  constexpr int AMASK = AS - 1;                // stage of K step kt under the block schedule: kt & AMASK
  constexpr int PT = 32 * MB * 128;            // elements of one partial tile per matrix
  constexpr int NW = NM * CPM;                 // weight copies per wave per block
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int nk = K >> 6;
  const int nblk = (nk + KSB - 1) / KSB;
  // Workgroups [0, units_grid) run the K parts of the split tiles (dispatched first, so they finish
  // early); the rest run whole tiles in an XCD-aware order: workgroup b runs on XCD b % 8, and each XCD
  // gets a contiguous run of tiles (n fastest) so the activation band it works on stays in its L2.
  const int b = (int)blockIdx.x;
  int tile, part = -1, kb0 = 0, kb1 = nblk;
  if (b < plan.units_grid) {
    if (b >= plan.units) return;
    tile = plan.full + b / plan.S;
    part = b - (b / plan.S) * plan.S;
    kb0 = part * plan.bps;
    kb1 = min(kb0 + plan.bps, nblk);
  } else {
    const int f = b - plan.units_grid;
    const int per = ((int)gridDim.x - plan.units_grid) >> 3;
    tile = (f & 7) * per + (f >> 3);
    if (tile >= plan.full) return;
  }
  const int kt0 = KSB * kb0, kt1 = min(KSB * kb1, nk);
  const int ntn = plan.ntn;
  const int tm = tile / ntn;
  const int tn = tile - tm * ntn;
  const int m0 = tm * 32 * MB;
  const int n0 = tn * 128;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;
  const int h = lane >> 5;
  const uint32_t rb = FMT == 1 ? (uint32_t)nk * 36u : (uint32_t)K;   // bytes per weight row
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  const uint32_t wlds = lds0 + AS * kNvAStage + wave * g_wave_wbytes<FMT>(GU);
  const uint8_t* wbuf = lds + AS * kNvAStage + wave * g_wave_wbytes<FMT>(GU);

  // Activation chunk p = 64 MB wave + 64 i + lane (copy i of the wave): tile row p >> 3, LDS chunk p & 7,
  // global chunk (p & 7) ^ ((row >> 1) & 7).  A wave's MB copies are consecutive kilobytes of the stage, so they go
  // out as one run with one M0 write.  Offsets are relative to the tile's first row (64-bit base), so they
  // stay below 32 * MB * K * 2 bytes.
  const uint8_t* a_tile = reinterpret_cast<const uint8_t*>(a16) + (size_t)m0 * K * 2;
  uint32_t aoff[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int p = 64 * MB * wave + 64 * i + lane, row = p >> 3, c = p & 7;
    aoff[i] = (uint32_t)(min(m0 + row, M - 1) - m0) * (uint32_t)K * 2u + (uint32_t)((c ^ ((row >> 1) & 7)) * 16);
  }
  // Weight copy j = CPM t + i of matrix t writes LDS slot s = 64 i + lane of the matrix's block buffer
  // (wbuf + MBYTES t).  NVFP4: column c = s / 9, chunk q = s % 9 of the column's 144-byte block (slots
  // 288..319 re-read chunks of slots 0..31), the column's block at 144 c.  FP8: column c = s / 8, slot
  // position p = s % 8 holds chunk p ^ ((c / 2) % 8) of the column's 128-byte block (a swizzle that keeps
  // the 16-byte fragment reads of 16 consecutive columns on distinct banks), the column's block at 128 c.
  // Offsets are relative to the wave's first column row (64-bit bases), so they stay below 32 rows.
  const int nw0 = min(n0 + 32 * wave, N - 1);
  const uint8_t* wbase0 = w0 + (size_t)nw0 * rb;
  const uint8_t* wbase1 = GU ? w1 + (size_t)nw0 * rb : wbase0;
  uint32_t woff[NW];
#pragma unroll
  for (int j = 0; j < NW; ++j) {
    int s = 64 * (j % CPM) + lane;
    int c, q;
    if constexpr (FMT == 1) {
      if (s >= 288) s -= 288;
      c = s / 9;
      q = s - 9 * c;
    } else {
      c = s >> 3;
      q = (s & 7) ^ ((c >> 1) & 7);
    }
    woff[j] = (uint32_t)(min(n0 + 32 * wave + c, N - 1) - nw0) * rb + 16u * (uint32_t)q;
  }
  // Copy i of a wave moves tile rows 8 MB wave + 8 i .. + 7.  Under the block schedule (32-row tiles, one
  // copy per wave, which waits for all of a wave's copies at once) a copy whose rows all lie past M is
  // skipped: those rows' outputs are never stored, so their LDS rows may hold anything.  The stepped
  // schedule counts copies in its waits and always issues them.
  auto copy_a = [&](int kt, int stage) {
    kt = min(kt, nk - 1);
    const uint8_t* base = a_tile + (size_t)kt * 128;
    const uint32_t sb = __builtin_amdgcn_readfirstlane(lds0 + stage * kNvAStage + 1024 * MB * wave);
    const uint8_t* bases[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i) bases[i] = base - 1024 * i;
    if (!BS || m0 + 8 * MB * wave < M) lds_copy16_run<MB>(aoff, bases, sb);
  };
  // A row whose K-step count r = nk % KSB is not 0 ends in a short block: it is copied as the last CB
  // bytes of the row (steps KSB - r .. KSB - 1 of the window are the valid ones; K >= g_min_k, so the
  // window starts inside the row) and read_block moves those steps down to positions 0 .. r-1.
  const int rtail = nk % KSB;
  // FP8 weight blocks of a plan with one row of tiles are read by exactly one workgroup and are whole
  // 128-byte lines (128 code bytes per column; rows start on a line when K and the matrix base are
  // multiples of 128 bytes): those copies carry the non-temporal hint (FP8, M = 8: 69.9 -> 65.0 us per
  // step).  NVFP4 blocks (144 bytes) share a line with the next block of the column, which the hint would
  // fetch twice (NVFP4, M = 8: 57.8 -> 62.6 us).
  const bool w_nt = FMT == 0 && BS && plan.ntm == 1 && (K & 127) == 0 && (((uintptr_t)w0 & 127) == 0) &&
                    (!GU || ((uintptr_t)w1 & 127) == 0);
  auto copy_w = [&](int blk) {
    blk = min(blk, nblk - 1);
    const uint32_t boff = (rtail && blk == nblk - 1) ? rb - (uint32_t)CB : (uint32_t)blk * CB;
    // runs of up to four copies, each run with one M0 write (copy j lands at wlds + 1024 j)
    uint32_t v[NW];
    const uint8_t* bases[NW];
#pragma unroll
    for (int j = 0; j < NW; ++j) {
      v[j] = woff[j] + boff;
      bases[j] = (j < CPM ? wbase0 : wbase1) - 1024 * (j & 3);
    }
#pragma unroll
    for (int g = 0; g < NW; g += 4) {
      const uint32_t lb = __builtin_amdgcn_readfirstlane(wlds + 1024 * g);
      if (w_nt) {
        if (g + 4 <= NW) lds_copy16_run_nt<4>(v + g, bases + g, lb);
        else lds_copy16_run_nt<(NW % 4 == 0 ? 4 : NW % 4)>(v + g, bases + g, lb);
      } else {
        if (g + 4 <= NW) lds_copy16_run<4>(v + g, bases + g, lb);
        else lds_copy16_run<(NW % 4 == 0 ? 4 : NW % 4)>(v + g, bases + g, lb);
      }
    }
  };

  f32x16 acc[NM][MB];
#pragma unroll
  for (int t = 0; t < NM; ++t)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[t][mb][r] = 0.f;

  // Registers of one weight block for this lane's column of matrix t.  NVFP4: record J's scale dword and
  // the 16 nibble bytes of its half h (bytes 36 J + 4 + 16 h .. + 15 of the block).  FP8: the code bytes of
  // K step J, half h (bytes 64 J + 32 h .. + 31), as two chunks.
  struct WBlockNv { uint32_t nib[4][4]; uint32_t d[4]; };
  struct WBlockF8 { u32x4 c[2][2]; };
  using WBlock = std::conditional_t<FMT == 1, WBlockNv, WBlockF8>;
  auto shift_block = [&](WBlock* wb, auto Sc) {   // step J <- step J + S
    constexpr int S = decltype(Sc)::value;
#pragma unroll
    for (int t = 0; t < NM; ++t)
#pragma unroll
      for (int J = 0; J + S < KSB; ++J) {
        if constexpr (FMT == 1) {
          wb[t].d[J] = wb[t].d[J + S];
#pragma unroll
          for (int e = 0; e < 4; ++e) wb[t].nib[J][e] = wb[t].nib[J + S][e];
        } else {
          wb[t].c[J][0] = wb[t].c[J + S][0];
          wb[t].c[J][1] = wb[t].c[J + S][1];
        }
      }
  };
  auto read_block = [&](WBlock* wb, int blk) {
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      if constexpr (FMT == 1) {
        const uint8_t* bp = wbuf + MBYTES * t + 144 * li;
#pragma unroll
        for (int J = 0; J < 4; ++J) wb[t].d[J] = *reinterpret_cast<const uint32_t*>(bp + 36 * J);
        u32x4 P = *reinterpret_cast<const u32x4*>(bp + 16 * h);          // record 0: chunks h, h+1
        u32x4 Q = *reinterpret_cast<const u32x4*>(bp + 16 * (1 + h));
        wb[t].nib[0][0] = P.y; wb[t].nib[0][1] = P.z; wb[t].nib[0][2] = P.w; wb[t].nib[0][3] = Q.x;
        P = *reinterpret_cast<const u32x4*>(bp + 16 * (2 + h));               // record 1: chunks 2+h, 3+h
        Q = *reinterpret_cast<const u32x4*>(bp + 16 * (3 + h));
        wb[t].nib[1][0] = P.z; wb[t].nib[1][1] = P.w; wb[t].nib[1][2] = Q.x; wb[t].nib[1][3] = Q.y;
        P = *reinterpret_cast<const u32x4*>(bp + 16 * (4 + h));               // record 2: chunks 4+h, 5+h
        Q = *reinterpret_cast<const u32x4*>(bp + 16 * (5 + h));
        wb[t].nib[2][0] = P.w; wb[t].nib[2][1] = Q.x; wb[t].nib[2][2] = Q.y; wb[t].nib[2][3] = Q.z;
        P = *reinterpret_cast<const u32x4*>(bp + 16 * (7 + h));               // record 3: chunk 7+h
        wb[t].nib[3][0] = P.x; wb[t].nib[3][1] = P.y; wb[t].nib[3][2] = P.z; wb[t].nib[3][3] = P.w;
      } else {
        const uint8_t* bp = wbuf + MBYTES * t + 128 * li;
        const int sw = (li >> 1) & 7;
#pragma unroll
        for (int J = 0; J < 2; ++J)
#pragma unroll
          for (int e = 0; e < 2; ++e)
            wb[t].c[J][e] = *reinterpret_cast<const u32x4*>(bp + 16 * ((4 * J + 2 * h + e) ^ sw));
      }
    }
    if (rtail && blk == nblk - 1) {
      if constexpr (FMT == 1) {
        if (rtail == 1) shift_block(wb, std::integral_constant<int, 3>{});
        else if (rtail == 2) shift_block(wb, std::integral_constant<int, 2>{});
        else shift_block(wb, std::integral_constant<int, 1>{});
      } else {
        shift_block(wb, std::integral_constant<int, 1>{});
      }
    }
  };
  auto read_a = [&](int stage, int s, AFrag* af) {
    const uint8_t* ast = lds + stage * kNvAStage;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      af[mb] = *reinterpret_cast<const AFrag*>(ast + (32 * mb + li) * 128 + (((4 * h + s) ^ ((li >> 1) & 7)) * 16));
  };
  // decode sub-step s of step J into exact f16 (NVFP4: E2M1 x E4M3 group scale; FP8: the E4M3 codes)
  // and run its MFMAs
  auto mfmas = [&](const WBlock* wb, int J, int s, const AFrag* af) {
    AFrag bfr[NM];
#pragma unroll
    for (int t = 0; t < NM; ++t) {
      if constexpr (ABF) {                                             // FP8 codes -> exact bf16
        const u32x4 ch = wb[t].c[J][s >> 1];
        const uint32_t wa = (s & 1) ? ch.z : ch.x, wb2 = (s & 1) ? ch.w : ch.y;
        const bf16x2 q0 = e4m3x2_bf16<false>(wa), q1 = e4m3x2_bf16<true>(wa);
        const bf16x2 q2 = e4m3x2_bf16<false>(wb2), q3 = e4m3x2_bf16<true>(wb2);
        bfr[t] = bf16x8{q0.x, q0.y, q1.x, q1.y, q2.x, q2.y, q3.x, q3.y};
        continue;
      }
      f16x2 p0, p1, p2, p3;
      if constexpr (FMT == 1) {
        const f16x2 dsc = e4m3x2_f16<false>(wb[t].d[J] >> (16 * h));   // groups 2h, 2h+1
        const uint32_t w = wb[t].nib[J][s];
        const _Float16 g = (s < 2) ? dsc.x : dsc.y;
        const f16x2 gg = {g, g};
        p0 = e2m1x2_f16<0>(w) * gg;
        p1 = e2m1x2_f16<1>(w) * gg;
        p2 = e2m1x2_f16<2>(w) * gg;
        p3 = e2m1x2_f16<3>(w) * gg;
      } else {
        const u32x4 ch = wb[t].c[J][s >> 1];                           // bytes 8 s .. 8 s + 7 of the half
        const uint32_t wa = (s & 1) ? ch.z : ch.x, wb2 = (s & 1) ? ch.w : ch.y;
        p0 = e4m3x2_f16<false>(wa);
        p1 = e4m3x2_f16<true>(wa);
        p2 = e4m3x2_f16<false>(wb2);
        p3 = e4m3x2_f16<true>(wb2);
      }
      if constexpr (!ABF) bfr[t] = AFrag{p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int t = 0; t < NM; ++t) {
        if constexpr (ABF) acc[t][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[t], acc[t][mb], 0, 0, 0);
        else acc[t][mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[mb], bfr[t], acc[t][mb], 0, 0, 0);
      }
#pragma unroll
    for (int i = 0; i < MB * NM; ++i) {      // one MFMA, one fragment read, two ALU ops at a time
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < MB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    }
  };

  WBlock wb[NM];
  AFrag af0[MB], af1[MB];
  if constexpr (!BS) {
    // Stepped schedule (128-row tiles: a K step's MFMAs are long enough to cover an activation copy).
    // Prologue: weight block 0, activation steps 0 and 1; wait for block 0 and step 0 (step 1 may fly),
    // read block 0 into registers and refill the buffer with block 1.
    copy_w(kb0);
    copy_a(kt0, 0);
    copy_a(kt0 + 1, 1);
    wait_vmem<MB>();
    __syncthreads();
    read_block(wb, kb0);
    wait_lds();
    copy_w(kb0 + 1);
    read_a(0, 0, af0);
    // K step kt (stage kt & 1, step J of the block in registers).
    auto step = [&](int kt, auto Jc) {
      constexpr int J = decltype(Jc)::value;
      read_a(kt & 1, 1, af1);
      mfmas(wb, J, 0, af0);
      __builtin_amdgcn_sched_barrier(0);
      read_a(kt & 1, 2, af0);
      mfmas(wb, J, 1, af1);
      __builtin_amdgcn_sched_barrier(0);
      read_a(kt & 1, 3, af1);
      mfmas(wb, J, 2, af0);
      __builtin_amdgcn_sched_barrier(0);
      // Step kt+1's activations were copied at the previous barrier; at step 0 of a block the copy of the
      // next weight block (issued after them) may still be in flight.
      if constexpr (J == 0) wait_vmem<NW>();
      else wait_vmem<0>();
      __syncthreads();
      copy_a(kt + 2, kt & 1);                  // every wave is done with this stage
      read_a((kt + 1) & 1, 0, af0);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(wb, J, 3, af1);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (J == KSB - 1) {            // next block: complete since the wait above
        read_block(wb, kt / KSB + 1);
        wait_lds();
        copy_w(kt / KSB + 2);
      }
    };
    for (int kt = kt0; kt < kt1; kt += KSB) {   // kt0 is a multiple of KSB: step J = kt % KSB
      step(kt, std::integral_constant<int, 0>{});
      if (kt + 1 < kt1) step(kt + 1, std::integral_constant<int, 1>{});
      if constexpr (KSB == 4) {
        if (kt + 2 < kt1) step(kt + 2, std::integral_constant<int, 2>{});
        if (kt + 3 < kt1) step(kt + 3, std::integral_constant<int, 3>{});
      }
    }
  } else {
    // Block schedule (narrow tiles, whose K steps are too short to cover a memory round trip): the
    // activations of a whole KSB-step block are copied together with its weights, into a ring of two
    // blocks' stages (stage kt & AMASK), so the copies of block b+1 fly during all the steps of block b
    // and the wait and the barrier come once per block.
    auto copy_a_blk = [&](int blk) {
#pragma unroll
      for (int j = 0; j < KSB; ++j) copy_a(KSB * blk + j, (KSB * blk + j) & AMASK);
    };
    copy_w(kb0);
    copy_a_blk(kb0);
    wait_vmem<0>();
    __syncthreads();
    read_block(wb, kb0);
    wait_lds();
    if (kb0 + 1 < kb1) {
      copy_w(kb0 + 1);
      copy_a_blk(kb0 + 1);
    }
    read_a(kt0 & AMASK, 0, af0);
    auto bstep = [&](int kt, auto Jc) {
      constexpr int J = decltype(Jc)::value;
      const int st = kt & AMASK;
      read_a(st, 1, af1);
      mfmas(wb, J, 0, af0);
      __builtin_amdgcn_sched_barrier(0);
      read_a(st, 2, af0);
      mfmas(wb, J, 1, af1);
      __builtin_amdgcn_sched_barrier(0);
      read_a(st, 3, af1);
      mfmas(wb, J, 2, af0);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (J < KSB - 1) read_a((kt + 1) & AMASK, 0, af0);   // same block: landed
      mfmas(wb, J, 3, af1);
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int blk = kb0; blk < kb1; ++blk) {
      const int kt = KSB * blk;
      bstep(kt, std::integral_constant<int, 0>{});
      if (kt + 1 < kt1) bstep(kt + 1, std::integral_constant<int, 1>{});
      if constexpr (KSB == 4) {
        if (kt + 2 < kt1) bstep(kt + 2, std::integral_constant<int, 2>{});
        if (kt + 3 < kt1) bstep(kt + 3, std::integral_constant<int, 3>{});
      }
      if (blk + 1 < kb1) {
        wait_vmem<0>();                        // block blk+1's copies landed (this wave's) ...
        __syncthreads();                       // ... and every wave's; all are done with block blk
        read_block(wb, blk + 1);
        wait_lds();
        if (blk + 2 < kb1) {                   // block blk+2 reuses block blk's stages
          copy_w(blk + 2);
          copy_a_blk(blk + 2);
        }
        read_a((KSB * blk + KSB) & AMASK, 0, af0);
      }
    }
  }
  wait_vmem<0>();                            // the trailing (clamped) copies land before the LDS is released

  if (part >= 0) {                           // raw partial tile [NM][32 MB][128], finished by nv_splitk_finish
    float* pt = partials + (size_t)b * NM * PT;
    const int col = 32 * wave + li;
#pragma unroll
    for (int t = 0; t < NM; ++t)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
          if (m0 + row < M) pt[t * PT + row * 128 + col] = acc[t][mb][r];   // the finish reads rows < M only
        }
    return;
  }

  const int ncol = n0 + 32 * wave + li;
  if (ncol >= N) return;
  const float c0 = FMT == 1 ? inv0 : cs0[ncol];
  const float c1 = FMT == 1 ? inv1 : (GU ? cs1[ncol] : 0.f);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 32 * mb + 8 * (r >> 2) + 4 * h + (r & 3);
      if (m < M) {
        const float rs = rowscale ? rowscale[m] : 1.0f;
        if constexpr (GU) {
          const float g = acc[0][mb][r] * rs * c0;
          const float u = acc[1][mb][r] * rs * c1;
          const float a = silu_f32(g) * u;
          if constexpr (A32) reinterpret_cast<float*>(out)[(size_t)m * N + ncol] = a;
          else reinterpret_cast<uint16_t*>(out)[(size_t)m * N + ncol] = __builtin_bit_cast(uint16_t, (_Float16)a);
        } else {
          reinterpret_cast<float*>(out)[(size_t)m * N + ncol] = acc[0][mb][r] * rs * c0;
        }
      }
    }
  }
}

// Epilogue of the split tiles: element (row, col) of split tile i adds its S parts in part order.
// A thread handles 4 consecutive columns of one tile row (16-byte partial loads); workgroup b handles 1024
// elements of split tile b / per_tile (a tile has bm * 128 elements).  Stores are vectors when N is a
// multiple of 4 and all 4 columns exist, else per column.
// Column factors as in the GEMM: cs0[n] / cs1[n] (FP8) when cs0 is not null, else inv0 / inv1.
constexpr int kFinishCols = 4;
// Workgroups per split tile: enough for the tile's rows below M when the whole batch lies in one tile
// row (short batches), else the whole tile.  bm * 128 is a multiple of 1024, so the covered elements stay
// inside the partial tile.
__host__ __device__ inline int nv_finish_per_tile(int M, const NvPlan& plan) {
  const int rows = (plan.ntm == 1 && M < plan.bm) ? M : plan.bm;
  return (rows * 128 + 256 * kFinishCols - 1) / (256 * kFinishCols);
}
// ACT32 (gate+up of FP8): act is stored as float32; otherwise as float16.
template <bool GU, bool ACT32>
__global__ void __launch_bounds__(256) nv_splitk_finish(int M, int N, NvPlan plan, const float* __restrict__ partials,
                                                       const float* __restrict__ rowscale,
                                                       const float* __restrict__ cs0, float inv0,
                                                       const float* __restrict__ cs1, float inv1,
                                                       void* __restrict__ out) {
  constexpr int NM = GU ? 2 : 1;
  const int per_tile = nv_finish_per_tile(M, plan);          // workgroups per split tile
  const int i = (int)blockIdx.x / per_tile;                   // split tile index
  const int e = (((int)blockIdx.x - i * per_tile) * 256 + (int)threadIdx.x) * kFinishCols;
  const int pt = plan.bm * 128;
  const int tile = plan.full + i;
  const int tm = tile / plan.ntn, tn = tile - tm * plan.ntn;
  const int m = tm * plan.bm + (e >> 7), n = tn * 128 + (e & 127);
  if (m >= M || n >= N) return;
  const float* p = partials + (size_t)i * plan.S * NM * pt + e;
  f32x4 acc[NM];
#pragma unroll
  for (int t = 0; t < NM; ++t) acc[t] = *reinterpret_cast<const f32x4*>(p + t * pt);
  for (int s = 1; s < plan.S; ++s)
#pragma unroll
    for (int t = 0; t < NM; ++t) acc[t] += *reinterpret_cast<const f32x4*>(p + (size_t)s * NM * pt + t * pt);
  const float rs = rowscale ? rowscale[m] : 1.0f;
  const bool vec = (N & 3) == 0 && n + kFinishCols <= N;
  if constexpr (GU && ACT32) {
    float a[kFinishCols];
#pragma unroll
    for (int j = 0; j < kFinishCols; ++j) {
      const int nj = min(n + j, N - 1);
      const float c0 = cs0 ? cs0[nj] : inv0;
      const float c1 = cs0 ? cs1[nj] : inv1;
      a[j] = silu_f32(acc[0][j] * rs * c0) * (acc[1][j] * rs * c1);
    }
    float* o = reinterpret_cast<float*>(out) + (size_t)m * N + n;
    if (vec) {
      *reinterpret_cast<f32x4*>(o) = f32x4{a[0], a[1], a[2], a[3]};
    } else {
#pragma unroll
      for (int j = 0; j < kFinishCols; ++j)
        if (n + j < N) o[j] = a[j];
    }
  } else if constexpr (GU) {
    uint16_t a[kFinishCols];
#pragma unroll
    for (int j = 0; j < kFinishCols; ++j) {
      const int nj = min(n + j, N - 1);
      const float c0 = cs0 ? cs0[nj] : inv0;
      const float c1 = cs0 ? cs1[nj] : inv1;
      const float g = acc[0][j] * rs * c0;
      const float u = acc[1][j] * rs * c1;
      a[j] = __builtin_bit_cast(uint16_t, (_Float16)(silu_f32(g) * u));
    }
    uint16_t* o = reinterpret_cast<uint16_t*>(out) + (size_t)m * N + n;
    if (vec) {
      *reinterpret_cast<u32x2*>(o) = u32x2{(uint32_t)a[0] | ((uint32_t)a[1] << 16), (uint32_t)a[2] | ((uint32_t)a[3] << 16)};
    } else {
#pragma unroll
      for (int j = 0; j < kFinishCols; ++j)
        if (n + j < N) o[j] = a[j];
    }
  } else {
    float y[kFinishCols];
#pragma unroll
    for (int j = 0; j < kFinishCols; ++j) {
      const int nj = min(n + j, N - 1);
      y[j] = acc[0][j] * rs * (cs0 ? cs0[nj] : inv0);
    }
    float* o = reinterpret_cast<float*>(out) + (size_t)m * N + n;
    if (vec) {
      *reinterpret_cast<f32x4*>(o) = f32x4{y[0], y[1], y[2], y[3]};
    } else {
#pragma unroll
      for (int j = 0; j < kFinishCols; ++j)
        if (n + j < N) o[j] = y[j];
    }
  }
}

template <int FMT, bool GU, int MB, bool BS, bool ABF, bool A32>
hipError_t nv_launch(int M, int K, int N, const NvPlan& plan, const uint16_t* a16, const float* rowscale,
                     const uint8_t* w0, const float* cs0, float inv0, const uint8_t* w1, const float* cs1,
                     float inv1, void* out, float* partials, hipStream_t st) {
  if (!raise_lds_limit<nv_gemm_kernel<FMT, GU, MB, BS, ABF, A32>>()) return hipErrorInvalidValue;   // up to 72 KB
  const int grid = plan.units_grid + (plan.full + 7) / 8 * 8;
  hipLaunchKernelGGL((nv_gemm_kernel<FMT, GU, MB, BS, ABF, A32>), dim3(grid), dim3(256), g_lds_bytes<FMT>(GU, MB, BS), st, M,
                     K, N, plan, a16, rowscale, w0, cs0, inv0, w1, cs1, inv1, out, partials);
  return hipGetLastError();
}

template <int FMT, bool GU, bool ABF, bool A32 = (FMT == 0)>
hipError_t nv_dispatch(int M, int K, int N, const uint16_t* a16, const float* rowscale, const uint8_t* w0,
                       const float* cs0, float inv0, const uint8_t* w1, const float* cs1, float inv1, void* out,
                       float* partials, hipStream_t st) {
  const NvPlan plan = nv_plan(FMT, M, K, N, GU);
  if (plan.units > 0 && partials == nullptr) return hipErrorInvalidValue;
  if (FMT == 1) cs0 = cs1 = nullptr;
  hipError_t e;
  switch (plan.bm) {
    case 32:
      e = nv_launch<FMT, GU, 1, true, ABF, A32>(M, K, N, plan, a16, rowscale, w0, cs0, inv0, w1, cs1, inv1, out, partials, st);
      break;
    case 64:
      e = nv_launch<FMT, GU, 2, false, ABF, A32>(M, K, N, plan, a16, rowscale, w0, cs0, inv0, w1, cs1, inv1, out, partials, st);
      break;
    default:
      e = nv_launch<FMT, GU, 4, false, ABF, A32>(M, K, N, plan, a16, rowscale, w0, cs0, inv0, w1, cs1, inv1, out, partials, st);
      break;
  }
  if (e != hipSuccess || plan.units == 0) return e;
  hipLaunchKernelGGL((nv_splitk_finish<GU, GU && A32>), dim3((plan.tiles - plan.full) * nv_finish_per_tile(M, plan)),
                     dim3(256), 0, st, M, N,
                     plan, partials, rowscale, cs0, inv0, cs1, inv1, out);
  return hipGetLastError();
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

// ---- W4A8: NVFP4 weights x per-token E4M3 activations -----------------------------------------------
//
// Activation quantization (page "Qwen3.8-27B-NVFP4", section "Implemented execution path": per-token
// dynamic 8-bit activations in a small workspace, one quantization of x shared by gate and up): each row
// is scaled by the power of two 2^-e that puts its largest magnitude in (224, 448] (exact) and rounded to
// E4M3 with round to nearest even (v_cvt_pk_fp8_f32).  Every E4M3 value is a float16, so the quantized
// row is stored as float16 values (the code's value, exactly) and the GEMMs are the float16 path's own:
// its decoded weights (E2M1 x E4M3 group scale) are exact float16 values too, so each MFMA product is the
// exact product of a quantized activation and a weight, accumulated in float32, and 2^e is the row scale
// its epilogue already applies.  (A form with one K = 16 fp8 MFMA per weight group and a float32 rescale
// of each group's result took 0.45 ms at M = 512 against 0.29 ms for this one: the rescale costs 16 FMAs
// per lane per MFMA.)
// E4M3 exponent of a row: smallest e with amax <= 448 * 2^e (amax = f 2^p, f in [0.5, 1): 448 = 0.875 * 2^9,
// so e = p - 9, plus one when f > 0.875); 0 for a zero or non-finite amax.
__device__ __forceinline__ int e4m3_token_exp(float amax) {
  if (!(amax > 0.f) || !(amax <= 3.0e38f)) return 0;
  int p;
  const float f = frexpf(amax, &p);
  return p - 9 + (f > 0.875f ? 1 : 0);
}
// 8 consecutive elements (as float32) scaled by 2^-e -> their E4M3 values as 8 float16 (16 bytes, in order).
__device__ __forceinline__ u32x4 e4m3_round8_f16(const float* v, int e) {
  float s[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = ldexpf(v[j], -e);
  int lo = 0, hi = 0;
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(s[0], s[1], lo, false);
  lo = __builtin_amdgcn_cvt_pk_fp8_f32(s[2], s[3], lo, true);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(s[4], s[5], hi, false);
  hi = __builtin_amdgcn_cvt_pk_fp8_f32(s[6], s[7], hi, true);
  return u32x4{as_u32(e4m3x2_f16<false>((uint32_t)lo)), as_u32(e4m3x2_f16<true>((uint32_t)lo)),
               as_u32(e4m3x2_f16<false>((uint32_t)hi)), as_u32(e4m3x2_f16<true>((uint32_t)hi))};
}
template <typename XT>
__device__ __forceinline__ void load8(const XT* row, int u, float* v) {
  if constexpr (std::is_same<XT, float>::value) {
    const u32x4 a = reinterpret_cast<const u32x4*>(row)[2 * u], b = reinterpret_cast<const u32x4*>(row)[2 * u + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(a[i]);
      v[4 + i] = __uint_as_float(b[i]);
    }
  } else {
    const u32x4 a = reinterpret_cast<const u32x4*>(row)[u];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(a[i] << 16);
      v[2 * i + 1] = __uint_as_float(a[i] & 0xFFFF0000u);
    }
  }
}
// One 256-thread workgroup per row; units of 8 elements, RU of them per thread kept in registers (the
// rest read again).  q [M][K] float16 (E4M3 values); rowscale[m] = 2^e.
template <typename XT, int RU>
__global__ void __launch_bounds__(256) quant_e4m3_kernel(int M, int K, const XT* __restrict__ x,
                                                         uint16_t* __restrict__ q, float* __restrict__ rowscale) {
  __shared__ float wmax[4];
  const int m = (int)blockIdx.x;
  const int t = (int)threadIdx.x;
  const int nu = K / 8;
  const XT* row = x + (size_t)m * K;
  float cache[RU][8];
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < RU; ++i) {
    const int u = t + 256 * i;
    if (u < nu) {
      load8<XT>(row, u, cache[i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(cache[i][j]));
    }
  }
  for (int u = t + 256 * RU; u < nu; u += 256) {
    float v[8];
    load8<XT>(row, u, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
  if ((t & 63) == 0) wmax[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const int e = e4m3_token_exp(amax);
  if (t == 0) rowscale[m] = ldexpf(1.0f, e);
  u32x4* o = reinterpret_cast<u32x4*>(q + (size_t)m * K);
#pragma unroll
  for (int i = 0; i < RU; ++i) {
    const int u = t + 256 * i;
    if (u < nu) o[u] = e4m3_round8_f16(cache[i], e);
  }
  for (int u = t + 256 * RU; u < nu; u += 256) {
    float v[8];
    load8<XT>(row, u, v);
    o[u] = e4m3_round8_f16(v, e);
  }
}

}  // namespace

hipError_t launch_rowscale_f16(int M, int K, const void* x, XType xt, uint16_t* x16, float* rowscale,
                               hipStream_t st) {
  // Rows of up to 5120 elements: four rows (waves) per workgroup, 10 (bf16) / 20 (float32) register chunks
  // per lane.  Longer rows: a workgroup per row, 10 / 20 register chunks per thread (K up to 20480 kept in
  // registers).
  if (K > 5120) {
    if (xt == X_BF16)
      hipLaunchKernelGGL((rowscale_f16_wg_kernel<uint16_t, 10>), dim3(M), dim3(256), 0, st, M, K,
                         reinterpret_cast<const uint16_t*>(x), x16, rowscale);
    else
      hipLaunchKernelGGL((rowscale_f16_wg_kernel<float, 20>), dim3(M), dim3(256), 0, st, M, K,
                         reinterpret_cast<const float*>(x), x16, rowscale);
    return hipGetLastError();
  }
  const dim3 grid((M + 3) / 4);
  if (xt == X_BF16)
    hipLaunchKernelGGL((rowscale_f16_kernel<uint16_t, 10>), grid, dim3(256), 0, st, M, K,
                       reinterpret_cast<const uint16_t*>(x), x16, rowscale);
  else
    hipLaunchKernelGGL((rowscale_f16_kernel<float, 20>), grid, dim3(256), 0, st, M, K,
                       reinterpret_cast<const float*>(x), x16, rowscale);
  return hipGetLastError();
}

size_t mfma_partial_bytes(int fmt, int M, int K, int N, bool gu) {
  if (K < g_min_k(fmt) || M <= 0) return 0;
  return nv_partial_bytes(nv_plan(fmt, M, K, N, gu), gu);
}

bool mfma_bf16_ok(int fmt, int K) { return fmt == 0 && K >= g_min_k(0); }

hipError_t launch_mfma_gateup(int fmt, int M, int K, int N, const uint16_t* x16, const float* rowscale,
                              const uint8_t* w0, const float* cs0, float inv0, const uint8_t* w1,
                              const float* cs1, float inv1, void* act16, float* partials, bool abf,
                              hipStream_t st) {
  if (abf) {
    if (!mfma_bf16_ok(fmt, K) || rowscale != nullptr) return hipErrorInvalidValue;
    return nv_dispatch<0, true, true>(M, K, N, x16, nullptr, w0, cs0, inv0, w1, cs1, inv1, act16, partials, st);
  }
  if (K >= g_min_k(fmt))
    return fmt == 1 ? nv_dispatch<1, true, false>(M, K, N, x16, rowscale, w0, cs0, inv0, w1, cs1, inv1, act16, partials, st)
                    : nv_dispatch<0, true, false>(M, K, N, x16, rowscale, w0, cs0, inv0, w1, cs1, inv1, act16, partials, st);
  if (fmt == 1)
    return gemm_dispatch<1, true>(M, K, N, x16, rowscale, w0, cs0, inv0, w1, cs1, inv1, act16, st);
  return gemm_dispatch<0, true>(M, K, N, x16, rowscale, w0, cs0, inv0, w1, cs1, inv1, act16, st);
}

hipError_t launch_mfma_linear(int fmt, int M, int K, int N, const uint16_t* a16, const float* rowscale,
                              const uint8_t* w, const float* cs, float inv, float* y, float* partials, bool abf,
                              hipStream_t st) {
  if (abf) {
    if (!mfma_bf16_ok(fmt, K) || rowscale != nullptr) return hipErrorInvalidValue;
    return nv_dispatch<0, false, true>(M, K, N, a16, nullptr, w, cs, inv, nullptr, nullptr, 0.f, y, partials, st);
  }
  if (K >= g_min_k(fmt))
    return fmt == 1 ? nv_dispatch<1, false, false>(M, K, N, a16, rowscale, w, cs, inv, nullptr, nullptr, 0.f, y, partials, st)
                    : nv_dispatch<0, false, false>(M, K, N, a16, rowscale, w, cs, inv, nullptr, nullptr, 0.f, y, partials, st);
  if (fmt == 1) return gemm_dispatch<1, false>(M, K, N, a16, rowscale, w, cs, inv, nullptr, nullptr, 0.f, y, st);
  return gemm_dispatch<0, false>(M, K, N, a16, rowscale, w, cs, inv, nullptr, nullptr, 0.f, y, st);
}

}  // namespace wq

namespace wq {

hipError_t launch_quant_e4m3(int M, int K, const void* x, XType xt, uint16_t* q, float* rowscale, hipStream_t st) {
  if (K % 8) return hipErrorInvalidValue;
  // units of 8 per thread kept in registers: 3 cover K = 6144, 9 cover K = 18432
  if (xt == X_BF16) {
    if (K <= 6144) hipLaunchKernelGGL((quant_e4m3_kernel<uint16_t, 3>), dim3(M), dim3(256), 0, st, M, K,
                                      reinterpret_cast<const uint16_t*>(x), q, rowscale);
    else hipLaunchKernelGGL((quant_e4m3_kernel<uint16_t, 9>), dim3(M), dim3(256), 0, st, M, K,
                            reinterpret_cast<const uint16_t*>(x), q, rowscale);
  } else if (xt == X_F32) {
    if (K <= 6144) hipLaunchKernelGGL((quant_e4m3_kernel<float, 3>), dim3(M), dim3(256), 0, st, M, K,
                                      reinterpret_cast<const float*>(x), q, rowscale);
    else hipLaunchKernelGGL((quant_e4m3_kernel<float, 9>), dim3(M), dim3(256), 0, st, M, K,
                            reinterpret_cast<const float*>(x), q, rowscale);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

size_t w4a8_partial_bytes(int M, int K, int N, bool gu) { return mfma_partial_bytes(1, M, K, N, gu); }

hipError_t launch_w4a8_gateup(int M, int K, int N, const uint16_t* xq, const float* sx, const uint8_t* w0, float inv0,
                              const uint8_t* w1, float inv1, float* act, float* partials, hipStream_t st) {
  if (K < g_min_k(1)) return hipErrorInvalidValue;
  return nv_dispatch<1, true, false, true>(M, K, N, xq, sx, w0, nullptr, inv0, w1, nullptr, inv1, act, partials, st);
}

hipError_t launch_w4a8_linear(int M, int K, int N, const uint16_t* aq, const float* sa, const uint8_t* w, float inv,
                              float* y, float* partials, hipStream_t st) {
  if (K < g_min_k(1)) return hipErrorInvalidValue;
  return nv_dispatch<1, false, false, false>(M, K, N, aq, sa, w, nullptr, inv, nullptr, nullptr, 0.f, y, partials, st);
}

}  // namespace wq
