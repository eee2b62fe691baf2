// M < 128 path, main kernels: HBM-streaming GEMVs tuned on MI355X for the decode shapes.
//
// Method: issue "tp>1 fp8w tail-MLP shard host-dequantizes every layer", section
// "Proposed fix" (SwiGLU MLP, float32 act); NVFP4 decode from page
// "Qwen3.8-27B-NVFP4", section "NVFP4 numerics as implemented" (the E4M3 group
// scale applied at every K=16 boundary).
//
// Two kernel shapes, chosen from measurements of the 5120 x 17408 decode:
//  * row kernels (gate+up): one wave per output row pair (gate row n, up row n); every weight load of the
//    pair is issued at once (2 x 5 KB for FP8 at K=5120), right after the loads of the workgroup's x
//    row, which is staged in LDS (one copy per 8 row pairs instead of one per wave); occupancy 8
//    waves/SIMD.  The weights stay in
//    registers while the m rows of a multi-row call are processed one by one.
//  * item kernels (down projection / single linear): a 16-wave workgroup owns RB output rows; the
//    activation row is staged once into LDS; the (row pair, K slot) work items -- a K slot is one unit per
//    lane -- are dealt round-robin to the waves, each wave streaming its items with the next D loads in
//    flight; each wave keeps one partial per row it touches and the workgroup adds the 16 partials of a
//    row in wave order.
//  * nv_lin_r32 (NVFP4 single linear with 16-bit activations, K % 256 == 0; the NVFP4 MLP's down
//    projection, whose act is float16): single-row items of 32 records moved by global->LDS copies,
//    rows interleaved over the grid (described at the kernel).
// The per-lane unit is 16 weights for both formats: an FP8 chunk (16 code bytes) or an NVFP4 group (the
// 8 nibble bytes qs[8q..8q+7] of a Block64 record and its scale byte d[q]).  Four lanes read one record,
// so the 36-byte records are covered without gaps and K = 5120 fills every lane (320 groups per row).
// Weight loads use clamped in-bounds addresses where a lane or item runs past the matrix and only the
// accumulation is guarded: a guarded load makes the compiler drain all outstanding loads before the
// next one.
// Fixed accumulation orders (bitwise reproducible; independent of M because m rows are processed one
// after another with the same schedule):
//  * FP8 units: the 8 code pairs go into two partials (even / odd 4-code quads); NVFP4 units: one
//    partial over the 16 weights in ascending k, then multiplied by the E4M3 group scale.
//  * row kernels: lane l owns units l, l+64, ... (ascending); FP8 s = p0 + p1 per row, NVFP4 the scaled
//    group partials summed in unit order; butterfly over 64 lanes (xor 32..1); times the channel scale
//    or 1/global_scale.
//  * item kernels: within a wave, items ascending, per row a butterfly over 64 lanes when the wave leaves
//    the row; then the workgroup sums the per-wave partials in wave order 0..15; times the channel scale
//    or 1/global_scale.
#include "dev_common.h"
#include "launch.h"

namespace wq {

namespace {

constexpr int kItemWaves = 16;   // waves per item-kernel workgroup
constexpr int kItemRows = 20;    // output rows per item-kernel workgroup
constexpr int kItemDepth = 2;    // loads in flight per wave (items)
constexpr int kRowWaves = 8;     // waves (row pairs) per row-kernel workgroup
constexpr int kStageRegs = 5;    // activation pieces per thread loaded ahead of the item prefetch
constexpr int kRowStageRegs = 2; // x pieces per thread loaded ahead of the row-kernel weights (K <= 8192)

__device__ __forceinline__ u32x4 ld_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ u32x2 ld8a4(const uint8_t* p) {
  u32x2 v;
  __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 8);
  return v;
}
__device__ __forceinline__ u32x4 ld16a4(const uint8_t* p) {
  u32x4 v;
  __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 16);
  return v;
}
template <int W>
__device__ __forceinline__ float gsum(float v) {
  static_assert(W == 64 || W == 16, "wave or row sum");
  if constexpr (W == 64) return wave64_sum(v);
  else return row16_sum(v);
}
__device__ __forceinline__ float e4m3_group(uint32_t d, int g) {
  return g == 0 ? e4m3_byte_f32<0>(d) : g == 1 ? e4m3_byte_f32<1>(d) : g == 2 ? e4m3_byte_f32<2>(d)
                                                                             : e4m3_byte_f32<3>(d);
}

// An activation row staged into LDS piece-major: piece q (16 bytes) of unit u at (q * U + u) * 16, where
// a unit holds 16 activations and PQ pieces make one unit, so consecutive lanes read consecutive pieces.
template <typename XT, int UNIT>
__device__ __forceinline__ void stage_units(uint8_t* lds, const XT* __restrict__ xm, int U) {
  constexpr int PQ = UNIT * (int)sizeof(XT) / 16;
  const u32x4* src = reinterpret_cast<const u32x4*>(xm);
  for (int i = threadIdx.x; i < U * PQ; i += blockDim.x) {
    const int u = i / PQ, q = i - u * PQ;
    *reinterpret_cast<u32x4*>(lds + ((size_t)q * U + u) * 16) = src[i];
  }
}


// The same staging split in two so that the activation loads can be issued before a weight prefetch
// (per-wave loads complete in order, so staging issued after the prefetch would wait for all of it);
// used by the single-row kernels (the multi-row ones would keep the registers live across m):
// issue() loads up to SPT pieces per thread into registers, finish() writes them to LDS and stages any
// remainder with a plain loop.
template <typename XT, int SPT>
struct StageRegs {
  u32x4 v[SPT];
  __device__ __forceinline__ void issue(const XT* __restrict__ xm, int U) {
    constexpr int PQ = 16 * (int)sizeof(XT) / 16;
    const u32x4* src = reinterpret_cast<const u32x4*>(xm);
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int i = threadIdx.x + j * (int)blockDim.x;
      if (i < U * PQ) v[j] = src[i];
    }
  }
  __device__ __forceinline__ void finish(uint8_t* lds, const XT* __restrict__ xm, int U) {
    constexpr int PQ = 16 * (int)sizeof(XT) / 16;
#pragma unroll
    for (int j = 0; j < SPT; ++j) {
      const int i = threadIdx.x + j * (int)blockDim.x;
      if (i < U * PQ) {
        const int u = i / PQ, q = i - u * PQ;
        *reinterpret_cast<u32x4*>(lds + ((size_t)q * U + u) * 16) = v[j];
      }
    }
    const u32x4* src = reinterpret_cast<const u32x4*>(xm);
    for (int i = threadIdx.x + SPT * (int)blockDim.x; i < U * PQ; i += blockDim.x) {
      const int u = i / PQ, q = i - u * PQ;
      *reinterpret_cast<u32x4*>(lds + ((size_t)q * U + u) * 16) = src[i];
    }
  }
};

// ---- FP8 gate+up row kernel (bf16 x) -------------------------------------------------------------
// kRowWaves waves per workgroup, one row pair each; the x row is staged once per workgroup into LDS
// (piece q of chunk c at (q * C + c) * 16) after the weight loads are issued, and read chunk by chunk.
// ONE: the call has a single activation row (compile-time loop bound).
template <int CH, bool ONE>
__global__ void __launch_bounds__(64 * kRowWaves) fp8_gu_row(int M, int K, int N, const uint16_t* __restrict__ x,
                                                          const uint8_t* __restrict__ wg, const float* __restrict__ sg,
                                                          const uint8_t* __restrict__ wu, const float* __restrict__ su,
                                                          float* __restrict__ act) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int C = K >> 4;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowWaves + (threadIdx.x >> 6);
  const int rl = min(row, N - 1);   // rows past N compute on row N-1 and store nothing
  // Single-row calls issue the x loads before the weight loads: loads of a wave complete in order, so
  // the workgroup barrier then waits only for x, not for every wave's weights.
  StageRegs<uint16_t, kRowStageRegs> sr;
  if constexpr (ONE) sr.issue(x, C);
  u32x4 w[2][CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int ch = min(lane + 64 * c, C - 1);
    w[0][c] = ld_stream(wg + (size_t)rl * K + 16 * ch);
    w[1][c] = ld_stream(wu + (size_t)rl * K + 16 * ch);
  }
  const int Mloop = ONE ? 1 : M;
  for (int m = 0; m < Mloop; ++m) {
    if constexpr (ONE) {
      sr.finish(lds, x, C);
    } else {
      if (m) __syncthreads();
      stage_units<uint16_t, 16>(lds, x + (size_t)m * K, C);
    }
    __syncthreads();
    float a[2][2] = {{0.f, 0.f}, {0.f, 0.f}};
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int ch = lane + 64 * c;
      if (ch < C) {
        const u32x4 x0 = *reinterpret_cast<const u32x4*>(lds + (size_t)ch * 16);
        const u32x4 x1 = *reinterpret_cast<const u32x4*>(lds + ((size_t)C + ch) * 16);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 v = w[t][c];
          float p0 = a[t][0], p1 = a[t][1];
          p0 = dot2_bf16(e4m3x2_bf16<false>(v.x), x0.x, p0);
          p0 = dot2_bf16(e4m3x2_bf16<true>(v.x), x0.y, p0);
          p1 = dot2_bf16(e4m3x2_bf16<false>(v.y), x0.z, p1);
          p1 = dot2_bf16(e4m3x2_bf16<true>(v.y), x0.w, p1);
          p0 = dot2_bf16(e4m3x2_bf16<false>(v.z), x1.x, p0);
          p0 = dot2_bf16(e4m3x2_bf16<true>(v.z), x1.y, p0);
          p1 = dot2_bf16(e4m3x2_bf16<false>(v.w), x1.z, p1);
          p1 = dot2_bf16(e4m3x2_bf16<true>(v.w), x1.w, p1);
          a[t][0] = p0;
          a[t][1] = p1;
        }
      }
    }
    if (row < N) {
      const float g = gsum<64>(a[0][0] + a[0][1]) * sg[row];
      const float u = gsum<64>(a[1][0] + a[1][1]) * su[row];
      if (lane == 0) act[(size_t)m * N + row] = silu_f32(g) * u;
    }
  }
}

// ---- NVFP4 gate+up row kernel (bf16 x), group mapping ---------------------------------------------
// Unit of work per lane: one 16-weight group = 8 nibble bytes (qs[8q..8q+7] of its record) plus the
// record's scale byte d[q].  Lane l owns groups l, l+64, ... of its row; lane 4j+q reads bytes
// [8q, 8q+12) of record j, i.e. the dword before its nibbles and the nibbles, so the quad's loads cover
// the record once and a wave's loads cover 16 records without gaps or overlap.  The dword before the
// nibbles of group 0 is the record's scale dword, which lane 4j passes to its quad (a DPP quad
// broadcast).  The loads carry the non-temporal hint: every byte is read by exactly one load (with
// separate loads for the nibbles and the scale byte the hint cost 4 us: the two loads share lines).
// Workgroup shape and x staging as in the FP8 row kernel.
// O16: act is stored as float16 bits (the NVFP4 MLP's act), else float32.
template <int CH, bool ONE, bool O16>
__global__ void __launch_bounds__(64 * kRowWaves) nv_gu_grp(int M, int K, int N, const uint16_t* __restrict__ x,
                                                         const uint8_t* __restrict__ bg, float inv_g,
                                                         const uint8_t* __restrict__ bu, float inv_u,
                                                         void* __restrict__ act) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int G = K >> 4;
  const size_t rb = (size_t)(K >> 6) * 36;
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kRowWaves + (threadIdx.x >> 6);
  const int rl = min(row, N - 1);   // rows past N compute on row N-1 and store nothing
  // Single-row calls issue the x loads before the weight loads: loads of a wave complete in order, so
  // the workgroup barrier then waits only for x, not for every wave's weights.
  StageRegs<uint16_t, kRowStageRegs> sr;
  if constexpr (ONE) sr.issue(x, G);
  u32x3_a4 wv[2][CH];   // record bytes [8q, 8q+12): .x the scale dword (q = 0), .y .z the group's nibbles
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int g = min(lane + 64 * c, G - 1);   // clamped: in bounds, never accumulated
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const uint8_t* p = (mt ? bu : bg) + (size_t)rl * rb + (size_t)(g >> 2) * 36 + 8 * (g & 3);
      wv[mt][c] = __builtin_nontemporal_load(reinterpret_cast<const u32x3_a4*>(p));   // 4-byte aligned
    }
  }
  const int Mloop = ONE ? 1 : M;
  for (int m = 0; m < Mloop; ++m) {
    if constexpr (ONE) {
      sr.finish(lds, x, G);
    } else {
      if (m) __syncthreads();
      stage_units<uint16_t, 16>(lds, x + (size_t)m * K, G);
    }
    __syncthreads();
    float acc[2] = {0.f, 0.f};
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int g = lane + 64 * c;
      // the record's scale dword from the quad's first lane (G is a multiple of 4, so quads never straddle
      // the clamped tail), then this group's byte d[q]
      uint32_t sq[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        sq[mt] = ((uint32_t)__builtin_amdgcn_mov_dpp((int)wv[mt][c].x, 0x00, 0xf, 0xf, false) >> (8 * (lane & 3))) &
                 0xffu;
      if (g < G) {
        const u32x4 x0 = *reinterpret_cast<const u32x4*>(lds + (size_t)g * 16);
        const u32x4 x1 = *reinterpret_cast<const u32x4*>(lds + ((size_t)G + g) * 16);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const u32x2 w = {wv[mt][c].y, wv[mt][c].z};
          float pt = 0.f;
          pt = dot2_bf16(e2m1x2_bf16<0>(w.x), x0.x, pt);
          pt = dot2_bf16(e2m1x2_bf16<1>(w.x), x0.y, pt);
          pt = dot2_bf16(e2m1x2_bf16<2>(w.x), x0.z, pt);
          pt = dot2_bf16(e2m1x2_bf16<3>(w.x), x0.w, pt);
          pt = dot2_bf16(e2m1x2_bf16<0>(w.y), x1.x, pt);
          pt = dot2_bf16(e2m1x2_bf16<1>(w.y), x1.y, pt);
          pt = dot2_bf16(e2m1x2_bf16<2>(w.y), x1.z, pt);
          pt = dot2_bf16(e2m1x2_bf16<3>(w.y), x1.w, pt);
          acc[mt] = fmaf(pt, e4m3_byte_f32<0>(sq[mt]), acc[mt]);
        }
      }
    }
    if (row < N) {
      const float gv = gsum<64>(acc[0]) * inv_g;
      const float uv = gsum<64>(acc[1]) * inv_u;
      const float a = silu_f32(gv) * uv;
      if (lane == 0) {
        if constexpr (O16) reinterpret_cast<uint16_t*>(act)[(size_t)m * N + row] = __builtin_bit_cast(uint16_t, (_Float16)a);
        else reinterpret_cast<float*>(act)[(size_t)m * N + row] = a;
      }
    }
  }
}

// Sum over one 16-weight group of E2M1 weight x float16 activation, float32 accumulation in ascending k:
// w0, w1 hold the group's 8 nibble bytes (low nibble first), x0, x1 its 16 activations (f16 pairs).
__device__ __forceinline__ float dot16_e2m1_f16(uint32_t w0, uint32_t w1, u32x4 x0, u32x4 x1, float acc) {
  acc = dot2_f16(e2m1x2_f16<0>(w0), as_f16x2(x0.x), acc);
  acc = dot2_f16(e2m1x2_f16<1>(w0), as_f16x2(x0.y), acc);
  acc = dot2_f16(e2m1x2_f16<2>(w0), as_f16x2(x0.z), acc);
  acc = dot2_f16(e2m1x2_f16<3>(w0), as_f16x2(x0.w), acc);
  acc = dot2_f16(e2m1x2_f16<0>(w1), as_f16x2(x1.x), acc);
  acc = dot2_f16(e2m1x2_f16<1>(w1), as_f16x2(x1.y), acc);
  acc = dot2_f16(e2m1x2_f16<2>(w1), as_f16x2(x1.z), acc);
  acc = dot2_f16(e2m1x2_f16<3>(w1), as_f16x2(x1.w), acc);
  return acc;
}
__device__ __forceinline__ float dot16_e2m1_bf16(uint32_t w0, uint32_t w1, u32x4 x0, u32x4 x1, float acc) {
  acc = dot2_bf16(e2m1x2_bf16<0>(w0), x0.x, acc);
  acc = dot2_bf16(e2m1x2_bf16<1>(w0), x0.y, acc);
  acc = dot2_bf16(e2m1x2_bf16<2>(w0), x0.z, acc);
  acc = dot2_bf16(e2m1x2_bf16<3>(w0), x0.w, acc);
  acc = dot2_bf16(e2m1x2_bf16<0>(w1), x1.x, acc);
  acc = dot2_bf16(e2m1x2_bf16<1>(w1), x1.y, acc);
  acc = dot2_bf16(e2m1x2_bf16<2>(w1), x1.z, acc);
  acc = dot2_bf16(e2m1x2_bf16<3>(w1), x1.w, acc);
  return acc;
}

// ---- item kernels ---------------------------------------------------------------------------------
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
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: cursor in SGPRs
  const int rbase = blockIdx.x * RB;
  const int NI = (RB / R) * T;
  const int nk = NI > wv ? (NI - wv + NW - 1) / NW : 0;
  const uint32_t lane_off = 16u * lane, max_off = 16u * (C - 1);
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
        // Row base is wave-uniform; the lane offset is clamped to the last chunk and rows to the last
        // row: in bounds, and never accumulated or stored.
        const uint32_t off = min(1024u * lc.t + lane_off, max_off);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int n = min(rbase + lc.g * R + r, N - 1);
          buf[b][r] = ld_stream(w + (size_t)n * K + off);
        }
      }
      ++lk;
      lc.step(NW, T);
    };
    if constexpr (ONE) {
      StageRegs<XT, kStageRegs> sr;
      sr.issue(xa, C);
#pragma unroll
      for (int b = 0; b < D; ++b) load(b);
      sr.finish(lds, xa, C);
    } else {
#pragma unroll
      for (int b = 0; b < D; ++b) load(b);
      stage_units<XT, 16>(lds, xa + (size_t)m * K, C);
    }
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

// NVFP4 single linear: y[m, n] = inv * sum_k xa[m, k] dq(blk[n, k]).  Same item schedule as the FP8
// kernel, with the 16-weight group (8 nibble bytes + its scale byte) as the per-lane unit.
// F16 (16-bit XT only): x holds float16 bits, else bfloat16 bits.
template <typename XT, bool ONE, bool F16>
__global__ void __launch_bounds__(64 * kItemWaves, 8) nv_lin_grp(int M, int K, int N, const XT* __restrict__ xa,
                                                              const uint8_t* __restrict__ blk, float inv,
                                                              float* __restrict__ y) {
  constexpr int R = 2, D = kItemDepth, NW = kItemWaves, RB = kItemRows;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ float part[NW][RB];
  const int G = K >> 4, T = (G + 63) >> 6;
  const size_t rb = (size_t)(K >> 6) * 36;
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform: cursor in SGPRs
  const int rbase = blockIdx.x * RB;
  const int NI = (RB / R) * T;
  const int nk = NI > wv ? (NI - wv + NW - 1) / NW : 0;
  // Byte offsets inside a row of group g = 64 t + lane: its nibbles at (g/4)*36 + 4 + 8*(g%4) and its
  // scale at (g/4)*36 + g%4; both increase with g, so clamping to group G-1 is one min each.
  const uint32_t q_lane = (lane >> 2) * 36u + 4u + 8u * (lane & 3), s_lane = (lane >> 2) * 36u + (lane & 3);
  const uint32_t q_max = ((G - 1) >> 2) * 36u + 4u + 8u * ((G - 1) & 3), s_max = ((G - 1) >> 2) * 36u + ((G - 1) & 3);
  const int Mloop = ONE ? 1 : M;
  for (int m = 0; m < Mloop; ++m) {
    if (m) __syncthreads();
    for (int i = threadIdx.x; i < NW * RB; i += blockDim.x) (&part[0][0])[i] = 0.f;
    u32x2 qb[D][R];
    uint32_t sb[D][R];
    ItemCursor lc;
    lc.init(wv, T);
    int lk = 0;
    auto load = [&](int b) {
      if (lk < nk) {
        // Row base is wave-uniform; offsets clamped to the last group and rows to the last row: in
        // bounds, and never accumulated or stored.
        const uint32_t qo = min(576u * lc.t + q_lane, q_max), so = min(576u * lc.t + s_lane, s_max);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int n = min(rbase + lc.g * R + r, N - 1);
          const uint8_t* p = blk + (size_t)n * rb;
          qb[b][r] = ld8a4(p + qo);
          sb[b][r] = p[so];
        }
      }
      ++lk;
      lc.step(NW, T);
    };
    if constexpr (ONE) {
      StageRegs<XT, kStageRegs> sr;
      sr.issue(xa, G);
#pragma unroll
      for (int b = 0; b < D; ++b) load(b);
      sr.finish(lds, xa, G);
    } else {
#pragma unroll
      for (int b = 0; b < D; ++b) load(b);
      stage_units<XT, 16>(lds, xa + (size_t)m * K, G);
    }
    __syncthreads();
    float acc[R] = {0.f, 0.f};
    int cur = -1;
    auto flush = [&]() {
      if (cur < 0) return;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float v = gsum<64>(acc[r]);
        acc[r] = 0.f;
        if (lane == 0) part[wv][cur * R + r] = v;
      }
    };
    ItemCursor cc;
    cc.init(wv, T);
    for (int k0 = 0; k0 < nk; k0 += D) {
#pragma unroll
      for (int b = 0; b < D; ++b) {
        const int k = k0 + b;
        if (k < nk) {
          const int gi = cc.g, g = lane + 64 * cc.t;
          cc.step(NW, T);
          if (gi != cur) {
            flush();
            cur = gi;
          }
          if (g < G) {
            if constexpr (sizeof(XT) == 4) {
              f32x4 xv[4];
#pragma unroll
              for (int qq = 0; qq < 4; ++qq) xv[qq] = *reinterpret_cast<const f32x4*>(lds + ((size_t)qq * G + g) * 16);
#pragma unroll
              for (int r = 0; r < R; ++r) {
                const u32x2 w = qb[b][r];
                float pt = 0.f;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                  const uint32_t wd = h ? w.y : w.x;
                  const f32x4 a0 = xv[2 * h], a1 = xv[2 * h + 1];
                  f32x2 e = e2m1x2_f32<0>(wd);
                  pt = fmaf(a0.x, e.x, pt);
                  pt = fmaf(a0.y, e.y, pt);
                  e = e2m1x2_f32<1>(wd);
                  pt = fmaf(a0.z, e.x, pt);
                  pt = fmaf(a0.w, e.y, pt);
                  e = e2m1x2_f32<2>(wd);
                  pt = fmaf(a1.x, e.x, pt);
                  pt = fmaf(a1.y, e.y, pt);
                  e = e2m1x2_f32<3>(wd);
                  pt = fmaf(a1.z, e.x, pt);
                  pt = fmaf(a1.w, e.y, pt);
                }
                acc[r] = fmaf(pt, e4m3_byte_f32<0>(sb[b][r]), acc[r]);
              }
            } else {
              const u32x4 x0 = *reinterpret_cast<const u32x4*>(lds + ((size_t)0 * G + g) * 16);
              const u32x4 x1 = *reinterpret_cast<const u32x4*>(lds + ((size_t)1 * G + g) * 16);
#pragma unroll
              for (int r = 0; r < R; ++r) {
                const u32x2 w = qb[b][r];
                const float pt = F16 ? dot16_e2m1_f16(w.x, w.y, x0, x1, 0.f) : dot16_e2m1_bf16(w.x, w.y, x0, x1, 0.f);
                acc[r] = fmaf(pt, e4m3_byte_f32<0>(sb[b][r]), acc[r]);
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
        y[(size_t)m * N + n] = v * inv;
      }
    }
  }
}

// NVFP4 single linear for 16-bit activations, K % 256 == 0: y[m, n] = inv * sum_k xa[m, k] dq(blk[n, k]).
// A 16-wave workgroup owns kR32Rows output rows, interleaved over the grid (local row i is row
// blockIdx + gridDim * i), so the rows the chip streams at any moment sit in two narrow windows of the
// matrix.  Work item (row i, slot t) = the 32 records [32 t, 32 t + 32) of the row, 1152 contiguous
// bytes; items are dealt round-robin to the waves.  Both the activation rows and the items move by
// global->LDS copies (kR32Depth items in flight per wave, explicit vmcnt waits): register loads of
// the same data made the compiler wait for every outstanding load at the top of the item loop.  The item
// copies carry the non-temporal hint (each weight byte is copied once).
// MR activation rows share one pass over the weights (each item is decoded once and used for all MR
// rows); a call with more rows makes ceil(M / MR) passes.
// Lane l of an item owns groups 2l, 2l+1 (record l / 2, 16 nibble bytes and 2 scale bytes).
// Accumulation order (fixed; independent of M and MR): per lane, group 2l then 2l+1, each a 16-weight
// partial in ascending k times its E4M3 scale; per wave and row, items ascending, a 64-lane sum
// (wave64_sum) when the wave leaves the row; per row, the 16 wave partials in wave order; times inv.
constexpr int kR32Rows = 20, kR32Depth = 2, kR32Item = 1152, kR32MaxMR = 3;
constexpr size_t r32_lds_bytes(int K, int MR) {
  return (size_t)MR * K * 2 + (size_t)kItemWaves * kR32Depth * kR32Item;
}

// 16 weights (8 nibble bytes in w0, w1, low nibble first) as eight 16-bit pairs in ascending k.
template <bool F16>
__device__ __forceinline__ void e2m1x16_decode(uint32_t w0, uint32_t w1, uint32_t* d) {
  if constexpr (F16) {
    d[0] = as_u32(e2m1x2_f16<0>(w0)); d[1] = as_u32(e2m1x2_f16<1>(w0));
    d[2] = as_u32(e2m1x2_f16<2>(w0)); d[3] = as_u32(e2m1x2_f16<3>(w0));
    d[4] = as_u32(e2m1x2_f16<0>(w1)); d[5] = as_u32(e2m1x2_f16<1>(w1));
    d[6] = as_u32(e2m1x2_f16<2>(w1)); d[7] = as_u32(e2m1x2_f16<3>(w1));
  } else {
    d[0] = __builtin_bit_cast(uint32_t, e2m1x2_bf16<0>(w0)); d[1] = __builtin_bit_cast(uint32_t, e2m1x2_bf16<1>(w0));
    d[2] = __builtin_bit_cast(uint32_t, e2m1x2_bf16<2>(w0)); d[3] = __builtin_bit_cast(uint32_t, e2m1x2_bf16<3>(w0));
    d[4] = __builtin_bit_cast(uint32_t, e2m1x2_bf16<0>(w1)); d[5] = __builtin_bit_cast(uint32_t, e2m1x2_bf16<1>(w1));
    d[6] = __builtin_bit_cast(uint32_t, e2m1x2_bf16<2>(w1)); d[7] = __builtin_bit_cast(uint32_t, e2m1x2_bf16<3>(w1));
  }
}
// acc + sum of the 16 products of decoded pairs d[0..7] and activation pairs x0, x1 in ascending k
template <bool F16>
__device__ __forceinline__ float dot16_pairs(const uint32_t* d, u32x4 x0, u32x4 x1, float acc) {
  const uint32_t xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if constexpr (F16) acc = dot2_f16(as_f16x2(d[i]), as_f16x2(xs[i]), acc);
    else acc = dot2_bf16(__builtin_bit_cast(bf16x2, d[i]), xs[i], acc);
  }
  return acc;
}

// ONE: the call has a single activation row (MR = 1; compile-time loop bound).
template <bool F16, int MR, bool ONE>
__global__ void __launch_bounds__(64 * kItemWaves) nv_lin_r32(int M, int K, int N, const uint16_t* __restrict__ xa,
                                                           const uint8_t* __restrict__ blk, float inv,
                                                           float* __restrict__ y) {
  constexpr int NW = kItemWaves, RB = kR32Rows, D = kR32Depth;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ float part[MR][NW][RB];
  const int U = K >> 5;                                // two-group units per row
  const int T = (U + 63) >> 6;                         // 32-record slots per row
  const uint32_t rb = (uint32_t)(K >> 6) * 36u;        // a multiple of 16
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NI = RB * T;
  const int nk = NI > wv ? (NI - wv + NW - 1) / NW : 0;
  const uint32_t lds0 = (uint32_t)(uintptr_t)lds;
  const uint32_t abytes = (uint32_t)K * 2u;            // one activation row
  const uint32_t ring = lds0 + MR * abytes + (uint32_t)wv * D * kR32Item;
  const uint8_t* ringp = lds + MR * abytes + wv * D * kR32Item;
  auto rowof = [&](int i) { return (int)blockIdx.x + (int)gridDim.x * i; };
  // copies of an item: chunk c < 72 at 1152 t + 16 c of the row; chunks past the row's end (last slot)
  // are clamped to its last chunk: in bounds, and they belong to units >= U, never used
  const uint32_t q0 = 16u * lane, q1 = 16u * (64 + (lane & 7));
  // the lane's unit inside an item: nibbles at 36 (l / 2) + 4 + 16 (l % 2), scale bytes at 36 (l / 2) + 2 (l % 2)
  const uint32_t qoff = (uint32_t)(lane >> 1) * 36u + 4u + 16u * (lane & 1);
  const uint32_t soff = (uint32_t)(lane >> 1) * 36u + 2u * (lane & 1);
  const int nslot = U * 4;                             // 16-byte activation pieces per row
  static_assert(!ONE || MR == 1, "single-row calls take one row per pass");
  const int Mloop = ONE ? 1 : M;
  for (int m0 = 0; m0 < Mloop; m0 += MR) {
    if (m0) __syncthreads();                           // the previous pass's LDS reads are done
    for (int i = threadIdx.x; i < MR * NW * RB; i += blockDim.x) (&part[0][0][0])[i] = 0.f;
    // activation rows m0 .. m0+MR-1 (past M: row M-1 again, never stored), piece-major: LDS slot
    // s = q U + u of row r holds piece 4 u + q of the row
#pragma unroll
    for (int r = 0; r < MR; ++r) {
      const uint16_t* xm = xa + (size_t)min(m0 + r, M - 1) * K;
      for (int j = 0; 64 * (wv + NW * j) < nslot; ++j) {
        const int sl = 64 * (wv + NW * j) + lane;
        if (sl < nslot) {
          const int q = sl / U, u = sl - q * U;
          lds_copy16((uint32_t)(4 * u + q) * 16u, xm,
                     __builtin_amdgcn_readfirstlane(lds0 + r * abytes + 1024u * (wv + NW * j)));
        }
      }
    }
    int lg = wv / T, lt = wv - (wv / T) * T, lk = 0;
    auto issue = [&](int stage) {
      const uint32_t st = ring + stage * kR32Item;
      const uint8_t* rowp = blk + (size_t)min(rowof(lg), N - 1) * rb;   // 64-bit row base, 32-bit offsets in the row
      const uint32_t off = 1152u * lt;
      lds_copy16_nt(min(off + q0, rb - 16u), rowp, __builtin_amdgcn_readfirstlane(st));
      if (lane < 8) lds_copy16_nt(min(off + q1, rb - 16u), rowp, __builtin_amdgcn_readfirstlane(st + 1024));
      ++lk;
      if (lk < nk) {                                   // past the wave's last item: repeat it (never used)
        lt += NW;
        while (lt >= T) { lt -= T; ++lg; }
      }
    };
#pragma unroll
    for (int d = 0; d < D; ++d) issue(d);
    wait_vmem<2 * D>();                                // this wave's activation copies landed ...
    __syncthreads();                                   // ... and every wave's
    float acc[MR];
#pragma unroll
    for (int r = 0; r < MR; ++r) acc[r] = 0.f;
    int cur = -1;
    auto flush = [&]() {
      if (cur < 0) return;
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const float v = wave64_sum(acc[r]);
        acc[r] = 0.f;
        if (lane == 0) part[r][wv][cur] = v;
      }
    };
    int cg = wv / T, ct = wv - (wv / T) * T;
    for (int k = 0; k < nk; ++k) {
      const int stage = k & (D - 1);
      wait_vmem<2 * (D - 1)>();                        // item k's two copies landed
      const int gi = cg, u = lane + 64 * ct;
      ct += NW;
      while (ct >= T) { ct -= T; ++cg; }
      if (gi != cur) {
        flush();
        cur = gi;
      }
      if (u < U) {
        const uint8_t* sp = ringp + stage * kR32Item;
        const uint32_t* wp = reinterpret_cast<const uint32_t*>(sp + qoff);
        const uint32_t w0 = wp[0], w1 = wp[1], w2 = wp[2], w3 = wp[3];
        const uint32_t sc = *reinterpret_cast<const uint16_t*>(sp + soff);
        const float s0 = e4m3_byte_f32<0>(sc), s1 = e4m3_byte_f32<1>(sc);
        if constexpr (MR == 1) {                       // decode fused into the dot products
          u32x4 xv[4];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) xv[qq] = *reinterpret_cast<const u32x4*>(lds + ((size_t)qq * U + u) * 16);
          const float p0 = F16 ? dot16_e2m1_f16(w0, w1, xv[0], xv[1], 0.f) : dot16_e2m1_bf16(w0, w1, xv[0], xv[1], 0.f);
          const float p1 = F16 ? dot16_e2m1_f16(w2, w3, xv[2], xv[3], 0.f) : dot16_e2m1_bf16(w2, w3, xv[2], xv[3], 0.f);
          acc[0] = fmaf(p0, s0, acc[0]);
          acc[0] = fmaf(p1, s1, acc[0]);
        } else {                                       // groups 2l and 2l+1 decoded once for all rows
          uint32_t d0[8], d1[8];
          e2m1x16_decode<F16>(w0, w1, d0);
          e2m1x16_decode<F16>(w2, w3, d1);
#pragma unroll
          for (int r = 0; r < MR; ++r) {
            const uint8_t* ar = lds + r * abytes;
            u32x4 xv[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) xv[qq] = *reinterpret_cast<const u32x4*>(ar + ((size_t)qq * U + u) * 16);
            const float p0 = dot16_pairs<F16>(d0, xv[0], xv[1], 0.f);
            const float p1 = dot16_pairs<F16>(d1, xv[2], xv[3], 0.f);
            acc[r] = fmaf(p0, s0, acc[r]);
            acc[r] = fmaf(p1, s1, acc[r]);
          }
        }
      }
      wait_lds();                                      // the stage's LDS reads are done before its refill
      issue(stage);                                    // item k + D
    }
    flush();
    wait_vmem<0>();                                    // trailing copies land before the LDS is reused
    __syncthreads();
    if (threadIdx.x < RB) {
      const int n = rowof(threadIdx.x);
      if (n < N) {
#pragma unroll
        for (int r = 0; r < MR; ++r) {
          if (m0 + r < M) {
            float v = 0.f;
            for (int ww = 0; ww < NW; ++ww) v += part[r][ww][threadIdx.x];
            y[(size_t)(m0 + r) * N + n] = v * inv;
          }
        }
      }
    }
  }
}

template <auto KERN>
bool lds_ok(size_t bytes) {
  return bytes <= 64 * 1024 || raise_lds_limit<KERN>();
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
  if (gu) return xt == X_BF16 && (K / 16 + 63) / 64 <= 8;
  if (xt != X_F32 && K % 256 == 0 && r32_lds_bytes(K, 1) <= kMaxItemLds) return true;
  return (size_t)K * (xt == X_F32 ? 4 : 2) <= kMaxItemLds;
}

hipError_t launch_fast_fp8(int M, int K, int N, const void* x, XType xt, const uint8_t* w0, const float* s0,
                           const uint8_t* w1, const float* s1, float* y, hipStream_t st) {
  if (w1 != nullptr) {
    const int CH = (K / 16 + 63) / 64;
    const dim3 grid((N + kRowWaves - 1) / kRowWaves), block(64 * kRowWaves);
    const size_t lds = (size_t)K * 2;
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    switch (CH) {
#define WQ_CASE(n)                                                                                         \
  case n:                                                                                                  \
    if (M == 1) hipLaunchKernelGGL((fp8_gu_row<n, true>), grid, block, lds, st, M, K, N, xb, w0, s0, w1, s1, y); \
    else hipLaunchKernelGGL((fp8_gu_row<n, false>), grid, block, lds, st, M, K, N, xb, w0, s0, w1, s1, y);      \
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
    if (!lds_ok<fp8_lin_items<T, O>>(lds)) return hipErrorInvalidValue;                                     \
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
                             const uint8_t* b1, float inv1, void* y, bool y16, hipStream_t st) {
  if (b1 != nullptr) {
    const int CH = (K / 16 + 63) / 64;
    const dim3 grid((N + kRowWaves - 1) / kRowWaves), block(64 * kRowWaves);
    const size_t lds = (size_t)K * 2;
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
    switch (CH) {
#define WQ_CASE(n)                                                                                           \
  case n:                                                                                                    \
    if (M == 1 && y16) hipLaunchKernelGGL((nv_gu_grp<n, true, true>), grid, block, lds, st, M, K, N, xb, b0, inv0, b1, inv1, y);  \
    else if (M == 1) hipLaunchKernelGGL((nv_gu_grp<n, true, false>), grid, block, lds, st, M, K, N, xb, b0, inv0, b1, inv1, y); \
    else if (y16) hipLaunchKernelGGL((nv_gu_grp<n, false, true>), grid, block, lds, st, M, K, N, xb, b0, inv0, b1, inv1, y);   \
    else hipLaunchKernelGGL((nv_gu_grp<n, false, false>), grid, block, lds, st, M, K, N, xb, b0, inv0, b1, inv1, y);           \
    break;
      WQ_CASE(1) WQ_CASE(2) WQ_CASE(3) WQ_CASE(4) WQ_CASE(5) WQ_CASE(6) WQ_CASE(7) WQ_CASE(8)
#undef WQ_CASE
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (y16) return hipErrorInvalidValue;                // a single linear writes float32
  float* yf = reinterpret_cast<float*>(y);
  if (xt != X_F32 && K % 256 == 0 && r32_lds_bytes(K, 1) <= kMaxItemLds) {
    // rows per pass: as many as fit (at most kR32MaxMR), never more than M
    int mr = 1;
    while (mr < kR32MaxMR && mr < M && r32_lds_bytes(K, mr + 1) <= kMaxItemLds) ++mr;
    const size_t lds = r32_lds_bytes(K, mr);
    const dim3 grid((N + kR32Rows - 1) / kR32Rows), block(64 * kItemWaves);
    const uint16_t* xb = reinterpret_cast<const uint16_t*>(x);
#define WQ_LAUNCH(F, R, O)                                                                                   \
  do {                                                                                                       \
    if (!lds_ok<nv_lin_r32<F, R, O>>(lds)) return hipErrorInvalidValue;                                      \
    hipLaunchKernelGGL((nv_lin_r32<F, R, O>), grid, block, lds, st, M, K, N, xb, b0, inv0, yf);              \
  } while (0)
#define WQ_MR(F)                                  \
  do {                                            \
    if (M == 1) WQ_LAUNCH(F, 1, true);            \
    else if (mr == 1) WQ_LAUNCH(F, 1, false);     \
    else if (mr == 2) WQ_LAUNCH(F, 2, false);     \
    else WQ_LAUNCH(F, 3, false);                  \
  } while (0)
    if (xt == X_F16) WQ_MR(true);
    else WQ_MR(false);
#undef WQ_MR
#undef WQ_LAUNCH
    return hipGetLastError();
  }
  const size_t lds = (size_t)K * (xt == X_F32 ? 4 : 2);
  const dim3 grid((N + kItemRows - 1) / kItemRows), block(64 * kItemWaves);
#define WQ_LAUNCH(T, O, F)                                                                                   \
  do {                                                                                                       \
    if (!lds_ok<nv_lin_grp<T, O, F>>(lds)) return hipErrorInvalidValue;                                      \
    hipLaunchKernelGGL((nv_lin_grp<T, O, F>), grid, block, lds, st, M, K, N, reinterpret_cast<const T*>(x), b0, inv0, yf); \
  } while (0)
  if (xt == X_F32) {
    if (M == 1) WQ_LAUNCH(float, true, false);
    else WQ_LAUNCH(float, false, false);
  } else if (xt == X_F16) {
    if (M == 1) WQ_LAUNCH(uint16_t, true, true);
    else WQ_LAUNCH(uint16_t, false, true);
  } else {
    if (M == 1) WQ_LAUNCH(uint16_t, true, false);
    else WQ_LAUNCH(uint16_t, false, false);
  }
#undef WQ_LAUNCH
  return hipGetLastError();
}

}  // namespace wq
