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
// The step moves ~7 MB, about 28 KB per CU, so it is bound by memory latency: both kernels
// issue all of a lane's weight loads at once (compile-time group count per lane) before
// staging the activations, so weights and activations arrive in one round trip.
// Kernel 1 (W13 + SwiGLU): one workgroup per (route, 4 consecutive n), a wave per n holding two
// 32-lane row groups (gate n, up n); for H < 1056 one per (route, 8 n) with four 16-lane row groups
// (gate n, up n, gate n+1, up n+1).  Lane j of a group owns the groups of 32 k  g = j, j+RL, ...: one
// coalesced 16-byte code load per group plus its scale and zero.  x sits in LDS, permuted so that each
// dword holds the pair (k, k+4) that matches the nibble extraction.  Order: per lane, groups ascending,
// inside a group 16 dot2 steps ascending; then the 16-lane rows summed by DPP (lane^1, lane^2, half-row
// and row mirrors) and, for 32-lane groups, the two rows added.
// Kernel 2 (W2 + ordered sum): for I <= 256 one workgroup per 16 outputs (32 when I <= 64), one
// wave per route, four (two) lanes per output row, each with a contiguous part of the row's groups;
// per (route, output) the parts' partials are combined pairwise and rounded to float16; then the
// workgroup's outputs sum the routes in order with fmaf.  Wider I: a workgroup per 32 outputs reading
// the rows as contiguous 16-byte pieces, or one row per thread.
// Decode (all kernels): each pair of nibbles becomes two float16 values with one v_and_or_b32, one
// exact subtraction and one packed fma (three-operand forms: masks in scalar registers).
#include <algorithm>
#include <utility>

#include "dev_common.h"
#include "launch.h"

namespace wq {

namespace {

constexpr int kGrpStride = 80;  // 32 f16 (64 B) + 16 B padding per group of 32 in LDS

// Copy rows of n16 halves (nrows contiguous rows starting at src) into LDS groups of 32 in (k, k+4)
// pair order, row r at lds + r * row_bytes.  The work is flattened over all rows, and each thread issues
// up to kStageAhead of its 16-byte loads before writing any of them (one memory round trip instead of
// one per row or per loop pass); any remainder goes through a plain loop.
constexpr int kStageAhead = 4;

__device__ __forceinline__ void stage_block(uint8_t* lds, int row_bytes, int bpr, int b, uint4 v) {
  const int rr = b / bpr, blk = b - rr * bpr;
  uint4 o;
  o.x = (v.x & 0xffffu) | (v.z << 16);
  o.y = (v.x >> 16) | (v.z & 0xffff0000u);
  o.z = (v.y & 0xffffu) | (v.w << 16);
  o.w = (v.y >> 16) | (v.w & 0xffff0000u);
  *reinterpret_cast<uint4*>(lds + rr * row_bytes + (blk >> 2) * kGrpStride + (blk & 3) * 16) = o;
}

__device__ __forceinline__ void stage_pairs(uint8_t* lds, const uint16_t* __restrict__ src, int n16, int nrows,
                                            int row_bytes) {
  const int bpr = n16 >> 3;  // 8-k blocks per row
  const int nb = nrows * bpr;
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4 v[kStageAhead];
#pragma unroll
  for (int j = 0; j < kStageAhead; ++j) {
    const int b = threadIdx.x + j * (int)blockDim.x;
    if (b < nb) v[j] = s4[b];
  }
#pragma unroll
  for (int j = 0; j < kStageAhead; ++j) {
    const int b = threadIdx.x + j * (int)blockDim.x;
    if (b < nb) stage_block(lds, row_bytes, bpr, b, v[j]);
  }
  for (int b = threadIdx.x + kStageAhead * (int)blockDim.x; b < nb; b += blockDim.x)
    stage_block(lds, row_bytes, bpr, b, s4[b]);
}

// Dot product of one group of 32 codes (16 bytes) with 32 LDS activations.
__device__ __forceinline__ float awq_group_dot(const u32x4 c, _Float16 s, _Float16 b, const uint8_t* xg,
                                               float acc, const AwqDecode& dc) {
  const f16x2 s2 = {s, s};
  const f16x2 b2 = {b, b};
#pragma unroll
  for (int dw = 0; dw < 4; ++dw) {
    const u32x4 xv = *reinterpret_cast<const u32x4*>(xg + 16 * dw);
    f16x2 p[4];
    awq_quad(c[dw], s2, b2, dc, p);
    acc = dot2_f16(p[0], as_f16x2(xv.x), acc);
    acc = dot2_f16(p[1], as_f16x2(xv.y), acc);
    acc = dot2_f16(p[2], as_f16x2(xv.z), acc);
    acc = dot2_f16(p[3], as_f16x2(xv.w), acc);
  }
  return acc;
}

template <int ML>
__device__ __forceinline__ _Float16 group_bias(const uint8_t* expert, const AwqLayout& L, int64_t idx, _Float16 s) {
  if constexpr (ML == 3) return awq_bias(expert[L.meta2_off + idx], s);
  else return f16_from_bits(reinterpret_cast<const uint16_t*>(expert + L.meta2_off)[idx]);
}
// The group's second metadata element as stored (zero byte or bias bits), and the bias made from it
// later: loading the raw values first lets every load of a lane be issued before any of them is used
// (a bias computed at load time makes the compiler wait for each group's metadata in turn).
template <int ML>
__device__ __forceinline__ uint32_t group_meta2_raw(const uint8_t* expert, const AwqLayout& L, int64_t idx) {
  if constexpr (ML == 3) return expert[L.meta2_off + idx];
  else return reinterpret_cast<const uint16_t*>(expert + L.meta2_off)[idx];
}
template <int ML>
__device__ __forceinline__ _Float16 group_bias_from_raw(uint32_t raw, _Float16 s) {
  if constexpr (ML == 3) return awq_bias(raw, s);
  else return f16_from_bits((uint16_t)raw);
}

// GPL: groups per lane (compile-time, so every weight load of a lane is issued at once before the
// activations are staged); 0 = runtime loop for shapes outside the unrolled range.
// W2 prefetch: while its own weight loads are in flight, each W13 workgroup also reads its share (one
// gridDim.y-th) of its route's W2 expert block, so that the W2 kernel finds those bytes in the
// memory-side cache instead of waiting a DRAM round trip.  The values only feed an empty asm at the end
// (kept live, never stored).  kPrefetchPerThread 16-byte loads per thread cover a 20-workgroup route of a
// 243 KB W2 expert (3-byte metadata) and most of a 4-byte one; loads past a workgroup's share repeat its
// last unit.
constexpr int kPrefetchPerThread = 3;   // (the end-of-kernel asm below names three)

template <int ML, int GPL, int RL>
__global__ void __launch_bounds__(256) awq_w13_kernel(int E, int H, int I, const uint16_t* __restrict__ x,
                                                      const int32_t* __restrict__ ids,
                                                      const uint8_t* __restrict__ bank, AwqLayout L,
                                                      uint16_t* __restrict__ act,
                                                      const uint8_t* __restrict__ w2bank, int64_t w2_expert_bytes) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const AwqDecode dc = awq_decode_consts();
  constexpr int NPW = 32 / RL;                         // n per wave: RL lanes per row, a gate and an up row each
  const int r = blockIdx.x;
  const int nb = blockIdx.y * 4 * NPW;
  const int e = ids[r];
  const int tid = threadIdx.x;
  if (e < 0 || e >= E) {  // invalid id: zero act row, no contribution
    if (tid < 4 * NPW && nb + tid < I) act[(size_t)r * I + nb + tid] = 0;
    return;
  }
  const int lane = tid & 63;
  const int j = lane & (RL - 1);
  const int rg = lane / RL;
  const int n = nb + NPW * (tid >> 6) + (rg >> 1);
  const int row = (rg & 1) ? n + I : n;
  const int G = H >> 5;
  const uint8_t* expert = bank + (size_t)e * L.expert_bytes;
  const uint8_t* codes = expert + (size_t)row * (H >> 1);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(expert + L.scale_off);
  float acc = 0.f;
  u32x4 pf[kPrefetchPerThread];
  // this workgroup's share of the route's W2 expert block, 16-byte units [u0, u1)
  const int64_t w2_units = w2_expert_bytes >> 4;
  const int64_t per_wg = (w2_units + gridDim.y - 1) / gridDim.y;
  const int64_t u0 = (int64_t)blockIdx.y * per_wg;
  const u32x4* w2e = reinterpret_cast<const u32x4*>(w2bank + (size_t)e * w2_expert_bytes);
  if constexpr (GPL > 0) {
    // Every load is unconditional, from a clamped in-bounds address (groups past G read group G-1 and are
    // not used): a load under a condition leaves a join at which the compiler copies the loaded register,
    // and the copy waits for the load, which serialises the memory round trips.  (I is a multiple of 8, so
    // every row n of the workgroup exists.)
    u32x4 c[GPL];
    uint32_t sraw[GPL], mraw[GPL];
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int g = min(j + RL * i, G - 1);
      const int64_t mi = (int64_t)row * G + g;
      // each code byte is read once, RL lanes x 16 bytes per load (whole 128-byte lines when a row's
      // H / 2 bytes are, as at H = 2560): the non-temporal hint (rotating experts, H = 2560: step 9.45 ->
      // 8.9 us); not for the W2 read-ahead below, which is there to leave the W2 bytes in the cache
      c[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(codes + 16 * g));
      sraw[i] = scales[mi];
      mraw[i] = group_meta2_raw<ML>(expert, L, mi);
    }
#pragma unroll
    for (int i = 0; i < kPrefetchPerThread; ++i)
      pf[i] = w2e[min(u0 + tid + 256 * i, min(u0 + per_wg, w2_units) - 1)];
    stage_pairs(lds, x, H, 1, 0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      if (j + RL * i < G) {
        const _Float16 sv = f16_from_bits((uint16_t)sraw[i]);
        acc = awq_group_dot(c[i], sv, group_bias_from_raw<ML>(mraw[i], sv), lds + (j + RL * i) * kGrpStride, acc,
                            dc);
      }
    }
  } else {
    stage_pairs(lds, x, H, 1, 0);
    __syncthreads();
    if (n < I) {
      for (int g = j; g < G; g += RL) {
        const u32x4 c = *reinterpret_cast<const u32x4*>(codes + 16 * g);
        const int64_t mi = (int64_t)row * G + g;
        const _Float16 s = f16_from_bits(scales[mi]);
        const _Float16 b = group_bias<ML>(expert, L, mi, s);
        acc = awq_group_dot(c, s, b, lds + g * kGrpStride, acc, dc);
      }
    }
  }
  acc = row16_sum(acc);                                // the row's lanes: DPP within 16 lanes ...
  if constexpr (RL == 32) acc += __shfl_xor(acc, 16, 64);   // ... then the two halves
  const float u = __shfl_down(acc, RL, 64);
  if (j == 0 && (rg & 1) == 0 && n < I) {
    const float gh = (float)(_Float16)acc;
    const float uh = (float)(_Float16)u;
    const _Float16 a = (_Float16)(silu_f32(gh) * uh);
    act[(size_t)r * I + n] = __builtin_bit_cast(uint16_t, a);
  }
  if constexpr (GPL > 0)   // the prefetched W2 bytes, consumed by nothing (only the wait at the very end)
    asm volatile("" ::"v"(pf[0]), "v"(pf[1]), "v"(pf[2]));
}

// Kernel 2 (W2 + ordered sum): one workgroup per kW2Rows outputs, one wave per route.  Wave r reads the
// route's kW2Rows consecutive rows (kW2Rows * I/2 contiguous code bytes) as 16-byte pieces
// p = lane + 64 j: piece p is group p % G of row p / G, and since the metadata planes are row-major its
// scale and zero are element p of the block's metadata run, so every load is coalesced.  The group
// partials go through LDS; per (route, row) they are added in group order, rounded to float16, and
// kW2Rows threads add the routes in order.  PPL = pieces per lane (compile-time: all loads at once).
constexpr int kW2Rows = 32;

template <int ML, int PPL>
__global__ void __launch_bounds__(1024) awq_w2_kernel(int E, int topk, int H, int I,
                                                      const int32_t* __restrict__ ids,
                                                      const float* __restrict__ router_w,
                                                      const uint8_t* __restrict__ bank, AwqLayout L,
                                                      const uint16_t* __restrict__ act, uint16_t* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const AwqDecode dc = awq_decode_consts();
  const int G = I >> 5;
  const int act_bytes = G * kGrpStride;  // per route
  float* part = reinterpret_cast<float*>(lds + topk * act_bytes);  // [topk][kW2Rows][G]
  float* ys = part + topk * kW2Rows * G;                           // [topk][kW2Rows]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int r = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int o0 = blockIdx.x * kW2Rows;
  const int nrows = min(kW2Rows, H - o0);
  const int np = nrows * G;
  const int e = ids[r];
  const bool live = e >= 0 && e < E;
  const uint8_t* expert = bank + (size_t)(live ? e : 0) * L.expert_bytes;
  const uint8_t* codes = expert + (size_t)o0 * (I >> 1);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(expert + L.scale_off);
  const int64_t m0 = (int64_t)o0 * G;
  u32x4 c[PPL];
  uint32_t sraw[PPL], mraw[PPL];
  if (live) {
#pragma unroll
    for (int j = 0; j < PPL; ++j) {
      const int pc = lane + 64 * j;
      if (pc < np) {
        c[j] = *reinterpret_cast<const u32x4*>(codes + 16 * pc);
        sraw[j] = scales[m0 + pc];
        mraw[j] = group_meta2_raw<ML>(expert, L, m0 + pc);
      }
    }
  }
  stage_pairs(lds, act, I, topk, act_bytes);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < PPL; ++j) {
    const int pc = lane + 64 * j;
    if (pc < np) {
      const int g = pc % G;
      const _Float16 sv = f16_from_bits((uint16_t)sraw[j]);
      part[(r * kW2Rows) * G + pc] =
          live ? awq_group_dot(c[j], sv, group_bias_from_raw<ML>(mraw[j], sv), lds + r * act_bytes + g * kGrpStride, 0.f,
                               dc)
               : 0.f;
    }
  }
  __syncthreads();
  for (int i = tid; i < topk * nrows; i += blockDim.x) {
    const int rr = i / nrows, row = i - rr * nrows;
    const float* pp = part + (rr * kW2Rows + row) * G;
    float y = 0.f;
    for (int g = 0; g < G; ++g) y += pp[g];
    ys[rr * kW2Rows + row] = (float)(_Float16)y;  // per-route float16 materialisation
  }
  __syncthreads();
  if (tid < nrows) {
    float sum = 0.f;
    for (int rr = 0; rr < topk; ++rr) {
      const int er = ids[rr];
      if (er >= 0 && er < E) sum = fmaf(router_w[rr], ys[rr * kW2Rows + tid], sum);
    }
    out[o0 + tid] = __builtin_bit_cast(uint16_t, (_Float16)sum);
  }
}

// Kernel 2, row-part form (G = I/32 <= 8): one workgroup per RPW = 64/LPR outputs, one wave per route;
// LPR lanes share a row: lane l handles row o0 + l % RPW and part h = l / RPW of its groups (part h:
// groups [h GP, min((h+1) GP, G)), GP = ceil(G/LPR)).  The lane's code and metadata loads are issued
// first; act is staged in LDS in (k, k+4) pair order (all RPW lanes of a part read the same addresses),
// and the routes' effective weights (0 for an invalid id) go to LDS beside it, all under one barrier.
// Order per (route, row): each group's 16 dot2 steps from 0, a part's group partials added in group order,
// the parts combined pairwise ((p0 + p1) + (p2 + p3) ...), rounded to float16; after a second barrier RPW
// threads add the routes in order with fmaf (an invalid route adds 0 * 0, which leaves the sum as it is).
constexpr int kMaxRoutes = 16;   // the entry point's top-k limit (one wave per route, 1024 threads)

template <int ML, int GP>
struct W2Lane {
  u32x4 c[GP];
  uint32_t sraw[GP], mraw[GP];
};

// The lane's unconditional loads from clamped addresses (an invalid id reads expert 0; groups past the
// part's count read group G-1), so that every load of the lane is in flight before any is used.
template <int ML, int GP>
__device__ __forceinline__ void w2_lane_load(W2Lane<ML, GP>& t, const uint8_t* expert, const AwqLayout& L, int o,
                                             int g0, int G, int I) {
  const uint8_t* codes = expert + (size_t)o * (I >> 1);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(expert + L.scale_off);
#pragma unroll
  for (int i = 0; i < GP; ++i) {
    const int g = min(g0 + i, G - 1);
    const int64_t mi = (int64_t)o * G + g;
    t.c[i] = *reinterpret_cast<const u32x4*>(codes + 16 * g);
    t.sraw[i] = scales[mi];
    t.mraw[i] = group_meta2_raw<ML>(expert, L, mi);
  }
}

// The route's value for the lane's row: group partials of the part in order, then the parts combined.
// Every partial is computed (a clamped group from its copy) and only the part's own are added, so that
// the uses are unconditional and the loads above stay where they are.
template <int ML, int GP, int LPR>
__device__ __forceinline__ float w2_lane_dot(const W2Lane<ML, GP>& t, const uint8_t* arow, int g0, int ng, int G,
                                             const AwqDecode& dc) {
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < GP; ++i) {
    const _Float16 sv = f16_from_bits((uint16_t)t.sraw[i]);
    const float p = awq_group_dot(t.c[i], sv, group_bias_from_raw<ML>(t.mraw[i], sv),
                                  arow + min(g0 + i, G - 1) * kGrpStride, 0.f, dc);
    acc = i < ng ? acc + p : acc;
  }
#pragma unroll
  for (int off = 64 / LPR; off < 64; off *= 2) acc += __shfl_xor(acc, off, 64);
  return acc;
}

template <int ML, int LPR, int GP>
__global__ void __launch_bounds__(1024) awq_w2_part_kernel(int E, int topk, int H, int I,
                                                           const int32_t* __restrict__ ids,
                                                           const float* __restrict__ router_w,
                                                           const uint8_t* __restrict__ bank, AwqLayout L,
                                                           const uint16_t* __restrict__ act, uint16_t* __restrict__ out) {
  constexpr int RPW = 64 / LPR;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];   // act rows, pair order
  __shared__ float ys[kMaxRoutes][RPW];
  __shared__ float wr[kMaxRoutes];
  const int G = I >> 5;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int r = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane % RPW, h = lane / RPW;
  const int o = blockIdx.x * RPW + row;
  const int g0 = h * GP;
  const int ng = min(max(G - g0, 0), GP);
  const int e = ids[r];
  const bool live = e >= 0 && e < E;
  W2Lane<ML, GP> t;
  w2_lane_load(t, bank + (size_t)(live ? e : 0) * L.expert_bytes, L, o, g0, G, I);
  if (tid < topk) {
    const int er = ids[tid];
    wr[tid] = er >= 0 && er < E ? router_w[tid] : 0.f;
  }
  stage_pairs(lds, act, I, topk, G * kGrpStride);
  __syncthreads();
  const AwqDecode dc = awq_decode_consts();
  const float y = w2_lane_dot<ML, GP, LPR>(t, lds + r * G * kGrpStride, g0, ng, G, dc);
  if (h == 0) ys[r][row] = live ? (float)(_Float16)y : 0.f;   // per-route float16
  __syncthreads();
  if (tid < RPW) {
    float sum = 0.f;
    for (int rr = 0; rr < topk; ++rr) sum = fmaf(wr[rr], ys[rr][tid], sum);
    out[blockIdx.x * RPW + tid] = __builtin_bit_cast(uint16_t, (_Float16)sum);
  }
}

// General W2 form (any I the entry point accepts): thread (r, o) computes y_r[o] over its row's groups
// with act[r] broadcast from LDS, rounds it to float16; then 32 threads sum the routes in order.
template <int ML>
__global__ void __launch_bounds__(512) awq_w2_rows_kernel(int E, int topk, int H, int I,
                                                     const int32_t* __restrict__ ids,
                                                     const float* __restrict__ router_w,
                                                     const uint8_t* __restrict__ bank, AwqLayout L,
                                                     const uint16_t* __restrict__ act, uint16_t* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const AwqDecode dc = awq_decode_consts();
  const int G = I >> 5;
  const int act_bytes = G * kGrpStride;  // per route
  float* ys = reinterpret_cast<float*>(lds + topk * act_bytes);  // [topk][32]
  const int tid = threadIdx.x;
  stage_pairs(lds, act, I, topk, act_bytes);
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
        acc = awq_group_dot(c, s, b, lds + r * act_bytes + g * kGrpStride, acc, dc);
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

// W2 row-part form for G groups per row: lanes per row and groups per lane part.  Two lanes per row for
// G <= 2, else kW2Lanes (more, smaller workgroups spread the step's dot products over more CUs).
constexpr int kW2Lanes = 4;
struct W2Form {
  int lpr, gp;
};
W2Form w2_form(int G) {
  if (G <= 2) return {2, 1};
  return {kW2Lanes, (G + kW2Lanes - 1) / kW2Lanes};
}

// Calls f(integral_constant<int, v>) for the v in Is... equal to x.
template <typename F, int... Is>
void dispatch_int(int x, F&& f, std::integer_sequence<int, Is...>) {
  (void)((x == Is ? (f(std::integral_constant<int, Is>{}), true) : false) || ...);
}

// f(ml, lpr, gp) with compile-time metadata layout, lanes per row and groups per part.
template <typename F>
void dispatch_w2(int meta_layout, W2Form form, F&& f) {
  static_assert(kW2Lanes == 4, "the part counts below assume four lanes per row (G <= 8: one or two groups)");
  auto with_ml = [&](auto ml) {
    if (form.lpr == 2) {
      f(ml, std::integral_constant<int, 2>{}, std::integral_constant<int, 1>{});
    } else {
      dispatch_int(form.gp, [&](auto gp) { f(ml, std::integral_constant<int, kW2Lanes>{}, gp); },
                   std::integer_sequence<int, 1, 2>{});
    }
  };
  if (meta_layout == 3) with_ml(std::integral_constant<int, 3>{});
  else with_ml(std::integral_constant<int, 4>{});
}

}  // namespace

hipError_t launch_moe_awq_m1(int E, int topk, int H, int I, const uint16_t* x, const int32_t* ids,
                             const float* router_w, const uint8_t* w13, const uint8_t* w2, int meta_layout,
                             uint16_t* act, uint16_t* out, hipStream_t st) {
  const AwqLayout L13 = awq_layout(2 * (int64_t)I, H, meta_layout);
  const AwqLayout L2 = awq_layout(H, I, meta_layout);
  const size_t lds13 = (size_t)(H / 32) * kGrpStride;
  // 32 lanes per row (4 n per workgroup) once a 16-lane row would hold 3 or more groups per lane
  const int rl = (H / 32 + 15) / 16 >= 3 ? 32 : 16;
  const dim3 g13(topk, (I + 128 / rl - 1) / (128 / rl));
  const int gpl13 = (H / 32 + rl - 1) / rl;  // groups per lane in W13
#define WQ_W13(ML, P)                                                                                          \
  if (rl == 32)                                                                                                \
    hipLaunchKernelGGL((awq_w13_kernel<ML, P, 32>), g13, dim3(256), lds13, st, E, H, I, x, ids, w13, L13, act, \
                       w2, L2.expert_bytes);                                                                   \
  else                                                                                                         \
    hipLaunchKernelGGL((awq_w13_kernel<ML, P, 16>), g13, dim3(256), lds13, st, E, H, I, x, ids, w13, L13, act, \
                       w2, L2.expert_bytes)
#define WQ_W13_ML(ML)                                                                     \
  switch (gpl13) {                                                                        \
    case 1: WQ_W13(ML, 1); break;                                                         \
    case 2: WQ_W13(ML, 2); break;                                                         \
    case 3: WQ_W13(ML, 3); break;                                                         \
    case 4: WQ_W13(ML, 4); break;                                                         \
    case 5: WQ_W13(ML, 5); break;                                                         \
    case 6: WQ_W13(ML, 6); break;                                                         \
    case 7: WQ_W13(ML, 7); break;                                                         \
    case 8: WQ_W13(ML, 8); break;                                                         \
    default: WQ_W13(ML, 0); break;                                                        \
  }
  if (meta_layout == 3) {
    WQ_W13_ML(3)
  } else {
    WQ_W13_ML(4)
  }
#undef WQ_W13_ML
#undef WQ_W13
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const size_t lds2 = (size_t)topk * (I / 32) * kGrpStride + (size_t)topk * kW2Rows * (I / 32 + 1) * 4;
  const int ppl2 = (kW2Rows * (I / 32) + 63) / 64;  // 16-byte pieces per lane in W2
  const int G2 = I / 32;                            // groups per W2 row
  if (G2 <= 8) {
    const W2Form f = w2_form(G2);
    const size_t ldsp = (size_t)topk * G2 * kGrpStride;
    const dim3 g2(H / (64 / f.lpr));
    auto go = [&](auto ml, auto lpr, auto gp) {
      hipLaunchKernelGGL((awq_w2_part_kernel<decltype(ml)::value, decltype(lpr)::value, decltype(gp)::value>), g2,
                         dim3(64 * topk), ldsp, st, E, topk, H, I, ids, router_w, w2, L2, act, out);
    };
    dispatch_w2(meta_layout, f, go);
  } else if (ppl2 <= 8 && lds2 <= 65536) {
    const dim3 g2((H + kW2Rows - 1) / kW2Rows);
#define WQ_W2(ML, P)                                                                                          \
  hipLaunchKernelGGL((awq_w2_kernel<ML, P>), g2, dim3(64 * topk), lds2, st, E, topk, H, I, ids, router_w, w2, L2, \
                     act, out)
#define WQ_W2_ML(ML)            \
  switch (ppl2) {               \
    case 1: WQ_W2(ML, 1); break; \
    case 2: WQ_W2(ML, 2); break; \
    case 3: WQ_W2(ML, 3); break; \
    case 4: WQ_W2(ML, 4); break; \
    case 5: WQ_W2(ML, 5); break; \
    case 6: WQ_W2(ML, 6); break; \
    case 7: WQ_W2(ML, 7); break; \
    default: WQ_W2(ML, 8); break; \
  }
    if (meta_layout == 3) {
      WQ_W2_ML(3)
    } else {
      WQ_W2_ML(4)
    }
#undef WQ_W2_ML
#undef WQ_W2
  } else {
    const size_t ldsr = (size_t)topk * (I / 32) * kGrpStride + (size_t)topk * 32 * 4;
    const int threads = (topk * 32 + 63) / 64 * 64;
    const dim3 g2((H + 31) / 32);
    if (meta_layout == 3)
      hipLaunchKernelGGL(awq_w2_rows_kernel<3>, g2, dim3(threads), ldsr, st, E, topk, H, I, ids, router_w, w2, L2,
                         act, out);
    else
      hipLaunchKernelGGL(awq_w2_rows_kernel<4>, g2, dim3(threads), ldsr, st, E, topk, H, I, ids, router_w, w2, L2,
                         act, out);
  }
  return hipGetLastError();
}

}  // namespace wq
