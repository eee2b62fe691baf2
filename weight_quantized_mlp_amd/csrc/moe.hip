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
// Kernel 1 (W13 + SwiGLU): one workgroup per (route, 8 consecutive n).  A wave holds
// four 16-lane row groups: (gate n, up n, gate n+1, up n+1); lane j of a group owns
// the groups of 32 k  g = j, j+16, ...: one coalesced 16-byte code load per group plus
// its scale and zero.  x sits in LDS, permuted so that each dword holds the pair
// (k, k+4) that matches the nibble extraction.  Order: per lane, groups ascending,
// inside a group 16 dot2 steps ascending; then a butterfly over the 16 lanes.
// Kernel 2 (W2 + ordered sum): one workgroup per 32 outputs, one wave per route reading the
// route's 32 rows as contiguous 16-byte group pieces; per (route, output) the group partials
// are added in group order and rounded to float16; then 32 threads sum the routes in order
// with fmaf.
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
// 243 KB W2 expert (3-byte metadata) and most of a 4-byte one.
constexpr int kPrefetchPerThread = 3;   // (the end-of-kernel asm below names three)

template <int ML, int GPL>
__global__ void __launch_bounds__(256) awq_w13_kernel(int E, int H, int I, const uint16_t* __restrict__ x,
                                                      const int32_t* __restrict__ ids,
                                                      const uint8_t* __restrict__ bank, AwqLayout L,
                                                      uint16_t* __restrict__ act,
                                                      const uint8_t* __restrict__ w2bank, int64_t w2_expert_bytes) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int r = blockIdx.x;
  const int nb = blockIdx.y * 8;
  const int e = ids[r];
  const int tid = threadIdx.x;
  if (e < 0 || e >= E) {  // invalid id: zero act row, no contribution
    if (tid < 8 && nb + tid < I) act[(size_t)r * I + nb + tid] = 0;
    return;
  }
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
      const int g = min(j + 16 * i, G - 1);
      const int64_t mi = (int64_t)row * G + g;
      c[i] = *reinterpret_cast<const u32x4*>(codes + 16 * g);
      sraw[i] = scales[mi];
      mraw[i] = group_meta2_raw<ML>(expert, L, mi);
    }
#pragma unroll
    for (int i = 0; i < kPrefetchPerThread; ++i)
      pf[i] = w2e[min(u0 + tid + 256 * i, (int64_t)w2_units - 1)];   // past the share: repeats a byte range
    stage_pairs(lds, x, H, 1, 0);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      if (j + 16 * i < G) {
        const _Float16 sv = f16_from_bits((uint16_t)sraw[i]);
        acc = awq_group_dot(c[i], sv, group_bias_from_raw<ML>(mraw[i], sv), lds + j * kGrpStride + 16 * i * kGrpStride,
                            acc);
      }
    }
  } else {
    stage_pairs(lds, x, H, 1, 0);
    __syncthreads();
    if (n < I) {
      for (int g = j; g < G; g += 16) {
        const u32x4 c = *reinterpret_cast<const u32x4*>(codes + 16 * g);
        const int64_t mi = (int64_t)row * G + g;
        const _Float16 s = f16_from_bits(scales[mi]);
        const _Float16 b = group_bias<ML>(expert, L, mi, s);
        acc = awq_group_dot(c, s, b, lds + g * kGrpStride, acc);
      }
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
          live ? awq_group_dot(c[j], sv, group_bias_from_raw<ML>(mraw[j], sv), lds + r * act_bytes + g * kGrpStride, 0.f)
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

// Kernel 2, row-pair form (G = I/32 <= 8): one workgroup per 32 outputs, one wave per route; lane l handles
// row o0 + (l & 31) and half h = l >> 5 of its groups (h = 0: groups [0, GH), h = 1: [GH, G), GH = ceil(G/2)).
// The lane loads its groups' codes and metadata and its route's act for those groups straight into
// registers (act is read by all 32 lanes of a half at the same addresses), so nothing is staged in LDS
// before the dot products.  Order per (route, row): each group's 16 dot2 steps from 0, the group partials
// of a half added in group order, then half 0 + half 1, rounded to float16; one barrier, then 32 threads
// add the routes in order with fmaf.
constexpr int kMaxRoutes = 16;   // the entry point's top-k limit (one wave per route, 1024 threads)

template <int ML, int GH>
__global__ void __launch_bounds__(1024) awq_w2_pair_kernel(int E, int topk, int H, int I,
                                                           const int32_t* __restrict__ ids,
                                                           const float* __restrict__ router_w,
                                                           const uint8_t* __restrict__ bank, AwqLayout L,
                                                           const uint16_t* __restrict__ act, uint16_t* __restrict__ out) {
  __shared__ float ys[kMaxRoutes][32];
  const int G = I >> 5;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int r = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int row = lane & 31, h = lane >> 5;
  const int o = blockIdx.x * 32 + row;
  const int g0 = h * GH;
  const int ng = h ? G - GH : GH;                     // this half's group count (0 < ng <= GH)
  const int e = ids[r];
  const bool live = e >= 0 && e < E;
  const uint8_t* expert = bank + (size_t)(live ? e : 0) * L.expert_bytes;
  const uint8_t* codes = expert + (size_t)o * (I >> 1);
  const uint16_t* scales = reinterpret_cast<const uint16_t*>(expert + L.scale_off);
  const u32x4* ar = reinterpret_cast<const u32x4*>(act + (size_t)r * I);   // 8 halves per 16-byte chunk
  // unconditional loads from clamped addresses (an invalid id reads expert 0; groups past this half's
  // count read group G-1), so that every load of the lane is in flight before any is used
  u32x4 c[GH], a[GH][4];
  uint32_t sraw[GH], mraw[GH];
#pragma unroll
  for (int i = 0; i < GH; ++i) {
    const int g = min(g0 + i, G - 1);
    const int64_t mi = (int64_t)o * G + g;
    c[i] = *reinterpret_cast<const u32x4*>(codes + 16 * g);
    sraw[i] = scales[mi];
    mraw[i] = group_meta2_raw<ML>(expert, L, mi);
  }
#pragma unroll
  for (int i = 0; i < GH; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) a[i][q] = ar[4 * min(g0 + i, G - 1) + q];
  // every group's partial is computed (a group past this half's count from its clamped copy) and only the
  // valid ones are added, in group order: with the uses unconditional the loads above stay where they are
  // (a conditional use lets the compiler sink its loads into the condition, one round trip each)
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < GH; ++i) {
    const _Float16 sv = f16_from_bits((uint16_t)sraw[i]), bv = group_bias_from_raw<ML>(mraw[i], sv);
    const f16x2 s2 = {sv, sv}, b2 = {bv, bv};
    float p = 0.f;
#pragma unroll
    for (int dw = 0; dw < 4; ++dw) {
      const u32x4 v = a[i][dw];               // k = 8 dw .. 8 dw + 7 of the group, natural order
      const uint32_t x04 = (v.x & 0xffffu) | (v.z << 16), x15 = (v.x >> 16) | (v.z & 0xffff0000u);
      const uint32_t x26 = (v.y & 0xffffu) | (v.w << 16), x37 = (v.y >> 16) | (v.w & 0xffff0000u);
      const uint32_t w = c[i][dw];
      p = dot2_f16(awq_pair<0>(w, s2, b2), as_f16x2(x04), p);
      p = dot2_f16(awq_pair<1>(w, s2, b2), as_f16x2(x15), p);
      p = dot2_f16(awq_pair<2>(w, s2, b2), as_f16x2(x26), p);
      p = dot2_f16(awq_pair<3>(w, s2, b2), as_f16x2(x37), p);
    }
    acc = i < ng ? acc + p : acc;
  }
  const float other = __shfl_xor(acc, 32, 64);      // the row's other half
  if (h == 0 && r < topk) ys[r][row] = live ? (float)(_Float16)(acc + other) : 0.f;   // per-route float16
  __syncthreads();
  if (tid < 32) {
    float sum = 0.f;
    for (int rr = 0; rr < topk; ++rr) {
      const int er = ids[rr];
      if (er >= 0 && er < E) sum = fmaf(router_w[rr], ys[rr][tid], sum);
    }
    out[blockIdx.x * 32 + tid] = __builtin_bit_cast(uint16_t, (_Float16)sum);
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
  const int gpl13 = (H / 32 + 15) / 16;  // groups per lane in W13
#define WQ_W13(ML, P)                                                                                     \
  hipLaunchKernelGGL((awq_w13_kernel<ML, P>), g13, dim3(256), lds13, st, E, H, I, x, ids, w13, L13, act, w2, \
                     L2.expert_bytes)
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
  const int gh = (I / 32 + 1) / 2;                  // groups per half row in the row-pair form
  if (gh <= 4) {
    const dim3 g2(H / 32);
#define WQ_W2P(ML, GH)                                                                                           \
  hipLaunchKernelGGL((awq_w2_pair_kernel<ML, GH>), g2, dim3(64 * topk), 0, st, E, topk, H, I, ids, router_w, w2, L2, \
                     act, out)
#define WQ_W2P_ML(ML)              \
  switch (gh) {                    \
    case 1: WQ_W2P(ML, 1); break;  \
    case 2: WQ_W2P(ML, 2); break;  \
    case 3: WQ_W2P(ML, 3); break;  \
    default: WQ_W2P(ML, 4); break; \
  }
    if (meta_layout == 3) {
      WQ_W2P_ML(3)
    } else {
      WQ_W2P_ML(4)
    }
#undef WQ_W2P_ML
#undef WQ_W2P
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
