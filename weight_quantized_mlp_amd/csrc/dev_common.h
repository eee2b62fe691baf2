// Device-side helpers shared by the gfx950 kernels of this library.
//
// Element decoders use the CDNA4 conversion instructions.  Their semantics were
// established by exhaustive checks on gfx950:
//   * v_cvt_pk_f32_fp8 decodes OCP E4M3 ("fn": bias 7, NaN at S.1111.111) exactly;
//   * the v_cvt_scalef32_pk_* conversions take only the exponent of their float
//     scale operand (a power of two), so they are used with scale 1.0, where they
//     return the exact E2M1 / E4M3 value, and the E4M3 group / channel scale is
//     applied by a separate exact or single-rounding multiply.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
// three dwords at a 4-byte-aligned address (record windows of the NVFP4 decode; global loads need only
// dword alignment)
typedef uint32_t u32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x2 __attribute__((ext_vector_type(2)));

// ---- element decoders ---------------------------------------------------------------------
// Two E4M3 bytes (bytes 0,1 or 2,3 of w) -> two exact float32.
template <bool HI>
__device__ __forceinline__ f32x2 e4m3x2_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(w, HI);
}
// Two E4M3 bytes -> two exact bf16 / f16 (every E4M3 value is representable in both).
template <bool HI>
__device__ __forceinline__ bf16x2 e4m3x2_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
}
template <bool HI>
__device__ __forceinline__ f16x2 e4m3x2_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}
// Two E2M1 nibbles of byte B of w (low nibble first) -> exact float32 / bf16 / f16.
template <int B>
__device__ __forceinline__ f32x2 e2m1x2_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
}
template <int B>
__device__ __forceinline__ bf16x2 e2m1x2_bf16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, B);
}
template <int B>
__device__ __forceinline__ f16x2 e2m1x2_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B);
}
// Single E4M3 byte B of w -> float32 (exact).
template <int B>
__device__ __forceinline__ float e4m3_byte_f32(uint32_t w) {
  f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(w, B >= 2);
  return (B & 1) ? v.y : v.x;
}

// ---- bit reinterpretation ---------------------------------------------------------------------
// Always reinterpret a scalar VALUE: in this toolchain __builtin_bit_cast applied to an
// ext-vector element expression (v.y) reads the vector's first element instead.
__device__ __forceinline__ f16x2 as_f16x2(uint32_t v) { return __builtin_bit_cast(f16x2, v); }
__device__ __forceinline__ uint32_t as_u32(f16x2 v) { return __builtin_bit_cast(uint32_t, v); }

// ---- dot products ---------------------------------------------------------------------------
// acc + a.x*b.x + a.y*b.y with float32 accumulation (bf16 and f16 operands).
__device__ __forceinline__ float dot2_bf16(bf16x2 a, uint32_t b_bits, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2, b_bits), acc, false);
}
__device__ __forceinline__ float dot2_f16(f16x2 a, f16x2 b, float acc) {
  return __builtin_amdgcn_fdot2(a, b, acc, false);
}

// ---- global->LDS copies ------------------------------------------------------------------------
// Copy 16 bytes per lane from sbase + voff into LDS at lds_base + 16 * lane (lds_base wave-uniform).
// M0 carries the LDS address; nothing else in the kernels that use it needs M0, so clobbering it is safe
// (the compiler warns about clobbering a reserved register in general).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_copy16(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_base)
               : "memory", "m0");
}
// The same copy with the non-temporal hint, for data read once (a decode kernel's weight stream).
__device__ __forceinline__ void lds_copy16_nt(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase),
               "s"(lds_base)
               : "memory", "m0");
}
// A run of N <= 4 such copies with one M0 write: copy k reads b[k] + v[k] + 1024 k into LDS at
// lds_base + 1024 k + 16 * lane.  The instruction's offset field adds 1024 k to both the global and the LDS
// address, so callers pass each global base lowered by 1024 k (only the sum is an address).  Rewriting M0
// before every copy cost 3% of the prefill GEMM's time.
template <int N>
__device__ __forceinline__ void lds_copy16_run(const uint32_t* v, const uint8_t* const* b, uint32_t lds_base) {
  static_assert(N >= 1 && N <= 4, "run length");
  if constexpr (N == 1) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(v[0]), "s"(b[0]),
                 "s"(lds_base)
                 : "memory", "m0");
  } else if constexpr (N == 2) {
    asm volatile(
        "s_mov_b32 m0, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2\n\tglobal_load_lds_dwordx4 %1, %3 offset:1024" ::"v"(
            v[0]),
        "v"(v[1]), "s"(b[0]), "s"(b[1]), "s"(lds_base)
        : "memory", "m0");
  } else if constexpr (N == 3) {
    asm volatile(
        "s_mov_b32 m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %3\n\tglobal_load_lds_dwordx4 %1, %4 offset:1024\n\t"
        "global_load_lds_dwordx4 %2, %5 offset:2048" ::"v"(v[0]),
        "v"(v[1]), "v"(v[2]), "s"(b[0]), "s"(b[1]), "s"(b[2]), "s"(lds_base)
        : "memory", "m0");
  } else {
    asm volatile(
        "s_mov_b32 m0, %8\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %4\n\tglobal_load_lds_dwordx4 %1, %5 offset:1024\n\t"
        "global_load_lds_dwordx4 %2, %6 offset:2048\n\tglobal_load_lds_dwordx4 %3, %7 offset:3072" ::"v"(v[0]),
        "v"(v[1]), "v"(v[2]), "v"(v[3]), "s"(b[0]), "s"(b[1]), "s"(b[2]), "s"(b[3]), "s"(lds_base)
        : "memory", "m0");
  }
}
#pragma clang diagnostic pop
// s_waitcnt vmcnt(N) with the other counters left alone (the copies above are invisible to the compiler's
// own counter tracking, so every wait on them is explicit).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }   // lgkmcnt(0)

// ---- reductions -----------------------------------------------------------------------------
// Butterfly sum over groups of W lanes (W = 16 or 64): xor offsets W/2, ..., 1.
// The order is fixed, so the result is bitwise reproducible and equal in all lanes.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = W / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Cross-lane sums through DPP (register-to-register, no LDS round trip).  row16_sum: the sum of each
// 16-lane row in every lane of that row, built from lane^1, lane^2 (quad permutes), then the half-row
// and row mirrors (which pair the already uniform quads and half rows).  wave64_sum: the four row
// sums added as (r0 + r1) + (r2 + r3), the same wave-uniform value in every lane.  Fixed order, so
// bitwise reproducible.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);   // row_half_mirror
  v += dpp_f32<0x140>(v);   // row_mirror
  return v;
}
__device__ __forceinline__ float wave64_sum(float v) {
  v = row16_sum(v);
  const int b = __builtin_bit_cast(int, v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

}  // namespace wq

namespace wq {

// ---- AWQ int4 group-32 -------------------------------------------------------------------------
// A dword of a code chunk holds 8 consecutive k (byte b: low nibble k=2b, high k=2b+1),
// i.e. the nibble of local k sits at bits [4k, 4k+4).  awq_pair<I> returns the pair
// (local k = I, local k = I + 4) dequantised as RN_f16(q * s + b) with one rounding,
// where b = RN_f16(-zero * s) is precomputed per group:
//   (nibble | 0x6400) is the half 1024 + q, minus 1024 is exactly q; then one packed fma.
template <int I>
__device__ __forceinline__ f16x2 awq_pair(uint32_t w, f16x2 s2, f16x2 b2) {
  const uint32_t t = ((w >> (4 * I)) & 0x000F000Fu) | 0x64006400u;
  const f16x2 q = __builtin_bit_cast(f16x2, t) - f16x2{(_Float16)1024.0f, (_Float16)1024.0f};
  return __builtin_elementwise_fma(q, s2, b2);
}

// The routed-step kernels' form of the same decode, the four pairs of one dword at a time.  The nibbles
// at bits [0, 4) and [4, 8) of each half already lie inside the float16 mantissa: OR-ing the exponent
// pattern of 1024 (0x6400) over the first gives the half 1024 + q, OR-ing that of 64 (0x5400) over the
// second (mantissa bits [4, 8)) gives 64 + q.  So one shift by 8 serves the dword's other two pairs, and
// each pair costs one v_and_or_b32, one exact subtraction and one packed fma.  The masks sit in scalar and
// the patterns in vector registers: the three-operand encoding takes no literal and one scalar operand.
struct AwqDecode {
  uint32_t m_lo, m_hi;      // 0x000F000F, 0x00F000F0 (scalar)
  uint32_t e1024, e64;      // 0x64006400, 0x54005400 (vector)
};
__device__ __forceinline__ AwqDecode awq_decode_consts() {
  AwqDecode d;
  asm("s_mov_b32 %0, 0xf000f" : "=s"(d.m_lo));
  asm("s_mov_b32 %0, 0xf000f0" : "=s"(d.m_hi));
  asm("v_mov_b32 %0, 0x64006400" : "=v"(d.e1024));
  asm("v_mov_b32 %0, 0x54005400" : "=v"(d.e64));
  return d;
}
// p[i] = the pair (local k = i, i + 4) of dword w, as awq_pair<i>.
__device__ __forceinline__ void awq_quad(uint32_t w, f16x2 s2, f16x2 b2, const AwqDecode& d, f16x2 (&p)[4]) {
  const uint32_t w8 = w >> 8;
  const f16x2 c1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f}, c64 = {(_Float16)-64.0f, (_Float16)-64.0f};
  p[0] = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, (w & d.m_lo) | d.e1024) + c1024, s2, b2);
  p[1] = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, (w & d.m_hi) | d.e64) + c64, s2, b2);
  p[2] = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, (w8 & d.m_lo) | d.e1024) + c1024, s2, b2);
  p[3] = __builtin_elementwise_fma(__builtin_bit_cast(f16x2, (w8 & d.m_hi) | d.e64) + c64, s2, b2);
}

// Per-group bias RN_f16(-zero * scale), a single half multiply.
__device__ __forceinline__ _Float16 awq_bias(uint32_t zero, _Float16 s) {
  const _Float16 nz = -(_Float16)(float)zero;
  return nz * s;
}

__device__ __forceinline__ _Float16 f16_from_bits(uint16_t b) { return __builtin_bit_cast(_Float16, b); }

}  // namespace wq
