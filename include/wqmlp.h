/*
 * wqmlp.h -- C ABI of the weight-only-quantized SwiGLU MLP library for MI355X (gfx950).
 *
 * The library computes, inside HIP kernels and with the weights left packed in
 * device memory, the dense SwiGLU MLP
 *
 *     act[m,i] = silu(sum_k x[m,k] * dq(gate[i,k])) * (sum_k x[m,k] * dq(up[i,k]))
 *     out[m,o] = sum_q act[m,q] * dq(down[o,q])
 *
 * (issue "tp>1 fp8w tail-MLP shard host-dequantizes every layer", section
 * "Proposed fix") for FP8 E4M3 per-output-channel and NVFP4 weights, and the
 * AWQ int4 group-32 routed-expert single-token step (pull request "[Kernel][SM70]
 * Add native-g32 AWQ QPN M1 operator", section "What it does").
 *
 * Conventions for every entry point:
 *   - Pointers are DEVICE pointers on the current HIP device unless stated.
 *     The caller owns every buffer; the library never allocates, frees or
 *     synchronises inside these calls (capturable into a hipGraph).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it and the call returns at once.
 *   - Tensors are dense row-major.  Every pointer must be 16-byte aligned.
 *   - Return value: WQ_OK or a negative WQ_E* code.  Argument errors are
 *     detected before anything is enqueued (pure arithmetic checks first,
 *     then the device/pointer/arch checks).  A failed launch returns
 *     WQ_ELAUNCH and wq_last_hip_error() gives the hipError_t.  There is no
 *     fallback path of any kind.
 *   - M == 0 (no activation rows) is a valid empty call: WQ_OK, nothing enqueued; the weights are
 *     still checked, while x, the output and the workspace may be NULL.
 */
#ifndef WQMLP_H
#define WQMLP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define WQ_ABI_VERSION 1

/* activation element types */
enum { WQ_F32 = 0, WQ_BF16 = 1, WQ_F16 = 2 };
/* weight formats */
enum { WQ_FMT_FP8W = 0, WQ_FMT_NVFP4 = 1 };
/* return codes */
enum {
  WQ_OK = 0,
  WQ_EINVAL = -1,     /* null pointer, bad shape, dtype, format or flags */
  WQ_EALIGN = -2,     /* a pointer is not 16-byte aligned */
  WQ_EOVERLAP = -3,   /* an output or the workspace overlaps an input or another output */
  WQ_EDEVICE = -4,    /* a pointer is not device memory of the current device */
  WQ_EARCH = -5,      /* the current device is not gfx950 */
  WQ_EWORKSPACE = -6, /* workspace missing or smaller than the query returns */
  WQ_ELAUNCH = -7,    /* kernel launch failed; see wq_last_hip_error() */
  WQ_ESCRATCH = -8    /* the call needs more than WQ_STATIC_SCRATCH_BYTES (mlp_fp8w_run_noalloc) */
};
/* path selection (flags bits 0-1).  AUTO picks the MFMA GEMM for M >= WQ_MFMA_MIN_ROWS, and for
 * 1 < M < WQ_MFMA_MIN_ROWS when M >= WQ_NARROW_MIN_ROWS_NVFP4 / WQ_NARROW_MIN_ROWS_FP8 (by format), the
 * call's weights (all matrices) hold at least WQ_NARROW_MIN_WEIGHT_BYTES and both dimensions are
 * multiples of 64; otherwise the GEMV.  The thresholds are the measured crossovers of the two paths
 * at hidden 5120, intermediate 17408 on MI355X (the GEMV streams the weights once per row, the GEMM
 * once per call). */
enum { WQ_PATH_AUTO = 0, WQ_PATH_GEMV = 1, WQ_PATH_MFMA = 2 };
/* stage selection (flags bits 2-3, MLP entry points only; default: both stages).
 * GATEUP_ONLY enqueues the gate/up projection + SwiGLU, leaving act in the
 * workspace; DOWN_ONLY enqueues the down projection from the act a previous
 * GATEUP_ONLY call (same shape, path and workspace) left there.  For callers
 * that interleave work or timing between the two stages. */
enum { WQ_STAGE_GATEUP_ONLY = 4, WQ_STAGE_DOWN_ONLY = 8 };
/* activation variant (flags bit 4; mlp_nvfp4_run and qlinear_run with NVFP4 weights, MFMA path only).
 * WQ_ACT_E4M3 selects the W4A8 variant (page "Qwen3.8-27B-NVFP4", section "Implemented execution
 * path": per-token dynamic 8-bit activations in a small workspace, one quantization of x shared by
 * gate and up).  Each row of the linear's input is scaled by the power of two 2^-e that puts its
 * largest magnitude in (224, 448] (exact) and rounded to E4M3 with round to nearest even.  Every E4M3
 * value is a float16, as is every decoded NVFP4 weight (E2M1 x E4M3 group scale), so the quantized rows
 * are held as float16 and the float16 MFMA GEMM forms each product exactly, accumulating in float32;
 * out = (1/gs) 2^e sum_k e2m1 * d_group * xq.  The MLP quantizes x for gate/up and its float32 act for
 * down.  The activation rounding is the variant's own error against the exact MLP (the page reports
 * 1.458e-2 for its INT8 form; section "Correctness and precision").  Both dimensions that act as K (H
 * and I for the MLP, K for the linear) must be multiples of 64 and at least 256; with WQ_PATH_GEMV,
 * with FP8 weights or with float16 x the call is WQ_EINVAL. */
enum { WQ_ACT_E4M3 = 16 };
#define WQ_MFMA_MIN_ROWS 128
#define WQ_NARROW_MIN_ROWS_NVFP4 3
#define WQ_NARROW_MIN_ROWS_FP8 2
#define WQ_NARROW_MIN_WEIGHT_BYTES (16u << 20)
/* largest top-k the routed-expert step accepts */
#define WQ_MOE_MAX_TOPK 16
/* largest value of every dimension (M, H, I, N, K, E); larger ones are WQ_EINVAL.  The kernels that
 * move data by global->LDS copies address it with 32-bit offsets inside one 128-row activation tile or
 * one weight row (64-bit bases), which this bound keeps below 2^31 bytes. */
#define WQ_MAX_DIM (1 << 23)
/* largest element count of any activation or output matrix: M x max(H, I) for the MLP, M x max(N, K)
 * for the single linear (2^36 float32 elements are 256 GiB); larger calls are WQ_EINVAL. */
#define WQ_MAX_ELEMS ((int64_t)1 << 36)

/* ABI version of the loaded library (WQ_ABI_VERSION). */
int wq_abi_version(void);
/* Static message for a return code. */
const char* wq_strerror(int rc);
/* hipError_t of the last WQ_ELAUNCH / WQ_EDEVICE on this host thread (0 if none). */
int wq_last_hip_error(void);

/*
 * Workspace (device bytes) that mlp_fp8w_run / mlp_nvfp4_run need for this
 * shape and path.  fmt: WQ_FMT_*; flags as for the run call.  Returns 0 for
 * invalid arguments or M == 0.
 *   GEMV path: act [M, I], float32 (FP8) or float16 (NVFP4).
 *   MFMA path: x as float16 [M, H] (row-scaled; unused for FP8 with bf16 x),
 *              per-row scales float32 [M],
 *              act float16 [M, I] (the down GEMM's operand),
 *              FP8 only: act float32 [M, I] and its per-row scales float32 [M],
 *              then float32 split-K partial tiles of at most 64 MiB; each
 *              region 256-byte aligned.  The size is a function of the shape
 *              alone.
 *   WQ_ACT_E4M3 (NVFP4): x's E4M3 values as float16 [M, H] (each row times the
 *              inverse of its scale), their row scales float32 [M], act
 *              float32 [M, I], act's E4M3 values as float16 [M, I], their row
 *              scales float32 [M], then the split-K partial tiles; each region
 *              256-byte aligned.  0 with WQ_PATH_GEMV or FP8.
 */
size_t mlp_workspace_bytes(int fmt, int64_t M, int64_t H, int64_t I, int flags);

/*
 * FP8 E4M3 per-output-channel W8A16 SwiGLU MLP.
 * Definition: issue "tp>1 fp8w tail-MLP shard ...", sections "Mechanism on the
 * tp>1 path" (dq[n,k] = F8E4M3ToF32(w[n,k]) * scale[n]) and "Proposed fix"
 * (the MLP equation, float32 act with no bf16 rounding).
 *   x       [M, H]  WQ_F32 or WQ_BF16 (x_dtype)
 *   w_gate  [I, H]  uint8 E4M3fn codes (OCP "fn": bias 7, NaN at 0x7F/0xFF)
 *   s_gate  [I]     float32 per-output-channel scales;  likewise w_up / s_up
 *   w_down  [H, I]  uint8 E4M3fn codes;  s_down [H] float32
 *   out     [M, H]  float32
 * flags: WQ_PATH_* | optional WQ_STAGE_* bit.
 * Shapes: H, I > 0 and multiples of 16 (GEMV) or 64 (MFMA).  Accumulation is
 * float32; silu(z) = z / (1 + exp(-z)).  The GEMV path (WQ_PATH_GEMV, or AUTO
 * below the row thresholds above) reduces each output over k in a fixed order
 * that does not depend on M, so results are bitwise reproducible and row m of
 * an M-row call equals a 1-row call on row m.  The MFMA path is reproducible
 * for a given shape; its split-K plan, and so its rounding, depends on M.
 * MFMA path numerics: with bf16 x the gate/up GEMM runs bf16 MFMAs on x as
 * given; float32 x is scaled per row by a power of two and rounded to float16
 * (bf16-representable values give the same bits either way); E4M3 codes decode
 * exactly; act = silu(g) * u is kept in float32 between the projections (as on
 * the GEMV path) and the down GEMM takes it as float16 after an exact
 * power-of-two scale per row (max |act| of the row in [2^14, 2^15)), which it
 * takes back out of the result: any finite act is accepted; each element is
 * rounded once (relative error at most 2^-11, or an absolute error below 2^-39
 * of the row's largest |act| for elements in float16's subnormal range).
 */
int mlp_fp8w_run(int64_t M, int64_t H, int64_t I, const void* x, int x_dtype,
                 const uint8_t* w_gate, const float* s_gate,
                 const uint8_t* w_up, const float* s_up,
                 const uint8_t* w_down, const float* s_down,
                 void* workspace, size_t workspace_bytes, float* out,
                 int flags, void* stream);

/*
 * mlp_fp8w_run without a workspace argument, for callers that cannot allocate
 * device memory (code under hipGraph capture, tight serving loops, harnesses that
 * forbid allocation).  Same arguments, definition, kernels and results as
 * mlp_fp8w_run with flags holding a WQ_PATH_* value only (stage bits are
 * WQ_EINVAL: the two-stage form hands act over in the scratch).  The scratch is a
 * static device array of WQ_STATIC_SCRATCH_BYTES inside the library, one per GPU,
 * held from the library's first use on that GPU until the process ends; a call
 * whose workspace (mlp_workspace_bytes) would exceed it returns WQ_ESCRATCH
 * before anything is enqueued (at hidden 5120 / intermediate 17408: every M up to
 * 32).  The call allocates nothing.  Every call on one GPU shares that GPU's
 * scratch and leaves its contents there: calls that may overlap in time on one
 * GPU (several streams or host threads) race, and must be ordered by the caller.
 */
#define WQ_STATIC_SCRATCH_BYTES ((size_t)32 << 20)
int mlp_fp8w_run_noalloc(int64_t M, int64_t H, int64_t I, const void* x, int x_dtype,
                         const uint8_t* w_gate, const float* s_gate,
                         const uint8_t* w_up, const float* s_up,
                         const uint8_t* w_down, const float* s_down,
                         float* out, int flags, void* stream);

/*
 * NVFP4 SwiGLU MLP on Block64 records.
 * Definition: page "Qwen3.8-27B-NVFP4", section "NVFP4 numerics as
 * implemented": E2M1 weights two per byte (low nibble = earlier weight), one
 * E4M3 scale per 16 consecutive input channels, and a per-tensor float32
 * global scale applied as 1/global_scale; the 36-byte record
 * {uint8 d[4]; uint8 qs[32]} covers 64 consecutive weights of one row, with
 * d[0..3] the groups in K order.  Records are row-major [rows, cols/64].
 *   x         [M, H]  WQ_F32 or WQ_BF16
 *   gate_blk  [I, H/64] records (36 B each); gate_global_scale float32 > 0
 *   up_blk    [I, H/64] records;             up_global_scale
 *   down_blk  [H, I/64] records;             down_global_scale
 *   out       [M, H]  float32
 * Shapes: H, I > 0 and multiples of 64.  Each K=16 group's partial sum is
 * scaled by its E4M3 group scale as it completes (GEMV) or the group scale is
 * folded exactly into the float16 decoded weight (MFMA); 1/global_scale
 * (rounded once to float32) multiplies the finished dot product.
 * act = silu(g) * u is rounded to float16 before the down projection on both
 * paths (the page's own kernels quantize activations more coarsely); |act|
 * must stay below 65504 (larger values overflow to inf and propagate into
 * out).  MFMA path: x rows are also scaled by a power of two and rounded to
 * float16.  GEMV path: bitwise M-independent as for mlp_fp8w_run.
 * flags may add WQ_ACT_E4M3 (the W4A8 variant above; MFMA path; act is then
 * kept in float32 and quantized per row like x).
 */
int mlp_nvfp4_run(int64_t M, int64_t H, int64_t I, const void* x, int x_dtype,
                  const uint8_t* gate_blk, float gate_global_scale,
                  const uint8_t* up_blk, float up_global_scale,
                  const uint8_t* down_blk, float down_global_scale,
                  void* workspace, size_t workspace_bytes, float* out,
                  int flags, void* stream);

/*
 * Bytes of a prepared AWQ bank holding E experts of one [N, K] matrix.
 * The metadata sizes are the pull request's ("[Kernel][SM70] Add native-g32
 * AWQ QPN M1 operator", section "What it does": a 3-byte {FP16 scale, u8 zero}
 * and a 4-byte {FP16 scale, FP16 bias} layout per group of 32); the pull
 * request gives no byte order, so the order below is this library's own.
 * Layout (per expert, experts stacked with this per-expert stride / E; every
 * plane 16-byte aligned):
 *   codes  [N][K/2] uint8: byte j of row n holds k=2j (low nibble), 2j+1 (high)
 *   scales [N][K/32] float16
 *   meta_layout 3: zeros [N][K/32] uint8      (3 bytes of metadata per group)
 *   meta_layout 4: bias  [N][K/32] float16 = RN_f16(-zero * scale)  (4 bytes)
 * Returns 0 for invalid arguments.
 */
size_t awq_bank_bytes(int64_t E, int64_t N, int64_t K, int meta_layout);

/*
 * AWQ int4 group-32 routed-expert single-token step.
 * Definition: pull request "[Kernel][SM70] Add native-g32 AWQ QPN M1
 * operator", section "What it does":
 *   dq = RN_f16(fma(q, scale, RN_f16(-zero * scale)))   (not RN_f16((q-zero)*scale))
 *   for each route r (router order): e = expert_ids[r];
 *     g = RN_f16(sum_k x[k]*dq13[e][n][k]),  u = RN_f16(sum_k x[k]*dq13[e][n+I][k])
 *     act[r][n] = RN_f16(silu(g) * u)                                   n < I
 *     y_r[o] = RN_f16(sum_q act[r][q] * dq2[e][o][q])
 *   out[o] = RN_f16(sum over valid r, in order, of router_w[r] * y_r[o]) with
 *   the sum in float32 from 0 (acc = fmaf(w_r, y_r, acc)).
 *   An id outside [0, E) contributes zero and its act row is zero; duplicate
 *   valid ids keep their separate router weights.
 *   x         [H]        float16 bits
 *   expert_ids[topk]     int32 (device)
 *   router_w  [topk]     float32 (device)
 *   w13_bank  E experts of [2I, H] (gate rows 0..I-1, up rows I..2I-1)
 *   w2_bank   E experts of [H, I]
 *   act       [topk, I]  float16 out (also the W13 stage's result)
 *   out       [H]        float16 out
 * Shapes: E >= 1, 1 <= topk <= WQ_MOE_MAX_TOPK, H and I positive multiples of 32,
 * H, I <= 16384, (H/32)*80 <= 65536 and topk*((I/32)*80 + 128) <= 65536 (the staged
 * activations must fit LDS); otherwise WQ_EINVAL.
 * Sums are float32; the order inside each dot product is fixed.
 */
int moe_awq_m1_run(int64_t E, int64_t topk, int64_t H, int64_t I,
                   const uint16_t* x, const int32_t* expert_ids, const float* router_w,
                   const void* w13_bank, const void* w2_bank, int meta_layout,
                   uint16_t* act, uint16_t* out, void* stream);

/*
 * Pack checkpoint NVFP4 tensors into Block64 records (one-time, device to device).
 *   weight_packed [N, K/2] uint8 (low nibble = earlier weight)
 *   weight_scale  [N, K/16] uint8 E4M3
 *   blk           [N, K/64, 36] uint8 out: blk[n][b] = weight_scale[n][4b..4b+3] ++ weight_packed[n][32b..32b+31]
 * K must be a positive multiple of 64 (page "Qwen3.8-27B-NVFP4", section "NVFP4
 * numerics as implemented": "the host packs these").  16-byte alignment is
 * not required for this call.
 */
int nvfp4_pack_block64(int64_t N, int64_t K, const uint8_t* weight_packed,
                       const uint8_t* weight_scale, uint8_t* blk, void* stream);

/*
 * Build a prepared AWQ bank (layout: awq_bank_bytes) from
 *   codes  [E, N, K] uint8 in 0..15 (one code per byte)
 *   scales [E, N, K/32] float16 bits
 *   zeros  [E, N, K/32] uint8
 * meta_layout 3 stores the zeros; meta_layout 4 stores bias = RN_f16(-zero * scale),
 * the half bias of the dequantisation boundary (pull request "[Kernel][SM70] Add
 * native-g32 AWQ QPN M1 operator", section "What it does"), so both layouts decode
 * to the same values.  bank must hold awq_bank_bytes(E, N, K, meta_layout) bytes
 * and be 16-byte aligned; the inputs need no alignment.  One-time, device to device.
 */
int awq_pack_bank(int64_t E, int64_t N, int64_t K, const uint8_t* codes,
                  const uint16_t* scales, const uint8_t* zeros, int meta_layout,
                  void* bank, void* stream);

/*
 * Debug decoders: each weight decoded on its own, one element per thread.  They use
 * the float32 conversions of the float32-activation GEMV kernels and the AWQ
 * kernels' half fma; the kernels that take bfloat16 or float16 operands decode with
 * the packed bfloat16 / float16 conversions instead, which these calls do not run
 * (the one-hot read-outs through qlinear_run and the MLP's gate/up stage reach those).
 */
/* FP8 ("tp>1 fp8w tail-MLP shard ...", section "Mechanism on the tp>1 path"):
 * out[n,k] = RN_f32(e4m3(w[n,k]) * s[n])                              [N, K] f32 */
int fp8w_dequant_f32(int64_t N, int64_t K, const uint8_t* w, const float* s, float* out, void* stream);
/* NVFP4 (page "Qwen3.8-27B-NVFP4", section "NVFP4 numerics as implemented"):
 * out[n,k] = RN_f32(e2m1(q) * e4m3(d) * RN_f32(1/global_scale))        [N, K] f32 */
int nvfp4_dequant_f32(int64_t N, int64_t K, const uint8_t* blk, float global_scale, float* out, void* stream);
/* AWQ (pull request "[Kernel][SM70] Add native-g32 AWQ QPN M1 operator", section
 * "What it does"): out[e,n,k] = dq as in moe_awq_m1_run          [E, N, K] f16 bits */
int awq_dequant_f16(int64_t E, int64_t N, int64_t K, const void* bank, int meta_layout,
                    uint16_t* out, void* stream);

/*
 * One quantised linear y[m,n] = sum_k x[m,k] * dq(W[n,k]) through the same
 * kernels as the MLP's down projection (GEMV) or its MFMA GEMM.
 *   fmt WQ_FMT_FP8W: w = [N, K] E4M3 codes, scale = [N] float32, global_scale ignored
 *   fmt WQ_FMT_NVFP4: w = Block64 [N, K/64], scale = NULL, global_scale as above
 *   x [M, K]: WQ_F32 or WQ_BF16; WQ_F16 for NVFP4 on the GEMV path only (the
 *   operand type of the NVFP4 MLP's down projection; AUTO then always takes the
 *   GEMV, and WQ_PATH_MFMA with it is WQ_EINVAL).
 *   y [M, N] float32.  Workspace: qlinear_workspace_bytes (the GEMV path needs
 *   none; the query does not know x's type and may ask for more than a float16
 *   call uses).
 * flags: a WQ_PATH_* value, plus WQ_ACT_E4M3 for NVFP4 (x quantized per row to
 * E4M3 as described there; MFMA path; K a multiple of 64, at least 256).
 * Shapes: K a positive multiple of 64 for NVFP4 and for the MFMA path, else of
 * 16; N any positive row count (partial tiles are masked, as in the tail case of
 * page "Qwen3.8-27B-NVFP4", section "Correctness and precision": 129 x 67 x 320).
 */
size_t qlinear_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, int flags);
int qlinear_run(int fmt, int64_t M, int64_t N, int64_t K, const void* x, int x_dtype,
                const uint8_t* w, const float* scale, float global_scale,
                void* workspace, size_t workspace_bytes, float* y, int flags, void* stream);

/*
 * Measurement helper, not a step of the method: a plain streaming read of `bytes`
 * (a positive multiple of 16) at src by `grid` workgroups (1 .. 2^20) of 256
 * threads, coalesced 16-byte loads in a grid-stride loop.  Its rate is the
 * achievable HBM read ceiling that the bandwidth-bound kernels are compared with,
 * beside the device's published peak.  sink: grid 32-bit words of device memory,
 * written only in the rare case that a lane's XOR fold of its data equals one fixed
 * value (so nothing is stored in practice, yet the loads cannot be removed).
 */
int wq_read_probe(const void* src, size_t bytes, uint32_t* sink, int grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WQMLP_H */
