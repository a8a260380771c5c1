/*
 * fp8q -- FP8 blockwise linear layer for AMD Instinct MI355X (gfx950).
 *
 * C ABI of the hot path: a dynamic per-token-group activation quantizer
 * (optionally fused after RMSNorm, or after residual add + RMSNorm), a
 * 128x128 weight-block quantizer, and
 * W8A8 GEMMs with per-K-block fp32 rescaling (plus per-tensor and MXFP8
 * variants).  Plain pointers and sizes only; every compute step runs in
 * hand-written HIP kernels on the caller's stream.
 *
 * Sources (page title, section):
 *   [SGL19]  "SGLang 源码完全拆解(十九):量化方法的注册与层分派"
 *   [SGLFP8] "[SGLang] FP8"
 *   [GLM17]  "GLM-5.3 推理全链路(十七):精度账本"
 *   [MKBK]   "量化" (HF quantization configs)
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Types.  bf16 and E4M3 values travel as their bit patterns (uint16_t and
 *   uint8_t).  E4M3 is the OCP "fn" variant: max 448, no infinities.
 *   UE8M0 scale bytes encode 2^(byte-127).
 * Layout.  Matrices are row-major with a leading dimension (row stride, in
 *   elements) `ld` >= the logical row length.  Every row buffer must be
 *   readable for its full `ld` elements (kernels read whole 16-byte chunks
 *   inside a row, but never write outside the logical [rows, K] region).
 * Alignment.  Matrix base pointers are 16-byte aligned; bf16 strides are
 *   multiples of 8 elements and E4M3 strides multiples of 16, so that every
 *   row starts on a 16-byte boundary.  Scale arrays are naturally aligned.
 * Memory.  Pointers are device pointers (except where stated).  The caller
 *   allocates every input and output; the library never allocates, frees,
 *   synchronizes or keeps pointers.  Work is enqueued asynchronously on
 *   `stream` (a hipStream_t; NULL = the null stream); buffers must stay alive
 *   until the stream has passed it.
 * Errors.  Arguments are checked before anything is launched ("fail at
 *   setup, not in the kernel", as the pages' config checks do: [SGL19]
 *   "配置对象还要过三道硬件检查"); on any error nothing is enqueued.  A launch
 *   failure reported by HIP returns FP8Q_ERR_LAUNCH.  The library prints
 *   nothing and never aborts.  M == 0 or N == 0 is a successful no-op.
 * Values.  Inputs must be finite; NaN/Inf inputs give unspecified (but
 *   memory-safe) outputs.
 * Determinism.  No atomics on floating-point data and fixed reduction
 *   orders: repeated calls give identical bits.  Calls are re-entrant across
 *   streams and host threads.  The only process-wide mutable state is:
 *   a per-device cache of the architecture and of kernel occupancies
 *   (filled once); an atomic launch counter that numbers split-K launches
 *   (the split-K workspace is the caller's and serves one launch at a time);
 *   and the launch-plan override set by fp8q_set_plan_override (tuning and
 *   tests; it changes tile shapes and splits, never the formula).  Nothing is
 *   read from the environment.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8Q_ABI_VERSION 3

typedef enum {
  FP8Q_OK = 0,
  FP8Q_ERR_NULL = 1,         /* a required pointer is NULL                      */
  FP8Q_ERR_SHAPE = 2,        /* negative extent, K <= 0, ld < row length, or an
                                extent beyond the limits (rows 2^26, K 2^30) */
  FP8Q_ERR_UNSUPPORTED = 3,  /* group/block/format/layout combination not offered */
  FP8Q_ERR_MISALIGNED = 4,   /* pointer or stride breaks the alignment rule     */
  FP8Q_ERR_DEVICE = 5,       /* current device is not gfx950, or HIP query failed */
  FP8Q_ERR_LAUNCH = 6,       /* HIP reported an error when launching            */
  FP8Q_ERR_VALUE = 7,        /* invalid scalar argument (e.g. eps <= 0)         */
  FP8Q_ERR_SCRATCH = 8       /* the problem needs more scratch than the
                                allocation-free entry point holds             */
} fp8q_status_t;

/* FP8Q_SCALE_F32_POW2: fp32 scales restricted to powers of two 2^e (e from the
 * round-up rule below), so that each one is exactly a UE8M0 value: its fp32
 * exponent field is the byte e + 127 ("block FP8 as an MXFP8 view"). */
typedef enum { FP8Q_SCALE_F32 = 0, FP8Q_SCALE_UE8M0 = 1, FP8Q_SCALE_F32_POW2 = 2 } fp8q_scale_fmt_t;
typedef enum { FP8Q_SCALES_ROW_MAJOR = 0, FP8Q_SCALES_COL_MAJOR = 1 } fp8q_scale_layout_t;
typedef enum { FP8Q_GRAN_BLOCK128 = 0, FP8Q_GRAN_PER_TENSOR = 1, FP8Q_GRAN_BLOCK128_POW2 = 2 } fp8q_gran_t;

/* Human-readable name of a status code (static storage, never NULL). */
const char* fp8q_status_string(fp8q_status_t s);

/* FP8Q_ABI_VERSION of the loaded library. */
int fp8q_abi_version(void);

/*
 * fp8q_set_plan_override -- force a GEMM launch plan (tuning and tests).
 *
 * The GEMM entry points choose tile shapes and tail splits from the problem
 * shape and the device's compute-unit count.  This call overrides that choice
 * for every later call in the process (all devices, all threads) until it is
 * called again; the results stay within the same bound (only the summation
 * order can change), so the override exists to pin each kernel variant in
 * tests and to measure them.  Calling it while another thread launches GEMMs
 * races with those launches.
 *   gemm_cfg     -1 automatic; 0: 256 x 256 prefill tiles; 1: 128 x 128 tiles
 *                (fp8q_gemm_blockscale[_splitk], fp8q_gemm_mxfp8, grouped GEMM).
 *   gemm_slots   0: plan for the device's CU count; n > 0: plan the persistent
 *                grid and its tail as if the device had n CUs.
 *   gemm_split   1 (default): balance a half-empty last round of tiles; 0: off.
 *   decode_wide  -1 automatic; 1: 96-channel decode column tiles; 0: 32-channel.
 *   split_wait_limit     -1: the default wait of a split tail tile's second K
 *                half for its partner's partial (2^22 polls); n >= 0: n polls.
 *   split_publish_delay  0 (default); n in 1..10000: the first K half sleeps
 *                n * ~3.4 us before publishing its partial.  With a short wait
 *                limit this drives the second half into computing the whole
 *                tile itself (the path taken if a partial never appeared);
 *                the output is then correct to the same bound, though its bits
 *                may differ from the split order's.
 * fp8q_set_plan_override(-1, 0, 1, -1, -1, 0) restores the automatic plans.
 * Errors: a value outside these ranges -> FP8Q_ERR_VALUE (nothing changed).
 */
fp8q_status_t fp8q_set_plan_override(int32_t gemm_cfg, int32_t gemm_slots, int32_t gemm_split,
                                     int32_t decode_wide, int32_t split_wait_limit,
                                     int32_t split_publish_delay);

/*
 * fp8q_quant_act_group -- dynamic per-token-group activation quantization.
 *
 * [GLM17] "第 1 站:RMSNorm 的两个出口" and [SGL19] "Triton 分块内核在做什么":
 * each run of `group_size` consecutive channels of a row gets its own scale
 * and is encoded to E4M3 with saturation ([SGL19] "从浮点到 FP8 的基本公式":
 * q = clamp(round(x/s), -448, 448), round-to-nearest-even).
 *
 *   x       bf16 [M, ldx]    input rows (logical length K).
 *   q       E4M3 [M, ldq]    output codes (only columns < K are written).
 *   scales  output, one per (row, group); G = ceil(K / group_size):
 *     group_size 128, fmt FP8Q_SCALE_F32: float, s = fp32(max(amax,1e-10)/448);
 *       q = E4M3(clamp(fp32(x / s))).
 *     group_size 32, fmt FP8Q_SCALE_UE8M0 (MXFP8, [SGLFP8] "4. 블록 양자화
 *       스케일 관리"): uint8 byte = e + 127 with e the smallest integer such
 *       that max(amax, 1e-10) <= 448 * 2^e (the round-up rule of [GLM17]
 *       "第 4 站:索引器"); q = E4M3(x * 2^-e).
 *     group_size 128, fmt FP8Q_SCALE_F32_POW2 (the power-of-two activation
 *       scales of [SGL19] "Triton 分块内核在做什么", act_scale_ue8m0): float
 *       s = 2^e with e as for MXFP8 over the 128-wide group; q = E4M3(x * 2^-e).
 *   layout  FP8Q_SCALES_ROW_MAJOR: scales[row * G + g];
 *           FP8Q_SCALES_COL_MAJOR: scales[g * M + row] (the [groups, rows]
 *           layout of [GLM17] "第 7 站:MoE").
 *   static_scale  if non-NULL: per-tensor static quantization with the given
 *           device fp32 scalar s ([SGL19] "激活量化的三种选择": a fixed
 *           input_scale); q = E4M3(clamp(fp32(x / s))); group_size, fmt and
 *           layout are ignored and `scales` may be NULL.  s must be > 0.
 * Errors: group_size/fmt pairs other than (128, F32), (128, F32_POW2) and
 *   (32, UE8M0) -> FP8Q_ERR_UNSUPPORTED.
 */
fp8q_status_t fp8q_quant_act_group(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                   int32_t group_size, int32_t fmt, int32_t layout,
                                   const float* static_scale,
                                   uint8_t* q, int64_t ldq, void* scales, void* stream);

/*
 * fp8q_rmsnorm_quant -- RMSNorm fused with group-128 dynamic quantization.
 *
 * [GLM17] "第 1 站:RMSNorm 的两个出口": y = x / sqrt(mean(x^2) + eps) * g with
 * bf16 input/output and high-precision statistics, followed by the per-token
 * group quantizer.  Computed per row as
 *   r = fp32(1 / sqrt(sum_k x_k^2 / K + eps))   (sum and root in fp64),
 *   y_k = bf16(fp32(fp32(x_k * r) * g_k)),
 *   (q, scales) = fp8q_quant_act_group(y, group 128, F32)  -- same bits as the
 *   unfused sequence.
 *
 *   x      bf16 [M, ldx];  gamma bf16 [K];  eps > 0 (finite).
 *   q      E4M3 [M, ldq];  scales float, layout as in fp8q_quant_act_group.
 *   y_out  optional bf16 [M, ldy] copy of the normalized rows (NULL = skip).
 */
fp8q_status_t fp8q_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, float eps,
                                 int64_t M, int64_t K, int64_t ldx, int32_t layout,
                                 uint8_t* q, int64_t ldq, float* scales,
                                 uint16_t* y_out, int64_t ldy, void* stream);

/*
 * fp8q_add_rmsnorm_quant -- residual add, RMSNorm and FP8 quantization in one pass.
 *
 * [GLM17] "第 1 站:RMSNorm 的两个出口": every decoder layer begins by adding
 * the sublayer output back into the bf16 residual stream and normalizing the
 * sum; with a static per-tensor activation scale, add, norm and the
 * fixed-scale cast form one kernel, with blockwise weights the per-token group
 * quantizer follows the norm.  Both exits are offered; the stream stays bf16
 * ("第 6 站:o_proj、残差流与 AllReduce 为什么停在 BF16").  Per row:
 *   z_k = bf16(x_k + h_k)   (the correctly rounded sum)  -> residual_out,
 *   r, y as in fp8q_rmsnorm_quant, computed on z,
 *   static_scale == NULL: (q, scales) = group-128 quantization of y with
 *                         fmt FP8Q_SCALE_F32 or FP8Q_SCALE_F32_POW2 (as in
 *                         fp8q_quant_act_group; `layout` likewise);
 *   static_scale != NULL: q = E4M3(clamp(fp32(y / s))) with the device fp32
 *                         scalar s > 0; `scales`, `fmt` and `layout` are
 *                         ignored and `scales` may be NULL.
 * The outputs are bit-identical to an add, then RMSNorm, then
 * fp8q_quant_act_group, run one after the other.
 *
 *   x             bf16 [M, ldx]  residual stream (input).
 *   h             bf16 [M, ldh]  sublayer output (input), or NULL: no add
 *                 (z = x; residual_out must then be NULL too).
 *   residual_out  bf16 [M, ldr]  updated stream z.  It may be x itself (same
 *                 pointer and ldr == ldx, the in-place update) or h itself;
 *                 any other overlap with x or h -> FP8Q_ERR_VALUE.
 *   gamma bf16 [K];  eps > 0 (finite);  q E4M3 [M, ldq];
 *   y_out optional bf16 [M, ldy] copy of the normalized rows (NULL = skip).
 * A sum that overflows bf16 gives an infinite z and unspecified q, scales, y.
 */
fp8q_status_t fp8q_add_rmsnorm_quant(const uint16_t* x, int64_t ldx, const uint16_t* h, int64_t ldh,
                                     uint16_t* residual_out, int64_t ldr, const uint16_t* gamma,
                                     float eps, int64_t M, int64_t K, int32_t fmt, int32_t layout,
                                     const float* static_scale, uint8_t* q, int64_t ldq,
                                     float* scales, uint16_t* y_out, int64_t ldy, void* stream);

/*
 * fp8q_quant_weight_block -- offline weight quantization.
 *
 * [SGL19] "建权重:先决定 scale 的形状": a [N, K] weight (row = output channel)
 * gets one scale per block_n x block_k sub-matrix on a ceil(N/block_n) x
 * ceil(K/block_k) grid; partial edge blocks are masked, not padded.  The
 * scale is the dequantization multiplier (weight_scale_inv), s = max|W|/448
 * over the block ([SGL19] "从浮点到 FP8 的基本公式").
 *
 *   (block_n, block_k, fmt):
 *     (128, 128, FP8Q_SCALE_F32)  -> float scale_inv [ceil(N/128), ceil(K/128)]
 *     (1, 32, FP8Q_SCALE_UE8M0)   -> uint8 scale_inv [N, ceil(K/32)] (MXFP8;
 *                                    any other MX block is rejected, the strict
 *                                    reading of [SGLFP8] "1. Fp8Config 초기화")
 *     (N, K, FP8Q_SCALE_F32)      -> per-tensor: one float at scale_inv[0]
 *                                    (scale_inv is also used as scratch).
 *     (128, 128, FP8Q_SCALE_F32_POW2) -> float scale_inv [ceil(N/128), ceil(K/128)],
 *                                    each 2^e with e the smallest integer such
 *                                    that max(amax, 1e-10) <= 448 * 2^e;
 *                                    q = E4M3(w * 2^-e).
 *   w bf16 [N, ldw];  q E4M3 [N, ldq].
 */
fp8q_status_t fp8q_quant_weight_block(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                      int32_t block_n, int32_t block_k, int32_t fmt,
                                      uint8_t* q, int64_t ldq, void* scale_inv, void* stream);

/*
 * fp8q_requant_weight_pow2 -- block-FP8 weights re-expressed with power-of-two scales.
 *
 * [SGL19] "分块路径的后处理": block FP8 may be used as an MXFP8 view, whose
 * hardware consumes power-of-two (UE8M0) scales ("前向:激活怎么量化,GEMM 走哪条
 * 内核" lists AMD's block-as-MXFP8 path; "为什么显式指定后端仍然可能被改写": a
 * kernel that needs UE8M0 scales cannot take fp32 block scales as they are).
 * For each 128x128 block with fp32 scale s: s' = the smallest power of two
 * >= s, q' = E4M3(decode(q) * s / s') (correctly rounded; never saturates).
 *
 *   q_in  E4M3 [N, ldi];  s_in float [ceil(N/128), ceil(K/128)] (positive,
 *         normal, finite -- other values give unspecified results).
 *   q_out E4M3 [N, ldo];  s_out float, same shape as s_in.
 *   In place is allowed: q_out == q_in with ldo == ldi, s_out == s_in;
 *   any other overlap between an output and an input -> FP8Q_ERR_VALUE.
 */
fp8q_status_t fp8q_requant_weight_pow2(const uint8_t* q_in, int64_t ldi, const float* s_in, int64_t N,
                                       int64_t K, uint8_t* q_out, int64_t ldo, float* s_out, void* stream);

/*
 * fp8q_gemm_blockscale -- Y = A * W^T with FP8 operands and fp32 scales.
 *
 * gran FP8Q_GRAN_BLOCK128 ([SGL19] "一条 GEMM 的三种缩放组合",
 * "Triton 分块内核在做什么"):
 *   Y[i,j] = bf16( sum_b P_b[i,j] * s_a[i,b] * s_w[j/128, b] + bias[j] ),
 *   P_b = sum over K block b (128 wide) of A[i,k]*W[j,k] (fp32 accumulate).
 *   a_scales float [M, ceil(K/128)] (a_layout ROW_MAJOR) or
 *            [ceil(K/128), M] (COL_MAJOR);
 *   w_scale_inv float [ceil(N/128), ceil(K/128)].
 * gran FP8Q_GRAN_PER_TENSOR: Y = bf16(s_a * s_w * sum_k A[i,k]*W[j,k] + bias[j])
 *   with a_scales and w_scale_inv each pointing at one float.
 * gran FP8Q_GRAN_BLOCK128_POW2: the FP8Q_GRAN_BLOCK128 formula and layouts,
 *   with every scale a power of two (FP8Q_SCALE_F32_POW2 quantizers,
 *   fp8q_requant_weight_pow2): the GEMM hands the scales' exponent bytes to
 *   the scaled MFMA, which applies them itself ([GLM17] "第 7 站:MoE——被排除在
 *   FP8 之外的门控与 dispatch 的量化": the scale becomes part of the matrix
 *   instruction and the per-element dequantization disappears).  A scale
 *   that is not a power of two is read as the power of two of its exponent
 *   field (its mantissa is ignored).
 *
 *   a    E4M3 [M, lda];  w E4M3 [N, ldw] (row = output channel);
 *   bias optional bf16 [N] (NULL = none);  y bf16 [M, ldy].
 */
fp8q_status_t fp8q_gemm_blockscale(const uint8_t* a, int64_t lda, const float* a_scales,
                                   int32_t a_layout, const uint8_t* w, int64_t ldw,
                                   const float* w_scale_inv, const uint16_t* bias,
                                   uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                   int32_t gran, void* stream);

/*
 * fp8q_gemm_blockscale_splitk -- fp8q_gemm_blockscale with K split into segments.
 *
 * [SGL19] "Triton 分块内核在做什么": with SPLIT_K > 1 the K dimension is cut
 * into segments, each accumulated into its own fp32 partial sum, and a
 * reduction kernel adds them; this changes the order of the floating-point
 * additions, so the result is not bit-identical to the single-accumulator
 * kernel (it is the same formula, within the same bound).  Here the split
 * serves two cases, both where whole tiles leave compute units idle:
 *  - decode shapes (M <= 64, K >= 12288): each of S segments streams its
 *    share of the weight on otherwise idle CUs; a second kernel adds the
 *    partials in segment order 0, 1, ..., S-1;
 *  - prefill shapes whose last round of 256 x 256 tiles is at most half
 *    full: each leftover tile is computed as two K halves by two workgroups.
 *    The first half runs first in its workgroup and leaves its fp32
 *    accumulators in the workspace; the second half runs last in the other
 *    workgroup and continues from those accumulators instead of zeros.
 *    Every output element so sees the same sequence of operations as in an
 *    unsplit tile: this split gives exactly the unsplit kernel's bits.  The
 *    continuing workgroup waits for the partial only up to a bound (the
 *    other never waits); if it has not appeared by then, it computes the
 *    whole tile itself (the same bits again).
 * Both orders are fixed: repeated calls give identical bits.  Other shapes,
 * or a workspace too small, run the unsplit kernels.  The prefill split keeps
 * three 8-byte words per leftover tile in the workspace after the partials:
 * two flag words, tagged with a per-launch value and reset to 0 by the last
 * workgroup that uses them, so whatever the workspace held before does not
 * matter and launches may be captured in a graph and replayed; and one
 * outcome word that the second half sets to (tag << 32) | 0x5AFE0003 when it
 * continued from the partial, or | 0x5AFE0002 when it computed the whole
 * tile (for inspection; the kernels never read it).  A workspace is used by
 * one launch at a time (launches that overlap on one workspace race).
 *
 *   Arguments as fp8q_gemm_blockscale (all three granularities), plus
 *   workspace  device memory for S * M * N fp32 partials (8-byte aligned),
 *              owned by the caller, contents ignored and overwritten; NULL
 *              with workspace_bytes 0 means: never split.
 * fp8q_gemm_splitk_workspace_size returns the bytes the current device's
 * split choice uses for an M x N x K problem (0: it would not split).
 */
size_t fp8q_gemm_splitk_workspace_size(int64_t M, int64_t N, int64_t K);
fp8q_status_t fp8q_gemm_blockscale_splitk(const uint8_t* a, int64_t lda, const float* a_scales,
                                          int32_t a_layout, const uint8_t* w, int64_t ldw,
                                          const float* w_scale_inv, const uint16_t* bias,
                                          uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                          int32_t gran, void* workspace, size_t workspace_bytes,
                                          void* stream);

/*
 * fp8q_gemm_blockscale_splitk_noalloc -- fp8q_gemm_blockscale_splitk without a
 * caller workspace, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).
 *
 * The same kernels and split choice as fp8q_gemm_blockscale_splitk (hence
 * the same bits); the partials and exchange words live in a device array of
 * FP8Q_SPLITK_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends.  Nothing in it needs to start at zero.  The call
 * allocates nothing (no hipMalloc, no hipFree).  Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other
 * threads) race and give undefined results; calls ordered on one stream are
 * safe.
 *   Arguments as fp8q_gemm_blockscale (all three granularities).
 * Errors: as fp8q_gemm_blockscale_splitk, and FP8Q_ERR_SCRATCH (nothing
 *   launched) when fp8q_gemm_splitk_workspace_size(M, N, K) exceeds
 *   FP8Q_SPLITK_SCRATCH_BYTES; FP8Q_ERR_DEVICE if the array's address cannot
 *   be obtained.
 */
#define FP8Q_SPLITK_SCRATCH_BYTES ((size_t)33 << 20)
fp8q_status_t fp8q_gemm_blockscale_splitk_noalloc(const uint8_t* a, int64_t lda, const float* a_scales,
                                                  int32_t a_layout, const uint8_t* w, int64_t ldw,
                                                  const float* w_scale_inv, const uint16_t* bias,
                                                  uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                                  int32_t gran, void* stream);

/*
 * fp8q_gemm_grouped_blockscale -- MoE expert GEMMs over expert-sorted rows.
 *
 * [SGL19] "MoE:专家权重多一个维度": expert weights carry one more dimension
 * (w13 [E, 2 I_p, H] with gate and up stacked, w2 [E, H, I_p]) and one scale
 * grid per expert; a grouped GEMM takes the activations sorted by expert into
 * one contiguous run per expert (the dispatch stage sorts them).  For each
 * expert e, rows offsets[e] .. offsets[e+1] - 1 of A:
 *   Y[i, j] = bf16( sum_b P_b[i,j] * s_a[i,b] * s_w[e][r(j), b] ),
 * the FP8Q_GRAN_BLOCK128 formula with expert e's weight and scales, where the
 * weight scale row r(j) = j / 128, or with stacked shards of `shard` rows
 * (w13: shard = I_p) r(j) = (j / shard) * ceil(shard/128) + (j % shard) / 128:
 * each shard has its own ceil grid, 2 * ceil(I_p/128) scale rows rather than
 * ceil(2 I_p / 128) (same section).
 *
 *   a E4M3 [M, lda] (expert-sorted rows);  a_scales float, [M, ceil(K/128)]
 *     (ROW_MAJOR) or [ceil(K/128), M] (COL_MAJOR).
 *   expert_offsets  device int32 [E + 1]: 0 = offsets[0] <= ... <=
 *     offsets[E] = M (rows of expert e are offsets[e] .. offsets[e+1] - 1;
 *     empty experts allowed).  Offsets outside [0, M] or decreasing give
 *     unspecified outputs but no access outside the operands.  1 <= E <= 1024.
 *   w E4M3: expert e's [N, ldw] matrix starts w_expert_stride bytes after
 *     expert e-1's (w_expert_stride >= N * ldw, a multiple of 16).
 *   w_scale_inv float [E, NBs, ceil(K/128)], NBs = ceil(N/128), or
 *     (N / shard) * ceil(shard/128) with shards; contiguous.
 *   shard  0 (one shard) or a divisor of N that is a multiple of 64.
 *   gran   FP8Q_GRAN_BLOCK128 or FP8Q_GRAN_BLOCK128_POW2 (power-of-two scales
 *     applied inside the MFMA, as in fp8q_gemm_blockscale).
 *   y bf16 [M, ldy].
 * K must be a multiple of 128 (FP8Q_ERR_UNSUPPORTED otherwise).
 */
fp8q_status_t fp8q_gemm_grouped_blockscale(const uint8_t* a, int64_t lda, const float* a_scales,
                                           int32_t a_layout, const int32_t* expert_offsets, int32_t E,
                                           const uint8_t* w, int64_t ldw, int64_t w_expert_stride,
                                           const float* w_scale_inv, int64_t shard, uint16_t* y,
                                           int64_t ldy, int64_t M, int64_t N, int64_t K, int32_t gran,
                                           void* stream);

/*
 * fp8q_gemm_mxfp8 -- MXFP8 GEMM: 1x32 blocks on both operands.
 *
 * [SGLFP8] "4. 블록 양자화 스케일 관리" (uint8 UE8M0 scales) and [SGL19]
 * "Triton 分块内核在做什么" (the scale multiply becomes an exponent add):
 *   Y[i,j] = bf16( sum_b P_b[i,j] * 2^(ea[i,b]-127) * 2^(ew[j,b]-127) + bias[j] ),
 *   b over 32-wide K blocks.
 *   a E4M3 [M, lda];  w E4M3 [N, ldw];  bias optional bf16 [N];  y bf16 [M, ldy].
 *   scale_layout FP8Q_SCALES_ROW_MAJOR: a_scales uint8 [M, ceil(K/32)],
 *                w_scales uint8 [N, ceil(K/32)];
 *                FP8Q_SCALES_COL_MAJOR: a_scales [ceil(K/32), M], w_scales
 *                [ceil(K/32), N] (the [groups, rows] layout of [GLM17] "第 7
 *                站:MoE——被排除在 FP8 之外的门控与 dispatch 的量化": a K block's scales
 *                of consecutive rows are contiguous); requires M > 64,
 *                K % 128 == 0 and M, N multiples of 4 (FP8Q_ERR_UNSUPPORTED
 *                otherwise).  fp8q_quant_act_group writes either layout, for
 *                activations and for weight rows alike.
 */
fp8q_status_t fp8q_gemm_mxfp8(const uint8_t* a, int64_t lda, const uint8_t* a_scales,
                              const uint8_t* w, int64_t ldw, const uint8_t* w_scales,
                              int32_t scale_layout, const uint16_t* bias, uint16_t* y, int64_t ldy,
                              int64_t M, int64_t N, int64_t K, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
