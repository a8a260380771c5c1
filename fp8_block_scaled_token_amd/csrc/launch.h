// Host-side launchers of the fp8q kernels (argument checking lives in api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

// Compute units of the current device (cached per device).
int device_cu_count();

// Launch-plan override (fp8q_set_plan_override): gemm_cfg -1/0/1,
// gemm_slots 0 or a CU count to plan for, gemm_split 0/1, decode_wide -1/0/1,
// split_wait_limit -1 (default) or polls, split_publish_delay sleeps (0).
struct PlanOverride {
  int gemm_cfg, gemm_slots, gemm_split, decode_wide, split_wait_limit, split_publish_delay;
};
PlanOverride plan_override();

// pow2: power-of-two fp32 scales (MX exponent rule on 128-wide groups)
hipError_t launch_quant_group128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                 uint8_t* q, int64_t ldq, float* scales, int col_major, int pow2,
                                 hipStream_t stream);
hipError_t launch_quant_group32mx(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  uint8_t* q, int64_t ldq, uint8_t* scales, int col_major,
                                  hipStream_t stream);
hipError_t launch_quant_static(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               const float* scale, uint8_t* q, int64_t ldq, hipStream_t stream);
hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M,
                                int64_t K, int64_t ldx, uint8_t* q, int64_t ldq, float* scales,
                                int col_major, uint16_t* y_out, int64_t ldy, hipStream_t stream);
// Residual add (z = bf16(x + h) written to z_out; none when h is null),
// RMSNorm of z, then the group-128 quantizer (power-of-two scales if pow2)
// or, with static_scale, the per-tensor static one.
hipError_t launch_add_rmsnorm_quant(const uint16_t* x, int64_t ldx, const uint16_t* h, int64_t ldh,
                                    uint16_t* z_out, int64_t ldz, const uint16_t* gamma, float eps,
                                    int64_t M, int64_t K, const float* static_scale, int pow2, uint8_t* q,
                                    int64_t ldq, float* scales, int col_major, uint16_t* y_out,
                                    int64_t ldy, hipStream_t stream);
hipError_t launch_weight_block128(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                  uint8_t* q, int64_t ldq, float* scale_inv, int pow2, hipStream_t stream);
// Block-FP8 codes and fp32 128x128 scales -> power-of-two scales (in place allowed).
hipError_t launch_requant_pow2(const uint8_t* q_in, int64_t ldi, const float* s_in, int64_t N, int64_t K,
                               uint8_t* q_out, int64_t ldo, float* s_out, hipStream_t stream);
hipError_t launch_weight_tensor(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                                int64_t ldq, float* scale_inv, hipStream_t stream);

// Scaled GEMMs: Y[M,N] (bf16) = A[M,K] (E4M3) * W[N,K]^T (E4M3).
//   gran 0: 128-block fp32 scales; gran 1: per-tensor fp32 scalars;
//   gran 2: 128-block power-of-two fp32 scales (applied inside the MFMA).
hipError_t launch_gemm_blockscale(const uint8_t* a, int64_t lda, const float* sa, int sa_col_major,
                                  const uint8_t* w, int64_t ldw, const float* sw,
                                  const uint16_t* bias, uint16_t* y, int64_t ldy, int64_t M,
                                  int64_t N, int64_t K, int gran, hipStream_t stream);
// Split-K variant of launch_gemm_blockscale: fp32 partials in `workspace`
// (decode shapes whose column tiles leave CUs idle, and the leftover tiles
// of a prefill GEMM's last round); otherwise, or when the workspace is too
// small, the unsplit kernels.
size_t gemm_splitk_workspace(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_blockscale_splitk(const uint8_t* a, int64_t lda, const float* sa, int sa_col_major,
                                         const uint8_t* w, int64_t ldw, const float* sw, const uint16_t* bias,
                                         uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, int gran,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream);
// Grouped (MoE) block GEMM over expert-sorted rows; hipErrorInvalidValue when
// the sizes exceed the kernel's 32-bit offsets (nothing is launched then).
hipError_t launch_gemm_grouped_blockscale(const uint8_t* a, int64_t lda, const float* sa, int sa_col_major,
                                          const int32_t* offsets, int E, const uint8_t* w, int64_t ldw,
                                          int64_t w_stride, const float* sw, int64_t shard, uint16_t* y,
                                          int64_t ldy, int64_t M, int64_t N, int64_t K, int pow2,
                                          hipStream_t stream);
// MX GEMM; col_major: scales [K/32][rows] (fast kernel only:
// hipErrorInvalidValue, nothing launched, where it does not apply).
hipError_t launch_gemm_mxfp8(const uint8_t* a, int64_t lda, const uint8_t* sa, const uint8_t* w,
                             int64_t ldw, const uint8_t* sw, int col_major, const uint16_t* bias, uint16_t* y,
                             int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream);

}  // namespace fp8q
