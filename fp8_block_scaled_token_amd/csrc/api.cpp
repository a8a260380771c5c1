// C ABI of fp8q: argument checking, device check, and kernel dispatch.
// The declarations and their contracts are in include/fp8q.h.
#include "fp8q.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <utility>

#include "launch.h"

namespace {

using fp8q_status = fp8q_status_t;

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950, 2 = something else
std::atomic<int> g_arch_ok[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

fp8q_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FP8Q_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int c = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return FP8Q_OK;
    if (c == 2) return FP8Q_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FP8Q_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FP8Q_OK : FP8Q_ERR_DEVICE;
}

fp8q_status launch_status(hipError_t e) { return e == hipSuccess ? FP8Q_OK : FP8Q_ERR_LAUNCH; }

// A row-major matrix operand: rows x K elements with stride ld, 16-byte rows.
fp8q_status check_matrix(const void* p, int64_t K, int64_t ld, int elem_bytes) {
  if (p == nullptr) return FP8Q_ERR_NULL;
  if (ld < K) return FP8Q_ERR_SHAPE;
  if (!aligned16(p) || (ld * elem_bytes) % 16 != 0) return FP8Q_ERR_MISALIGNED;
  return FP8Q_OK;
}

// Byte range [lo, hi) of a row-major [rows, cols] matrix with stride ld
// (elements of elem bytes); a contiguous array is one row.
struct Span {
  uintptr_t lo, hi;
};
Span span(const void* p, int64_t rows, int64_t ld, int64_t cols, int elem) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(p);
  return {b, b + static_cast<uintptr_t>(((rows - 1) * ld + cols) * elem)};
}
bool overlap(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }

#define FP8Q_TRY(expr)                 \
  do {                                 \
    const fp8q_status s_ = (expr);     \
    if (s_ != FP8Q_OK) return s_;      \
  } while (0)

// Launch-grid limits: rows (M, N) up to 2^26, K up to 2^30.
constexpr int64_t kMaxRows = int64_t(1) << 26;
constexpr int64_t kMaxK = int64_t(1) << 30;

std::atomic<int> g_cu_count[kMaxDevices];

// Scratch of fp8q_gemm_blockscale_splitk_noalloc: one copy per GPU, held
// until the process ends.  In host code `scratch` only names the symbol;
// its device address comes from hipGetSymbolAddress (once per device, with
// that device current) and is kept per device in g_scratch.
__device__ __attribute__((aligned(256))) unsigned char scratch[FP8Q_SPLITK_SCRATCH_BYTES];
std::atomic<void*> g_scratch[kMaxDevices];

void* scratch_address(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p != nullptr) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
  g_scratch[dev].store(q, std::memory_order_release);
  return q;
}

// fp8q_set_plan_override's values (automatic plans by default)
std::atomic<int> g_ov_cfg{-1}, g_ov_slots{0}, g_ov_split{1}, g_ov_wide{-1}, g_ov_wait{-1}, g_ov_delay{0};

}  // namespace

namespace fp8q {

// Compute units of the current device (cached per device; 256 if unknown).
int device_cu_count() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

PlanOverride plan_override() {
  return {g_ov_cfg.load(std::memory_order_relaxed),   g_ov_slots.load(std::memory_order_relaxed),
          g_ov_split.load(std::memory_order_relaxed), g_ov_wide.load(std::memory_order_relaxed),
          g_ov_wait.load(std::memory_order_relaxed),  g_ov_delay.load(std::memory_order_relaxed)};
}

}  // namespace fp8q

extern "C" {

const char* fp8q_status_string(fp8q_status_t s) {
  switch (s) {
    case FP8Q_OK: return "ok";
    case FP8Q_ERR_NULL: return "null pointer argument";
    case FP8Q_ERR_SHAPE: return "invalid shape (negative extent, K <= 0, ld < K, or beyond the size limits)";
    case FP8Q_ERR_UNSUPPORTED: return "unsupported group/block/format/layout combination";
    case FP8Q_ERR_MISALIGNED: return "misaligned pointer or stride (rows must start on 16-byte boundaries)";
    case FP8Q_ERR_DEVICE: return "current HIP device is not gfx950 (or device query failed)";
    case FP8Q_ERR_LAUNCH: return "kernel launch failed";
    case FP8Q_ERR_VALUE: return "invalid scalar argument";
    case FP8Q_ERR_SCRATCH: return "problem needs more split-K scratch than the allocation-free entry point holds";
  }
  return "unknown status";
}

int fp8q_abi_version(void) { return FP8Q_ABI_VERSION; }

fp8q_status_t fp8q_set_plan_override(int32_t gemm_cfg, int32_t gemm_slots, int32_t gemm_split,
                                     int32_t decode_wide, int32_t split_wait_limit,
                                     int32_t split_publish_delay) {
  if (gemm_cfg < -1 || gemm_cfg > 1 || gemm_slots < 0 || gemm_slots > 4096 || gemm_split < 0 ||
      gemm_split > 1 || decode_wide < -1 || decode_wide > 1 || split_wait_limit < -1 ||
      split_publish_delay < 0 || split_publish_delay > 10000)
    return FP8Q_ERR_VALUE;
  g_ov_cfg.store(gemm_cfg, std::memory_order_relaxed);
  g_ov_slots.store(gemm_slots, std::memory_order_relaxed);
  g_ov_split.store(gemm_split, std::memory_order_relaxed);
  g_ov_wide.store(decode_wide, std::memory_order_relaxed);
  g_ov_wait.store(split_wait_limit, std::memory_order_relaxed);
  g_ov_delay.store(split_publish_delay, std::memory_order_relaxed);
  return FP8Q_OK;
}

fp8q_status_t fp8q_quant_act_group(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                   int32_t group_size, int32_t fmt, int32_t layout,
                                   const float* static_scale, uint8_t* q, int64_t ldq,
                                   void* scales, void* stream) {
  if (M < 0 || K <= 0 || M > kMaxRows || K > kMaxK) return FP8Q_ERR_SHAPE;
  if (static_scale == nullptr) {
    const bool g128 = group_size == 128 && (fmt == FP8Q_SCALE_F32 || fmt == FP8Q_SCALE_F32_POW2);
    const bool g32 = group_size == 32 && fmt == FP8Q_SCALE_UE8M0;
    if (!g128 && !g32) return FP8Q_ERR_UNSUPPORTED;
    if (layout != FP8Q_SCALES_ROW_MAJOR && layout != FP8Q_SCALES_COL_MAJOR) return FP8Q_ERR_UNSUPPORTED;
  }
  if (M == 0) return FP8Q_OK;
  FP8Q_TRY(check_matrix(x, K, ldx, 2));
  FP8Q_TRY(check_matrix(q, K, ldq, 1));
  if (static_scale == nullptr && scales == nullptr) return FP8Q_ERR_NULL;
  if (static_scale == nullptr && fmt != FP8Q_SCALE_UE8M0 && (reinterpret_cast<uintptr_t>(scales) & 3u))
    return FP8Q_ERR_MISALIGNED;
  FP8Q_TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int colm = layout == FP8Q_SCALES_COL_MAJOR;
  hipError_t e;
  if (static_scale != nullptr)
    e = fp8q::launch_quant_static(x, M, K, ldx, static_scale, q, ldq, st);
  else if (group_size == 128)
    e = fp8q::launch_quant_group128(x, M, K, ldx, q, ldq, static_cast<float*>(scales), colm,
                                    fmt == FP8Q_SCALE_F32_POW2, st);
  else
    e = fp8q::launch_quant_group32mx(x, M, K, ldx, q, ldq, static_cast<uint8_t*>(scales), colm, st);
  return launch_status(e);
}

fp8q_status_t fp8q_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M,
                                 int64_t K, int64_t ldx, int32_t layout, uint8_t* q, int64_t ldq,
                                 float* scales, uint16_t* y_out, int64_t ldy, void* stream) {
  if (M < 0 || K <= 0 || M > kMaxRows || K > kMaxK) return FP8Q_ERR_SHAPE;
  if (layout != FP8Q_SCALES_ROW_MAJOR && layout != FP8Q_SCALES_COL_MAJOR) return FP8Q_ERR_UNSUPPORTED;
  if (!(eps > 0.0f) || !std::isfinite(eps)) return FP8Q_ERR_VALUE;
  if (M == 0) return FP8Q_OK;
  FP8Q_TRY(check_matrix(x, K, ldx, 2));
  FP8Q_TRY(check_matrix(q, K, ldq, 1));
  if (gamma == nullptr || scales == nullptr) return FP8Q_ERR_NULL;
  if (!aligned16(gamma)) return FP8Q_ERR_MISALIGNED;
  if (reinterpret_cast<uintptr_t>(scales) & 3u) return FP8Q_ERR_MISALIGNED;
  if (y_out != nullptr) FP8Q_TRY(check_matrix(y_out, K, ldy, 2));
  FP8Q_TRY(check_device());
  return launch_status(fp8q::launch_rmsnorm_quant(x, gamma, eps, M, K, ldx, q, ldq, scales,
                                                   layout == FP8Q_SCALES_COL_MAJOR, y_out, ldy,
                                                   static_cast<hipStream_t>(stream)));
}

fp8q_status_t fp8q_add_rmsnorm_quant(const uint16_t* x, int64_t ldx, const uint16_t* h, int64_t ldh,
                                     uint16_t* residual_out, int64_t ldr, const uint16_t* gamma,
                                     float eps, int64_t M, int64_t K, int32_t fmt, int32_t layout,
                                     const float* static_scale, uint8_t* q, int64_t ldq,
                                     float* scales, uint16_t* y_out, int64_t ldy, void* stream) {
  if (M < 0 || K <= 0 || M > kMaxRows || K > kMaxK) return FP8Q_ERR_SHAPE;
  if (static_scale == nullptr) {
    if (layout != FP8Q_SCALES_ROW_MAJOR && layout != FP8Q_SCALES_COL_MAJOR) return FP8Q_ERR_UNSUPPORTED;
    if (fmt != FP8Q_SCALE_F32 && fmt != FP8Q_SCALE_F32_POW2) return FP8Q_ERR_UNSUPPORTED;
  }
  if (!(eps > 0.0f) || !std::isfinite(eps)) return FP8Q_ERR_VALUE;
  if (h == nullptr && residual_out != nullptr) return FP8Q_ERR_VALUE;
  if (M == 0) return FP8Q_OK;
  FP8Q_TRY(check_matrix(x, K, ldx, 2));
  if (h != nullptr) {
    FP8Q_TRY(check_matrix(h, K, ldh, 2));
    FP8Q_TRY(check_matrix(residual_out, K, ldr, 2));
  }
  FP8Q_TRY(check_matrix(q, K, ldq, 1));
  if (gamma == nullptr || (static_scale == nullptr && scales == nullptr)) return FP8Q_ERR_NULL;
  if (!aligned16(gamma)) return FP8Q_ERR_MISALIGNED;
  if (static_scale == nullptr && (reinterpret_cast<uintptr_t>(scales) & 3u)) return FP8Q_ERR_MISALIGNED;
  if (static_scale != nullptr && (reinterpret_cast<uintptr_t>(static_scale) & 3u)) return FP8Q_ERR_MISALIGNED;
  if (y_out != nullptr) FP8Q_TRY(check_matrix(y_out, K, ldy, 2));
  if (h != nullptr) {
    // the residual output is x or h exactly, or disjoint from both
    for (const auto& in : {std::make_pair(x, ldx), std::make_pair(h, ldh)}) {
      if (in.first == residual_out && in.second == ldr) continue;
      if (overlap(span(in.first, M, in.second, K, 2), span(residual_out, M, ldr, K, 2))) return FP8Q_ERR_VALUE;
    }
  }
  FP8Q_TRY(check_device());
  return launch_status(fp8q::launch_add_rmsnorm_quant(x, ldx, h, ldh, residual_out, ldr, gamma, eps, M, K,
                                                       static_scale, fmt == FP8Q_SCALE_F32_POW2, q, ldq,
                                                       scales, layout == FP8Q_SCALES_COL_MAJOR, y_out, ldy,
                                                       static_cast<hipStream_t>(stream)));
}

fp8q_status_t fp8q_quant_weight_block(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                      int32_t block_n, int32_t block_k, int32_t fmt, uint8_t* q,
                                      int64_t ldq, void* scale_inv, void* stream) {
  if (N < 0 || K <= 0 || N > kMaxRows || K > kMaxK) return FP8Q_ERR_SHAPE;
  enum { BLOCK, BLOCK_POW2, MX, TENSOR } kind;
  if (block_n == 128 && block_k == 128 && fmt == FP8Q_SCALE_F32) kind = BLOCK;
  else if (block_n == 128 && block_k == 128 && fmt == FP8Q_SCALE_F32_POW2) kind = BLOCK_POW2;
  else if (block_n == 1 && block_k == 32 && fmt == FP8Q_SCALE_UE8M0) kind = MX;
  else if (block_n == N && block_k == K && fmt == FP8Q_SCALE_F32) kind = TENSOR;
  else return FP8Q_ERR_UNSUPPORTED;
  if (N == 0) return FP8Q_OK;
  FP8Q_TRY(check_matrix(w, K, ldw, 2));
  FP8Q_TRY(check_matrix(q, K, ldq, 1));
  if (scale_inv == nullptr) return FP8Q_ERR_NULL;
  if (kind != MX && (reinterpret_cast<uintptr_t>(scale_inv) & 3u)) return FP8Q_ERR_MISALIGNED;
  FP8Q_TRY(check_device());
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (kind == BLOCK || kind == BLOCK_POW2)
    e = fp8q::launch_weight_block128(w, N, K, ldw, q, ldq, static_cast<float*>(scale_inv), kind == BLOCK_POW2, st);
  else if (kind == MX) e = fp8q::launch_quant_group32mx(w, N, K, ldw, q, ldq, static_cast<uint8_t*>(scale_inv), 0, st);
  else e = fp8q::launch_weight_tensor(w, N, K, ldw, q, ldq, static_cast<float*>(scale_inv), st);
  return launch_status(e);
}

fp8q_status_t fp8q_requant_weight_pow2(const uint8_t* q_in, int64_t ldi, const float* s_in, int64_t N,
                                       int64_t K, uint8_t* q_out, int64_t ldo, float* s_out, void* stream) {
  if (N < 0 || K <= 0 || N > kMaxRows || K > kMaxK) return FP8Q_ERR_SHAPE;
  if (N == 0) return FP8Q_OK;
  FP8Q_TRY(check_matrix(q_in, K, ldi, 1));
  FP8Q_TRY(check_matrix(q_out, K, ldo, 1));
  if (s_in == nullptr || s_out == nullptr) return FP8Q_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(s_in) & 3u) || (reinterpret_cast<uintptr_t>(s_out) & 3u))
    return FP8Q_ERR_MISALIGNED;
  // outputs: in place on their own input, else disjoint from every input and
  // from each other
  const int64_t nscales = ((N + 127) / 128) * ((K + 127) / 128);
  const Span qi = span(q_in, N, ldi, K, 1), qo = span(q_out, N, ldo, K, 1);
  const Span si = span(s_in, 1, nscales, nscales, 4), so = span(s_out, 1, nscales, nscales, 4);
  if (!(q_out == q_in && ldo == ldi) && overlap(qo, qi)) return FP8Q_ERR_VALUE;
  if (s_out != s_in && overlap(so, si)) return FP8Q_ERR_VALUE;
  if (overlap(qo, si) || overlap(so, qi) || overlap(qo, so)) return FP8Q_ERR_VALUE;
  FP8Q_TRY(check_device());
  return launch_status(fp8q::launch_requant_pow2(q_in, ldi, s_in, N, K, q_out, ldo, s_out,
                                                  static_cast<hipStream_t>(stream)));
}

fp8q_status_t fp8q_gemm_blockscale(const uint8_t* a, int64_t lda, const float* a_scales,
                                   int32_t a_layout, const uint8_t* w, int64_t ldw,
                                   const float* w_scale_inv, const uint16_t* bias, uint16_t* y,
                                   int64_t ldy, int64_t M, int64_t N, int64_t K, int32_t gran,
                                   void* stream) {
  if (M < 0 || N < 0 || K <= 0 || M > kMaxRows || N > kMaxRows || K > kMaxK) return FP8Q_ERR_SHAPE;
  if ((M / 128 + 1) * (N / 128 + 1) >= (int64_t(1) << 24)) return FP8Q_ERR_SHAPE;   // tile grid
  if (gran != FP8Q_GRAN_BLOCK128 && gran != FP8Q_GRAN_PER_TENSOR && gran != FP8Q_GRAN_BLOCK128_POW2)
    return FP8Q_ERR_UNSUPPORTED;
  if (a_layout != FP8Q_SCALES_ROW_MAJOR && a_layout != FP8Q_SCALES_COL_MAJOR) return FP8Q_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return FP8Q_OK;
  FP8Q_TRY(check_matrix(a, K, lda, 1));
  FP8Q_TRY(check_matrix(w, K, ldw, 1));
  FP8Q_TRY(check_matrix(y, N, ldy, 2));
  if (a_scales == nullptr || w_scale_inv == nullptr) return FP8Q_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(a_scales) & 3u) || (reinterpret_cast<uintptr_t>(w_scale_inv) & 3u))
    return FP8Q_ERR_MISALIGNED;
  if (bias != nullptr && (reinterpret_cast<uintptr_t>(bias) & 1u)) return FP8Q_ERR_MISALIGNED;
  FP8Q_TRY(check_device());
  return launch_status(fp8q::launch_gemm_blockscale(a, lda, a_scales, a_layout == FP8Q_SCALES_COL_MAJOR,
                                                     w, ldw, w_scale_inv, bias, y, ldy, M, N, K,
                                                     gran, static_cast<hipStream_t>(stream)));
}

size_t fp8q_gemm_splitk_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1 || M > kMaxRows || N > kMaxRows || K > kMaxK) return 0;
  if (check_device() != FP8Q_OK) return 0;
  return fp8q::gemm_splitk_workspace(M, N, K);
}

fp8q_status_t fp8q_gemm_blockscale_splitk(const uint8_t* a, int64_t lda, const float* a_scales,
                                          int32_t a_layout, const uint8_t* w, int64_t ldw,
                                          const float* w_scale_inv, const uint16_t* bias,
                                          uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                          int32_t gran, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  if (M < 0 || N < 0 || K <= 0 || M > kMaxRows || N > kMaxRows || K > kMaxK) return FP8Q_ERR_SHAPE;
  if ((M / 128 + 1) * (N / 128 + 1) >= (int64_t(1) << 24)) return FP8Q_ERR_SHAPE;
  if (gran != FP8Q_GRAN_BLOCK128 && gran != FP8Q_GRAN_PER_TENSOR && gran != FP8Q_GRAN_BLOCK128_POW2)
    return FP8Q_ERR_UNSUPPORTED;
  if (a_layout != FP8Q_SCALES_ROW_MAJOR && a_layout != FP8Q_SCALES_COL_MAJOR) return FP8Q_ERR_UNSUPPORTED;
  if (workspace == nullptr && workspace_bytes != 0) return FP8Q_ERR_NULL;
  if (M == 0 || N == 0) return FP8Q_OK;
  FP8Q_TRY(check_matrix(a, K, lda, 1));
  FP8Q_TRY(check_matrix(w, K, ldw, 1));
  FP8Q_TRY(check_matrix(y, N, ldy, 2));
  if (a_scales == nullptr || w_scale_inv == nullptr) return FP8Q_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(a_scales) & 3u) || (reinterpret_cast<uintptr_t>(w_scale_inv) & 3u) ||
      (reinterpret_cast<uintptr_t>(workspace) & 7u))
    return FP8Q_ERR_MISALIGNED;
  if (bias != nullptr && (reinterpret_cast<uintptr_t>(bias) & 1u)) return FP8Q_ERR_MISALIGNED;
  FP8Q_TRY(check_device());
  return launch_status(fp8q::launch_gemm_blockscale_splitk(
      a, lda, a_scales, a_layout == FP8Q_SCALES_COL_MAJOR, w, ldw, w_scale_inv, bias, y, ldy, M, N, K, gran,
      workspace, workspace_bytes, static_cast<hipStream_t>(stream)));
}

fp8q_status_t fp8q_gemm_blockscale_splitk_noalloc(const uint8_t* a, int64_t lda, const float* a_scales,
                                                  int32_t a_layout, const uint8_t* w, int64_t ldw,
                                                  const float* w_scale_inv, const uint16_t* bias,
                                                  uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K,
                                                  int32_t gran, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || M > kMaxRows || N > kMaxRows || K > kMaxK) return FP8Q_ERR_SHAPE;
  if ((M / 128 + 1) * (N / 128 + 1) >= (int64_t(1) << 24)) return FP8Q_ERR_SHAPE;
  if (gran != FP8Q_GRAN_BLOCK128 && gran != FP8Q_GRAN_PER_TENSOR && gran != FP8Q_GRAN_BLOCK128_POW2)
    return FP8Q_ERR_UNSUPPORTED;
  if (a_layout != FP8Q_SCALES_ROW_MAJOR && a_layout != FP8Q_SCALES_COL_MAJOR) return FP8Q_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return FP8Q_OK;
  FP8Q_TRY(check_matrix(a, K, lda, 1));
  FP8Q_TRY(check_matrix(w, K, ldw, 1));
  FP8Q_TRY(check_matrix(y, N, ldy, 2));
  if (a_scales == nullptr || w_scale_inv == nullptr) return FP8Q_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(a_scales) & 3u) || (reinterpret_cast<uintptr_t>(w_scale_inv) & 3u))
    return FP8Q_ERR_MISALIGNED;
  if (bias != nullptr && (reinterpret_cast<uintptr_t>(bias) & 1u)) return FP8Q_ERR_MISALIGNED;
  FP8Q_TRY(check_device());
  if (fp8q::gemm_splitk_workspace(M, N, K) > FP8Q_SPLITK_SCRATCH_BYTES) return FP8Q_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FP8Q_ERR_DEVICE;
  void* ws = scratch_address(dev);
  if (ws == nullptr) return FP8Q_ERR_DEVICE;
  return launch_status(fp8q::launch_gemm_blockscale_splitk(
      a, lda, a_scales, a_layout == FP8Q_SCALES_COL_MAJOR, w, ldw, w_scale_inv, bias, y, ldy, M, N, K, gran,
      ws, FP8Q_SPLITK_SCRATCH_BYTES, static_cast<hipStream_t>(stream)));
}

fp8q_status_t fp8q_gemm_grouped_blockscale(const uint8_t* a, int64_t lda, const float* a_scales,
                                           int32_t a_layout, const int32_t* expert_offsets, int32_t E,
                                           const uint8_t* w, int64_t ldw, int64_t w_expert_stride,
                                           const float* w_scale_inv, int64_t shard, uint16_t* y,
                                           int64_t ldy, int64_t M, int64_t N, int64_t K, int32_t gran,
                                           void* stream) {
  if (M < 0 || N < 0 || K <= 0 || M > kMaxRows || N > kMaxRows || K > kMaxK) return FP8Q_ERR_SHAPE;
  if (E < 1 || E > 1024 || shard < 0) return FP8Q_ERR_SHAPE;
  if (gran != FP8Q_GRAN_BLOCK128 && gran != FP8Q_GRAN_BLOCK128_POW2) return FP8Q_ERR_UNSUPPORTED;
  if (a_layout != FP8Q_SCALES_ROW_MAJOR && a_layout != FP8Q_SCALES_COL_MAJOR) return FP8Q_ERR_UNSUPPORTED;
  if (K % 128 != 0) return FP8Q_ERR_UNSUPPORTED;
  if (shard > 0 && (N % shard != 0 || shard % 64 != 0)) return FP8Q_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return FP8Q_OK;
  FP8Q_TRY(check_matrix(a, K, lda, 1));
  FP8Q_TRY(check_matrix(w, K, ldw, 1));
  FP8Q_TRY(check_matrix(y, N, ldy, 2));
  if (a_scales == nullptr || w_scale_inv == nullptr || expert_offsets == nullptr) return FP8Q_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(a_scales) & 3u) || (reinterpret_cast<uintptr_t>(w_scale_inv) & 3u) ||
      (reinterpret_cast<uintptr_t>(expert_offsets) & 3u))
    return FP8Q_ERR_MISALIGNED;
  if (w_expert_stride < N * ldw) return FP8Q_ERR_SHAPE;
  if (w_expert_stride % 16 != 0) return FP8Q_ERR_MISALIGNED;
  FP8Q_TRY(check_device());
  const hipError_t e = fp8q::launch_gemm_grouped_blockscale(
      a, lda, a_scales, a_layout == FP8Q_SCALES_COL_MAJOR, expert_offsets, E, w, ldw, w_expert_stride,
      w_scale_inv, shard, y, ldy, M, N, K, gran == FP8Q_GRAN_BLOCK128_POW2, static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return FP8Q_ERR_SHAPE;     // beyond the kernel's offset limits
  return launch_status(e);
}

fp8q_status_t fp8q_gemm_mxfp8(const uint8_t* a, int64_t lda, const uint8_t* a_scales,
                              const uint8_t* w, int64_t ldw, const uint8_t* w_scales,
                              int32_t scale_layout, const uint16_t* bias, uint16_t* y, int64_t ldy,
                              int64_t M, int64_t N, int64_t K, void* stream) {
  if (M < 0 || N < 0 || K <= 0 || M > kMaxRows || N > kMaxRows || K > kMaxK) return FP8Q_ERR_SHAPE;
  if ((M / 128 + 1) * (N / 128 + 1) >= (int64_t(1) << 24)) return FP8Q_ERR_SHAPE;   // tile grid
  if (scale_layout != FP8Q_SCALES_ROW_MAJOR && scale_layout != FP8Q_SCALES_COL_MAJOR) return FP8Q_ERR_UNSUPPORTED;
  if (scale_layout == FP8Q_SCALES_COL_MAJOR && (M <= 64 || K % 128 != 0 || M % 4 != 0 || N % 4 != 0))
    return FP8Q_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return FP8Q_OK;
  FP8Q_TRY(check_matrix(a, K, lda, 1));
  FP8Q_TRY(check_matrix(w, K, ldw, 1));
  FP8Q_TRY(check_matrix(y, N, ldy, 2));
  if (a_scales == nullptr || w_scales == nullptr) return FP8Q_ERR_NULL;
  if (scale_layout == FP8Q_SCALES_COL_MAJOR &&
      ((reinterpret_cast<uintptr_t>(a_scales) & 3u) || (reinterpret_cast<uintptr_t>(w_scales) & 3u)))
    return FP8Q_ERR_MISALIGNED;
  if (bias != nullptr && (reinterpret_cast<uintptr_t>(bias) & 1u)) return FP8Q_ERR_MISALIGNED;
  FP8Q_TRY(check_device());
  const hipError_t e = fp8q::launch_gemm_mxfp8(a, lda, a_scales, w, ldw, w_scales,
                                               scale_layout == FP8Q_SCALES_COL_MAJOR, bias, y, ldy, M, N, K,
                                               static_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidValue) return FP8Q_ERR_UNSUPPORTED;   // column-major beyond the fast kernel's limits
  return launch_status(e);
}

}  // extern "C"
