// Scaled FP8 GEMM kernels of the blockwise linear layer (gfx950).
//
// Y[M,N] (bf16) = A[M,K] (E4M3 activations) * W[N,K]^T (E4M3 weights, one row
// per output channel), fp32 accumulation, three scale modes on one skeleton:
//
//  MODE_BLOCK   Y_ij = sum_b P_b[i,j] * s_a[i,b] * s_w[j/128,b]; the scales
//               depend on the K block b, so each 128-wide partial sum is
//               rescaled before it is accumulated ([SGL19] "一条 GEMM 的三种缩放组合";
//               "Triton 分块内核在做什么": one weight scale per tile per K step).
//  MODE_TENSOR  scalar scales leave the sum: Y = s_a * s_w * sum_k (same
//               section: the per-tensor case degenerates to one multiply).
//  MODE_MX      1x32 UE8M0 scales consumed by the scaled MFMA itself
//               ([SGLFP8] "4. 블록 양자화 스케일 관리"; [SGL19] "Triton 分块内核在做什么":
//               scale multiplies become exponent adds).
//  MODE_BMX     block scales restricted to powers of two (block FP8 read as
//               an MXFP8 view, [SGL19] "分块路径的后处理", "前向:激活怎么量化,
//               GEMM 走哪条内核"; the scale as part of the MMA, [GLM17] "第 7 站:
//               MoE——被排除在 FP8 之外的门控与 dispatch 的量化"): the formula of MODE_BLOCK, with
//               the exponent bytes handed to the scaled MFMA (fast kernel
//               only; the other kernels run these scales in MODE_BLOCK,
//               which gives the same sum, as the products by powers of two
//               are exact).
//
// Page titles: [SGL19] "SGLang 源码完全拆解(十九):量化方法的注册与层分派",
// [SGLFP8] "[SGLang] FP8", [GLM17] "GLM-5.3 推理全链路(十七):精度账本".
//
// The contraction runs on v_mfma_*_16x16x128_f8f6f4: one instruction is
// exactly one 128-wide K block of a 16x16 output tile, so P_b comes out of a
// single MFMA and the block rescale is 4 VALU FMAs per lane (operand layout in
// gemm_common.h).
//
// Prefill shapes with K % 128 == 0 go to the fast kernel of gemm_fast.hip.
// The two general kernels here take every other shape:
//  * gemm_lds_kernel (prefill): BM x BN workgroup tiles, 4 waves, A and W
//    tiles double-buffered through LDS (16-byte chunks XOR-swizzled by row to
//    spread banks), tiles mapped XCD-aware (consecutive workgroups land on
//    different XCDs, so each XCD is given a contiguous run of tiles).
//  * gemm_decode_kernel (M <= 64): HBM-bound weight streaming; each wave
//    loads its MFMA fragments straight from global memory and owns every
//    4th K block; the 4 partial accumulators are summed in fixed order
//    through LDS (deterministic).
#include "gemm_common.h"

namespace fp8q {

// ============================================================================
// Prefill kernel: LDS double buffering.

template <int BM, int BN, int WM, int WN, int MODE>
__global__ __launch_bounds__(256, 2) void gemm_lds_kernel(GemmArgs p) {
  static_assert(WM * WN == 4, "four waves");
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 16, TN = WTN / 16;
  static_assert(TM >= 1 && TN >= 1, "wave tile at least 16x16");
  static_assert(WTN <= 128 && 128 % WTN == 0, "one weight-scale block per wave");
  constexpr int ACH = BM * 8 / 256;      // 16-byte chunks of A per thread per stage
  constexpr int WCH = BN * 8 / 256;
  static_assert(ACH >= 1 && WCH >= 1, "tile too small for 256 threads");
  constexpr int STAGE = (BM + BN) * 128;

  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];
  __shared__ __attribute__((aligned(16))) uint32_t lds_sa[2][BM];   // fp32 bits or 4 MX bytes
  __shared__ __attribute__((aligned(16))) uint32_t lds_sw[2][BN];   // MX bytes (MODE_MX only)

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave / WN, wn = wave % WN;
  int tm, tn;
  tile_of(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  // ---- global -> register staging
  uint4 ra[ACH], rw[WCH];
  uint32_t rsa = 0, rsw = 0;
  const int ld_c = t & 7;          // chunk column of this thread
  const int ld_r = t >> 3;         // first row of this thread (rows ld_r + 32*i)

  auto load_stage = [&](int kb) {
    const int k = kb * 128 + ld_c * 16;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int row = min(m0 + ld_r + 32 * i, p.M - 1);
      ra[i] = load_chunk(p.a, p.lda, row, k, p.K);
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int row = min(n0 + ld_r + 32 * i, p.N - 1);
      rw[i] = load_chunk(p.w, p.ldw, row, k, p.K);
    }
    if (MODE == MODE_BLOCK) {
      if (t < BM) {
        const int row = min(m0 + t, p.M - 1);
        const float* sa = static_cast<const float*>(p.sa);
        rsa = __float_as_uint(p.sa_col_major ? sa[(int64_t)kb * p.M + row]
                                             : sa[(int64_t)row * p.KB + kb]);
      }
    } else if (MODE == MODE_MX) {
      const uint8_t* sa = static_cast<const uint8_t*>(p.sa);
      const uint8_t* sw = static_cast<const uint8_t*>(p.sw);
      if (t < BM) {
        const int row = min(m0 + t, p.M - 1);
        rsa = 0;
#pragma unroll
        for (int s = 0; s < 4; ++s) rsa |= (uint32_t)mx_byte(sa, row, kb * 4 + s, p.KB32) << (8 * s);
      }
      if (t < BN) {
        const int row = min(n0 + t, p.N - 1);
        rsw = 0;
#pragma unroll
        for (int s = 0; s < 4; ++s) rsw |= (uint32_t)mx_byte(sw, row, kb * 4 + s, p.KB32) << (8 * s);
      }
    }
  };

  auto store_stage = [&](int st) {
    uint8_t* base = lds + st * STAGE;
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
      const int row = ld_r + 32 * i;
      *reinterpret_cast<uint4*>(base + row * 128 + ((ld_c ^ (row & 7)) << 4)) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < WCH; ++i) {
      const int row = ld_r + 32 * i;
      *reinterpret_cast<uint4*>(base + (BM + row) * 128 + ((ld_c ^ (row & 7)) << 4)) = rw[i];
    }
    if (MODE != MODE_TENSOR && t < BM) lds_sa[st][t] = rsa;
    if (MODE == MODE_MX && t < BN) lds_sw[st][t] = rsw;
  };

  auto read_frag = [&](const uint8_t* base, int row) {
    Frag f;
    const int c0 = lane >> 4;          // 16-byte chunks c0 and c0 + 4 of the row
    f.u[0] = *reinterpret_cast<const uint4*>(base + row * 128 + ((c0 ^ (row & 7)) << 4));
    f.u[1] = *reinterpret_cast<const uint4*>(base + row * 128 + (((c0 + 4) ^ (row & 7)) << 4));
    return f;
  };

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // weight-scale block of this wave's columns (MODE_BLOCK)
  const int wblk = min((n0 + wn * WTN) / 128, p.NB - 1);
  const float* swp = static_cast<const float*>(p.sw);

  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int kb = 0; kb < p.KB; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < p.KB) load_stage(kb + 1);
    const uint8_t* base = lds + cur * STAGE;

    Frag fa[TM], fb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = read_frag(base, wm * WTM + 16 * i + (lane & 15));
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = read_frag(base + BM * 128, wn * WTN + 16 * j + (lane & 15));

    if (MODE == MODE_BLOCK) {
      const float swv = swp[(int64_t)wblk * p.KB + kb];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint4 sx4 = *reinterpret_cast<const uint4*>(&lds_sa[cur][wm * WTM + 16 * i + 4 * (lane >> 4)]);
        const float sc[4] = {__uint_as_float(sx4.x) * swv, __uint_as_float(sx4.y) * swv,
                             __uint_as_float(sx4.z) * swv, __uint_as_float(sx4.w) * swv};
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const v4f P = mfma_plain(fa[i].v, fb[j].v, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(P[r], sc[r], acc[i][j][r]);
        }
      }
    } else if (MODE == MODE_TENSOR) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_plain(fa[i].v, fb[j].v, acc[i][j]);
    } else {
      const int sh = 8 * (lane >> 4);
      int sav[TM], swv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) sav[i] = (lds_sa[cur][wm * WTM + 16 * i + (lane & 15)] >> sh) & 0xFF;
#pragma unroll
      for (int j = 0; j < TN; ++j) swv[j] = (lds_sw[cur][wn * WTN + 16 * j + (lane & 15)] >> sh) & 0xFF;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_mx(fa[i].v, fb[j].v, acc[i][j], sav[i], swv[j]);
    }

    if (kb + 1 < p.KB) store_stage(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: optional per-tensor multiply, bias, bf16 rounding
  float mul = 1.0f;
  if (MODE == MODE_TENSOR)
    mul = static_cast<const float*>(p.sa)[0] * static_cast<const float*>(p.sw)[0];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + wn * WTN + 16 * j + (lane & 15);
    const float b = (p.bias != nullptr && col < p.N) ? __uint_as_float((uint32_t)p.bias[col] << 16) : 0.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      store_tile_bf16(p, acc[i][j], m0 + wm * WTM + 16 * i + 4 * (lane >> 4), col, mul, b);
  }
}

// ============================================================================
// Decode kernel (small M): weight streaming, K split over the 4 waves.

template <int TM, int TN, int MODE>
__global__ __launch_bounds__(256) void gemm_decode_kernel(GemmArgs p) {
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int n0 = blockIdx.x * (16 * TN);
  const int m0 = blockIdx.y * (16 * TM);
  const int kq = (lane >> 4) * 16;      // this lane's chunks: K [kq, +16) and [64 + kq, +16)

  int arow[TM], wrow[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) arow[i] = min(m0 + 16 * i + (lane & 15), p.M - 1);
#pragma unroll
  for (int j = 0; j < TN; ++j) wrow[j] = min(n0 + 16 * j + (lane & 15), p.N - 1);

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  Frag fa[2][TM], fb[2][TN];
  auto load = [&](int buf, int kb) {
    const int k = kb * 128 + kq;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      fb[buf][j].u[0] = load_chunk(p.w, p.ldw, wrow[j], k, p.K);
      fb[buf][j].u[1] = load_chunk(p.w, p.ldw, wrow[j], k + 64, p.K);
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      fa[buf][i].u[0] = load_chunk(p.a, p.lda, arow[i], k, p.K);
      fa[buf][i].u[1] = load_chunk(p.a, p.lda, arow[i], k + 64, p.K);
    }
  };

  auto compute = [&](int buf, int kb) {
    if (MODE == MODE_BLOCK) {
      const float* sa = static_cast<const float*>(p.sa);
      const float* sw = static_cast<const float*>(p.sw);
      float sx[TM][4];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = min(m0 + 16 * i + 4 * (lane >> 4) + r, p.M - 1);
          sx[i][r] = p.sa_col_major ? sa[(int64_t)kb * p.M + row] : sa[(int64_t)row * p.KB + kb];
        }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int blk = min((n0 + 16 * j) / 128, p.NB - 1);
        const float swv = sw[(int64_t)blk * p.KB + kb];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const v4f P = mfma_plain(fa[buf][i].v, fb[buf][j].v, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(P[r], sx[i][r] * swv, acc[i][j][r]);
        }
      }
    } else if (MODE == MODE_TENSOR) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_plain(fa[buf][i].v, fb[buf][j].v, acc[i][j]);
    } else {
      const uint8_t* sa = static_cast<const uint8_t*>(p.sa);
      const uint8_t* sw = static_cast<const uint8_t*>(p.sw);
      const int kb32 = kb * 4 + (lane >> 4);
      int sav[TM], swv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) sav[i] = mx_byte(sa, arow[i], kb32, p.KB32);
#pragma unroll
      for (int j = 0; j < TN; ++j) swv[j] = mx_byte(sw, wrow[j], kb32, p.KB32);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_mx(fa[buf][i].v, fb[buf][j].v, acc[i][j], sav[i], swv[j]);
    }
  };

  // K blocks wave, wave+4, wave+8, ...: prefetch the next one while computing
  int kb = wave;
  if (kb < p.KB) load(0, kb);
  while (kb < p.KB) {
    const int nxt = kb + 4;
    if (nxt < p.KB) load(1, nxt);
    compute(0, kb);
    kb = nxt;
    if (kb >= p.KB) break;
    const int nxt2 = kb + 4;
    if (nxt2 < p.KB) load(0, nxt2);
    compute(1, kb);
    kb = nxt2;
  }

  // fixed-order sum of the four waves' partials: ((w0 + w1) + w2) + w3
  __shared__ v4f red[3][TM * TN][64];
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) red[wave - 1][i * TN + j][lane] = acc[i][j];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v4f o = red[w][i * TN + j][lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = acc[i][j][r] + o[r];
      }

  float mul = 1.0f;
  if (MODE == MODE_TENSOR)
    mul = static_cast<const float*>(p.sa)[0] * static_cast<const float*>(p.sw)[0];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + 16 * j + (lane & 15);
    const float b = (p.bias != nullptr && col < p.N) ? __uint_as_float((uint32_t)p.bias[col] << 16) : 0.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i) store_tile_bf16(p, acc[i][j], m0 + 16 * i + 4 * (lane >> 4), col, mul, b);
  }
}

// ============================================================================
// Host side

static inline int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

template <int MODE>
static hipError_t launch_mode(GemmArgs p, hipStream_t stream) {
  if (p.M <= 64 && gemm_decode_eligible(p)) return launch_gemm_decode(p, MODE, stream);
  if (p.M <= 64) {
    // decode: one 16-row MFMA tile row per 16 rows of M; 6 column tiles per
    // workgroup (96 columns) when N is large enough to fill the chip
    const int TMn = cdiv(p.M, 16);
    const dim3 block(256);
#define FP8Q_DEC(TMv, TNv)                                                            \
  hipLaunchKernelGGL((gemm_decode_kernel<TMv, TNv, MODE>), dim3(cdiv(p.N, 16 * TNv), 1), block, 0, \
                     stream, p)
    const bool wide = p.N >= 256 * 96;
    if (TMn == 1) { if (wide) FP8Q_DEC(1, 6); else FP8Q_DEC(1, 2); }
    else if (TMn == 2) { if (wide) FP8Q_DEC(2, 6); else FP8Q_DEC(2, 2); }
    else if (TMn == 3) { if (wide) FP8Q_DEC(3, 4); else FP8Q_DEC(3, 2); }
    else { if (wide) FP8Q_DEC(4, 4); else FP8Q_DEC(4, 2); }
#undef FP8Q_DEC
    return hipGetLastError();
  }
  if (gemm_fast_eligible(p, MODE)) return launch_gemm_fast(p, MODE, stream);
  constexpr int BM = 128, BN = 128;
  p.tiles_m = cdiv(p.M, BM);
  p.tiles_n = cdiv(p.N, BN);
  const dim3 grid(p.tiles_m * p.tiles_n), block(256);
  hipLaunchKernelGGL((gemm_lds_kernel<BM, BN, 2, 2, MODE>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_gemm_blockscale(const uint8_t* a, int64_t lda, const float* sa, int sa_col_major,
                                  const uint8_t* w, int64_t ldw, const float* sw,
                                  const uint16_t* bias, uint16_t* y, int64_t ldy, int64_t M,
                                  int64_t N, int64_t K, int gran, hipStream_t stream) {
  GemmArgs p{};
  p.a = a; p.lda = lda; p.sa = sa; p.sa_col_major = sa_col_major;
  p.w = w; p.ldw = ldw; p.sw = sw; p.bias = bias; p.y = y; p.ldy = ldy;
  p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.KB = cdiv(K, 128); p.KB32 = cdiv(K, 32); p.NB = cdiv(N, 128);
  p.m_end = p.M;
  if (gran == 1) return launch_mode<MODE_TENSOR>(p, stream);
  if (gran == 2 && p.M > 64 && gemm_fast_eligible(p, MODE_BMX)) return launch_gemm_fast(p, MODE_BMX, stream);
  return launch_mode<MODE_BLOCK>(p, stream);
}

namespace {

GemmArgs block_args(const uint8_t* a, int64_t lda, const float* sa, int sa_col_major, const uint8_t* w,
                    int64_t ldw, const float* sw, const uint16_t* bias, uint16_t* y, int64_t ldy, int64_t M,
                    int64_t N, int64_t K) {
  GemmArgs p{};
  p.a = a; p.lda = lda; p.sa = sa; p.sa_col_major = sa_col_major;
  p.w = w; p.ldw = ldw; p.sw = sw; p.bias = bias; p.y = y; p.ldy = ldy;
  p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.KB = cdiv(K, 128); p.KB32 = cdiv(K, 32); p.NB = cdiv(N, 128);
  p.m_end = p.M;
  return p;
}

}  // namespace

size_t gemm_splitk_workspace(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1) return 0;
  const GemmArgs p = block_args(nullptr, K, nullptr, 0, nullptr, K, nullptr, nullptr, nullptr, N, M, N, K);
  if (M > 64) return gemm_fast_eligible(p, MODE_BLOCK) ? gemm_fast_tail_workspace(p) : 0u;
  const int s = decode_splits(p);
  return s > 1 ? (size_t)s * (size_t)M * (size_t)N * 4u : 0u;
}

hipError_t launch_gemm_blockscale_splitk(const uint8_t* a, int64_t lda, const float* sa, int sa_col_major,
                                         const uint8_t* w, int64_t ldw, const float* sw, const uint16_t* bias,
                                         uint16_t* y, int64_t ldy, int64_t M, int64_t N, int64_t K, int gran,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  GemmArgs p = block_args(a, lda, sa, sa_col_major, w, ldw, sw, bias, y, ldy, M, N, K);
  if (p.M > 64 && workspace != nullptr && gemm_fast_eligible(p, MODE_BLOCK)) {
    // prefill: the last round's leftover tiles split along K
    const size_t need = gemm_fast_tail_workspace(p);
    if (need > 0 && workspace_bytes >= need) {
      p.partial = static_cast<float*>(workspace);
      return launch_gemm_fast(p, gran == 1 ? MODE_TENSOR : gran == 2 ? MODE_BMX : MODE_BLOCK, stream);
    }
  }
  if (p.M <= 64 && workspace != nullptr && gemm_decode_eligible(p)) {
    int s = decode_splits(p);
    const int64_t fit = (int64_t)(workspace_bytes / ((size_t)M * (size_t)N * 4u));
    if (s > fit) s = (int)fit;
    if (s >= 2) {
      p.partial = static_cast<float*>(workspace);
      return launch_gemm_decode_split(p, gran == 1 ? MODE_TENSOR : MODE_BLOCK, s, stream);
    }
  }
  return launch_gemm_blockscale(a, lda, sa, sa_col_major, w, ldw, sw, bias, y, ldy, M, N, K, gran, stream);
}

hipError_t launch_gemm_grouped_blockscale(const uint8_t* a, int64_t lda, const float* sa, int sa_col_major,
                                          const int32_t* offsets, int E, const uint8_t* w, int64_t ldw,
                                          int64_t w_stride, const float* sw, int64_t shard, uint16_t* y,
                                          int64_t ldy, int64_t M, int64_t N, int64_t K, int pow2,
                                          hipStream_t stream) {
  GemmArgs p{};
  p.a = a; p.lda = lda; p.sa = sa; p.sa_col_major = sa_col_major;
  p.w = w; p.ldw = ldw; p.sw = sw; p.bias = nullptr; p.y = y; p.ldy = ldy;
  p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.KB = cdiv(K, 128); p.KB32 = cdiv(K, 32);
  p.shard = (int)shard;
  p.shard_blocks = cdiv(shard, 128);
  p.NB = shard ? (int)(N / shard) * p.shard_blocks : cdiv(N, 128);
  p.m_end = p.M;
  if (!gemm_grouped_eligible(p, E, w_stride)) return hipErrorInvalidValue;
  return launch_gemm_grouped(p, offsets, E, w_stride, pow2 ? MODE_BMX : MODE_BLOCK, stream);
}

hipError_t launch_gemm_mxfp8(const uint8_t* a, int64_t lda, const uint8_t* sa, const uint8_t* w,
                             int64_t ldw, const uint8_t* sw, int col_major, const uint16_t* bias, uint16_t* y,
                             int64_t ldy, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  GemmArgs p{};
  p.a = a; p.lda = lda; p.sa = sa; p.sa_col_major = col_major;
  p.w = w; p.ldw = ldw; p.sw = sw; p.bias = bias; p.y = y; p.ldy = ldy;
  p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.KB = cdiv(K, 128); p.KB32 = cdiv(K, 32); p.NB = cdiv(N, 128);
  p.m_end = p.M;
  if (col_major) {
    // [K/32][rows] scales: the fast kernel reads them (whole dwords of four rows)
    if (!gemm_fast_eligible(p, MODE_MX) || p.M % 4 || p.N % 4) return hipErrorInvalidValue;
    return launch_gemm_fast(p, MODE_MXC, stream);
  }
  return launch_mode<MODE_MX>(p, stream);
}

}  // namespace fp8q
