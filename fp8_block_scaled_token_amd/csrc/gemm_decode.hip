// Decode-shaped scaled FP8 GEMM for gfx950 (M <= 64, K % 128 == 0): the
// weight-streaming path of fp8q_gemm_blockscale / fp8q_gemm_mxfp8.
//
// With few activation rows every weight byte is used for at most four 16-row
// MFMA tiles, so the kernel is bound by how fast the weight matrix streams
// out of HBM.  The design keeps as many bytes in flight per CU as possible
// and nothing else on the critical path:
//  * A workgroup (4 waves) owns a column tile of 16*TN output channels for
//    all rows; wave w multiplies K blocks w, w+4, w+8, ... and the four
//    partial sums are added in a fixed order at the end (deterministic).
//  * Each wave streams its blocks' weight fragments, activation fragments
//    and scale words with direct-to-LDS loads (buffer_load ... lds) into a
//    ring of S stages of its own, S - 1 blocks ahead of the one it
//    multiplies.  The ring belongs to one wave, so the K loop needs no
//    workgroup barrier: the wave waits for its own loads (vmcnt) and for its
//    own LDS reads before refilling a stage (lgkmcnt).
//  * Fragments sit in LDS in the XOR-swizzled layout of the prefill kernel:
//    a 1 KB load covers eight 128-byte K-block rows, lane i fetching chunk
//    (i % 8) ^ (i / 8) of row i / 8.
//  * Split-K (when the column tiles alone leave CUs idle): grid row s takes
//    K blocks [s * split_kb, (s + 1) * split_kb) and writes its fp32 partial
//    sums instead of the output; splitk_reduce_kernel adds the splits in
//    order s = 0, 1, ... (fixed, so repeated calls give the same bits; the
//    order differs from the unsplit kernel's, so the bits may differ from
//    it) and applies the epilogue.
// Arithmetic per K block is that of the other kernels: one
// v_mfma_scale_f32_16x16x128_f8f6f4 per 16x16 tile and K block, then the
// block rescale (block mode), nothing (per-tensor, scaled in the epilogue)
// or the E8M0 scales inside the MFMA (MX).
#include <cstdlib>

#include "dma.h"
#include "gemm_common.h"
#include "launch.h"

namespace fp8q {

using namespace dma;

namespace {

// LDS layout: per wave a ring of S stages, then a 1 KB sink per wave.  A
// stage holds TN weight fragments (2 KB each), TM activation fragments, the
// activation scale words (16 per row tile: the row's fp32 block scale, or
// its four MX bytes) and the weight scale words (block mode: the fp32 scale
// of each 128-column block the tile touches, at most two; MX: the four bytes
// of each of the 16*TN rows), each kind in whole 64-word loads.
template <int TM_, int TN_, int S_, int MODE_>
struct DecTile {
  static constexpr int TM = TM_, TN = TN_, S = S_, MODE = MODE_;
  static constexpr int WB = TN * 2048, AB = TM * 2048;
  static constexpr int SC_OFF = WB + AB;
  static constexpr int SW_WORDS = MODE == MODE_MX ? 16 * TN : MODE == MODE_BLOCK ? 2 : 0;
  static constexpr int SA_LOADS = MODE == MODE_TENSOR ? 0 : (16 * TM + 63) / 64;
  static constexpr int SW_LOADS = (SW_WORDS + 63) / 64;
  static constexpr int SW_WORD0 = 64 * SA_LOADS;          // first weight word
  static constexpr int STAGE = SC_OFF + (SA_LOADS + SW_LOADS) * 256;
  static constexpr int RING = S * STAGE;
  static constexpr int SINK_OFF = 4 * RING;
  static constexpr int LDS_BYTES = SINK_OFF + 4 * 1024;
  // direct-to-LDS loads per K block and wave
  static constexpr int LOADS = 2 * TN + 2 * TM + SA_LOADS + SW_LOADS;
  static_assert(LOADS * (S - 1) < 64, "vmcnt range");
  static_assert(STAGE % 256 == 0, "scale loads stay 256-byte aligned");
  static_assert(LDS_BYTES <= 160 * 1024, "the rings fit in the CU's LDS");
};

}  // namespace

template <class D>
__global__ __launch_bounds__(256) void gemm_decode_dma_kernel(GemmArgs p) {
  constexpr int TM = D::TM, TN = D::TN, S = D::S, MODE = D::MODE, LOADS = D::LOADS;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[D::LDS_BYTES];
  const int lane = threadIdx.x & 63, l16 = lane & 15, lq = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n0 = blockIdx.x * (16 * TN);
  // this grid row's K blocks [kb0, KB)
  const int kb0 = p.split_kb ? (int)blockIdx.y * p.split_kb : 0;
  const int KB = p.split_kb ? min(p.KB, kb0 + p.split_kb) : p.KB;

  const i32x4 rA = rsrc(p.a, (int64_t)p.M * p.lda);
  const i32x4 rW = rsrc(p.w, (int64_t)p.N * p.ldw);

  // ---- per-lane offsets (the K block adds kb * 128 in the scalar offset)
  // fragment load h (0, 1) of a 16-row tile starting at row r0 covers rows
  // r0 + 8h + lane/8; rows past M or N fall outside the descriptor
  const int lrow = lane >> 3, lchunk = (lane & 7) ^ (lane >> 3);
  uint32_t offW[TN][2], offA[TM][2];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) offW[j][h] = (uint32_t)((n0 + 16 * j + 8 * h + lrow) * (int)p.ldw + lchunk * 16);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int h = 0; h < 2; ++h) offA[i][h] = (uint32_t)((16 * i + 8 * h + lrow) * (int)p.lda + lchunk * 16);

  // Scale words: activation load t covers activation rows 64t + lane,
  // weight load t weight words 64t + lane.  A word's array offset is
  // base + kb * step, recomputed per block with one multiply-add (the
  // column-major activation scales advance by M words per K block, the
  // others by one word or four bytes).
  constexpr int SL = D::SA_LOADS + D::SW_LOADS;
  uint32_t sbase[SL > 0 ? SL : 1], sstep[SL > 0 ? SL : 1];
#pragma unroll
  for (int t = 0; t < SL; ++t) {
    bool live;
    uint32_t base, step;
    if (t < D::SA_LOADS) {                                // activation row q
      const int q = 64 * t + lane;
      live = q < 16 * TM && q < p.M;
      if (MODE == MODE_BLOCK) {
        base = p.sa_col_major ? (uint32_t)q * 4u : (uint32_t)(q * p.KB) * 4u;
        step = p.sa_col_major ? (uint32_t)p.M * 4u : 4u;
      } else {
        base = (uint32_t)(q * p.KB32);
        step = 4u;
      }
    } else if (MODE == MODE_BLOCK) {                      // weight block n0/128 + b
      const int b = 64 * (t - D::SA_LOADS) + lane, blk = n0 / 128 + b;
      live = b < 2 && blk < p.NB;
      base = (uint32_t)(blk * p.KB) * 4u;
      step = 4u;
    } else {                                              // MX weight row
      const int b = 64 * (t - D::SA_LOADS) + lane, row = n0 + b;
      live = b < 16 * TN && row < p.N;
      base = (uint32_t)(row * p.KB32);
      step = 4u;
    }
    sbase[t] = live ? base : OOB;
    sstep[t] = live ? step : 0u;
  }
  i32x4 rSA = rA, rSW = rW;
  if (MODE == MODE_BLOCK) {
    rSA = rsrc(p.sa, (int64_t)p.M * p.KB * 4);
    rSW = rsrc(p.sw, (int64_t)p.NB * p.KB * 4);
  } else if (MODE == MODE_MX) {
    rSA = rsrc(p.sa, (int64_t)p.M * p.KB32);
    rSW = rsrc(p.sw, (int64_t)p.N * p.KB32);
  }

  const uint32_t smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const uint32_t ring = smem_base + wave * D::RING;
  const uint32_t sink = smem_base + D::SINK_OFF + wave * 1024;

  // Loads of K block kb into stage st of this wave's ring; past the last
  // block they read nothing and write zeros into the sink (every block
  // issues the same number of loads: the waits count them).
  auto issue = [&](int st, int kb) {
    const bool valid = kb < KB;
    const int kbv = valid ? kb : 0;
    const uint32_t stage = ring + st * D::STAGE;
    i32x4 rw = rW, ra = rA;
    rw.z = valid ? rw.z : 0;
    ra.z = valid ? ra.z : 0;
    const uint32_t kofs = (uint32_t)kbv * 128u;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      // weights are read once per launch: streamed
      for (int h = 0; h < 2; ++h) dma16_nt(rw, valid ? stage + (2 * j + h) * 1024 : sink, offW[j][h], kofs);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) dma16(ra, valid ? stage + D::WB + (2 * i + h) * 1024 : sink, offA[i][h], kofs);
#pragma unroll
    for (int t = 0; t < SL; ++t) {
      i32x4 rs = t < D::SA_LOADS ? rSA : rSW;
      rs.z = valid ? rs.z : 0;
      const uint32_t off = sbase[t] == OOB ? OOB : sbase[t] + (uint32_t)kbv * sstep[t];
      dma4(rs, valid ? stage + D::SC_OFF + t * 256 : sink, off, 0u);
    }
  };

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto read_frag = [&](const uint8_t* base, int row) {
    Frag f;
    f.u[0] = *reinterpret_cast<const uint4*>(base + swz(row, lq));
    f.u[1] = *reinterpret_cast<const uint4*>(base + swz(row, lq + 4));
    return f;
  };

  // multiply the block in stage st: standard layout, activations as the
  // first operand (lane holds rows 4*(lane/16) + r, column lane % 16)
  auto compute = [&](int st) {
    const uint8_t* stg = smem + wave * D::RING + st * D::STAGE;
    const uint32_t* sw_words = reinterpret_cast<const uint32_t*>(stg + D::SC_OFF);
    Frag fb[TN], fa[TM];
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = read_frag(stg + j * 2048, l16);
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[i] = read_frag(stg + D::WB + i * 2048, l16);
    if constexpr (MODE == MODE_BLOCK) {
      float sx[TM][4];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const uint4 w4 = *reinterpret_cast<const uint4*>(sw_words + 16 * i + 4 * lq);
        sx[i][0] = __uint_as_float(w4.x);
        sx[i][1] = __uint_as_float(w4.y);
        sx[i][2] = __uint_as_float(w4.z);
        sx[i][3] = __uint_as_float(w4.w);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const float swv = __uint_as_float(sw_words[D::SW_WORD0 + (n0 + 16 * j) / 128 - n0 / 128]);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const v4f P = mfma_plain(fa[i].v, fb[j].v, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(P[r], sx[i][r] * swv, acc[i][j][r]);
        }
      }
    } else if constexpr (MODE == MODE_TENSOR) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_plain(fa[i].v, fb[j].v, acc[i][j]);
    } else {
      const int sh = 8 * lq;
      int sab[TM], swb[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) sab[i] = (int)((sw_words[16 * i + l16] >> sh) & 0xFF);
#pragma unroll
      for (int j = 0; j < TN; ++j) swb[j] = (int)((sw_words[D::SW_WORD0 + 16 * j + l16] >> sh) & 0xFF);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_mx(fa[i].v, fb[j].v, acc[i][j], sab[i], swb[j]);
    }
  };

  // ---- K loop: blocks kb = wave + 4t.  At step t the stage of block t - 1
  // (whose LDS reads are waited for) is refilled with block t + S - 1; then
  // the wave waits until only the loads of blocks t + 1 .. t + S - 1 are in
  // flight, i.e. block t has landed, and multiplies it.
  const int kw = kb0 + wave;                 // this wave's first block
  const int T = KB > kw ? (KB - kw + 3) / 4 : 0;
#pragma unroll
  for (int s = 0; s < S - 1; ++s) issue(s, kw + 4 * s);
  for (int t = 0; t < T; ++t) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    issue((t + S - 1) % S, kw + 4 * (t + S - 1));
    wait_vmcnt<LOADS * (S - 1)>();
    compute(t % S);
  }
  // everything this wave issued has landed (the sink included) before the
  // ring memory is reused for the partial sums
  wait_vmcnt<0>();
  __syncthreads();

  // fixed-order sum of the four waves' partials: ((w0 + w1) + w2) + w3
  v4f* red = reinterpret_cast<v4f*>(smem);     // [3][TM * TN][64]
  static_assert(3 * TM * TN * 64 * 16 <= D::LDS_BYTES, "partials fit in LDS");
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) red[((wave - 1) * TM * TN + i * TN + j) * 64 + lane] = acc[i][j];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v4f o = red[(w * TM * TN + i * TN + j) * 64 + lane];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[i][j][r] = acc[i][j][r] + o[r];
      }

  if (p.split_kb) {
    // fp32 partial sums of this split: element (row, col) at
    // partial[(split * M + row) * N + col]; lane holds rows 16i + 4*(lane/16) + r
    float* part = p.partial + (int64_t)blockIdx.y * p.M * p.N;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + 16 * j + l16;
      if (col >= p.N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * i + 4 * lq + r;
          if (row < p.M) part[(int64_t)row * p.N + col] = acc[i][j][r];
        }
    }
    return;
  }
  float mul = 1.0f;
  if (MODE == MODE_TENSOR)
    mul = static_cast<const float*>(p.sa)[0] * static_cast<const float*>(p.sw)[0];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + 16 * j + l16;
    const float b = (p.bias != nullptr && col < p.N) ? __uint_as_float((uint32_t)p.bias[col] << 16) : 0.0f;
#pragma unroll
    for (int i = 0; i < TM; ++i) store_tile_bf16(p, acc[i][j], 16 * i + 4 * lq, col, mul, b);
  }
}

// y = bf16(sum over splits s = 0, 1, ... of partial[s] (in that order),
// times the per-tensor scale product if any, plus bias).  Thread t handles
// four consecutive columns of one row.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(GemmArgs p, int splits, int per_tensor) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cols4 = (p.N + 3) / 4;
  const int64_t row = q / cols4;
  const int c0 = (int)(q % cols4) * 4;
  if (row >= p.M) return;
  float mul = 1.0f;
  if (per_tensor) mul = static_cast<const float*>(p.sa)[0] * static_cast<const float*>(p.sw)[0];
  const int64_t plane = (int64_t)p.M * p.N;
  for (int c = c0; c < c0 + 4 && c < p.N; ++c) {
    const float* src = p.partial + row * p.N + c;
    float v = src[0];
    for (int s = 1; s < splits; ++s) v = v + src[s * plane];
    if (per_tensor) v = v * mul;
    const float b = p.bias != nullptr ? __uint_as_float((uint32_t)p.bias[c] << 16) : 0.0f;
    p.y[row * p.ldy + c] = (uint16_t)f32_to_bf16_bits(v + b);
  }
}

namespace {

template <int MODE, int TM, int TN, int S>
void launch_dec(const GemmArgs& p, hipStream_t stream, int splits = 1) {
  using D = DecTile<TM, TN, S, MODE>;
  hipLaunchKernelGGL(gemm_decode_dma_kernel<D>, dim3((p.N + 16 * TN - 1) / (16 * TN), splits), dim3(256), 0, stream,
                     p);
}

// Column tiles per workgroup and ring depth: six column tiles (96
// channels) when that still gives every CU a workgroup, else two (more
// workgroups, deeper rings); fewer where the rings would not fit in LDS.
// plan_override().decode_wide (fp8q_set_plan_override) may force the six or
// the two column-tile configuration.
template <int MODE, int TM>
void launch_dec_tm(const GemmArgs& p, hipStream_t stream) {
  const int forced = plan_override().decode_wide;
  const bool wide = forced >= 0 ? forced != 0 : p.N >= 96 * device_cu_count();
  if (wide) {
    if constexpr (TM <= 3) launch_dec<MODE, TM, 6, 2>(p, stream);
    else launch_dec<MODE, TM, 4, 2>(p, stream);
  } else {
    if constexpr (TM <= 2) launch_dec<MODE, TM, 2, 4>(p, stream);
    else launch_dec<MODE, TM, 2, 3>(p, stream);
  }
}

template <int MODE>
void launch_dec_mode(const GemmArgs& p, hipStream_t stream) {
  const int tm = (p.M + 15) / 16;
  if (tm == 1) launch_dec_tm<MODE, 1>(p, stream);
  else if (tm == 2) launch_dec_tm<MODE, 2>(p, stream);
  else if (tm == 3) launch_dec_tm<MODE, 3>(p, stream);
  else launch_dec_tm<MODE, 4>(p, stream);
}

}  // namespace

bool gemm_decode_eligible(const GemmArgs& p) {
  const int64_t lim = (int64_t(1) << 31) - 1;
  return p.M >= 1 && p.M <= 64 && p.K % 128 == 0 && (int64_t)(p.N + 96) * p.ldw < lim &&
         (int64_t)64 * p.lda < lim && (int64_t)p.M * p.KB * 4 < lim && (int64_t)(p.NB + 2) * p.KB * 4 < lim &&
         (int64_t)(p.N + 96) * p.KB32 < lim;
}

// Split count of the split-K path: as many K runs as keep every CU busy
// with the narrow (two column tiles, 32 channels) configuration, at least
// eight K blocks per run, at most 8 runs -- and no split below 96 K blocks:
// the reduction kernel and its launch cost about as much as a short K loop
// saves (measured at M = 32: K 7168 loses 2 us of 12; K 14336 gains 5 of
// 18, K 28672 gains 23 of 44).
int decode_splits(const GemmArgs& p) {
  if (!gemm_decode_eligible(p) || p.KB < 96) return 1;
  const int cus = device_cu_count();
  const int wgs = (p.N + 31) / 32;
  int s = cus / (wgs > 0 ? wgs : 1);
  s = s < p.KB / 8 ? s : p.KB / 8;
  s = s < 8 ? s : 8;
  return s < 1 ? 1 : s;
}

template <int MODE>
void launch_dec_split(const GemmArgs& p, int splits, hipStream_t stream) {
  const int tm = (p.M + 15) / 16;
  if (tm == 1) launch_dec<MODE, 1, 2, 4>(p, stream, splits);
  else if (tm == 2) launch_dec<MODE, 2, 2, 4>(p, stream, splits);
  else if (tm == 3) launch_dec<MODE, 3, 2, 3>(p, stream, splits);
  else launch_dec<MODE, 4, 2, 3>(p, stream, splits);
}

hipError_t launch_gemm_decode_split(GemmArgs p, int mode, int splits, hipStream_t stream) {
  p.split_kb = (p.KB + splits - 1) / splits;
  splits = (p.KB + p.split_kb - 1) / p.split_kb;            // no empty split
  if (mode == MODE_BLOCK) launch_dec_split<MODE_BLOCK>(p, splits, stream);
  else if (mode == MODE_TENSOR) launch_dec_split<MODE_TENSOR>(p, splits, stream);
  else launch_dec_split<MODE_MX>(p, splits, stream);
  const int64_t threads = (int64_t)p.M * ((p.N + 3) / 4);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, p, splits,
                     mode == MODE_TENSOR ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_gemm_decode(GemmArgs p, int mode, hipStream_t stream) {
  if (mode == MODE_BLOCK) launch_dec_mode<MODE_BLOCK>(p, stream);
  else if (mode == MODE_TENSOR) launch_dec_mode<MODE_TENSOR>(p, stream);
  else launch_dec_mode<MODE_MX>(p, stream);
  return hipGetLastError();
}

}  // namespace fp8q
