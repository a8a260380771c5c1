// Shared pieces of the scaled FP8 GEMM kernels (gfx950): argument block,
// MFMA wrappers, tile ordering and the bf16 epilogue store.
//
// Operand layout of v_mfma_*_16x16x128_f8f6f4 (A and B alike), measured on
// the device: lane l supplies row (l % 16) of its operand; its first 16 bytes
// are K [16*(l/16), +16) of the 128-wide block and its last 16 bytes are
// K [64 + 16*(l/16), +16).  The E8M0 scale of lane l applies to row (l % 16)
// and the 32-wide K block number (l / 16) in natural K order, i.e. to
// K [32*(l/16), +32).  The 16x16 fp32 result has rows 4*(l/16) + r (r = 0..3)
// and column l % 16 in lane l.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace fp8q {

enum { MODE_BLOCK = 0, MODE_TENSOR = 1, MODE_MX = 2, MODE_BMX = 3, MODE_MXC = 4 };  // MXC: MX, scales [K/32][rows]

struct GemmArgs {
  const uint8_t* a;
  int64_t lda;
  const void* sa;       // float* (BLOCK/TENSOR) or uint8_t* (MX)
  int sa_col_major;
  const uint8_t* w;
  int64_t ldw;
  const void* sw;       // float* (BLOCK/TENSOR) or uint8_t* (MX)
  const uint16_t* bias;
  uint16_t* y;
  int64_t ldy;
  int M, N, K;
  int KB;               // number of 128-wide K blocks
  int KB32;             // number of 32-wide K blocks (MX scale columns)
  int NB;               // number of weight scale rows
  int tiles_m, tiles_n;
  int m_end;            // output rows at or past m_end are not stored (M, or an expert's end)
  int shard;            // stacked weight shards of `shard` rows each (0: one shard), see below
  int shard_blocks;     // ceil(shard / 128)
  int split_kb;         // split-K: K blocks per split (0: no split); split s = blockIdx.y
  float* partial;       // split-K: fp32 partial sums [splits][M][N] (row stride N); split
                        // tail tiles: 256 KB per leftover tile, then an 8-byte exchange word each
  uint32_t tag;         // split tail tiles: this launch's exchange tag (never 0)
  int wait_limit;       // split tail tiles: polls before the second K half stops waiting
  int publish_delay;    // split tail tiles: sleeps before publishing (tests only; normally 0)
};

// Weight scale row of output channel j: j / 128, or with stacked shards
// (j / shard) * ceil(shard / 128) + (j % shard) / 128.
__host__ __device__ __forceinline__ int weight_scale_row(const GemmArgs& p, int j) {
  return p.shard ? (j / p.shard) * p.shard_blocks + (j % p.shard) / 128 : j / 128;
}

union Frag {
  v8i v;
  uint4 u[2];
};

// Keep the first `valid` bytes of a 16-byte chunk (0 < valid < 16).
__device__ __forceinline__ uint4 keep_bytes(uint4 c, int valid) {
  uint32_t d[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int nb = valid - 4 * i;
    if (nb <= 0) d[i] = 0u;
    else if (nb < 4) d[i] &= (1u << (8 * nb)) - 1u;
  }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

// 16 bytes of row `row` starting at column k (k % 16 == 0); bytes >= K are 0.
// Never touches memory past roundup(K, 16) <= ld.
__device__ __forceinline__ uint4 load_chunk(const uint8_t* base, int64_t ld, int64_t row, int k, int K) {
  const int valid = K - k;
  if (valid >= 16) return ld16(base + row * ld + k);
  if (valid <= 0) return make_uint4(0, 0, 0, 0);
  return keep_bytes(ld16(base + row * ld + k), valid);
}

__device__ __forceinline__ v4f mfma_plain(const v8i& a, const v8i& b, const v4f& c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_mx(const v8i& a, const v8i& b, const v4f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// MX scale byte of (row, 32-block kb32) or the neutral 127 past the last block.
__device__ __forceinline__ int mx_byte(const uint8_t* s, int64_t row, int kb32, int KB32) {
  return kb32 < KB32 ? (int)s[row * KB32 + kb32] : 127;
}

// Tile index -> (tile_m, tile_n), walking groups of GROUP_M tile rows so that
// consecutive indices share A rows and W rows.
__device__ __forceinline__ void group_walk(int idx, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GROUP_M = 8;
  const int width = GROUP_M * tiles_n;
  const int group = idx / width;
  const int first_m = group * GROUP_M;
  const int gsize = min(tiles_m - first_m, GROUP_M);
  const int in_group = idx - group * width;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Workgroup id -> (tile_m, tile_n): neighbouring tiles meet in one XCD's L2.
__device__ __forceinline__ void tile_of(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
  group_walk(xcd_contiguous(pid, tiles_m * tiles_n), tiles_m, tiles_n, tm, tn);
}

__device__ __forceinline__ void store_tile_bf16(const GemmArgs& p, const v4f& acc, int row0, int col,
                                                float mul, float bias) {
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int row = row0 + r;
    if (row < p.M && col < p.N) {
      float v = acc[r];
      if (mul != 1.0f) v = v * mul;
      v = v + bias;
      p.y[(int64_t)row * p.ldy + col] = (uint16_t)f32_to_bf16_bits(v);
    }
  }
}

// Fast prefill path (gemm_fast.hip): shapes it accepts, and its launcher.
bool gemm_fast_eligible(const GemmArgs& p, int mode);
// With p.partial set (at least gemm_fast_tail_workspace(p) bytes), the
// leftover tiles of the last round are split along K between two
// workgroups instead of into half-height tiles.
size_t gemm_fast_tail_workspace(const GemmArgs& p);
hipError_t launch_gemm_fast(GemmArgs p, int mode, hipStream_t stream);

// Grouped (MoE) path on the fast kernel's tiles: expert-sorted rows,
// offsets [E + 1] on the device, expert weights w_stride bytes apart.
bool gemm_grouped_eligible(const GemmArgs& p, int E, int64_t w_stride);
hipError_t launch_gemm_grouped(GemmArgs p, const int32_t* offsets, int E, int64_t w_stride, int mode,
                               hipStream_t stream);

// Decode path (gemm_decode.hip): shapes it accepts, and its launcher.
bool gemm_decode_eligible(const GemmArgs& p);
hipError_t launch_gemm_decode(GemmArgs p, int mode, hipStream_t stream);
// Split-K decode: the K blocks are cut into `splits` runs of p.split_kb, one
// grid row each, whose fp32 partial sums go to p.partial; a second kernel adds
// them in split order and applies the epilogue.  decode_splits() is the
// split count launch_gemm_decode_split uses for a shape (1: no split).
int decode_splits(const GemmArgs& p);
hipError_t launch_gemm_decode_split(GemmArgs p, int mode, int splits, hipStream_t stream);

}  // namespace fp8q
