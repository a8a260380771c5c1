// Prefill-shaped scaled FP8 GEMM for gfx950 (the fast path of
// fp8q_gemm_blockscale / fp8q_gemm_mxfp8).
//
// Same arithmetic as the generic kernels (block rescale per 128-wide K block,
// per-tensor, or MX scales inside the MFMA; see gemm_kernels.hip), organised
// for throughput:
//  * 256 x 128 workgroup tile, 4 waves in a 2 x 2 grid, 128 x 64 per wave
//    (8 x 4 MFMA tiles of 16 x 16): each K block a wave reads 12 operand
//    fragments from LDS for 32 MFMAs.
//  * Operands move global -> LDS with buffer_load ... lds (no VGPR staging).
//    Such a load writes 16 bytes per lane to consecutive LDS addresses, so the
//    XOR row swizzle of the LDS tile is produced by choosing, per lane, which
//    16-byte chunk of global memory to fetch.  Rows past M or N fall outside
//    the buffer descriptor and read as zero.
//  * Three LDS stages: K block kb+2 streams in while kb is multiplied; one
//    barrier per K block.
//  * Workgroup ids are renumbered XCD-aware and walked in groups of tile rows
//    (tile_of), so tiles sharing A rows or W rows meet in the same L2.
// Preconditions (checked by the launcher): K % 128 == 0, every operand and
// scale array smaller than 2^31 bytes, M > 64.
#include <cstdlib>

#include "gemm_common.h"

namespace fp8q {

namespace {

constexpr int FBN = 128;                      // workgroup tile width (one weight-scale block)

// Byte offset of 16-byte chunk c (0..7) of tile row r in a swizzled LDS tile.
__device__ __forceinline__ int swz(int r, int c) { return (r << 7) | ((c ^ (r & 7)) << 4); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (stride 0): reads at byte offsets >= `bytes` return 0.
__device__ __forceinline__ i32x4 rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
  r.z = __builtin_amdgcn_readfirstlane((int)bytes);
  r.w = 0x00020000;
  return r;
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct-to-LDS loads: lane i's 16 (or 4) bytes land at LDS address
// lds + 16*i (4*i); `lds` must be wave-uniform.
// Written as inline assembly on purpose: the compiler cannot tell which LDS
// stage a direct-to-LDS load fills, and would otherwise make every LDS read
// wait for all of them.  These loads are therefore invisible to the
// compiler's vmcnt bookkeeping; the kernel waits for them explicitly
// (wait_vmcnt) and issues no other vector-memory loads inside its K loop.
__device__ __forceinline__ void dma16(const i32x4& r, uint32_t lds, int voffset) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(r), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const i32x4& r, uint32_t lds, int voffset) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(r), "s"(lds)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

}  // namespace

// BM x 128 workgroup tile, NW waves in a WM x (NW/WM) grid, NS LDS stages
// (each stage one LDS object: A tile, W tile, scale words).
template <int MODE, int BM, int NW, int NS>
__global__ __launch_bounds__(NW * 64) void gemm_fast_kernel(GemmArgs p) {
  constexpr int BN = FBN;
  constexpr int WM = (NW == 8 && BM == 256) ? 4 : 2, WN = NW / WM;
  constexpr int WTM = BM / WM, WTN = BN / WN;          // wave tile
  constexpr int TM = WTM / 16, TN = WTN / 16;
  constexpr int ABYTES = BM * 128, WBYTES = BN * 128;  // one K block of A / W
  constexpr int A_PER = (ABYTES / 1024) / NW;          // 1 KB DMA instructions per wave
  constexpr int W_PER = (WBYTES / 1024) / NW;
  constexpr int RA = BM / NW, RW = BN / NW;            // scale rows per wave
  constexpr int S_WORDS_NW = 128 * NW;                 // A scales, then W scales / copies
  constexpr int STAGE_BYTES = ABYTES + WBYTES + S_WORDS_NW * 4;
  static_assert(A_PER >= 1 && W_PER >= 1 && RA <= 64 && RW <= 64, "tile too small for NW waves");
  static_assert(WTN <= 128 && 128 % WTN == 0, "one weight-scale block per wave");
  static_assert(NS >= 2 && NS <= 4, "2..4 stages");
  __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE_BYTES], st1[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[NS > 2 ? STAGE_BYTES : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[NS > 3 ? STAGE_BYTES : 16];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WN, wn = wave % WN;
  int tm, tn;
  tile_of(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const i32x4 rA = rsrc(p.a, (int64_t)p.M * p.lda);
  const i32x4 rW = rsrc(p.w, (int64_t)p.N * p.ldw);
  const i32x4 rSA =
      rsrc(p.sa, MODE == MODE_MX ? (int64_t)p.M * p.KB32 : (MODE == MODE_BLOCK ? (int64_t)p.M * p.KB * 4 : 4));
  const i32x4 rSW =
      rsrc(p.sw, MODE == MODE_MX ? (int64_t)p.N * p.KB32 : (MODE == MODE_BLOCK ? (int64_t)p.NB * p.KB * 4 : 4));

  // DMA source offsets.  DMA instruction i of wave w fills LDS kilobyte
  // A_PER*w + i, i.e. tile rows 8*(A_PER*w + i) + lane/8 with lane % 8 the
  // physical chunk; the logical chunk to fetch is (lane % 8) ^ (row % 8) =
  // (lane % 8) ^ (lane / 8).
  const int lrow = lane >> 3, lchunk = (lane & 7) ^ (lane >> 3);
  const int offA = (m0 + 8 * A_PER * wave + lrow) * (int)p.lda + lchunk * 16;
  const int offW = (n0 + 8 * W_PER * wave + lrow) * (int)p.ldw + lchunk * 16;
  const int lda8 = 8 * (int)p.lda, ldw8 = 8 * (int)p.ldw;
  // scale rows: lane l of wave w fetches A row RA*w + l % RA (word 64w + l),
  // and (MX) W row RW*w + l % RW (word 64*NW + 64w + l)
  const int srow = m0 + RA * wave + (lane % RA);
  const int swrow = n0 + RW * wave + (lane % RW);
  const int wblk = n0 / 128;

  auto stage = [&](auto S) -> uint8_t* {
    if constexpr (decltype(S)::value == 0) return st0;
    else if constexpr (decltype(S)::value == 1) return st1;
    else if constexpr (decltype(S)::value == 2) return st2;
    else return st3;
  };
  auto stage_s = [&](auto S) -> uint32_t* { return reinterpret_cast<uint32_t*>(stage(S) + ABYTES + WBYTES); };

  // DMA instructions per wave per stage (the vmcnt bookkeeping relies on it)
  constexpr int NLOAD = A_PER + W_PER + (MODE == MODE_TENSOR ? 0 : 2);

  auto issue = [&](auto S, int kb) {
    const uint32_t base = __builtin_amdgcn_readfirstlane(lds_addr(stage(S)));
    const uint32_t a = base + wave * A_PER * 1024;
    const uint32_t w = base + ABYTES + wave * W_PER * 1024;
    const uint32_t sc = base + ABYTES + WBYTES + wave * 256;
    const int kofs = kb * 128;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) dma16(rA, a + i * 1024, offA + i * lda8 + kofs);
#pragma unroll
    for (int i = 0; i < W_PER; ++i) dma16(rW, w + i * 1024, offW + i * ldw8 + kofs);
    if constexpr (MODE == MODE_BLOCK) {
      const int e = p.sa_col_major ? kb * p.M + srow : srow * p.KB + kb;
      dma4(rSA, sc, e * 4);
      // the tile's weight-block scale, same address in every lane
      dma4(rSW, sc + 256 * NW, (wblk * p.KB + kb) * 4);
    } else if constexpr (MODE == MODE_MX) {
      dma4(rSA, sc, srow * p.KB32 + kb * 4);
      dma4(rSW, sc + 256 * NW, swrow * p.KB32 + kb * 4);
    }
  };
  // word index of A-scale row r / W-scale row c within a stage's scale words
  auto sa_word = [](int r) { return 64 * (r / RA) + (r % RA); };
  auto sw_word = [](int c) { return 64 * NW + 64 * (c / RW) + (c % RW); };

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  auto read_frag = [&](const uint8_t* base, int row) {
    Frag f;
    const int c0 = lane >> 4;
    f.u[0] = *reinterpret_cast<const uint4*>(base + swz(row, c0));
    f.u[1] = *reinterpret_cast<const uint4*>(base + swz(row, c0 + 4));
    return f;
  };

  auto compute = [&](auto S) {
    const uint8_t* a = stage(S);
    const uint8_t* w = stage(S) + ABYTES;
    const uint32_t* s = stage_s(S);
    Frag fb[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = read_frag(w, wn * WTN + 16 * j + (lane & 15));
    if constexpr (MODE == MODE_BLOCK) {
      const float swv = __uint_as_float(s[64 * NW + wave * 64]);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const Frag fa = read_frag(a, wm * WTM + 16 * i + (lane & 15));
        // rows 4*(lane/16) + r of this 16-row tile are consecutive scale words
        const int r0 = wm * WTM + 16 * i + 4 * (lane >> 4);
        const uint4 sx4 = *reinterpret_cast<const uint4*>(s + sa_word(r0));
        const float sc[4] = {__uint_as_float(sx4.x) * swv, __uint_as_float(sx4.y) * swv,
                             __uint_as_float(sx4.z) * swv, __uint_as_float(sx4.w) * swv};
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const v4f P = mfma_plain(fa.v, fb[j].v, v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(P[r], sc[r], acc[i][j][r]);
        }
      }
    } else if constexpr (MODE == MODE_TENSOR) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const Frag fa = read_frag(a, wm * WTM + 16 * i + (lane & 15));
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_plain(fa.v, fb[j].v, acc[i][j]);
      }
    } else {
      const int sh = 8 * (lane >> 4);
      int swb[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) swb[j] = (s[sw_word(wn * WTN + 16 * j + (lane & 15))] >> sh) & 0xFF;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const Frag fa = read_frag(a, wm * WTM + 16 * i + (lane & 15));
        const int sab = (s[sa_word(wm * WTM + 16 * i + (lane & 15))] >> sh) & 0xFF;
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_mx(fa.v, fb[j].v, acc[i][j], sab, swb[j]);
      }
    }
  };

  // step kb: stage S = kb % NS holds block kb.  Blocks kb+1 .. kb+NS-2 may
  // still be in flight; block kb+NS-1 is issued into the stage freed by kb-1.
  auto step = [&](auto S, auto S_issue, int kb) {
    const int ahead = min(p.KB - 1 - kb, NS - 2);     // blocks issued after kb
    if constexpr (NS == 2) {
      wait_vmcnt<0>();
    } else if constexpr (NS == 3) {
      if (ahead >= 1) wait_vmcnt<NLOAD>(); else wait_vmcnt<0>();
    } else {
      if (ahead >= 2) wait_vmcnt<2 * NLOAD>(); else if (ahead == 1) wait_vmcnt<NLOAD>(); else wait_vmcnt<0>();
    }
    // plain s_barrier: a __syncthreads() fence would wait for every load in flight
    __builtin_amdgcn_s_barrier();
    if (kb + NS - 1 < p.KB) issue(S_issue, kb + NS - 1);
    compute(S);
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;

  issue(S0{}, 0);
  if (NS > 2 && p.KB > 1) issue(S1{}, 1);
  if (NS > 3 && p.KB > 2) issue(S2{}, 2);
  for (int kb = 0; kb < p.KB; kb += NS) {
    if constexpr (NS == 2) {
      step(S0{}, S1{}, kb);
      if (kb + 1 < p.KB) step(S1{}, S0{}, kb + 1);
    } else if constexpr (NS == 3) {
      step(S0{}, S2{}, kb);
      if (kb + 1 < p.KB) step(S1{}, S0{}, kb + 1);
      if (kb + 2 < p.KB) step(S2{}, S1{}, kb + 2);
    } else {
      step(S0{}, S3{}, kb);
      if (kb + 1 < p.KB) step(S1{}, S0{}, kb + 1);
      if (kb + 2 < p.KB) step(S2{}, S1{}, kb + 2);
      if (kb + 3 < p.KB) step(S3{}, S2{}, kb + 3);
    }
  }

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

// Tile configuration: 0 = 256x128 tile, 8 waves, 3 stages (one workgroup
// per CU); 1 = 128x128 tile, 4 waves, 2 stages (two workgroups per CU, whose
// independent barriers overlap).  Measured on MI355X: 1 is faster for the
// block and per-tensor modes, 0 for MX.  FP8Q_GEMM_CFG overrides (tuning).
static int gemm_fast_cfg(int mode) {
  static const int forced = [] {
    const char* e = getenv("FP8Q_GEMM_CFG");
    return e ? atoi(e) : -1;
  }();
  if (forced == 0 || forced == 1) return forced;
  return mode == MODE_MX ? 0 : 1;
}

static int cfg_bm(int cfg) { return cfg == 1 ? 128 : 256; }

bool gemm_fast_eligible(const GemmArgs& p, int mode) {
  const int bm = cfg_bm(gemm_fast_cfg(mode));
  const int64_t a_bytes = (int64_t)p.M * p.lda + bm * p.lda;     // + rows past M of the last tile
  const int64_t w_bytes = (int64_t)p.N * p.ldw + FBN * p.ldw;
  const int64_t lim = (int64_t(1) << 31) - 1;
  return p.M > 64 && p.K % 128 == 0 && a_bytes < lim && w_bytes < lim &&
         (int64_t)(p.M + bm) * p.KB * 4 < lim && (int64_t)(p.M + bm) * p.KB32 < lim &&
         (int64_t)(p.N + FBN) * p.KB32 < lim;
}

template <int MODE>
static void launch_cfg(const GemmArgs& p, int cfg, hipStream_t stream) {
  const dim3 grid(p.tiles_m * p.tiles_n);
  if (cfg == 1) hipLaunchKernelGGL((gemm_fast_kernel<MODE, 128, 4, 2>), grid, dim3(256), 0, stream, p);
  else hipLaunchKernelGGL((gemm_fast_kernel<MODE, 256, 8, 3>), grid, dim3(512), 0, stream, p);
}

hipError_t launch_gemm_fast(GemmArgs p, int mode, hipStream_t stream) {
  const int cfg = gemm_fast_cfg(mode);
  const int bm = cfg_bm(cfg);
  p.tiles_m = (p.M + bm - 1) / bm;
  p.tiles_n = (p.N + FBN - 1) / FBN;
  if (mode == MODE_BLOCK) launch_cfg<MODE_BLOCK>(p, cfg, stream);
  else if (mode == MODE_TENSOR) launch_cfg<MODE_TENSOR>(p, cfg, stream);
  else launch_cfg<MODE_MX>(p, cfg, stream);
  return hipGetLastError();
}

}  // namespace fp8q
