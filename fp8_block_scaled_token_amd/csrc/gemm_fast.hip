// Prefill-shaped scaled FP8 GEMM for gfx950 (the fast path of
// fp8q_gemm_blockscale / fp8q_gemm_mxfp8).
//
// Same arithmetic as the generic kernels (block rescale per 128-wide K block,
// per-tensor, or MX scales inside the MFMA; see gemm_kernels.hip), organised
// for throughput on CDNA4:
//  * Large workgroup tiles.  One K block of a BM x BN tile moves
//    (BM + BN) * 128 bytes from L2 through the CU's vector cache into LDS;
//    at the fp8 MFMA rate a 128 x 128 tile would need that path's whole
//    bandwidth, a 256 x 256 tile needs half of it.  The big configuration
//    is 256 x 256 with 8 waves (2 x 4, 128 x 64 per wave: 8 x 4 MFMA tiles),
//    one workgroup per CU; the small one is 128 x 128 with 4 waves, two
//    workgroups per CU, for shapes with few tiles.
//  * Operands move global -> LDS with buffer_load ... lds (no VGPR staging).
//    Such a load writes 16 bytes per lane to consecutive LDS addresses, so the
//    XOR row swizzle of the LDS tile is produced by choosing, per lane, which
//    16-byte chunk of global memory to fetch.  Rows past M or N fall outside
//    the buffer descriptor and read as zero.
//  * Two LDS stages, one barrier per K block; the loop body is a single basic
//    block so the scheduler can interleave the block-mode rescale FMAs of one
//    16-row tile with the MFMAs of the next.
//  * Tail balancing: when the last round of tiles would leave at least half
//    of the CUs idle, those tiles are split into two half-height tiles, which
//    fill the machine and take half as long.
//  * Workgroup ids are renumbered XCD-aware and tiles walked in groups of
//    tile rows, so tiles sharing A rows or W rows meet in the same L2.
// Preconditions (checked by the launcher): K % 128 == 0, every operand and
// scale array smaller than 2^31 bytes, M > 64.
#include <cstdlib>
#include <utility>

#include "gemm_common.h"
#include "launch.h"

// K blocks between an L2 prefetch touch and the operand loads it serves
// (0 disables the touches).
#ifndef FP8Q_PREFETCH_DISTANCE
#define FP8Q_PREFETCH_DISTANCE 3
#endif

namespace fp8q {

namespace {

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
// compiler's vmcnt bookkeeping; the kernel waits for them explicitly and
// issues no other vector-memory loads inside its K loop.
__device__ __forceinline__ void dma16(const i32x4& r, uint32_t lds, uint32_t voffset) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(r), "s"(lds)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const i32x4& r, uint32_t lds, uint32_t voffset) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voffset), "s"(r), "s"(lds)
               : "memory", "m0");
}

// Added to a load offset that must not read memory: every descriptor covers
// fewer than 2^31 bytes, so the load falls out of range and writes zeros.
constexpr uint32_t OOB = 0x80000000u;

template <int... I, typename F>
__device__ __forceinline__ void static_for_impl(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(std::make_integer_sequence<int, N>{}, f);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// Wait until at most N of this wave's global loads are in flight and all of
// its LDS reads have returned, then a workgroup barrier.  One asm statement
// with a memory clobber, so no LDS access moves across it.  (A
// __syncthreads() fence would wait for every global load.)
template <int N>
__device__ __forceinline__ void wait_vmcnt_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" : : "n"(N) : "memory");
}

}  // namespace

// Geometry of one fast-kernel configuration: BM x BN workgroup tile, WM x WN
// waves.  Stage layout in LDS (2 stages): A tile [BM][128] and W tile
// [BN][128], both swizzled; then 64 A-scale words per wave, then 64 W-scale
// words per wave.
template <int MODE_, int BM_, int BN_, int WM_, int WN_, int NTN_>
struct FastTile {
  static constexpr int MODE = MODE_, BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  // tile columns of one XCD's concurrently running group of tiles (the XCD's
  // workgroup slots divided by the group height of group_walk)
  static constexpr int NTN = NTN_;
  static constexpr int NW = WM * WN;
  static constexpr int WTN = BN / WN, TN = WTN / 16;
  static constexpr int ABYTES = BM * 128, WBYTES = BN * 128;
  static constexpr int A_PER = ABYTES / 1024 / NW;  // 1 KB loads per wave per stage
  static constexpr int W_PER = WBYTES / 1024 / NW;
  static constexpr int SA_OFF = ABYTES + WBYTES;
  static constexpr int SW_OFF = SA_OFF + NW * 256;
  static constexpr int STAGE = SW_OFF + NW * 256;
  static constexpr int NS = 2;
  static constexpr int PF_OFF = NS * STAGE;            // 256 bytes per wave: prefetch sink
  static constexpr int LDS_BYTES = PF_OFF + NW * 256;
  static_assert(BM == 32 * NW && BN == 32 * NW, "each wave fetches the scales of 32 rows");
  static_assert(A_PER * NW * 1024 == ABYTES && W_PER * NW * 1024 == WBYTES, "whole 1 KB loads");
  static_assert(WTN <= 128 && 128 % WTN == 0, "one weight-scale block per wave");
  static_assert(STAGE % 1024 == 0, "stages stay 1 KB aligned");
};

// One tile: rows [m0, m0 + RM) x columns [n0, n0 + BN), RM = BM (full) or
// BM / 2 (HALF).
template <class T, bool HALF>
__device__ __forceinline__ void fast_tile(const GemmArgs& p, uint8_t* smem, int m0, int n0, int gm, int gn) {
  constexpr int MODE = T::MODE, BN = T::BN, WN = T::WN;
  constexpr int RM = HALF ? T::BM / 2 : T::BM;
  constexpr int WTM = RM / T::WM, TM = WTM / 16, WTN = T::WTN, TN = T::TN;
  constexpr int A_PER = T::A_PER, W_PER = T::W_PER, STAGE = T::STAGE;
  constexpr int ABYTES = T::ABYTES, SA_OFF = T::SA_OFF, SW_OFF = T::SW_OFF;
  static_assert(TM >= 1, "wave tile at least 16 rows");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;

  const i32x4 rA = rsrc(p.a, (int64_t)p.M * p.lda);
  const i32x4 rW = rsrc(p.w, (int64_t)p.N * p.ldw);
  const i32x4 rSA =
      rsrc(p.sa, MODE == MODE_MX ? (int64_t)p.M * p.KB32 : (MODE == MODE_BLOCK ? (int64_t)p.M * p.KB * 4 : 4));
  const i32x4 rSW =
      rsrc(p.sw, MODE == MODE_MX ? (int64_t)p.N * p.KB32 : (MODE == MODE_BLOCK ? (int64_t)p.NB * p.KB * 4 : 4));

  // Load i of wave w fills LDS kilobyte (A_PER*w + i) of the A tile, i.e.
  // tile rows 8*(A_PER*w + i) + lane/8 with lane % 8 the physical chunk; the
  // logical chunk to fetch is (lane % 8) ^ (row % 8) = (lane % 8) ^ (lane / 8).
  // A half tile needs only its first RM rows: the other loads are kept (for
  // the vmcnt count) but read nothing.
  const int lrow = lane >> 3, lchunk = (lane & 7) ^ (lane >> 3);
  const int offA = (m0 + 8 * A_PER * wave + lrow) * (int)p.lda + lchunk * 16;
  const int offW = (n0 + 8 * W_PER * wave + lrow) * (int)p.ldw + lchunk * 16;
  const int lda8 = 8 * (int)p.lda, ldw8 = 8 * (int)p.ldw;
  // scales: lane l of wave w fetches A row 32w + l % 32 (and, MX, W row
  // 32w + l % 32) into scale word 64w + l; block mode: W block n0/128 + l % NBLK
  constexpr int NBLK = BN / 128 > 0 ? BN / 128 : 1;
  const int srow = m0 + 32 * wave + (lane & 31);
  const int swrow = n0 + 32 * wave + (lane & 31);
  const int sa_row = p.sa_col_major ? srow : srow * p.KB;   // block-mode A scale (row, kb)
  const int sa_kstride = p.sa_col_major ? p.M : 1;
  const int wblk = n0 / 128 + lane % NBLK;
  const uint32_t smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));

  // Fill stage `st` with K block kb.  Past the last block the loads are kept
  // (so every step issues the same number) but read nothing and write zeros
  // into the free stage.
  auto issue = [&](int st, int kb) {
    const bool valid = kb < p.KB;
    const uint32_t oob = valid ? 0u : OOB;
    const uint32_t base = smem_base + st * STAGE;
    const uint32_t a = base + wave * A_PER * 1024;
    const uint32_t w = base + ABYTES + wave * W_PER * 1024;
    const int kofs = valid ? kb * 128 : 0;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const bool live = !HALF || (A_PER * wave + i) * 8 < RM;
      dma16(rA, a + i * 1024, (uint32_t)(offA + i * lda8 + kofs) + (live ? oob : OOB));
    }
#pragma unroll
    for (int i = 0; i < W_PER; ++i) dma16(rW, w + i * 1024, (uint32_t)(offW + i * ldw8 + kofs) + oob);
    const int kbv = valid ? kb : 0;
    const uint32_t sa_lds = base + SA_OFF + wave * 256, sw_lds = base + SW_OFF + wave * 256;
    if constexpr (MODE == MODE_BLOCK) {
      dma4(rSA, sa_lds, (uint32_t)((sa_row + kbv * sa_kstride) * 4) + oob);
      dma4(rSW, sw_lds, (uint32_t)((wblk * p.KB + kbv) * 4) + oob);
    } else if constexpr (MODE == MODE_MX) {
      dma4(rSA, sa_lds, (uint32_t)(srow * p.KB32 + kbv * 4) + oob);
      dma4(rSW, sw_lds, (uint32_t)(swrow * p.KB32 + kbv * 4) + oob);
    }
  };
  // L2 prefetch.  Tiles running together on one XCD share operand rows: the
  // NTN tiles of a tile row read the same A rows, the 8 tiles of a tile
  // column (group_walk's group height) the same W rows.  Every workgroup
  // touches one line (the 128 bytes of a K block) of its share of those rows,
  // PFD K blocks ahead, so that the operand loads find them in L2.  The
  // touches go to a per-wave LDS sink; they are issued after the operand
  // loads of a step and may stay in flight until the next step's wait.
  constexpr int PFD = FP8Q_PREFETCH_DISTANCE;
  constexpr int PA = RM / T::NTN / T::NW, PW = BN / 8 / T::NW;   // rows per wave
  static_assert(PA >= 1 && PA <= 64 && PW >= 1 && PW <= 64, "prefetch slice");
  const uint32_t pfa = (uint32_t)(m0 + gn * (RM / T::NTN) + wave * PA + lane) * (uint32_t)p.lda;
  const uint32_t pfw = (uint32_t)(n0 + gm * (BN / 8) + wave * PW + lane) * (uint32_t)p.ldw;
  const uint32_t pf_lds = smem_base + T::PF_OFF + wave * 256;
  auto prefetch = [&](int kb) {
    const bool valid = PFD > 0 && kb < p.KB;
    const uint32_t kofs = valid ? (uint32_t)kb * 128u : 0u;
    dma4(rA, pf_lds, (valid && lane < PA) ? pfa + kofs : OOB);
    dma4(rW, pf_lds, (valid && lane < PW) ? pfw + kofs : OOB);
  };

  // scale word of tile row r / tile column c
  auto s_word = [](int r) { return 64 * (r >> 5) + (r & 31); };

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

  // Block mode rescale, software-pipelined: the MFMAs of 16-row tile i give
  // P (fp32 partial products of this K block); P is folded into the
  // accumulators (acc += P * s_a * s_w) while the MFMAs of tile i + 1 run.
  // The last tile's P is folded at the start of the next K block (or before
  // the epilogue).
  v4f Pq[TN];
  float scq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < TN; ++j) Pq[j] = v4f{0.f, 0.f, 0.f, 0.f};
  auto fold = [&](auto I) {
    constexpr int i = decltype(I)::value;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(Pq[j][r], scq[r], acc[i][j][r]);
  };

  const int arow = wm * WTM + (lane & 15);           // fragment row of 16-row tile 0
  const int brow = wn * WTN + (lane & 15);
  auto compute = [&](int st) {
    const uint8_t* a = smem + st * STAGE;
    const uint8_t* w = a + ABYTES;
    const uint32_t* sa = reinterpret_cast<const uint32_t*>(a + SA_OFF);
    const uint32_t* sw = reinterpret_cast<const uint32_t*>(a + SW_OFF);
    Frag fb[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = read_frag(w, brow + 16 * j);
    if constexpr (MODE == MODE_BLOCK) {
      const float swv = __uint_as_float(sw[wave * 64 + (wn * WTN) / 128]);
      // rows 4*(lane/16) + r of a 16-row tile are consecutive scale words
      const int srow0 = wm * WTM + 4 * (lane >> 4);
      Frag fa = read_frag(a, arow);
      uint4 sx4 = *reinterpret_cast<const uint4*>(sa + s_word(srow0));
      static_for<TM>([&](auto I) {
        constexpr int i = decltype(I)::value;
        Frag fn;
        uint4 sxn;
        if constexpr (i + 1 < TM) {
          fn = read_frag(a, arow + 16 * (i + 1));
          sxn = *reinterpret_cast<const uint4*>(sa + s_word(srow0 + 16 * (i + 1)));
        }
        v4f Pn[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) Pn[j] = mfma_plain(fa.v, fb[j].v, v4f{0.f, 0.f, 0.f, 0.f});
        fold(std::integral_constant<int, (i == 0 ? TM - 1 : i - 1)>{});
#pragma unroll
        for (int j = 0; j < TN; ++j) Pq[j] = Pn[j];
        scq[0] = __uint_as_float(sx4.x) * swv;
        scq[1] = __uint_as_float(sx4.y) * swv;
        scq[2] = __uint_as_float(sx4.z) * swv;
        scq[3] = __uint_as_float(sx4.w) * swv;
        if constexpr (i + 1 < TM) {
          fa = fn;
          sx4 = sxn;
        }
      });
    } else if constexpr (MODE == MODE_TENSOR) {
      static_for<TM>([&](auto I) {
        constexpr int i = decltype(I)::value;
        const Frag fa = read_frag(a, arow + 16 * i);
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_plain(fa.v, fb[j].v, acc[i][j]);
      });
    } else {
      const int sh = 8 * (lane >> 4);
      int swb[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) swb[j] = (sw[s_word(brow + 16 * j)] >> sh) & 0xFF;
      static_for<TM>([&](auto I) {
        constexpr int i = decltype(I)::value;
        const Frag fa = read_frag(a, arow + 16 * i);
        const int sab = (sa[s_word(arow + 16 * i)] >> sh) & 0xFF;
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = mfma_mx(fa.v, fb[j].v, acc[i][j], sab, swb[j]);
      });
    }
  };

  // Main loop, one K block per iteration: wait for this wave's loads of
  // block kb, barrier (every wave's part of block kb has landed and no wave
  // still reads the stage of block kb-1), refill that stage with block kb+1,
  // multiply block kb.
  // The two prefetch touches issued after a step's loads may stay in flight.
  static_assert(T::NS == 2, "the wait count below assumes two stages");
  issue(0, 0);
  prefetch(PFD - 1);
  int cs = 0;
  for (int kb = 0; kb < p.KB; ++kb) {
    wait_vmcnt_barrier<2>();
    issue(cs ^ 1, kb + 1);
    prefetch(kb + PFD);
    compute(cs);
    cs ^= 1;
  }
  // the predicated-off loads still write LDS: let them land before exit
  wait_vmcnt<0>();
  if constexpr (MODE == MODE_BLOCK) fold(std::integral_constant<int, TM - 1>{});

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

// Workgroups [0, full) take whole tiles (in XCD-contiguous group order);
// the remaining tiles of that order are split into two half-height tiles,
// one per workgroup.
template <class T>
__global__ __launch_bounds__(T::NW * 64) void gemm_fast_kernel(GemmArgs p, int full) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];
  const int total = p.tiles_m * p.tiles_n;
  const int b = blockIdx.x;
  int tm, tn;
  if (b < full) {
    group_walk(xcd_contiguous(b, full), p.tiles_m, p.tiles_n, tm, tn);
    fast_tile<T, false>(p, smem, tm * T::BM, tn * T::BN, tm % 8, tn % T::NTN);
  } else {
    const int h = xcd_contiguous(b - full, 2 * (total - full));
    group_walk(full + (h >> 1), p.tiles_m, p.tiles_n, tm, tn);
    fast_tile<T, true>(p, smem, tm * T::BM + (h & 1) * (T::BM / 2), tn * T::BN, tm % 8, tn % T::NTN);
  }
}

namespace {

// Configuration 0: 256 x 256 tiles, 8 waves, one workgroup per CU.
// Configuration 1: 128 x 128 tiles, 4 waves, two workgroups per CU.
// Tuning and test overrides, read at every call: FP8Q_GEMM_CFG=0/1 forces a
// configuration, FP8Q_GEMM_SPLIT=0 disables the half-tile tail balancing,
// FP8Q_GEMM_SLOTS=n plans for n CUs instead of the device's count.
int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  return e ? atoi(e) : dflt;
}

int cu_count() {
  const int forced = env_int("FP8Q_GEMM_SLOTS", 0);
  return forced > 0 ? forced : device_cu_count();
}

struct Plan {
  int cfg;       // 0 = 256 x 256, 1 = 128 x 128
  int tiles_m, tiles_n;
  int full;      // workgroups that take whole tiles
  int grid;
};

// Tiles of one configuration and how many of them to split: when the last
// round would occupy at most half of the workgroup slots, split it.
Plan plan_cfg(const GemmArgs& p, int cfg, int slots, bool split) {
  const int bm = cfg == 0 ? 256 : 128, bn = bm;
  Plan pl;
  pl.cfg = cfg;
  pl.tiles_m = (p.M + bm - 1) / bm;
  pl.tiles_n = (p.N + bn - 1) / bn;
  const int total = pl.tiles_m * pl.tiles_n;
  const int rem = total % slots;
  const int tail = (split && total > slots && rem > 0 && 2 * rem <= slots) ? rem : 0;
  pl.full = total - tail;
  pl.grid = total + tail;
  return pl;
}

// Estimated time in units of one 256 x 256 tile on one CU; the 128 x 128
// configuration runs two tiles per CU at a lower MFMA efficiency.
double plan_cost(const Plan& pl, int cus) {
  const int slots = pl.cfg == 0 ? cus : 2 * cus;
  const int total = pl.tiles_m * pl.tiles_n;
  const int tail = total - pl.full;
  const double rounds = (pl.full + slots - 1) / slots + (tail > 0 ? 0.5 : 0.0);
  const double per_round = pl.cfg == 0 ? 1.0 : 0.5 / 0.8;
  return rounds * per_round;
}

Plan choose_plan(const GemmArgs& p) {
  const int forced = env_int("FP8Q_GEMM_CFG", -1);
  const bool split = env_int("FP8Q_GEMM_SPLIT", 1) != 0;
  const int cus = cu_count();
  const Plan big = plan_cfg(p, 0, cus, split), small = plan_cfg(p, 1, 2 * cus, split);
  if (forced == 0) return big;
  if (forced == 1) return small;
  return plan_cost(big, cus) <= plan_cost(small, cus) ? big : small;
}

template <int MODE>
void launch_plan(GemmArgs p, const Plan& pl, hipStream_t stream) {
  p.tiles_m = pl.tiles_m;
  p.tiles_n = pl.tiles_n;
  if (pl.cfg == 0) {
    using T = FastTile<MODE, 256, 256, 2, 4, 4>;
    hipLaunchKernelGGL(gemm_fast_kernel<T>, dim3(pl.grid), dim3(T::NW * 64), 0, stream, p, pl.full);
  } else {
    using T = FastTile<MODE, 128, 128, 2, 2, 8>;
    hipLaunchKernelGGL(gemm_fast_kernel<T>, dim3(pl.grid), dim3(T::NW * 64), 0, stream, p, pl.full);
  }
}

}  // namespace

bool gemm_fast_eligible(const GemmArgs& p, int /*mode*/) {
  const int bm = 256, bn = 256;  // the larger configuration bounds both
  const int64_t a_bytes = (int64_t)p.M * p.lda + bm * p.lda;     // + rows past M of the last tile
  const int64_t w_bytes = (int64_t)p.N * p.ldw + bn * p.ldw;
  const int64_t lim = (int64_t(1) << 31) - 1;
  return p.M > 64 && p.K % 128 == 0 && a_bytes < lim && w_bytes < lim &&
         (int64_t)(p.M + bm) * p.KB * 4 < lim && (int64_t)(p.M + bm) * p.KB32 < lim &&
         (int64_t)(p.N + bn) * p.KB32 < lim && (int64_t)(p.NB + 2) * p.KB * 4 < lim;
}

hipError_t launch_gemm_fast(GemmArgs p, int mode, hipStream_t stream) {
  const Plan pl = choose_plan(p);
  if (mode == MODE_BLOCK) launch_plan<MODE_BLOCK>(p, pl, stream);
  else if (mode == MODE_TENSOR) launch_plan<MODE_TENSOR>(p, pl, stream);
  else launch_plan<MODE_MX>(p, pl, stream);
  return hipGetLastError();
}

}  // namespace fp8q
