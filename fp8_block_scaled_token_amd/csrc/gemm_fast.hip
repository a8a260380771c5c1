// Prefill-shaped scaled FP8 GEMM for gfx950 (the fast path of
// fp8q_gemm_blockscale / fp8q_gemm_mxfp8).
//
// Same arithmetic as the generic kernels (block rescale per 128-wide K block,
// per-tensor, or MX scales inside the MFMA; see gemm_kernels.hip), organised
// for throughput on CDNA4:
//  * Transposed MFMA tiles.  Each 16x16x128 MFMA takes a weight fragment as
//    its first operand and an activation fragment as its second, so a lane
//    holds four consecutive output COLUMNS of one output ROW.  In block mode
//    the four partial products of a lane then share one activation scale:
//    the per-K-block rescale is 4 FMAs per MFMA plus one scale product per
//    16 rows, close to the VALU issue slots that an fp8 MFMA leaves free
//    (three to four wave64 instructions per MFMA on one SIMD, measured).
//    The epilogue exchanges bf16 pairs across the four lanes of a row and
//    writes 16-byte runs.
//  * Large workgroup tiles.  One K block of a BM x BN tile moves
//    (BM + BN) * 128 bytes from L2 through the CU's vector cache into LDS;
//    the big configuration is 256 x 256 with 8 waves (2 x 4, 128 rows x 64
//    columns per wave), one workgroup per CU; the small one is 128 x 128 with
//    4 waves, two workgroups per CU, for shapes with few tiles.
//  * Operands move global -> LDS with buffer_load ... lds (no VGPR staging).
//    Such a load writes 16 bytes per lane to consecutive LDS addresses, so the
//    XOR row swizzle of the LDS tile is produced by choosing, per lane, which
//    16-byte chunk of global memory to fetch.  The per-lane offsets are fixed
//    for the whole K loop and the K position travels in the scalar offset,
//    so issuing a K block costs no vector instructions.  Rows past M or N are
//    given an offset outside the buffer descriptor and read as zero.
//  * Two LDS stages, one barrier per K block; the K loop body is a single
//    basic block so the scheduler can interleave the block-mode rescale FMAs
//    of one 16-row tile with the MFMAs of the next.
//  * Tail balancing: when the last round of tiles would leave at least half
//    of the CUs idle, those tiles are split into two half-height tiles, which
//    fill the machine and take half as long -- or, given a workspace, into
//    their two K halves, the second continuing from the first's fp32
//    accumulators (full-height tiles, the same bits as unsplit).  The
//    grouped (MoE) kernel sizes an expert's last row tile to its rows: a
//    half- or three-quarter-height tile where they fit.
//  * Workgroup ids are renumbered XCD-aware and tiles walked in groups of
//    tile rows, so tiles sharing A rows or W rows meet in the same L2, and
//    every workgroup touches its share of the operand lines a few K blocks
//    ahead so that the LDS loads find them in L2.
// Preconditions (checked by the launcher): K % 128 == 0, every operand and
// scale array smaller than 2^31 bytes, M > 64.
#include <utility>

#include <atomic>

#include "dma.h"
#include "gemm_common.h"
#include "launch.h"

// K blocks between an L2 prefetch touch and the operand loads it serves
// (0 disables the touches).
#ifndef FP8Q_PREFETCH_DISTANCE
#define FP8Q_PREFETCH_DISTANCE 3
#endif
// 16-row tiles between the LDS read of an activation fragment and its use.
#ifndef FP8Q_A_LOOKAHEAD
#define FP8Q_A_LOOKAHEAD 1
#endif
// Issue points after the first over which a K block's loads are spread.
#ifndef FP8Q_LOAD_SLOTS
#define FP8Q_LOAD_SLOTS 4
#endif

namespace fp8q {

using namespace dma;

// Geometry of one fast-kernel configuration: BM x BN workgroup tile, WM x WN
// waves.  Stage layout in LDS (2 stages): A tile [BM][128] and W tile
// [BN][128], both swizzled; then the scale words of the stage's K block: BM
// activation-scale words, then BN weight-scale words (MX: one word = the four
// 32-wide blocks of a row; block mode: only the first BN/128 words are used).
template <int MODE_, int BM_, int BN_, int WM_, int WN_, int NTN_>
struct FastTile {
  static constexpr int MODE = MODE_, BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  // fp32 scale words (block mode, and its power-of-two view)
  static constexpr bool FP32S = MODE == MODE_BLOCK || MODE == MODE_BMX;
  // MX scale bytes, row-major ([rows][K/32]) or column-major ([K/32][rows])
  static constexpr bool MXS = MODE == MODE_MX || MODE == MODE_MXC;
  // tile columns of one XCD's concurrently running group of tiles (the XCD's
  // workgroup slots divided by the group height of group_walk)
  static constexpr int NTN = NTN_;
  static constexpr int NW = WM * WN;
  static constexpr int WTN = BN / WN, TN = WTN / 16;
  static constexpr int ABYTES = BM * 128, WBYTES = BN * 128;
  static constexpr int A_PER = ABYTES / 1024 / NW;  // 1 KB loads per wave per stage
  static constexpr int W_PER = WBYTES / 1024 / NW;
  static constexpr int SA_OFF = ABYTES + WBYTES;
  static constexpr int SW_OFF = SA_OFF + BM * 4;
  static constexpr int STAGE = ((SW_OFF + BN * 4) + 1023) / 1024 * 1024;
  static constexpr int NS = 2;
  // 1 KB per wave: sink for prefetch touches and for loads past the last K
  // block, so that those never write a stage
  static constexpr int SINK_OFF = NS * STAGE;
  // a split tail tile's consumer decision (one word, broadcast to all waves)
  static constexpr int XCH_OFF = SINK_OFF + NW * 1024;
  static constexpr int LDS_BYTES = XCH_OFF + 16;
  static_assert(LDS_BYTES <= 160 * 1024, "fits the CU's LDS");
  // scale loads: one 64-word load per wave covers the BM + BN scale words
  static constexpr int SCALE_LOADS = MODE == MODE_TENSOR ? 0 : 1;
  static_assert(NW * 64 == BM + BN, "one scale word per lane");
  static_assert(A_PER * NW * 1024 == ABYTES && W_PER * NW * 1024 == WBYTES, "whole 1 KB loads");
  static_assert(WTN <= 128 && 128 % WTN == 0, "one weight-scale block per wave");
  static_assert(STAGE % 1024 == 0, "stages stay 1 KB aligned");
};

// One tile: rows [m0, m0 + RM) x columns [n0, n0 + BN), RM = BM * RQ / 4:
// a whole tile (RQ = 4), or a short one for the last rows of an expert in
// the grouped GEMM (3/4: RQ = 3) or a half-height tile (RQ = 2).
// `preloaded`: the previous tile of this workgroup already issued this tile's
// first K block (and its touches) before its epilogue.  `has_next`: issue the
// first K block of the next tile (nm0, nn0, ngm, ngn) before this tile's
// epilogue, so that its latency overlaps the output stores.
// K range of a tile and, for the two K halves of a split tail tile, how the
// halves meet (the exchange below).  The producer computes K blocks
// [0, KB/2) as its workgroup's first item and leaves its fp32 accumulators in
// `part`; the consumer computes [KB/2, KB) as its workgroup's last item,
// starting from those accumulators instead of zeros, and writes the output.
// Each output element thus sees the same sequence of rescaled block products
// as in an unsplit tile, so the split changes no bit of the result.  If the
// partial has not appeared when the consumer arrives (within the wait
// limit), the consumer computes the whole tile itself.
// Cache policy bits of a buffer access (SC0 | SC1): system scope, i.e. a
// store writes through to memory and a load misses the caches.
constexpr int kCacheSystem = 1 | 16;

struct TileK {
  int kb0, kb1;        // K blocks [kb0, kb1)
  int next_kb0;        // first K block of the next tile (issued early when has_next)
  int role;            // 0: whole tile, 1: producer, 2: consumer (the two K halves of a tile)
  float* part;         // 256 KB partial slot of the pair
  uint64_t* flags;     // the pair's words: [0] producer's flag, [1] consumer's flag, [2] outcome
  uint32_t tag;        // this launch's tag (never 0)
  // the previous item was a producer's K half: publish its partial (these
  // flag words) once this tile's first wait has seen its stores complete
  uint64_t* publish;
};

// Words of a split tail tile pair.  Only system-scope loads and stores touch
// them (each completes at memory; no read-modify-write), so the two
// workgroups, on different XCDs, agree without a coherent cache:
//   producer: partial -> memory, then flags[0] = PUBLISHED; later (at the
//             end of the kernel) it reads flags[1] and, if the consumer has
//             given up, resets both flag words;
//   consumer: waits (bounded) for flags[0] == PUBLISHED and then resets it;
//             past the limit it writes flags[1] = GAVE_UP, reads flags[0]
//             once more, and either consumes after all (resetting both) or
//             computes the whole tile itself.
// Each side's store completes before its read of the other's word, so at
// least one of them sees the other's word: either the consumer finds the
// partial or the producer finds the give-up (or both; both then reset both
// words).  The last one to act leaves both flag words 0, so a graph replay,
// which reuses the tag, starts from a clean state.  A word counts only if it
// holds this launch's tag and marker: whatever else the workspace held is
// ignored.  flags[2] records the consumer's outcome (CONSUMED or GAVE_UP with
// the tag) for inspection; nothing reads it on the device.
constexpr uint32_t kPublished = 0x5AFE0001u, kGaveUp = 0x5AFE0002u, kConsumed = 0x5AFE0003u;
__device__ __forceinline__ uint64_t flag_word(uint32_t tag, uint32_t marker) {
  // formed where it is used (rarely): kept opaque so that the compiler does
  // not hoist the word out of the tile loop and hold a register for it
  uint64_t w = ((uint64_t)tag << 32) | marker;
  asm volatile("" : "+s"(w));
  return w;
}
__device__ __forceinline__ void flag_store(uint64_t* w, uint64_t v) {
  __hip_atomic_store(w, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
__device__ __forceinline__ uint64_t flag_load(uint64_t* w) {
  return __hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Returns true when this workgroup, the consumer of a split tail tile, gave
// up waiting for its partner's partial: nothing was written, and the caller
// then computes the whole tile (the producer writes no output either).
template <class T, int RQ, bool SPLIT, bool NTW = false>
__device__ __forceinline__ bool fast_tile(const GemmArgs& p, uint8_t* smem, int m0, int n0, int gm, int gn,
                                          bool preloaded, bool has_next, int nm0, int nn0, int ngm, int ngn,
                                          const TileK& tk) {
  constexpr int MODE = T::MODE, BM = T::BM, BN = T::BN, WN = T::WN, NW = T::NW;
  constexpr bool FP32S = T::FP32S, MXC = MODE == MODE_MXC;
  static_assert(RQ >= 2 && RQ <= 4, "tile height in quarters");
  constexpr int RM = T::BM * RQ / 4;
  constexpr int WTM = RM / T::WM, TM = WTM / 16, WTN = T::WTN, TN = T::TN;
  // a short tile's activation rows are spread over all waves too
  constexpr int A_PER = RM * 128 / 1024 / NW, W_PER = T::W_PER, STAGE = T::STAGE;
  static_assert(A_PER >= 1 && A_PER * NW * 1024 == RM * 128, "whole 1 KB activation loads");
  constexpr int ABYTES = T::ABYTES, SA_OFF = T::SA_OFF, SW_OFF = T::SW_OFF;
  static_assert(TM >= 1, "wave tile at least 16 rows");

  const int lane = threadIdx.x & 63, l16 = lane & 15, lq = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;

  const i32x4 rA = rsrc(p.a, (int64_t)p.M * p.lda);
  const i32x4 rW = rsrc(p.w, (int64_t)p.N * p.ldw);

  // ---- per-lane load offsets of a tile (fixed for its whole K loop)
  // Load i of wave w fills LDS kilobyte (A_PER*w + i) of the A tile, i.e.
  // tile rows 8*(A_PER*w + i) + lane/8 with lane % 8 the physical chunk; the
  // logical chunk to fetch is (lane % 8) ^ (row % 8) = (lane % 8) ^ (lane / 8).
  // Scale words: lane l of wave w fetches word q = 64w + l of the stage's
  // scale area.  Activation words are ordered [wm][row % 16][row tile] so a
  // lane reads the TM scales of its rows as consecutive words; MX weight
  // words likewise [wn][row % 16][row tile].  Block mode: weight word b
  // (b < WN) is the scale of the 128-row weight block that holds wave
  // column b's channels n0 + b*WTN .. +WTN (one block: WTN divides 128 and
  // the shard size).
  // L2 prefetch rows: tiles running together on one XCD share operand rows:
  // the NTN tiles of a tile row read the same A rows, the 8 tiles of a tile
  // column (group_walk's group height) the same W rows.  Every workgroup
  // touches one line (the 128 bytes of a K block) of its share of those rows.
  constexpr int PFD = FP8Q_PREFETCH_DISTANCE;
  constexpr int PA = RM / T::NTN / NW, PW = BN / 8 / NW;   // rows per wave
  static_assert(PA >= 1 && PA <= 64 && PW >= 1 && PW <= 64, "prefetch slice");
  struct Offs {
    uint32_t a[A_PER], w[W_PER], s, pfa, pfw;
  };
  // `ln` is the lane index; the next tile's offsets are computed from an
  // opaque copy of it so that no lane-dependent partial term of this tile's
  // offsets is kept alive through the K loop for reuse
  auto make_offs = [&](int tm0, int tn0, int tgm, int tgn, int ln) {
    const int lrow = ln >> 3, lchunk = (ln & 7) ^ (ln >> 3);
    Offs o;
#pragma unroll
    for (int i = 0; i < A_PER; ++i)
      o.a[i] = (uint32_t)((tm0 + 8 * (A_PER * wave + i) + lrow) * (int)p.lda + lchunk * 16);
#pragma unroll
    for (int i = 0; i < W_PER; ++i)
      o.w[i] = (uint32_t)((tn0 + 8 * (W_PER * wave + i) + lrow) * (int)p.ldw + lchunk * 16);
    o.s = OOB;
    if constexpr (MODE != MODE_TENSOR) {
      const int q = 64 * wave + ln;
      if (q < BM) {
        const int g = q / WTM, rem = q % WTM;             // q < RM only when g < WM
        const int row = tm0 + g * WTM + 16 * (rem % TM) + rem / TM;
        const bool live = q < RM && row < p.M;
        if (FP32S) {
          o.s = live ? (uint32_t)(p.sa_col_major ? row * 4 : row * p.KB * 4) : OOB;
        } else if (MXC) {
          // MX, [K/32][M] bytes: dword q holds rows 4r .. 4r+3 of 32-wide
          // block qb of the K block (M % 4 == 0: whole dwords in or out)
          const int qb = q / (BM / 4), r = tm0 + 4 * (q % (BM / 4));
          o.s = (r < p.M && r < tm0 + RM) ? (uint32_t)(qb * p.M + r) : OOB;
        } else {
          o.s = live ? (uint32_t)(row * p.KB32) : OOB;
        }
      } else {
        const int qw = q - BM;
        if (FP32S) {
          const int col = tn0 + qw * WTN;
          o.s = (qw < WN && col < p.N) ? (uint32_t)(weight_scale_row(p, col) * p.KB * 4) : OOB;
        } else if (MXC) {
          const int qb = qw / (BN / 4), c = tn0 + 4 * (qw % (BN / 4));
          o.s = c < p.N ? (uint32_t)(qb * p.N + c) : OOB;
        } else {
          const int g = qw / WTN, rem = qw % WTN;
          const int row = tn0 + g * WTN + 16 * (rem % TN) + rem / TN;
          o.s = row < p.N ? (uint32_t)(row * p.KB32) : OOB;
        }
      }
    }
    const int pra = tm0 + tgn * (RM / T::NTN) + wave * PA + ln;
    const int prw = tn0 + tgm * (BN / 8) + wave * PW + ln;
    o.pfa = (PFD > 0 && ln < PA && pra < p.M) ? (uint32_t)pra * (uint32_t)p.lda : OOB;
    o.pfw = (PFD > 0 && ln < PW && prw < p.N) ? (uint32_t)prw * (uint32_t)p.ldw : OOB;
    return o;
  };
  const Offs cur = make_offs(m0, n0, gm, gn, lane);

  const bool wave_is_a = 64 * wave < BM;    // waves below BM/64 fetch activation scales
  i32x4 rSA = rA, rSW = rW;
  if constexpr (FP32S) {
    rSA = rsrc(p.sa, (int64_t)p.M * p.KB * 4);
    rSW = rsrc(p.sw, (int64_t)p.NB * p.KB * 4);
  } else if constexpr (T::MXS) {
    rSA = rsrc(p.sa, (int64_t)p.M * p.KB32);
    rSW = rsrc(p.sw, (int64_t)p.N * p.KB32);
  }
  // the scalar offset of a K block: block-mode column-major activation
  // scales advance by M words, every other scale array by one word (block)
  // or four bytes (MX) per K block
  uint32_t kstepS = (FP32S && p.sa_col_major && wave_is_a) ? (uint32_t)p.M * 4u : 4u;
  if (MXC) kstepS = wave_is_a ? (uint32_t)p.M * 4u : (uint32_t)p.N * 4u;
  const i32x4 rS = wave_is_a ? rSA : rSW;
  const uint32_t smem_base = __builtin_amdgcn_readfirstlane(lds_addr(smem));

  const uint32_t sink = smem_base + T::SINK_OFF + wave * 1024;

  // Loads of one K block, numbered l = 0 .. NLD-1 (A_PER activation loads,
  // W_PER weight loads, then the scale load).  issue_load(l, st, kb, o) fills
  // its part of stage `st` with K block kb of the tile whose offsets are o.
  // Past the last block the descriptors cover nothing: the loads are still
  // issued (every block issues the same number) but read nothing and write
  // zeros into this wave's sink.
  const int KB = tk.kb1;                     // loads of blocks at or past it read nothing
  constexpr int NLD = A_PER + W_PER + T::SCALE_LOADS;
  auto issue_load = [&](auto L, int st, int kb, const Offs& o) {
    constexpr int l = decltype(L)::value;
    const bool valid = kb < KB;
    const int kbv = valid ? kb : 0;
    const uint32_t base = smem_base + st * STAGE;
    if constexpr (l < A_PER) {
      i32x4 r = rA;
      r.z = valid ? r.z : 0;
      dma16(r, valid ? base + (wave * A_PER + l) * 1024 : sink, o.a[l], (uint32_t)kbv * 128u);
    } else if constexpr (l < A_PER + W_PER) {
      i32x4 r = rW;
      r.z = valid ? r.z : 0;
      const uint32_t dst = valid ? base + ABYTES + (wave * W_PER + l - A_PER) * 1024 : sink;
      if constexpr (NTW) dma16_nt(r, dst, o.w[l - A_PER], (uint32_t)kbv * 128u);
      else dma16(r, dst, o.w[l - A_PER], (uint32_t)kbv * 128u);
    } else {
      i32x4 r = rS;
      r.z = valid ? r.z : 0;
      dma4(r, valid ? base + SA_OFF + wave * 256 : sink, o.s, (uint32_t)kbv * kstepS);
    }
  };
  // L2 prefetch touches of K block kb (PFD blocks ahead of the loads they
  // serve), into the sink; past the last K block they read nothing.  They are
  // issued after the operand loads of a step and may stay in flight until
  // the next step's wait.
  auto prefetch = [&](int kb, const Offs& o) {
    const bool valid = PFD > 0 && kb < KB;
    i32x4 ra = rA, rw = rW;
    ra.z = valid ? ra.z : 0;
    rw.z = valid ? rw.z : 0;
    const uint32_t kofs = valid ? (uint32_t)kb * 128u : 0u;
    dma4(ra, sink, o.pfa, kofs);
    dma4(rw, sink, o.pfw, kofs);
  };

  // A consumer (second K half of a split tail tile) first waits for its
  // producer's partial: thread 0 polls the flag (bounded) and passes the
  // decision to every wave through LDS.  Giving up leaves everything to the
  // caller, which computes the whole tile.
  bool from_partial = false;
  if (SPLIT && tk.role == 2) {
    int* decision = reinterpret_cast<int*>(smem + T::XCH_OFF);
    if (threadIdx.x == 0) {
      const uint64_t pub = flag_word(tk.tag, kPublished);
      bool seen = flag_load(tk.flags) == pub;
      for (int n = 0; !seen && n < p.wait_limit; ++n) {
        __builtin_amdgcn_s_sleep(2);
        seen = flag_load(tk.flags) == pub;
      }
      if (!seen) {
        flag_store(tk.flags + 1, flag_word(tk.tag, kGaveUp));
        wait_vmcnt<0>();
        seen = flag_load(tk.flags) == pub;
        if (seen) flag_store(tk.flags + 1, 0);
      }
      if (seen) flag_store(tk.flags, 0);
      flag_store(tk.flags + 2, flag_word(tk.tag, seen ? kConsumed : kGaveUp));
      *decision = seen ? 1 : 0;
    }
    __syncthreads();
    if (*decision == 0) {
      // this half's first K block was issued early into stage 0: let it land
      // before the whole tile refills that stage
      wait_vmcnt<0>();
      return true;
    }
    from_partial = true;
  }

  // acc[i][j]: output rows m0 + wm*WTM + 16i + lane%16, columns
  // n0 + wn*WTN + 16j + 4*(lane/16) + r (r = 0..3).  A consumer starts from
  // the producer's accumulators (read past the caches; they were written
  // through to memory).  Partial layout: float4 ((wave * TM + i) * TN + j) *
  // 64 + lane, i.e. every store and load of a wave is 1 KB contiguous.
  v4f acc[TM][TN];
  if (SPLIT && from_partial) {
    const int vo = (wave * TM * TN * 64 + lane) * 16;
    const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(tk.part, 0, T::BM * T::BN * 4, 0x00020000);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_bit_cast(v4f, __builtin_amdgcn_raw_buffer_load_b128(rl, vo, (i * TN + j) * 1024,
                                                                                 kCacheSystem));
    // wait for them here, with a wait the compiler sees (vmcnt 0; expcnt and
    // lgkmcnt unconstrained): it then places no wait for them inside the K
    // loop, which would drain the operand loads of every block.  (The first
    // wait below would wait for them anyway: they follow this tile's first
    // block's loads.)
    __builtin_amdgcn_s_waitcnt(0x0F70);
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
  }

  // n consecutive scale words from LDS: 16-byte reads where n is a multiple
  // of 4 (the run then starts 16-byte aligned), else 8-byte reads where n is
  // even, else single words
  auto read_words = [&](const uint32_t* src, uint32_t* dst, auto NN) {
    constexpr int n = decltype(NN)::value;
    if constexpr (n % 4 == 0) {
#pragma unroll
      for (int i = 0; i < n; i += 4) {
        const uint4 s4 = *reinterpret_cast<const uint4*>(src + i);
        dst[i] = s4.x; dst[i + 1] = s4.y; dst[i + 2] = s4.z; dst[i + 3] = s4.w;
      }
    } else if constexpr (n % 2 == 0) {
#pragma unroll
      for (int i = 0; i < n; i += 2) {
        const uint2 s2 = *reinterpret_cast<const uint2*>(src + i);
        dst[i] = s2.x; dst[i + 1] = s2.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < n; ++i) dst[i] = src[i];
    }
  };

  auto read_frag = [&](const uint8_t* base, int row) {
    Frag f;
    f.u[0] = *reinterpret_cast<const uint4*>(base + swz(row, lq));
    f.u[1] = *reinterpret_cast<const uint4*>(base + swz(row, lq + 4));
    return f;
  };

  // Block mode rescale, software-pipelined: the MFMAs of 16-row tile i give
  // P (fp32 partial products of this K block); P is folded into the
  // accumulators (acc += P * s_a * s_w, one scale per lane) while the MFMAs
  // of tile i + 1 run.  The last tile's P is folded during the first tile of
  // the next K block (or before the epilogue).
  v4f Pq[TN];
  float cq = 0.f;
#pragma unroll
  for (int j = 0; j < TN; ++j) Pq[j] = v4f{0.f, 0.f, 0.f, 0.f};
  auto fold_one = [&](auto I, int j) {
    constexpr int i = decltype(I)::value;
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(Pq[j][r], cq, acc[i][j][r]);
  };

  const int arow = wm * WTM + l16;            // fragment row of 16-row tile 0
  const int brow = wn * WTN + l16;

  // Operands carried from one K block to the next: the weight fragments, the
  // first LA activation fragments and the scales of the block about to be
  // multiplied are read from LDS while the previous block's last MFMAs run.
  // Activation fragments live in a ring of LA + 1 registers sets: the one of
  // 16-row tile i is read LA tiles before its MFMAs.
  constexpr int LA = TM > FP8Q_A_LOOKAHEAD ? FP8Q_A_LOOKAHEAD : TM - 1 > 0 ? TM - 1 : 1;
  static_assert(LA >= 1 && LA < TM, "activation fragment lookahead");
  Frag fb[TN], fr[LA + 1];
  uint32_t sav[TM] = {}, swb[TN] = {};    // activation / weight scale words
  float swv = 0.f;                        // block mode: this wave's weight scale
  int swe = 127;                          // power-of-two view: its exponent byte
  // the weight fragments and the scales of the block in stage st
  auto read_w = [&](int st) {
    const uint8_t* a = smem + st * STAGE;
    const uint8_t* w = a + ABYTES;
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[j] = read_frag(w, brow + 16 * j);
    if constexpr (MXC) {
      // [sub-block][row] bytes: this lane's sub-block lq, its rows
#pragma unroll
      for (int i = 0; i < TM; ++i) sav[i] = a[SA_OFF + lq * BM + arow + 16 * i];
#pragma unroll
      for (int j = 0; j < TN; ++j) swb[j] = a[SW_OFF + lq * BN + brow + 16 * j];
    } else if constexpr (MODE == MODE_MX) {
      read_words(reinterpret_cast<const uint32_t*>(a + SA_OFF) + wm * WTM + l16 * TM, sav,
                 std::integral_constant<int, TM>{});
      read_words(reinterpret_cast<const uint32_t*>(a + SW_OFF) + wn * WTN + l16 * TN, swb,
                 std::integral_constant<int, TN>{});
    } else if constexpr (MODE != MODE_TENSOR) {
      read_words(reinterpret_cast<const uint32_t*>(a + SA_OFF) + wm * WTM + l16 * TM, sav,
                 std::integral_constant<int, TM>{});
    }
    if constexpr (MODE == MODE_BLOCK)
      swv = __uint_as_float(reinterpret_cast<const uint32_t*>(a + SW_OFF)[wn]);
    if constexpr (MODE == MODE_BMX)
      swe = (int)((reinterpret_cast<const uint32_t*>(a + SW_OFF)[wn] >> 23) & 0xFFu);
  };
  auto load_regs = [&](int st) {
    read_w(st);
    const uint8_t* a = smem + st * STAGE;
#pragma unroll
    for (int i = 0; i < LA; ++i) fr[i] = read_frag(a, arow + 16 * i);
  };

  // The MFMAs (and block-mode folds) of 16-row tile i of the block in stage
  // st; the activation fragment of tile i + LA is read meanwhile.
  auto mfma_tile = [&](auto I, const Frag& fa) {
    constexpr int i = decltype(I)::value;
    if constexpr (MODE == MODE_BLOCK) {
      // fold column tile j of the previous 16-row tile (its MFMA was issued
      // TN MFMAs ago), then reuse its registers for this tile's product
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        fold_one(std::integral_constant<int, (i == 0 ? TM - 1 : i - 1)>{}, j);
        Pq[j] = mfma_plain(fb[j].v, fa.v, v4f{0.f, 0.f, 0.f, 0.f});
        // keep this order of FMAs and MFMAs (only LDS reads and scalar
        // instructions may move across): the scheduler would otherwise
        // hoist folds next to the MFMAs whose results they read
        __builtin_amdgcn_sched_barrier(0x0104);
      }
      cq = __uint_as_float(sav[i]) * swv;
    } else if constexpr (MODE == MODE_TENSOR) {
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma_plain(fb[j].v, fa.v, acc[i][j]);
    } else if constexpr (MODE == MODE_BMX) {
      // power-of-two fp32 scales: the exponent field is the UE8M0 byte the
      // scaled MFMA applies to all four 32-wide parts of the 128-wide block,
      // so the rescale happens inside the MFMA and the accumulators carry
      // across K blocks
      const int sab = (int)((sav[i] >> 23) & 0xFFu);
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mfma_mx(fb[j].v, fa.v, acc[i][j], swe, sab);
    } else {
      // scale byte of this lane's 32-wide K block (lane / 16): in each word
      // (row-major scales) or already the byte (column-major)
      const int sh = MXC ? 0 : 8 * lq;
      const int sab = (int)((sav[i] >> sh) & 0xFF);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = mfma_mx(fb[j].v, fa.v, acc[i][j], (int)((swb[j] >> sh) & 0xFF), sab);
    }
  };
  auto tile = [&](auto I, int st) {
    constexpr int i = decltype(I)::value;
    const uint8_t* a = smem + st * STAGE;
    if constexpr (i + LA < TM) fr[(i + LA) % (LA + 1)] = read_frag(a, arow + 16 * (i + LA));
    mfma_tile(I, fr[i % (LA + 1)]);
  };

  // Main loop.  Block kb sits in stage kb % 2 and block kb + 1 is being
  // loaded into the other stage.  Once this wave has issued its last LDS
  // read of block kb (the fragment of the last 16-row tile), it waits for its
  // own loads of block kb + 1 and meets the other waves at the barrier: after
  // it, block kb + 1 is complete in LDS and nobody reads stage kb % 2 any
  // more, which is refilled with block kb + 2.  The last LA tiles' MFMAs then
  // overlap the reads of block kb + 1's first operands.  The two prefetch
  // touches issued after a block's loads are the only loads issued after
  // them, hence the wait for at most 2 loads in flight.  (SLOTS - 1 < TM - LA:
  // every slot of block kb + 1 is issued before that barrier.)
  static_assert(T::NS == 2, "the wait count below assumes two stages");
  // The loads of a block are spread over SLOTS issue points: slot 0 right
  // after the barrier that frees their stage, slot s >= 1 before 16-row tile
  // s - 1 of the next block, so that the vector-memory queue never receives
  // a whole block's loads at once (a full queue stalls the issuing wave and
  // with it its MFMAs).  The prefetch touches follow the last slot.
  constexpr int SLOTS = 1 + (TM - LA - 1 < FP8Q_LOAD_SLOTS ? TM - LA - 1 : FP8Q_LOAD_SLOTS);
  constexpr int PER = (NLD + SLOTS - 1) / SLOTS;
  auto issue_slot = [&](auto S, int st, int kb) {
    constexpr int sl = decltype(S)::value;
    static_for<NLD>([&](auto L) {
      if constexpr (decltype(L)::value / PER == sl) issue_load(L, st, kb, cur);
    });
    if constexpr (sl == SLOTS - 1) prefetch(kb + PFD - 1, cur);
  };
  auto issue_all = [&](int st, int kb, const Offs& o) {
    static_for<NLD>([&](auto L) { issue_load(L, st, kb, o); });
    prefetch(kb + PFD - 1, o);
  };
  const int kb0 = tk.kb0;
  if (preloaded) {
    // block kb0 was issued before the previous tile's output stores: wait
    // for everything (the stores have had the loads' latency to drain)
    wait_vmcnt_barrier<0>();
  } else {
    issue_all(0, kb0, cur);
    wait_vmcnt_barrier<2>();
  }
  // Every wave's stores of the previous item (a producer's partial, issued
  // before this tile's loads) have completed: publish it.
  if (SPLIT && tk.publish != nullptr && threadIdx.x == 0) {
    // a bounded delay before publishing, only when the launch plan asks for
    // one (tests of the give-up path)
    for (int n = 0; n < p.publish_delay; ++n) __builtin_amdgcn_s_sleep(127);
    flag_store(tk.publish, flag_word(p.tag, kPublished));
  }
  static_for<SLOTS>([&](auto S) { if constexpr (decltype(S)::value == 0) issue_slot(S, 1, kb0 + 1); });
  load_regs(0);
  for (int kb = kb0; kb < KB; ++kb) {
    const int st = (kb - kb0) & 1;
    static_for<TM>([&](auto I) {
      constexpr int i = decltype(I)::value;
      // the rest of block kb + 1's loads (its slot 0 was issued at the
      // previous barrier)
      if constexpr (i + 1 < SLOTS) issue_slot(std::integral_constant<int, i + 1>{}, st ^ 1, kb + 1);
      if constexpr (i == TM - LA) {
        wait_vmcnt_barrier<2>();
        issue_slot(std::integral_constant<int, 0>{}, st, kb + 2);
      }
      tile(I, st);
    });
    // keep the next block's reads behind the last tile's MFMAs, which still
    // read the weight fragments being replaced.  After the last block this
    // reads a stale stage (possibly while the next tile's first loads land
    // in it): harmless, the values are never used, and reading
    // unconditionally keeps the old and new fragments from being live at once.
    __builtin_amdgcn_sched_barrier(0);
    load_regs(st ^ 1);
  }
  // After the last barrier of the K loop no wave reads a stage any more:
  // start the next tile's first K block now.
  if (has_next) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    issue_all(0, tk.next_kb0, make_offs(nm0, nn0, ngm, ngn, ln));
  }
  if constexpr (MODE == MODE_BLOCK) {
#pragma unroll
    for (int j = 0; j < TN; ++j) fold_one(std::integral_constant<int, TM - 1>{}, j);
  }

  // A producer's K half ends here: its accumulators go to the pair's
  // partial slot, written through to memory (system-scope cache policy), so
  // that the consumer, on another XCD whose L2 is not coherent with this
  // one, reads them past its caches without an L2 write-back.  The stores
  // are not waited for here: the next tile's first wait covers them, and
  // the flag is raised after it (TileK::publish).
  // (SPLIT: only the kernel that may split its tail carries this code, so
  // the others keep their registers.)
  if (SPLIT && tk.role == 1) {
    const int vo = (wave * TM * TN * 64 + lane) * 16;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(tk.part, 0, T::BM * T::BN * 4, 0x00020000);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), rs, vo, (i * TN + j) * 1024,
                                               kCacheSystem);
    return false;
  }
  const int m_end = p.m_end;

  // Epilogue.  After the MFMAs, lane (r16, q) = (lane % 16, lane / 16) holds
  // for column tile j the four columns 16j + 4q + 0..3 of row r16 (+16i).
  // The four lanes of a row exchange their bf16 pairs with two rounds of
  // lane swaps (a 4 x 4 transpose over q and j), after which lane (r16, q)
  // holds the sixteen contiguous columns 16q .. 16q + 15 and writes them as
  // two 16-byte stores: half as many store instructions, each carrying
  // 16-byte runs, as storing the MFMA layout directly.
  static_assert(TN == 4, "the epilogue transpose is 4 x 4");
  float mul = 1.0f;
  if (MODE == MODE_TENSOR)
    mul = static_cast<const float*>(p.sa)[0] * static_cast<const float*>(p.sw)[0];
  float bias[TN][4];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int col = n0 + wn * WTN + 16 * j + 4 * lq + r;
      bias[j][r] = (p.bias != nullptr && col < p.N) ? __uint_as_float((uint32_t)p.bias[col] << 16) : 0.0f;
    }
  const int col0 = n0 + wn * WTN + 16 * lq;           // this lane's columns after the exchange
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    // D[j][h]: bf16 pair h (columns 16j + 4q + 2h, +1) of column tile j
    uint32_t d[TN][2];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = acc[i][j][r];
        if (MODE == MODE_TENSOR) v[r] = v[r] * mul;
        v[r] = v[r] + bias[j][r];
      }
      d[j][0] = pack_bf16x2(v[0], v[1]);
      d[j][1] = pack_bf16x2(v[2], v[3]);
    }
    // round 1 swaps lane halves (q 0,1 <-> q 2,3) between tiles j and j + 2,
    // round 2 swaps lane quarters (q 1 <-> q 0, q 3 <-> q 2) between the
    // results: e[x] then holds columns 16q + 4x + 0..3 (x = source lane q)
    uint32_t e[4][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const auto s02 = __builtin_amdgcn_permlane32_swap(d[0][h], d[2][h], false, false);
      const auto s13 = __builtin_amdgcn_permlane32_swap(d[1][h], d[3][h], false, false);
      const auto t01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
      const auto t23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
      e[0][h] = t01[0];
      e[1][h] = t01[1];
      e[2][h] = t23[0];
      e[3][h] = t23[1];
    }
    const int row = m0 + wm * WTM + 16 * i + l16;
    if (row >= m_end) continue;
    uint16_t* yr = p.y + (int64_t)row * p.ldy;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int c = col0 + 8 * half;
      const uint4 o = make_uint4(e[2 * half][0], e[2 * half][1], e[2 * half + 1][0], e[2 * half + 1][1]);
      if (c + 8 <= p.N) {
        *reinterpret_cast<uint4*>(yr + c) = o;
      } else {
        const uint32_t w[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int t = 0; t < 8; ++t)
          if (c + t < p.N) yr[c + t] = (uint16_t)(w[t >> 1] >> ((t & 1) * 16));
      }
    }
  }
  return false;
}

// Work items [0, full) are whole tiles (in XCD-contiguous group order); the
// remaining tiles of that order are split into two half-height tiles, items
// [full, items) -- or, with `ksplit` (a workspace in p.partial), into their
// two K halves: items full + 2t and full + 2t + 1 are the first and second
// K half of leftover tile t, which meet through the pair's partial slot and
// flag words (see TileK).  The kernel is persistent: workgroup g takes
// items g, g + G, g + 2G, ... (G = gridDim.x, at most one workgroup per
// slot), so the workgroups of a round start together and keep their XCD
// (item % 8), and no workgroup is launched per tile.  full is a multiple of
// G and items - full <= G, so a workgroup holds at most one K half; a first
// K half (the producer's) is moved to the front of its workgroup's items and
// a second one stays last, so the partial is written while the consumer
// still works on its whole tiles.  Between two tiles no barrier is needed: a
// wave issues the next tile's first LDS writes only after the last K-loop
// barrier of the previous tile, after which nobody reads a stage, and the
// next tile's first barrier waits for every wave.  A producer never waits,
// so the waits cannot form a cycle; a consumer stops waiting after
// p.wait_limit polls and then computes the whole tile itself.
template <class T, bool KSPLIT>
__global__ __launch_bounds__(T::NW * 64) void gemm_fast_kernel(GemmArgs p, int full, int items) {
  constexpr bool ksplit = KSPLIT;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];
  const int total = p.tiles_m * p.tiles_n;
  const int G = gridDim.x;
  // item -> tile origin and prefetch group coordinates; the kind: 0 whole
  // tile, 1 half-height tile, 2 K half
  auto decode = [&](int x, int& m0, int& n0, int& gm, int& gn) {
    int tm, tn, kind = 0;
    if (x < full) {
      group_walk(xcd_contiguous(x, full), p.tiles_m, p.tiles_n, tm, tn);
      m0 = tm * T::BM;
    } else if (ksplit) {
      group_walk(full + ((x - full) >> 1), p.tiles_m, p.tiles_n, tm, tn);
      m0 = tm * T::BM;
      kind = 2;
    } else {
      const int h = xcd_contiguous(x - full, 2 * (total - full));
      group_walk(full + (h >> 1), p.tiles_m, p.tiles_n, tm, tn);
      m0 = tm * T::BM + (h & 1) * (T::BM / 2);
      kind = 1;
    }
    n0 = tn * T::BN;
    gm = tm % 8;
    gn = tn % T::NTN;
    return kind;
  };
  const int g = blockIdx.x;
  const int half_kb = p.KB / 2;
  const int tails = (items - full) / 2;
  // this workgroup's items in order: g, g + G, ... (< items), except that a
  // first K half (full + g, the last of them) is moved to the front
  const bool front = ksplit && g < items - full && (g & 1) == 0;
  auto next_item = [&](int x) {
    if (front && x == full + g) return g;
    const int y = x + G;
    return (y >= items || (front && y == full + g)) ? -1 : y;
  };
  bool preloaded = false;
  uint64_t* publish = nullptr;         // flag words of a partial stored by the previous item
  uint64_t* produced = nullptr;        // flag words of this workgroup's K half as producer
  int redo_m0 = -1, redo_n0 = 0, redo_gm = 0, redo_gn = 0;
  for (int b = g >= items ? -1 : (front ? full + g : g); b >= 0; b = next_item(b)) {
    int m0, n0, gm, gn, nm0 = 0, nn0 = 0, ngm = 0, ngn = 0;
    const int kind = decode(b, m0, n0, gm, gn);
    const int nb = next_item(b);
    // the next tile's first block is issued early between tiles of one
    // kind, and between a whole tile and a K half either way (at that
    // tile's first block)
    const int nkind = nb >= 0 ? decode(nb, nm0, nn0, ngm, ngn) : -1;
    const bool has_next = nkind >= 0 && (nkind == kind || (kind == 0 && nkind == 2) || (kind == 2 && nkind == 0));
    TileK tk{0, p.KB, 0, 0, nullptr, nullptr, p.tag, publish};
    if (nkind == 2) tk.next_kb0 = ((nb - full) & 1) ? half_kb : 0;
    if (kind == 2) {
      const int t = (b - full) >> 1, second = (b - full) & 1;
      tk.kb0 = second ? half_kb : 0;
      tk.kb1 = second ? p.KB : half_kb;
      tk.role = second ? 2 : 1;
      tk.part = p.partial + (int64_t)t * (T::BM * T::BN);
      tk.flags = reinterpret_cast<uint64_t*>(p.partial + (int64_t)tails * (T::BM * T::BN)) + 3 * t;
    }
    bool redo;
    if (kind == 1)
      redo = fast_tile<T, 2, KSPLIT>(p, smem, m0, n0, gm, gn, preloaded, has_next, nm0, nn0, ngm, ngn, tk);
    else
      redo = fast_tile<T, 4, KSPLIT>(p, smem, m0, n0, gm, gn, preloaded, has_next, nm0, nn0, ngm, ngn, tk);
    if (KSPLIT && redo) {
      redo_m0 = m0; redo_n0 = n0; redo_gm = gm; redo_gn = gn;
    }
    publish = nullptr;
    if (KSPLIT && tk.role == 1) publish = produced = tk.flags;
    preloaded = has_next;
  }
  if (KSPLIT && publish != nullptr) {
    // a producer's K half with no tile after it: wait for its stores here
    wait_vmcnt_barrier<0>();
    if (threadIdx.x == 0) flag_store(publish, flag_word(p.tag, kPublished));
  }
  if (KSPLIT && redo_m0 >= 0) {
    // the partner's half did not appear in time: the whole tile here (a K
    // half is its workgroup's last item, so nothing was issued early and
    // nothing follows)
    const TileK whole{0, p.KB, 0, 0, nullptr, nullptr, p.tag, nullptr};   // role 0: a whole tile
    fast_tile<T, 4, false>(p, smem, redo_m0, redo_n0, redo_gm, redo_gn, false, false, 0, 0, 0, 0, whole);
  }
  if (KSPLIT && produced != nullptr && threadIdx.x == 0) {
    // the producer's read of the consumer's flag, after its own flag store
    // has completed
    wait_vmcnt<0>();
    if (flag_load(produced + 1) == flag_word(p.tag, kGaveUp)) {
      flag_store(produced, 0);
      flag_store(produced + 1, 0);
    }
  }
  // the last touches and past-the-end loads still write the LDS sink: let
  // them land before the workgroup ends
  wait_vmcnt<0>();
}

// Grouped GEMM over expert-sorted rows (MoE experts): rows offsets[e] ..
// offsets[e+1] of A multiply expert e's weight w + e * w_stride with its
// scales sw + e * sw_stride.  Items are the tiles of every expert, expert
// after expert (an expert's tiles in group_walk order), counted on the device
// from the offsets: each workgroup sums the per-expert tile counts in LDS
// (a scan) and finds an item's expert by binary search.  Offsets are clamped
// to [0, M] and made non-decreasing, so any offsets keep every access inside
// the operands (outputs are then unspecified).  A tile's rows past its
// expert's end are computed from the next expert's rows and not stored.  The
// next tile's first K block is issued early only when it belongs to the same
// expert (its weight descriptor is the same).
struct GroupArgs {
  const int32_t* offsets;   // [E + 1]
  int E;
  int64_t w_stride;         // bytes between experts' weights
  int64_t sw_stride;        // scale words between experts' scale grids
};

constexpr int kMaxExperts = 1024;

template <class T>
__global__ __launch_bounds__(T::NW * 64) void gemm_grouped_kernel(GemmArgs p, GroupArgs g) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem[T::LDS_BYTES];
  __shared__ int tiles_before[kMaxExperts];    // inclusive scan of per-expert tile counts
  constexpr int NT = T::NW * 64, PER = (kMaxExperts + NT - 1) / NT;
  const int E = g.E;
  // expert e's rows [row_begin(e), row_end(e)), clamped into [0, M]; e may
  // differ between lanes (the counting loop below), so nothing here assumes
  // a wave-uniform e
  auto clampM = [&](int o) { return o < 0 ? 0 : (o > p.M ? p.M : o); };
  auto row_begin = [&](int e) { return clampM(g.offsets[e]); };
  auto row_end = [&](int e) {
    const int b = clampM(g.offsets[e]), x = clampM(g.offsets[e + 1]);
    return x < b ? b : x;
  };
  for (int t = threadIdx.x; t < E; t += NT)
    tiles_before[t] = (row_end(t) - row_begin(t) + T::BM - 1) / T::BM * p.tiles_n;
  __syncthreads();
  for (int d = 1; d < E; d <<= 1) {
    int v[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int t = threadIdx.x + i * NT;
      v[i] = (t < E && t >= d) ? tiles_before[t - d] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int t = threadIdx.x + i * NT;
      if (t < E) tiles_before[t] += v[i];
    }
    __syncthreads();
  }
  const int items = __builtin_amdgcn_readfirstlane(tiles_before[E - 1]);
  // item -> expert (first e with tiles_before[e] > x), tile origin, and the
  // tile's height in quarters of BM: an expert's last row tile holding at
  // most BM/2 (3BM/4) rows computes only that many (and loads only those
  // activation rows)
  auto decode = [&](int x, int& e, int& m0, int& n0, int& gm, int& gn) {
    // branch-free binary search (straight-line code: a loop here made the
    // register allocator spill around the tile bodies); e = the number of
    // experts whose inclusive count is <= x
    int lo = 0;
#pragma unroll
    for (int step = kMaxExperts / 2; step > 0; step >>= 1) {
      const int c = lo + step;
      const int v = __builtin_amdgcn_readfirstlane(tiles_before[c <= E ? c - 1 : 0]);
      lo = (c <= E && v <= x) ? c : lo;
    }
    e = lo;
    const int li = x - (e ? __builtin_amdgcn_readfirstlane(tiles_before[e - 1]) : 0);
    // x is wave-uniform, hence e: its rows are made uniform (SGPRs)
    const int r0 = __builtin_amdgcn_readfirstlane(row_begin(e));
    const int cnt = __builtin_amdgcn_readfirstlane(row_end(e)) - r0;
    const int tiles_m = (cnt + T::BM - 1) / T::BM;
    int tm, tn;
    group_walk(li, tiles_m, p.tiles_n, tm, tn);
    m0 = r0 + tm * T::BM;
    n0 = tn * T::BN;
    gm = tm % 8;
    gn = tn % T::NTN;
    const int left = cnt - tm * T::BM;
    return left <= T::BM / 2 ? 2 : left <= 3 * T::BM / 4 ? 3 : 4;
  };
  bool preloaded = false;
  // the next item's decode is carried into the next iteration
  int e = 0, m0 = 0, n0 = 0, gm = 0, gn = 0;
  int rq = 4;
  if ((int)blockIdx.x < items) rq = decode(blockIdx.x, e, m0, n0, gm, gn);
  for (int b = blockIdx.x; b < items; b += gridDim.x) {
    int ne = -1, nm0 = 0, nn0 = 0, ngm = 0, ngn = 0;
    const int nb = b + gridDim.x;
    int nrq = 4;
    if (nb < items) nrq = decode(nb, ne, nm0, nn0, ngm, ngn);
    const bool has_next = ne == e && nrq == rq;
    GemmArgs pe = p;
    pe.w = p.w + e * g.w_stride;
    pe.sw = static_cast<const float*>(p.sw) + e * g.sw_stride;
    pe.m_end = __builtin_amdgcn_readfirstlane(row_end(e));
    const TileK tk{0, p.KB, 0, 0, nullptr, nullptr, 0u, nullptr};
    if (rq == 2)
      fast_tile<T, 2, false, true>(pe, smem, m0, n0, gm, gn, preloaded, has_next, nm0, nn0, ngm, ngn, tk);
    else if (rq == 3)
      fast_tile<T, 3, false, true>(pe, smem, m0, n0, gm, gn, preloaded, has_next, nm0, nn0, ngm, ngn, tk);
    else
      fast_tile<T, 4, false, true>(pe, smem, m0, n0, gm, gn, preloaded, has_next, nm0, nn0, ngm, ngn, tk);
    preloaded = has_next;
    e = ne; m0 = nm0; n0 = nn0; gm = ngm; gn = ngn; rq = nrq;
  }
  wait_vmcnt<0>();
}

namespace {

// Configuration 0: 256 x 256 tiles, 8 waves, one workgroup per CU.
// Configuration 1: 128 x 128 tiles, 4 waves, two workgroups per CU.
// plan_override() (fp8q_set_plan_override) may force a configuration,
// disable the tail balancing, or plan for another CU count.
int cu_count() {
  const int forced = plan_override().gemm_slots;
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
  const PlanOverride ov = plan_override();
  const int forced = ov.gemm_cfg;
  const bool split = ov.gemm_split != 0;
  const int cus = cu_count();
  const Plan big = plan_cfg(p, 0, cus, split), small = plan_cfg(p, 1, 2 * cus, split);
  if (forced == 0) return big;
  if (forced == 1) return small;
  return plan_cost(big, cus) <= plan_cost(small, cus) ? big : small;
}

// Workspace of the split tail (configuration 0 only): 256 x 256 fp32 per
// leftover tile, then three 8-byte words each (two flags, the outcome); 0
// when the plan has no tail, or when K is below 32 blocks: for a short K
// loop the exchange of a 256 KB partial costs about what the split saves.
size_t tail_workspace(const Plan& pl, const GemmArgs& p) {
  const int tail = pl.tiles_m * pl.tiles_n - pl.full;
  if (pl.cfg != 0 || tail <= 0 || p.KB < 32) return 0;
  return (size_t)tail * (256u * 256u * 4u + 24u);
}

std::atomic<uint32_t> g_tag{0};

template <int MODE>
void launch_plan(GemmArgs p, const Plan& pl, hipStream_t stream) {
  p.tiles_m = pl.tiles_m;
  p.tiles_n = pl.tiles_n;
  // persistent grid: one workgroup per slot (configuration 0 holds one
  // workgroup per CU, configuration 1 two), never more than the items
  const int slots = (pl.cfg == 0 ? 1 : 2) * cu_count();
  const int grid = pl.grid < slots ? pl.grid : slots;
  // with a workspace, the leftover tiles are split along K instead of in
  // half-height tiles; a fresh tag per launch marks its exchange words
  const int ksplit = p.partial != nullptr && tail_workspace(pl, p) > 0;
  if (ksplit) {
    uint32_t n = ++g_tag;
    if (n == 0) n = ++g_tag;
    p.tag = n;
    const PlanOverride ov = plan_override();
    p.wait_limit = ov.split_wait_limit >= 0 ? ov.split_wait_limit : (1 << 22);
    p.publish_delay = ov.split_publish_delay;
  }
  if (pl.cfg == 0) {
    using T = FastTile<MODE, 256, 256, 2, 4, 4>;
    if (ksplit)
      hipLaunchKernelGGL((gemm_fast_kernel<T, true>), dim3(grid), dim3(T::NW * 64), 0, stream, p, pl.full, pl.grid);
    else
      hipLaunchKernelGGL((gemm_fast_kernel<T, false>), dim3(grid), dim3(T::NW * 64), 0, stream, p, pl.full, pl.grid);
  } else {
    using T = FastTile<MODE, 128, 128, 2, 2, 8>;
    hipLaunchKernelGGL((gemm_fast_kernel<T, false>), dim3(grid), dim3(T::NW * 64), 0, stream, p, pl.full, pl.grid);
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

bool gemm_grouped_eligible(const GemmArgs& p, int E, int64_t w_stride) {
  const int64_t lim = (int64_t(1) << 31) - 1;
  return E >= 1 && E <= kMaxExperts && p.K % 128 == 0 && (int64_t)(p.M + 256) * p.lda < lim &&
         (int64_t)p.N * p.ldw + 256 * p.ldw < lim && (int64_t)(p.M + 256) * p.KB * 4 < lim &&
         (int64_t)(p.NB + 2) * p.KB * 4 < lim && (int64_t)(E - 1) * w_stride < (int64_t(1) << 62) &&
         (p.shard == 0 || p.shard % 64 == 0);
}

hipError_t launch_gemm_grouped(GemmArgs p, const int32_t* offsets, int E, int64_t w_stride, int mode,
                               hipStream_t stream) {
  // Tiles of 256 rows unless experts average fewer than 112 rows: an expert
  // of c rows takes ceil(c/256) tiles of 256 or ceil(c/128) of 128, and just
  // above 128 rows the second 128-row tile is nearly empty yet re-reads the
  // expert's whole weight (measured: 291 against 333 us at 129 rows).
  const int forced = plan_override().gemm_cfg;
  const int cfg = forced >= 0 ? forced : ((int64_t)p.M >= 112 * (int64_t)E ? 0 : 1);
  const int bm = cfg == 0 ? 256 : 128;
  p.tiles_n = (p.N + bm - 1) / bm;
  p.tiles_m = 0;
  const GroupArgs g{offsets, E, w_stride, (int64_t)p.NB * p.KB};
  // persistent: one workgroup per slot; the item count is known on the device only
  const int grid = (cfg == 0 ? 1 : 2) * cu_count();
#define FP8Q_GROUPED(MODEV)                                                                           \
  do {                                                                                                \
    if (cfg == 0) {                                                                                   \
      using T = FastTile<MODEV, 256, 256, 2, 4, 4>;                                                   \
      hipLaunchKernelGGL(gemm_grouped_kernel<T>, dim3(grid), dim3(T::NW * 64), 0, stream, p, g);      \
    } else {                                                                                          \
      using T = FastTile<MODEV, 128, 128, 2, 2, 8>;                                                   \
      hipLaunchKernelGGL(gemm_grouped_kernel<T>, dim3(grid), dim3(T::NW * 64), 0, stream, p, g);      \
    }                                                                                                 \
  } while (0)
  if (mode == MODE_BMX) FP8Q_GROUPED(MODE_BMX);
  else FP8Q_GROUPED(MODE_BLOCK);
#undef FP8Q_GROUPED
  return hipGetLastError();
}

size_t gemm_fast_tail_workspace(const GemmArgs& p) { return tail_workspace(choose_plan(p), p); }

hipError_t launch_gemm_fast(GemmArgs p, int mode, hipStream_t stream) {
  const Plan pl = choose_plan(p);
  if (mode == MODE_BLOCK) launch_plan<MODE_BLOCK>(p, pl, stream);
  else if (mode == MODE_TENSOR) launch_plan<MODE_TENSOR>(p, pl, stream);
  else if (mode == MODE_BMX) launch_plan<MODE_BMX>(p, pl, stream);
  else if (mode == MODE_MXC) launch_plan<MODE_MXC>(p, pl, stream);
  else launch_plan<MODE_MX>(p, pl, stream);
  return hipGetLastError();
}

}  // namespace fp8q
