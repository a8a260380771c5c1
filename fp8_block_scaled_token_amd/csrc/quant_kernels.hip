// Quantizer kernels of the FP8 blockwise linear layer (gfx950).
//
//  * quant_group128   dynamic per-token-group activation quantizer, fp32 scale
//                     per 128 channels ([GLM17] "第 1 站:RMSNorm 的两个出口";
//                     [SGL19] "Triton 分块内核在做什么").
//  * quant_group32mx  MXFP8 1x32 blocks with UE8M0 scale bytes ([SGLFP8]
//                     "4. 블록 양자화 스케일 관리"; round-up exponent of [GLM17]
//                     "第 4 站:索引器——FP8 与排名稳定性").
//  * quant_static     per-tensor static scale ([SGL19] "激活量化的三种选择").
//  * rmsnorm_quant    RMSNorm -> bf16 -> group-128 quantizer in one pass,
//                     optionally preceded by the residual add and with the
//                     static per-tensor exit instead of group scales ([GLM17]
//                     "第 1 站:RMSNorm 的两个出口").
//  * weight_block     128x128 weight blocks and the per-tensor weight scale
//                     ([SGL19] "建权重:先决定 scale 的形状", "从浮点到 FP8 的基本公式").
//
// Page titles: [SGL19] "SGLang 源码完全拆解(十九):量化方法的注册与层分派",
// [SGLFP8] "[SGLang] FP8", [GLM17] "GLM-5.3 推理全链路(十七):精度账本".
//
// Work layout of the row quantizers: one 64-lane wave owns a segment of
// 512*CH consecutive elements of one row.  Load c of lane l covers the 8
// elements [seg0 + 512c + 8l, +8): every load instruction of the wave reads one
// contiguous kilobyte, and the 16 lanes of a DPP row hold exactly one
// 128-element group (4 lanes hold one 32-element MX block), so group maxima
// are DPP reductions that leave the maximum in every lane of the row.  Every
// lane then computes the scale s and its reciprocal r of its own groups
// itself, without a division and without a lane exchange (group_scales: a
// product refined by its exact FMA residual, and the hardware reciprocal
// refined by a Newton step, both equal to the IEEE quotients), and lane l
// stores the scale of chunk l % 16 of its DPP row (store_group_scales), so
// the wave's row-major scales go out as one coalesced store.  Segments that
// lie wholly inside the row take an unmasked path; only a row's last segment
// masks.  Quantization is HBM-bound: every lane issues all CH loads first.
#include "device_common.h"
#include "launch.h"

namespace fp8q {

__device__ __forceinline__ float absmax8(const uint4& raw) {
  float v[8];
  unpack8(raw, v);
  float m = fabsf(v[0]);
#pragma unroll
  for (int e = 1; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
  return m;
}

// Group scales of a wave segment.  amax[c] holds, in every lane of 16-lane
// row g, the max of group 4c + g, and every lane computes the scale of that
// group itself, s = fp32(max(amax, 1e-10) / 448), and its reciprocal
// r = fp32(1 / s), without a division or a lane exchange:
//   s0 = RN(a * RN(1/448)), refined by its exact residual a - 448 s0 (FMA);
//   r from the hardware reciprocal of s, refined by one Newton step (FMAs).
// amax is a bf16 value or the floor, a set of ~20600 inputs; a host test runs
// every one of them (with every reciprocal estimate within 2 ulp) and finds
// both results equal to the IEEE quotients.  s_mine: the scale that lane l
// stores, that of chunk l % 16 (lanes with l % 16 < CH; see
// store_group_scales).
template <int CH>
__device__ __forceinline__ void group_scales(const float (&amax)[CH], float (&s)[CH],
                                             float (&r)[CH], float& s_mine) {
  static_assert(CH <= 16, "one lane per group");
  constexpr float kInv448 = 1.0f / kFp8Max;           // RN(1/448), folded at compile time
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const float a = fmaxf(amax[c], kAmaxFloor);
    const float s0 = a * kInv448;
    const float e = __builtin_fmaf(-s0, kFp8Max, a);
    s[c] = __builtin_fmaf(e, kInv448, s0);
    const float r0 = __builtin_amdgcn_rcpf(s[c]);
    const float t = __builtin_fmaf(-s[c], r0, 1.0f);
    r[c] = __builtin_fmaf(r0, t, r0);
    // (selected here, with constant indices, so that s stays in registers)
    if (c == 0 || (int)(threadIdx.x & 15) == c) s_mine = s[c];
  }
}

// Codes of 8 values with a scale derived from their group's (or block's, or
// tensor's) maximum: |x| <= amax and s = RN(max(amax, 1e-10)/448) >=
// (amax/448)(1 - 2^-24), so |x/s| <= 448 (1 + 2^-23) < 464.  The hardware
// conversion rounds every magnitude up to 464 to nearest-even E4M3 and so
// maps (448, 464) to 448 itself (measured on gfx950): the saturating clamp of
// the quantization formula is implied and not executed here.  (Static scales,
// which bound nothing, clamp explicitly.)
__device__ __forceinline__ uint2 quant8(const uint4& raw, float s, float r) {
  float v[8], t[8];
  unpack8(raw, v);
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = div_by_scale(v[e], s, r);
  return encode8(t);
}

// Scale byte e + 127 for a block max a (>= 1e-10, a normal fp32 number
// m * 2^E, 1 <= m < 2): 448 = 1.75 * 2^8, so the smallest e with a <= 448*2^e
// is E - 8 when m <= 1.75 and E - 7 otherwise.
__device__ __forceinline__ uint32_t ue8m0_byte(float amax) {
  const uint32_t b = __float_as_uint(fmaxf(amax, kAmaxFloor));
  const uint32_t biased = b >> 23;            // E + 127 (a > 0, normal)
  const uint32_t man = b & 0x7FFFFFu;
  return biased - 8u + (man > 0x600000u ? 1u : 0u);
}

// x * 2^-e is exact and |x| <= amax <= 448 * 2^e, so no clamp is needed.
__device__ __forceinline__ uint2 quant8_mx(const uint4& raw, uint32_t byte) {
  // 2^-e = 2^(127 - byte) as an fp32 bit pattern (byte <= 253 for bf16 input)
  const float inv = __uint_as_float((254u - byte) << 23);
  float v[8], t[8];
  unpack8(raw, v);
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = v[e] * inv;
  return encode8(t);
}

// Power-of-two group scales (the MX exponent rule on 128-wide groups):
// amax[c] as in group_scales; byte[c] is the UE8M0 byte of this lane's group
// in chunk c, s_mine the fp32 scale 2^(byte-127) that lane l stores (chunk
// l % 16, as in group_scales).
template <int CH>
__device__ __forceinline__ void pow2_group_scales(const float (&amax)[CH], uint32_t (&byte)[CH], float& s_mine) {
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    byte[c] = ue8m0_byte(amax[c]);
    if (c == 0 || (int)(threadIdx.x & 15) == c) s_mine = __uint_as_float(byte[c] << 23);
  }
}

// Store the wave's group scales: lane l with c = l % 16 < CH holds the scale
// of group first_group + 4c + l / 16 (chunk c, 16-lane row l / 16).
template <int CH>
__device__ __forceinline__ void store_group_scales(float* scales, float s_mine, int64_t first_group,
                                                   int64_t G, int64_t M, int64_t row, int col_major) {
  const int lane = threadIdx.x & 63, c = lane & 15;
  const int64_t g = first_group + 4 * c + (lane >> 4);
  if (c < CH && g < G) {
    if (col_major) scales[g * M + row] = s_mine;
    else scales[row * G + g] = s_mine;
  }
}

// --------------------------------------------------------------------------
// Group-128 dynamic quantizer (fp32 scales)

// Workgroup b (after XCD-contiguous renumbering) owns rows 4*(b / segs) + wave
// of segment b % segs: each XCD handles a contiguous band of rows.
__device__ __forceinline__ void row_block(int segs, int64_t& row, int64_t& seg) {
  const int b = xcd_contiguous(blockIdx.x, gridDim.x);
  row = (int64_t)(b / segs) * 4 + (threadIdx.x >> 6);
  seg = b % segs;
}

// POW2: scales restricted to powers of two (2^e, e by the MX round-up rule),
// stored as fp32; codes x * 2^-e.
template <int CH, bool POW2>
__global__ __launch_bounds__(256) void quant_group128_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ scales, int col_major, int segs) {
  const int lane = threadIdx.x & 63;
  int64_t row, seg;
  row_block(segs, row, seg);
  if (row >= M) return;
  const int64_t seg0 = seg * (512 * CH);
  const uint16_t* xr = x + row * ldx;
  uint8_t* qr = q + row * ldq;
  const bool full = seg0 + 512 * CH <= K;

  uint4 raw[CH];
  if (full) {
    const uint16_t* xs = xr + seg0 + 8 * lane;
#pragma unroll
    for (int c = 0; c < CH; ++c) raw[c] = ld16_nt(xs + 512 * c);
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t k0 = seg0 + 512 * c + 8 * lane;
      raw[c] = (k0 < K) ? load8_bf16_masked(xr, k0, K) : make_uint4(0, 0, 0, 0);
    }
  }
  float amax[CH], s[CH], r[CH], s_mine;
  uint32_t byte[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) amax[c] = max_row16(absmax8(raw[c]));
  if constexpr (POW2) pow2_group_scales<CH>(amax, byte, s_mine);
  else group_scales<CH>(amax, s, r, s_mine);
  auto codes = [&](int c) { return POW2 ? quant8_mx(raw[c], byte[c]) : quant8(raw[c], s[c], r[c]); };
  if (full) {
    uint8_t* qs = qr + seg0 + 8 * lane;
#pragma unroll
    for (int c = 0; c < CH; ++c) st8(qs + 512 * c, codes(c));
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t k0 = seg0 + 512 * c + 8 * lane;
      const uint2 o = codes(c);
      if (k0 < K) store8_masked(qr, k0, K, o);
    }
  }
  store_group_scales<CH>(scales, s_mine, seg0 / 128, (K + 127) >> 7, M, row, col_major);
}

// --------------------------------------------------------------------------
// MXFP8 1x32 quantizer (UE8M0 scale bytes)

template <int CH>
__global__ __launch_bounds__(256) void quant_group32mx_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
    uint8_t* __restrict__ q, int64_t ldq, uint8_t* __restrict__ scales, int col_major, int segs) {
  const int lane = threadIdx.x & 63;
  int64_t row, seg;
  row_block(segs, row, seg);
  if (row >= M) return;
  const int64_t seg0 = seg * (512 * CH);
  const uint16_t* xr = x + row * ldx;
  uint8_t* qr = q + row * ldq;
  const int64_t G = (K + 31) >> 5;
  const bool full = seg0 + 512 * CH <= K;

  uint4 raw[CH];
  if (full) {
    const uint16_t* xs = xr + seg0 + 8 * lane;
#pragma unroll
    for (int c = 0; c < CH; ++c) raw[c] = ld16_nt(xs + 512 * c);
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t k0 = seg0 + 512 * c + 8 * lane;
      raw[c] = (k0 < K) ? load8_bf16_masked(xr, k0, K) : make_uint4(0, 0, 0, 0);
    }
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t k0 = seg0 + 512 * c + 8 * lane;
    const uint32_t byte = ue8m0_byte(max_quad(absmax8(raw[c])));
    const uint2 o = quant8_mx(raw[c], byte);
    if (full) st8(qr + k0, o);
    else if (k0 < K) store8_masked(qr, k0, K, o);
    const int64_t g = (seg0 + 512 * c) / 32 + (lane >> 2);
    if ((lane & 3) == 0 && g < G) {
      if (col_major) scales[g * M + row] = (uint8_t)byte;
      else scales[row * G + g] = (uint8_t)byte;
    }
  }
}

// --------------------------------------------------------------------------
// Static per-tensor quantizer (any positive scale: IEEE division per element)

template <int CH>
__global__ __launch_bounds__(256) void quant_static_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
    const float* __restrict__ scale, uint8_t* __restrict__ q, int64_t ldq, int segs) {
  const int lane = threadIdx.x & 63;
  int64_t row, seg;
  row_block(segs, row, seg);
  if (row >= M) return;
  const int64_t seg0 = seg * (512 * CH);
  const uint16_t* xr = x + row * ldx;
  uint8_t* qr = q + row * ldq;
  const float s = *scale;
  const bool full = seg0 + 512 * CH <= K;
  uint4 raw[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t k0 = seg0 + 512 * c + 8 * lane;
    raw[c] = full ? ld16_nt(xr + k0) : (k0 < K) ? load8_bf16_masked(xr, k0, K) : make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t k0 = seg0 + 512 * c + 8 * lane;
    float v[8], t[8];
    unpack8(raw[c], v);
#pragma unroll
    for (int e = 0; e < 8; ++e) t[e] = clamp448(v[e] / s);   // IEEE division
    const uint2 o = encode8(t);
    if (full) st8_nt(qr + k0, o);   // streaming store: 3-16 % faster here (measured)
    else if (k0 < K) store8_masked(qr, k0, K, o);
  }
}

// --------------------------------------------------------------------------
// RMSNorm fused with the group-128 quantizer.  A 4-wave workgroup handles a
// row at a time; wave w covers the segment of 512*CH elements starting at
// (4i + w) * 512*CH in pass i.  The per-wave fp64 partial sums of squares
// meet in LDS and are added in wave order (deterministic).
//
// ADD: the row first becomes z = bf16(x + h), which is written to the
// residual output and is what the norm reads.  EXIT: how the normalized row
// is quantized -- group-128 fp32 scales, one fixed per-tensor scale (no
// group scales), or group-128 power-of-two scales.
//
// rmsnorm_quant_rows_kernel (K <= 4 * 512*CH): the workgroup owns a run of
// consecutive rows (runs in XCD-contiguous order) and keeps a row in
// registers from the sum of squares to the quantization; the next row's
// loads are issued before the current row is computed, so HBM traffic
// overlaps the arithmetic.  gamma is loaded once.
// rmsnorm_quant_kernel (longer rows): one row per workgroup, read twice (with
// ADD the sum is formed in both passes and stored in the second, so a
// residual output that is x itself is read before it is overwritten).

struct RmsArgs {
  const uint16_t* x;
  const uint16_t* gamma;
  float eps;
  int64_t M, K, ldx;
  uint8_t* q;
  int64_t ldq;
  float* scales;
  int col_major;
  uint16_t* y_out;
  int64_t ldy;
  const uint16_t* h;         // ADD: sublayer output
  int64_t ldh;
  uint16_t* z_out;           // ADD: updated residual stream
  int64_t ldz;
  const float* static_scale; // EXIT_STATIC: per-tensor scale
};

// STREAM: the row is read once (activations, the sublayer output); the norm
// weight, which every workgroup reads, is loaded without the streaming hint.
template <int CH, bool STREAM = true>
__device__ __forceinline__ void load_row_seg(uint4 (&raw)[CH], const uint16_t* xr, int64_t seg0, int64_t K) {
  const int lane = threadIdx.x & 63;
  if (seg0 + 512 * CH <= K) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const uint16_t* p = xr + seg0 + 512 * c + 8 * lane;
      raw[c] = STREAM ? ld16_nt(p) : ld16(p);
    }
  } else {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t k0 = seg0 + 512 * c + 8 * lane;
      raw[c] = (k0 < K) ? load8_bf16_masked(xr, k0, K) : make_uint4(0, 0, 0, 0);
    }
  }
}

// z = bf16(x + h) for a segment, in place in x: one fp32 addition and one
// round-to-nearest-even to bf16.  The fp32 sum of two bf16 values rounded to
// bf16 is the correctly rounded sum (24 >= 2*8 + 1 bits: the double rounding
// is innocuous); zero padding past K stays zero.
template <int CH>
__device__ __forceinline__ void add_seg(uint4 (&x)[CH], const uint4 (&h)[CH]) {
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    float a[8], b[8];
    unpack8(x[c], a);
    unpack8(h[c], b);
    uint32_t o[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) o[e >> 1] = pack_bf16x2(a[e] + b[e], a[e + 1] + b[e + 1]);
    x[c] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

template <int CH>
__device__ __forceinline__ void store_row_seg(uint16_t* zr, const uint4 (&z)[CH], int64_t seg0, int64_t K) {
  const int lane = threadIdx.x & 63;
  const bool full = seg0 + 512 * CH <= K;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t k0 = seg0 + 512 * c + 8 * lane;
    if (full) *reinterpret_cast<uint4*>(zr + k0) = z[c];
    else if (k0 < K) store8_bf16_masked(zr, k0, K, z[c]);
  }
}

// fp64 sum of squares of a segment (squares of bf16 values are exact); one
// accumulation chain per chunk, so the chains overlap instead of forming
// one dependent chain of 8*CH fused multiply-adds
template <int CH>
__device__ __forceinline__ double sumsq_seg(const uint4 (&raw)[CH], double ss) {
  double part[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    float v[8];
    unpack8(raw[c], v);
    double t = 0.0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const double d = (double)v[e];
      t = __builtin_fma(d, d, t);
    }
    part[c] = t;
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) ss += part[c];
  return ss;
}

// r = fp32(1 / sqrt(sum / K + eps)) from the wave partials; `part` holds one
// slot per wave, written here, and the caller's barrier discipline keeps a
// slot set from being overwritten while another wave still reads it.
// fp32 rounding of 1/sqrt(v) for v > 0 (normal): the hardware estimate
// refined by two Newton steps in fp64, y <- y + y (1/2 - (v/2) y^2), each of
// which squares the relative error, to within a few fp64 ulps of the exact
// value; the fp32 rounding is then that of the exact value unless this lies
// within about 2^-50 of an fp32 rounding boundary.
__device__ __forceinline__ float rsqrt_f64_to_f32(double v) {
  const double h = 0.5 * v;
  double y = __builtin_amdgcn_rsq(v);
  y = __builtin_fma(y, __builtin_fma(-h * y, y, 0.5), y);
  y = __builtin_fma(y, __builtin_fma(-h * y, y, 0.5), y);
  return (float)y;
}

__device__ __forceinline__ float rms_inv(double ss, double* part, double inv_k, float eps) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  ss = sum_wave_f64(ss);
  if (lane == 0) part[wave] = ss;
  __syncthreads();
  ss = ((part[0] + part[1]) + part[2]) + part[3];
  return rsqrt_f64_to_f32(__builtin_fma(ss, inv_k, (double)eps));
}

enum { EXIT_GROUP = 0, EXIT_STATIC = 1, EXIT_POW2 = 2 };

// y = bf16((x * r) * g) for one segment, then its quantization: group
// scales, the static scale s (q = E4M3(clamp(fp32(y / s))), IEEE division),
// or power-of-two group scales.
template <int CH, int EXIT>
__device__ __forceinline__ void norm_quant_seg(const RmsArgs& a, uint4 (&raw)[CH], const float (&gf)[CH][8],
                                               float rn, float s_stat, int64_t row, int64_t seg0) {
  const int lane = threadIdx.x & 63;
  const int64_t K = a.K;
  const bool full = seg0 + 512 * CH <= K;
  uint8_t* qr = a.q + row * a.ldq;
  uint16_t* yr = a.y_out != nullptr ? a.y_out + row * a.ldy : nullptr;
  // y[c]: the bf16 values of y as fp32, unpacked once from their rounding
  // and used by both the group maximum and the quotients
  float amax[CH], y[CH][8];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t k0 = seg0 + 512 * c + 8 * lane;
    float v[8];
    unpack8(raw[c], v);
    const float* g = gf[c];
    uint32_t yb[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) yb[e >> 1] = pack_bf16x2((v[e] * rn) * g[e], (v[e + 1] * rn) * g[e + 1]);
    raw[c] = make_uint4(yb[0], yb[1], yb[2], yb[3]);      // raw now holds bf16 y
    if (yr != nullptr) {
      if (full) *reinterpret_cast<uint4*>(yr + k0) = raw[c];
      else if (k0 < K) store8_bf16_masked(yr, k0, K, raw[c]);
    }
    unpack8(raw[c], y[c]);
    if (EXIT != EXIT_STATIC) {
      float m = fabsf(y[c][0]);
#pragma unroll
      for (int e = 1; e < 8; ++e) m = fmaxf(m, fabsf(y[c][e]));
      amax[c] = max_row16(m);
    }
  }
  if (EXIT == EXIT_STATIC) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int64_t k0 = seg0 + 512 * c + 8 * lane;
      float t[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = clamp448(y[c][e] / s_stat);   // IEEE division
      const uint2 o = encode8(t);
      if (full) st8_nt(qr + k0, o);
      else if (k0 < K) store8_masked(qr, k0, K, o);
    }
    return;
  }
  float s[CH], r[CH], s_mine;
  uint32_t byte[CH];
  if constexpr (EXIT == EXIT_POW2) pow2_group_scales<CH>(amax, byte, s_mine);
  else group_scales<CH>(amax, s, r, s_mine);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t k0 = seg0 + 512 * c + 8 * lane;
    float t[8];
    if constexpr (EXIT == EXIT_POW2) {
      // 2^-e = 2^(127 - byte) exactly; x * 2^-e is exact (see quant8_mx)
      const float inv = __uint_as_float((254u - byte[c]) << 23);
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = y[c][e] * inv;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = div_by_scale(y[c][e], s[c], r[c]);
    }
    const uint2 o = encode8(t);
    if (full) st8_nt(qr + k0, o);
    else if (k0 < K) store8_masked(qr, k0, K, o);
  }
  store_group_scales<CH>(a.scales, s_mine, seg0 / 128, (K + 127) >> 7, a.M, row, a.col_major);
}

template <int CH, bool ADD, int EXIT>
__global__ __launch_bounds__(256) void rmsnorm_quant_rows_kernel(RmsArgs a, int rows_per_wg) {
  __shared__ double part[2][4];
  const int wave = threadIdx.x >> 6;
  const int64_t r0 = (int64_t)xcd_contiguous(blockIdx.x, gridDim.x) * rows_per_wg;
  const int64_t r1 = r0 + rows_per_wg < a.M ? r0 + rows_per_wg : a.M;
  if (r0 >= a.M) return;                       // whole workgroup
  const int64_t seg0 = (int64_t)wave * (512 * CH);
  const float s_stat = EXIT == EXIT_STATIC ? *a.static_scale : 1.0f;
  uint4 cur[CH], nxt[CH];
  uint4 hcur[ADD ? CH : 1], hnxt[ADD ? CH : 1];
  float gf[CH][8];          // gamma of this wave's segment, unpacked once
  {
    uint4 gr[CH];
    load_row_seg<CH, false>(gr, a.gamma, seg0, a.K);
#pragma unroll
    for (int c = 0; c < CH; ++c) unpack8(gr[c], gf[c]);
  }
  auto load = [&](uint4 (&xb)[CH], uint4 (&hb)[ADD ? CH : 1], int64_t row) {
    load_row_seg<CH>(xb, a.x + row * a.ldx, seg0, a.K);
    if constexpr (ADD) load_row_seg<CH>(hb, a.h + row * a.ldh, seg0, a.K);
  };
  load(cur, hcur, r0);
  const double inv_k = 1.0 / (double)a.K;
  // one row: its successor's loads go into the other buffers first
  auto step = [&](uint4 (&buf)[CH], uint4 (&hbuf)[ADD ? CH : 1], uint4 (&other)[CH],
                  uint4 (&hother)[ADD ? CH : 1], int64_t row) {
    if (row + 1 < r1) load(other, hother, row + 1);
    if constexpr (ADD) {
      add_seg<CH>(buf, hbuf);
      if (seg0 < a.K) store_row_seg<CH>(a.z_out + row * a.ldz, buf, seg0, a.K);
    }
    // the two slot sets alternate; the barrier inside rms_inv of row i+1
    // orders every read of set (i & 1) before the writes of row i+2
    const float rn = rms_inv(sumsq_seg<CH>(buf, 0.0), part[(row - r0) & 1], inv_k, a.eps);
    if (seg0 < a.K) norm_quant_seg<CH, EXIT>(a, buf, gf, rn, s_stat, row, seg0);
  };
  // rows alternate between the two buffer sets (no copies between rows)
  for (int64_t row = r0; row < r1; row += 2) {
    step(cur, hcur, nxt, hnxt, row);
    if (row + 1 < r1) step(nxt, hnxt, cur, hcur, row + 1);
  }
}

template <int CH, bool ADD, int EXIT>
__global__ __launch_bounds__(256) void rmsnorm_quant_kernel(RmsArgs a) {
  __shared__ double part[4];
  const int wave = threadIdx.x >> 6;
  const int64_t row = xcd_contiguous(blockIdx.x, gridDim.x);
  const uint16_t* xr = a.x + row * a.ldx;
  const uint16_t* hr = ADD ? a.h + row * a.ldh : nullptr;
  constexpr int64_t SEG = 512 * CH;
  const int64_t npass = (a.K + 4 * SEG - 1) / (4 * SEG);
  const float s_stat = EXIT == EXIT_STATIC ? *a.static_scale : 1.0f;
  uint4 raw[CH], gr[CH];
  double ss = 0.0;
  for (int64_t it = 0; it < npass; ++it) {
    // first of two reads: keep the lines cached for the second
    load_row_seg<CH, false>(raw, xr, (4 * it + wave) * SEG, a.K);
    if constexpr (ADD) {
      load_row_seg<CH, false>(gr, hr, (4 * it + wave) * SEG, a.K);
      add_seg<CH>(raw, gr);
    }
    ss = sumsq_seg<CH>(raw, ss);
  }
  const float rn = rms_inv(ss, part, 1.0 / (double)a.K, a.eps);
  for (int64_t it = 0; it < npass; ++it) {
    const int64_t seg0 = (4 * it + wave) * SEG;
    if (seg0 >= a.K) break;
    load_row_seg<CH>(raw, xr, seg0, a.K);
    if constexpr (ADD) {
      load_row_seg<CH>(gr, hr, seg0, a.K);
      add_seg<CH>(raw, gr);
      store_row_seg<CH>(a.z_out + row * a.ldz, raw, seg0, a.K);
    }
    load_row_seg<CH, false>(gr, a.gamma, seg0, a.K);
    float gf[CH][8];
#pragma unroll
    for (int c = 0; c < CH; ++c) unpack8(gr[c], gf[c]);
    norm_quant_seg<CH, EXIT>(a, raw, gf, rn, s_stat, row, seg0);
  }
}

// --------------------------------------------------------------------------
// Weight blocks.  One 256-thread workgroup per 128x128 block: thread t holds
// the 8-column chunk (t % 16) of rows t/16 + 16i, i = 0..7 (each 16-lane row
// of a wave reads one 256-byte block row contiguously).
//   MODE 0: block scale = block amax / 448; quantize; write scale.
//   MODE 1: per-tensor pass 1 -- fold the block amax into *slot (integer max
//           of the non-negative fp32 bit patterns: order independent).
//   MODE 2: per-tensor pass 2 -- quantize with s from the tensor amax in *slot.
//   MODE 3: block scale = the power of two 2^e of the MX round-up rule;
//           codes w * 2^-e.

template <int MODE>
__global__ __launch_bounds__(256) void weight_block_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, int64_t ldw,
    uint8_t* __restrict__ q, int64_t ldq, float* __restrict__ scale_out,
    uint32_t* __restrict__ slot, int64_t KB) {
  __shared__ float red[4];
  const int t = threadIdx.x;
  const int64_t bn = blockIdx.y, bk = blockIdx.x;
  const int64_t k0 = bk * 128 + 8 * (t & 15);
  uint4 raw[8];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t n = bn * 128 + (t >> 4) + 16 * i;
    raw[i] = (n < N && k0 < K) ? load8_bf16_masked(w + n * ldw, k0, K) : make_uint4(0, 0, 0, 0);
    if (MODE != 2) m = fmaxf(m, absmax8(raw[i]));
  }
  float amax;
  if (MODE != 2) {
    m = max_wave(m);
    if ((t & 63) == 0) red[t >> 6] = m;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    if (MODE == 1) {
      if (t == 0) atomicMax(slot, __float_as_uint(amax));
      return;
    }
  } else {
    amax = __uint_as_float(*slot);
  }
  if constexpr (MODE == 3) {
    const uint32_t byte = ue8m0_byte(amax);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t n = bn * 128 + (t >> 4) + 16 * i;
      if (n < N && k0 < K) store8_masked(q + n * ldq, k0, K, quant8_mx(raw[i], byte));
    }
    if (t == 0) scale_out[bn * KB + bk] = __uint_as_float(byte << 23);
    return;
  }
  const float s = fmaxf(amax, kAmaxFloor) / kFp8Max;
  const float r = 1.0f / s;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t n = bn * 128 + (t >> 4) + 16 * i;
    if (n < N && k0 < K) store8_masked(q + n * ldq, k0, K, quant8(raw[i], s, r));
  }
  if (MODE == 0 && t == 0) scale_out[bn * KB + bk] = s;
}

// fp32 product a * b rounded to odd: the nearest-rounded product, moved one
// ulp toward the exact value (whose remainder an FMA gives exactly) when it is
// inexact and its last bit is even.  Rounding that to a format at least two
// bits narrower is the correct rounding of the exact product.
__device__ __forceinline__ float mul_round_odd(float a, float b) {
  const float p = a * b;
  const float e = __builtin_fmaf(a, b, -p);
  uint32_t bits = __float_as_uint(p);
  if (e != 0.0f && (bits & 1u) == 0u) bits += ((__float_as_uint(e) ^ bits) & 0x80000000u) ? 0xFFFFFFFFu : 1u;
  return __uint_as_float(bits);
}

// Re-quantization of one 128x128 block-FP8 block to a power-of-two scale:
// s' = the smallest power of two >= s, codes E4M3(decode(q) * (s / s')).  For
// a positive normal s = 1.f * 2^E, s' = 2^E when f = 0 and 2^(E+1) otherwise,
// and s / s' (1 or 0.1f in binary) keeps s's mantissa.  The exact product of
// a 4-bit code value and that 24-bit ratio can need 28 bits, and its
// nearest fp32 value can be an E4M3 rounding midpoint that the exact value is
// not; the product is therefore rounded to odd in fp32 before the E4M3
// conversion rounds it to nearest-even.  |decode(q)| <= 448 and s / s' <= 1,
// so nothing saturates.  In place is allowed (q_out == q_in, s_out == s_in):
// every thread reads its codes before writing them, and the scale is written
// after a barrier that follows every thread's read of it.
__global__ __launch_bounds__(256) void requant_pow2_kernel(
    const uint8_t* q_in, int64_t ldi, const float* s_in, int64_t N, int64_t K,
    uint8_t* q_out, int64_t ldo, float* s_out, int64_t KB) {
  const int t = threadIdx.x;
  const int64_t bn = blockIdx.y, bk = blockIdx.x;
  const int64_t k0 = bk * 128 + 8 * (t & 15);
  const uint32_t b = __float_as_uint(s_in[bn * KB + bk]);
  const uint32_t f = b & 0x7FFFFFu;
  const uint32_t eb = (b >> 23) + (f ? 1u : 0u);              // biased exponent of s'
  const float mul = __uint_as_float(f | ((f ? 126u : 127u) << 23));
#pragma unroll 4
  for (int i = 0; i < 8; ++i) {
    const int64_t n = bn * 128 + (t >> 4) + 16 * i;
    if (n >= N || k0 >= K) continue;
    const uint8_t* src = q_in + n * ldi;
    uint2 c;
    if (k0 + 8 <= K) {
      c = *reinterpret_cast<const uint2*>(src + k0);
    } else {
      uint32_t w[2] = {0u, 0u};
      for (int e = 0; k0 + e < K; ++e) w[e >> 2] |= (uint32_t)src[k0 + e] << (8 * (e & 3));
      c = make_uint2(w[0], w[1]);
    }
    float v[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t word = h ? c.y : c.x;
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
      v[4 * h + 0] = mul_round_odd(lo[0], mul);
      v[4 * h + 1] = mul_round_odd(lo[1], mul);
      v[4 * h + 2] = mul_round_odd(hi[0], mul);
      v[4 * h + 3] = mul_round_odd(hi[1], mul);
    }
    store8_masked(q_out + n * ldo, k0, K, encode8(v));
  }
  __syncthreads();
  if (t == 0) s_out[bn * KB + bk] = __uint_as_float(eb << 23);
}

__global__ void zero_slot_kernel(uint32_t* slot) { *slot = 0u; }

// amax bits in slot -> fp32 scale, in place (after MODE 2 has read it).
__global__ void finalize_tensor_scale_kernel(uint32_t* slot) {
  const float amax = __uint_as_float(*slot);
  *reinterpret_cast<float*>(slot) = fmaxf(amax, kAmaxFloor) / kFp8Max;
}

// --------------------------------------------------------------------------
// Host launchers

static inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Row quantizers: segments of 512*CH elements per wave.  Rows of at most 512
// take one chunk; longer rows take 2, or 3, 5 or 7 when the row is an odd
// number of whole 512-element chunks that one of them divides (a ragged
// last segment runs the masked path: 12 % slower at K = 7168, measured),
// else 2 with a masked last segment.  Two chunks per wave measured best or
// equal for the group, MX and static quantizers on 2048x7168, 4096x6144 and
// 8192x7168 (against 1, 3, 4 and 7: MX 2-7 % and static 0-3 % faster than
// with 4 or 7, the group quantizer within 1 %).
static inline int row_chunks(int64_t K) {
  if (K <= 512) return 1;
  if (K % 1024 == 512) {
    const int64_t n = K / 512;
    for (const int c : {3, 5, 7})
      if (n % c == 0) return c;
  }
  return 2;
}

// LAUNCH(C) for the chunk count row_chunks chose
#define FP8Q_BY_CHUNKS(ch, LAUNCH) \
  do {                              \
    switch (ch) {                   \
      case 1: LAUNCH(1); break;     \
      case 3: LAUNCH(3); break;     \
      case 5: LAUNCH(5); break;     \
      case 7: LAUNCH(7); break;     \
      default: LAUNCH(2); break;    \
    }                               \
  } while (0)

// 1-D grid of ceil(M/4) * segs workgroups; the kernels index it with int.
static inline bool row_grid_fits(int64_t M, int64_t segs) { return ceil_div(M, 4) * segs <= 0x7FFFFFFF; }
static inline dim3 row_grid(int64_t M, int64_t segs) { return dim3((unsigned)(ceil_div(M, 4) * segs)); }

hipError_t launch_quant_group128(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                 uint8_t* q, int64_t ldq, float* scales, int col_major, int pow2,
                                 hipStream_t stream) {
  const int ch = row_chunks(K);
  const int segs = (int)ceil_div(K, 512 * ch);
  if (!row_grid_fits(M, segs)) return hipErrorInvalidConfiguration;
  const dim3 grid = row_grid(M, segs), block(256);
#define FP8Q_G128(CH, P2) \
  hipLaunchKernelGGL((quant_group128_kernel<CH, P2>), grid, block, 0, stream, x, M, K, ldx, q, ldq, scales, col_major, segs)
#define FP8Q_G128_P2(CH) FP8Q_G128(CH, true)
#define FP8Q_G128_F(CH) FP8Q_G128(CH, false)
  if (pow2) FP8Q_BY_CHUNKS(ch, FP8Q_G128_P2);
  else FP8Q_BY_CHUNKS(ch, FP8Q_G128_F);
#undef FP8Q_G128_F
#undef FP8Q_G128_P2
#undef FP8Q_G128
  return hipGetLastError();
}

hipError_t launch_quant_group32mx(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                  uint8_t* q, int64_t ldq, uint8_t* scales, int col_major,
                                  hipStream_t stream) {
  const int ch = row_chunks(K);
  const int segs = (int)ceil_div(K, 512 * ch);
  if (!row_grid_fits(M, segs)) return hipErrorInvalidConfiguration;
  const dim3 grid = row_grid(M, segs), block(256);
#define FP8Q_MX(CH) \
  hipLaunchKernelGGL(quant_group32mx_kernel<CH>, grid, block, 0, stream, x, M, K, ldx, q, ldq, scales, col_major, segs)
  FP8Q_BY_CHUNKS(ch, FP8Q_MX);
#undef FP8Q_MX
  return hipGetLastError();
}

hipError_t launch_quant_static(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                               const float* scale, uint8_t* q, int64_t ldq, hipStream_t stream) {
  const int ch = row_chunks(K);
  const int segs = (int)ceil_div(K, 512 * ch);
  if (!row_grid_fits(M, segs)) return hipErrorInvalidConfiguration;
  const dim3 grid = row_grid(M, segs), block(256);
#define FP8Q_ST(CH) \
  hipLaunchKernelGGL(quant_static_kernel<CH>, grid, block, 0, stream, x, M, K, ldx, scale, q, ldq, segs)
  FP8Q_BY_CHUNKS(ch, FP8Q_ST);
#undef FP8Q_ST
  return hipGetLastError();
}

namespace {

// 256-thread workgroups of `kern` that one CU holds at once (at least 1)
int resident_wgs(const void* kern) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, 256, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

template <bool ADD, int EXIT>
hipError_t dispatch_rmsnorm(const RmsArgs& a, hipStream_t stream) {
  const dim3 block(256);
  if (a.K > 4 * 512 * 8) {   // long rows: one workgroup per row, two reads
    hipLaunchKernelGGL((rmsnorm_quant_kernel<4, ADD, EXIT>), dim3((unsigned)a.M), block, 0, stream, a);
    return hipGetLastError();
  }
  // up to four workgroups per CU, each a run of consecutive rows (measured
  // best against two per CU and against one workgroup per row); never more
  // than fit at once, so that no CU runs a second round of runs
#ifndef FP8Q_RMS_WGS_PER_CU
#define FP8Q_RMS_WGS_PER_CU 4
#endif
#define FP8Q_RMS(CH)                                                                                   \
  do {                                                                                                 \
    const auto kern = rmsnorm_quant_rows_kernel<CH, ADD, EXIT>;                                        \
    static const int fit = resident_wgs(reinterpret_cast<const void*>(kern));                          \
    const int64_t wgs = (int64_t)device_cu_count() * (fit < FP8Q_RMS_WGS_PER_CU ? fit : FP8Q_RMS_WGS_PER_CU); \
    const int rows = (int)ceil_div(a.M, wgs);                                                          \
    hipLaunchKernelGGL(kern, dim3((unsigned)ceil_div(a.M, rows)), block, 0, stream, a, rows);          \
  } while (0)
  const int64_t K = a.K;
  if (K <= 2048) FP8Q_RMS(1);
  else if (K <= 4096) FP8Q_RMS(2);
  else if (K <= 6144) FP8Q_RMS(3);
  else if (K <= 8192) FP8Q_RMS(4);
  else if (K <= 12288) FP8Q_RMS(6);
  else FP8Q_RMS(8);
#undef FP8Q_RMS
  return hipGetLastError();
}

}  // namespace

hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* gamma, float eps, int64_t M,
                                int64_t K, int64_t ldx, uint8_t* q, int64_t ldq, float* scales,
                                int col_major, uint16_t* y_out, int64_t ldy, hipStream_t stream) {
  const RmsArgs a{x, gamma, eps, M, K, ldx, q, ldq, scales, col_major, y_out, ldy,
                  nullptr, 0, nullptr, 0, nullptr};
  return dispatch_rmsnorm<false, EXIT_GROUP>(a, stream);
}

hipError_t launch_add_rmsnorm_quant(const uint16_t* x, int64_t ldx, const uint16_t* h, int64_t ldh,
                                    uint16_t* z_out, int64_t ldz, const uint16_t* gamma, float eps,
                                    int64_t M, int64_t K, const float* static_scale, int pow2, uint8_t* q,
                                    int64_t ldq, float* scales, int col_major, uint16_t* y_out,
                                    int64_t ldy, hipStream_t stream) {
  const RmsArgs a{x, gamma, eps, M, K, ldx, q, ldq, scales, col_major, y_out, ldy,
                  h, ldh, z_out, ldz, static_scale};
  if (h == nullptr) {
    if (static_scale != nullptr) return dispatch_rmsnorm<false, EXIT_STATIC>(a, stream);
    return pow2 ? dispatch_rmsnorm<false, EXIT_POW2>(a, stream) : dispatch_rmsnorm<false, EXIT_GROUP>(a, stream);
  }
  if (static_scale != nullptr) return dispatch_rmsnorm<true, EXIT_STATIC>(a, stream);
  return pow2 ? dispatch_rmsnorm<true, EXIT_POW2>(a, stream) : dispatch_rmsnorm<true, EXIT_GROUP>(a, stream);
}

hipError_t launch_weight_block128(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                  uint8_t* q, int64_t ldq, float* scale_inv, int pow2, hipStream_t stream) {
  const int64_t KB = ceil_div(K, 128);
  const dim3 grid((unsigned)KB, (unsigned)ceil_div(N, 128)), block(256);
  if (pow2)
    hipLaunchKernelGGL(weight_block_kernel<3>, grid, block, 0, stream, w, N, K, ldw, q, ldq, scale_inv,
                       (uint32_t*)nullptr, KB);
  else
    hipLaunchKernelGGL(weight_block_kernel<0>, grid, block, 0, stream, w, N, K, ldw, q, ldq, scale_inv,
                       (uint32_t*)nullptr, KB);
  return hipGetLastError();
}

hipError_t launch_requant_pow2(const uint8_t* q_in, int64_t ldi, const float* s_in, int64_t N, int64_t K,
                               uint8_t* q_out, int64_t ldo, float* s_out, hipStream_t stream) {
  const int64_t KB = ceil_div(K, 128);
  const dim3 grid((unsigned)KB, (unsigned)ceil_div(N, 128)), block(256);
  hipLaunchKernelGGL(requant_pow2_kernel, grid, block, 0, stream, q_in, ldi, s_in, N, K, q_out, ldo, s_out, KB);
  return hipGetLastError();
}

hipError_t launch_weight_tensor(const uint16_t* w, int64_t N, int64_t K, int64_t ldw, uint8_t* q,
                                int64_t ldq, float* scale_inv, hipStream_t stream) {
  const int64_t KB = ceil_div(K, 128);
  const dim3 grid((unsigned)KB, (unsigned)ceil_div(N, 128)), block(256);
  uint32_t* slot = reinterpret_cast<uint32_t*>(scale_inv);
  hipLaunchKernelGGL(zero_slot_kernel, dim3(1), dim3(1), 0, stream, slot);
  hipLaunchKernelGGL(weight_block_kernel<1>, grid, block, 0, stream, w, N, K, ldw, q, ldq,
                     (float*)nullptr, slot, KB);
  hipLaunchKernelGGL(weight_block_kernel<2>, grid, block, 0, stream, w, N, K, ldw, q, ldq,
                     (float*)nullptr, slot, KB);
  hipLaunchKernelGGL(finalize_tensor_scale_kernel, dim3(1), dim3(1), 0, stream, slot);
  return hipGetLastError();
}

}  // namespace fp8q
