// Device helpers shared by the fp8q kernels (gfx950 only).
//
// Arithmetic notes
// * The library is compiled with -ffp-contract=off: every multiply and add is
//   rounded as written; fused multiply-adds appear only where __builtin_fmaf
//   is spelled out.
// * fp32 denormals are kept (no flush-to-zero) and fp32 division is the
//   compiler's correctly rounded IEEE division.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8q {

constexpr float kFp8Max = 448.0f;   // largest finite OCP E4M3 value
constexpr float kAmaxFloor = 1e-10f;

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- bf16 <-> f32

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Unpack 8 bf16 (one 16-byte chunk) into fp32.
__device__ __forceinline__ void unpack8(const uint4& c, float v[8]) {
  v[0] = bf16_lo(c.x); v[1] = bf16_hi(c.x);
  v[2] = bf16_lo(c.y); v[3] = bf16_hi(c.y);
  v[4] = bf16_lo(c.z); v[5] = bf16_hi(c.z);
  v[6] = bf16_lo(c.w); v[7] = bf16_hi(c.w);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; overflow -> inf).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (v_cvt_pk_bf16_f32: round to nearest even).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 b = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
  return __builtin_bit_cast(uint32_t, b);
}

// ------------------------------------------------------------------ E4M3 encode

// Two fp32 values (already clamped to +-448) -> two E4M3 bytes in the low or
// high half of `old`, using the hardware conversion (round to nearest even).
template <bool HI>
__device__ __forceinline__ uint32_t cvt_pk_e4m3(float a, float b, uint32_t old) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI);
}

__device__ __forceinline__ float clamp448(float t) {
  return __builtin_amdgcn_fmed3f(t, -kFp8Max, kFp8Max);
}

// Encode 8 clamped fp32 values into 8 E4M3 bytes.
__device__ __forceinline__ uint2 encode8(const float t[8]) {
  uint32_t w0 = cvt_pk_e4m3<false>(t[0], t[1], 0u);
  w0 = cvt_pk_e4m3<true>(t[2], t[3], w0);
  uint32_t w1 = cvt_pk_e4m3<false>(t[4], t[5], 0u);
  w1 = cvt_pk_e4m3<true>(t[6], t[7], w1);
  return make_uint2(w0, w1);
}

// ------------------------------------------------------------ x / s in fp32

// fp32 quotient x / s for the quantizer's operand domain, given r = RN(1/s):
// y = RN(x*r) is refined once with the exact negated residual y*s - x (one
// FMA) -- Markstein's correction.  Computing the residual as y*s - x (rather
// than x - y*s) keeps the sign of a zero x, so the sequence is odd in x.  For
// every bf16 x with |x| <= amax and s = RN(max(amax, 1e-10)/448), amax a bf16
// value, the result equals the IEEE quotient x / s wherever either is at
// least 2^-10, and both lie below 2^-10 (so both encode to the E4M3 zero of
// the sign of x) everywhere else; a host-side test enumerates that finite
// domain.
__device__ __forceinline__ float div_by_scale(float x, float s, float r) {
  const float y = x * r;
  const float e = __builtin_fmaf(y, s, -x);
  return __builtin_fmaf(-e, r, y);
}

// ------------------------------------------------------- cross-lane max / sum

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// Cross-lane maxima of NON-NEGATIVE, non-NaN fp32 values: on such values the
// order of the bit patterns as unsigned integers is the numeric order, so the
// DPP steps are integer maxima (no NaN canonicalisation needed).

// Max over each aligned group of 4 lanes (quad), result in every lane.
__device__ __forceinline__ float max_quad(float v) {
  uint32_t u = __float_as_uint(v);
  u = max(u, dpp_u<0xB1>(u));     // quad_perm [1,0,3,2]
  u = max(u, dpp_u<0x4E>(u));     // quad_perm [2,3,0,1]
  return __uint_as_float(u);
}

// Max over each aligned row of 16 lanes, result in every lane.
__device__ __forceinline__ float max_row16(float v) {
  uint32_t u = __float_as_uint(max_quad(v));
  u = max(u, dpp_u<0x141>(u));    // row_half_mirror: lanes 0-3 <-> 4-7
  u = max(u, dpp_u<0x140>(u));    // row_mirror: lanes 0-7 <-> 8-15
  return __uint_as_float(u);
}

// Max over the whole 64-lane wave (every lane gets the result).
__device__ __forceinline__ float max_wave(float v) {
  uint32_t u = __float_as_uint(max_row16(v));
  u = max(u, (uint32_t)__shfl_xor((int)u, 16));
  u = max(u, (uint32_t)__shfl_xor((int)u, 32));
  return __uint_as_float(u);
}

// fp64 value of a DPP partner lane (both 32-bit halves moved alike)
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = dpp_u<CTRL>((uint32_t)u), hi = dpp_u<CTRL>((uint32_t)(u >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// v plus the value of the partner lane in the other 16-lane row of a row
// pair (HALF32 false) or in the other half of the wave (HALF32 true), via
// the lane-swap instructions (VALU, no LDS round trip)
template <bool HALF32>
__device__ __forceinline__ double add_swapped_f64(double v) {
  const uint64_t u = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  uint32_t plo, phi;
  if constexpr (HALF32) {
    const auto sl = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto sh = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const bool upper = (threadIdx.x & 32) != 0;
    plo = upper ? sl[0] : sl[1];
    phi = upper ? sh[0] : sh[1];
  } else {
    const auto sl = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
    const auto sh = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
    const bool odd = (threadIdx.x & 16) != 0;
    plo = odd ? sl[0] : sl[1];
    phi = odd ? sh[0] : sh[1];
  }
  return v + __longlong_as_double((long long)(((uint64_t)phi << 32) | plo));
}

// Sum over the 64-lane wave, the same bits in every lane: each step adds a
// lane's value and its partner's (fp64 addition is commutative, so partners
// compute the same sum): quads, half-rows and rows by DPP, then row pairs
// and wave halves by lane swaps.
__device__ __forceinline__ double sum_wave_f64(double v) {
  v += dpp_f64<0xB1>(v);     // quad_perm [1,0,3,2]
  v += dpp_f64<0x4E>(v);     // quad_perm [2,3,0,1]
  v += dpp_f64<0x141>(v);    // row_half_mirror
  v += dpp_f64<0x140>(v);    // row_mirror
  v = add_swapped_f64<false>(v);
  return add_swapped_f64<true>(v);
}

// ------------------------------------------------------------- work mapping

// Hardware hands consecutive workgroup ids to the 8 XCDs in turn.  Renumber
// ids 0..total-1 so that each XCD receives a contiguous run (a bijection):
// neighbouring work items then share that XCD's L2, and partial cache lines
// written by neighbours (column-major scales) are completed in one L2.
__device__ __forceinline__ int xcd_contiguous(int pid, int total) {
  const int xcd = pid & 7, idx = pid >> 3;
  const int per = total >> 3, rem = total & 7;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
}

// ------------------------------------------------------------- memory access

__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void st8(void* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }

// Streaming forms (non-temporal hint) for data a kernel touches once: an
// activation row that is read once, a row of codes written once.  On gfx950
// the hint lifts the quantizers' read-bf16 / write-byte stream by ~10 % (the
// one-shot quantizers gain from it on their loads; the row-walking RMSNorm
// quantizer and the static quantizer also on their code stores, where the
// group and MX quantizers measured 1-8 % slower with it).
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 ld16_nt(const void* p) {
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void st8_nt(void* p, uint2 v) {
  __builtin_nontemporal_store((u32x2){v.x, v.y}, reinterpret_cast<u32x2*>(p));
}

// Load 8 bf16 starting at column k0 of a row of logical length K; columns >= K
// read as zero.  Whole chunk via one 16-byte load when it lies inside [0, K);
// otherwise element by element.
__device__ __forceinline__ uint4 load8_bf16_masked(const uint16_t* row, int64_t k0, int64_t K) {
  if (k0 + 8 <= K) return ld16(row + k0);
  uint32_t w[4] = {0u, 0u, 0u, 0u};
  for (int e = 0; e < 8; ++e) {
    if (k0 + e < K) w[e >> 1] |= (uint32_t)row[k0 + e] << ((e & 1) * 16);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Store 8 bytes at column k0 of a row of logical length K (bytes >= K dropped).
__device__ __forceinline__ void store8_masked(uint8_t* row, int64_t k0, int64_t K, uint2 v) {
  if (k0 + 8 <= K) { st8(row + k0, v); return; }
  for (int e = 0; e < 8; ++e) {
    if (k0 + e < K) {
      uint32_t w = e < 4 ? v.x : v.y;
      row[k0 + e] = (uint8_t)(w >> ((e & 3) * 8));
    }
  }
}

__device__ __forceinline__ void store8_bf16_masked(uint16_t* row, int64_t k0, int64_t K, uint4 v) {
  if (k0 + 8 <= K) { *reinterpret_cast<uint4*>(row + k0) = v; return; }
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  for (int e = 0; e < 8; ++e)
    if (k0 + e < K) row[k0 + e] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
}

}  // namespace fp8q
