// Direct-to-LDS loading helpers of the FP8 GEMM kernels (gfx950): buffer
// descriptors, the LDS tile swizzle, explicitly counted waits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace fp8q {
namespace dma {

// Byte offset of 16-byte chunk c (0..7) of tile row r in a swizzled LDS tile.
__device__ __forceinline__ int swz(int r, int c) { return (r << 7) | ((c ^ (r & 7)) << 4); }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Raw buffer descriptor (stride 0): lanes whose offset is >= `bytes` read 0.
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

// Direct-to-LDS loads: lane i's 16 (or 4) bytes from base + voffset + soffset
// land at LDS address lds + 16*i (4*i); `lds` and `soffset` are wave-uniform.
// Written as inline assembly on purpose: the compiler cannot tell which LDS
// stage a direct-to-LDS load fills, and would otherwise make every LDS read
// wait for all of them.  These loads are therefore invisible to the
// compiler's vmcnt bookkeeping; the kernel waits for them explicitly and
// issues no other vector-memory loads inside its K loop.
// Every caller keeps voffset + soffset below the descriptor's size for a lane
// whose voffset is below it, so the loads stay inside their arrays whether or
// not the range check includes the scalar offset.
__device__ __forceinline__ void dma16(const i32x4& r, uint32_t lds, uint32_t voffset, uint32_t soffset) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds"
               :
               : "v"(voffset), "s"(r), "s"(lds), "s"(soffset)
               : "memory", "m0");
}
// The same with the non-temporal hint, for operand bytes a launch reads once
// (a decode GEMM's weights, an expert's weights in the grouped GEMM): they
// stream through the caches instead of displacing lines that are re-read.
__device__ __forceinline__ void dma16_nt(const i32x4& r, uint32_t lds, uint32_t voffset, uint32_t soffset) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, %3 offen nt lds"
               :
               : "v"(voffset), "s"(r), "s"(lds), "s"(soffset)
               : "memory", "m0");
}
__device__ __forceinline__ void dma4(const i32x4& r, uint32_t lds, uint32_t voffset, uint32_t soffset) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, %3 offen lds"
               :
               : "v"(voffset), "s"(r), "s"(lds), "s"(soffset)
               : "memory", "m0");
}

// A lane offset that must not read memory: every descriptor covers fewer
// than 2^31 bytes and every scalar offset is below 2^31, so the load falls
// out of range (and the sum does not wrap) and writes zeros.
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

}  // namespace dma
}  // namespace fp8q
