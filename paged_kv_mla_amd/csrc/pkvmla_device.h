// Device-side helpers shared by the decode, merge and gather kernels (gfx950).
#ifndef PKVMLA_DEVICE_H_
#define PKVMLA_DEVICE_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pkvmla_internal.h"

#define LDS_AS __attribute__((address_space(3)))

namespace pkvmla {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef __bf16 bf16x4_t __attribute__((__vector_size__(8)));
typedef float f32x4_t __attribute__((__vector_size__(16)));
typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));

// ---------------------------------------------------------------------------
// LDS tile layout (one stage, 36864 bytes):
//   [0, 32768)      ckv rows: token t at t*1024, its 16-byte chunk c (dims
//                   8c..8c+7) at chunk position c ^ swz16(t)
//   [32768, 36864)  kpe rows: token t at 32768 + t*128, chunk c at c ^ swz8(t)
// The XOR swizzles keep every MFMA operand read free of bank conflicts for
// both a 64-bank (16 lanes x 16 B or 32 lanes x 8 B per cycle) and a 32-bank
// LDS: 16 consecutive tokens reading one chunk cover all 16 16-byte slots of
// 256 bytes, and the transposed V reads (8 tokens x 2 chunks per 32 lanes)
// do too.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz16(int t) {
  return (((t >> 2) ^ (t >> 3)) & 1) | ((t & 7) << 1);
}
__device__ __forceinline__ int swz8(int t) {
  return (t ^ (t >> 3)) & 7;
}
__device__ __forceinline__ int lds_ckv_off(int t, int c) {
  return t * 1024 + ((c ^ swz16(t)) << 4);
}
__device__ __forceinline__ int lds_kpe_off(int t, int c) {
  return kTile * 1024 + t * 128 + ((c ^ swz8(t)) << 4);
}

// gfx9 s_waitcnt immediate: wait until at most N vector-memory ops are
// outstanding (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Direct HBM -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4) from
// a per-lane 64-bit address: lane i of the wave lands at LDS byte
// lds_base + 16*i.  Issued through inline asm so that the compiler neither
// reorders it nor inserts its own conservative vector-memory waits before
// every LDS read; completion is tracked explicitly with s_waitcnt vmcnt before
// the workgroup barrier that publishes a tile.  M0 (the LDS base register of
// the instruction) is saved and restored.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(gptr), "s"(lds_base)
      : "memory");
}

// A wave-uniform pointer moved to scalar registers (the value is the same in
// every lane; readfirstlane makes that explicit to the compiler).
__device__ __forceinline__ const void* to_sgpr(const void* ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}

// The same copy from a wave-uniform 64-bit base (SGPR pair) plus a 32-bit
// per-lane byte offset: the address arithmetic stays on the scalar unit.
// Both copies carry a memory clobber: no compiler-generated load or store
// moves across them, so the issue order of vector-memory operations (which
// the explicit vmcnt waits count) is the program order.
__device__ __forceinline__ void dma16_s(const void* sbase_any, uint32_t voff, uint32_t lds_base) {
  const void* sbase = to_sgpr(sbase_any);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory");
}

// Maximum over the four 16-lane rows (lanes l, l^16, l^32, l^48 hold one head)
// with the gfx950 row-swap permutes, which stay in the VALU.
__device__ __forceinline__ float max_over_rows(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float y = fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
  const uint32_t v = __builtin_bit_cast(uint32_t, y);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)b[0]), __builtin_bit_cast(float, (uint32_t)b[1]));
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Lane id computed afresh (volatile asm: never hoisted, merged or spilled).
// Code that runs once per work unit derives its lane constants from it, so
// they do not occupy registers through the hot loop or get spilled (a spill
// reload waits for every copy in flight).
__device__ __forceinline__ int lane_id_fresh() {
  int x;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
  return x;
}

// Workgroup barrier that orders LDS traffic (every LDS access of this wave has
// completed) without waiting for outstanding vector-memory loads: tile copies
// in flight keep flying across it.  The memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __syncthreads();
}

}  // namespace pkvmla

#endif  // PKVMLA_DEVICE_H_
