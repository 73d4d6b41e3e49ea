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
// Swizzles chosen by measuring LDS bank-conflict cycles on gfx950: with the
// chunk position c ^ (t mod 16) the QK operand reads (ds_read_b128: 16
// tokens, one chunk each) take 4 LDS cycles per instruction, the conflict-free
// minimum; the transposed V reads (ds_read_b64_tr_b16) then take 4 cycles
// instead of 2.  No XOR of this form serves both (the b128 reads want lanes
// 2k, 2k+1 on adjacent chunks, the transposed reads want 8 consecutive tokens
// on distinct chunk pairs), and QK moves 4.5x more bytes per tile than PV.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz16(int t) {
  return t & 15;
}
__device__ __forceinline__ int swz8(int t) {
  return t & 7;
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

// Copies with M0 already holding the LDS base: global address = sbase + voff +
// OFF and LDS address = M0 + OFF + 16 * lane (the instruction offset moves both
// sides).  set_m0 loads M0; the compiler itself never uses M0 in these
// kernels, so it stays valid between the copies of one tile.
__device__ __forceinline__ void set_m0(uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0" : : "s"(lds_base) : "memory");
}
template <int OFF>
__device__ __forceinline__ void dma16_m0(const void* sbase_any, uint32_t voff) {
  static_assert(OFF >= 0 && OFF < 4096, "instruction offset range");
  const void* sbase = to_sgpr(sbase_any);
  asm volatile("global_load_lds_dwordx4 %0, %1 offset:%2" : : "v"(voff), "s"(sbase), "i"(OFF) : "memory");
}
// Per-lane 64-bit address form with M0 already set (offset 0).
__device__ __forceinline__ void dma16_m0v(const void* gptr) {
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(gptr) : "memory");
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

// Timing runs: each workgroup stores its start and end on the 100 MHz
// real-time counter into its own pair of a launch's record (plain stores to
// distinct words, no atomics: a single word updated by every workgroup would
// itself delay the launch it measures).  One lane per workgroup.
__device__ __forceinline__ void stamp_start(unsigned long long* stamps) {
  if (stamps) stamps[2 * blockIdx.x] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ void stamp_end(unsigned long long* stamps) {
  if (stamps) stamps[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
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
