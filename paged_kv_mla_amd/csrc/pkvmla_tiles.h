// KV tile stream shared by the decode kernels: the producer walk over a
// workgroup's work units and the direct-to-LDS copies of one 32-token tile.
#ifndef PKVMLA_TILES_H_
#define PKVMLA_TILES_H_

#include "pkvmla_device.h"

namespace pkvmla {

// Index tables (schedule, page lists) are read through the constant address
// space: they never change while a kernel runs, and wave-uniform reads from it
// always become scalar loads (a vector load would have to be waited for with a
// vmcnt that also waits for the tile copies in flight).
#define PKVMLA_CONST_AS __attribute__((address_space(4)))
typedef const PKVMLA_CONST_AS int32_t* idx_ptr;

// Wait until at most n (wave-uniform, >= 0) of this wave's vector-memory
// operations are outstanding: the largest encodable count <= n, so the wait
// is never weaker than asked.  The counter holds at most 63 operations (issue
// stalls beyond), so 63 or more later operations imply completion.
__device__ __forceinline__ void wait_vm_le(int n) {
  if (n >= 63) return;
  if (n >= 54) wait_vmcnt<54>();
  else if (n >= 45) wait_vmcnt<45>();
  else if (n >= 36) wait_vmcnt<36>();
  else if (n >= 27) wait_vmcnt<27>();
  else if (n >= 18) wait_vmcnt<18>();
  else if (n >= 9) wait_vmcnt<9>();
  else wait_vmcnt<0>();
}

// Producer side of the tile stream: the unit and tile whose copies go out
// next.  All fields are wave-uniform (scalar registers).
struct TileStream {
  int u, u_end;           // unit of the next tile; end of the workgroup's list
  int tile, ntiles;       // tile index inside that unit, tiles in the unit
  int kv0, kv1;           // token range of the unit
  idx_ptr pages;          // page list of the unit's sequence
  int g;                  // stream position of the next tile
  int pid;                // page id of the next tile's first token (prefetched)
};

__device__ __forceinline__ void stream_load_unit(TileStream& s, idx_ptr units, idx_ptr seq_indptr,
                                                 idx_ptr seq_indices, int log2_ps) {
  idx_ptr rec = units + (size_t)s.u * kUnitInts;
  const int seq = rec[1];
  s.kv0 = rec[2];
  s.kv1 = rec[3];
  s.ntiles = (s.kv1 - s.kv0 + kTile - 1) / kTile;
  s.tile = 0;
  s.pages = seq_indices + seq_indptr[seq];
  s.pid = s.pages[s.kv0 >> log2_ps];
}

__device__ __forceinline__ void stream_advance(TileStream& s, idx_ptr units, idx_ptr seq_indptr,
                                               idx_ptr seq_indices, int log2_ps) {
  ++s.g;
  if (++s.tile < s.ntiles) {
    s.pid = s.pages[(s.kv0 + s.tile * kTile) >> log2_ps];
  } else if (++s.u < s.u_end) {
    stream_load_unit(s, units, seq_indptr, seq_indices, log2_ps);
  }
}

// Scalar description of one tile's copies, computed once per tile so that
// each copy instruction costs a few scalar operations.
struct TileCopy {
  const char* crow;       // BIG: ckv row of the tile's first token
  const char* krow;       // BIG: kpe row of the tile's first token
  idx_ptr pages;          // !BIG: page list, with tok0 and log2_ps below
  int tok0, last, log2_ps;
  uint32_t st;            // LDS stage base
  // BIG, whole tiles (last == kTile - 1): this wave's two ckv row groups and
  // its kpe block as ready scalar bases, so a copy needs no address arithmetic
  // (scalar ALU work between the MFMAs of the k-loop costs more than it looks:
  // about four clocks per instruction, in dependent chains)
  const char* g0;
  const char* g1;
  const char* kb;
  bool full;
};

__device__ __forceinline__ TileCopy tile_copy(const TileStream& s, const char* __restrict__ ckv,
                                              const char* __restrict__ kpe, int log2_ps,
                                              uint32_t stage_base, int wave) {
  TileCopy c;
  c.tok0 = s.kv0 + s.tile * kTile;
  c.last = min(s.kv1 - 1 - c.tok0, kTile - 1);
  c.log2_ps = log2_ps;
  c.pages = s.pages;
  c.st = stage_base;
  const int64_t rowbase = ((int64_t)(uint32_t)s.pid << log2_ps) + (c.tok0 & ((1 << log2_ps) - 1));
  c.crow = ckv + rowbase * (kCkvDim * 2);
  c.krow = kpe + rowbase * (kKpeDim * 2);
  c.full = c.last == kTile - 1;
  c.g0 = c.crow + (4 * wave) * (kCkvDim * 2);
  c.g1 = c.crow + (4 * wave + 16) * (kCkvDim * 2);
  c.kb = c.krow + (8 * wave) * (kKpeDim * 2);
  return c;
}

// The copies of a tile are four shares ("copy slots", one per wave of a
// four-wave workgroup, or two per copy wave of the role-split kernel).  The
// share of slot `wave`: the ckv rows
// t = 4*wave + j and t = 4*wave + j + 16 (j = 0..3; one 1 KB row per
// instruction) and the kpe block of tokens 8*wave .. 8*wave+7 (one instruction,
// 128 bytes per token).  The 16-byte chunks of a row are XOR-swizzled on the
// global side so they land in the LDS layout of pkvmla_device.h; rows t and
// t + 16 share their swizzle, so a wave needs four lane offsets for its ckv
// rows and one for its kpe block.  Those offsets live in registers that are
// never rewritten: a copy reads its address registers only when the CU's
// memory pipeline accepts it (about one copy every 23 clocks per CU), and a
// write to such a register before that stalls the wave.
// Tokens past kv_end copy the last valid ckv row (finite data whose
// probability is later zero: a NaN there would survive the zero weight).
// One M0 value serves four consecutive ckv rows: the instruction offset (0, 1,
// 2 or 3 KB) moves the LDS destination and the global source alike, and the
// scalar base of a row absorbs its page and its clamping.
// BIG: a page holds whole tiles (page_size >= 32), so one page id serves the
// tile and every address is a scalar base plus a lane offset.
constexpr int kCopyWaves = 4;
constexpr int kCopiesPerWave = kTile / kCopyWaves + 1;

struct CopyLanes {
  uint32_t v0, v1, v2, v3;  // ckv rows with swizzle 4*wave + j
  uint32_t vk;              // kpe block (the same for every wave)
};

__device__ __forceinline__ CopyLanes copy_lanes(int wave) {
  const uint32_t lane = (uint32_t)lane_id_fresh();
  const uint32_t w4 = (uint32_t)(4 * wave);
  CopyLanes L;
  L.v0 = (lane ^ (w4 + 0u)) << 4;
  L.v1 = (lane ^ (w4 + 1u)) << 4;
  L.v2 = (lane ^ (w4 + 2u)) << 4;
  L.v3 = (lane ^ (w4 + 3u)) << 4;
  // token 8*wave + lane/8 (swz8 = lane/8), chunk lane % 8
  L.vk = (lane >> 3) * (uint32_t)(kKpeDim * 2) + (((lane & 7u) ^ (lane >> 3)) << 4);
  return L;
}

// Copy part k (0..kCopiesPerWave-1) of this wave's share: parts 0..7 are the
// ckv rows (4*wave + k%4 + 16*(k/4)), part 8 the kpe block.  Parts must be
// issued in order with no other M0 user in between: M0 is loaded at parts 0,
// 4 and 8 only.
template <bool BIG>
__device__ __forceinline__ void tile_copy_part(const TileCopy& c, const char* __restrict__ ckv,
                                               const char* __restrict__ kpe, int wave, const int k,
                                               const CopyLanes& L) {
  const int ps_mask = (1 << c.log2_ps) - 1;
  auto row_of = [&](int t) -> int64_t {  // global row of tile token t (clamped), !BIG
    const int tok = c.tok0 + min(t, c.last);
    return ((int64_t)(uint32_t)c.pages[tok >> c.log2_ps] << c.log2_ps) + (tok & ps_mask);
  };
  if (k < 8) {
    const int j = k & 3;
    const int t0 = 4 * wave + 16 * (k >> 2);  // first row of the group of four
    const int t = t0 + j;
    if (j == 0) set_m0(c.st + (uint32_t)t0 * 1024u);
    // global source = base + voff + j KB: the base of row t is its own row
    // address minus j KB
    const char* rowp = BIG ? c.crow + (int64_t)min(t, c.last) * (kCkvDim * 2)
                           : ckv + row_of(t) * (kCkvDim * 2);
    const char* base = rowp - j * 1024;
    // (!BIG: the persistent offsets do not pay for their registers there)
    const CopyLanes& LL = BIG ? L : copy_lanes(wave);
    switch (j) {
      case 0: dma16_m0<0>(base, LL.v0); break;
      case 1: dma16_m0<1024>(base, LL.v1); break;
      case 2: dma16_m0<2048>(base, LL.v2); break;
      default: dma16_m0<3072>(base, LL.v3); break;
    }
  } else {
    set_m0(c.st + kTile * 1024 + (uint32_t)wave * 1024u);
    if constexpr (BIG) {
      // Units start on tile boundaries and a page holds whole tiles, so all
      // 32 kpe rows of the tile lie inside the tile's page; rows past kv_end
      // are copied unclamped (their scores are replaced by -inf with a select
      // before the softmax, so whatever they hold never reaches the output).
      dma16_m0<0>(c.krow + wave * 8 * (kKpeDim * 2), L.vk);
    } else {
      // lane group j = lane / 8 copies token 8*wave + j (clamped)
      const int lane = lane_id_fresh();
      const int tl = 8 * wave + (lane >> 3);
      const uint32_t kchunk = (uint32_t)(((lane & 7) ^ swz8(tl)) << 4);
      int64_t row = row_of(8 * wave);
#pragma unroll
      for (int kk = 1; kk < 8; ++kk) row = ((lane >> 3) == kk) ? row_of(8 * wave + kk) : row;
      dma16_m0v(kpe + row * (kKpeDim * 2) + kchunk);
    }
  }
}

// Part k of a whole tile's copies (BIG and full): ready bases, no clamping.
__device__ __forceinline__ void tile_copy_part_full(const TileCopy& c, int wave, const int k,
                                                    const CopyLanes& L) {
  if (k < 8) {
    const int j = k & 3;
    if (j == 0) set_m0(c.st + (uint32_t)(4 * wave + 16 * (k >> 2)) * 1024u);
    const char* base = k < 4 ? c.g0 : c.g1;
    switch (j) {
      case 0: dma16_m0<0>(base, L.v0); break;
      case 1: dma16_m0<1024>(base, L.v1); break;
      case 2: dma16_m0<2048>(base, L.v2); break;
      default: dma16_m0<3072>(base, L.v3); break;
    }
  } else {
    set_m0(c.st + kTile * 1024 + (uint32_t)wave * 1024u);
    dma16_m0<0>(c.kb, L.vk);
  }
}

template <bool BIG>
__device__ __forceinline__ void tile_copy_wave(const TileCopy& c, const char* __restrict__ ckv,
                                               const char* __restrict__ kpe, int wave,
                                               const CopyLanes& L) {
#pragma unroll
  for (int k = 0; k < kCopiesPerWave; ++k) tile_copy_part<BIG>(c, ckv, kpe, wave, k, L);
}

}  // namespace pkvmla

#endif  // PKVMLA_TILES_H_
