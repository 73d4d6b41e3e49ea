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

// The unit record carries its page list's start and its first page id, so a
// unit's first copies wait for one load (the record), not three.
__device__ __forceinline__ void stream_load_unit(TileStream& s, idx_ptr units, idx_ptr seq_indices) {
  idx_ptr rec = units + (size_t)s.u * kUnitInts;
  s.kv0 = rec[2];
  s.kv1 = rec[3];
  s.ntiles = (s.kv1 - s.kv0 + kTile - 1) / kTile;
  s.tile = 0;
  s.pages = seq_indices + rec[6];
  s.pid = rec[7];
}

__device__ __forceinline__ void stream_advance(TileStream& s, idx_ptr units, idx_ptr seq_indices,
                                               int log2_ps) {
  ++s.g;
  if (++s.tile < s.ntiles) {
    s.pid = s.pages[(s.kv0 + s.tile * kTile) >> log2_ps];
  } else if (++s.u < s.u_end) {
    stream_load_unit(s, units, seq_indices);
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
  // its kpe block as ready scalar bases, so a copy needs at most one scalar
  // multiply-add (for a ckv row stride other than 1 KB)
  // (scalar ALU work between the MFMAs of the k-loop costs more than it looks:
  // about four clocks per instruction, in dependent chains)
  const char* g0;
  const char* g1;
  const char* kb;
  uint32_t row0;          // BIG: cache row of the tile's first token
  int cs, ks;             // row strides of the ckv and kpe caches, bytes
  bool full;
};

__device__ __forceinline__ TileCopy tile_copy(const TileStream& s, const char* __restrict__ ckv,
                                              const char* __restrict__ kpe, int log2_ps,
                                              uint32_t stage_base, int wave, int cs, int ks) {
  TileCopy c;
  c.tok0 = s.kv0 + s.tile * kTile;
  c.last = min(s.kv1 - 1 - c.tok0, kTile - 1);
  c.log2_ps = log2_ps;
  c.pages = s.pages;
  c.st = stage_base;
  const int64_t rowbase = ((int64_t)(uint32_t)s.pid << log2_ps) + (c.tok0 & ((1 << log2_ps) - 1));
  c.row0 = (uint32_t)rowbase;
  c.cs = cs;
  c.ks = ks;
  c.crow = ckv + rowbase * cs;
  c.krow = kpe + rowbase * ks;
  c.full = c.last == kTile - 1;
  c.g0 = c.crow + (int64_t)(4 * wave) * cs;
  c.g1 = c.crow + (int64_t)(4 * wave + 16) * cs;
  c.kb = c.krow + (int64_t)(8 * wave) * ks;
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

// ks: the kpe cache's row stride in bytes (128 for a [pages, page_size, 64]
// tensor, 1152 for the kpe view of a combined [pages, page_size, 576] one).
__device__ __forceinline__ CopyLanes copy_lanes(int wave, int ks) {
  const uint32_t lane = (uint32_t)lane_id_fresh();
  const uint32_t w4 = (uint32_t)(4 * wave);
  CopyLanes L;
  L.v0 = (lane ^ (w4 + 0u)) << 4;
  L.v1 = (lane ^ (w4 + 1u)) << 4;
  L.v2 = (lane ^ (w4 + 2u)) << 4;
  L.v3 = (lane ^ (w4 + 3u)) << 4;
  // token 8*wave + lane/8 (swz8 = lane/8), chunk lane % 8
  L.vk = (lane >> 3) * (uint32_t)ks + (((lane & 7u) ^ (lane >> 3)) << 4);
  return L;
}

// One copy slot's share of a tile that is not one ready block of rows (page
// size below 32, or a unit's partial last tile): the cache rows of the slot's
// 8 ckv tokens (4*wave + j and 4*wave + 16 + j) and 8 kpe tokens (8*wave + k)
// are resolved first, clamped to the last valid token, in one batch of scalar
// page-id loads with one wait; then its 9 copies go out (M0 loaded three
// times, as in the whole-tile path).
// PACKED: the caches' rows are 1 KB (ckv) and 128 B (kpe) apart, so row
// addresses are shifts; otherwise they take the runtime strides.
template <bool BIG, bool PACKED>
__device__ __forceinline__ void tile_copy_slot(const TileCopy& c, const char* __restrict__ ckv,
                                               const char* __restrict__ kpe, int wave,
                                               const CopyLanes& L) {
  // slot tokens: ckv rows 4*wave + j, 4*wave + 16 + j; kpe tokens 8*wave + k
  auto tok_of = [&](int i) { return i < 4 ? 4 * wave + i : i < 8 ? 4 * wave + 12 + i : 8 * wave + i - 8; };
  uint32_t rows[16];
  if constexpr (BIG) {
#pragma unroll
    for (int i = 0; i < 16; ++i) rows[i] = c.row0 + (uint32_t)min(tok_of(i), c.last);  // one page
  } else {
    // all 16 page-id loads go out before the first use (one wait, not 16)
    const int ps_mask = (1 << c.log2_ps) - 1;
    uint32_t pid[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) pid[i] = (uint32_t)c.pages[(c.tok0 + min(tok_of(i), c.last)) >> c.log2_ps];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      rows[i] = (pid[i] << c.log2_ps) + (uint32_t)((c.tok0 + min(tok_of(i), c.last)) & ps_mask);
  }
  const uint32_t* rc = rows;
  const uint32_t* rk = rows + 8;
  // ckv: the source of row t is its row address; the copy's instruction
  // offset (j KB) moves source and LDS destination alike, so the base is
  // the row address minus j KB
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    set_m0(c.st + (uint32_t)(4 * wave + 16 * g) * 1024u);
    const size_t cs = PACKED ? (size_t)(kCkvDim * 2) : (size_t)c.cs;
    dma16_m0<0>(ckv + (size_t)rc[4 * g + 0] * cs, L.v0);
    dma16_m0<1024>(ckv + (size_t)rc[4 * g + 1] * cs - 1024, L.v1);
    dma16_m0<2048>(ckv + (size_t)rc[4 * g + 2] * cs - 2048, L.v2);
    dma16_m0<3072>(ckv + (size_t)rc[4 * g + 3] * cs - 3072, L.v3);
  }
  // kpe: lane group g8 = lane / 8 copies token 8*wave + g8 (chunk swizzle
  // g8, since 8*wave is a multiple of 8)
  set_m0(c.st + kTile * 1024 + (uint32_t)wave * 1024u);
  const int lane = lane_id_fresh();
  const int g8 = lane >> 3;
  uint32_t row = rk[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) row = g8 == k ? rk[k] : row;
  const uint32_t kchunk = (uint32_t)(((lane & 7) ^ g8) << 4);
  dma16_m0v(kpe + (size_t)row * (PACKED ? (size_t)(kKpeDim * 2) : (size_t)c.ks) + kchunk);
}

// Part k of a whole tile's copies (BIG and full): ready bases, no clamping.
__device__ __forceinline__ void tile_copy_part_full(const TileCopy& c, int wave, const int k,
                                                    const CopyLanes& L) {
  if (k < 8) {
    const int j = k & 3;
    if (j == 0) set_m0(c.st + (uint32_t)(4 * wave + 16 * (k >> 2)) * 1024u);
    // row 4*wave + 16*(k/4) + j sits j row strides past the group's base; the
    // instruction offset adds j KB, so the base takes j * (stride - 1 KB)
    const char* base = (k < 4 ? c.g0 : c.g1) + (int64_t)j * (c.cs - 1024);
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

}  // namespace pkvmla

#endif  // PKVMLA_TILES_H_
