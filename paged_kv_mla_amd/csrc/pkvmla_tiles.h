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
};

__device__ __forceinline__ TileCopy tile_copy(const TileStream& s, const char* __restrict__ ckv,
                                              const char* __restrict__ kpe, int log2_ps,
                                              uint32_t stage_base) {
  TileCopy c;
  c.tok0 = s.kv0 + s.tile * kTile;
  c.last = min(s.kv1 - 1 - c.tok0, kTile - 1);
  c.log2_ps = log2_ps;
  c.pages = s.pages;
  c.st = stage_base;
  const int64_t rowbase = ((int64_t)(uint32_t)s.pid << log2_ps) + (c.tok0 & ((1 << log2_ps) - 1));
  c.crow = ckv + rowbase * (kCkvDim * 2);
  c.krow = kpe + rowbase * (kKpeDim * 2);
  return c;
}

// One wave's share of a tile's copies in a four-wave workgroup: ckv rows
// 8*wave .. 8*wave+7 (one 1 KB row per instruction, 16-byte chunks
// XOR-swizzled on the global side so they land in the LDS layout of
// pkvmla_device.h) and the kpe block of tokens 8*wave .. 8*wave+7 (one
// instruction, 128 bytes per token).  Tokens past kv_end copy the last valid
// row: every copied row is finite data whose probability is later set to zero.
// One M0 value serves four consecutive ckv rows: the instruction offset (0, 1,
// 2 or 3 KB) moves the LDS destination and the global source alike, and the
// scalar base of a row absorbs its page and its clamping.
// BIG: a page holds whole tiles (page_size >= 32), so one page id serves the
// tile and every address is a scalar base plus a lane offset.
constexpr int kCopyWaves = 4;
constexpr int kCopiesPerWave = kTile / kCopyWaves + 1;

template <bool BIG>
__device__ __forceinline__ void tile_copy_wave(const TileCopy& c, const char* __restrict__ ckv,
                                               const char* __restrict__ kpe, int wave) {
  constexpr int R = kTile / kCopyWaves;
  const int lane = lane_id_fresh();
  const int ps_mask = (1 << c.log2_ps) - 1;
  auto row_of = [&](int t) -> int64_t {  // global row of tile token t (clamped), !BIG
    const int tok = c.tok0 + min(t, c.last);
    return ((int64_t)(uint32_t)c.pages[tok >> c.log2_ps] << c.log2_ps) + (tok & ps_mask);
  };
#pragma unroll
  for (int k = 0; k < R; ++k) {
    const int t = R * wave + k;
    const int kq = k & 3;  // row within its group of four
    if (kq == 0) set_m0(c.st + (uint32_t)t * 1024u);
    const uint32_t voff = ((uint32_t)lane << 4) ^ (uint32_t)(swz16(t) << 4);
    // global source = base + voff + kq KB: the base of row t is its own row
    // address minus kq KB
    const char* rowp = BIG ? c.crow + (int64_t)min(t, c.last) * (kCkvDim * 2)
                           : ckv + row_of(t) * (kCkvDim * 2);
    const char* base = rowp - kq * 1024;
    switch (kq) {
      case 0: dma16_m0<0>(base, voff); break;
      case 1: dma16_m0<1024>(base, voff); break;
      case 2: dma16_m0<2048>(base, voff); break;
      default: dma16_m0<3072>(base, voff); break;
    }
  }
  const int tl = 8 * wave + (lane >> 3);  // this lane's kpe token
  const uint32_t kchunk = (uint32_t)(((lane & 7) ^ swz8(tl)) << 4);
  set_m0(c.st + kTile * 1024 + (uint32_t)wave * 1024u);
  if constexpr (BIG) {
    dma16_m0<0>(c.krow, (uint32_t)min(tl, c.last) * (kKpeDim * 2) + kchunk);
  } else {
    // lane group j = lane / 8 copies token 8*wave + j (clamped)
    int64_t row = row_of(8 * wave);
#pragma unroll
    for (int kk = 1; kk < 8; ++kk) row = ((lane >> 3) == kk) ? row_of(8 * wave + kk) : row;
    dma16_m0v(kpe + row * (kKpeDim * 2) + kchunk);
  }
}

}  // namespace pkvmla

#endif  // PKVMLA_TILES_H_
