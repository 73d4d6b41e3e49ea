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
// Slot tokens: ckv rows 4*wave + j and 4*wave + 16 + j (i = 0..7), kpe tokens
// 8*wave + k (i = 8..15).
__device__ __forceinline__ int slot_token(int wave, int i) {
  return i < 4 ? 4 * wave + i : i < 8 ? 4 * wave + 12 + i : 8 * wave + i - 8;
}

// Cache rows of a slot's 16 tokens, clamped to the tile's last valid token.
template <bool BIG>
__device__ __forceinline__ void slot_rows(const TileCopy& c, int wave, uint32_t* rows) {
  if constexpr (BIG) {
#pragma unroll
    for (int i = 0; i < 16; ++i) rows[i] = c.row0 + (uint32_t)min(slot_token(wave, i), c.last);  // one page
  } else {
    // all 16 page-id loads go out before the first use (one wait, not 16)
    const int ps_mask = (1 << c.log2_ps) - 1;
    uint32_t pid[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      pid[i] = (uint32_t)c.pages[(c.tok0 + min(slot_token(wave, i), c.last)) >> c.log2_ps];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      rows[i] = (pid[i] << c.log2_ps) + (uint32_t)((c.tok0 + min(slot_token(wave, i), c.last)) & ps_mask);
  }
}

template <bool BIG, bool PACKED>
__device__ __forceinline__ void tile_copy_slot(const TileCopy& c, const char* __restrict__ ckv,
                                               const char* __restrict__ kpe, int wave,
                                               const CopyLanes& L) {
  uint32_t rows[16];
  slot_rows<BIG>(c, wave, rows);
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

// ---------------------------------------------------------------------------
// fp8 (OCP E4M3) caches: a slot's share of a tile goes HBM -> registers ->
// bf16 -> LDS, into the same swizzled bf16 layout as the direct copies, so
// the QK and PV waves read the tile unchanged.  Every E4M3 value is exactly a
// bf16 value (3 mantissa bits, exponents 2^-9 .. 2^8), so the widening is
// exact; the caches' scales are applied in fp32 by the consumers.
// A slot's registers: its 8 ckv rows as four 16-byte loads (lanes 0..31 and
// 32..63 take rows 2i and 2i+1 of the slot, 16 codes each: bf16 chunks 2c
// and 2c+1 of the row) and its 8 kpe rows as one 8-byte load (lane l: token
// 8*wave + l/8, chunk l%8).  Row strides cs and ks are in bytes.
// ---------------------------------------------------------------------------
struct Fp8Slot {
  u32x4_t c[4];
  uint32_t k[2];
};

// Loads through the global address space: a generic (flat) load would also
// count on lgkmcnt, so the LDS-store wait before each barrier would wait for
// the next tile's loads too.
#define PKVMLA_GLOBAL_AS __attribute__((address_space(1)))
typedef const PKVMLA_GLOBAL_AS char* gchar_ptr;
__device__ __forceinline__ u32x4_t gload16(gchar_ptr p) {
  return *reinterpret_cast<const PKVMLA_GLOBAL_AS u32x4_t*>(p);
}
typedef uint32_t u32x2_t __attribute__((__vector_size__(8)));
__device__ __forceinline__ u32x2_t gload8(gchar_ptr p) {
  return *reinterpret_cast<const PKVMLA_GLOBAL_AS u32x2_t*>(p);
}

template <bool BIG>
__device__ __forceinline__ void fp8_slot_load(const TileCopy& c, const char* __restrict__ ckv,
                                              const char* __restrict__ kpe, int wave, Fp8Slot& r) {
  uint32_t rows[16];
  slot_rows<BIG>(c, wave, rows);
  const int lane = lane_id_fresh();
  const int half = lane >> 5, cl = lane & 31;
  const gchar_ptr gc = (gchar_ptr)ckv;
  const gchar_ptr gk = (gchar_ptr)kpe;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t row = half ? rows[2 * i + 1] : rows[2 * i];
    r.c[i] = gload16(gc + (size_t)row * c.cs + cl * 16);
  }
  const int g8 = lane >> 3;
  uint32_t row = rows[8];
#pragma unroll
  for (int k = 1; k < 8; ++k) row = g8 == k ? rows[8 + k] : row;
  const u32x2_t kv = gload8(gk + (size_t)row * c.ks + (lane & 7) * 8);
  r.k[0] = kv[0];
  r.k[1] = kv[1];
}

// Per-lane constants of one copy slot: the byte offsets of its loads from
// the tile's first ckv and kpe rows (whole tiles of one page: rows t at
// t * stride) and the LDS offsets (within a stage) of its bf16 chunks.
struct Fp8Lanes {
  uint32_t gc[4], gk;
  uint32_t lc[8], lk;
};

__device__ __forceinline__ Fp8Lanes fp8_lanes(int wave, int cs, int ks) {
  const int lane = lane_id_fresh();
  const int half = lane >> 5, cl = lane & 31;
  Fp8Lanes L;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = slot_token(wave, 2 * i + half);
    L.gc[i] = (uint32_t)(t * cs + cl * 16);
    L.lc[2 * i] = (uint32_t)lds_ckv_off(t, 2 * cl);
    L.lc[2 * i + 1] = (uint32_t)lds_ckv_off(t, 2 * cl + 1);
  }
  const int t = 8 * wave + (lane >> 3);
  L.gk = (uint32_t)(t * ks + (lane & 7) * 8);
  L.lk = (uint32_t)lds_kpe_off(t, lane & 7);
  return L;
}

// A whole tile of one page (BIG and full): scalar row bases plus the lane
// offsets, no clamping.
__device__ __forceinline__ void fp8_slot_load_full(const TileCopy& c, const Fp8Lanes& L, Fp8Slot& r) {
  const gchar_ptr crow = (gchar_ptr)to_sgpr(c.crow);
  const gchar_ptr krow = (gchar_ptr)to_sgpr(c.krow);
#pragma unroll
  for (int i = 0; i < 4; ++i) r.c[i] = gload16(crow + L.gc[i]);
  const u32x2_t kv = gload8(krow + L.gk);
  r.k[0] = kv[0];
  r.k[1] = kv[1];
}

// Four codes (one dword) to four bf16 (two dwords), exactly.
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t v) {
  const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false);
  const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

__device__ __forceinline__ void fp8_slot_store(LDS_AS char* stage, const Fp8Lanes& L,
                                               const Fp8Slot& r) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint2 a = fp8x4_to_bf16x4(r.c[i][0]), b = fp8x4_to_bf16x4(r.c[i][1]);
    const uint2 d = fp8x4_to_bf16x4(r.c[i][2]), e = fp8x4_to_bf16x4(r.c[i][3]);
    *(LDS_AS u32x4_t*)(stage + L.lc[2 * i]) = u32x4_t{a.x, a.y, b.x, b.y};
    *(LDS_AS u32x4_t*)(stage + L.lc[2 * i + 1]) = u32x4_t{d.x, d.y, e.x, e.y};
  }
  const uint2 a = fp8x4_to_bf16x4(r.k[0]), b = fp8x4_to_bf16x4(r.k[1]);
  *(LDS_AS u32x4_t*)(stage + L.lk) = u32x4_t{a.x, a.y, b.x, b.y};
}

}  // namespace pkvmla

#endif  // PKVMLA_TILES_H_
