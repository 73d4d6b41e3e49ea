// Fused absorbed-MLA decode kernel with split wave roles, for 64 and 128 query
// heads on gfx950.
//
// A workgroup of ten waves keeps 64 query heads of its work units (split-KV
// segments: a token range [kv_begin, kv_end) of one request's page list); at
// 128 heads two workgroups, one per head group, walk the same token ranges on
// the same XCD, so each KV tile comes from HBM once and from L2 the second
// time.  The waves split by role:
//   QK waves (0..3)  wave r holds Q for heads 16r..16r+15 and computes
//                    S^T[token, head] = K[token, 576] . Q^T[576, head] with
//                    MFMA 16x16x32 bf16 (K from LDS), then the softmax of those
//                    heads (running max m, running sum l), and publishes
//                    P^T[token, head] in bf16 and the rescale factors in LDS;
//   PV waves (4..7)  wave 4+r accumulates O^T[dim, head] += V^T[dim, token] .
//                    P^T[token, head] for dims 128r..128r+127 and all 64 heads
//                    (128 accumulator registers), one tile behind the QK waves,
//                    and writes the unit's output rows;
//   copy waves (8, 9) issue the HBM -> LDS copies of the KV tiles (direct
//                    LDS loads), each half of every tile.
// A copy instruction holds its wave until the CU's memory pipeline accepts it
// (about one 1 KB copy every 23 clocks per CU, 36 per tile), so copies issued
// from a computing wave stall its MFMAs; the copy waves take that wait
// instead.  Ten waves put three on two of the SIMDs, so every wave gets at
// most 168 registers (the PV waves' 128 accumulators fit with a V prefetch
// depth of two).
//
// Pipeline.  A first barrier follows the copy waves' issue of tile 0 (the QK
// waves load their queries only then, so those loads do not delay the tile),
// a second one tile 0's landing.  Then iteration i runs QK and softmax of
// tile i on the QK waves and PV of tile i-1 (with the epilogue when tile i-1
// ends a unit) on the PV waves, while the copy waves issue tile i+2 right
// after the barrier and then wait, with an exact s_waitcnt vmcnt, until their
// share of tile i+1 has landed; then one barrier.  The PV waves write no LDS,
// so they enter that barrier without waiting for their own reads: the first V
// fragments of their next tile (landed, and resident two more iterations) are
// read before it and arrive while the waves wait there.  KV tiles of 32 tokens
// live in a 4-stage LDS ring (two tiles in flight), P^T and the per-head
// factors in two-deep exchange buffers.  A copy wave keeps at most two tiles'
// shares (36 operations) in flight: the vmcnt counter holds at most 63, and a
// wave with more outstanding cannot wait for them exactly.
//
// At 16 and 32 heads (bf16 caches) progress counters in LDS replace the
// per-tile barrier, and each role waits only for what its next step needs:
// a copy wave publishes the tiles whose share has landed (after its exact
// vmcnt wait) and refills a stage once the PV waves have finished the tile
// four back; a QK wave scores tile i once it has landed and writes P^T into
// an exchange buffer once the PV waves have finished tile i-2 (the same
// parity), then publishes i+1; a PV wave takes tile t once every QK wave has
// published it and the next tile has landed, and publishes t+1 once its
// reads have returned.  Every dependency points at strictly earlier work,
// and every wait is bounded.  At 64 heads the PV waves' registers leave no
// room for the waits (the variant spilled), and the barrier stays.
//
// Row-block units (the level-0 launch of a cascade plan).  The 64 rows of a
// workgroup are then not the heads of one request but 64 consecutive query
// rows rho = b * H + head of a prefix group (four requests at 16 heads, two at
// 32, one at 64, half of one at 128), all scoring the same shared-prefix tile
// from LDS.  Such a unit's record holds the block's first row, the offset of
// its rows in the partial-state rows (rho + offset) and the end of the
// group's rows in place of request, slot and gathered-row index; its rows
// always write partial states, which the merge combines with the suffix's.
// The same units serve several new query tokens per request (16 or 32 heads):
// the 64 rows are t * H + head of 4 or 2 tokens of one request over its own
// pages, each QK wave's 16 rows the heads of one token t, masked at that
// token's causal bound (positions below t + the record's second field); a
// block the schedule left whole writes out and lse itself (slot kRowsDirect).
//
// Masking.  Only the last tile of a unit can be partial, except in row blocks
// of query tokens, where a wave's token may see a tile partly or not at all.
// A partial tile's ckv slots past kv_end copy the last valid row (finite
// data), its kpe slots the page's own rows; the QK waves set the scores of
// slots they may not see to -inf (a select) before the softmax, so they add
// exactly zero to PV.

#include <hip/hip_runtime.h>
#include <math.h>

#include "pkvmla_tiles.h"

namespace pkvmla {

namespace {

// A workgroup holds HB head blocks of 16 heads (HB = 1, 2 or 4): HB QK waves,
// kRsPvWaves PV waves, kRsCopyWaves copy waves.
constexpr int kRsPvWaves = 4;
constexpr int kRsCopyWaves = 2;
constexpr int kRsMaxHB = 4;
// fp8 caches: four copy waves (one per SIMD: their loads, widening and LDS
// stores are VALU work), one copy slot each
constexpr int kRsCopyWavesFp8 = 4;
__host__ __device__ constexpr int rs_threads(int hb, bool fp8 = false) {
  return (hb + kRsPvWaves + (fp8 ? kRsCopyWavesFp8 : kRsCopyWaves)) * 64;
}
constexpr int kRsRing = 4;     // LDS stages: PV tile, QK tile, two tiles in flight
constexpr int kRsAhead = 2;    // k-steps between a K fragment's LDS read and its MFMA
constexpr int kRsVAhead = 2;   // dim blocks between a V fragment's LDS read and its MFMAs
                               // (two: the register budget at ten waves, HB = 4)
constexpr int kRsDBW = 8;      // output-dim blocks of 16 per PV wave (128 dims)
static_assert(kCopyWaves == 2 * kRsCopyWaves, "each copy wave issues two copy slots' shares");
// A copy wave keeps at most (kRsRing - 2) tiles of its two slots' copies in
// flight.  The vmcnt counter of a wave holds at most 63 operations: with more
// outstanding, an exact s_waitcnt (including the last one before the
// workgroup retires) no longer covers every copy still writing LDS.
static_assert((kRsRing - 2) * 2 * kCopiesPerWave < 64, "copies in flight exceed the vmcnt range");

// LDS layout
constexpr int kXpOff = kRsRing * kStageBytes;         // P^T exchange: [parity][hb] 1 KB blocks
constexpr int kXaOff = kXpOff + 2 * kRsMaxHB * 1024;  // rescale factors: [parity][li][hb] floats
constexpr int kXlOff = kXaOff + 2 * 64 * 4;        // unit row sums:   [parity][li][hb] floats
// progress counters (bf16 caches): tiles landed per copy wave, tiles whose
// P^T is published per QK wave, tiles finished per PV wave
constexpr int kLandedOff = kXlOff + 2 * 64 * 4;
constexpr int kReadyOff = kLandedOff + 4 * kRsCopyWaves;
constexpr int kDoneOff = kReadyOff + 4 * kRsMaxHB;
constexpr int kRsLds = kDoneOff + 4 * kRsPvWaves;
static_assert(kRsLds <= 160 * 1024, "LDS budget");

// Bounded wait until each of the n LDS counters c[0..n-1] holds at least
// target; false when the wave gave up after `limit` polls (the plan's wait
// limit, 2^20 by default: about 0.1 s).  A QK or PV wave whose wait gave up
// writes NaN for every unit it finishes afterwards, so a protocol error ends
// the workgroup and shows as non-finite results, never as a workgroup that
// does not end or as plausible wrong values (a stalled copy wave stalls the
// QK and PV waves' waits in turn).
template <int N>
__device__ __forceinline__ bool counters_reach(const volatile LDS_AS int* c, int target) {
  int m = c[0];
#pragma unroll
  for (int j = 1; j < N; ++j) m = min(m, c[j]);
  return __builtin_amdgcn_readfirstlane(m) >= target;
}
template <int N>
__device__ __forceinline__ bool wait_counters(const volatile LDS_AS int* c, int target, int limit) {
  // the first poll straight-line (it usually succeeds), the loop only after it
  bool ok = limit > 0 && counters_reach<N>(c, target);
  if (!ok) {
    for (int it = 1; it < limit; ++it) {
      __builtin_amdgcn_s_sleep(1);
      if (counters_reach<N>(c, target)) {
        ok = true;
        break;
      }
    }
  }
  asm volatile("" ::: "memory");  // no LDS access moves above the wait
  return ok;
}
// Publishes v in the wave's counter once all of the wave's LDS accesses
// issued so far have completed (their data written, or read out).
__device__ __forceinline__ void publish_counter(volatile LDS_AS int* c, int v) {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt open
  asm volatile("" ::: "memory");
  *c = v;
}

// Unit cursor: the unit and tile a role is at, with the unit's fields.  For
// a row-block unit, b is its first query row, slot the offset of its rows in
// the partial-state rows, and rend the end of its group's rows.  A unit whose
// slot is kChainNext hands its softmax state to the next unit of the list
// (the same request's rows over another sequence): it writes nothing, and the
// next unit (cont) starts from its running max, row sums and outputs.
struct UnitCursor {
  int u;        // unit index
  int tile;     // tile index within the unit
  int ntiles;   // tiles in the unit
  int b, kv0, kv1, slot, rend;
  int caus;     // row blocks of query tokens: token t sees positions below t + caus
  bool cont;    // this unit continues the previous one's state
};

__device__ __forceinline__ void cursor_load(UnitCursor& c, idx_ptr units) {
  idx_ptr rec = units + (size_t)c.u * kUnitInts;
  c.b = rec[0];
  c.caus = rec[1];
  c.kv0 = rec[2];
  c.kv1 = rec[3];
  c.slot = rec[4];
  c.rend = rec[5];
  c.ntiles = (c.kv1 - c.kv0 + kTile - 1) / kTile;
  c.tile = 0;
}

__device__ __forceinline__ void cursor_next(UnitCursor& c, idx_ptr units, int u_end) {
  if (++c.tile >= c.ntiles) {
    c.cont = c.slot == kChainNext;
    if (++c.u < u_end) cursor_load(c, units);
  }
}

}  // namespace

// PACKED: the caches are packed [pages, page_size, 512] and [.., 64] tensors
// (row strides 1 KB and 128 B, compile-time constants); otherwise the row
// strides cs_arg and ks_arg (bytes) apply, e.g. the two views of one
// [pages, page_size, 576] cache.  ROWS: the units are row blocks (above).
// FP8: the caches hold OCP E4M3 codes (row strides in bytes); the copy waves
// widen each tile to bf16 in LDS, the score is ckv part + kpe_ratio * kpe
// part (kpe_ratio = kpe scale / ckv scale; the ckv scale is folded into
// sm_scale by the host) and the output rows take v_scale (the ckv scale).
template <bool BIG, int HB, bool PACKED, bool ROWS, bool FP8>
__global__ void __launch_bounds__(rs_threads(HB, FP8), 1)
mla_decode_rs_kernel(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
                     const uint16_t* __restrict__ ckv_cache, const uint16_t* __restrict__ kpe_cache,
                     uint16_t* __restrict__ out, float* __restrict__ lse_out,
                     uint16_t* __restrict__ part_o, float* __restrict__ part_lse,
                     const int32_t* __restrict__ wg_indptr_g, const int32_t* __restrict__ units_g,
                     const int32_t* __restrict__ seq_indices_g, int H, int n_hg, int n_lanes,
                     int log2_ps, float sm_scale, float C, float thr, int cs_arg,
                     int ks_arg, unsigned long long* stamps, float v_scale, float kpe_ratio,
                     int qo_log2h, int wait_limit) {
  const int cs = PACKED ? kCkvDim * 2 : cs_arg;
  const int ks = PACKED ? kKpeDim * 2 : ks_arg;
  // the two table pointers are read from the kernel arguments up front, with
  // the others, not in a dependent round trip just before their first use
  const int32_t* wgp = wg_indptr_g;
  const int32_t* unp = units_g;
  asm volatile("" : "+s"(wgp), "+s"(unp));
  const idx_ptr wg_indptr = (idx_ptr)wgp;
  const idx_ptr units = (idx_ptr)unp;
  const idx_ptr seq_indices = (idx_ptr)seq_indices_g;
  __shared__ __attribute__((aligned(1024))) char smem_raw[kRsLds];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;

  constexpr int HEADS = 16 * HB;  // heads per workgroup
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // QK waves 0..HB-1 (r: head block), PV waves HB..HB+3 (r: dim quarter),
  // then the copy waves
  const int r = wave < HB ? wave : wave - HB;
  // Block -> (head group, lane): the head groups of one lane are 8 blocks
  // apart, which the dispatcher places on the same XCD.
  const int hg = (int)(blockIdx.x >> 3) % n_hg;
  const int sl = (int)(blockIdx.x / (8 * n_hg)) * 8 + (int)(blockIdx.x & 7);
  // timing runs: workgroup start and end (wave 0 ends after the final
  // barrier, which every wave of the workgroup passes)
  const bool stamp_lane = stamps && threadIdx.x == 0;
  if (stamp_lane) stamp_start(stamps);
  if (sl >= n_lanes || wg_indptr[sl] >= wg_indptr[sl + 1]) {
    if (stamp_lane) stamp_end(stamps);
    return;
  }
  const int u_begin = wg_indptr[sl];
  const int u_end = wg_indptr[sl + 1];
  const char* ckv = reinterpret_cast<const char*>(ckv_cache);
  const char* kpe = reinterpret_cast<const char*>(kpe_cache);

  // 16 and 32 heads with bf16 caches: the roles synchronise through the
  // progress counters (each waits only for what its next step reads or
  // overwrites); 64 heads, and fp8 caches: one workgroup barrier per tile
  // (at 64 heads the PV waves' registers leave no room for the waits)
  constexpr bool FLAGS = !FP8 && HB < 4;
  volatile LDS_AS int* landed = (volatile LDS_AS int*)(smem + kLandedOff);
  volatile LDS_AS int* ready = (volatile LDS_AS int*)(smem + kReadyOff);
  volatile LDS_AS int* done = (volatile LDS_AS int*)(smem + kDoneOff);
  bool waits_ok = true;  // (counters) every wait of this wave so far succeeded
  // Tiles of the workgroup (with barriers every role runs the same number).
  // The first four units' bounds are loaded together (indices clamped to the
  // last unit, so every load is in the table; the empty asm keeps the compiler
  // from sinking each load into its own conditional), one round trip where a
  // loop would take one per unit.
  int G = 0;
  {
    int kb[4], ke[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      idx_ptr rec = units + (size_t)min(u_begin + k, u_end - 1) * kUnitInts;
      kb[k] = rec[2];
      ke[k] = rec[3];
    }
    asm volatile("" : "+s"(kb[0]), "+s"(ke[0]), "+s"(kb[1]), "+s"(ke[1]), "+s"(kb[2]), "+s"(ke[2]),
                 "+s"(kb[3]), "+s"(ke[3]));
#pragma unroll
    for (int k = 0; k < 4; ++k) G += u_begin + k < u_end ? (ke[k] - kb[k] + kTile - 1) / kTile : 0;
  }
  for (int u = u_begin + 4; u < u_end; ++u) {
    idx_ptr rec = units + (size_t)u * kUnitInts;
    G += (rec[3] - rec[2] + kTile - 1) / kTile;
  }

  if (wave < HB) {
    // ======================= QK and softmax role =======================
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int li = lane & 15;
    const int head = hg * HEADS + r * 16 + li;
    // the query row of this lane in a unit (rows past a row block's group
    // load the group's last row and write nothing)
    auto q_row = [&](int b, int rend) -> int {
      return ROWS ? min(b + hg * HEADS + r * 16 + li, rend - 1) : b * H + head;
    };
    int offA[2], offK[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      offA[tb] = lds_ckv_off(tb * 16 + li, g);
      offK[tb] = lds_kpe_off(tb * 16 + li, g);
    }
    UnitCursor cq;
    cq.u = u_begin;
    cq.cont = false;
    cursor_load(cq, units);
    // the unit's query: lane (g, li) holds Q[head][ks*32 + g*8 .. +7]
    bf16x8_t q[18];
    auto load_q = [&](int row) {
      const char* qn = reinterpret_cast<const char*>(q_nope + (size_t)row * kCkvDim);
      const char* qp = reinterpret_cast<const char*>(q_pe + (size_t)row * kKpeDim);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks)
        q[ks] = *reinterpret_cast<const bf16x8_t*>(qn + (ks * 32 + g * 8) * 2);
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2)
        q[16 + k2] = *reinterpret_cast<const bf16x8_t*>(qp + (k2 * 32 + g * 8) * 2);
    };
    if (FLAGS) ready[r] = 0;
    // the query loads go out after the copy waves have issued tile 0, so that
    // tile's copies do not queue behind them in the memory pipeline
    lds_barrier();
    load_q(q_row(cq.b, cq.rend));
    float m_run = -INFINITY, l_run = 0.f;

    if (!FLAGS) lds_barrier();  // tile 0 has landed
    int land_seen = 0;  // landed tiles, as last read
    for (int i = 0; i <= G; ++i) {
      if (i < G) {
        // tile i has landed (usually known from the read during the last
        // tile's softmax)
        if (FLAGS && land_seen < i + 1)
          waits_ok &= wait_counters<kRsCopyWaves>(landed, i + 1, wait_limit);
        const int stage = i % kRsRing;
        const int par = i & 1;
        if (cq.tile == 0 && !cq.cont) {
          m_run = -INFINITY;
          l_run = 0.f;
        }
        // ---- QK: S^T = K . Q^T, 18 k-steps x 2 token blocks ----
        const int so = stage * kStageBytes;
        int oA0 = offA[0], oA1 = offA[1], oK0 = offK[0], oK1 = offK[1];
        asm volatile("" : "+v"(oA0), "+v"(oA1), "+v"(oK0), "+v"(oK1));
        auto ldA = [&](int ks, int tb) -> bf16x8_t {
          const int base = tb ? (ks < 16 ? oA1 : oK1) : (ks < 16 ? oA0 : oK0);
          const int off = ks < 16 ? ((so + base) ^ (ks << 6)) : ((so + base) ^ ((ks - 16) << 6));
          return *(const LDS_AS bf16x8_t*)(smem + off);
        };
        // The k-loop runs at raised issue priority: when both waves of a SIMD
        // have an MFMA ready the QK wave's goes first, so its softmax (VALU)
        // overlaps the PV wave's MFMAs instead of following them.  Each K
        // fragment is read AH k-steps ahead (the scheduling barriers keep the
        // compiler from sinking the reads next to their MFMAs).
        __builtin_amdgcn_s_setprio(3);
        constexpr int AH = kRsAhead;
        bf16x8_t A[AH + 1][2];
#pragma unroll
        for (int pp = 0; pp < AH; ++pp) {
          A[pp][0] = ldA(pp, 0);
          A[pp][1] = ldA(pp, 1);
        }
        f32x4_t acc[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
        // (FP8: the two kpe k-steps accumulate apart, to take their own scale)
        f32x4_t acck[2] = {f32x4_t{0.f, 0.f, 0.f, 0.f}, f32x4_t{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int ks = 0; ks < 18; ++ks) {
          if (ks + AH < 18) {
            A[(ks + AH) % (AH + 1)][0] = ldA(ks + AH, 0);
            A[(ks + AH) % (AH + 1)][1] = ldA(ks + AH, 1);
          }
#pragma unroll
          for (int tb = 0; tb < 2; ++tb) {
            if (FP8 && ks >= 16)
              acck[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[ks % (AH + 1)][tb], q[ks], acck[tb], 0, 0, 0);
            else
              acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[ks % (AH + 1)][tb], q[ks], acc[tb], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        __builtin_amdgcn_s_setprio(0);
        // Q of the next unit goes out once the last k-step has read this
        // unit's, so its latency hides behind the softmax and the barrier
        if (cq.tile == cq.ntiles - 1 && cq.u + 1 < u_end && cq.slot != kChainNext) {
          idx_ptr nrec = units + (size_t)(cq.u + 1) * kUnitInts;
          load_q(q_row(nrec[0], ROWS ? nrec[5] : 0));
        }
        if (FLAGS) land_seen = min(landed[0], landed[1]);
        // ---- softmax of this tile: lane (g, li) holds tokens tb*16 + g*4 + k ----
        // tokens of the tile this wave's rows see: the unit's end, and in
        // row blocks of query tokens the causal bound of the wave's token (its
        // 16 rows are heads of one token); 0 or less: none (a whole tile
        // masked, possible only in row blocks)
        int kv_lim = cq.kv1;
        if (ROWS && qo_log2h >= 0) kv_lim = min(kv_lim, ((cq.b + hg * HEADS + r * 16) >> qo_log2h) + cq.caus);
        const int valid = min(kv_lim - (cq.kv0 + cq.tile * kTile), kTile);
        float sv[8];
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int k = 0; k < 4; ++k) sv[tb * 4 + k] = FP8 ? fmaf(kpe_ratio, acck[tb][k], acc[tb][k]) : acc[tb][k];
        if (valid < kTile) {  // a unit's partial last tile (uniform branch)
#pragma unroll
          for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int k = 0; k < 4; ++k)
              sv[tb * 4 + k] = tb * 16 + g * 4 + k < valid ? sv[tb * 4 + k] : -INFINITY;
        }
        float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        mx = fmaxf(mx, fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
        mx = max_over_rows(mx);
        // lazy running max: m moves only when the tile max exceeds it by more
        // than thr (probabilities stay <= 2^thr*C); the first tile always sets it
        const bool grow = mx > m_run + thr;
        const float m_new = grow ? mx : m_run;
        // (row blocks: a row may see nothing yet, m stays -inf; the factor is
        // then 0, as on any unit's first tile, and the probabilities 0)
        const float alpha = ROWS && m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * C);
        m_run = m_new;
        const float mc = ROWS && m_run == -INFINITY ? 0.f : m_run * C;
        float pv[8];
        bf16x8_t pT;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          pv[k] = __builtin_amdgcn_exp2f(fmaf(sv[k], C, -mc));
          pT[k] = (__bf16)pv[k];
        }
        // the lane's share of the row sum as a tree (depth 3, not 8)
        const float ps = ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
        l_run = l_run * alpha + ps;
        // the exchange buffers of this parity held tile i-2's: the PV waves
        // have read them once they have finished tile i-2
        if (FLAGS && i >= 2) waits_ok &= wait_counters<kRsPvWaves>(done, i - 1, wait_limit);
        *(LDS_AS bf16x8_t*)(smem + kXpOff + (par * kRsMaxHB + r) * 1024 + lane * 16) = pT;
        if (g == 0) *(LDS_AS float*)(smem + kXaOff + (par * 64 + li * 4 + r) * 4) = alpha;
        if (cq.tile == cq.ntiles - 1 && cq.slot != kChainNext) {
          // unit done: row sums for the PV waves, lse for the output
          float l = l_run;
          l += __shfl_xor(l, 16);
          l += __shfl_xor(l, 32);
          float lse = m_run * sm_scale + __builtin_amdgcn_logf(l) * 0.69314718055994531f;
          if (FLAGS && !waits_ok) lse = __builtin_nanf("");
          if (g == 0) {
            *(LDS_AS float*)(smem + kXlOff + (par * 64 + li * 4 + r) * 4) = l;
            if (ROWS) {
              const int row = cq.b + hg * HEADS + r * 16 + li;
              if (row < cq.rend) {
                if (cq.slot == kRowsDirect) lse_out[row] = lse;
                else part_lse[cq.slot + row] = lse;
              }
            } else if (cq.slot < 0) {
              lse_out[(size_t)cq.b * H + head] = lse;
            } else {
              part_lse[(size_t)cq.slot * H + head] = lse;
            }
          }
        }
        if (FLAGS) {
          publish_counter(ready + r, i + 1);
          land_seen = __builtin_amdgcn_readfirstlane(land_seen);
        }
        cursor_next(cq, units, u_end);
      }
      if (!FLAGS) lds_barrier();
    }
    if (!FLAGS && stamp_lane) stamp_end(stamps);
  } else if (wave < HB + kRsPvWaves) {
    // ======================= PV and epilogue role =======================
    const int lane0 = threadIdx.x & 63;
    const int g0 = lane0 >> 4;
    const int li0 = lane0 & 15;
    int offV[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      const int tV = tb * 16 + g0 * 4 + (li0 >> 2);
      const int qq = li0 & 3;
      offV[tb] = lds_ckv_off(tV, qq >> 1) + (qq & 1) * 8;
    }
    if (FLAGS) done[r] = 0;
    lds_barrier();  // tile 0's copies are out
    if (!FLAGS) lds_barrier();  // tile 0 has landed

    UnitCursor cp;
    cp.u = u_begin;
    cp.cont = false;
    cursor_load(cp, units);
    // O (128 VGPRs, MFMAs in VGPR form) starts at zero once.  A tile whose
    // rescale factors are not all 1 multiplies O by them before its MFMAs
    // (rare: the running max moves only in steps of more than the threshold);
    // the factors are exactly 0 on a unit's first tile (the running max
    // starts at -inf), which clears the previous unit.
    f32x4_t o[kRsDBW][HB];
#pragma unroll
    for (int db = 0; db < kRsDBW; ++db)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) o[db][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // ---- iteration 0: the QK waves take tile 0 ----
    if (!FLAGS) lds_barrier();
    constexpr int VP = kRsVAhead;
    int oV0 = offV[0], oV1 = offV[1];
    asm volatile("" : "+v"(oV0), "+v"(oV1));
    auto ldV = [&](int so, int db, int tb) -> bf16x4_t {
      const int dbg = r * kRsDBW + db;
      return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
          (LDS_AS bf16x4_t*)(smem + ((so + (tb ? oV1 : oV0)) ^ (dbg << 5))));
    };
    // the first dim block's V fragments of the next tile, read before the
    // barrier that starts its iteration (one block: the register budget)
    if (FLAGS) waits_ok &= wait_counters<kRsCopyWaves>(landed, 1, wait_limit);
    bf16x4_t vn0 = ldV(0, 0, 0), vn1 = ldV(0, 0, 1);

    // ---- iteration t+1: PV of tile t, copies of tile t+3 ----
    for (int t = 0; t < G; ++t) {
      const int stage = t % kRsRing;
      const int par = t & 1;
      if (FLAGS) {
        // P^T of tile t is published, and tile t+1 has landed (its first V
        // block is read after this tile's MFMAs; the QK waves need it now)
        waits_ok &= wait_counters<HB>(ready, t + 1, wait_limit);
        if (t + 1 < G) waits_ok &= wait_counters<kRsCopyWaves>(landed, t + 2, wait_limit);
      }
      const int lane = lane_id_fresh();
      bf16x8_t pB[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb)
        pB[hb] = *(const LDS_AS bf16x8_t*)(smem + kXpOff + (par * kRsMaxHB + hb) * 1024 + lane * 16);
      const f32x4_t a4 = *(const LDS_AS f32x4_t*)(smem + kXaOff + (par * 64 + (lane & 15) * 4) * 4);
      bool need = false;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) need |= a4[hb] != 1.0f;
      const bool rescale = __builtin_amdgcn_ballot_w64(need) != 0;
      __builtin_amdgcn_sched_barrier(0);
      const int so = stage * kStageBytes;
      if (rescale) {
#pragma unroll
        for (int db = 0; db < kRsDBW; ++db)
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) o[db][hb] *= a4[hb];
      }
      {
        bf16x4_t V[VP + 1][2];
        V[0][0] = vn0;
        V[0][1] = vn1;
#pragma unroll
        for (int pp = 1; pp < VP; ++pp) {
          V[pp][0] = ldV(so, pp, 0);
          V[pp][1] = ldV(so, pp, 1);
        }
#pragma unroll
        for (int db = 0; db < kRsDBW; ++db) {
          if (db + VP < kRsDBW) {
            V[(db + VP) % (VP + 1)][0] = ldV(so, db + VP, 0);
            V[(db + VP) % (VP + 1)][1] = ldV(so, db + VP, 1);
          }
          const bf16x8_t a = __builtin_shufflevector(V[db % (VP + 1)][0], V[db % (VP + 1)][1], 0, 1,
                                                     2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
            o[db][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pB[hb], o[db][hb], 0, 0, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // the next tile's first V fragments (that tile landed before this
      // iteration began; the QK waves read it now)
      if (t + 1 < G) {
        const int so1 = ((t + 1) % kRsRing) * kStageBytes;
        vn0 = ldV(so1, 0, 0);
        vn1 = ldV(so1, 0, 1);
      }
      if (cp.tile == cp.ntiles - 1 && cp.slot != kChainNext) {
        // ---- epilogue: this wave's 128 dims of the unit's 64 heads ----
        const int le = lane_id_fresh();
        const int ge = le >> 4, lie = le & 15;
        const f32x4_t l4 = *(const LDS_AS f32x4_t*)(smem + kXlOff + (par * 64 + lie * 4) * 4);
        float linv[HB];
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          linv[hb] = __builtin_amdgcn_rcpf(l4[hb]) * (FP8 ? v_scale : 1.f);
          // (row blocks: a row that saw no token of this piece has O = 0 and
          // l = 0; its state is (0, -inf), weight 0 in the merge)
          if (ROWS) linv[hb] = l4[hb] > 0.f ? linv[hb] : 0.f;
        }
        if (FLAGS && !waits_ok) {
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) linv[hb] = __builtin_nanf("");
        }
        // Lane (g, li) holds dims r*128 + db*16 + g*4 .. +3 of head hb*16 + li.
        // For a pair of dim blocks (2dp, 2dp+1) one row swap (rows 0<->1 and
        // 2<->3, v_permlane16_swap) gives every lane 8 consecutive dims: even
        // rows dims (g/2)*8 .. +7 of block 2dp, odd rows those of block 2dp+1.
        // So each lane stores 16 bytes, half the store instructions of
        // 8-byte stores.
        const uint32_t col = (uint32_t)(lie * kCkvDim + r * (kRsDBW * 16) + (ge >> 1) * 8);
        // a whole request's rows go to out, a split unit's to its partial slot
        // (both bf16)
        // (a row block's rows: partial-state rows from its first row plus
        // the unit's offset, or out's own rows for a whole block of query
        // tokens; head blocks past the block's rows store nothing)
        char* obase = reinterpret_cast<char*>(
            ROWS ? (cp.slot == kRowsDirect ? out + (size_t)(cp.b + hg * HEADS) * kCkvDim
                                           : part_o + (size_t)(cp.slot + cp.b + hg * HEADS) * kCkvDim)
            : cp.slot < 0 ? out + ((size_t)cp.b * H + hg * HEADS) * kCkvDim
                          : part_o + ((size_t)cp.slot * H + hg * HEADS) * kCkvDim);
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          if (ROWS && cp.b + hg * HEADS + hb * 16 >= cp.rend) break;
          const uint32_t row = col + (uint32_t)hb * 16 * kCkvDim;
#pragma unroll
          for (int dp = 0; dp < kRsDBW / 2; ++dp) {
            const uint2 x = __builtin_bit_cast(
                uint2, __builtin_convertvector(o[2 * dp][hb] * linv[hb], bf16x4_t));  // RNE
            const uint2 y = __builtin_bit_cast(
                uint2, __builtin_convertvector(o[2 * dp + 1][hb] * linv[hb], bf16x4_t));
            const auto s0 = __builtin_amdgcn_permlane16_swap(x.x, y.x, false, false);
            const auto s1 = __builtin_amdgcn_permlane16_swap(x.y, y.y, false, false);
            const uint32_t blk = (uint32_t)(2 * dp + (ge & 1));
            *reinterpret_cast<uint4*>(obase + (row + blk * 16) * 2) =
                make_uint4((uint32_t)s0[0], (uint32_t)s1[0], (uint32_t)s0[1], (uint32_t)s1[1]);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      cursor_next(cp, units, u_end);
      if (FLAGS) {
        // tile t's stage and exchange buffers are free once this wave's reads
        // of them have returned
        publish_counter(done + r, t + 1);
      } else {
        // this role writes no LDS, and its reads still in flight are of a tile
        // that stays resident for two more iterations: no wait before the barrier
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
      }
    }
    // (with counters no barrier ends the workgroup: its end is the first PV
    // wave's)
    if (FLAGS && stamps && threadIdx.x == HB * 64) stamp_end(stamps);
  } else if constexpr (FP8) {
    // ================= copy role, fp8 caches =================
    // copy wave cw loads copy slot cw of every tile into registers (five
    // loads), widens it to bf16 and stores it to the tile's LDS stage.  Two
    // register buffers alternate by tile parity: at step i the loads of tile
    // i+2 go out, then tile i+1 (loaded one step earlier) is widened and
    // stored, and the barrier publishes it once the wave's LDS stores have
    // completed.  The compiler waits for the loads a store uses; no wait here
    // covers the loads still in flight.
    const int cw = wave - (HB + kRsPvWaves);
    const Fp8Lanes FL = fp8_lanes(cw, cs, ks);
    TileStream ts;
    ts.u = u_begin;
    ts.u_end = u_end;
    ts.g = 0;
    stream_load_unit(ts, units, seq_indices);
    Fp8Slot b0, b1;
    // Every step loads a tile: once the stream is exhausted, the last tile's
    // rows again (valid memory, never stored).  With no branch around the
    // loads of a step, the compiler's wait before a store counts exactly the
    // five loads issued after that buffer's.
    TileCopy keep;
    auto load_tile = [&](Fp8Slot& buf) __attribute__((always_inline)) {
      const bool more = ts.u < ts.u_end;
      if (more) keep = tile_copy(ts, ckv, kpe, log2_ps, 0u, cw, cs, ks);
      if (BIG && keep.full) fp8_slot_load_full(keep, FL, buf);
      else fp8_slot_load<BIG>(keep, ckv, kpe, cw, buf);
      if (more) stream_advance(ts, units, seq_indices, log2_ps);
    };
    auto store_tile = [&](const Fp8Slot& buf, int g) __attribute__((always_inline)) {
      fp8_slot_store(smem + (g % kRsRing) * kStageBytes, FL, buf);
    };
    // this wave's LDS stores are complete, then the workgroup barrier (no
    // fence: loads of the next tile stay in flight across it)
    auto publish = [&]() __attribute__((always_inline)) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt left open
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    };
    load_tile(b0);  // tile 0
    publish();      // the QK waves load their queries from here on
    load_tile(b1);  // tile 1
    store_tile(b0, 0);
    publish();
    // steps s = 0 .. G (one barrier each), two per pass: step s loads tile
    // s+2 into the buffer of tile s (stored at step s-1) and stores tile s+1
    for (int i = 0;; i += 2) {
      load_tile(b0);
      if (i + 1 < G) store_tile(b1, i + 1);
      publish();
      if (i >= G) break;
      load_tile(b1);
      if (i + 2 < G) store_tile(b0, i + 2);
      publish();
      if (i + 1 >= G) break;
    }
  } else {
    // ======================= copy role =======================
    // copy wave cw issues copy slots 2cw and 2cw+1 of every tile (18 copies;
    // at most two tiles, 36 operations, in flight)
    const int cw = wave - (HB + kRsPvWaves);
    CopyLanes CLw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) CLw[h] = copy_lanes(2 * cw + h, ks);
    TileStream ts;
    ts.u = u_begin;
    ts.u_end = u_end;
    ts.g = 0;
    stream_load_unit(ts, units, seq_indices);
    int vmc = 0;
    int rv0 = 0, rv1 = 0, rv2 = 0, rv3 = 0;
    auto book_tile = [&]() {
      vmc += 2 * kCopiesPerWave;
      const int st = ts.g % kRsRing;
      rv0 = st == 0 ? vmc : rv0;
      rv1 = st == 1 ? vmc : rv1;
      rv2 = st == 2 ? vmc : rv2;
      rv3 = st == 3 ? vmc : rv3;
      stream_advance(ts, units, seq_indices, log2_ps);
    };
    auto vmc_of = [&](int gidx) {
      const int st = gidx % kRsRing;
      return st == 0 ? rv0 : st == 1 ? rv1 : st == 2 ? rv2 : rv3;
    };
    auto issue_tile = [&]() {
      const uint32_t sb = smem_base + (uint32_t)(ts.g % kRsRing) * kStageBytes;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int w = 2 * cw + h;
        const TileCopy c = tile_copy(ts, ckv, kpe, log2_ps, sb, w, cs, ks);
        if (BIG && c.full) {
#pragma unroll
          for (int k = 0; k < kCopiesPerWave; ++k) tile_copy_part_full(c, w, k, CLw[h]);
        } else {
          tile_copy_slot<BIG, PACKED>(c, ckv, kpe, w, CLw[h]);
        }
      }
      book_tile();
    };
    if (FLAGS) landed[cw] = 0;
    if (ts.u < ts.u_end) issue_tile();
    lds_barrier();  // the QK waves load their queries from here on
    if constexpr (FLAGS) {
      // Tile t goes into stage t mod 4 once the PV waves have finished tile
      // t-4 (the QK waves finished it before), and the wave then waits, with
      // an exact vmcnt, for its share of tile t-1: at most two tiles in flight.
      for (int t = 1; t < G; ++t) {
        if (t >= kRsRing) wait_counters<kRsPvWaves>(done, t - kRsRing + 1, wait_limit);
        issue_tile();
        wait_vm_le(vmc - vmc_of(t - 1));
        asm volatile("" ::: "memory");
        landed[cw] = t;  // tiles 0 .. t-1 have landed
      }
      wait_vmcnt<0>();
      asm volatile("" ::: "memory");
      landed[cw] = G;
    } else {
      if (ts.u < ts.u_end) issue_tile();
      wait_vm_le(vmc - vmc_of(0));
      lds_barrier();
      for (int i = 0; i <= G; ++i) {
        // tile i+2 into the stage PV(i-2) released at the last barrier
        if (ts.u < ts.u_end) issue_tile();
        if (i + 1 < G) wait_vm_le(vmc - vmc_of(i + 1));
        lds_barrier();
      }
      wait_vmcnt<0>();
    }
  }
}

int decode_rs_head_blocks(int waves, int heads_per_wave, int num_heads, int head_groups) {
  if (heads_per_wave != 16 || head_groups < 1) return 0;
  const int hb = waves - kRsPvWaves;
  if ((hb != 1 && hb != 2 && hb != 4) || num_heads != 16 * hb * head_groups) return 0;
  return hb;
}

bool launch_decode_rs(const DecodeParams& p, hipStream_t stream, hipError_t* err) {
  // row-block units: 64 rows per workgroup at every head count
  const int hb = p.row_blocks ? (p.waves == 4 + kRsPvWaves && p.heads_per_wave == 16 ? 4 : 0)
                              : decode_rs_head_blocks(p.waves, p.heads_per_wave, p.num_heads,
                                                      p.head_groups);
  if (!hb) return false;
  const bool big = p.log2_ps >= 5;
  const bool packed = p.ckv_stride == kCkvDim * 2 && p.kpe_stride == kKpeDim * 2;
  const dim3 grid(decode_grid(p.n_lanes, p.head_groups)), block(rs_threads(hb, p.fp8 != 0));
#define PKVMLA_RS_ARGS                                                                   \
  p.q_nope, p.q_pe, p.ckv, p.kpe, p.out, p.lse, p.part_o, p.part_lse, p.wg_indptr, p.units, \
      p.seq_indices, p.num_heads, p.head_groups, p.n_lanes, p.log2_ps, p.sm_scale,     \
      p.score_log2, p.rescale_thr, p.ckv_stride, p.kpe_stride, p.stamps, p.v_scale,    \
      p.kpe_ratio, p.qo_log2h, p.wait_limit
#define PKVMLA_RS_LAUNCH3(HBV, PK, RB, F8)                                                     \
  if (big) mla_decode_rs_kernel<true, HBV, PK, RB, F8><<<grid, block, 0, stream>>>(PKVMLA_RS_ARGS); \
  else mla_decode_rs_kernel<false, HBV, PK, RB, F8><<<grid, block, 0, stream>>>(PKVMLA_RS_ARGS);
  // fp8 caches always take the runtime row strides
#define PKVMLA_RS_LAUNCH(HBV, RB)                                   \
  if (p.fp8) { PKVMLA_RS_LAUNCH3(HBV, false, RB, true) }            \
  else if (packed) { PKVMLA_RS_LAUNCH3(HBV, true, RB, false) }      \
  else { PKVMLA_RS_LAUNCH3(HBV, false, RB, false) }
  if (p.row_blocks) {
    PKVMLA_RS_LAUNCH(4, true)
  } else {
    switch (hb) {
      case 1: PKVMLA_RS_LAUNCH(1, false) break;
      case 2: PKVMLA_RS_LAUNCH(2, false) break;
      default: PKVMLA_RS_LAUNCH(4, false) break;
    }
  }
#undef PKVMLA_RS_LAUNCH
#undef PKVMLA_RS_LAUNCH3
#undef PKVMLA_RS_ARGS
  *err = hipGetLastError();
  return true;
}

}  // namespace pkvmla
