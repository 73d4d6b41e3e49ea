// Fused absorbed-MLA decode kernel for 64 and 128 query heads on gfx950.
//
// One workgroup of four waves per CU runs a list of work units (split-KV
// segments: a token range [kv_begin, kv_end) of one request's page list) and
// keeps every query head of the unit:
//   QK   wave w computes S^T[token, head] = K[token, 576] . Q^T[576, head] for
//        its own 16*NB heads (MFMA 16x16x32 bf16; K from LDS, Q in registers),
//   softmax of those heads (running max m, running sum l),
//   PV   wave w accumulates O^T[dim, head] += V^T[dim, token] . P^T[token, head]
//        for its own 128 output dims and all 64*NB heads; V^T is read from the
//        same LDS tile with ds_read_b64_tr_b16 and P^T of every wave comes
//        through a small LDS exchange.
// Splitting PV by output dims reads each V element once per workgroup; QK has
// to read the whole K tile once per wave (each wave holds different heads).
//
// Pipeline.  KV tiles of 32 tokens form one continuous stream over all units
// of the workgroup (a tile of the next unit can be in flight while the current
// unit finishes); each wave copies its share of a tile straight from HBM into
// a 3-stage LDS ring with global_load_lds_dwordx4.  While PV reads tile t and
// QK reads tile t+1, one tile (t+2) is in flight: 36 KB per CU keeps HBM
// streaming at full rate on a full chip.  Its copies go out one per k-step
// over the first nine k-steps of QK(t+1): the CU's memory pipeline accepts
// about one 1 KB copy every 23 clocks, and the four waves meet at a barrier
// every tile, so a burst of 36 copies would hold all of them for about 800
// clocks.  The copies take their lane offsets from registers that are never
// rewritten (a copy reads its address registers only when it is accepted).
// Inside a unit, the softmax of tile t is computed between the MFMAs of
// QK(t+1), so the VALU work overlaps the matrix cores.  Every wave counts the
// vector-memory operations it has issued; waiting for a tile is an s_waitcnt
// vmcnt with the exact number of later operations, so copies of later tiles,
// the next query and the epilogue stores of the previous unit stay in flight.
//
// Masking.  Only the last tile of a unit can be partial.  Its ckv slots past
// kv_end are filled with the last valid token's row (finite data), its kpe
// slots with the page's own rows past kv_end, and those slots' scores are
// set to -inf (a select) before the softmax, so they add exactly zero to PV.

#include <hip/hip_runtime.h>
#include <math.h>

#include "pkvmla_tiles.h"

namespace pkvmla {

namespace {

constexpr int kWaves = 4;
static_assert(kWaves == kCopyWaves, "the tile copies assume four waves");
constexpr int kDmaW = kCopiesPerWave;   // copy instructions per wave and tile: 8 ckv rows + 1 kpe block
constexpr int kRing = 3;                // LDS stages: PV tile, QK tile, one tile in flight
constexpr int kQkAhead = 2;             // k-steps between a K fragment's LDS read and its MFMA

}  // namespace

template <int NB, bool BIG>
__global__ void __launch_bounds__(kWaves * 64, 1)
mla_decode_w4_kernel(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
                     const uint16_t* __restrict__ ckv_cache, const uint16_t* __restrict__ kpe_cache,
                     uint16_t* __restrict__ out, float* __restrict__ lse_out,
                     float* __restrict__ part_o, float* __restrict__ part_lse,
                     const int32_t* __restrict__ wg_indptr_g, const int32_t* __restrict__ units_g,
                     const int32_t* __restrict__ seq_indptr_g,
                     const int32_t* __restrict__ seq_indices_g, int n_lanes, int log2_ps,
                     float sm_scale, float C, float thr) {
  const idx_ptr wg_indptr = (idx_ptr)wg_indptr_g;
  const idx_ptr units = (idx_ptr)units_g;
  const idx_ptr seq_indptr = (idx_ptr)seq_indptr_g;
  const idx_ptr seq_indices = (idx_ptr)seq_indices_g;
  constexpr int HBN = kWaves * NB;   // head blocks of 16 in the workgroup
  constexpr int H = HBN * 16;
  constexpr int DBW = 8;             // output-dim blocks of 16 per wave (128 dims)
  // LDS: the ring, the P^T exchange (1 KB per head block), then per-head
  // floats laid out [li][head block]: rescale factors and row sums.
  constexpr int xp_off = kRing * kStageBytes;
  constexpr int xa_off = xp_off + HBN * 1024;
  constexpr int xl_off = xa_off + HBN * 64;
  // q_pe of the unit's request: head block hb, rope k-step k2 at
  // qp_off + (hb * 2 + k2) * 1 KB, lane (g, li) at 16 * lane (the MFMA B layout)
  constexpr int qp_off = (xl_off + HBN * 64 + 1023) / 1024 * 1024;
  constexpr int lds_bytes = qp_off + HBN * 2048;
  static_assert(lds_bytes <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem_raw[lds_bytes];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;    // 16-lane group
  const int li = lane & 15;
  const int sl = blockIdx.x;
  if (sl >= n_lanes) return;
  const int u_begin = wg_indptr[sl];
  const int u_end = wg_indptr[sl + 1];
  if (u_begin >= u_end) return;
  const char* ckv = reinterpret_cast<const char*>(ckv_cache);
  const char* kpe = reinterpret_cast<const char*>(kpe_cache);

  // Per-lane LDS offsets inside a stage.
  // QK A operand: token tb*16 + li, chunk ks*4 + g  -> base ^ (ks << 6)
  // PV V^T operand (transposed read): source lane (g, r = li/4, q = li%4)
  // addresses token tb*16 + g*4 + r, dims db*16 + 4q..4q+3 -> base ^ (db << 5)
  int offA[2], offK[2], offV[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int tA = tb * 16 + li;
    offA[tb] = lds_ckv_off(tA, g);
    offK[tb] = lds_kpe_off(tA, g);
    const int tV = tb * 16 + g * 4 + (li >> 2);
    const int q = li & 3;
    offV[tb] = lds_ckv_off(tV, q >> 1) + (q & 1) * 8;
  }

  // ---- tile stream: the first kRing tiles ----
  TileStream ts;
  ts.u = u_begin;
  ts.u_end = u_end;
  ts.g = 0;
  stream_load_unit(ts, units, seq_indptr, seq_indices, log2_ps);
  int vmc = 0;  // vector-memory ops this wave has issued
  // vmc right after the latest tile of each ring stage (named scalars, not an
  // array: an indexed array would be placed in scratch memory)
  int rv0 = 0, rv1 = 0, rv2 = 0;
  // the stream's next tile: its scalar context, its copy parts, then booking
  // (vmc, ring stage) and advancing the stream
  auto book_tile = [&]() {
    vmc += kDmaW;
    const int st = ts.g % kRing;
    rv0 = st == 0 ? vmc : rv0;
    rv1 = st == 1 ? vmc : rv1;
    rv2 = st == 2 ? vmc : rv2;
    stream_advance(ts, units, seq_indptr, seq_indices, log2_ps);
  };
  auto issue_one = [&]() {
    const TileCopy c = tile_copy(ts, ckv, kpe, log2_ps,
                                 smem_base + (uint32_t)(ts.g % kRing) * kStageBytes, wave);
    tile_copy_wave<BIG>(c, ckv, kpe, wave, copy_lanes(wave));
    book_tile();
  };
  // the stream may issue tile j once tiles < j - kRing + 1 are consumed
  auto may_issue = [&](int consumed) { return ts.u < ts.u_end && ts.g < consumed + kRing; };
  auto maybe_issue = [&](int consumed) {
    if (may_issue(consumed)) issue_one();
  };
  auto vmc_of = [&](int gidx) {
    const int st = gidx % kRing;
    return st == 0 ? rv0 : st == 1 ? rv1 : rv2;
  };
#pragma unroll 1
  for (int i = 0; i < kRing - 1; ++i)
    if (ts.u < ts.u_end) issue_one();

  // Q^T operand for a whole unit: lane (g, li) holds
  // Q[head nb*16 + li][ks*32 + g*8 .. +7]; the q_nope k-steps (0..15) stay in
  // registers, the two q_pe k-steps are copied into LDS (16 fewer registers,
  // which buys a deeper K prefetch).  Each wave reads only its own q_pe
  // blocks, after its own copies have landed.
  bf16x8_t q[NB][16];
  int q_vmc = 0;
  // (a request's rows as a scalar base, lanes as 32-bit offsets: few address registers)
  auto load_q = [&](int b) {
    const char* qn = reinterpret_cast<const char*>(q_nope + (size_t)b * H * kCkvDim);
    const char* qp = reinterpret_cast<const char*>(q_pe + (size_t)b * H * kKpeDim);
    const uint32_t lq = (uint32_t)lane_id_fresh();
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t h = (uint32_t)(wave * (16 * NB) + nb * 16) + (lq & 15);
      const uint32_t on = (h * kCkvDim + (lq >> 4) * 8) * 2;
      const uint32_t op = (h * kKpeDim + (lq >> 4) * 8) * 2;
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) q[nb][ks] = *reinterpret_cast<const bf16x8_t*>(qn + on + ks * 64);
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        set_m0(smem_base + (uint32_t)(qp_off + ((wave * NB + nb) * 2 + k2) * 1024));
        dma16_m0<0>(qp, op + (uint32_t)k2 * 64);
      }
    }
    vmc += 18 * NB;
    q_vmc = vmc;
  };
  load_q(units[(size_t)u_begin * kUnitInts + 0]);

  int gc = 0;  // stream position of the current unit's first tile
  for (int u = u_begin; u < u_end; ++u) {
    idx_ptr rec = units + (size_t)u * kUnitInts;
    const int b = rec[0];
    const int kv0 = rec[2];
    const int kv1 = rec[3];
    const int slot = rec[4];
    const int n = (kv1 - kv0 + kTile - 1) / kTile;

    // the query and this wave's copies of the unit's first tile have landed
    wait_vm_le(vmc - max(q_vmc, vmc_of(gc)));
    lds_barrier();  // (the stream is already kRing tiles ahead here)

    // Per-lane offsets and the lane id go through an empty asm once per tile:
    // otherwise the compiler hoists every derived operand address out of the
    // loops and spills them, and a spill reload waits for all outstanding
    // copies.
    auto fresh = [&](int (&oA)[2], int (&oK)[2], int (&oV)[2]) {
      oA[0] = offA[0]; oA[1] = offA[1]; oK[0] = offK[0]; oK[1] = offK[1];
      oV[0] = offV[0]; oV[1] = offV[1];
      asm volatile("" : "+v"(oA[0]), "+v"(oA[1]), "+v"(oK[0]), "+v"(oK[1]), "+v"(oV[0]), "+v"(oV[1]));
    };
    // this lane's q_pe fragment of head block nb, rope k-step k2
    auto ldQpe = [&](int nb, int k2) -> bf16x8_t {
      const int off = qp_off + ((wave * NB + nb) * 2 + k2) * 1024 + lane_id_fresh() * 16;
      return *(const LDS_AS bf16x8_t*)(smem + off);
    };

    // ---- QK of one stage into acc (fresh), with `mid(ks)` after each k-step ----
    auto qk = [&](int stage, const int (&oA)[2], const int (&oK)[2], f32x4_t (&acc)[2][NB],
                  auto&& mid) {
      const int so = stage * kStageBytes;
      auto ldA = [&](int ks, int tb) -> bf16x8_t {
        const int off = ks < 16 ? ((so + oA[tb]) ^ (ks << 6)) : ((so + oK[tb]) ^ ((ks - 16) << 6));
        return *(const LDS_AS bf16x8_t*)(smem + off);
      };
      f32x4_t acc2[2][NB];  // odd k-steps (NB == 1: keeps dependent MFMAs apart)
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          acc[tb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          acc2[tb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      // K fragments are read kQkAhead k-steps ahead of their MFMAs (LDS latency
      // under load exceeds one k-step of matrix work)
      constexpr int AH = kQkAhead;
      bf16x8_t A[AH + 1][2];
#pragma unroll
      for (int pp = 0; pp < AH; ++pp) {
        A[pp][0] = ldA(pp, 0);
        A[pp][1] = ldA(pp, 1);
      }
      // q_pe fragments: read from LDS a few k-steps before the rope k-steps
      constexpr int QPE_AT = 12;
      bf16x8_t qpe[NB][2];
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        if (ks + AH < 18) {
          A[(ks + AH) % (AH + 1)][0] = ldA(ks + AH, 0);
          A[(ks + AH) % (AH + 1)][1] = ldA(ks + AH, 1);
        }
        if (ks == QPE_AT) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            qpe[nb][0] = ldQpe(nb, 0);
            qpe[nb][1] = ldQpe(nb, 1);
          }
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const bf16x8_t bq = ks < 16 ? q[nb][ks & 15] : qpe[nb][(ks - 16) & 1];
            if (NB == 1 && (ks & 1))
              acc2[tb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[ks % (AH + 1)][tb], bq, acc2[tb][nb], 0, 0, 0);
            else
              acc[tb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[ks % (AH + 1)][tb], bq, acc[tb][nb], 0, 0, 0);
          }
        mid(ks);
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (NB == 1) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[tb][0] += acc2[tb][0];
      }
    };

    // ---- softmax state of this wave's heads ----
    float m_run[NB], l_run[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_run[nb] = -INFINITY;
      l_run[nb] = 0.f;
    }
    f32x4_t o[DBW][HBN];
#pragma unroll
    for (int db = 0; db < DBW; ++db)
#pragma unroll
      for (int hb = 0; hb < HBN; ++hb) o[db][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // Softmax of one tile's scores, in pieces that can sit between MFMAs.
    // Per lane: heads nb*16 + li, tokens tb*16 + g*4 + i.
    struct SoftmaxTmp {
      float sv[NB][8];
      float mx[NB];
      float alpha[NB];
      bf16x8_t pT[NB];
    };
    // valid < kTile (a unit's last tile): slots t >= valid get -inf
    auto sm_load = [&](SoftmaxTmp& T, const f32x4_t (&s)[2][NB], int valid) {
      const int gm = valid < kTile ? (lane_id_fresh() >> 4) : 0;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = tb * 16 + gm * 4 + i;
            T.sv[nb][tb * 4 + i] = (valid >= kTile || t < valid) ? s[tb][nb][i] : -INFINITY;
          }
    };
    auto sm_max = [&](SoftmaxTmp& T) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float mx = fmaxf(fmaxf(T.sv[nb][0], T.sv[nb][1]), fmaxf(T.sv[nb][2], T.sv[nb][3]));
        mx = fmaxf(mx, fmaxf(fmaxf(T.sv[nb][4], T.sv[nb][5]), fmaxf(T.sv[nb][6], T.sv[nb][7])));
        T.mx[nb] = mx;
      }
    };
    auto sm_rows = [&](SoftmaxTmp& T) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) T.mx[nb] = max_over_rows(T.mx[nb]);
    };
    // Lazy running max: the reference m moves only when the tile max exceeds it
    // by more than rescale_thr (probabilities stay <= 2^8, exact in fp32 and in
    // bf16's range), so O is rarely rescaled.  The first tile always sets m.
    auto sm_alpha = [&](SoftmaxTmp& T) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const bool grow = T.mx[nb] > m_run[nb] + thr;
        const float m_new = grow ? T.mx[nb] : m_run[nb];
        T.alpha[nb] = __builtin_amdgcn_exp2f((m_run[nb] - m_new) * C);
        m_run[nb] = m_new;
      }
    };
    auto sm_exp = [&](SoftmaxTmp& T, int k0, int k1) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float mc = m_run[nb] * C;
#pragma unroll
        for (int k = k0; k < k1; ++k) T.sv[nb][k] = __builtin_amdgcn_exp2f(fmaf(T.sv[nb][k], C, -mc));
      }
    };
    auto sm_sum = [&](SoftmaxTmp& T) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float ps = (T.sv[nb][0] + T.sv[nb][1]) + (T.sv[nb][2] + T.sv[nb][3]);
        ps += (T.sv[nb][4] + T.sv[nb][5]) + (T.sv[nb][6] + T.sv[nb][7]);
        l_run[nb] = l_run[nb] * T.alpha[nb] + ps;
#pragma unroll
        for (int k = 0; k < 8; ++k) T.pT[nb][k] = (__bf16)T.sv[nb][k];
      }
    };
    auto sm_publish = [&](SoftmaxTmp& T) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int hb = wave * NB + nb;
        *(LDS_AS bf16x8_t*)(smem + xp_off + hb * 1024 + lane * 16) = T.pT[nb];
        if (g == 0) *(LDS_AS float*)(smem + xa_off + (li * HBN + hb) * 4) = T.alpha[nb];
      }
    };

    // ---- PV of one stage: rescale when a head's max moved, then this
    // wave's dims for every head ----
    auto pv = [&](int stage, const int (&oV)[2], bool may_rescale) {
      bf16x8_t pB[HBN];
      float alpha[HBN];
#pragma unroll
      for (int hb = 0; hb < HBN; ++hb)
        pB[hb] = *(const LDS_AS bf16x8_t*)(smem + xp_off + hb * 1024 + lane * 16);
#pragma unroll
      for (int h4 = 0; h4 < HBN / 4; ++h4) {
        const f32x4_t a4 = *(const LDS_AS f32x4_t*)(smem + xa_off + (li * HBN + h4 * 4) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) alpha[h4 * 4 + i] = a4[i];
      }
      if (may_rescale) {
        bool need = false;
#pragma unroll
        for (int hb = 0; hb < HBN; ++hb) need |= alpha[hb] != 1.0f;
        if (__builtin_amdgcn_ballot_w64(need)) {
          // The empty asm statements pin the accumulators to AGPRs so the
          // MFMAs keep their AGPR form; the multiply goes through VGPRs.
#pragma unroll
          for (int db = 0; db < DBW; ++db)
#pragma unroll
            for (int hb = 0; hb < HBN; ++hb) {
              asm volatile("" : "+a"(o[db][hb]));
              o[db][hb] *= alpha[hb];
              asm volatile("" : "+a"(o[db][hb]));
            }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      const int so = stage * kStageBytes;
      auto ldV = [&](int db, int tb) -> bf16x4_t {
        const int dbg = wave * DBW + db;
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4_t*)(smem + ((so + oV[tb]) ^ (dbg << 5))));
      };
      constexpr int VP = 2;
      bf16x4_t V[VP + 1][2];
#pragma unroll
      for (int pp = 0; pp < VP; ++pp) {
        V[pp][0] = ldV(pp, 0);
        V[pp][1] = ldV(pp, 1);
      }
#pragma unroll
      for (int db = 0; db < DBW; ++db) {
        if (db + VP < DBW) {
          V[(db + VP) % (VP + 1)][0] = ldV(db + VP, 0);
          V[(db + VP) % (VP + 1)][1] = ldV(db + VP, 1);
        }
        const bf16x8_t a = __builtin_shufflevector(V[db % (VP + 1)][0], V[db % (VP + 1)][1], 0, 1,
                                                   2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int hb = 0; hb < HBN; ++hb)
          o[db][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pB[hb], o[db][hb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // ---- prologue: scores of the unit's first tile ----
    f32x4_t sacc[2][NB];
    {
      int oA[2], oK[2], oV[2];
      fresh(oA, oK, oV);
      qk(gc % kRing, oA, oK, sacc, [&](int) {});
    }

    // ---- all tiles but the last: QK(t+1) with the softmax of tile t in between ----
    // (the copies' lane offsets stay in registers through the unit's tiles)
    const CopyLanes CL = copy_lanes(wave);
    for (int t = 0; t + 1 < n; ++t) {
      const int gi = gc + t;
      wait_vm_le(vmc - vmc_of(gi + 1));
      lds_barrier();  // tile t+1 landed everywhere; PV(t-1) and its exchange are consumed
      int oA[2], oK[2], oV[2];
      fresh(oA, oK, oV);
      SoftmaxTmp T;
      f32x4_t snext[2][NB];
      // the copies of tile gi+2 go into the stage PV(gi-1) just released
      const bool iss = may_issue(gi);
      // BIG whole tiles: one copy part per k-step (k-steps 0..8), from ready
      // bases.  The CU's memory pipeline takes a copy about every 23 clocks,
      // so a burst of 36 copies would hold the waves (which meet at a barrier
      // every tile) for about 800.  A unit's last (partial) tile, and the
      // small-page path with its per-row page lookups, issue their share at
      // once before the k-loop.
      TileCopy cp{};
      bool spread = false;
      if (iss) {
        cp = tile_copy(ts, ckv, kpe, log2_ps, smem_base + (uint32_t)(ts.g % kRing) * kStageBytes, wave);
        if (BIG && cp.full) {
          spread = true;
        } else {
          tile_copy_wave<BIG>(cp, ckv, kpe, wave, CL);
          book_tile();
        }
      }
      qk((gi + 1) % kRing, oA, oK, snext, [&](int ks) {
        if (spread && ks < kDmaW) {
          tile_copy_part_full(cp, wave, ks, CL);
          if (ks == kDmaW - 1) book_tile();
        }
        switch (ks) {
          case 0: sm_load(T, sacc, kTile); sm_max(T); break;
          case 1: sm_rows(T); break;
          case 2: sm_alpha(T); break;
          case 3: sm_exp(T, 0, 2); break;
          case 4: sm_exp(T, 2, 4); break;
          case 5: sm_exp(T, 4, 6); break;
          case 6: sm_exp(T, 6, 8); break;
          case 7: sm_sum(T); break;
          case 8: sm_publish(T); break;
          default: break;
        }
      });
      lds_barrier();  // P^T and rescale factors of tile t published
      pv(gi % kRing, oV, t > 0);
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sacc[tb][nb] = snext[tb][nb];
    }

    // ---- last tile of the unit ----
    const int gl = gc + n - 1;
    lds_barrier();  // PV(gl-1) and its exchange are consumed
    // (no copy here: the next unit's first tile is still in flight and the
    // query of the next unit goes out now)
    if (u + 1 < u_end) load_q(units[(size_t)(u + 1) * kUnitInts + 0]);
    {
      int oA[2], oK[2], oV[2];
      fresh(oA, oK, oV);
      SoftmaxTmp T;
      sm_load(T, sacc, kv1 - (kv0 + (n - 1) * kTile));
      sm_max(T);
      sm_rows(T);
      sm_alpha(T);
      sm_exp(T, 0, 8);
      sm_sum(T);
      sm_publish(T);
      lds_barrier();
      pv(gl % kRing, oV, n > 1);
    }

    // ---- epilogue: row sums of every head, then this wave's dims ----
    const int le = lane_id_fresh();
    const int ge = le >> 4, lie = le & 15;
    float lse_v[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float l = l_run[nb];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      lse_v[nb] = m_run[nb] * sm_scale + __builtin_amdgcn_logf(l) * 0.69314718055994531f;
      if (ge == 0) *(LDS_AS float*)(smem + xl_off + (lie * HBN + wave * NB + nb) * 4) = l;
    }
    lds_barrier();  // row sums published; PV(gl) done everywhere
    maybe_issue(gl + 1);
    float linv[HBN];
#pragma unroll
    for (int h4 = 0; h4 < HBN / 4; ++h4) {
      const f32x4_t l4 = *(const LDS_AS f32x4_t*)(smem + xl_off + (lie * HBN + h4 * 4) * 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) linv[h4 * 4 + i] = __builtin_amdgcn_rcpf(l4[i]);
    }
    // lane (g, li) holds dims wave*128 + db*16 + g*4 .. +3 of head hb*16 + li;
    // one head block at a time keeps the products' live range short
    const uint32_t col = (uint32_t)(lie * kCkvDim + wave * (DBW * 16) + ge * 4);
    char* obase = reinterpret_cast<char*>(out + (size_t)b * H * kCkvDim);
    char* pbase = reinterpret_cast<char*>(part_o + (size_t)max(slot, 0) * H * kCkvDim);
#pragma unroll
    for (int hb = 0; hb < HBN; ++hb) {
      const uint32_t row = col + (uint32_t)hb * 16 * kCkvDim;
      f32x4_t v[DBW];
#pragma unroll
      for (int db = 0; db < DBW; ++db) v[db] = o[db][hb] * linv[hb];
      if (slot < 0) {
#pragma unroll
        for (int db = 0; db < DBW; ++db)
          *reinterpret_cast<bf16x4_t*>(obase + row * 2 + db * 32) =
              __builtin_convertvector(v[db], bf16x4_t);  // RNE
      } else {
#pragma unroll
        for (int db = 0; db < DBW; ++db)
          *reinterpret_cast<f32x4_t*>(pbase + row * 4 + db * 64) = v[db];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    vmc += DBW * HBN;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int h = (wave * NB + nb) * 16 + lie;
      if (ge == 0) {
        if (slot < 0) lse_out[(size_t)b * H + h] = lse_v[nb];
        else part_lse[(size_t)slot * H + h] = lse_v[nb];
      }
    }
    gc += n;
  }
  // no copy may still be writing LDS when the workgroup retires
  wait_vmcnt<0>();
}

bool launch_decode_w4(const DecodeParams& p, hipStream_t stream, hipError_t* err) {
  if (p.waves != kWaves || p.head_groups != 1) return false;
  const bool big = p.log2_ps >= 5;
  const dim3 grid(p.n_lanes), block(kWaves * 64);
#define PKVMLA_W4_ARGS                                                                   \
  p.q_nope, p.q_pe, p.ckv, p.kpe, p.out, p.lse, p.part_o, p.part_lse, p.wg_indptr, p.units, \
      p.seq_indptr, p.seq_indices, p.n_lanes, p.log2_ps, p.sm_scale, p.score_log2, p.rescale_thr
  if (p.heads_per_wave == 32) {
    if (big) mla_decode_w4_kernel<2, true><<<grid, block, 0, stream>>>(PKVMLA_W4_ARGS);
    else mla_decode_w4_kernel<2, false><<<grid, block, 0, stream>>>(PKVMLA_W4_ARGS);
  } else if (p.heads_per_wave == 16) {
    if (big) mla_decode_w4_kernel<1, true><<<grid, block, 0, stream>>>(PKVMLA_W4_ARGS);
    else mla_decode_w4_kernel<1, false><<<grid, block, 0, stream>>>(PKVMLA_W4_ARGS);
  } else {
    return false;
  }
#undef PKVMLA_W4_ARGS
  *err = hipGetLastError();
  return true;
}

}  // namespace pkvmla
