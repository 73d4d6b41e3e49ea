// HIP kernels for absorbed-form MLA paged decode on gfx950 (MI355X).
//
// One workgroup runs a list of work units; a unit is a contiguous token range
// [kv_begin, kv_end) of one request's page list (a split-KV segment).  For a
// unit the workgroup holds every query head of the request: wave w owns heads
// [w*16*NB, (w+1)*16*NB).  KV tiles of 32 tokens stream HBM -> LDS through the
// page table with direct-to-LDS loads (global_load_lds_dwordx4) into an
// NSTAGE-deep ring, so the shared latent tile is fetched once per workgroup and
// read by all waves.  Per tile and wave:
//   QK  S^T[token, head] = K[token, 576] . Q^T[576, head]     (MFMA 16x16x32 bf16,
//       K from LDS, Q held in registers for the whole unit)
//   online softmax per head (running max m, running sum l, rescale of O)
//   PV  O^T[dim, head] += V^T[dim, token] . P^T[token, head]  (V^T read from the
//       same LDS tile with ds_read_b64_tr_b16, P^T straight from the QK result)
// The epilogue writes bf16 out and fp32 lse, or an fp32 partial state that the
// merge kernel combines by log-sum-exp.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

#include "pkvmla_device.h"

namespace pkvmla {

// Loads per tile issued by `wave`: the 32 ckv rows go round-robin over the
// waves, the 4 kpe blocks (8 tokens each) to waves 0..3.
template <int NW>
__device__ __forceinline__ constexpr int loads_per_tile(int wave) {
  return kTile / NW + ((NW >= 4) ? (wave < 4 ? 1 : 0) : 4 / NW);
}

// Page ids of one KV tile, as far as this wave needs them to issue its loads.
// Read with wave-uniform addresses, i.e. through the scalar cache, one tile
// ahead of the copies that use them, so the scalar-load latency never sits
// between a tile becoming free and its next copy starting.  When a page holds
// whole tiles (page_size >= 32; tiles start at multiples of 32 tokens) one id
// serves the entire tile.  Otherwise each token's id is read unclamped (the
// device index table carries kIndexPad valid trailing entries, so the read
// stays inside it) and tokens past kv_end use the row of the last valid token
// instead: slots past kv_len and unlisted pages are never copied, and every
// copied row is finite data whose probability is masked to exactly zero.
template <int NW, bool BIG>
struct TilePages {
  static constexpr int kRows = kTile / NW;                  // ckv rows copied by this wave
  static constexpr int kKpe = (4 + NW - 1) / NW;            // kpe blocks of 8 tokens (bound)
  static constexpr int kIds = BIG ? 1 : kRows;
  static constexpr int kKpeIds = (BIG || NW == 1) ? 1 : kKpe * 8;  // one wave reuses its ckv ids
  int pc[kIds];
  int pk[kKpeIds];
  int plast;  // page id of the last valid token of the tile
};

template <int NW, bool BIG>
__device__ __forceinline__ void load_tile_pages(TilePages<NW, BIG>& tp,
                                                const int32_t* __restrict__ pages, int log2_ps,
                                                int tok0, int kv_end, int wave) {
  if constexpr (BIG) {
    tp.pc[0] = pages[tok0 >> log2_ps];
  } else {
    const int last = min(kv_end - 1 - tok0, kTile - 1);
    tp.plast = pages[(tok0 + last) >> log2_ps];
#pragma unroll
    for (int k = 0; k < TilePages<NW, BIG>::kRows; ++k)
      tp.pc[k] = pages[(tok0 + k * NW + wave) >> log2_ps];
    if constexpr (NW > 1) {
#pragma unroll
      for (int jj = 0; jj < TilePages<NW, BIG>::kKpe; ++jj) {
        const int j = jj * NW + wave;
#pragma unroll
        for (int k = 0; k < 8; ++k)
          tp.pk[jj * 8 + k] = (j < 4) ? pages[(tok0 + 8 * j + k) >> log2_ps] : 0;
      }
    }
  }
}

// Issue the direct-to-LDS loads [K0, K1) of this wave's share of one KV tile:
// index k < kRows is ckv row k*NW + wave, then kpe block (k - kRows)*NW + wave
// (8 tokens, 64 lanes x 16 bytes).  Splitting the issue lets the loads of the
// next tile go out between the MFMAs of the current one.
// K0/K1 are compile-time constants at every call site once the caller's loop
// is unrolled, so the page-id arrays are always indexed statically.
template <int NW, bool BIG>
__device__ __forceinline__ void issue_dma(const TilePages<NW, BIG>& tp,
                                          const uint16_t* __restrict__ ckv,
                                          const uint16_t* __restrict__ kpe, int log2_ps, int tok0,
                                          int kv_end, uint32_t stage_base, int wave, int lane,
                                          const int K0, const int K1) {
  constexpr int kRows = TilePages<NW, BIG>::kRows;
  constexpr int kKpe = TilePages<NW, BIG>::kKpe;
  const int ps_mask = (1 << log2_ps) - 1;
  const int last = kv_end - 1 - tok0;
  const char* ckv_b = reinterpret_cast<const char*>(ckv);
  const char* kpe_b = reinterpret_cast<const char*>(kpe);
  size_t base = 0, row_last = 0;
  if constexpr (BIG) {
    base = ((size_t)(uint32_t)tp.pc[0] << log2_ps) + (size_t)(tok0 & ps_mask);
  } else {
    const int tlast = min(last, kTile - 1);
    row_last = ((size_t)(uint32_t)tp.plast << log2_ps) + (size_t)((tok0 + tlast) & ps_mask);
  }
#pragma unroll
  for (int k = K0; k < K1 && k < kRows; ++k) {
    const int t = k * NW + wave;
    size_t row;
    if constexpr (BIG) {
      row = base + (size_t)min(t, last);
    } else {
      const size_t row_t = ((size_t)(uint32_t)tp.pc[k] << log2_ps) + (size_t)((tok0 + t) & ps_mask);
      row = t <= last ? row_t : row_last;
    }
    dma16(ckv_b + row * (kCkvDim * 2) + ((lane ^ swz16(t)) << 4), stage_base + t * 1024);
  }
#pragma unroll
  for (int jj = (K0 > kRows ? K0 - kRows : 0); jj < kKpe && kRows + jj < K1; ++jj) {
    const int j = jj * NW + wave;
    if (j < 4) {
      const int t = 8 * j + (lane >> 3);
      size_t row;
      if constexpr (BIG) {
        row = base + (size_t)min(t, last);
      } else {
        int pg;
        if constexpr (NW == 1) {
          pg = tp.pc[8 * j];
#pragma unroll
          for (int k = 1; k < 8; ++k) pg = ((lane >> 3) == k) ? tp.pc[8 * j + k] : pg;
        } else {
          pg = tp.pk[jj * 8];
#pragma unroll
          for (int k = 1; k < 8; ++k) pg = ((lane >> 3) == k) ? tp.pk[jj * 8 + k] : pg;
        }
        const size_t row_t = ((size_t)(uint32_t)pg << log2_ps) + (size_t)((tok0 + t) & ps_mask);
        row = t <= last ? row_t : row_last;
      }
      dma16(kpe_b + row * (kKpeDim * 2) + (((lane & 7) ^ swz8(t)) << 4),
            stage_base + kTile * 1024 + j * 1024);
    }
  }
}

// All of this wave's loads of one KV tile.
template <int NW, bool BIG>
__device__ __forceinline__ void issue_tile(const TilePages<NW, BIG>& tp,
                                           const uint16_t* __restrict__ ckv,
                                           const uint16_t* __restrict__ kpe, int log2_ps,
                                           int tok0, int kv_end, uint32_t stage_base,
                                           int wave, int lane) {
  issue_dma<NW, BIG>(tp, ckv, kpe, log2_ps, tok0, kv_end, stage_base, wave, lane, 0, 64);
}

// Wait until this wave's loads of all but the last `pending` issued tiles landed.
template <int NW, int PENDING>
__device__ __forceinline__ void wait_tiles(int wave) {
  if constexpr (NW >= 8) {
    if (wave < 4) wait_vmcnt<PENDING * loads_per_tile<NW>(0)>();
    else wait_vmcnt<PENDING * loads_per_tile<NW>(4)>();
  } else {
    wait_vmcnt<PENDING * loads_per_tile<NW>(0)>();
  }
}

// ---------------------------------------------------------------------------
// Fused decode kernel.  NW waves x NB head blocks of 16 = heads per request.
// ---------------------------------------------------------------------------
template <int NW, int NB, int NSTAGE, bool BIG>
__global__ void __launch_bounds__(NW * 64)
mla_decode_kernel(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
                  const uint16_t* __restrict__ ckv, const uint16_t* __restrict__ kpe,
                  uint16_t* __restrict__ out, float* __restrict__ lse_out,
                  uint16_t* __restrict__ part_o, float* __restrict__ part_lse,
                  const int32_t* __restrict__ wg_indptr, const int32_t* __restrict__ units,
                  const int32_t* __restrict__ seq_indptr,
                  const int32_t* __restrict__ seq_indices, int H, int n_hg, int n_lanes,
                  int log2_ps, float sm_scale, float C, float rescale_thr) {
  static_assert(NSTAGE >= 2, "need at least double buffering");
  static_assert(kTile / NW * NW == kTile, "waves must divide the tile");
  constexpr int HBN = NW * NB;       // head blocks of 16 in the workgroup
  constexpr int DBW = 32 / NW;       // output-dim blocks of 16 owned by each wave in PV
  constexpr int NDMA = kTile / NW + (4 + NW - 1) / NW;
  constexpr int DMA_PER_STEP = (NDMA + 17) / 18;
  // LDS: NSTAGE tile stages, then the P^T exchange (1 KB per head block) and
  // one float per head (rescale factors, later row sums).
  constexpr int xp_off = NSTAGE * kStageBytes;
  constexpr int xa_off = xp_off + HBN * 1024;
  __shared__ __attribute__((aligned(1024))) char smem_raw[xa_off + HBN * 16 * 4];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;    // 16-lane group
  const int li = lane & 15;
  // Workgroups are dispatched round-robin over the 8 XCDs (block b on XCD
  // b % 8).  The head-group replicas of one schedule lane take blocks
  // b, b+8, ..., so they share an XCD's L2 and start together: the KV tile
  // they all read comes from HBM once.
  const int hg = (blockIdx.x >> 3) % n_hg;
  const int sl = (blockIdx.x / (8 * n_hg)) * 8 + (blockIdx.x & 7);
  if (sl >= n_lanes) return;
  const int head0 = hg * (NW * NB * 16);
  const int u_begin = wg_indptr[sl];
  const int u_end = wg_indptr[sl + 1];

  // Per-lane LDS offsets that do not depend on the unit (stage-relative).
  // QK A operand: token t = tb*16 + li, chunk ks*4 + g  -> base ^ (ks << 6)
  int offA[2], offK[2];
  // PV V^T operand (transposed read): source lane (g, r = li/4, q = li%4)
  // addresses token tb*16 + g*4 + r, dims db*16 + 4q..4q+3 -> base ^ (db << 5)
  int offV[2];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int tA = tb * 16 + li;
    offA[tb] = lds_ckv_off(tA, g);
    offK[tb] = lds_kpe_off(tA, g);
    const int tV = tb * 16 + g * 4 + (li >> 2);
    const int q = li & 3;
    offV[tb] = lds_ckv_off(tV, q >> 1) + (q & 1) * 8;
  }

  for (int u = u_begin; u < u_end; ++u) {
    const int32_t* rec = units + (size_t)u * kUnitInts;
    const int b = rec[0];
    const int seq = rec[1];
    const int kv0 = rec[2];
    const int kv1 = rec[3];
    const int slot = rec[4];
    const int32_t* pages = seq_indices + seq_indptr[seq];
    const int ntiles = (kv1 - kv0 + kTile - 1) / kTile;

    __syncthreads();  // all waves are done with the previous unit's stages

    // Tile 0 first, then the query; one full vector-memory wait covers both, so
    // the compiler's own wait tracking sees the query registers as complete
    // before the loop (it does not see the tile loads, which are inline asm).
    TilePages<NW, BIG> tp;
    load_tile_pages<NW, BIG>(tp, pages, log2_ps, kv0, kv1, wave);
    issue_tile<NW, BIG>(tp, ckv, kpe, log2_ps, kv0, kv1, smem_base, wave, lane);

    // Q^T operand, registers for the whole unit: lane (g, li) holds
    // Q[head nb*16 + li][ks*32 + g*8 .. +7].
    bf16x8_t q[NB][18];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int h = head0 + wave * (16 * NB) + nb * 16 + li;
      const bf16x8_t* qn = reinterpret_cast<const bf16x8_t*>(
          q_nope + ((size_t)b * H + h) * kCkvDim + g * 8);
      const bf16x8_t* qp = reinterpret_cast<const bf16x8_t*>(
          q_pe + ((size_t)b * H + h) * kKpeDim + g * 8);
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) q[nb][ks] = qn[ks * 4];
      q[nb][16] = qp[0];
      q[nb][17] = qp[4];
    }
    wait_vmcnt<0>();

#pragma unroll
    for (int s = 1; s < NSTAGE - 1; ++s) {
      if (s < ntiles) {
        load_tile_pages<NW, BIG>(tp, pages, log2_ps, kv0 + s * kTile, kv1, wave);
        issue_tile<NW, BIG>(tp, ckv, kpe, log2_ps, kv0 + s * kTile, kv1,
                            smem_base + s * kStageBytes, wave, lane);
      }
    }
    // page ids of the next tile to issue are always fetched one iteration early
    if (NSTAGE - 1 < ntiles)
      load_tile_pages<NW, BIG>(tp, pages, log2_ps, kv0 + (NSTAGE - 1) * kTile, kv1, wave);

    // Softmax state of this wave's own heads (rows of S it computes).
    float m_run[NB], l_run[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_run[nb] = -INFINITY;
      l_run[nb] = 0.f;
    }
    // PV accumulators: this wave's DBW output-dim blocks for all HBN head blocks.
    f32x4_t o[DBW][HBN];
#pragma unroll
    for (int db = 0; db < DBW; ++db)
#pragma unroll
      for (int hb = 0; hb < HBN; ++hb) o[db][hb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int it = 0; it < ntiles; ++it) {
      // this wave's loads of tile `it` have landed (later tiles may still fly)
      const int later = min(NSTAGE - 2, ntiles - 1 - it);
      if (NSTAGE >= 4 && later >= 2) wait_tiles<NW, (NSTAGE >= 4 ? 2 : 0)>(wave);
      else if (NSTAGE >= 3 && later >= 1) wait_tiles<NW, (NSTAGE >= 3 ? 1 : 0)>(wave);
      else wait_tiles<NW, 0>(wave);
      __syncthreads();  // tile `it` landed for every wave; tile it-1 and its P exchange are consumed
      // Per-lane LDS offsets and the lane id go through an empty asm each tile:
      // otherwise the compiler hoists every derived operand address out of
      // the loop and spills them, and a spill reload inside the loop would
      // wait for all outstanding tile loads.
      int oA0 = offA[0], oA1 = offA[1], oK0 = offK[0], oK1 = offK[1], oV0 = offV[0], oV1 = offV[1];
      int lane_o = lane;
      asm volatile("" : "+v"(oA0), "+v"(oA1), "+v"(oK0), "+v"(oK1), "+v"(oV0), "+v"(oV1), "+v"(lane_o));
      const int nt = it + NSTAGE - 1;          // tile whose loads go out during this QK
      const bool issue = nt < ntiles;
      const uint32_t nt_base = smem_base + (nt % NSTAGE) * kStageBytes;
      const int nt_tok0 = kv0 + nt * kTile;
      const int stage_off = (it % NSTAGE) * kStageBytes;
      const int tok0 = kv0 + it * kTile;
      const int valid = kv1 - tok0;

      // ---- QK: 18 k-steps of 32 dims, A fragments prefetched, next tile's
      // loads interleaved (DMA_PER_STEP per k-step) ----
      f32x4_t sacc[2][NB];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sacc[tb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int a0 = stage_off + oA0, a1 = stage_off + oA1;
      const int k0 = stage_off + oK0, k1 = stage_off + oK1;
      auto ldA = [&](int ks, int tb) -> bf16x8_t {
        const int off = ks < 16 ? ((tb ? a1 : a0) ^ (ks << 6)) : ((tb ? k1 : k0) ^ ((ks - 16) << 6));
        return *(const LDS_AS bf16x8_t*)(smem + off);
      };
      constexpr int AP = NB >= 2 ? 1 : 2;
      bf16x8_t A[AP + 1][2];
#pragma unroll
      for (int pp = 0; pp < AP; ++pp) {
        A[pp][0] = ldA(pp, 0);
        A[pp][1] = ldA(pp, 1);
      }
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
        if (issue) {
          issue_dma<NW, BIG>(tp, ckv, kpe, log2_ps, nt_tok0, kv1, nt_base, wave, lane_o,
                             ks * DMA_PER_STEP, (ks + 1) * DMA_PER_STEP);
        }
        if (ks + AP < 18) {
          A[(ks + AP) % (AP + 1)][0] = ldA(ks + AP, 0);
          A[(ks + AP) % (AP + 1)][1] = ldA(ks + AP, 1);
        }
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            sacc[tb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[ks % (AP + 1)][tb], q[nb][ks],
                                                                   sacc[tb][nb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (issue && nt + 1 < ntiles)
        load_tile_pages<NW, BIG>(tp, pages, log2_ps, kv0 + (nt + 1) * kTile, kv1, wave);

      // ---- online softmax of this wave's heads (per lane: one head, 8 tokens) ----
      bf16x8_t pT[NB];
      float alpha_own[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float sv[8];
        float mx = -INFINITY;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = tb * 16 + g * 4 + i;
            const float v = (t < valid) ? sacc[tb][nb][i] : -INFINITY;
            sv[tb * 4 + i] = v;
            mx = fmaxf(mx, v);
          }
        mx = max_over_rows(mx);
        // Lazy running max: the reference m moves only when the tile max exceeds
        // it by more than rescale_thr (probabilities stay <= 2^8, exact in
        // fp32/bf16 range), so O is rarely rescaled.  The first tile always sets m.
        const bool grow = mx > m_run[nb] + rescale_thr;
        const float m_new = grow ? mx : m_run[nb];
        alpha_own[nb] = __builtin_amdgcn_exp2f((m_run[nb] - m_new) * C);
        m_run[nb] = m_new;
        const float mc = m_new * C;
        float psum = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sv[k], C, -mc));
          psum += e;
          pT[nb][k] = (__bf16)e;
        }
        l_run[nb] = l_run[nb] * alpha_own[nb] + psum;
      }

      // ---- exchange: every wave's P^T fragments and rescale factors ----
      bf16x8_t pB[HBN];
      float alpha[HBN];
      if constexpr (NW == 1) {
#pragma unroll
        for (int hb = 0; hb < HBN; ++hb) {
          pB[hb] = pT[hb];
          alpha[hb] = alpha_own[hb];
        }
      } else {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int hb = wave * NB + nb;
          *(LDS_AS bf16x8_t*)(smem + xp_off + hb * 1024 + lane * 16) = pT[nb];
          if (g == 0) *(LDS_AS float*)(smem + xa_off + (hb * 16 + li) * 4) = alpha_own[nb];
        }
        __syncthreads();
#pragma unroll
        for (int hb = 0; hb < HBN; ++hb) {
          pB[hb] = *(const LDS_AS bf16x8_t*)(smem + xp_off + hb * 1024 + lane * 16);
          alpha[hb] = *(const LDS_AS float*)(smem + xa_off + (hb * 16 + li) * 4);
        }
      }
      // Rescale O only when some head's reference max moved (never on the
      // unit's first tile, where O is still zero).  The empty asm statements
      // pin the accumulators to AGPRs so the MFMAs keep their AGPR form; the
      // multiply itself goes through VGPRs (compiler-generated moves).
      if (it > 0) {
        bool need = false;
#pragma unroll
        for (int hb = 0; hb < HBN; ++hb) need |= alpha[hb] != 1.0f;
        if (__builtin_amdgcn_ballot_w64(need)) {
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

      // ---- PV over this wave's dims: V^T fragments (transposed reads of the
      // same LDS tile) feed HBN MFMAs each ----
      const int v0 = stage_off + oV0, v1 = stage_off + oV1;
      auto ldV = [&](int db, int tb) -> bf16x4_t {
        const int dbg = wave * DBW + db;
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4_t*)(smem + ((tb ? v1 : v0) ^ (dbg << 5))));
      };
      constexpr int VP = 2;
      bf16x4_t V[VP + 1][2];
#pragma unroll
      for (int pp = 0; pp < VP && pp < DBW; ++pp) {
        V[pp][0] = ldV(pp, 0);
        V[pp][1] = ldV(pp, 1);
      }
#pragma unroll
      for (int db = 0; db < DBW; ++db) {
        if (db + VP < DBW) {
          V[(db + VP) % (VP + 1)][0] = ldV(db + VP, 0);
          V[(db + VP) % (VP + 1)][1] = ldV(db + VP, 1);
        }
        const bf16x8_t a = __builtin_shufflevector(V[db % (VP + 1)][0], V[db % (VP + 1)][1], 0, 1, 2,
                                                   3, 4, 5, 6, 7);
#pragma unroll
        for (int hb = 0; hb < HBN; ++hb)
          o[db][hb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pB[hb], o[db][hb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- epilogue: row sums and maxima of every head, then this wave's dims ----
    float linv[HBN], lse_v[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float l = l_run[nb];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      l_run[nb] = l;
      lse_v[nb] = m_run[nb] * sm_scale + __builtin_amdgcn_logf(l) * 0.69314718055994531f;
    }
    if constexpr (NW == 1) {
#pragma unroll
      for (int hb = 0; hb < HBN; ++hb) linv[hb] = 1.0f / l_run[hb];
    } else {
      __syncthreads();  // every wave is done reading the exchange area
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        if (g == 0) *(LDS_AS float*)(smem + xa_off + ((wave * NB + nb) * 16 + li) * 4) = l_run[nb];
      __syncthreads();
#pragma unroll
      for (int hb = 0; hb < HBN; ++hb) linv[hb] = 1.0f / *(const LDS_AS float*)(smem + xa_off + (hb * 16 + li) * 4);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int h = head0 + (wave * NB + nb) * 16 + li;
      if (g == 0) {
        if (slot < 0) lse_out[(size_t)b * H + h] = lse_v[nb];
        else part_lse[(size_t)slot * H + h] = lse_v[nb];
      }
    }
#pragma unroll
    for (int hb = 0; hb < HBN; ++hb) {
      const int h = head0 + hb * 16 + li;
      // a whole request's row goes to out, a split unit's to its partial slot (both bf16)
      uint16_t* orow = (slot < 0 ? out + ((size_t)b * H + h) * kCkvDim
                                 : part_o + ((size_t)slot * H + h) * kCkvDim) +
                       wave * (DBW * 16) + g * 4;
#pragma unroll
      for (int db = 0; db < DBW; ++db) {
        const f32x4_t v = o[db][hb] * linv[hb];
        const uint32_t lo = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
        *reinterpret_cast<uint2*>(orow + db * 16) = make_uint2(lo, hi);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split-KV merge: per (request, head) combine the partial states by
// log-sum-exp: lse = M + ln sum_i e^(lse_i - M), out = sum_i e^(lse_i - lse) o_i.
// The partial outputs o_i are bf16 (each already normalized by its own row
// sum), the combination runs in fp32.  Block: 4 heads x 64 lanes, 8 dims per
// lane (one 16-byte load per partial row).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) mla_merge_kernel(MergeParams p) {
  const int32_t* mr = p.merges + (size_t)blockIdx.x * kMergeInts;
  const int b = mr[0], s0 = mr[1], n = mr[2];
  const int H = p.num_heads;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int d0 = (threadIdx.x & 63) * 8;
  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, p.part_lse[(size_t)(s0 + i) * H + h]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int i = 0; i < n; ++i) {
    const size_t base = (size_t)(s0 + i) * H + h;
    const float w = __builtin_amdgcn_exp2f((p.part_lse[base] - M) * 1.4426950408889634f);
    const uint4 x = *reinterpret_cast<const uint4*>(p.part_o + base * kCkvDim + d0);
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[2 * k] = fmaf(w, __builtin_bit_cast(float, xw[k] << 16), acc[2 * k]);
      acc[2 * k + 1] = fmaf(w, __builtin_bit_cast(float, xw[k] & 0xFFFF0000u), acc[2 * k + 1]);
    }
    wsum += w;
  }
  const float inv = 1.0f / wsum;
  uint32_t packed[4];
#pragma unroll
  for (int k = 0; k < 4; ++k)
    packed[k] = (uint32_t)f32_to_bf16_rne(acc[2 * k] * inv) |
                ((uint32_t)f32_to_bf16_rne(acc[2 * k + 1] * inv) << 16);
  *reinterpret_cast<uint4*>(p.out + ((size_t)b * H + h) * kCkvDim + d0) =
      make_uint4(packed[0], packed[1], packed[2], packed[3]);
  if ((threadIdx.x & 63) == 0)
    p.lse[(size_t)b * H + h] = M + __builtin_amdgcn_logf(wsum) * 0.69314718055994531f;
}

// ---------------------------------------------------------------------------
// Gather through the decode kernel's load path: issue_tile into LDS, then copy
// each valid token's ckv and kpe chunks back out of the swizzled tile.
// ---------------------------------------------------------------------------
template <bool BIG>
__global__ void __launch_bounds__(256)
mla_gather_kernel(const uint16_t* __restrict__ ckv, const uint16_t* __restrict__ kpe,
                  uint16_t* __restrict__ rows, const int32_t* __restrict__ units,
                  const int32_t* __restrict__ seq_indptr,
                  const int32_t* __restrict__ seq_indices, int log2_ps) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kStageBytes];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int32_t* rec = units + (size_t)blockIdx.x * kUnitInts;
  const int seq = rec[1], kv0 = rec[2], kv1 = rec[3], row0 = rec[5];
  const int32_t* pages = seq_indices + seq_indptr[seq];
  for (int tok0 = kv0; tok0 < kv1; tok0 += kTile) {
    __syncthreads();
    TilePages<4, BIG> tp;
    load_tile_pages<4, BIG>(tp, pages, log2_ps, tok0, kv1, wave);
    issue_tile<4, BIG>(tp, ckv, kpe, log2_ps, tok0, kv1, smem_base, wave, lane);
    wait_vmcnt<0>();
    __syncthreads();
    const int n = min(kTile, kv1 - tok0);
    for (int idx = threadIdx.x; idx < n * 72; idx += 256) {
      const int t = idx / 72, c = idx % 72;
      const int src = c < 64 ? lds_ckv_off(t, c) : lds_kpe_off(t, c - 64);
      const u32x4_t v = *(const LDS_AS u32x4_t*)(smem + src);
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(rows + ((size_t)row0 + (tok0 - kv0) + t) * 576) + c;
      *dst = v;
    }
  }
}

// ---------------------------------------------------------------------------
// Host side: configuration table and launchers.
// ---------------------------------------------------------------------------
bool kernel_config_for(int num_heads, KernelConfig* cfg) {
  switch (num_heads) {
    case 16: *cfg = KernelConfig{5, 16, 4, 1, 2, 1}; break;
    case 32: *cfg = KernelConfig{6, 16, 4, 1, 2, 1}; break;
    case 64: *cfg = KernelConfig{8, 16, 4, 1, 4, 1}; break;
    case 128: *cfg = KernelConfig{8, 16, 4, 1, 4, 2}; break;
    default: return false;
  }
  // Experiments only: PKVMLA_CONFIG="waves,heads_per_wave,stages,wg_per_cu,fixed,head_groups"
  // overrides the table when that kernel shape exists for num_heads.
  if (const char* e = getenv("PKVMLA_CONFIG")) {
    KernelConfig c{};
    if (sscanf(e, "%d,%d,%d,%d,%d,%d", &c.waves, &c.heads_per_wave, &c.stages, &c.wg_per_cu,
               &c.fixed_cost, &c.head_groups) == 6 &&
        c.head_groups >= 1 && c.wg_per_cu >= 1 && c.fixed_cost >= 0) {
      const bool rs = c.stages == 4 &&
                      decode_rs_head_blocks(c.waves, c.heads_per_wave, num_heads, c.head_groups);
      const bool generic = c.heads_per_wave == 16 && c.stages == 2 &&
                           (c.waves == 1 || c.waves == 2) &&
                           c.waves * c.heads_per_wave * c.head_groups == num_heads;
      if (rs || generic) *cfg = c;
    }
  }
  return true;
}

int decode_grid(int n_lanes, int head_groups) {
  return ((n_lanes + 7) / 8) * 8 * head_groups;
}

#define PKVMLA_DECODE_ARGS                                                               \
  p.q_nope, p.q_pe, p.ckv, p.kpe, p.out, p.lse, p.part_o, p.part_lse, p.wg_indptr, p.units, \
      p.seq_indptr, p.seq_indices, p.num_heads, p.head_groups, p.n_lanes, p.log2_ps,      \
      p.sm_scale, p.score_log2, p.rescale_thr

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.n_lanes <= 0) return hipSuccess;
  hipError_t err = hipSuccess;
  if (launch_decode_rs(p, stream, &err)) return err;
  const int grid = decode_grid(p.n_lanes, p.head_groups);
  // big: every page holds whole 32-token tiles (page_size >= 32)
  const int key = p.waves * 10000 + p.heads_per_wave * 100 + p.stages * 10 + (p.log2_ps >= 5);
  switch (key) {
#define PKVMLA_CASE(W, NB, S, BIG)                                                         \
  case W * 10000 + NB * 1600 + S * 10 + BIG:                                               \
    mla_decode_kernel<W, NB, S, BIG><<<grid, W * 64, 0, stream>>>(PKVMLA_DECODE_ARGS);     \
    break;
    PKVMLA_CASE(1, 1, 2, 0) PKVMLA_CASE(1, 1, 2, 1)
    PKVMLA_CASE(2, 1, 2, 0) PKVMLA_CASE(2, 1, 2, 1)
    PKVMLA_CASE(4, 1, 4, 0) PKVMLA_CASE(4, 1, 4, 1)
    PKVMLA_CASE(4, 2, 4, 0) PKVMLA_CASE(4, 2, 4, 1)
#undef PKVMLA_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeParams& p, int n_merges, hipStream_t stream) {
  if (n_merges <= 0) return hipSuccess;
  dim3 grid(n_merges, p.num_heads / 4);
  mla_merge_kernel<<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherParams& p, int n_units, hipStream_t stream) {
  if (n_units <= 0) return hipSuccess;
  if (p.log2_ps >= 5)
    mla_gather_kernel<true><<<n_units, 256, 0, stream>>>(p.ckv, p.kpe, p.rows, p.units,
                                                         p.seq_indptr, p.seq_indices, p.log2_ps);
  else
    mla_gather_kernel<false><<<n_units, 256, 0, stream>>>(p.ckv, p.kpe, p.rows, p.units,
                                                          p.seq_indptr, p.seq_indices, p.log2_ps);
  return hipGetLastError();
}

}  // namespace pkvmla
