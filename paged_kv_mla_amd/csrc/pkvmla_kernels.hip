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

#include "pkvmla_internal.h"

#define LDS_AS __attribute__((address_space(3)))
#define GLB_AS __attribute__((address_space(1)))

namespace pkvmla {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(16)));
typedef __bf16 bf16x4_t __attribute__((__vector_size__(8)));
typedef float f32x4_t __attribute__((__vector_size__(16)));
typedef uint32_t u32x4_t __attribute__((__vector_size__(16)));

// ---------------------------------------------------------------------------
// LDS tile layout (one stage, 36864 bytes):
//   [0, 32768)      ckv rows: token t at t*1024, its 16-byte chunk c (dims
//                   8c..8c+7) at chunk position c ^ swz16(t)
//   [32768, 36864)  kpe rows: token t at 32768 + t*128, chunk c at c ^ (t & 7)
// The XOR swizzles keep the MFMA operand reads free of bank conflicts: 16
// consecutive tokens reading one chunk hit 16 different 16-byte bank groups,
// and the transposed V reads (4 tokens x 2 chunks per 16 lanes) hit 8.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz16(int t) {
  return ((t & 3) << 1) | ((t >> 2) & 1) | (t & 8);
}
__device__ __forceinline__ int lds_ckv_off(int t, int c) {
  return t * 1024 + ((c ^ swz16(t)) << 4);
}
__device__ __forceinline__ int lds_kpe_off(int t, int c) {
  return kTile * 1024 + t * 128 + ((c ^ (t & 7)) << 4);
}

// gfx9 s_waitcnt immediate: wait until at most N vector-memory ops are
// outstanding (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Direct HBM -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane i
// of the wave lands at LDS byte lds_base + 16*i.  Issued through inline asm so
// that the compiler neither reorders it nor inserts its own conservative
// vector-memory waits before every LDS read; completion is tracked explicitly
// with s_waitcnt vmcnt before the workgroup barrier that publishes a tile.
// M0 (the LDS base register of the instruction) is saved and restored.
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

// Loads per tile issued by `wave`: the 32 ckv rows go round-robin over the
// waves, the 4 kpe blocks (8 tokens each) to waves 0..3.
template <int NW>
__device__ __forceinline__ constexpr int loads_per_tile(int wave) {
  return kTile / NW + ((NW >= 4) ? (wave < 4 ? 1 : 0) : 4 / NW);
}

// Issue this wave's share of the direct-to-LDS loads of one KV tile.
// Tokens past kv_end are clamped to the last valid token (finite data; their
// scores are masked and their probabilities are exactly zero), so slots past
// kv_len and unlisted pages are never read.  Every page id is read with a
// wave-uniform address, i.e. through the scalar cache, so the vector-memory
// counter only ever tracks the tile loads themselves.
template <int NW>
__device__ __forceinline__ void issue_tile(const uint16_t* __restrict__ ckv,
                                           const uint16_t* __restrict__ kpe,
                                           const int32_t* __restrict__ pages, int log2_ps,
                                           int tok0, int kv_end, uint32_t stage_base,
                                           int wave, int lane) {
  const int ps_mask = (1 << log2_ps) - 1;
#pragma unroll
  for (int k = 0; k < kTile / NW; ++k) {
    const int t = k * NW + wave;
    const int tok = min(tok0 + t, kv_end - 1);
    const int page = pages[tok >> log2_ps];
    const size_t row = ((size_t)(uint32_t)page << log2_ps) + (size_t)(tok & ps_mask);
    const char* src = reinterpret_cast<const char*>(ckv) + row * (kCkvDim * 2) +
                      ((lane ^ swz16(t)) << 4);
    dma16(src, stage_base + t * 1024);
  }
  // kpe: 4 loads of 8 tokens (64 lanes x 16 bytes); lane -> token 8j + lane/8
#pragma unroll
  for (int jj = 0; jj < (4 + NW - 1) / NW; ++jj) {
    const int j = jj * NW + wave;
    if (j < 4) {
      int pg = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int tk = min(tok0 + 8 * j + k, kv_end - 1);
        const int pk = pages[tk >> log2_ps];
        pg = ((lane >> 3) == k) ? pk : pg;
      }
      const int t = 8 * j + (lane >> 3);
      const int tok = min(tok0 + t, kv_end - 1);
      const size_t row = ((size_t)(uint32_t)pg << log2_ps) + (size_t)(tok & ps_mask);
      const char* src = reinterpret_cast<const char*>(kpe) + row * (kKpeDim * 2) +
                        (((lane & 7) ^ (t & 7)) << 4);
      dma16(src, stage_base + kTile * 1024 + j * 1024);
    }
  }
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

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// Fused decode kernel.  NW waves x NB head blocks of 16 = heads per request.
// ---------------------------------------------------------------------------
template <int NW, int NB, int NSTAGE>
__global__ void __launch_bounds__(NW * 64)
mla_decode_kernel(const uint16_t* __restrict__ q_nope, const uint16_t* __restrict__ q_pe,
                  const uint16_t* __restrict__ ckv, const uint16_t* __restrict__ kpe,
                  uint16_t* __restrict__ out, float* __restrict__ lse_out,
                  float* __restrict__ part_o, float* __restrict__ part_lse,
                  const int32_t* __restrict__ wg_indptr, const int32_t* __restrict__ units,
                  const int32_t* __restrict__ seq_indptr,
                  const int32_t* __restrict__ seq_indices, int H, int log2_ps,
                  float sm_scale, float C) {
  static_assert(NSTAGE >= 2, "need at least double buffering");
  static_assert(kTile / NW * NW == kTile, "waves must divide the tile");
  __shared__ __attribute__((aligned(1024))) char smem_raw[NSTAGE * kStageBytes];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;    // 16-lane group
  const int li = lane & 15;
  const int u_begin = wg_indptr[blockIdx.x];
  const int u_end = wg_indptr[blockIdx.x + 1];

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
    issue_tile<NW>(ckv, kpe, pages, log2_ps, kv0, kv1, smem_base, wave, lane);

    // Q^T operand, registers for the whole unit: lane (g, li) holds
    // Q[head nb*16 + li][ks*32 + g*8 .. +7].
    bf16x8_t q[NB][18];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int h = wave * (16 * NB) + nb * 16 + li;
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
      if (s < ntiles)
        issue_tile<NW>(ckv, kpe, pages, log2_ps, kv0 + s * kTile, kv1,
                       smem_base + s * kStageBytes, wave, lane);
    }

    float m_run[NB], l_run[NB];
    f32x4_t o[NB][32];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_run[nb] = -INFINITY;
      l_run[nb] = 0.f;
#pragma unroll
      for (int db = 0; db < 32; ++db) o[nb][db] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    for (int it = 0; it < ntiles; ++it) {
      // this wave's loads of tile `it` have landed (later tiles may still fly)
      const int later = min(NSTAGE - 2, ntiles - 1 - it);
      if (NSTAGE >= 4 && later >= 2) wait_tiles<NW, (NSTAGE >= 4 ? 2 : 0)>(wave);
      else if (NSTAGE >= 3 && later >= 1) wait_tiles<NW, (NSTAGE >= 3 ? 1 : 0)>(wave);
      else wait_tiles<NW, 0>(wave);
      __syncthreads();  // every wave's loads of tile `it` landed; tile it-1 is consumed
      {
        const int nt = it + NSTAGE - 1;
        if (nt < ntiles)
          issue_tile<NW>(ckv, kpe, pages, log2_ps, kv0 + nt * kTile, kv1,
                         smem_base + (nt % NSTAGE) * kStageBytes, wave, lane);
      }
      const int stage_off = (it % NSTAGE) * kStageBytes;
      const int tok0 = kv0 + it * kTile;
      const int valid = kv1 - tok0;

      // ---- QK: 18 k-steps of 32 dims, A fragments prefetched two steps ahead ----
      f32x4_t sacc[2][NB];
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sacc[tb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      const int a0 = stage_off + offA[0], a1 = stage_off + offA[1];
      const int k0 = stage_off + offK[0], k1 = stage_off + offK[1];
      auto ldA = [&](int ks, int tb) -> bf16x8_t {
        const int off = ks < 16 ? ((tb ? a1 : a0) ^ (ks << 6)) : ((tb ? k1 : k0) ^ ((ks - 16) << 6));
        return *(const LDS_AS bf16x8_t*)(smem + off);
      };
      // prefetch distance: two k-steps, one when 32 heads per wave leave no room
      constexpr int AP = NB >= 2 ? 1 : 2;
      bf16x8_t A[AP + 1][2];
#pragma unroll
      for (int pp = 0; pp < AP; ++pp) {
        A[pp][0] = ldA(pp, 0);
        A[pp][1] = ldA(pp, 1);
      }
#pragma unroll
      for (int ks = 0; ks < 18; ++ks) {
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

      // ---- online softmax (per lane: one head, 8 tokens of the tile) ----
      bf16x8_t pT[NB];
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
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[nb], mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run[nb] - m_new) * C);
        m_run[nb] = m_new;
        const float mc = m_new * C;
        float psum = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sv[k], C, -mc));
          psum += e;
          pT[nb][k] = (__bf16)e;
        }
        l_run[nb] = l_run[nb] * alpha + psum;
        // Rescale O only when some head's running max moved (never on the
        // unit's first tile, where O is still zero).  The empty asm statements
        // pin the accumulators to AGPRs so the MFMAs keep their AGPR form; the
        // multiply itself goes through VGPRs (compiler-generated moves).
        if (it > 0 && __builtin_amdgcn_ballot_w64(alpha != 1.0f)) {
#pragma unroll
          for (int db = 0; db < 32; ++db) {
            asm volatile("" : "+a"(o[nb][db]));
            o[nb][db] *= alpha;
            asm volatile("" : "+a"(o[nb][db]));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- PV: 32 blocks of 16 output dims, V^T fragments prefetched two ahead ----
      const int v0 = stage_off + offV[0], v1 = stage_off + offV[1];
      auto ldV = [&](int db, int tb) -> bf16x4_t {
        return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (LDS_AS bf16x4_t*)(smem + ((tb ? v1 : v0) ^ (db << 5))));
      };
      bf16x4_t V[3][2];
      V[0][0] = ldV(0, 0);
      V[0][1] = ldV(0, 1);
      V[1][0] = ldV(1, 0);
      V[1][1] = ldV(1, 1);
#pragma unroll
      for (int db = 0; db < 32; ++db) {
        if (db + 2 < 32) {
          V[(db + 2) % 3][0] = ldV(db + 2, 0);
          V[(db + 2) % 3][1] = ldV(db + 2, 1);
        }
        const bf16x8_t a = __builtin_shufflevector(V[db % 3][0], V[db % 3][1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          o[nb][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pT[nb], o[nb][db], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // ---- epilogue ----
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      float l = l_run[nb];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      const float inv = 1.0f / l;
      const float lse_v = m_run[nb] * sm_scale + __builtin_amdgcn_logf(l) * 0.69314718055994531f;
      const int h = wave * (16 * NB) + nb * 16 + li;
      if (slot < 0) {
        uint16_t* orow = out + ((size_t)b * H + h) * kCkvDim + g * 4;
#pragma unroll
        for (int db = 0; db < 32; ++db) {
          const f32x4_t v = o[nb][db] * inv;
          const uint32_t lo = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
          *reinterpret_cast<uint2*>(orow + db * 16) = make_uint2(lo, hi);
        }
        if (g == 0) lse_out[(size_t)b * H + h] = lse_v;
      } else {
        float* prow = part_o + ((size_t)slot * H + h) * kCkvDim + g * 4;
#pragma unroll
        for (int db = 0; db < 32; ++db)
          *reinterpret_cast<f32x4_t*>(prow + db * 16) = o[nb][db] * inv;
        if (g == 0) part_lse[(size_t)slot * H + h] = lse_v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Split-KV merge: per (request, head) combine the partial states by
// log-sum-exp: lse = M + ln sum_i e^(lse_i - M), out = sum_i e^(lse_i - lse) o_i.
// Block: 4 heads x 64 lanes, 8 dims per lane.
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
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(p.part_o + base * kCkvDim + d0);
    const f32x4_t x0 = src[0], x1 = src[1];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      acc[k] = fmaf(w, x0[k], acc[k]);
      acc[4 + k] = fmaf(w, x1[k], acc[4 + k]);
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
    issue_tile<4>(ckv, kpe, pages, log2_ps, tok0, kv1, smem_base, wave, lane);
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
    case 16: *cfg = KernelConfig{1, 16, 2, 2, 1}; return true;
    case 32: *cfg = KernelConfig{2, 16, 2, 2, 1}; return true;
    case 64: *cfg = KernelConfig{4, 16, 4, 1, 2}; return true;
    case 128: *cfg = KernelConfig{4, 32, 4, 1, 2}; return true;
    default: return false;
  }
}

#define PKVMLA_DECODE_ARGS                                                               \
  p.q_nope, p.q_pe, p.ckv, p.kpe, p.out, p.lse, p.part_o, p.part_lse, p.wg_indptr, p.units, \
      p.seq_indptr, p.seq_indices, p.num_heads, p.log2_ps, p.sm_scale, p.score_log2

hipError_t launch_decode(const DecodeParams& p, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  switch (p.num_heads) {
    case 16: mla_decode_kernel<1, 1, 2><<<grid, 64, 0, stream>>>(PKVMLA_DECODE_ARGS); break;
    case 32: mla_decode_kernel<2, 1, 2><<<grid, 128, 0, stream>>>(PKVMLA_DECODE_ARGS); break;
    case 64: mla_decode_kernel<4, 1, 4><<<grid, 256, 0, stream>>>(PKVMLA_DECODE_ARGS); break;
    case 128: mla_decode_kernel<4, 2, 4><<<grid, 256, 0, stream>>>(PKVMLA_DECODE_ARGS); break;
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
  mla_gather_kernel<<<n_units, 256, 0, stream>>>(p.ckv, p.kpe, p.rows, p.units, p.seq_indptr,
                                                 p.seq_indices, p.log2_ps);
  return hipGetLastError();
}

}  // namespace pkvmla
