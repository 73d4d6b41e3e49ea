// Host side of the decode path and the two helper kernels on gfx950 (MI355X):
// the kernel-configuration table, the decode launcher (the fused role-split
// kernel lives in pkvmla_decode_rs.hip), the split-KV merge, and the
// page-table gather that checks the decode kernel's copy path bit for bit.

#include <hip/hip_runtime.h>
#include <math.h>

#include <mutex>

#include "pkvmla_tiles.h"

namespace pkvmla {

// ---------------------------------------------------------------------------
// Split-KV merge: per (request, head) combine the partial states by
// log-sum-exp: lse = M + ln sum_i e^(lse_i - M), out = sum_i e^(lse_i - lse) o_i.
// The partial outputs o_i are bf16 (each already normalized by its own row
// sum), the combination runs in fp32.  Block: 4 heads x 64 lanes, 8 dims per
// lane (one 16-byte load per partial row).  One pass: the states are read in
// chunks of four (their loads in flight together) and folded into a running
// (M, weight sum, weighted sum), so a request with at most four states costs
// one round trip to memory (and the same bits as a max-first two-pass merge;
// with more states, the rescaled sums round differently).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) mla_merge_kernel(MergeParams p) {
  constexpr int kChunk = 4;  // partial states whose loads are in flight together
  // timing runs: the block's start and end on the real-time counter
  const uint32_t sb = blockIdx.y * gridDim.x + blockIdx.x;
  if (p.stamps && threadIdx.x == 0) p.stamps[2 * sb] = __builtin_amdgcn_s_memrealtime();
  // The record and the slot list are read-only tables, read with scalar
  // loads: the slot numbers then sit in scalar registers, and no wait for a
  // vector load of the list stands between a chunk's partial-state loads
  // (which would take a round trip per state).  The record is one load.
  const idx_ptr mr = (idx_ptr)p.merges + (size_t)blockIdx.x * kMergeInts;
  int b = mr[0], s0 = mr[1], n = mr[2], kind = mr[3];
  asm volatile("" : "+s"(b), "+s"(s0), "+s"(n), "+s"(kind));
  if (n <= 0) {  // an unused record slot of a plan with fixed launches
    if (p.stamps && threadIdx.x == 0) p.stamps[2 * sb + 1] = __builtin_amdgcn_s_memrealtime();
    return;
  }
  // kind 1: the request's slots are listed (a cascade plan's prefix states
  // sit in its level-0 row blocks' slots)
  const idx_ptr list = kind == 1 ? (idx_ptr)p.slot_list + s0 : nullptr;
  const int H = p.num_heads;
  const int h = blockIdx.y * 4 + (threadIdx.x >> 6);
  const int d0 = (threadIdx.x & 63) * 8;
  constexpr float kLog2e = 1.4426950408889634f;
  float M = -INFINITY, wsum = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < n; i0 += kChunk) {
    // chunk entries past the last state re-read the last one (valid memory)
    // and carry weight 0 (a select, so they add exactly nothing)
    uint4 x[kChunk];
    float lv[kChunk];
    int slot[kChunk];
    if (list) {  // one uniform branch, so the chunk's list loads go out together
#pragma unroll
      for (int j = 0; j < kChunk; ++j) slot[j] = list[min(i0 + j, n - 1)];
    } else {
#pragma unroll
      for (int j = 0; j < kChunk; ++j) slot[j] = s0 + min(i0 + j, n - 1);
    }
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const size_t base = (size_t)slot[j] * H + h;
      lv[j] = p.part_lse[base];
      x[j] = *reinterpret_cast<const uint4*>(p.part_o + base * kCkvDim + d0);
    }
    float cm = M;
#pragma unroll
    for (int j = 0; j < kChunk; ++j) cm = fmaxf(cm, lv[j]);
    // rescale what is folded so far to the new maximum (the first chunk has
    // nothing folded: factor 0 on zeros)
    const float f = cm == M ? 1.f : __builtin_amdgcn_exp2f((M - cm) * kLog2e);
    M = cm;
    wsum *= f;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] *= f;
#pragma unroll
    for (int j = 0; j < kChunk; ++j) {
      const float w = i0 + j < n ? __builtin_amdgcn_exp2f((lv[j] - M) * kLog2e) : 0.f;
      const uint32_t xw[4] = {x[j].x, x[j].y, x[j].z, x[j].w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[2 * k] = fmaf(w, __builtin_bit_cast(float, xw[k] << 16), acc[2 * k]);
        acc[2 * k + 1] = fmaf(w, __builtin_bit_cast(float, xw[k] & 0xFFFF0000u), acc[2 * k + 1]);
      }
      wsum += w;
    }
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
  if (p.stamps && threadIdx.x == 0) p.stamps[2 * sb + 1] = __builtin_amdgcn_s_memrealtime();
}

// ---------------------------------------------------------------------------
// Gather through the decode kernel's copy path: every tile of the block's unit
// goes HBM -> LDS exactly as the decode kernel's copy waves issue it (the
// whole-tile path for full tiles of big pages, the batched per-slot path
// otherwise; four waves, one copy slot each), then each valid token's ckv and
// kpe chunks are copied back out of the swizzled tile, row-major.
// ---------------------------------------------------------------------------
template <bool BIG>
__global__ void __launch_bounds__(kCopyWaves * 64)
mla_gather_kernel(const uint16_t* __restrict__ ckv_cache, const uint16_t* __restrict__ kpe_cache,
                  uint16_t* __restrict__ rows, const int32_t* __restrict__ units_g,
                  const int32_t* __restrict__ seq_indices_g, int log2_ps, int cs, int ks) {
  __shared__ __attribute__((aligned(1024))) char smem_raw[kStageBytes];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const uint32_t smem_base = (uint32_t)(uintptr_t)smem;
  const idx_ptr units = (idx_ptr)units_g;
  const idx_ptr seq_indices = (idx_ptr)seq_indices_g;
  const char* ckv = reinterpret_cast<const char*>(ckv_cache);
  const char* kpe = reinterpret_cast<const char*>(kpe_cache);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // copy slot
  const CopyLanes CL = copy_lanes(wave, ks);
  idx_ptr rec = units + (size_t)blockIdx.x * kUnitInts;
  const int kv0 = rec[2], kv1 = rec[3], row0 = rec[5];
  TileStream ts;
  ts.u = blockIdx.x;
  ts.u_end = blockIdx.x + 1;
  ts.g = 0;
  stream_load_unit(ts, units, seq_indices);
  for (int tok0 = kv0; tok0 < kv1; tok0 += kTile) {
    __syncthreads();  // the previous tile has been read out
    const TileCopy c = tile_copy(ts, ckv, kpe, log2_ps, smem_base, wave, cs, ks);
    if (BIG && c.full) {
#pragma unroll
      for (int k = 0; k < kCopiesPerWave; ++k) tile_copy_part_full(c, wave, k, CL);
    } else {
      tile_copy_slot<BIG, true>(c, ckv, kpe, wave, CL);  // the gather reads packed caches
    }
    stream_advance(ts, units, seq_indices, log2_ps);
    wait_vmcnt<0>();
    __syncthreads();
    const int n = min(kTile, kv1 - tok0);
    for (int idx = threadIdx.x; idx < n * 72; idx += kCopyWaves * 64) {
      const int t = idx / 72, ch = idx % 72;
      const int src = ch < 64 ? lds_ckv_off(t, ch) : lds_kpe_off(t, ch - 64);
      const u32x4_t v = *(const LDS_AS u32x4_t*)(smem + src);
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(rows + ((size_t)row0 + (tok0 - kv0) + t) * 576) + ch;
      *dst = v;
    }
  }
  // no copy may still be writing LDS when the workgroup retires
  wait_vmcnt<0>();
}

// ---------------------------------------------------------------------------
// Host side: configuration table and launchers.
// ---------------------------------------------------------------------------
// Per head count: compute waves (one QK wave per 16 heads and four PV waves;
// two copy waves come on top), heads per QK wave, LDS stages, workgroups per
// CU, fixed schedule cost of a unit in tiles, head groups (workgroups that
// share a token range, each holding 64 of 128 heads).
bool kernel_config_for(int num_heads, KernelConfig* cfg) {
  switch (num_heads) {
    case 16: *cfg = KernelConfig{5, 16, 4, 1, 2, 1}; break;
    case 32: *cfg = KernelConfig{6, 16, 4, 1, 2, 1}; break;
    case 64: *cfg = KernelConfig{8, 16, 4, 1, 4, 1}; break;
    case 128: *cfg = KernelConfig{8, 16, 4, 1, 4, 2}; break;
    default: return false;
  }
  return true;
}

// ---------------------------------------------------------------------------
// Static scratch for callers that cannot allocate.  pkvmla_run_noalloc keeps
// the split workspace (partial outputs and their lse) here instead of in the
// plan's own buffer.  Each device that loads the library holds one copy until
// the process ends; runs on one device share it (calls that overlap on one
// device race).  The host never passes `scratch` itself to a kernel: in host
// code that name is a stand-in, not a device address.  Its address on each
// device comes from hipGetSymbolAddress, once per device, with that device
// current.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_address(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device) return hipErrorInvalidDevice;  // the caller makes it current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

int decode_grid(int n_lanes, int head_groups) {
  return ((n_lanes + 7) / 8) * 8 * head_groups;
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.n_lanes <= 0) return hipSuccess;
  hipError_t err = hipSuccess;
  if (launch_decode_rs(p, stream, &err)) return err;
  return hipErrorInvalidValue;  // no kernel for this configuration
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
    mla_gather_kernel<true><<<n_units, kCopyWaves * 64, 0, stream>>>(
        p.ckv, p.kpe, p.rows, p.units, p.seq_indices, p.log2_ps, p.ckv_stride,
        p.kpe_stride);
  else
    mla_gather_kernel<false><<<n_units, kCopyWaves * 64, 0, stream>>>(
        p.ckv, p.kpe, p.rows, p.units, p.seq_indices, p.log2_ps, p.ckv_stride,
        p.kpe_stride);
  return hipGetLastError();
}

}  // namespace pkvmla
