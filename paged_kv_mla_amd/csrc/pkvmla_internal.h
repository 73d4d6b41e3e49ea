// Internal declarations shared by the host library and the HIP kernels.
#ifndef PKVMLA_INTERNAL_H_
#define PKVMLA_INTERNAL_H_

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace pkvmla {

constexpr int kCkvDim = 512;        // head_dim_ckv = kv_lora_rank
constexpr int kKpeDim = 64;         // head_dim_kpe = qk_rope_head_dim
constexpr int kTile = 32;           // KV tokens per tile
constexpr int kUnitInts = 8;        // b, seq, kv_begin, kv_end, slot, row, page_base, first_page
                                    // (page_base: start of seq's page list in seq_indices;
                                    //  first_page: the page of token kv_begin)
constexpr int kMergeInts = 4;       // b, first_slot (or first list entry), count, kind
// Slot field of a unit that hands its softmax state to the next unit of its
// workgroup's list instead of writing it (a chained cascade request: its last
// prefix piece, then its suffix).
constexpr int32_t kChainNext = INT32_MIN;
// Slot field of a row-block unit that writes its rows' out and lse itself
// (a block of several query tokens left whole by the schedule).
constexpr int32_t kRowsDirect = INT32_MIN + 1;
constexpr int kStageBytes = kTile * kCkvDim * 2 + kTile * kKpeDim * 2;  // 36864
constexpr int kIndexPad = 64;       // margin of valid page ids after the device index table

// Kernel shape for one head count.
struct KernelConfig {
  int waves;          // waves per workgroup
  int heads_per_wave; // 16 * head blocks
  int stages;         // LDS ring depth (tiles)
  int wg_per_cu;      // resident workgroups per CU the schedule assumes
  int fixed_cost;     // schedule cost of one segment, in tiles
  int head_groups;    // workgroups sharing one token range, each with H / head_groups heads
};

bool kernel_config_for(int num_heads, KernelConfig* cfg);

struct DecodeParams {
  const uint16_t* q_nope;    // [B][H][512] bf16
  const uint16_t* q_pe;      // [B][H][64]  bf16
  const uint16_t* ckv;       // [P][ps] rows of 512 bf16, ckv_stride bytes apart
  const uint16_t* kpe;       // [P][ps] rows of 64 bf16, kpe_stride bytes apart
  int32_t ckv_stride, kpe_stride;  // row strides in bytes (1024 and 128 when contiguous)
  uint16_t* out;             // [B][H][512] bf16
  float* lse;                // [B][H]
  uint16_t* part_o;          // [slots][H][512] bf16 (normalized partial outputs)
  float* part_lse;           // [slots][H]
  const int32_t* wg_indptr;  // [grid + 1]
  const int32_t* units;      // [n_units][8]
  const int32_t* seq_indices;
  int32_t num_heads;
  int32_t head_groups;
  int32_t n_lanes;           // schedule lanes (workgroups per head group)
  int32_t waves, heads_per_wave, stages;
  int32_t log2_ps;
  int32_t row_blocks;        // units are row blocks of a cascade plan's level 0
  float sm_scale;
  float score_log2;          // sm_scale * log2(e)
  float rescale_thr;         // raw-score margin before the running max moves (8 / score_log2)
  unsigned long long* stamps;  // null, or {earliest start, latest end} of the launch's
                               // waves on the 100 MHz real-time clock (timing runs only)
  int32_t fp8;               // caches hold OCP E4M3 codes (ckv, kpe as bytes)
  float v_scale;             // fp8: ckv scale (output rows); else unused
  float kpe_ratio;           // fp8: kpe scale / ckv scale; else unused
  int32_t qo_log2h;          // row blocks of several query tokens: log2 H (query token
                             // t = row >> qo_log2h sees positions below t + the unit's
                             // second field); -1: no causal bound
  int32_t wait_limit;        // polls before a progress-counter wait gives up
};

struct MergeParams {
  const uint16_t* part_o;    // [slots][H][512] bf16
  const float* part_lse;
  const int32_t* merges;     // [n_merges][4]: b, first, count, kind (0: slots first ..
                             // first + count - 1; 1: slots slot_list[first .. first + count - 1])
  const int32_t* slot_list;
  uint16_t* out;
  float* lse;
  int32_t num_heads;
  unsigned long long* stamps;  // null, or per-block {start, end} records (timing runs)
};

struct GatherParams {
  const uint16_t* ckv;
  const uint16_t* kpe;
  uint16_t* rows;            // [n_rows][576]
  int32_t ckv_stride, kpe_stride;  // cache row strides in bytes
  const int32_t* units;
  const int32_t* seq_indices;
  int32_t log2_ps;
};

// Static split workspace of pkvmla_run_noalloc: its size, and its address on
// a device (looked up once per device, with that device current).
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
hipError_t scratch_address(int device, void** ptr);

int decode_grid(int n_lanes, int head_groups);
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);
// Role-split kernel (16, 32 or 64 heads per workgroup, one or more head
// groups); false when the configuration is not its own, else *err holds the
// launch status.
bool launch_decode_rs(const DecodeParams& p, hipStream_t stream, hipError_t* err);
// Head blocks of 16 per workgroup of the role-split kernel for a configuration
// (waves = head blocks + 4 PV waves), or 0 when it is not that kernel's.
int decode_rs_head_blocks(int waves, int heads_per_wave, int num_heads, int head_groups);
hipError_t launch_merge(const MergeParams& p, int n_merges, hipStream_t stream);
hipError_t launch_gather(const GatherParams& p, int n_units, hipStream_t stream);

}  // namespace pkvmla

#endif  // PKVMLA_INTERNAL_H_
