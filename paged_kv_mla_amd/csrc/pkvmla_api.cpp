// C ABI of the MLA paged-decode library: argument validation, plan lifetime,
// schedule upload and kernel dispatch.  See include/pkvmla.h for the contract.
#include "pkvmla.h"

#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <string>
#include <vector>

#include "pkvmla_internal.h"
#include "pkvmla_schedule.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return PKVMLA_OK;
}

#define PKVMLA_HIP(call)                                                              \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess)                                                             \
      return fail(e_ == hipErrorOutOfMemory ? PKVMLA_ENOMEM : PKVMLA_EHIP, "%s: %s", #call, \
                  hipGetErrorString(e_));                                             \
  } while (0)

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

struct pkvmla_plan_s {
  int device = 0;
  int32_t batch = 0, num_heads = 0, page_size = 0, log2_ps = 0;
  int32_t ckv_dim = 0, kpe_dim = 0, num_pages = 0;
  float sm_scale = 0.f;
  int32_t is_cascade = 0, num_groups = 0, num_cu = 0;
  int32_t num_requests = 0;  // requests of a plan with several query tokens per request
  int32_t is_qo = 0;
  pkvmla::KernelConfig cfg{};
  pkvmla::Schedule sched;
  int32_t num_seqs = 0;
  int64_t n_indices = 0;
  // Capacities fixed at creation: the device tables, the split workspace and
  // every launch configuration are sized by them, so a later page-table update
  // changes no pointer and no grid (a captured HIP graph stays valid).
  int32_t cap_lanes = 0;     // schedule lanes (workgroups per head group)
  int32_t cap_units = 0;     // unit records: work items + lanes bound the splits
  int32_t cap_merges = 0;    // merge records: one per request at most
  int64_t cap_indices = 0;   // page ids
  int64_t index_capacity_request = 0;  // caller's page-id capacity (0: the first table's)
  // Launch shapes: exact (lanes in use; the merge kernel only when a request
  // is split) or, for a plan built with a capacity, fixed at the capacities so
  // that the kernels a captured graph replays stay right after updates.
  int fixed_launch = 0;
  int32_t cap_slots = 0;     // partial-state slots of the split workspace
  // cascade plans: level 0, row blocks of each group's query rows over its
  // shared prefix (a launch of its own before the suffixes), and the merge's
  // slot lists
  pkvmla::KernelConfig cfg0{};
  pkvmla::RowSchedule sched0;
  std::vector<int32_t> slot_list;
  int32_t cap_lanes0 = 0, cap_units0 = 0, cap_list = 0;
  // cascade in one launch: each request's suffix chained after its prefix
  // piece (64 heads or more, every prefix non-empty, ordinary plans)
  int32_t cascade_chain = 0;
  size_t off_wg = 0, off_units = 0, off_merges = 0, off_sip = 0, off_sl = 0, off_si = 0;
  size_t off_wg0 = 0, off_units0 = 0, off_list = 0;
  // device tables (one allocation) and split workspace
  int32_t* d_tables = nullptr;
  int32_t* d_wg_indptr = nullptr;
  int32_t* d_units = nullptr;
  int32_t* d_merges = nullptr;
  int32_t* d_seq_indptr = nullptr;
  int32_t* d_seq_lens = nullptr;
  int32_t* d_seq_indices = nullptr;
  int32_t* d_wg0 = nullptr;
  int32_t* d_units0 = nullptr;
  int32_t* d_slot_list = nullptr;
  void* d_part = nullptr;  // part_o bf16 [slots][H][512] then part_lse fp32 [slots][H]
  size_t table_ints = 0;
  // optional per-run timing: every workgroup's start and end stamps, per run
  // slot [kTimingSlots][timing_wgs0 + timing_wgs + timing_wgsm][2] (the
  // level-0 decode launch's workgroups, the decode launch's, then the merge
  // launch's blocks), the grids each run launched, and in mode 2 a HIP event
  // pair around the decode launches (events created up front)
  static constexpr int kTimingSlots = 256;
  hipEvent_t ev[2 * kTimingSlots] = {};
  unsigned long long* d_stamps = nullptr;
  int32_t timing_wgs0 = 0, timing_wgs = 0, timing_wgsm = 0;
  int32_t timing_grid[kTimingSlots][3] = {};
  int timing = 0;
  int64_t timed_runs = 0;
  int32_t wait_limit = 1 << 20;  // polls before a progress-counter wait gives up
};

namespace {

// Common checks of the scalar plan parameters.
int check_shape(int32_t batch, int32_t num_pages, int32_t num_heads, int32_t ckv_dim,
                int32_t kpe_dim, int32_t page_size, float sm_scale, int32_t* log2_ps,
                float* scale) {
  if (batch < 1) return fail(PKVMLA_EINVAL, "batch must be >= 1 (got %d)", batch);
  if (num_pages < 1) return fail(PKVMLA_EINVAL, "num_pages must be >= 1 (got %d)", num_pages);
  if (ckv_dim != pkvmla::kCkvDim || kpe_dim != pkvmla::kKpeDim)
    return fail(PKVMLA_EUNSUPPORTED,
                "head_dim_ckv must be kv_lora_rank = 512 and head_dim_kpe qk_rope_head_dim = 64 "
                "(got %d, %d)",
                ckv_dim, kpe_dim);
  pkvmla::KernelConfig cfg;
  if (!pkvmla::kernel_config_for(num_heads, &cfg))
    return fail(PKVMLA_EUNSUPPORTED, "num_heads must be one of 16, 32, 64, 128 (got %d)",
                num_heads);
  if (page_size < 1) return fail(PKVMLA_EINVAL, "page_size must be >= 1 (got %d)", page_size);
  if (page_size > 256 || (page_size & (page_size - 1)) != 0)
    return fail(PKVMLA_EUNSUPPORTED, "page_size must be a power of two <= 256 (got %d)",
                page_size);
  if ((int64_t)num_pages * page_size > (int64_t)INT32_MAX)
    return fail(PKVMLA_EUNSUPPORTED, "num_pages * page_size must fit in int32");
  if (!std::isfinite(sm_scale) || sm_scale < 0.f)
    return fail(PKVMLA_EINVAL, "sm_scale must be finite and >= 0 (0 = default)");
  int l = 0;
  while ((1 << l) < page_size) ++l;
  *log2_ps = l;
  *scale = sm_scale == 0.f ? (float)(1.0 / std::sqrt((double)(ckv_dim + kpe_dim))) : sm_scale;
  return PKVMLA_OK;
}

// Validate one CSR page list: indptr[n+1], indices, lens[n].
int check_pages(const char* what, const int32_t* indptr, const int32_t* indices,
                const int32_t* lens, int32_t n, int32_t num_pages, int32_t page_size,
                int32_t min_len) {
  if (!indptr || !lens) return fail(PKVMLA_EINVAL, "%s: null indptr or lens", what);
  if (indptr[0] != 0) return fail(PKVMLA_EINVAL, "%s: indptr[0] must be 0", what);
  for (int32_t b = 0; b < n; ++b) {
    if (indptr[b + 1] < indptr[b])
      return fail(PKVMLA_EINVAL, "%s: indptr must be non-decreasing (at %d)", what, b);
    if (lens[b] < min_len)
      return fail(PKVMLA_EINVAL, "%s: length[%d] = %d is below %d", what, b, lens[b], min_len);
    const int64_t cap = (int64_t)(indptr[b + 1] - indptr[b]) * page_size;
    if (lens[b] > cap)
      return fail(PKVMLA_EINVAL, "%s: length[%d] = %d exceeds its %d pages x page_size %d", what,
                  b, lens[b], indptr[b + 1] - indptr[b], page_size);
  }
  if (indptr[n] > 0 && !indices) return fail(PKVMLA_EINVAL, "%s: null indices", what);
  for (int64_t i = 0; i < indptr[n]; ++i)
    if (indices[i] < 0 || indices[i] >= num_pages)
      return fail(PKVMLA_EINVAL, "%s: page index %d at %lld outside [0, %d)", what, indices[i],
                  (long long)i, num_pages);
  return PKVMLA_OK;
}

// The page fields of unit records: the sequence's page-list start and the page
// of the unit's first token.
// The sequence is the record's second field, or seq_of[unit] when given (row
// blocks of several query tokens keep their causal offset there).
void fill_page_fields(std::vector<int32_t>* units, const std::vector<int32_t>& seq_indptr,
                      const std::vector<int32_t>& seq_indices, int32_t page_size,
                      const std::vector<int32_t>* seq_of = nullptr) {
  for (size_t i = 0; i < units->size(); i += pkvmla::kUnitRecordInts) {
    int32_t* u = &(*units)[i];
    const int32_t base = seq_indptr[seq_of ? (*seq_of)[i / pkvmla::kUnitRecordInts] : u[1]];
    u[6] = base;
    u[7] = seq_indices[(size_t)base + (size_t)(u[2] / page_size)];
  }
}

// Build the schedule for `items` into *sched, with the page fields of its unit
// records (the sequence's page-list start and the page of the unit's first
// token, so a workgroup's first copies need one dependent load, the record,
// instead of three).
int build_plan_schedule(const pkvmla_plan_s* P, const std::vector<pkvmla::WorkItem>& items,
                        const std::vector<int32_t>& seq_indptr,
                        const std::vector<int32_t>& seq_indices, pkvmla::Schedule* sched) {
  if (!pkvmla::build_schedule(items, P->batch, P->cap_lanes, pkvmla::kTile, P->cfg.fixed_cost,
                              sched))
    return fail(PKVMLA_EINVAL, "schedule construction failed");
  if (sched->total_rows > INT32_MAX) return fail(PKVMLA_EUNSUPPORTED, "too many tokens");
  fill_page_fields(&sched->units, seq_indptr, seq_indices, P->page_size);
  return PKVMLA_OK;
}

// Write the schedule and the sequences' page tables into the capacity-sized
// device tables (one copy on `stream`, then a wait for it: the host staging
// buffer is local).  Entries past the live ones: wg_indptr repeats its last
// value (empty lanes), merge records have count 0 (skipped).
int upload_tables(pkvmla_plan_s* P, const pkvmla::Schedule& sched,
                  const std::vector<int32_t>& seq_indptr, const std::vector<int32_t>& seq_lens,
                  const std::vector<int32_t>& seq_indices, hipStream_t stream,
                  const pkvmla::RowSchedule* sched0 = nullptr,
                  const std::vector<int32_t>* slot_list = nullptr) {
  // every table must fit its region of the allocation: a schedule beyond the
  // plan's capacities is an error, never an overflow into the next table
  const std::vector<int32_t>& wg = sched.wg_indptr;
  if ((int64_t)wg.size() > (int64_t)P->cap_lanes + 1 ||
      (int64_t)sched.units.size() > (int64_t)P->cap_units * pkvmla::kUnitRecordInts ||
      (int64_t)sched.merges.size() > (int64_t)P->cap_merges * pkvmla::kMergeRecordInts ||
      sched.n_slots > P->cap_slots ||
      (int64_t)seq_indptr.size() > (int64_t)(P->off_sl - P->off_sip) ||
      (int64_t)seq_lens.size() > (int64_t)(P->off_si - P->off_sl) ||
      (int64_t)seq_indices.size() > (int64_t)(P->table_ints - P->off_si) ||
      (sched0 && ((int64_t)sched0->wg_indptr.size() > (int64_t)P->cap_lanes0 + 1 ||
                  (int64_t)sched0->units.size() > (int64_t)P->cap_units0 * pkvmla::kUnitRecordInts ||
                  sched0->n_slots > P->cap_slots ||
                  (int64_t)slot_list->size() > (int64_t)P->cap_list)))
    return fail(PKVMLA_EUNSUPPORTED, "schedule exceeds the plan's tables");
  std::vector<int32_t> host(P->table_ints, 0);
  for (int32_t l = 0; l <= P->cap_lanes; ++l)
    host[P->off_wg + l] = l < (int32_t)wg.size() ? wg[l] : wg.back();
  std::copy(sched.units.begin(), sched.units.end(), host.begin() + P->off_units);
  std::copy(sched.merges.begin(), sched.merges.end(), host.begin() + P->off_merges);
  std::copy(seq_indptr.begin(), seq_indptr.end(), host.begin() + P->off_sip);
  std::copy(seq_lens.begin(), seq_lens.end(), host.begin() + P->off_sl);
  std::copy(seq_indices.begin(), seq_indices.end(), host.begin() + P->off_si);
  if (sched0) {
    const std::vector<int32_t>& wg0 = sched0->wg_indptr;
    for (int32_t l = 0; l <= P->cap_lanes0; ++l)
      host[P->off_wg0 + l] = l < (int32_t)wg0.size() ? wg0[l] : wg0.back();
    std::copy(sched0->units.begin(), sched0->units.end(), host.begin() + P->off_units0);
    std::copy(slot_list->begin(), slot_list->end(), host.begin() + P->off_list);
  }
  PKVMLA_HIP(hipMemcpyAsync(P->d_tables, host.data(), P->table_ints * sizeof(int32_t),
                            hipMemcpyHostToDevice, stream));
  PKVMLA_HIP(hipStreamSynchronize(stream));
  P->num_seqs = (int32_t)seq_lens.size();
  P->n_indices = (int64_t)seq_indices.size();
  return PKVMLA_OK;
}

// Level 0 of a cascade plan (its groups and prefix lengths).
struct Level0Groups {
  const int32_t* group_req_indptr;
  int32_t num_groups;
  const int32_t* prefix_lens;
};

// A cascade plan's schedules: level 1 over the suffix items (every unit
// writing a partial state numbered after level 0's), level 0 over the row
// blocks, the merge records and slot list.
int build_cascade_schedules(const pkvmla_plan_s* P, const Level0Groups& l0,
                            const std::vector<pkvmla::WorkItem>& items,
                            const std::vector<int32_t>& seq_indptr,
                            const std::vector<int32_t>& seq_indices, pkvmla::Schedule* sched,
                            pkvmla::RowSchedule* sched0, std::vector<int32_t>* slot_list) {
  int rc = build_plan_schedule(P, items, seq_indptr, seq_indices, sched);
  if (rc) return rc;
  if (!pkvmla::build_row_schedule(l0.group_req_indptr, l0.num_groups, l0.prefix_lens,
                                  P->num_heads, P->cap_lanes0, pkvmla::kTile, sched0))
    return fail(PKVMLA_EUNSUPPORTED, "level-0 schedule construction failed (too many rows)");
  fill_page_fields(&sched0->units, seq_indptr, seq_indices, P->page_size);
  int64_t slot = sched0->n_slots;
  for (size_t i = 0; i < sched->units.size(); i += pkvmla::kUnitRecordInts)
    sched->units[i + 4] = (int32_t)slot++;
  if (slot > INT32_MAX / 2) return fail(PKVMLA_EUNSUPPORTED, "too many partial states");
  sched->n_slots = (int32_t)slot;
  pkvmla::build_cascade_merges(*sched0, sched->units, P->batch, P->num_heads, &sched->merges,
                               slot_list);
  return PKVMLA_OK;
}

// The host tables of a cascade plan, as the caller passes them.
struct CascadeTables {
  const int32_t* group_req_indptr;
  int32_t num_groups;
  const int32_t* prefix_indptr;
  const int32_t* prefix_indices;
  const int32_t* prefix_lens;
  const int32_t* kv_indptr;
  const int32_t* kv_indices;
  const int32_t* kv_lens;
  int32_t batch;
};

int check_cascade(const CascadeTables& t, int32_t num_pages, int32_t page_size) {
  if (t.num_groups < 1 || !t.group_req_indptr)
    return fail(PKVMLA_EINVAL, "num_groups must be >= 1 with a group_req_indptr");
  if (t.group_req_indptr[0] != 0 || t.group_req_indptr[t.num_groups] != t.batch)
    return fail(PKVMLA_EINVAL, "group_req_indptr must run from 0 to batch");
  for (int32_t g = 0; g < t.num_groups; ++g)
    if (t.group_req_indptr[g + 1] < t.group_req_indptr[g])
      return fail(PKVMLA_EINVAL, "group_req_indptr must be non-decreasing (at %d)", g);
  int rc = check_pages("prefix", t.prefix_indptr, t.prefix_indices, t.prefix_lens, t.num_groups,
                       num_pages, page_size, 0);
  if (rc) return rc;
  rc = check_pages("suffix", t.kv_indptr, t.kv_indices, t.kv_lens, t.batch, num_pages, page_size,
                   0);
  if (rc) return rc;
  for (int32_t g = 0; g < t.num_groups; ++g)
    for (int32_t b = t.group_req_indptr[g]; b < t.group_req_indptr[g + 1]; ++b)
      if (t.prefix_lens[g] + t.kv_lens[b] < 1)
        return fail(PKVMLA_EINVAL, "request %d attends no token (prefix and suffix empty)", b);
  return PKVMLA_OK;
}

// Sequences (G prefix lists, then one suffix list per request) and the
// level-1 items (each request over its suffix; empty ones get no unit).
void cascade_sequences(const CascadeTables& t, std::vector<int32_t>* sip, std::vector<int32_t>* sl,
                       std::vector<int32_t>* si, std::vector<pkvmla::WorkItem>* items) {
  const int32_t G = t.num_groups, B = t.batch;
  sip->clear();
  sl->clear();
  for (int32_t g = 0; g <= G; ++g) sip->push_back(t.prefix_indptr[g]);
  for (int32_t b = 1; b <= B; ++b) sip->push_back(t.prefix_indptr[G] + t.kv_indptr[b]);
  for (int32_t g = 0; g < G; ++g) sl->push_back(t.prefix_lens[g]);
  for (int32_t b = 0; b < B; ++b) sl->push_back(t.kv_lens[b]);
  si->assign(t.prefix_indices, t.prefix_indices + t.prefix_indptr[G]);
  si->insert(si->end(), t.kv_indices, t.kv_indices + t.kv_indptr[B]);
  items->clear();
  for (int32_t b = 0; b < B; ++b) items->push_back(pkvmla::WorkItem{b, G + b, t.kv_lens[b]});
}

static_assert(pkvmla::kChainNext == pkvmla::kChainNextSlot, "chained-unit slot marker");

// The one-launch (chained) cascade schedule, in the plan's tables: its units
// in the level-0 table, no level-1 units.
int build_chain_tables(const pkvmla_plan_s* P, const Level0Groups& l0, const int32_t* kv_lens,
                       const std::vector<int32_t>& seq_indptr,
                       const std::vector<int32_t>& seq_indices, pkvmla::Schedule* sched,
                       pkvmla::RowSchedule* sched0, std::vector<int32_t>* slot_list) {
  if (!pkvmla::build_chain_schedule(l0.group_req_indptr, l0.num_groups, l0.prefix_lens, kv_lens,
                                    P->batch, P->cap_lanes0, pkvmla::kTile, sched0,
                                    &sched->merges, slot_list))
    return fail(PKVMLA_EUNSUPPORTED, "chained cascade schedule construction failed");
  fill_page_fields(&sched0->units, seq_indptr, seq_indices, P->page_size);
  sched->grid = 0;
  sched->wg_indptr.assign(1, 0);
  sched->units.clear();
  sched->n_slots = sched0->n_slots;
  sched->total_rows = 0;
  return PKVMLA_OK;
}

// A plan with several new tokens per request, laid out in row blocks.
struct QoRows {
  const int32_t* qo_indptr;
  const int32_t* kv_lens;
  int32_t num_requests;
};

static_assert(pkvmla::kRowsDirect == pkvmla::kRowsDirectSlot, "direct row-block slot marker");

// Query-token index of a plan with several new tokens per request: every
// request brings 1 .. kv_len of them.
int check_qo(const int32_t* qo_indptr, const int32_t* kv_lens, int32_t batch) {
  if (!qo_indptr) return fail(PKVMLA_EINVAL, "null qo_indptr");
  if (qo_indptr[0] != 0) return fail(PKVMLA_EINVAL, "qo_indptr[0] must be 0");
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
    if (n < 1) return fail(PKVMLA_EINVAL, "request %d has %lld query tokens (>= 1 needed)", b, (long long)n);
    if (n > kv_lens[b])
      return fail(PKVMLA_EINVAL, "request %d: %lld query tokens but kv_len %d (the new tokens are part "
                  "of the KV)", b, (long long)n, kv_lens[b]);
  }
  return PKVMLA_OK;
}

// One work item per query token: row qo_indptr[b] + j over sequence b, of its
// causal length (position + 1).
std::vector<pkvmla::WorkItem> qo_token_items(const int32_t* qo_indptr, const int32_t* kv_lens,
                                             int32_t batch) {
  std::vector<pkvmla::WorkItem> items((size_t)qo_indptr[batch]);
  for (int32_t b = 0; b < batch; ++b) {
    const int32_t n = qo_indptr[b + 1] - qo_indptr[b];
    for (int32_t j = 0; j < n; ++j)
      items[qo_indptr[b] + j] = pkvmla::WorkItem{qo_indptr[b] + j, b, kv_lens[b] - n + 1 + j};
  }
  return items;
}

// The tables of a row-block plan: its units in the level-0 table, merges per
// query token over a slot list, no level-1 units.
int build_qo_row_tables(const pkvmla_plan_s* P, const int32_t* qo_indptr, const int32_t* kv_lens,
                        int32_t batch, const std::vector<int32_t>& seq_indptr,
                        const std::vector<int32_t>& seq_indices, pkvmla::Schedule* sched,
                        pkvmla::RowSchedule* sched0, std::vector<int32_t>* slot_list) {
  std::vector<int32_t> unit_seq;
  if (!pkvmla::build_qo_row_schedule(qo_indptr, kv_lens, batch, P->num_heads, P->cap_lanes0,
                                     pkvmla::kTile, P->cfg0.fixed_cost, sched0, &unit_seq,
                                     &sched->merges, slot_list))
    return fail(PKVMLA_EUNSUPPORTED, "row-block schedule construction failed (too many query rows)");
  fill_page_fields(&sched0->units, seq_indptr, seq_indices, P->page_size, &unit_seq);
  sched->grid = 0;
  sched->wg_indptr.assign(1, 0);
  sched->units.clear();
  sched->n_slots = sched0->n_slots;
  sched->total_rows = 0;
  return PKVMLA_OK;
}

bool chain_eligible(const pkvmla_plan_s* P, const Level0Groups& l0) {
  if (P->fixed_launch || P->num_heads < 64) return false;
  for (int32_t g = 0; g < l0.num_groups; ++g)
    if (l0.prefix_lens[g] <= 0) return false;
  return true;
}

// Fix the capacities, build the schedule, allocate and upload the device tables.
// With `l0` (cascade plans) the items are the suffixes; the level-0 row-block
// schedule is built beside them, every suffix unit writes a partial state
// after the level-0 slots, and each request's merge lists all of its states.
int finish_plan(pkvmla_plan_s* P, const std::vector<pkvmla::WorkItem>& items,
                const std::vector<int32_t>& seq_indptr, const std::vector<int32_t>& seq_lens,
                const std::vector<int32_t>& seq_indices, hipStream_t stream,
                const Level0Groups* l0 = nullptr, const QoRows* qo = nullptr) {
  PKVMLA_HIP(hipGetDevice(&P->device));
  PKVMLA_HIP(hipDeviceGetAttribute(&P->num_cu, hipDeviceAttributeMultiprocessorCount, P->device));
  // the schedule's lanes: each lane's token ranges are replicated over the head groups
  P->cap_lanes = std::max(1, P->num_cu * P->cfg.wg_per_cu / P->cfg.head_groups);
  // a lane boundary splits at most one work item, so units <= items + lanes - 1
  P->cap_units = (int32_t)items.size() + P->cap_lanes;
  P->cap_merges = P->batch;
  P->cap_indices = std::max<int64_t>((int64_t)seq_indices.size(), P->index_capacity_request);
  int rc;
  P->cap_slots = P->cap_units;
  if (l0) {
    // level-0 capacities, for any groups and prefixes of this batch and head
    // count: nb <= lanes gives one unit per lane (at most 64 / H requests,
    // at least one, per unit), nb > lanes one unit per block (blocks <=
    // rows / 64 + groups, one slot per request)
    const int64_t H = P->num_heads, B = P->batch;
    P->cap_lanes0 = std::max(1, P->num_cu / P->cfg0.head_groups);
    const int64_t blocks = (B * H + 63) / 64 + l0->num_groups;
    const int64_t u0 = std::max<int64_t>(P->cap_lanes0, blocks);
    const int64_t s0 = std::max<int64_t>((int64_t)P->cap_lanes0 * std::max<int64_t>(1, 64 / H), B);
    const int64_t slots = s0 + B + P->cap_lanes;
    if (u0 > INT32_MAX / pkvmla::kUnitRecordInts || slots > INT32_MAX / 2)
      return fail(PKVMLA_EUNSUPPORTED, "too many query rows for a cascade plan");
    P->cap_units0 = (int32_t)u0;
    P->cap_slots = (int32_t)slots;
    P->cap_list = (int32_t)slots;
    P->cascade_chain = chain_eligible(P, *l0) ? 1 : 0;
    if (P->cascade_chain) {
      // pieces: at most one per lane (batch <= lanes) or one per request;
      // plus a suffix unit per request; a slot per piece or chain at most
      const int64_t pieces = std::max<int64_t>(P->cap_lanes0, B);
      P->cap_units0 = (int32_t)std::max<int64_t>(u0, pieces + B);
      P->cap_slots = (int32_t)std::max<int64_t>(slots, pieces + B);
      P->cap_list = P->cap_slots;
      std::vector<int32_t> kvl(seq_lens.begin() + l0->num_groups, seq_lens.end());
      rc = build_chain_tables(P, *l0, kvl.data(), seq_indptr, seq_indices, &P->sched,
                              &P->sched0, &P->slot_list);
    } else {
      rc = build_cascade_schedules(P, *l0, items, seq_indptr, seq_indices, &P->sched,
                                   &P->sched0, &P->slot_list);
    }
  } else if (qo) {
    // every unit in the level-0 table (row blocks of the 64-row kernel), no
    // level-1 units; merges per query token over slot lists
    P->cap_lanes0 = std::max(1, P->num_cu / P->cfg0.head_groups);
    rc = build_qo_row_tables(P, qo->qo_indptr, qo->kv_lens, qo->num_requests, seq_indptr,
                             seq_indices, &P->sched, &P->sched0, &P->slot_list);
    if (rc) return rc;
    if (P->fixed_launch) {
      // any query-token split of the same T tokens over the same B requests:
      // blocks <= T * H / 64 + B, a unit per block plus one per lane cut, a
      // walk slot per unit holding 64 / H partial slots, as many list entries
      const int64_t per = pkvmla::kQoBlockRows / P->num_heads;
      const int64_t blocks = ((int64_t)P->batch * P->num_heads + pkvmla::kQoBlockRows - 1) /
                                 pkvmla::kQoBlockRows + qo->num_requests;
      const int64_t units = blocks + P->cap_lanes0;
      if (units * per > INT32_MAX / 2 || units > INT32_MAX / pkvmla::kUnitRecordInts)
        return fail(PKVMLA_EUNSUPPORTED, "too many query rows for a plan with a capacity");
      P->cap_units0 = (int32_t)units;
      P->cap_slots = (int32_t)(units * per);
      P->cap_list = (int32_t)(units * per);
    } else {
      P->cap_units0 = (int32_t)(P->sched0.units.size() / pkvmla::kUnitRecordInts);
      P->cap_slots = std::max(1, P->sched0.n_slots);
      P->cap_list = (int32_t)P->slot_list.size();
    }
  } else {
    rc = build_plan_schedule(P, items, seq_indptr, seq_indices, &P->sched);
  }
  if (rc) return rc;

  // 64-int aligned sub-buffers inside one allocation
  auto pad = [](size_t n) { return (n + 63) & ~size_t(63); };
  P->off_wg = 0;
  P->off_units = P->off_wg + pad((size_t)P->cap_lanes + 1);
  P->off_merges = P->off_units + pad((size_t)P->cap_units * pkvmla::kUnitRecordInts);
  P->off_wg0 = P->off_merges + pad((size_t)P->cap_merges * pkvmla::kMergeRecordInts);
  const bool has_l0 = l0 || qo;
  P->off_units0 = P->off_wg0 + pad(has_l0 ? (size_t)P->cap_lanes0 + 1 : 0);
  P->off_list = P->off_units0 + pad((size_t)P->cap_units0 * pkvmla::kUnitRecordInts);
  P->off_sip = P->off_list + pad((size_t)P->cap_list);
  P->off_sl = P->off_sip + pad(seq_indptr.size());
  P->off_si = P->off_sl + pad(seq_lens.size());
  // every page-id read of the kernels lies inside its sequence's list (tile
  // starts below kv_end, tokens clamped to the last valid one); the kIndexPad
  // trailing entries (page 0, a valid id) are a margin beyond that
  P->table_ints = P->off_si + pad((size_t)P->cap_indices + pkvmla::kIndexPad);
  PKVMLA_HIP(hipMalloc(&P->d_tables, P->table_ints * sizeof(int32_t)));
  P->d_wg_indptr = P->d_tables + P->off_wg;
  P->d_units = P->d_tables + P->off_units;
  P->d_merges = P->d_tables + P->off_merges;
  P->d_seq_indptr = P->d_tables + P->off_sip;
  P->d_seq_lens = P->d_tables + P->off_sl;
  P->d_seq_indices = P->d_tables + P->off_si;
  P->d_wg0 = P->d_tables + P->off_wg0;
  P->d_units0 = P->d_tables + P->off_units0;
  P->d_slot_list = P->d_tables + P->off_list;
  // split workspace for the largest slot count any schedule can need
  // (flat plans: slots <= units)
  const size_t rows = (size_t)P->cap_slots * P->num_heads;
  PKVMLA_HIP(hipMalloc(&P->d_part, rows * (pkvmla::kCkvDim * sizeof(uint16_t) + sizeof(float))));
  return upload_tables(P, P->sched, seq_indptr, seq_lens, seq_indices, stream,
                       has_l0 ? &P->sched0 : nullptr, has_l0 ? &P->slot_list : nullptr);
}

void free_plan(pkvmla_plan_s* P) {
  if (!P) return;
  for (hipEvent_t& e : P->ev)
    if (e) (void)hipEventDestroy(e);
  if (P->d_tables) (void)hipFree(P->d_tables);
  if (P->d_part) (void)hipFree(P->d_part);
  if (P->d_stamps) (void)hipFree(P->d_stamps);
  delete P;
}

}  // namespace

extern "C" {

const char* pkvmla_last_error(void) { return g_last_error.c_str(); }

int pkvmla_kernel_config(int32_t num_heads, int32_t* cfg7) {
  if (!cfg7) return fail(PKVMLA_EINVAL, "null output");
  pkvmla::KernelConfig c;
  if (!pkvmla::kernel_config_for(num_heads, &c))
    return fail(PKVMLA_EUNSUPPORTED, "num_heads must be one of 16, 32, 64, 128 (got %d)",
                num_heads);
  cfg7[0] = pkvmla::kTile;
  cfg7[1] = c.waves;
  cfg7[2] = c.heads_per_wave;
  cfg7[3] = c.stages;
  cfg7[4] = c.wg_per_cu;
  cfg7[5] = c.fixed_cost;
  cfg7[6] = c.head_groups;
  return ok();
}

int pkvmla_schedule_host(const int32_t* items, int32_t n_items, int32_t batch, int32_t num_wg,
                         int32_t tile, int32_t fixed_cost, int32_t* wg_indptr, int64_t cap_wg,
                         int32_t* units, int64_t cap_units, int32_t* merges, int64_t cap_merges,
                         int32_t* counts) {
  if ((!items && n_items > 0) || !counts || n_items < 0)
    return fail(PKVMLA_EINVAL, "null or negative argument");
  if (num_wg < 1 || tile < 1 || fixed_cost < 0 || batch < 1)
    return fail(PKVMLA_EINVAL, "num_wg, tile, batch must be >= 1 and fixed_cost >= 0");
  std::vector<pkvmla::WorkItem> v((size_t)n_items);
  for (int32_t i = 0; i < n_items; ++i) {
    v[i] = pkvmla::WorkItem{items[3 * i], items[3 * i + 1], items[3 * i + 2]};
    if (v[i].req < 0 || v[i].req >= batch || v[i].len < 0)
      return fail(PKVMLA_EINVAL, "item %d: request out of range or negative length", i);
  }
  pkvmla::Schedule s;
  if (!pkvmla::build_schedule(v, batch, num_wg, tile, fixed_cost, &s))
    return fail(PKVMLA_EINVAL, "schedule construction failed");
  counts[0] = s.grid;
  counts[1] = (int32_t)(s.units.size() / pkvmla::kUnitRecordInts);
  counts[2] = (int32_t)(s.merges.size() / pkvmla::kMergeRecordInts);
  if ((int64_t)s.wg_indptr.size() > cap_wg || (int64_t)s.units.size() > cap_units ||
      (int64_t)s.merges.size() > cap_merges)
    return fail(PKVMLA_EINVAL, "output capacity too small (need %zu, %zu, %zu)",
                s.wg_indptr.size(), s.units.size(), s.merges.size());
  if (!s.wg_indptr.empty() && !wg_indptr) return fail(PKVMLA_EINVAL, "null wg_indptr");
  if (!s.units.empty() && !units) return fail(PKVMLA_EINVAL, "null units");
  if (!s.merges.empty() && !merges) return fail(PKVMLA_EINVAL, "null merges");
  std::copy(s.wg_indptr.begin(), s.wg_indptr.end(), wg_indptr);
  std::copy(s.units.begin(), s.units.end(), units);
  std::copy(s.merges.begin(), s.merges.end(), merges);
  return ok();
}

int pkvmla_schedule_rows_host(const int32_t* group_req_indptr, int32_t num_groups,
                               const int32_t* prefix_lens, int32_t num_heads, int32_t num_wg,
                               int32_t tile, int32_t* wg_indptr, int64_t cap_wg, int32_t* units,
                               int64_t cap_units, int32_t* counts) {
  if (!group_req_indptr || !prefix_lens || !counts || num_groups < 1)
    return fail(PKVMLA_EINVAL, "null argument or num_groups < 1");
  if (num_wg < 1 || tile < 1 || num_heads < 16 || num_heads % 16)
    return fail(PKVMLA_EINVAL, "num_wg, tile must be >= 1, num_heads a multiple of 16");
  if (group_req_indptr[0] != 0) return fail(PKVMLA_EINVAL, "group_req_indptr[0] must be 0");
  for (int32_t g = 0; g < num_groups; ++g)
    if (group_req_indptr[g + 1] < group_req_indptr[g] || prefix_lens[g] < 0)
      return fail(PKVMLA_EINVAL, "group %d: decreasing indptr or negative prefix length", g);
  pkvmla::RowSchedule s;
  if (!pkvmla::build_row_schedule(group_req_indptr, num_groups, prefix_lens, num_heads, num_wg,
                                  tile, &s))
    return fail(PKVMLA_EINVAL, "row schedule construction failed");
  counts[0] = s.grid;
  counts[1] = (int32_t)(s.units.size() / pkvmla::kUnitRecordInts);
  counts[2] = s.n_slots;
  if ((int64_t)s.wg_indptr.size() > cap_wg || (int64_t)s.units.size() > cap_units)
    return fail(PKVMLA_EINVAL, "output capacity too small (need %zu, %zu)", s.wg_indptr.size(),
                s.units.size());
  if (!s.wg_indptr.empty() && !wg_indptr) return fail(PKVMLA_EINVAL, "null wg_indptr");
  if (!s.units.empty() && !units) return fail(PKVMLA_EINVAL, "null units");
  std::copy(s.wg_indptr.begin(), s.wg_indptr.end(), wg_indptr);
  std::copy(s.units.begin(), s.units.end(), units);
  return ok();
}

int pkvmla_schedule_chain_host(const int32_t* group_req_indptr, int32_t num_groups,
                                const int32_t* prefix_lens, const int32_t* kv_lens, int32_t batch,
                                int32_t num_wg, int32_t tile, int32_t* wg_indptr, int64_t cap_wg,
                                int32_t* units, int64_t cap_units, int32_t* merges,
                                int64_t cap_merges, int32_t* slot_list, int64_t cap_list,
                                int32_t* counts) {
  if (!group_req_indptr || !prefix_lens || !kv_lens || !counts || num_groups < 1 || batch < 1)
    return fail(PKVMLA_EINVAL, "null argument, num_groups < 1 or batch < 1");
  if (num_wg < 1 || tile < 1) return fail(PKVMLA_EINVAL, "num_wg and tile must be >= 1");
  if (group_req_indptr[0] != 0 || group_req_indptr[num_groups] != batch)
    return fail(PKVMLA_EINVAL, "group_req_indptr must run from 0 to batch");
  for (int32_t g = 0; g < num_groups; ++g)
    if (group_req_indptr[g + 1] < group_req_indptr[g] || prefix_lens[g] < 1)
      return fail(PKVMLA_EINVAL, "group %d: decreasing indptr or empty prefix", g);
  for (int32_t b = 0; b < batch; ++b)
    if (kv_lens[b] < 0) return fail(PKVMLA_EINVAL, "negative suffix length at %d", b);
  pkvmla::RowSchedule s;
  std::vector<int32_t> m, l;
  if (!pkvmla::build_chain_schedule(group_req_indptr, num_groups, prefix_lens, kv_lens, batch,
                                    num_wg, tile, &s, &m, &l))
    return fail(PKVMLA_EINVAL, "chain schedule construction failed");
  counts[0] = s.grid;
  counts[1] = (int32_t)(s.units.size() / pkvmla::kUnitRecordInts);
  counts[2] = (int32_t)(m.size() / pkvmla::kMergeRecordInts);
  counts[3] = (int32_t)l.size();
  if ((int64_t)s.wg_indptr.size() > cap_wg || (int64_t)s.units.size() > cap_units ||
      (int64_t)m.size() > cap_merges || (int64_t)l.size() > cap_list)
    return fail(PKVMLA_EINVAL, "output capacity too small");
  if (!wg_indptr || (!s.units.empty() && !units) || (!m.empty() && !merges) ||
      (!l.empty() && !slot_list))
    return fail(PKVMLA_EINVAL, "null output");
  std::copy(s.wg_indptr.begin(), s.wg_indptr.end(), wg_indptr);
  std::copy(s.units.begin(), s.units.end(), units);
  std::copy(m.begin(), m.end(), merges);
  std::copy(l.begin(), l.end(), slot_list);
  return ok();
}

int pkvmla_schedule_qo_rows_host(const int32_t* qo_indptr, const int32_t* kv_lens,
                                 int32_t batch, int32_t num_heads, int32_t num_wg, int32_t tile,
                                 int32_t fixed_cost, int32_t* wg_indptr, int64_t cap_wg,
                                 int32_t* units, int64_t cap_units, int32_t* merges,
                                 int64_t cap_merges, int32_t* slot_list, int64_t cap_list,
                                 int32_t* counts) {
  if (!qo_indptr || !kv_lens || !counts || batch < 1)
    return fail(PKVMLA_EINVAL, "null argument or batch < 1");
  if (num_wg < 1 || tile < 1 || fixed_cost < 0)
    return fail(PKVMLA_EINVAL, "num_wg and tile must be >= 1, fixed_cost >= 0");
  if (num_heads != 16 && num_heads != 32)
    return fail(PKVMLA_EUNSUPPORTED, "row blocks of query tokens need 16 or 32 heads (got %d)",
                num_heads);
  if (qo_indptr[0] != 0) return fail(PKVMLA_EINVAL, "qo_indptr[0] must be 0");
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t n = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
    if (n < 1 || n > kv_lens[b])
      return fail(PKVMLA_EINVAL, "request %d: %lld query tokens for kv_len %d", b, (long long)n,
                  kv_lens[b]);
  }
  pkvmla::RowSchedule s;
  std::vector<int32_t> seq, m, l;
  if (!pkvmla::build_qo_row_schedule(qo_indptr, kv_lens, batch, num_heads, num_wg, tile,
                                     fixed_cost, &s, &seq, &m, &l))
    return fail(PKVMLA_EINVAL, "row-block schedule construction failed");
  counts[0] = s.grid;
  counts[1] = (int32_t)(s.units.size() / pkvmla::kUnitRecordInts);
  counts[2] = (int32_t)(m.size() / pkvmla::kMergeRecordInts);
  counts[3] = (int32_t)l.size();
  counts[4] = s.n_slots;
  counts[5] = pkvmla::qo_uses_row_blocks(qo_indptr, batch, num_heads) ? 1 : 0;
  if ((int64_t)s.wg_indptr.size() > cap_wg || (int64_t)s.units.size() > cap_units ||
      (int64_t)m.size() > cap_merges || (int64_t)l.size() > cap_list)
    return fail(PKVMLA_EINVAL, "output capacity too small");
  if (!wg_indptr || (!s.units.empty() && !units) || (!m.empty() && !merges) ||
      (!l.empty() && !slot_list))
    return fail(PKVMLA_EINVAL, "null output");
  std::copy(s.wg_indptr.begin(), s.wg_indptr.end(), wg_indptr);
  std::copy(s.units.begin(), s.units.end(), units);
  std::copy(m.begin(), m.end(), merges);
  std::copy(l.begin(), l.end(), slot_list);
  return ok();
}

int pkvmla_plan_create_with_capacity(const int32_t* kv_indptr, const int32_t* kv_indices,
                                     const int32_t* kv_lens, int32_t batch, int32_t num_pages,
                                     int32_t num_heads, int32_t ckv_dim, int32_t kpe_dim,
                                     int32_t page_size, float sm_scale, int64_t index_capacity,
                                     void* stream, pkvmla_plan* out) {
  if (!out) return fail(PKVMLA_EINVAL, "null plan output pointer");
  *out = nullptr;
  int32_t log2_ps;
  float scale;
  int rc = check_shape(batch, num_pages, num_heads, ckv_dim, kpe_dim, page_size, sm_scale,
                       &log2_ps, &scale);
  if (rc) return rc;
  rc = check_pages("kv", kv_indptr, kv_indices, kv_lens, batch, num_pages, page_size, 1);
  if (rc) return rc;
  if (index_capacity < 0) return fail(PKVMLA_EINVAL, "index_capacity must be >= 0");
  if (index_capacity > 0 && index_capacity < kv_indptr[batch])
    return fail(PKVMLA_EINVAL, "index_capacity %lld is below the table's %d page ids",
                (long long)index_capacity, kv_indptr[batch]);

  pkvmla_plan_s* P = new pkvmla_plan_s();
  P->batch = batch;
  P->num_heads = num_heads;
  P->page_size = page_size;
  P->log2_ps = log2_ps;
  P->ckv_dim = ckv_dim;
  P->kpe_dim = kpe_dim;
  P->num_pages = num_pages;
  P->sm_scale = scale;
  P->index_capacity_request = index_capacity;
  P->fixed_launch = index_capacity > 0 ? 1 : 0;
  pkvmla::kernel_config_for(num_heads, &P->cfg);
  std::vector<pkvmla::WorkItem> items((size_t)batch);
  for (int32_t b = 0; b < batch; ++b) items[b] = pkvmla::WorkItem{b, b, kv_lens[b]};
  std::vector<int32_t> sip(kv_indptr, kv_indptr + batch + 1);
  std::vector<int32_t> sl(kv_lens, kv_lens + batch);
  std::vector<int32_t> si(kv_indices, kv_indices + kv_indptr[batch]);
  rc = finish_plan(P, items, sip, sl, si, (hipStream_t)stream);
  if (rc) {
    std::string msg = g_last_error;
    free_plan(P);
    g_last_error = msg;
    return rc;
  }
  *out = P;
  return ok();
}

int pkvmla_plan_create_qo(const int32_t* qo_indptr, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* kv_lens, int32_t batch,
                          int32_t num_pages, int32_t num_heads, int32_t ckv_dim, int32_t kpe_dim,
                          int32_t page_size, float sm_scale, void* stream, pkvmla_plan* out) {
  return pkvmla_plan_create_qo_with_capacity(qo_indptr, kv_indptr, kv_indices, kv_lens, batch,
                                             num_pages, num_heads, ckv_dim, kpe_dim, page_size,
                                             sm_scale, PKVMLA_QO_AUTO, 0, stream, out);
}

int pkvmla_plan_create_qo_layout(const int32_t* qo_indptr, const int32_t* kv_indptr,
                                 const int32_t* kv_indices, const int32_t* kv_lens, int32_t batch,
                                 int32_t num_pages, int32_t num_heads, int32_t ckv_dim,
                                 int32_t kpe_dim, int32_t page_size, float sm_scale,
                                 int32_t layout, void* stream, pkvmla_plan* out) {
  return pkvmla_plan_create_qo_with_capacity(qo_indptr, kv_indptr, kv_indices, kv_lens, batch,
                                             num_pages, num_heads, ckv_dim, kpe_dim, page_size,
                                             sm_scale, layout, 0, stream, out);
}

int pkvmla_plan_create_qo_with_capacity(const int32_t* qo_indptr, const int32_t* kv_indptr,
                                        const int32_t* kv_indices, const int32_t* kv_lens,
                                        int32_t batch, int32_t num_pages, int32_t num_heads,
                                        int32_t ckv_dim, int32_t kpe_dim, int32_t page_size,
                                        float sm_scale, int32_t layout, int64_t index_capacity,
                                        void* stream, pkvmla_plan* out) {
  if (!out) return fail(PKVMLA_EINVAL, "null plan output pointer");
  *out = nullptr;
  int32_t log2_ps;
  float scale;
  int rc = check_shape(batch, num_pages, num_heads, ckv_dim, kpe_dim, page_size, sm_scale,
                       &log2_ps, &scale);
  if (rc) return rc;
  rc = check_pages("kv", kv_indptr, kv_indices, kv_lens, batch, num_pages, page_size, 1);
  if (rc) return rc;
  rc = check_qo(qo_indptr, kv_lens, batch);
  if (rc) return rc;
  if (index_capacity < 0) return fail(PKVMLA_EINVAL, "index_capacity must be >= 0");
  if (index_capacity > 0 && index_capacity < kv_indptr[batch])
    return fail(PKVMLA_EINVAL, "index_capacity %lld is below the table's %d page ids",
                (long long)index_capacity, kv_indptr[batch]);
  if (layout != PKVMLA_QO_AUTO && layout != PKVMLA_QO_TOKENS && layout != PKVMLA_QO_ROW_BLOCKS)
    return fail(PKVMLA_EINVAL, "unknown query-token layout %d", layout);
  if (layout == PKVMLA_QO_ROW_BLOCKS && num_heads != 16 && num_heads != 32)
    return fail(PKVMLA_EUNSUPPORTED, "row blocks of query tokens need 16 or 32 heads (got %d)",
                num_heads);
  const bool rows_layout = layout == PKVMLA_QO_ROW_BLOCKS ||
                           (layout == PKVMLA_QO_AUTO &&
                            pkvmla::qo_uses_row_blocks(qo_indptr, batch, num_heads));
  const int32_t rows = qo_indptr[batch];
  pkvmla_plan_s* P = new pkvmla_plan_s();
  P->batch = rows;  // one query row per (request, new token)
  P->num_requests = batch;
  P->is_qo = rows_layout ? 2 : 1;
  P->num_heads = num_heads;
  P->page_size = page_size;
  P->log2_ps = log2_ps;
  P->ckv_dim = ckv_dim;
  P->kpe_dim = kpe_dim;
  P->num_pages = num_pages;
  P->sm_scale = scale;
  P->index_capacity_request = index_capacity;
  P->fixed_launch = index_capacity > 0 ? 1 : 0;
  pkvmla::kernel_config_for(num_heads, &P->cfg);
  // Query row r = qo_indptr[b] + j sits at position kv_len - qo_len + j and
  // attends tokens 0 .. that position of request b's page list (causal among
  // the request's new tokens, every earlier token visible).  Either one work
  // item of that length over sequence b per query token, or row blocks of
  // 64 query rows (several tokens' heads), each over the whole sequence with
  // the causal bound per row, so one KV tile serves all of them.
  std::vector<pkvmla::WorkItem> items;
  std::vector<int32_t> sip(kv_indptr, kv_indptr + batch + 1);
  std::vector<int32_t> sl(kv_lens, kv_lens + batch);
  std::vector<int32_t> si(kv_indices, kv_indices + kv_indptr[batch]);
  if (rows_layout) {
    P->cfg0 = pkvmla::KernelConfig{8, 16, 4, 1, 4, 1};
    const QoRows qr{qo_indptr, kv_lens, batch};
    rc = finish_plan(P, items, sip, sl, si, (hipStream_t)stream, nullptr, &qr);
  } else {
    items = qo_token_items(qo_indptr, kv_lens, batch);
    rc = finish_plan(P, items, sip, sl, si, (hipStream_t)stream);
  }
  if (rc) {
    std::string msg = g_last_error;
    free_plan(P);
    g_last_error = msg;
    return rc;
  }
  *out = P;
  return ok();
}

int pkvmla_plan_create(const int32_t* kv_indptr, const int32_t* kv_indices,
                       const int32_t* kv_lens, int32_t batch, int32_t num_pages,
                       int32_t num_heads, int32_t ckv_dim, int32_t kpe_dim, int32_t page_size,
                       float sm_scale, void* stream, pkvmla_plan* out) {
  return pkvmla_plan_create_with_capacity(kv_indptr, kv_indices, kv_lens, batch, num_pages,
                                          num_heads, ckv_dim, kpe_dim, page_size, sm_scale, 0,
                                          stream, out);
}

int pkvmla_plan_update(pkvmla_plan P, const int32_t* kv_indptr, const int32_t* kv_indices,
                       const int32_t* kv_lens, void* stream) {
  if (!P) return fail(PKVMLA_EINVAL, "null plan");
  if (P->is_cascade) return fail(PKVMLA_EINVAL, "a cascade plan is updated with pkvmla_plan_update_cascade");
  if (P->is_qo) return fail(PKVMLA_EINVAL, "a plan with several query tokens per request is updated with pkvmla_plan_update_qo");
  int rc = check_pages("kv", kv_indptr, kv_indices, kv_lens, P->batch, P->num_pages,
                       P->page_size, 1);
  if (rc) return rc;
  if ((int64_t)kv_indptr[P->batch] > P->cap_indices)
    return fail(PKVMLA_EINVAL, "%d page ids exceed the plan's capacity of %lld",
                kv_indptr[P->batch], (long long)P->cap_indices);
  int dev = -1;
  PKVMLA_HIP(hipGetDevice(&dev));
  if (dev != P->device)
    return fail(PKVMLA_EINVAL, "plan was built on device %d, current device is %d", P->device,
                dev);
  std::vector<pkvmla::WorkItem> items((size_t)P->batch);
  for (int32_t b = 0; b < P->batch; ++b) items[b] = pkvmla::WorkItem{b, b, kv_lens[b]};
  std::vector<int32_t> sip(kv_indptr, kv_indptr + P->batch + 1);
  std::vector<int32_t> sl(kv_lens, kv_lens + P->batch);
  std::vector<int32_t> si(kv_indices, kv_indices + kv_indptr[P->batch]);
  pkvmla::Schedule sched;
  rc = build_plan_schedule(P, items, sip, si, &sched);
  if (rc) return rc;
  if ((int64_t)sched.units.size() > (int64_t)P->cap_units * pkvmla::kUnitRecordInts ||
      sched.grid > P->cap_lanes || sched.n_slots > P->cap_units)
    return fail(PKVMLA_EINVAL, "schedule exceeds the plan's capacities");
  // the plan takes the new schedule only once its tables are on the device
  rc = upload_tables(P, sched, sip, sl, si, (hipStream_t)stream);
  if (rc) return rc;
  P->sched = std::move(sched);
  return ok();
}

int pkvmla_plan_update_qo(pkvmla_plan P, const int32_t* qo_indptr, const int32_t* kv_indptr,
                          const int32_t* kv_indices, const int32_t* kv_lens, void* stream) {
  if (!P) return fail(PKVMLA_EINVAL, "null plan");
  if (!P->is_qo) return fail(PKVMLA_EINVAL, "not a plan with several query tokens per request");
  const int32_t B = P->num_requests;
  int rc = check_pages("kv", kv_indptr, kv_indices, kv_lens, B, P->num_pages, P->page_size, 1);
  if (rc) return rc;
  rc = check_qo(qo_indptr, kv_lens, B);
  if (rc) return rc;
  if (qo_indptr[B] != P->batch)
    return fail(PKVMLA_EINVAL, "%d query tokens, the plan's tensors have %d", qo_indptr[B], P->batch);
  if ((int64_t)kv_indptr[B] > P->cap_indices)
    return fail(PKVMLA_EINVAL, "%d page ids exceed the plan's capacity of %lld", kv_indptr[B],
                (long long)P->cap_indices);
  int dev = -1;
  PKVMLA_HIP(hipGetDevice(&dev));
  if (dev != P->device)
    return fail(PKVMLA_EINVAL, "plan was built on device %d, current device is %d", P->device,
                dev);
  std::vector<int32_t> sip(kv_indptr, kv_indptr + B + 1);
  std::vector<int32_t> sl(kv_lens, kv_lens + B);
  std::vector<int32_t> si(kv_indices, kv_indices + kv_indptr[B]);
  pkvmla::Schedule sched;
  pkvmla::RowSchedule sched0;
  std::vector<int32_t> list;
  if (P->is_qo == 2) {
    // the plan keeps its layout (row blocks) whatever the new split
    rc = build_qo_row_tables(P, qo_indptr, kv_lens, B, sip, si, &sched, &sched0, &list);
    if (rc) return rc;
    if (sched0.grid > P->cap_lanes0 ||
        (int64_t)sched0.units.size() > (int64_t)P->cap_units0 * pkvmla::kUnitRecordInts ||
        sched.n_slots > P->cap_slots || (int64_t)list.size() > P->cap_list ||
        (int64_t)sched.merges.size() > (int64_t)P->cap_merges * pkvmla::kMergeRecordInts)
      return fail(PKVMLA_EINVAL, "schedule exceeds the plan's capacities");
    rc = upload_tables(P, sched, sip, sl, si, (hipStream_t)stream, &sched0, &list);
    if (rc) return rc;
    P->sched = std::move(sched);
    P->sched0 = std::move(sched0);
    P->slot_list = std::move(list);
    return ok();
  }
  rc = build_plan_schedule(P, qo_token_items(qo_indptr, kv_lens, B), sip, si, &sched);
  if (rc) return rc;
  if ((int64_t)sched.units.size() > (int64_t)P->cap_units * pkvmla::kUnitRecordInts ||
      sched.grid > P->cap_lanes || sched.n_slots > P->cap_slots)
    return fail(PKVMLA_EINVAL, "schedule exceeds the plan's capacities");
  rc = upload_tables(P, sched, sip, sl, si, (hipStream_t)stream);
  if (rc) return rc;
  P->sched = std::move(sched);
  return ok();
}

int pkvmla_plan_create_cascade_with_capacity(
    const int32_t* group_req_indptr, int32_t num_groups, const int32_t* prefix_indptr,
    const int32_t* prefix_indices, const int32_t* prefix_lens, const int32_t* kv_indptr,
    const int32_t* kv_indices, const int32_t* kv_lens, int32_t batch, int32_t num_pages,
    int32_t num_heads, int32_t ckv_dim, int32_t kpe_dim, int32_t page_size, float sm_scale,
    int64_t index_capacity, void* stream, pkvmla_plan* out) {
  if (!out) return fail(PKVMLA_EINVAL, "null plan output pointer");
  *out = nullptr;
  int32_t log2_ps;
  float scale;
  int rc = check_shape(batch, num_pages, num_heads, ckv_dim, kpe_dim, page_size, sm_scale,
                       &log2_ps, &scale);
  if (rc) return rc;
  const CascadeTables t{group_req_indptr, num_groups, prefix_indptr, prefix_indices, prefix_lens,
                        kv_indptr, kv_indices, kv_lens, batch};
  rc = check_cascade(t, num_pages, page_size);
  if (rc) return rc;
  if (index_capacity < 0) return fail(PKVMLA_EINVAL, "index_capacity must be >= 0");
  const int64_t n_ids = (int64_t)prefix_indptr[num_groups] + kv_indptr[batch];
  if (index_capacity > 0 && index_capacity < n_ids)
    return fail(PKVMLA_EINVAL, "index_capacity %lld is below the tables' %lld page ids",
                (long long)index_capacity, (long long)n_ids);

  pkvmla_plan_s* P = new pkvmla_plan_s();
  P->batch = batch;
  P->num_heads = num_heads;
  P->page_size = page_size;
  P->log2_ps = log2_ps;
  P->ckv_dim = ckv_dim;
  P->kpe_dim = kpe_dim;
  P->num_pages = num_pages;
  P->sm_scale = scale;
  P->is_cascade = 1;
  P->num_groups = num_groups;
  P->index_capacity_request = index_capacity;
  P->fixed_launch = index_capacity > 0 ? 1 : 0;
  pkvmla::kernel_config_for(num_heads, &P->cfg);
  // level 0: 64 query rows per workgroup (four head blocks), a whole request
  // per lane above 64 heads (its head groups)
  P->cfg0 = pkvmla::KernelConfig{8, 16, 4, 1, 4, num_heads > 64 ? num_heads / 64 : 1};
  std::vector<int32_t> sip, sl, si;
  std::vector<pkvmla::WorkItem> items;
  cascade_sequences(t, &sip, &sl, &si, &items);
  const Level0Groups l0{group_req_indptr, num_groups, prefix_lens};
  rc = finish_plan(P, items, sip, sl, si, (hipStream_t)stream, &l0);
  if (rc) {
    std::string msg = g_last_error;
    free_plan(P);
    g_last_error = msg;
    return rc;
  }
  *out = P;
  return ok();
}

int pkvmla_plan_create_cascade(const int32_t* group_req_indptr, int32_t num_groups,
                               const int32_t* prefix_indptr, const int32_t* prefix_indices,
                               const int32_t* prefix_lens, const int32_t* kv_indptr,
                               const int32_t* kv_indices, const int32_t* kv_lens, int32_t batch,
                               int32_t num_pages, int32_t num_heads, int32_t ckv_dim,
                               int32_t kpe_dim, int32_t page_size, float sm_scale, void* stream,
                               pkvmla_plan* out) {
  return pkvmla_plan_create_cascade_with_capacity(
      group_req_indptr, num_groups, prefix_indptr, prefix_indices, prefix_lens, kv_indptr,
      kv_indices, kv_lens, batch, num_pages, num_heads, ckv_dim, kpe_dim, page_size, sm_scale, 0,
      stream, out);
}

int pkvmla_plan_update_cascade(pkvmla_plan P, const int32_t* group_req_indptr,
                               const int32_t* prefix_indptr, const int32_t* prefix_indices,
                               const int32_t* prefix_lens, const int32_t* kv_indptr,
                               const int32_t* kv_indices, const int32_t* kv_lens, void* stream) {
  if (!P) return fail(PKVMLA_EINVAL, "null plan");
  if (!P->is_cascade) return fail(PKVMLA_EINVAL, "not a cascade plan (use pkvmla_plan_update)");
  const CascadeTables t{group_req_indptr, P->num_groups, prefix_indptr, prefix_indices,
                        prefix_lens, kv_indptr, kv_indices, kv_lens, P->batch};
  int rc = check_cascade(t, P->num_pages, P->page_size);
  if (rc) return rc;
  const int64_t n_ids = (int64_t)prefix_indptr[P->num_groups] + kv_indptr[P->batch];
  if (n_ids > P->cap_indices)
    return fail(PKVMLA_EINVAL, "%lld page ids exceed the plan's capacity of %lld",
                (long long)n_ids, (long long)P->cap_indices);
  int dev = -1;
  PKVMLA_HIP(hipGetDevice(&dev));
  if (dev != P->device)
    return fail(PKVMLA_EINVAL, "plan was built on device %d, current device is %d", P->device,
                dev);
  std::vector<int32_t> sip, sl, si;
  std::vector<pkvmla::WorkItem> items;
  cascade_sequences(t, &sip, &sl, &si, &items);
  pkvmla::Schedule sched;
  pkvmla::RowSchedule sched0;
  std::vector<int32_t> list;
  const Level0Groups l0{group_req_indptr, P->num_groups, prefix_lens};
  if (P->cascade_chain) {
    // a plan in the one-launch layout keeps it (an update that would need the
    // two-level layout, an empty prefix, is refused: its launches differ)
    if (!chain_eligible(P, l0))
      return fail(PKVMLA_EUNSUPPORTED, "this plan runs its cascade in one launch, which needs "
                  "every prefix non-empty (build it with an index_capacity to update freely)");
    rc = build_chain_tables(P, l0, kv_lens, sip, si, &sched, &sched0, &list);
  } else {
    rc = build_cascade_schedules(P, l0, items, sip, si, &sched, &sched0, &list);
  }
  if (rc) return rc;
  if ((int64_t)sched.units.size() > (int64_t)P->cap_units * pkvmla::kUnitRecordInts ||
      sched.grid > P->cap_lanes || sched0.grid > P->cap_lanes0 ||
      (int64_t)sched0.units.size() > (int64_t)P->cap_units0 * pkvmla::kUnitRecordInts ||
      sched.n_slots > P->cap_slots || (int64_t)list.size() > P->cap_list)
    return fail(PKVMLA_EINVAL, "schedule exceeds the plan's capacities");
  // the plan takes the new schedules only once its tables are on the device
  rc = upload_tables(P, sched, sip, sl, si, (hipStream_t)stream, &sched0, &list);
  if (rc) return rc;
  P->sched = std::move(sched);
  P->sched0 = std::move(sched0);
  P->slot_list = std::move(list);
  return ok();
}

}  // extern "C"

namespace {

// Bytes of split workspace the plan's runs can touch: partial outputs (bf16)
// and lse (fp32) for every partial slot a schedule of this plan can use.
size_t workspace_bytes(const pkvmla_plan_s* P) {
  const size_t slots = P->fixed_launch ? (size_t)P->cap_slots : (size_t)P->sched.n_slots;
  return slots * (size_t)P->num_heads * (pkvmla::kCkvDim * sizeof(uint16_t) + sizeof(float));
}

// KV cache element type of a run: bf16, or OCP E4M3 codes with per-tensor
// scales (a value is scale * code value).
struct KvFormat {
  int fp8;
  float ckv_scale, kpe_scale;
};

int run_impl(pkvmla_plan P, const void* q_nope, const void* q_pe, const void* ckv_cache,
             const void* kpe_cache, int64_t ckv_row_stride, int64_t kpe_row_stride, void* out,
             float* lse, void* stream, void* workspace, size_t workspace_slots,
             KvFormat kv = KvFormat{0, 1.f, 1.f});

}  // namespace

extern "C" {

int pkvmla_run_strided(pkvmla_plan P, const void* q_nope, const void* q_pe,
                       const void* ckv_cache, const void* kpe_cache, int64_t ckv_row_stride,
                       int64_t kpe_row_stride, void* out, float* lse, void* stream) {
  if (!P) return fail(PKVMLA_EINVAL, "null plan");
  return run_impl(P, q_nope, q_pe, ckv_cache, kpe_cache, ckv_row_stride, kpe_row_stride, out,
                  lse, stream, P->d_part, (size_t)P->cap_slots);
}

int pkvmla_run_noalloc(pkvmla_plan P, const void* q_nope, const void* q_pe,
                       const void* ckv_cache, const void* kpe_cache, void* out, float* lse,
                       void* stream) {
  if (!P) return fail(PKVMLA_EINVAL, "null plan");
  const size_t need = workspace_bytes(P);
  if (need > pkvmla::kScratchBytes)
    return fail(PKVMLA_EUNSUPPORTED,
                "the plan's split workspace needs %zu bytes, more than the %zu bytes of static "
                "scratch (use pkvmla_run)",
                need, pkvmla::kScratchBytes);
  int dev = -1;
  PKVMLA_HIP(hipGetDevice(&dev));
  if (dev != P->device)
    return fail(PKVMLA_EINVAL, "plan was built on device %d, current device is %d", P->device,
                dev);
  void* ws = nullptr;
  PKVMLA_HIP(pkvmla::scratch_address(dev, &ws));
  // the scratch holds as many slots as fit; the plan's need is within that
  const size_t slots = pkvmla::kScratchBytes /
                       ((size_t)P->num_heads * (pkvmla::kCkvDim * sizeof(uint16_t) + sizeof(float)));
  return run_impl(P, q_nope, q_pe, ckv_cache, kpe_cache, pkvmla::kCkvDim, pkvmla::kKpeDim, out,
                  lse, stream, ws, slots);
}

int pkvmla_run_fp8(pkvmla_plan P, const void* q_nope, const void* q_pe, const void* ckv_cache,
                   const void* kpe_cache, int64_t ckv_row_stride, int64_t kpe_row_stride,
                   float ckv_scale, float kpe_scale, void* out, float* lse, void* stream) {
  if (!P) return fail(PKVMLA_EINVAL, "null plan");
  if (!(std::isfinite(ckv_scale) && ckv_scale > 0.f && std::isfinite(kpe_scale) &&
        kpe_scale > 0.f))
    return fail(PKVMLA_EINVAL, "fp8 cache scales must be finite and > 0 (got %g, %g)",
                (double)ckv_scale, (double)kpe_scale);
  // strides in bytes: ckv rows in 16-byte loads, kpe rows in 8-byte loads
  if (ckv_row_stride < pkvmla::kCkvDim || kpe_row_stride < pkvmla::kKpeDim ||
      (ckv_row_stride & 15) || (kpe_row_stride & 7) || ckv_row_stride > (1 << 20) ||
      kpe_row_stride > (1 << 20))
    return fail(PKVMLA_EINVAL,
                "fp8 row strides (bytes) must be >= 512 and a multiple of 16 (ckv), >= 64 and "
                "a multiple of 8 (kpe), <= 2^20 (got %lld, %lld)",
                (long long)ckv_row_stride, (long long)kpe_row_stride);
  if ((reinterpret_cast<uintptr_t>(kpe_cache) & 7u))
    return fail(PKVMLA_EINVAL, "the fp8 kpe cache must be 8-byte aligned");
  return run_impl(P, q_nope, q_pe, ckv_cache, kpe_cache, ckv_row_stride, kpe_row_stride, out,
                  lse, stream, P->d_part, (size_t)P->cap_slots,
                  KvFormat{1, ckv_scale, kpe_scale});
}

}  // extern "C"

namespace {

int run_impl(pkvmla_plan P, const void* q_nope, const void* q_pe, const void* ckv_cache,
             const void* kpe_cache, int64_t ckv_row_stride, int64_t kpe_row_stride, void* out,
             float* lse, void* stream, void* workspace, size_t workspace_slots, KvFormat kv) {
  if (!P) return fail(PKVMLA_EINVAL, "null plan");
  if (!q_nope || !q_pe || !ckv_cache || !kpe_cache || !out || !lse)
    return fail(PKVMLA_EINVAL, "null tensor pointer");
  // bf16 strides in elements: whole 16-byte chunks, at least one row, and
  // every row offset (pages x page_size rows) inside 32-bit row arithmetic
  // (fp8 strides, in bytes, are checked by pkvmla_run_fp8)
  if (!kv.fp8 && (ckv_row_stride < pkvmla::kCkvDim || kpe_row_stride < pkvmla::kKpeDim ||
                  (ckv_row_stride & 7) || (kpe_row_stride & 7) || ckv_row_stride > (1 << 20) ||
                  kpe_row_stride > (1 << 20)))
    return fail(PKVMLA_EINVAL,
                "row strides must be multiples of 8 elements, >= 512 (ckv) and >= 64 (kpe), "
                "<= 2^20 (got %lld, %lld)",
                (long long)ckv_row_stride, (long long)kpe_row_stride);
  if (!aligned16(q_nope) || !aligned16(q_pe) || !aligned16(ckv_cache) ||
      (!kv.fp8 && !aligned16(kpe_cache)) || !aligned16(out) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(PKVMLA_EINVAL, "device pointers must be 16-byte aligned (lse 4-byte)");
  int dev = -1;
  PKVMLA_HIP(hipGetDevice(&dev));
  if (dev != P->device)
    return fail(PKVMLA_EINVAL, "plan was built on device %d, current device is %d", P->device,
                dev);
  hipStream_t s = (hipStream_t)stream;
  // workspace layout: part_o bf16 [slots][H][512], then part_lse fp32 [slots][H]
  const size_t part_o_elems = workspace_slots * P->num_heads * pkvmla::kCkvDim;
  uint16_t* part_o = static_cast<uint16_t*>(workspace);
  pkvmla::DecodeParams d{};
  d.q_nope = static_cast<const uint16_t*>(q_nope);
  d.q_pe = static_cast<const uint16_t*>(q_pe);
  d.ckv = static_cast<const uint16_t*>(ckv_cache);
  d.kpe = static_cast<const uint16_t*>(kpe_cache);
  const int64_t esize = kv.fp8 ? 1 : 2;  // bytes per cache element
  d.ckv_stride = (int32_t)(ckv_row_stride * esize);
  d.kpe_stride = (int32_t)(kpe_row_stride * esize);
  d.out = static_cast<uint16_t*>(out);
  d.lse = lse;
  d.part_o = part_o;
  d.part_lse = part_o ? reinterpret_cast<float*>(part_o + part_o_elems) : nullptr;
  d.wg_indptr = P->d_wg_indptr;
  d.units = P->d_units;
  d.seq_indices = P->d_seq_indices;
  d.num_heads = P->num_heads;
  d.head_groups = P->cfg.head_groups;
  // lanes past the schedule's have no units (their workgroups return at once)
  // (row-block plans of query tokens have every unit in the level-0 table)
  d.n_lanes = P->is_qo == 2 ? 0 : P->fixed_launch ? P->cap_lanes : P->sched.grid;
  d.waves = P->cfg.waves;
  d.heads_per_wave = P->cfg.heads_per_wave;
  d.stages = P->cfg.stages;
  d.log2_ps = P->log2_ps;
  // fp8: the ckv scale multiplies every score (the kpe part is rescaled by
  // kpe_ratio in the kernel) and every output row
  const double eff_scale = (double)P->sm_scale * (kv.fp8 ? (double)kv.ckv_scale : 1.0);
  d.sm_scale = (float)eff_scale;
  d.score_log2 = (float)(eff_scale * 1.4426950408889634);
  d.rescale_thr = (float)(8.0 / (eff_scale * 1.4426950408889634));
  d.fp8 = kv.fp8;
  d.v_scale = kv.ckv_scale;
  d.kpe_ratio = kv.fp8 ? (float)((double)kv.kpe_scale / (double)kv.ckv_scale) : 1.f;
  const int slot_ev = (int)(P->timed_runs % pkvmla_plan_s::kTimingSlots);
  unsigned long long* rec =
      P->timing ? P->d_stamps + (size_t)slot_ev * 2 *
                                    (P->timing_wgs0 + P->timing_wgs + P->timing_wgsm)
                : nullptr;
  d.stamps = rec ? rec + 2 * (size_t)P->timing_wgs0 : nullptr;
  if (P->timing == 2) PKVMLA_HIP(hipEventRecord(P->ev[2 * slot_ev], s));
  int32_t grid0 = 0;
  d.qo_log2h = -1;
  d.wait_limit = P->wait_limit;
  if ((P->is_cascade || P->is_qo == 2) && (P->sched0.grid > 0 || P->fixed_launch)) {
    // level 0: the groups' query rows over their shared prefixes, or the row
    // blocks of several query tokens per request (causal bound per row)
    pkvmla::DecodeParams d0 = d;
    d0.qo_log2h = P->is_qo == 2 ? (P->num_heads == 16 ? 4 : 5) : -1;
    d0.wg_indptr = P->d_wg0;
    d0.units = P->d_units0;
    d0.head_groups = P->cfg0.head_groups;
    d0.n_lanes = P->fixed_launch ? P->cap_lanes0 : P->sched0.grid;
    d0.waves = P->cfg0.waves;
    d0.heads_per_wave = P->cfg0.heads_per_wave;
    d0.stages = P->cfg0.stages;
    d0.row_blocks = P->cascade_chain ? 0 : 1;
    d0.stamps = rec;
    grid0 = d0.n_lanes > 0 ? pkvmla::decode_grid(d0.n_lanes, d0.head_groups) : 0;
    PKVMLA_HIP(pkvmla::launch_decode(d0, s));
  }
  PKVMLA_HIP(pkvmla::launch_decode(d, s));
  if (P->timing) {
    if (P->timing == 2) PKVMLA_HIP(hipEventRecord(P->ev[2 * slot_ev + 1], s));
    P->timing_grid[slot_ev][0] = grid0;
    P->timing_grid[slot_ev][1] = d.n_lanes > 0 ? pkvmla::decode_grid(d.n_lanes, d.head_groups) : 0;
    P->timing_grid[slot_ev][2] = 0;
  }
  // fixed launches cover every merge record slot (records past the live ones
  // have count 0 and are skipped by the kernel)
  const int n_merges = P->fixed_launch
                           ? P->cap_merges
                           : (int)(P->sched.merges.size() / pkvmla::kMergeRecordInts);
  if (n_merges > 0) {
    pkvmla::MergeParams m{};
    m.part_o = d.part_o;
    m.part_lse = d.part_lse;
    m.merges = P->d_merges;
    m.slot_list = P->d_slot_list;
    m.out = d.out;
    m.lse = lse;
    m.num_heads = P->num_heads;
    m.stamps = rec ? rec + 2 * (size_t)(P->timing_wgs0 + P->timing_wgs) : nullptr;
    if (rec) P->timing_grid[slot_ev][2] = n_merges * (P->num_heads / 4);
    PKVMLA_HIP(pkvmla::launch_merge(m, n_merges, s));
  }
  if (P->timing) ++P->timed_runs;
  return ok();
}

}  // namespace

extern "C" {

int pkvmla_run(pkvmla_plan P, const void* q_nope, const void* q_pe, const void* ckv_cache,
               const void* kpe_cache, void* out, float* lse, void* stream) {
  return pkvmla_run_strided(P, q_nope, q_pe, ckv_cache, kpe_cache, pkvmla::kCkvDim,
                            pkvmla::kKpeDim, out, lse, stream);
}

void pkvmla_plan_destroy(pkvmla_plan P) { free_plan(P); }

int pkvmla_plan_set_wait_limit(pkvmla_plan P, int32_t polls) {
  if (!P) return fail(PKVMLA_EINVAL, "null plan");
  if (polls < 0) return fail(PKVMLA_EINVAL, "wait limit must be >= 0");
  P->wait_limit = polls;
  return ok();
}

int pkvmla_plan_set_timing(pkvmla_plan P, int32_t enable) {
  if (!P) return fail(PKVMLA_EINVAL, "null plan");
  if (enable < 0 || enable > 2) return fail(PKVMLA_EINVAL, "timing mode must be 0, 1 or 2");
  if (enable == 2 && !P->ev[0]) {
    // timing-only events: no system-scope fence (cache write-back and
    // invalidation) at each record, which would add its own cost to the
    // interval and to the kernels that follow
    for (hipEvent_t& e : P->ev) PKVMLA_HIP(hipEventCreateWithFlags(&e, hipEventDisableSystemFence));
  }
  if (enable) {
    // records for the largest launches the plan can make (its capacities)
    const bool has_l0 = P->is_cascade || P->is_qo == 2;
    const int32_t w0 = has_l0 ? pkvmla::decode_grid(std::max(P->cap_lanes0, 1), P->cfg0.head_groups) : 0;
    const int32_t w1 = pkvmla::decode_grid(std::max(P->cap_lanes, 1), P->cfg.head_groups);
    const int32_t wm = std::max(P->cap_merges, 1) * (P->num_heads / 4);
    if (!P->d_stamps || w0 != P->timing_wgs0 || w1 != P->timing_wgs || wm != P->timing_wgsm) {
      if (P->d_stamps) {
        PKVMLA_HIP(hipDeviceSynchronize());
        PKVMLA_HIP(hipFree(P->d_stamps));
        P->d_stamps = nullptr;
      }
      const size_t n = (size_t)pkvmla_plan_s::kTimingSlots * 2 * (size_t)(w0 + w1 + wm);
      PKVMLA_HIP(hipMalloc(&P->d_stamps, n * sizeof(unsigned long long)));
      P->timing_wgs0 = w0;
      P->timing_wgs = w1;
      P->timing_wgsm = wm;
    }
  }
  P->timing = enable;
  P->timed_runs = 0;
  return ok();
}

namespace {

// Per recorded run (oldest first): the span of its decode launches (earliest
// workgroup start to latest workgroup end) and its start, in real-time
// counter ticks (100 MHz).
int timing_records(pkvmla_plan P, std::vector<unsigned long long>* start,
                   std::vector<unsigned long long>* span,
                   std::vector<unsigned long long>* merge_start = nullptr) {
  PKVMLA_HIP(hipDeviceSynchronize());
  const int64_t K = pkvmla_plan_s::kTimingSlots;
  const int64_t n = std::min<int64_t>(P->timed_runs, K);
  const size_t per = 2 * (size_t)(P->timing_wgs0 + P->timing_wgs + P->timing_wgsm);
  std::vector<unsigned long long> all(std::max<size_t>(1, (size_t)K * per));
  if (n > 0)
    PKVMLA_HIP(hipMemcpy(all.data(), P->d_stamps, (size_t)K * per * sizeof(unsigned long long),
                         hipMemcpyDeviceToHost));
  start->clear();
  span->clear();
  if (merge_start) merge_start->clear();
  for (int64_t r = P->timed_runs - n; r < P->timed_runs; ++r) {
    const int64_t slot = r % K;
    const unsigned long long* rec = all.data() + (size_t)slot * per;
    unsigned long long lo = ~0ull, hi = 0;
    auto scan = [&](const unsigned long long* x, int32_t wgs) {
      for (int32_t b = 0; b < wgs; ++b) {
        lo = std::min(lo, x[2 * b]);
        hi = std::max(hi, x[2 * b + 1]);
      }
    };
    scan(rec, P->timing_grid[slot][0]);
    scan(rec + 2 * (size_t)P->timing_wgs0, P->timing_grid[slot][1]);
    start->push_back(lo);
    span->push_back(hi >= lo ? hi - lo : 0);
    if (merge_start) {
      // earliest merge block start (0: the run launched no merge)
      const unsigned long long* mrec = rec + 2 * (size_t)(P->timing_wgs0 + P->timing_wgs);
      unsigned long long ms = ~0ull;
      for (int32_t b = 0; b < P->timing_grid[slot][2]; ++b) ms = std::min(ms, mrec[2 * b]);
      merge_start->push_back(P->timing_grid[slot][2] > 0 ? ms : 0);
    }
  }
  return PKVMLA_OK;
}

}  // namespace

int pkvmla_plan_timing(pkvmla_plan P, double* event_ms, double* span_ms, int64_t* n_runs) {
  if (!P || !event_ms || !span_ms || !n_runs) return fail(PKVMLA_EINVAL, "null argument");
  std::vector<unsigned long long> start, span;
  int rc = timing_records(P, &start, &span);
  if (rc) return rc;
  const int64_t n = (int64_t)span.size();
  double tot = 0.0, sp = 0.0;
  for (int64_t i = 0; i < n; ++i) {
    if (P->timing == 2 && P->ev[0]) {
      const int64_t slot = (P->timed_runs - n + i) % pkvmla_plan_s::kTimingSlots;
      float ms = 0.f;
      PKVMLA_HIP(hipEventElapsedTime(&ms, P->ev[2 * slot], P->ev[2 * slot + 1]));
      tot += ms;
    }
    sp += (double)span[i] * 1e-5;  // 100 MHz ticks -> ms
  }
  *event_ms = tot;
  *span_ms = sp;
  *n_runs = n;
  return ok();
}

int pkvmla_plan_timing_runs(pkvmla_plan P, double* span_us, double* start_us,
                            double* merge_start_us, int64_t cap, int64_t* n_runs) {
  if (!P || !n_runs) return fail(PKVMLA_EINVAL, "null argument");
  std::vector<unsigned long long> start, span, mstart;
  int rc = timing_records(P, &start, &span, &mstart);
  if (rc) return rc;
  const int64_t n = (int64_t)span.size();
  *n_runs = n;
  if (n > cap || (n > 0 && (!span_us || !start_us || !merge_start_us)))
    return fail(PKVMLA_EINVAL, "output capacity too small (%lld runs)", (long long)n);
  for (int64_t i = 0; i < n; ++i) {
    span_us[i] = (double)span[i] * 1e-2;
    start_us[i] = (double)(start[i] - start[0]) * 1e-2;
    merge_start_us[i] = mstart[i] ? (double)(mstart[i] - start[0]) * 1e-2 : -1.0;
  }
  return ok();
}

int pkvmla_plan_export(pkvmla_plan P, int32_t* buf, int64_t cap, int64_t* used) {
  if (!P || !used) return fail(PKVMLA_EINVAL, "null plan or used pointer");
  const int64_t n_wg = (int64_t)P->sched.wg_indptr.size();
  const int64_t n_u = (int64_t)P->sched.units.size();
  const int64_t n_m = (int64_t)P->sched.merges.size();
  const int64_t n_wg0 = (int64_t)P->sched0.wg_indptr.size();
  const int64_t n_u0 = (int64_t)P->sched0.units.size();
  const int64_t n_sl = (int64_t)P->slot_list.size();
  const int64_t need = 32 + n_wg + n_u + n_m + (P->num_seqs + 1) + P->num_seqs + P->n_indices +
                       n_wg0 + n_u0 + n_sl;
  *used = need;
  if (!buf || cap < need) return fail(PKVMLA_EINVAL, "buffer too small: need %lld int32", (long long)need);
  PKVMLA_HIP(hipDeviceSynchronize());
  memset(buf, 0, 32 * sizeof(int32_t));
  buf[0] = 1;
  buf[1] = P->batch;
  buf[2] = P->num_heads;
  buf[3] = P->page_size;
  buf[4] = P->ckv_dim;
  buf[5] = P->kpe_dim;
  buf[6] = pkvmla::kTile;
  buf[7] = P->cfg.waves;
  buf[8] = P->cfg.heads_per_wave;
  buf[9] = P->cfg.stages;
  buf[10] = P->cfg.wg_per_cu;
  buf[11] = P->cfg.fixed_cost;
  buf[12] = P->sched.grid;
  buf[13] = (int32_t)(n_u / pkvmla::kUnitRecordInts);
  buf[14] = (int32_t)(n_m / pkvmla::kMergeRecordInts);
  buf[15] = P->sched.n_slots;
  buf[16] = P->num_seqs;
  buf[17] = (int32_t)P->n_indices;
  buf[18] = P->num_cu;
  memcpy(&buf[19], &P->sm_scale, sizeof(float));
  buf[20] = P->is_cascade;
  buf[21] = P->num_groups;
  buf[22] = P->cfg.head_groups;
  buf[23] = pkvmla::decode_grid(P->fixed_launch ? P->cap_lanes : P->sched.grid,
                                P->cfg.head_groups);
  buf[24] = P->fixed_launch;
  buf[25] = (int32_t)std::min<int64_t>(P->cap_indices, INT32_MAX);
  buf[26] = P->is_qo;
  buf[27] = P->num_requests;
  buf[28] = P->sched0.grid;
  buf[29] = (int32_t)(n_u0 / pkvmla::kUnitRecordInts);
  buf[30] = (int32_t)n_sl;
  buf[31] = P->cascade_chain;
  int32_t* dst = buf + 32;
  auto pull = [&](const int32_t* src, int64_t n) -> hipError_t {
    hipError_t e = n ? hipMemcpy(dst, src, n * sizeof(int32_t), hipMemcpyDeviceToHost) : hipSuccess;
    dst += n;
    return e;
  };
  PKVMLA_HIP(pull(P->d_wg_indptr, n_wg));
  PKVMLA_HIP(pull(P->d_units, n_u));
  PKVMLA_HIP(pull(P->d_merges, n_m));
  PKVMLA_HIP(pull(P->d_seq_indptr, P->num_seqs + 1));
  PKVMLA_HIP(pull(P->d_seq_lens, P->num_seqs));
  PKVMLA_HIP(pull(P->d_seq_indices, P->n_indices));
  PKVMLA_HIP(pull(P->d_wg0, n_wg0));
  PKVMLA_HIP(pull(P->d_units0, n_u0));
  PKVMLA_HIP(pull(P->d_slot_list, n_sl));
  return ok();
}

int pkvmla_gather_rows(pkvmla_plan P, int64_t* n_rows) {
  if (!P || !n_rows) return fail(PKVMLA_EINVAL, "null argument");
  int64_t n = P->sched.total_rows;
  for (size_t i = 0; i < P->sched0.units.size(); i += pkvmla::kUnitRecordInts)
    n += P->sched0.units[i + 3] - P->sched0.units[i + 2];
  *n_rows = n;
  return ok();
}

int pkvmla_gather(pkvmla_plan P, const void* ckv_cache, const void* kpe_cache, void* rows,
                  void* stream) {
  if (!P) return fail(PKVMLA_EINVAL, "null plan");
  int64_t n_rows = 0;
  (void)pkvmla_gather_rows(P, &n_rows);
  if (!ckv_cache || !kpe_cache || (!rows && n_rows > 0))
    return fail(PKVMLA_EINVAL, "null tensor pointer");
  if (!aligned16(ckv_cache) || !aligned16(kpe_cache) || !aligned16(rows))
    return fail(PKVMLA_EINVAL, "device pointers must be 16-byte aligned");
  int dev = -1;
  PKVMLA_HIP(hipGetDevice(&dev));
  if (dev != P->device)
    return fail(PKVMLA_EINVAL, "plan was built on device %d, current device is %d", P->device,
                dev);
  pkvmla::GatherParams g{};
  g.ckv = static_cast<const uint16_t*>(ckv_cache);
  g.kpe = static_cast<const uint16_t*>(kpe_cache);
  g.rows = static_cast<uint16_t*>(rows);
  g.units = P->d_units;
  g.seq_indices = P->d_seq_indices;
  g.log2_ps = P->log2_ps;
  g.ckv_stride = pkvmla::kCkvDim * 2;
  g.kpe_stride = pkvmla::kKpeDim * 2;
  const int n_units = (int)(P->sched.units.size() / pkvmla::kUnitRecordInts);
  if (!P->is_cascade && P->is_qo != 2) {
    PKVMLA_HIP(pkvmla::launch_gather(g, n_units, (hipStream_t)stream));
    return ok();
  }
  // cascade: the level-0 pieces (prefix tokens, once per row-block piece)
  // then the suffix units; query-token row blocks: their pieces; as gather
  // records (request and sequence fields unused, row = tokens before); a
  // temporary table, and a wait before it is freed
  std::vector<int32_t> gu;
  int64_t row = 0;
  auto add = [&](const std::vector<int32_t>& us) {
    for (size_t i = 0; i < us.size(); i += pkvmla::kUnitRecordInts) {
      gu.insert(gu.end(), {0, us[i + 1], us[i + 2], us[i + 3], -1, (int32_t)row, us[i + 6], us[i + 7]});
      row += us[i + 3] - us[i + 2];
    }
  };
  add(P->sched0.units);
  add(P->sched.units);
  if (gu.empty()) return ok();
  if (row > INT32_MAX) return fail(PKVMLA_EUNSUPPORTED, "too many rows");
  int32_t* d_gu = nullptr;
  PKVMLA_HIP(hipMalloc(&d_gu, gu.size() * sizeof(int32_t)));
  hipError_t e = hipMemcpy(d_gu, gu.data(), gu.size() * sizeof(int32_t), hipMemcpyHostToDevice);
  if (e == hipSuccess) {
    g.units = d_gu;
    e = pkvmla::launch_gather(g, (int)(gu.size() / pkvmla::kUnitRecordInts), (hipStream_t)stream);
  }
  const hipError_t e2 = hipStreamSynchronize((hipStream_t)stream);
  (void)hipFree(d_gu);
  PKVMLA_HIP(e);
  PKVMLA_HIP(e2);
  return ok();
}

}  // extern "C"
