// Host-side split-KV scheduler (pure C++, no HIP).
#ifndef PKVMLA_SCHEDULE_H_
#define PKVMLA_SCHEDULE_H_

#include <stdint.h>

#include <vector>

namespace pkvmla {

// req, seq, kv_begin, kv_end, slot, row, page_base, first_page; the scheduler
// leaves the last two 0, the plan fills them from the page tables
constexpr int kUnitRecordInts = 8;
constexpr int kMergeRecordInts = 4;  // req, first_slot, count, 0
// slot field of a unit whose state carries into the next unit (the kernels'
// kChainNext)
constexpr int32_t kChainNextSlot = INT32_MIN;

struct WorkItem {
  int32_t req;  // request whose query heads attend
  int32_t seq;  // page list (sequence) attended
  int32_t len;  // tokens of that sequence
};

struct Schedule {
  int32_t grid = 0;
  int32_t n_slots = 0;
  int64_t total_rows = 0;
  std::vector<int32_t> wg_indptr;  // grid + 1
  std::vector<int32_t> units;      // n_units * 8
  std::vector<int32_t> merges;     // n_merges * 4
};

bool build_schedule(const std::vector<WorkItem>& items, int32_t batch, int32_t num_wg,
                    int32_t tile, int32_t fixed, Schedule* s);

// Level 0 of a cascade plan: the shared prefix of each group scored by row
// blocks of its query rows (rho = b * H + head).  Unit records:
// row0, group, kv_begin, kv_end, slot offset (first slot * H - row0), row_end,
// then the two page fields the plan fills.  Slots 0 .. n_slots - 1, each
// unit taking one per request of its rows, in emission order.
struct RowSchedule {
  int32_t grid = 0;
  int32_t n_slots = 0;
  std::vector<int32_t> wg_indptr;  // grid + 1
  std::vector<int32_t> units;      // n_units * 8
};

// Rows per block at a head count (64, or a whole request above 64 heads).
inline int32_t row_block_rows(int32_t num_heads) { return num_heads > 64 ? num_heads : 64; }

bool build_row_schedule(const int32_t* group_req_indptr, int32_t num_groups,
                        const int32_t* prefix_lens, int32_t num_heads, int32_t num_wg,
                        int32_t tile, RowSchedule* s);

// A cascade in one launch (num_heads >= 64, every group's prefix non-empty):
// each request's rows are one block, cut over the lanes as in
// build_row_schedule, and the request's suffix (if any) follows the block's
// last piece on that lane, chained to it (kChainNext in the piece's slot
// field: the state carries into the suffix unit).  Unit records are flat
// ones: request, sequence (group g for a prefix piece, G + b for a suffix),
// kv_begin, kv_end, slot, 0, then the two page fields the plan fills.  A
// request with one state (one piece) writes out directly (slot -1); one with
// several pieces gets a partial slot per state (slots numbered in emission
// order) and a merge record (b, first list entry, count, 1) over its slots.
bool build_chain_schedule(const int32_t* group_req_indptr, int32_t num_groups,
                          const int32_t* prefix_lens, const int32_t* kv_lens, int32_t batch,
                          int32_t num_wg, int32_t tile, RowSchedule* s,
                          std::vector<int32_t>* merges, std::vector<int32_t>* slot_list);

// Merge records (b, first list entry, count, 1) and the slot list of a
// cascade plan: per request its level-0 slots (level-0 emission order) then
// its level-1 slots (the `l1` units' slot fields, emission order).
void build_cascade_merges(const RowSchedule& l0, const std::vector<int32_t>& l1_units,
                          int32_t batch, int32_t num_heads, std::vector<int32_t>* merges,
                          std::vector<int32_t>* slot_list);

// Several new query tokens per request as row blocks (16 or 32 heads): request
// b's query rows t * H + h (its tokens t = qo_indptr[b] .. qo_indptr[b+1] - 1)
// in blocks of 64, each block over the positions its last token sees, with
// the causal bound per row.  The layout is used when some request brings more
// than one token (qo_indptr[batch] > batch); otherwise the plan has one work
// item per query token.
constexpr int32_t kQoBlockRows = 64;
// slot field of a row-block unit that writes out and lse directly (the
// kernels' kRowsDirect)
constexpr int32_t kRowsDirectSlot = INT32_MIN + 1;
bool qo_uses_row_blocks(const int32_t* qo_indptr, int32_t batch, int32_t num_heads);

// The row-block schedule: the blocks are the items of build_schedule's walk
// (`fixed`: the 64-row kernel's cost per segment; length t_last + c_b, t_last
// the block's last token), whose units become records
// row0, c_b, kv_begin, kv_end, slot field, row_end, 0, 0 with
// c_b = kv_lens[b] - n_b + 1 - qo_indptr[b] (token t sees the positions below
// t + c_b) and slot field kRowsDirectSlot (a whole block) or
// walk slot * 64 - row0 (partial row = field + row, slots of H rows).  A split
// block gives one merge record (t, first list entry, count, 1) per token t,
// its list the token's slot in each piece.  unit_seq: the request (sequence)
// of each unit, for the page fields.  n_slots counts slots of H rows.
bool build_qo_row_schedule(const int32_t* qo_indptr, const int32_t* kv_lens, int32_t batch,
                           int32_t num_heads, int32_t num_wg, int32_t tile, int32_t fixed,
                           RowSchedule* s, std::vector<int32_t>* unit_seq,
                           std::vector<int32_t>* merges, std::vector<int32_t>* slot_list);

}  // namespace pkvmla

#endif  // PKVMLA_SCHEDULE_H_
