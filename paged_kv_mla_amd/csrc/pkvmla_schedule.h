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

}  // namespace pkvmla

#endif  // PKVMLA_SCHEDULE_H_
