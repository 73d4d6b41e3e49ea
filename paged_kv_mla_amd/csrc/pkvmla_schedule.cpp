// Split-KV work schedule (host only, no GPU).
//
// Balances the attention work of a decode batch over a fixed workgroup budget
// W.  Work items are (request, sequence, length); each is cut into segments
// ("units") on KV-tile boundaries.  A unit costs its tile count plus a fixed
// per-segment cost (query load and epilogue).  The greedy walk fills workgroup
// after workgroup up to a cost cap; the cap is the smallest value at or above
// the even share ceil(C / W) for which the walk needs at most W workgroups,
// so the split overhead never piles up on the last workgroup.  Requests cut
// into more than one unit write partial states (bf16 outputs normalized by
// their own row sums, fp32 lse) into consecutive slots and get one merge row.
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "pkvmla_schedule.h"

namespace pkvmla {

namespace {

struct RawUnit {
  int32_t wg, req, seq, kv_begin, kv_end;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// One greedy pass at a given cap; returns the number of workgroups used.
int64_t walk(const std::vector<WorkItem>& items, int32_t tile, int32_t fixed, int64_t cap,
             std::vector<RawUnit>* out) {
  out->clear();
  int64_t w = 0, used = 0;
  for (const WorkItem& it : items) {
    if (it.len <= 0) continue;
    const int64_t tiles = ceil_div(it.len, tile);
    int64_t t = 0;
    while (t < tiles) {
      const int64_t room = cap - used - fixed;
      if (room <= 0) {
        ++w;
        used = 0;
        continue;
      }
      const int64_t take = std::min(tiles - t, room);
      const int64_t end = std::min<int64_t>((t + take) * tile, it.len);
      out->push_back(RawUnit{(int32_t)w, it.req, it.seq, (int32_t)(t * tile), (int32_t)end});
      used += take + fixed;
      t += take;
    }
  }
  return out->empty() ? 0 : w + 1;
}

}  // namespace

bool build_schedule(const std::vector<WorkItem>& items, int32_t batch, int32_t num_wg,
                    int32_t tile, int32_t fixed, Schedule* s) {
  if (num_wg < 1 || tile < 1 || fixed < 0 || batch < 0) return false;
  int64_t total = 0;
  for (const WorkItem& it : items)
    if (it.len > 0) total += ceil_div(it.len, tile) + fixed;
  int64_t cap = std::max<int64_t>(ceil_div(total, num_wg), (int64_t)fixed + 1);
  std::vector<RawUnit> raw;
  int64_t grid = walk(items, tile, fixed, cap, &raw);
  while (grid > num_wg) {
    ++cap;
    grid = walk(items, tile, fixed, cap, &raw);
  }

  std::vector<int32_t> count(batch, 0);
  for (const RawUnit& r : raw) {
    if (r.req < 0 || r.req >= batch) return false;
    ++count[r.req];
  }
  s->grid = (int32_t)grid;
  s->units.assign(raw.size() * kUnitRecordInts, 0);
  s->merges.clear();
  s->wg_indptr.assign(grid + 1, 0);
  std::vector<int32_t> first(batch, -1);
  int32_t slot = 0;
  int64_t row = 0;
  for (size_t i = 0; i < raw.size(); ++i) {
    const RawUnit& r = raw[i];
    int32_t sl = -1;
    if (count[r.req] > 1) {
      if (first[r.req] < 0) first[r.req] = slot;
      sl = slot++;
    }
    int32_t* u = &s->units[i * kUnitRecordInts];
    u[0] = r.req;
    u[1] = r.seq;
    u[2] = r.kv_begin;
    u[3] = r.kv_end;
    u[4] = sl;
    u[5] = (int32_t)row;
    row += r.kv_end - r.kv_begin;
    s->wg_indptr[r.wg + 1] += 1;
  }
  for (int32_t b = 0; b < batch; ++b) {
    if (count[b] > 1) {
      s->merges.push_back(b);
      s->merges.push_back(first[b]);
      s->merges.push_back(count[b]);
      s->merges.push_back(0);
    }
  }
  for (int64_t w = 0; w < grid; ++w) s->wg_indptr[w + 1] += s->wg_indptr[w];
  s->n_slots = slot;
  s->total_rows = row;
  return true;
}

}  // namespace pkvmla
