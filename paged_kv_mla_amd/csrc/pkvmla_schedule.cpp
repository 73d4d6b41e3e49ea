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
#include <array>
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

// Level-0 schedule.  Blocks: for each group with a non-empty prefix, its rows
// [first request * H, end request * H) cut into blocks of row_block_rows(H).
// With nb blocks on W lanes:
//   nb <= W: every block is cut into S = floor(W / nb) token pieces (never
//     more pieces than the prefix has tiles), piece s of block k on lane
//     k * S + s.  Lanes are placed round-robin on the eight XCDs (lane l on
//     XCD l mod 8): with S = 1 every lane walks its prefix from the first
//     tile at the same time, so the workgroups of one XCD read each tile from
//     its L2 after the first; with S a multiple of 8 each XCD streams only
//     its own pieces of every prefix.
//   nb > W: block k goes whole to lane k mod W.
// Piece s of a prefix of T tiles covers tiles [s*T/P, (s+1)*T/P) (P pieces).
bool build_row_schedule(const int32_t* group_req_indptr, int32_t num_groups,
                        const int32_t* prefix_lens, int32_t num_heads, int32_t num_wg,
                        int32_t tile, RowSchedule* s) {
  if (num_wg < 1 || tile < 1 || num_heads < 1 || num_groups < 0) return false;
  struct Block {
    int32_t g, row0, row_end, len;
  };
  std::vector<Block> blocks;
  const int32_t rb = row_block_rows(num_heads);
  for (int32_t g = 0; g < num_groups; ++g) {
    if (prefix_lens[g] <= 0) continue;
    const int64_t r0 = (int64_t)group_req_indptr[g] * num_heads;
    const int64_t r1 = (int64_t)group_req_indptr[g + 1] * num_heads;
    for (int64_t r = r0; r < r1; r += rb)
      blocks.push_back(Block{g, (int32_t)r, (int32_t)std::min<int64_t>(r + rb, r1), prefix_lens[g]});
  }
  const int64_t nb = (int64_t)blocks.size();
  std::vector<std::vector<std::array<int32_t, 4>>> lane_units;  // block, kv_begin, kv_end
  if (nb == 0) {
    s->grid = 0;
  } else if (nb <= num_wg) {
    const int64_t S = num_wg / nb;
    s->grid = (int32_t)(nb * S);
    lane_units.assign((size_t)s->grid, {});
    for (int64_t k = 0; k < nb; ++k) {
      const int64_t T = ceil_div(blocks[k].len, tile);
      const int64_t P = std::min<int64_t>(S, T);
      for (int64_t p = 0; p < P; ++p) {
        const int64_t t0 = p * T / P, t1 = (p + 1) * T / P;
        lane_units[(size_t)(k * S + p)].push_back(
            {(int32_t)k, (int32_t)(t0 * tile), (int32_t)std::min<int64_t>(t1 * tile, blocks[k].len), 0});
      }
    }
  } else {
    s->grid = num_wg;
    lane_units.assign((size_t)num_wg, {});
    for (int64_t k = 0; k < nb; ++k)
      lane_units[(size_t)(k % num_wg)].push_back({(int32_t)k, 0, blocks[k].len, 0});
  }
  s->wg_indptr.assign((size_t)s->grid + 1, 0);
  s->units.clear();
  int64_t slot = 0;
  for (int32_t l = 0; l < s->grid; ++l) {
    for (const auto& u : lane_units[(size_t)l]) {
      const Block& b = blocks[(size_t)u[0]];
      const int64_t off = slot * num_heads - b.row0;
      if (off < INT32_MIN || off > INT32_MAX) return false;
      s->units.insert(s->units.end(), {b.row0, b.g, u[1], u[2], (int32_t)off, b.row_end, 0, 0});
      slot += (b.row_end - b.row0) / num_heads;
    }
    s->wg_indptr[(size_t)l + 1] = (int32_t)(s->units.size() / kUnitRecordInts);
  }
  if (slot > INT32_MAX) return false;
  s->n_slots = (int32_t)slot;
  return true;
}

bool build_chain_schedule(const int32_t* group_req_indptr, int32_t num_groups,
                          const int32_t* prefix_lens, const int32_t* kv_lens, int32_t batch,
                          int32_t num_wg, int32_t tile, RowSchedule* s,
                          std::vector<int32_t>* merges, std::vector<int32_t>* slot_list) {
  if (num_wg < 1 || tile < 1 || batch < 1 || num_groups < 1) return false;
  std::vector<int32_t> group(batch, -1);
  for (int32_t g = 0; g < num_groups; ++g) {
    if (prefix_lens[g] <= 0) return false;  // every request needs a prefix block
    for (int32_t b = group_req_indptr[g]; b < group_req_indptr[g + 1]; ++b) group[b] = g;
  }
  // per lane: (request, kv_begin, kv_end, is_last_piece)
  std::vector<std::vector<std::array<int32_t, 4>>> lanes;
  std::vector<int32_t> pieces(batch, 0);
  if (batch <= num_wg) {
    const int64_t S = num_wg / batch;
    s->grid = (int32_t)(batch * S);
    lanes.assign((size_t)s->grid, {});
    for (int32_t b = 0; b < batch; ++b) {
      const int64_t L = prefix_lens[group[b]];
      const int64_t T = ceil_div(L, tile);
      const int64_t P = std::min<int64_t>(S, T);
      pieces[b] = (int32_t)P;
      for (int64_t p = 0; p < P; ++p) {
        const int64_t t0 = p * T / P, t1 = (p + 1) * T / P;
        lanes[(size_t)(b * S + p)].push_back(
            {b, (int32_t)(t0 * tile), (int32_t)std::min<int64_t>(t1 * tile, L), p == P - 1});
      }
    }
  } else {
    s->grid = num_wg;
    lanes.assign((size_t)num_wg, {});
    for (int32_t b = 0; b < batch; ++b) {
      pieces[b] = 1;
      lanes[(size_t)(b % num_wg)].push_back({b, 0, prefix_lens[group[b]], 1});
    }
  }
  std::vector<std::vector<int32_t>> per(batch);
  s->wg_indptr.assign((size_t)s->grid + 1, 0);
  s->units.clear();
  int32_t slot = 0;
  for (int32_t l = 0; l < s->grid; ++l) {
    for (const auto& u : lanes[(size_t)l]) {
      const int32_t b = u[0];
      const bool chain = u[3] && kv_lens[b] > 0;
      int32_t sl = -1;
      if (chain) {
        sl = kChainNextSlot;
      } else if (pieces[b] > 1) {
        per[b].push_back(slot);
        sl = slot++;
      }
      s->units.insert(s->units.end(), {b, group[b], u[1], u[2], sl, 0, 0, 0});
      if (chain) {
        int32_t sl2 = -1;
        if (pieces[b] > 1) {
          per[b].push_back(slot);
          sl2 = slot++;
        }
        s->units.insert(s->units.end(), {b, num_groups + b, 0, kv_lens[b], sl2, 0, 0, 0});
      }
    }
    s->wg_indptr[(size_t)l + 1] = (int32_t)(s->units.size() / kUnitRecordInts);
  }
  s->n_slots = slot;
  merges->clear();
  slot_list->clear();
  for (int32_t b = 0; b < batch; ++b) {
    if (per[b].empty()) continue;
    merges->insert(merges->end(), {b, (int32_t)slot_list->size(), (int32_t)per[b].size(), 1});
    slot_list->insert(slot_list->end(), per[b].begin(), per[b].end());
  }
  return true;
}

void build_cascade_merges(const RowSchedule& l0, const std::vector<int32_t>& l1_units,
                          int32_t batch, int32_t num_heads, std::vector<int32_t>* merges,
                          std::vector<int32_t>* slot_list) {
  std::vector<std::vector<int32_t>> per(batch);
  for (size_t i = 0; i < l0.units.size(); i += kUnitRecordInts) {
    const int32_t* u = &l0.units[i];
    const int32_t first = (u[4] + u[0]) / num_heads;  // slot of the block's first request
    for (int32_t b = u[0] / num_heads; b < u[5] / num_heads; ++b)
      per[b].push_back(first + (b - u[0] / num_heads));
  }
  for (size_t i = 0; i < l1_units.size(); i += kUnitRecordInts)
    per[l1_units[i]].push_back(l1_units[i + 4]);
  merges->clear();
  slot_list->clear();
  for (int32_t b = 0; b < batch; ++b) {
    merges->insert(merges->end(), {b, (int32_t)slot_list->size(), (int32_t)per[b].size(), 1});
    slot_list->insert(slot_list->end(), per[b].begin(), per[b].end());
  }
}

}  // namespace pkvmla

namespace pkvmla {

// A 64-row workgroup costs about what a 16- or 32-head one costs per tile, so
// row blocks pay as soon as one request brings two tokens (its tiles then
// serve both), and only a batch of single tokens keeps one item per token.
bool qo_uses_row_blocks(const int32_t* qo_indptr, int32_t batch, int32_t num_heads) {
  return (num_heads == 16 || num_heads == 32) && qo_indptr[batch] > batch;
}

// Row blocks of several new tokens per request.  The blocks are the work items
// of the flat walk (item k over its request's sequence, up to the positions its
// last token sees: no tile past them has a visible position for any row); its
// units and merges are then rewritten for rows: slot field kRowsDirectSlot for
// a whole block, else walk slot * 64 - row0 (so walk slot s holds the 64 / H
// partial slots of H rows from s * 64 / H on, one per token of the block); a
// split block's merge becomes one merge per token over a list of its slots.
bool build_qo_row_schedule(const int32_t* qo_indptr, const int32_t* kv_lens, int32_t batch,
                           int32_t num_heads, int32_t num_wg, int32_t tile, int32_t fixed,
                           RowSchedule* s, std::vector<int32_t>* unit_seq,
                           std::vector<int32_t>* merges, std::vector<int32_t>* slot_list) {
  if ((num_heads != 16 && num_heads != 32) || batch < 1) return false;
  struct Block {
    int32_t b, row0, row_end;
  };
  std::vector<Block> blocks;
  std::vector<WorkItem> items;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t lo = (int64_t)qo_indptr[b] * num_heads;
    const int64_t hi = (int64_t)qo_indptr[b + 1] * num_heads;
    if (hi > INT32_MAX) return false;
    const int32_t c = kv_lens[b] - (qo_indptr[b + 1] - qo_indptr[b]) + 1 - qo_indptr[b];
    for (int64_t r = lo; r < hi; r += kQoBlockRows) {
      const int32_t r1 = (int32_t)std::min<int64_t>(r + kQoBlockRows, hi);
      // the block's work ends where its last token's causal range ends
      items.push_back(WorkItem{(int32_t)blocks.size(), b, r1 / num_heads - 1 + c});
      blocks.push_back(Block{b, (int32_t)r, r1});
    }
  }
  Schedule flat;
  if (!build_schedule(items, (int32_t)blocks.size(), num_wg, tile, fixed, &flat)) return false;
  const int32_t per = kQoBlockRows / num_heads;
  if ((int64_t)flat.n_slots * per > INT32_MAX / 2) return false;
  s->grid = flat.grid;
  s->wg_indptr = flat.wg_indptr;
  s->units = flat.units;
  s->n_slots = flat.n_slots * per;
  unit_seq->clear();
  for (size_t i = 0; i < s->units.size(); i += kUnitRecordInts) {
    int32_t* u = &s->units[i];
    const Block& k = blocks[(size_t)u[0]];
    const int32_t n = qo_indptr[k.b + 1] - qo_indptr[k.b];
    unit_seq->push_back(k.b);
    const int32_t slot = u[4];
    u[0] = k.row0;
    u[1] = kv_lens[k.b] - n + 1 - qo_indptr[k.b];  // token t sees positions < t + u[1]
    u[4] = slot < 0 ? kRowsDirectSlot : slot * kQoBlockRows - k.row0;
    u[5] = k.row_end;
    u[6] = 0;
    u[7] = 0;
  }
  merges->clear();
  slot_list->clear();
  for (size_t i = 0; i < flat.merges.size(); i += kMergeRecordInts) {
    const Block& k = blocks[(size_t)flat.merges[i]];
    const int32_t first = flat.merges[i + 1], count = flat.merges[i + 2];
    for (int32_t j = 0; j < (k.row_end - k.row0) / num_heads; ++j) {
      merges->insert(merges->end(),
                     {k.row0 / num_heads + j, (int32_t)slot_list->size(), count, 1});
      for (int32_t p = 0; p < count; ++p) slot_list->push_back((first + p) * per + j);
    }
  }
  return true;
}

}  // namespace pkvmla
