// Randomized invariant checks of the host schedulers (pkvmla_schedule.cpp),
// built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py.  Pure C++: no GPU, no HIP.
//
// For every random case:
//   build_schedule        every token of every item is covered exactly once,
//                         units per lane are contiguous, slots are unique and
//                         merges list each split request's slots;
//   build_row_schedule    every (group row, prefix token) pair is covered
//                         exactly once, slots are unique and in range;
//   build_chain_schedule  every request's prefix and suffix tokens are covered
//                         once, a chained unit is followed by its request's
//                         suffix, and every state is output or merged once;
//   build_cascade_merges  each request lists exactly its own slots.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <random>
#include <vector>

#include "pkvmla_schedule.h"

using namespace pkvmla;

static int g_fail = 0;
#define CHECK(c)                                                            \
  do {                                                                      \
    if (!(c)) {                                                             \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c);       \
      ++g_fail;                                                             \
      return;                                                               \
    }                                                                       \
  } while (0)

static void flat_case(std::mt19937& rng) {
  const int B = 1 + rng() % 40, W = 1 + rng() % 300, tile = 1 << (4 + rng() % 3);
  const int fixed = rng() % 4;
  std::vector<WorkItem> items;
  for (int b = 0; b < B; ++b) items.push_back(WorkItem{b, b, (int32_t)(rng() % 5000)});
  Schedule s;
  CHECK(build_schedule(items, B, W, tile, fixed, &s));
  CHECK(s.grid <= W && (int)s.wg_indptr.size() == s.grid + 1);
  std::vector<std::vector<char>> cov(B);
  for (int b = 0; b < B; ++b) cov[b].assign(items[b].len, 0);
  std::vector<int> slot_seen(s.n_slots, 0);
  for (size_t i = 0; i < s.units.size(); i += kUnitRecordInts) {
    const int32_t* u = &s.units[i];
    CHECK(u[0] >= 0 && u[0] < B && u[2] >= 0 && u[2] < u[3] && u[3] <= items[u[0]].len);
    for (int t = u[2]; t < u[3]; ++t) {
      CHECK(!cov[u[0]][t]);
      cov[u[0]][t] = 1;
    }
    if (u[4] >= 0) {
      CHECK(u[4] < s.n_slots && !slot_seen[u[4]]);
      slot_seen[u[4]] = 1;
    }
  }
  for (int b = 0; b < B; ++b)
    for (char c : cov[b]) CHECK(c);
  for (size_t i = 0; i < s.merges.size(); i += kMergeRecordInts) {
    const int32_t* m = &s.merges[i];
    CHECK(m[2] >= 2 && m[1] >= 0 && m[1] + m[2] <= s.n_slots);
  }
}

static void cascade_case(std::mt19937& rng) {
  const int G = 1 + rng() % 5, W = 1 + rng() % 300, tile = 32;
  const int H = 16 << (rng() % 4);
  std::vector<int32_t> gi(1, 0), pl;
  for (int g = 0; g < G; ++g) {
    gi.push_back(gi.back() + (int32_t)(rng() % 7));
    pl.push_back((int32_t)(rng() % 3000));
  }
  const int B = gi.back();
  if (B == 0) return;
  std::vector<int32_t> kl(B);
  for (int b = 0; b < B; ++b) kl[b] = (int32_t)(rng() % 700);
  // two-level: rows
  RowSchedule r;
  CHECK(build_row_schedule(gi.data(), G, pl.data(), H, W, tile, &r));
  std::vector<std::vector<int>> cov(B);
  for (int b = 0; b < B; ++b) {
    int g = 0;
    while (gi[g + 1] <= b) ++g;
    cov[b].assign(pl[g], 0);
  }
  std::vector<int> slot_seen(r.n_slots, 0);
  for (size_t i = 0; i < r.units.size(); i += kUnitRecordInts) {
    const int32_t* u = &r.units[i];
    CHECK(u[0] % H == 0 && u[5] % H == 0 && u[0] < u[5]);
    for (int b = u[0] / H; b < u[5] / H; ++b) {
      CHECK(b < B);
      for (int t = u[2]; t < u[3]; ++t) {
        CHECK(t < (int)cov[b].size() && !cov[b][t]);
        cov[b][t] = 1;
      }
      const int slot = (u[4] + u[0]) / H + b - u[0] / H;
      CHECK(slot >= 0 && slot < r.n_slots && !slot_seen[slot]);
      slot_seen[slot] = 1;
    }
  }
  for (int b = 0; b < B; ++b)
    for (int c : cov[b]) CHECK(c);
  std::vector<int32_t> l1;  // one suffix unit per request, slots after level 0's
  for (int b = 0; b < B; ++b)
    if (kl[b] > 0) l1.insert(l1.end(), {b, G + b, 0, kl[b], r.n_slots + (int32_t)(l1.size() / 8), 0, 0, 0});
  std::vector<int32_t> merges, list;
  build_cascade_merges(r, l1, B, H, &merges, &list);
  CHECK((int)merges.size() == 4 * B);
  std::vector<int> listed(r.n_slots + l1.size() / 8, 0);
  for (int b = 0; b < B; ++b) {
    const int32_t* m = &merges[4 * b];
    CHECK(m[0] == b && m[3] == 1 && m[1] + m[2] <= (int)list.size());
    for (int k = 0; k < m[2]; ++k) {
      const int sl = list[m[1] + k];
      CHECK(sl >= 0 && sl < (int)listed.size() && !listed[sl]);
      listed[sl] = 1;
    }
  }
  for (int x : listed) CHECK(x);
  // one launch (every prefix non-empty)
  for (auto& p : pl) p = p > 0 ? p : 1 + (int32_t)(rng() % 100);
  RowSchedule c;
  std::vector<int32_t> cm, cl;
  CHECK(build_chain_schedule(gi.data(), G, pl.data(), kl.data(), B, W, tile, &c, &cm, &cl));
  // the plan's table bounds: a unit per prefix piece (at most max(W, B)) and
  // per suffix (B); as many slots at most
  const int64_t cap = std::max<int64_t>(W, B) + B;
  CHECK((int64_t)(c.units.size() / kUnitRecordInts) <= cap && c.n_slots <= cap &&
        (int64_t)cl.size() <= cap);
  std::vector<int> pre(B, 0), outs(B, 0);
  std::vector<std::vector<char>> sufcov(B);
  for (int b = 0; b < B; ++b) sufcov[b].assign((size_t)std::max(kl[b], 0), 0);
  std::vector<int> seen(c.n_slots, 0);
  for (size_t i = 0; i < c.units.size(); i += kUnitRecordInts) {
    const int32_t* u = &c.units[i];
    const int b = u[0];
    CHECK(b >= 0 && b < B);
    if (u[1] < G) {
      pre[b] += u[3] - u[2];
      if (u[4] == kChainNextSlot) {
        CHECK(i + kUnitRecordInts < c.units.size());
        const int32_t* n = u + kUnitRecordInts;
        CHECK(n[0] == b && n[1] == G + b && n[2] == 0 && n[3] > 0 && n[3] <= kl[b]);
      }
    } else {
      // a request's suffix, each token once
      CHECK(u[1] == G + b && u[2] % tile == 0 && u[2] < u[3] && u[3] <= kl[b]);
      for (int t = u[2]; t < u[3]; ++t) {
        CHECK(!sufcov[b][t]);
        sufcov[b][t] = 1;
      }
    }
    if (u[4] == -1) ++outs[b];
    if (u[4] >= 0) {
      CHECK(u[4] < c.n_slots && !seen[u[4]]);
      seen[u[4]] = 1;
    }
  }
  for (int b = 0; b < B; ++b) {
    int g = 0;
    while (gi[g + 1] <= b) ++g;
    CHECK(pre[b] == pl[g]);
    for (char x : sufcov[b]) CHECK(x);
  }
  std::vector<int> merged(B, 0);
  for (size_t i = 0; i < cm.size(); i += 4) merged[cm[i]] = 1;
  for (int b = 0; b < B; ++b) CHECK((outs[b] == 1) != (merged[b] == 1));
}

int main(int argc, char** argv) {
  const int n = argc > 1 ? atoi(argv[1]) : 2000;
  std::mt19937 rng(20251);
  for (int i = 0; i < n; ++i) {
    flat_case(rng);
    cascade_case(rng);
  }
  printf("%d cases, %d failures\n", n, g_fail);
  return g_fail ? 1 : 0;
}
