"""Independent re-derivation of the split-KV work schedule.

Test infrastructure only.  The pages describe no scheduler; the rule below is
this library's own design, restated here from its written specification so the
plan the C library builds (host function and uploaded device tables) can be
checked bit for bit.  It shares no code with the C implementation.

Rule (all integers):
  * Work items are (request b, sequence s, length L): a flat plan has one item
    per request with s = b; a cascade plan has, per request, the group prefix
    (s = group id, L = prefix length) then the request's own suffix
    (s = G + b, L = suffix length).  Items with L = 0 are skipped.
  * tiles(L) = ceil(L / TILE).  Every segment also costs FIXED tiles.
    C = sum over items of (tiles(L) + FIXED); W is the workgroup budget
    (compute units x workgroups per CU).
  * walk(cap): go through the items in order with a tile cursor t and a
    current workgroup w holding u cost units.  While t < tiles(L):
    room = cap - u - FIXED; if room <= 0, open the next workgroup (w += 1,
    u = 0) and retry; else take = min(tiles(L) - t, room), emit the unit
    (w, b, s, t*TILE, min((t + take) * TILE, L)), u += take + FIXED,
    t += take.
  * cap is the smallest integer >= max(ceil(C / W), FIXED + 1) for which
    walk(cap) uses at most W workgroups; the grid is the number it uses.
  * A request with exactly one unit writes out and lse directly (slot -1);
    otherwise each of its units gets the next partial slot in emission order
    and a merge row (b, first slot, count) is added in request order.
  * row = number of tokens in all earlier units (emission order): where the
    unit's tokens start in the gathered-rows view.
"""

from __future__ import annotations

import numpy as np

PLAN_TILE = 32          # KV tokens per tile
UNIT_INTS = 8           # int32 per unit record: b, seq, kv_begin, kv_end, slot, row,
                        # page_base, first_page (the last two: unit_page_fields)
MERGE_INTS = 4          # int32 per merge record: b, first_slot, count, 0

# Per head count: (compute waves per workgroup: QK and PV, heads per QK wave,
# LDS stages, workgroups per CU, fixed cost per segment in tiles, head
# groups).  These mirror the library's plan parameters; nothing below
# computes with them except the lane count.  The
# schedule has (CUs x workgroups per CU) / head groups lanes.  The library
# exports the values it uses; the tests compare them with this table.
_KERNEL_CONFIGS = {
    16: (5, 16, 4, 1, 2, 1),
    32: (6, 16, 4, 1, 2, 1),
    64: (8, 16, 4, 1, 4, 1),
    128: (8, 16, 4, 1, 4, 2),
}


def kernel_config(num_heads: int):
    waves, hpw, stages, wg_per_cu, fixed, hg = _KERNEL_CONFIGS[int(num_heads)]
    return dict(waves=waves, heads_per_wave=hpw, stages=stages,
                wg_per_cu=wg_per_cu, fixed_cost=fixed, head_groups=hg, tile=PLAN_TILE)


def flat_items(kv_lens):
    return [(b, b, int(L)) for b, L in enumerate(kv_lens)]


def qo_items(qo_indptr, kv_lens):
    """One item per query row of a plan with several new tokens per request:
    row qo_indptr[b] + j over request b's pages, causal length
    kv_lens[b] - n_b + 1 + j (its position plus one)."""
    items = []
    for b in range(len(kv_lens)):
        n = int(qo_indptr[b + 1]) - int(qo_indptr[b])
        for j in range(n):
            items.append((int(qo_indptr[b]) + j, b, int(kv_lens[b]) - n + 1 + j))
    return items


def cascade_items(group_req_indptr, prefix_lens, kv_lens):
    G = len(prefix_lens)
    items = []
    for g in range(G):
        for b in range(int(group_req_indptr[g]), int(group_req_indptr[g + 1])):
            items.append((b, g, int(prefix_lens[g])))
            items.append((b, G + b, int(kv_lens[b])))
    items.sort(key=lambda it: it[0])  # stable: prefix before suffix per request
    return items


def schedule_ref(items, batch: int, num_wg: int, tile: int = PLAN_TILE, fixed: int = 1):
    """Returns (wg_indptr int32 [grid+1], units int32 [n,8], merges int32 [m,4])."""
    if num_wg < 1:
        raise ValueError("num_wg must be >= 1")

    def tiles(L):
        return -(-L // tile)

    def walk(cap):
        raw = []  # (w, b, s, kv_begin, kv_end)
        w, u = 0, 0
        for (b, s, L) in items:
            if L <= 0:
                continue
            T = tiles(L)
            t = 0
            while t < T:
                room = cap - u - fixed
                if room <= 0:
                    w += 1
                    u = 0
                    continue
                take = min(T - t, room)
                raw.append((w, b, s, t * tile, min((t + take) * tile, L)))
                u += take + fixed
                t += take
        return raw, (w + 1) if raw else 0

    C = sum(tiles(L) + fixed for (_, _, L) in items if L > 0)
    cap = max(-(-C // num_wg), fixed + 1)
    raw, grid = walk(cap)
    while grid > num_wg:
        cap += 1
        raw, grid = walk(cap)

    per_req = np.zeros(batch, dtype=np.int64)
    for r in raw:
        per_req[r[1]] += 1
    units = np.zeros((len(raw), UNIT_INTS), dtype=np.int32)
    first_slot = {}
    slot = 0
    row = 0
    for i, (wi, b, s, k0, k1) in enumerate(raw):
        if per_req[b] == 1:
            sl = -1
        else:
            sl = slot
            first_slot.setdefault(b, slot)
            slot += 1
        units[i, :6] = (b, s, k0, k1, sl, row)
        row += k1 - k0
    merges = [(b, first_slot[b], int(per_req[b]), 0) for b in range(batch) if per_req[b] > 1]
    merges = np.asarray(merges, dtype=np.int32).reshape(-1, MERGE_INTS)
    wg_indptr = np.zeros(grid + 1, dtype=np.int32)
    for r in raw:
        wg_indptr[r[0] + 1] += 1
    wg_indptr = np.cumsum(wg_indptr).astype(np.int32)
    return wg_indptr, units, merges


def unit_page_fields(units, seq_indptr, seq_indices, page_size: int):
    """The two page fields of each unit record, from the sequences' page tables:
    page_base = seq_indptr[seq] (where the sequence's page list starts in
    seq_indices) and first_page = the page holding token kv_begin, i.e.
    seq_indices[page_base + kv_begin // page_size].  Returns a filled copy."""
    out = np.array(units, dtype=np.int32, copy=True)
    seq_indptr = np.asarray(seq_indptr, dtype=np.int64)
    seq_indices = np.asarray(seq_indices, dtype=np.int64)
    for i in range(out.shape[0]):
        seq, k0 = int(out[i, 1]), int(out[i, 2])
        base = int(seq_indptr[seq])
        out[i, 6] = base
        out[i, 7] = seq_indices[base + k0 // page_size]
    return out
