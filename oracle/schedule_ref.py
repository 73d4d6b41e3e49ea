"""Independent re-derivation of the split-KV work schedule.

Test infrastructure only.  The pages describe no scheduler; the rule below is
this library's own design, restated here from its written specification so the
plan the C library builds (host function and uploaded device tables) can be
checked bit for bit.  It shares no code with the C implementation.

Rule (all integers):
  * Work items are (request b, sequence s, length L): a flat plan has one item
    per request with s = b; a cascade plan's level 1 has one per request for
    its own suffix (s = G + b, L = suffix length; sequences 0..G-1 are the
    groups' prefixes).  Items with L = 0 are skipped.
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


QO_BLOCK_ROWS = 64            # query rows per row block of a qo plan
QO_ROWS_DIRECT = -(2 ** 31) + 1   # slot field of a row block that writes out and lse itself
QO_ROWS_FIXED = 4             # fixed cost per segment of the 64-row kernel (its config)


def qo_uses_rows(qo_indptr, num_heads: int) -> bool:
    """Layout rule of a plan with several new tokens per request: row blocks
    (qo_rows_ref) when H is 16 or 32 and some request brings more than one
    query token (qo_indptr[B] > B); otherwise one work item per query token
    (qo_items)."""
    B = len(qo_indptr) - 1
    return int(num_heads) in (16, 32) and int(qo_indptr[B]) > B


def qo_rows_ref(qo_indptr, kv_lens, num_heads: int, num_wg: int, tile: int = PLAN_TILE,
                fixed: int = QO_ROWS_FIXED, pages=None):
    """Row-block schedule of a plan with several new tokens per request
    (H = 16 or 32), restated from its rule:

    * request b's rows [qo_indptr[b] * H, qo_indptr[b+1] * H) are cut into
      blocks of 64 (the last may be short), in request order; block k of
      request b is a work item (k, b, t_last + c_b) of the flat walk
      (schedule_ref, batch = number of blocks, the 64-row kernel's fixed cost),
      t_last being the block's last token: the positions its last token sees,
      the most any of its rows sees (the causal bound itself is per row);
    * each walk unit (k, b, kv_begin, kv_end, slot) becomes the record
      (row0, c_b, kv_begin, kv_end, slot field, row_end, page fields) with
      c_b = kv_lens[b] - n_b + 1 - qo_indptr[b], so that token t
      (rows t * H ..) sees the positions below t + c_b; slot field
      QO_ROWS_DIRECT for a block the walk left whole, else
      walk slot * 64 - row0 (partial row = walk slot * 64 + rho - row0, so
      walk slot s holds partial slots s * 64/H .. of H rows each);
    * each walk merge (k, first, count) gives, for every token t of block k
      in order, the merge record (t, list position, count, 1) and the list
      entries (first + i) * 64/H + (t - row0 / H), i = 0 .. count - 1;
    * page fields (optional `pages` = (kv_indptr, kv_indices, page_size)):
      those of unit_page_fields for sequence b.

    Returns (wg_indptr, units [n, 8], merges [m, 4], slot_list, n_slots) with
    n_slots in slots of H rows."""
    H = int(num_heads)
    assert H in (16, 32)
    per = QO_BLOCK_ROWS // H
    blocks = []   # (b, row0, row_end)
    for b in range(len(kv_lens)):
        lo, hi = int(qo_indptr[b]) * H, int(qo_indptr[b + 1]) * H
        for r in range(lo, hi, QO_BLOCK_ROWS):
            blocks.append((b, r, min(r + QO_BLOCK_ROWS, hi)))
    def reach(b, r1):     # positions seen by the block's last token (rows .. r1 - 1)
        n = int(qo_indptr[b + 1]) - int(qo_indptr[b])
        return (r1 // H - 1) + int(kv_lens[b]) - n + 1 - int(qo_indptr[b])
    items = [(k, b, reach(b, r1)) for k, (b, _, r1) in enumerate(blocks)]
    wg, fu, fm = schedule_ref(items, len(blocks), num_wg, tile, fixed)
    units = np.zeros_like(fu)
    walk_slots = 0
    for i in range(fu.shape[0]):
        k, b, k0, k1, sl = (int(x) for x in fu[i, :5])
        _, r0, r1 = blocks[k]
        n = int(qo_indptr[b + 1]) - int(qo_indptr[b])
        c = int(kv_lens[b]) - n + 1 - int(qo_indptr[b])
        if sl < 0:
            field = QO_ROWS_DIRECT
        else:
            field = sl * QO_BLOCK_ROWS - r0
            walk_slots = max(walk_slots, sl + 1)
        units[i, :6] = (r0, c, k0, k1, field, r1)
    merges, slot_list = [], []
    for (k, first, count, _) in fm:
        _, r0, r1 = blocks[int(k)]
        for j in range((r1 - r0) // H):
            merges.append((r0 // H + j, len(slot_list), int(count), 1))
            slot_list.extend((int(first) + i) * per + j for i in range(int(count)))
    if pages is not None:
        kv_indptr, kv_indices, page_size = pages
        withseq = units.copy()
        withseq[:, 1] = [blocks[int(fu[i, 0])][0] for i in range(fu.shape[0])]
        filled = unit_page_fields(withseq, kv_indptr, kv_indices, page_size)
        units[:, 6:] = filled[:, 6:]
    return (wg, units, np.asarray(merges, np.int32).reshape(-1, MERGE_INTS),
            np.asarray(slot_list, np.int32), walk_slots * per)


def suffix_items(num_groups: int, kv_lens):
    """Level-1 items of a cascade plan: request b over its suffix (sequence
    G + b)."""
    return [(b, num_groups + b, int(L)) for b, L in enumerate(kv_lens)]


def row_schedule_ref(group_req_indptr, prefix_lens, num_heads: int, num_wg: int,
                     tile: int = PLAN_TILE):
    """Level 0 of a cascade plan (its shared prefixes), restated from the rule:

    * query rows rho = b * H + h; group g owns rows [gi[g] * H, gi[g+1] * H);
      each group with a non-empty prefix has blocks of R = max(64, H) rows
      starting at its first row (the last one may be short), in group order;
    * nb blocks, W lanes.  nb <= W: S = W // nb pieces per block, P = min(S,
      tiles) of them for a prefix of `tiles` tiles, piece p covering tiles
      p*tiles//P .. (p+1)*tiles//P - 1 (tokens clipped to the prefix length),
      on lane k*S + p for block k; grid = nb * S.  nb > W: block k whole on
      lane k % W; grid = W;
    * units in lane order (a lane's in block order): (row0, g, kv_begin,
      kv_end, offset, row_end, 0, 0), slots counted from 0 in that order, a
      unit taking (row_end - row0) / H of them, offset = first slot * H - row0.

    Returns (wg_indptr [grid+1], units [n, 8], n_slots)."""
    H = int(num_heads)
    R = max(64, H)
    blocks = []
    for g in range(len(prefix_lens)):
        L = int(prefix_lens[g])
        if L <= 0:
            continue
        lo, hi = int(group_req_indptr[g]) * H, int(group_req_indptr[g + 1]) * H
        r = lo
        while r < hi:
            blocks.append((g, r, min(r + R, hi), L))
            r += R
    nb = len(blocks)
    if nb == 0:
        return np.zeros(1, np.int32), np.zeros((0, UNIT_INTS), np.int32), 0
    if nb <= num_wg:
        S = num_wg // nb
        grid = nb * S
        lanes = [[] for _ in range(grid)]
        for k, (g, r0, r1, L) in enumerate(blocks):
            T = -(-L // tile)
            P = min(S, T)
            for p in range(P):
                t0, t1 = p * T // P, (p + 1) * T // P
                lanes[k * S + p].append((k, t0 * tile, min(t1 * tile, L)))
    else:
        grid = num_wg
        lanes = [[] for _ in range(grid)]
        for k, (g, r0, r1, L) in enumerate(blocks):
            lanes[k % num_wg].append((k, 0, L))
    units, wg = [], [0]
    slot = 0
    for lane in lanes:
        for (k, k0, k1) in lane:
            g, r0, r1, _ = blocks[k]
            units.append((r0, g, k0, k1, slot * H - r0, r1, 0, 0))
            slot += (r1 - r0) // H
        wg.append(len(units))
    return (np.asarray(wg, np.int32), np.asarray(units, np.int32).reshape(-1, UNIT_INTS), slot)


CHAIN_NEXT = -(2 ** 31)   # slot field: the unit's state carries into the next unit


def cascade_chain_ref(group_req_indptr, prefix_lens, kv_lens, num_wg: int, tile: int = PLAN_TILE):
    """A cascade in one launch (64 heads or more, every prefix non-empty).

    Request b (in group g) is one block over the g prefix of L tiles' tokens.
    B requests on W lanes: B <= W gives S = W // B pieces per request (P =
    min(S, tiles) of them; piece p covers tiles p*T//P .. (p+1)*T//P - 1, on
    lane b*S + p); B > W puts request b whole on lane b % W.  Right after the
    last piece of b, on its lane, comes b's suffix (sequence G + b, tokens
    0 .. kv_lens[b]) when it is non-empty; that piece's slot field is
    CHAIN_NEXT (its state carries into the suffix unit).  A request with one
    piece writes out directly (slot -1); otherwise every state (each earlier
    piece, and the last piece or its chain) takes the next slot in emission
    order, and the request gets a merge record (b, first list entry, count, 1)
    listing its slots.  Unit records: (b, seq, kv_begin, kv_end, slot, 0, page
    fields 0, 0).  Returns dict(wg0, units0, merges, slot_list, n_slots)."""
    G = len(prefix_lens)
    B = len(kv_lens)
    grp = np.zeros(B, np.int64)
    for g in range(G):
        assert int(prefix_lens[g]) > 0
        grp[int(group_req_indptr[g]):int(group_req_indptr[g + 1])] = g
    if B <= num_wg:
        S = num_wg // B
        grid = B * S
        lanes = [[] for _ in range(grid)]
        P = []
        for b in range(B):
            L = int(prefix_lens[grp[b]])
            T = -(-L // tile)
            n = min(S, T)
            P.append(n)
            for p in range(n):
                t0, t1 = p * T // n, (p + 1) * T // n
                lanes[b * S + p].append((b, t0 * tile, min(t1 * tile, L), p == n - 1))
    else:
        grid = num_wg
        lanes = [[] for _ in range(grid)]
        P = [1] * B
        for b in range(B):
            lanes[b % num_wg].append((b, 0, int(prefix_lens[grp[b]]), True))
    units, wg, per = [], [0], [[] for _ in range(B)]
    slot = 0
    for lane in lanes:
        for (b, k0, k1, last) in lane:
            chain = last and int(kv_lens[b]) > 0

            def take():
                nonlocal slot
                if P[b] == 1:
                    return -1
                per[b].append(slot)
                slot += 1
                return slot - 1
            units.append((b, int(grp[b]), k0, k1, CHAIN_NEXT if chain else take(), 0, 0, 0))
            if chain:
                units.append((b, G + b, 0, int(kv_lens[b]), take(), 0, 0, 0))
        wg.append(len(units))
    merges, slot_list = [], []
    for b in range(B):
        if per[b]:
            merges.append((b, len(slot_list), len(per[b]), 1))
            slot_list.extend(per[b])
    return dict(wg0=np.asarray(wg, np.int32),
                units0=np.asarray(units, np.int64).astype(np.int32).reshape(-1, UNIT_INTS),
                merges=np.asarray(merges, np.int32).reshape(-1, MERGE_INTS),
                slot_list=np.asarray(slot_list, np.int32), n_slots=slot)


def cascade_plan_ref(group_req_indptr, prefix_lens, kv_lens, num_heads: int, num_wg: int,
                     num_wg0: int, tile: int = PLAN_TILE, fixed: int = 1):
    """The two schedules of a cascade plan and its merge lists.

    Level 1 is the split-KV walk over the suffix items with every unit given a
    partial slot, numbered after level 0's in emission order.  Request b's
    merge lists its level-0 slots (each level-0 unit whose rows hold b, in
    level-0 emission order: the unit's first slot + b - row0 / H) and then its
    level-1 slots; merge records are (b, first list entry, count, 1).

    Returns dict(wg0, units0, wg, units, merges, slot_list)."""
    H = int(num_heads)
    wg0, units0, n0 = row_schedule_ref(group_req_indptr, prefix_lens, H, num_wg0, tile)
    B = len(kv_lens)
    wg, units, _ = schedule_ref(suffix_items(len(prefix_lens), kv_lens), B, num_wg, tile, fixed)
    units = units.copy()
    units[:, 4] = n0 + np.arange(units.shape[0])
    per = [[] for _ in range(B)]
    for u in units0:
        first = (int(u[4]) + int(u[0])) // H
        for b in range(int(u[0]) // H, int(u[5]) // H):
            per[b].append(first + b - int(u[0]) // H)
    for u in units:
        per[int(u[0])].append(int(u[4]))
    merges, slot_list = [], []
    for b in range(B):
        merges.append((b, len(slot_list), len(per[b]), 1))
        slot_list.extend(per[b])
    return dict(wg0=wg0, units0=units0, wg=wg, units=units,
                merges=np.asarray(merges, np.int32).reshape(-1, MERGE_INTS),
                slot_list=np.asarray(slot_list, np.int32))


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
