"""CPU: pins for the split-KV schedule re-derivation (hand-worked cases and
structural invariants that hold for any valid schedule)."""

import numpy as np
import pytest

from oracle.schedule_ref import schedule_ref, flat_items, kernel_config
from mla_workloads import config_lens, CONFIGS


def test_hand_worked_small_many_workgroups():
    # lens 1,17,64,200 -> tiles 1,1,2,7; fixed 1 -> C = 15, cap = max(1, 2) = 2:
    # every workgroup takes one tile, the 7-tile request is cut seven ways.
    wg, units, merges = schedule_ref(flat_items([1, 17, 64, 200]), 4, num_wg=512, tile=32, fixed=1)
    expect = [(0, 0, 0, 1, -1), (1, 1, 0, 17, -1), (2, 2, 0, 32, 0), (2, 2, 32, 64, 1)]
    expect += [(3, 3, 32 * k, min(32 * k + 32, 200), 2 + k) for k in range(7)]
    assert [tuple(u[:5]) for u in units] == expect
    assert wg.tolist() == list(range(12))
    assert merges.tolist() == [[2, 0, 2, 0], [3, 2, 7, 0]]


def test_hand_worked_small_two_workgroups():
    # C = 15, cap = 8: the first workgroup takes requests 0..2 (cost 7), the
    # last one takes all of request 3.
    wg, units, merges = schedule_ref(flat_items([1, 17, 64, 200]), 4, num_wg=2, tile=32, fixed=1)
    assert [tuple(u[:5]) for u in units] == [(0, 0, 0, 1, -1), (1, 1, 0, 17, -1),
                                            (2, 2, 0, 64, -1), (3, 3, 0, 200, -1)]
    assert wg.tolist() == [0, 3, 4]
    assert merges.shape == (0, 4)


def check_schedule(items, batch, num_wg, tile, fixed):
    wg, units, merges = schedule_ref(items, batch, num_wg, tile, fixed)
    grid = len(wg) - 1
    assert 0 < grid <= num_wg
    assert np.all(np.diff(wg) >= 1)              # every launched workgroup has work
    # exact coverage of every (request, sequence, token) once, tile-aligned cuts
    cover = {}
    for u in units:
        b, s, k0, k1, slot = map(int, u[:5])
        assert 0 <= k0 < k1 and k0 % tile == 0
        cover.setdefault((b, s), []).append((k0, k1))
    for (b, s, L) in items:
        if L == 0:
            assert (b, s) not in cover
            continue
        segs = sorted(cover[(b, s)])
        assert segs[0][0] == 0 and segs[-1][1] == L
        assert all(a[1] == c[0] for a, c in zip(segs[:-1], segs[1:]))
    # slots: -1 iff the request has one unit; otherwise unique, consecutive per request
    nreq = np.bincount(units[:, 0], minlength=batch)
    slots = units[:, 4]
    assert np.all((slots == -1) == (nreq[units[:, 0]] == 1))
    used = slots[slots >= 0]
    assert sorted(used.tolist()) == list(range(len(used)))
    for b, s0, n, _ in merges.tolist():
        assert nreq[b] == n > 1
        assert sorted(slots[units[:, 0] == b].tolist()) == list(range(s0, s0 + n))
    assert len(merges) == int((nreq > 1).sum())
    return wg, units, merges


@pytest.mark.parametrize("name", ["tiny", "deepseek", "long", "ragged"])
@pytest.mark.parametrize("num_cu", [256, 80, 1])
def test_flat_schedule_invariants(name, num_cu):
    lens = config_lens(name)
    kc = kernel_config(CONFIGS[name]["num_heads"])
    check_schedule(flat_items(lens), len(lens), num_cu * kc["wg_per_cu"], kc["tile"],
                   kc["fixed_cost"])


def test_deepseek_balance():
    """On 256 CUs no workgroup carries more than cap + one segment of slack."""
    lens = config_lens("deepseek")
    kc = kernel_config(128)
    wg, units, _ = schedule_ref(flat_items(lens), len(lens), 256, kc["tile"], kc["fixed_cost"])
    cost = np.zeros(len(wg) - 1)
    for w in range(len(wg) - 1):
        for u in units[wg[w]:wg[w + 1]]:
            cost[w] += -(-(int(u[3]) - int(u[2])) // kc["tile"]) + kc["fixed_cost"]
    assert len(wg) - 1 <= 256
    assert cost.max() <= cost.mean() * 1.15


def test_row_schedule_hand_cases():
    """Level-0 schedules worked out by hand from the rule."""
    from oracle.schedule_ref import row_schedule_ref
    # one group of two requests at 16 heads (32 rows, one block), 64-token
    # prefix (2 tiles), 512 lanes: S = 512 pieces asked, 2 tiles give 2 pieces
    wg, units, ns = row_schedule_ref([0, 2, 5], [64, 0], 16, 512)
    assert len(wg) == 513 and wg[1] == 1 and wg[2] == 2 and wg[-1] == 2
    assert units.tolist() == [[0, 0, 0, 32, 0, 32, 0, 0], [0, 0, 32, 64, 32, 32, 0, 0]]
    assert ns == 4     # two requests per piece
    # three requests at 128 heads (a block each), 2 lanes: blocks 0 and 2 on
    # lane 0, block 1 on lane 1; slots in lane order 0, 1 | 2
    wg, units, ns = row_schedule_ref([0, 3], [100], 128, 2)
    assert wg.tolist() == [0, 2, 3]
    assert units.tolist() == [[0, 0, 0, 100, 0, 128, 0, 0], [256, 0, 0, 100, -128, 384, 0, 0],
                              [128, 0, 0, 100, 128, 256, 0, 0]]
    assert ns == 3
    # 32 heads, 5 requests: rows 0..159 -> blocks of 64, 64, 32 rows; 7 lanes:
    # S = 2 pieces each of a 3-tile prefix: tiles [0,1) and [1,3)
    wg, units, ns = row_schedule_ref([0, 5], [70], 32, 7)
    assert wg.tolist() == [0, 1, 2, 3, 4, 5, 6]
    assert [u[:6] for u in units.tolist()] == [
        [0, 0, 0, 32, 0, 64], [0, 0, 32, 70, 64, 64],
        [64, 0, 0, 32, 64, 128], [64, 0, 32, 70, 128, 128],
        [128, 0, 0, 32, 128, 160], [128, 0, 32, 70, 160, 160]]
    assert ns == 10


def test_cascade_plan_merge_lists_hand_case():
    """Two groups ([0, 2) with a 64-token prefix, [2, 5) with none), suffixes
    3, 0, 40, 2, 1 at 16 heads; 512 level-0 lanes, 512 level-1 lanes."""
    from oracle.schedule_ref import cascade_plan_ref
    r = cascade_plan_ref([0, 2, 5], [64, 0], [3, 0, 40, 2, 1], 16, 512, 512, 32, 1)
    # level 0: piece 0 (lane 0) holds slots 0, 1 (requests 0, 1), piece 1
    # (lane 1) slots 2, 3.  Level 1: cost 2 + 3 + 2 + 2 = 9 on 512 lanes gives
    # the minimum cap 2, one tile per unit: request 2's 40 tokens take two
    # units.  Slots 4..8 in emission order.
    assert r["units"][:, :5].tolist() == [[0, 2, 0, 3, 4], [2, 4, 0, 32, 5], [2, 4, 32, 40, 6],
                                          [3, 5, 0, 2, 7], [4, 6, 0, 1, 8]]
    assert r["merges"].tolist() == [[0, 0, 3, 1], [1, 3, 2, 1], [2, 5, 2, 1], [3, 7, 1, 1],
                                    [4, 8, 1, 1]]
    assert r["slot_list"].tolist() == [0, 2, 4, 1, 3, 5, 6, 7, 8]


def test_chain_schedule_hand_cases():
    """One-launch cascade schedules worked out by hand from the rule."""
    from oracle.schedule_ref import cascade_chain_ref, CHAIN_NEXT
    # two requests, one group, 100-token prefix (4 tiles), suffixes 10 and 0,
    # 4 lanes: S = 2 pieces each; tiles [0,2) and [2,4) of 4
    r = cascade_chain_ref([0, 2], [100], [10, 0], 4)
    assert r["wg0"].tolist() == [0, 1, 3, 4, 5]
    assert [u[:5] for u in r["units0"].tolist()] == [
        [0, 0, 0, 64, 0],               # request 0 piece 0: slot 0
        [0, 0, 64, 100, CHAIN_NEXT],    # piece 1, state carried into ...
        [0, 1, 0, 10, 1],               # ... its suffix (sequence G + 0): slot 1
        [1, 0, 0, 64, 2],               # request 1 (empty suffix): pieces in slots 2, 3
        [1, 0, 64, 100, 3]]
    assert r["merges"].tolist() == [[0, 0, 2, 1], [1, 2, 2, 1]]
    assert r["slot_list"].tolist() == [0, 1, 2, 3]
    # three requests on 2 lanes: whole requests round robin, one state each
    r = cascade_chain_ref([0, 3], [40], [5, 6, 0], 2)
    assert r["wg0"].tolist() == [0, 3, 5]
    assert [u[:5] for u in r["units0"].tolist()] == [
        [0, 0, 0, 40, CHAIN_NEXT], [0, 1, 0, 5, -1], [2, 0, 0, 40, -1],
        [1, 0, 0, 40, CHAIN_NEXT], [1, 2, 0, 6, -1]]
    assert r["merges"].shape == (0, 4)


def test_cascade_config_schedule():
    from oracle.schedule_ref import cascade_plan_ref
    prefix, suffix = config_lens("cascade")
    B = len(suffix)
    kc = kernel_config(128)
    r = cascade_plan_ref([0, B], [prefix], suffix, 128, 128, 128, kc["tile"], kc["fixed_cost"])
    # one lane per request, each walking the whole prefix from its first tile
    assert len(r["wg0"]) == B + 1 and r["units0"].shape[0] == B
    assert (r["units0"][:, 2] == 0).all() and (r["units0"][:, 3] == prefix).all()
    assert r["merges"][:, 2].min() >= 2      # a prefix state and at least one suffix state


def test_unit_page_fields_hand_case():
    """Page fields worked out by hand: sequence 0 owns pages [7, 3], sequence 1
    pages [9, 1, 4] (page size 16).  A unit of sequence 1 starting at token 32
    begins in its third page, id 4; one of sequence 0 at token 16, in page 3."""
    from oracle.schedule_ref import unit_page_fields
    units = np.zeros((3, 8), np.int32)
    units[0, :4] = (0, 0, 0, 16)
    units[1, :4] = (1, 1, 32, 40)
    units[2, :4] = (0, 0, 16, 20)
    got = unit_page_fields(units, [0, 2, 5], [7, 3, 9, 1, 4], 16)
    assert got[:, 6].tolist() == [0, 2, 0]
    assert got[:, 7].tolist() == [7, 4, 3]
    assert np.array_equal(got[:, :6], units[:, :6])   # the schedule fields are untouched


def test_qo_rows_layout_rule_hand_cases():
    """Row blocks at 16 or 32 heads when some request has two or more tokens."""
    from oracle.schedule_ref import qo_uses_rows
    assert qo_uses_rows([0, 2], 16)
    assert not qo_uses_rows([0, 1], 32)          # one token: a plain decode
    assert not qo_uses_rows([0, 1, 2, 3], 16)    # one token each
    assert qo_uses_rows([0, 2], 32)
    assert not qo_uses_rows([0, 4], 64)          # 64 heads or more: one item per token
    assert not qo_uses_rows([0, 4], 128)
    assert qo_uses_rows([0, 1, 2, 3, 5], 16)     # one request with two tokens


def test_qo_rows_schedule_hand_case():
    """H = 16, requests with 5 and 2 new tokens, kv_lens 100 and 40, 8 lanes.
    Blocks: rows [0, 64) and [64, 80) of request 0, [80, 112) of request 1.
    Causal offsets: 100 - 5 + 1 - 0 = 96 and 40 - 2 + 1 - 5 = 34, so the
    blocks' last tokens 3, 4 and 6 reach 99, 100 and 40 positions: items of
    4, 4 and 2 tiles at fixed cost 4, C = 22.  cap 5 (one tile per unit)
    needs 10 lanes, cap 6 (two tiles) needs 5: request 0's blocks are cut at
    position 64 into walk slots 0, 1 and 2, 3; the last block stays whole."""
    from oracle.schedule_ref import qo_rows_ref, QO_ROWS_DIRECT
    wg, units, merges, slot_list, n_slots = qo_rows_ref([0, 5, 7], [100, 40], 16, 8)
    assert wg.tolist() == [0, 1, 2, 3, 4, 5]
    assert [u[:6] for u in units.tolist()] == [
        [0, 96, 0, 64, 0, 64], [0, 96, 64, 99, 64, 64],
        [64, 96, 0, 64, 64, 80], [64, 96, 64, 100, 128, 80],
        [80, 34, 0, 40, QO_ROWS_DIRECT, 112]]
    # four 16-row slots per walk slot: token t of block 0 sits in slots t and
    # 4 + t; token 4 (block 1, rows 64..79) in walk slots 2 and 3's first
    assert merges.tolist() == [[0, 0, 2, 1], [1, 2, 2, 1], [2, 4, 2, 1], [3, 6, 2, 1],
                               [4, 8, 2, 1]]
    assert slot_list.tolist() == [0, 4, 1, 5, 2, 6, 3, 7, 8, 12]
    assert n_slots == 16


@pytest.mark.parametrize("seed", range(40))
def test_qo_rows_schedule_invariants(seed):
    """Any qo row-block schedule: the block's pieces tile [0, t_last + c)
    exactly once, t_last being its last token (so every row's causal range
    [0, t + c) is covered and no tile lies wholly past all of them); every
    partial row is written by exactly one (piece, token) and read by that
    token's merge alone; whole blocks have no merge."""
    from oracle.schedule_ref import qo_rows_ref, QO_ROWS_DIRECT
    rng = np.random.default_rng(seed)
    H = int(rng.choice([16, 32]))
    B = int(rng.integers(1, 7))
    qo = rng.integers(1, 20, size=B)
    kv = np.maximum(qo, rng.integers(1, 3000, size=B))
    qo_indptr = np.concatenate([[0], np.cumsum(qo)]).astype(np.int32)
    W = int(rng.integers(1, 300))
    wg, units, merges, slot_list, n_slots = qo_rows_ref(qo_indptr, kv, H, W)
    assert 0 < len(wg) - 1 <= W and np.all(np.diff(wg) >= 1)
    cover, writers = {}, {}
    for u in units.tolist():
        r0, c, k0, k1, sl, r1 = u[:6]
        assert 0 <= k0 < k1 and r0 % H == 0 and r1 % H == 0 and 0 < r1 - r0 <= 64
        cover.setdefault(r0, []).append((k0, k1, sl))
        for t in range(r0 // H, r1 // H):
            b = int(np.searchsorted(qo_indptr, t, side="right")) - 1
            n = int(qo[b])
            assert t + c == int(kv[b]) - n + 1 + (t - int(qo_indptr[b]))   # causal limit
            if sl != QO_ROWS_DIRECT:
                s = (sl + t * H) // H
                assert (sl + t * H) % H == 0 and 0 <= s < n_slots
                assert s not in writers
                writers[s] = t
    ends = {u[0]: (u[5], u[1]) for u in units.tolist()}
    for r0, pieces in cover.items():
        pieces.sort()
        r1, c = ends[r0]
        assert pieces[0][0] == 0 and pieces[-1][1] == (r1 // H - 1) + c
        assert all(pieces[i][1] == pieces[i + 1][0] for i in range(len(pieces) - 1))
        assert (len(pieces) == 1) == (pieces[0][2] == QO_ROWS_DIRECT)
    merged = {}
    for (t, pos, cnt, kind) in merges.tolist():
        assert kind == 1 and t not in merged
        merged[t] = slot_list[pos:pos + cnt].tolist()
        assert all(writers[s] == t for s in merged[t])
    assert sorted(s for v in merged.values() for s in v) == sorted(writers)
