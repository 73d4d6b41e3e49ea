"""CPU: pins for the split-KV schedule re-derivation (hand-worked cases and
structural invariants that hold for any valid schedule)."""

import numpy as np
import pytest

from oracle.schedule_ref import schedule_ref, flat_items, cascade_items, kernel_config
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


def test_cascade_items_and_schedule():
    items = cascade_items(np.array([0, 2, 5]), np.array([64, 0]), np.array([3, 0, 40, 0, 1]))
    assert items == [(0, 0, 64), (0, 2, 3), (1, 0, 64), (1, 3, 0), (2, 1, 0), (2, 4, 40),
                     (3, 1, 0), (3, 5, 0), (4, 1, 0), (4, 6, 1)]
    wg, units, merges = check_schedule(items, 5, 512, 32, 1)
    # request 3 has no tokens at all in this hand-made table: it gets no unit
    assert 3 not in set(units[:, 0].tolist())


def test_cascade_config_schedule():
    prefix, suffix = config_lens("cascade")
    B = len(suffix)
    kc = kernel_config(128)
    items = cascade_items(np.array([0, B]), np.array([prefix]), suffix)
    wg, units, merges = check_schedule(items, B, 256, kc["tile"], kc["fixed_cost"])
    assert len(merges) == B          # every request has prefix and suffix units


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
