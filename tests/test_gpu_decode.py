"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small cases compare every element; full-size workloads compare every request
too, in the same launch configuration the benchmark times.  Integer work (page-table gather, plan
tables) is compared bit for bit.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.schedule_ref import (schedule_ref, flat_items, cascade_plan_ref, cascade_chain_ref,
                                 qo_items, kernel_config, unit_page_fields)
from mla_workloads import (make_flat, make_cascade, make_config, make_qo, stress_variant,
                           stress_variant_cascade, poison_unreferenced, permute_pages,
                           STRESS_KINDS)
from gpu_helpers import (Dev, run_gpu, oracle_flat, oracle_cascade, oracle_qo, compare, bits_of,
                         dev_bf16)

pytestmark = pytest.mark.gpu

# a plain import: a library that fails to build or load fails this suite
import paged_kv_mla_amd as pk  # noqa: E402


def note(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield


def small(seed, lens, H=16, ps=16, pool=None, extra=0, sm_scale=None):
    return make_flat(f"s{seed}", seed, len(lens), H, ps, list(lens), pool_pages=pool,
                     extra_pages=extra, sm_scale=sm_scale)


# ------------------------------------------------------------- integer paths
GATHER_CASES = {
    "tiny": lambda: make_config("tiny"),
    "tiny_perm_poison": lambda: poison_unreferenced(permute_pages(make_config("tiny"), 3)),
    "ps1_scatter": lambda: small(61, [1, 2, 33, 95, 64], H=16, ps=1),
    "ps64_extra_pages": lambda: small(62, [1, 64, 65, 300], H=128, ps=64, extra=1),
    "ps256": lambda: small(63, [5, 511, 700], H=32, ps=256),
    # one page per tile: the smallest page size of the whole-tile copy path
    "ps32_tile_pages": lambda: small(64, [1, 31, 32, 33, 95, 97], H=128, ps=32),
    "ps8": lambda: small(65, [3, 8, 9, 40, 161], H=64, ps=8),
}


@pytest.mark.parametrize("name", sorted(GATHER_CASES))
def test_gather_bit_exact(name):
    inp = GATHER_CASES[name]()
    note(f"gather {name}")
    plan = pk.plan_for(inp)
    d = Dev(inp)
    rows = plan.gather(d.ckv, d.kpe)
    torch.cuda.synchronize()
    ref = oracle.gather_ref(inp.ckv, inp.kpe, inp.kv_indptr, inp.kv_indices, inp.kv_lens,
                            inp.page_size)
    assert np.array_equal(bits_of(rows), ref)


def test_gather_bit_exact_cascade():
    cas = make_cascade("cg", 64, 5, 16, 16, [32, 48], [1, 20, 0, 33, 5], groups=2)
    note("gather cascade")
    plan = pk.plan_for(cas)
    rows = plan.gather(dev_bf16(cas.ckv), dev_bf16(cas.kpe))
    # expected: each level-0 piece's prefix tokens, then each suffix unit's
    # tokens (the token ranges from the oracle's own schedule re-derivation)
    ex = plan.export()
    r = cascade_plan_ref(cas.group_req_indptr, cas.prefix_lens, cas.kv_lens, 16,
                         max(1, ex.num_cu // ex.head_groups), ex.num_cu, 32, int(ex.header[11]))
    G = cas.num_groups
    seq_indptr = np.concatenate([cas.prefix_indptr, cas.prefix_indptr[G] + cas.kv_indptr[1:]])
    seq_indices = np.concatenate([cas.prefix_indices[:cas.prefix_indptr[G]], cas.kv_indices])
    seq_lens = np.concatenate([cas.prefix_lens, cas.kv_lens])
    full = oracle.gather_ref(cas.ckv, cas.kpe, seq_indptr, seq_indices, seq_lens, cas.page_size)
    start = np.concatenate([[0], np.cumsum(seq_lens)])
    ref = [full[start[u[1]] + u[2]:start[u[1]] + u[3]]
           for u in np.concatenate([r["units0"], r["units"]])]
    ref = np.concatenate(ref) if ref else np.zeros((0, 576), np.uint16)
    assert np.array_equal(bits_of(rows), ref)


@pytest.mark.parametrize("name", ["tiny", "deepseek", "ragged"])
def test_plan_export_bit_exact(name):
    from mla_workloads import config_lens, CONFIGS
    cfg = CONFIGS[name]
    lens = config_lens(name)
    # page tables only matter for the seq tables: a simple contiguous layout
    ps = cfg["page_size"]
    npg = (lens.astype(np.int64) + ps - 1) // ps
    indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    indices = np.arange(indptr[-1], dtype=np.int32)[::-1].copy()
    note(f"export {name}")
    plan = pk.plan(indptr, indices, lens, cfg["num_heads"], ps, int(indptr[-1]))
    ex = plan.export()
    kc = kernel_config(cfg["num_heads"])
    hdr = ex.header
    assert list(hdr[:7]) == [1, len(lens), cfg["num_heads"], ps, 512, 64, kc["tile"]]
    assert list(hdr[7:12]) == [kc["waves"], kc["heads_per_wave"], kc["stages"],
                               kc["wg_per_cu"], kc["fixed_cost"]]
    assert ex.head_groups == kc["head_groups"]
    lanes = max(1, ex.num_cu * int(hdr[10]) // ex.head_groups)
    wg, units, merges = schedule_ref(flat_items(lens), len(lens), lanes, kc["tile"], int(hdr[11]))
    units = unit_page_fields(units, indptr, indices, ps)
    np.testing.assert_array_equal(ex.wg_indptr, wg)
    np.testing.assert_array_equal(ex.units, units)
    np.testing.assert_array_equal(ex.merges, merges)
    np.testing.assert_array_equal(ex.seq_indptr, indptr)
    np.testing.assert_array_equal(ex.seq_lens, lens)
    np.testing.assert_array_equal(ex.seq_indices, indices)
    assert ex.sm_scale == np.float32(1.0 / math.sqrt(576))


@pytest.mark.parametrize("H", [16, 64, 128])
def test_plan_export_cascade(H):
    cas = make_cascade("ce", 65 + H, 6, H, 16, [32, 48], [1, 20, 0, 33, 5, 7], groups=2)
    note(f"export cascade H{H}")
    ex = pk.plan_for(cas).export()
    kc = kernel_config(H)
    hdr = ex.header
    lanes = max(1, ex.num_cu * int(hdr[10]) // ex.head_groups)
    hg0 = max(1, H // 64)
    G = cas.num_groups
    seq_indptr = np.concatenate([cas.prefix_indptr, cas.prefix_indptr[G] + cas.kv_indptr[1:]])
    seq_indices = np.concatenate([cas.prefix_indices[:cas.prefix_indptr[G]], cas.kv_indices])
    # 64 heads or more with every prefix non-empty: one launch, suffixes chained
    chained = H >= 64 and (cas.prefix_lens > 0).all()
    assert int(hdr[31]) == int(chained)
    if chained:
        r = cascade_chain_ref(cas.group_req_indptr, cas.prefix_lens, cas.kv_lens,
                              max(1, ex.num_cu // hg0), kc["tile"])
        assert ex.units.shape[0] == 0 and ex.wg_indptr.tolist() == [0]
    else:
        r = cascade_plan_ref(cas.group_req_indptr, cas.prefix_lens, cas.kv_lens, H, lanes,
                             max(1, ex.num_cu // hg0), kc["tile"], int(hdr[11]))
        np.testing.assert_array_equal(ex.units, unit_page_fields(r["units"], seq_indptr,
                                                                 seq_indices, cas.page_size))
        np.testing.assert_array_equal(ex.wg_indptr, r["wg"])
    np.testing.assert_array_equal(ex.units0, unit_page_fields(r["units0"], seq_indptr,
                                                              seq_indices, cas.page_size))
    np.testing.assert_array_equal(ex.merges, r["merges"])
    np.testing.assert_array_equal(ex.slot_list, r["slot_list"])
    np.testing.assert_array_equal(ex.wg_indptr0, r["wg0"])
    np.testing.assert_array_equal(ex.seq_lens, np.concatenate([cas.prefix_lens, cas.kv_lens]))
    np.testing.assert_array_equal(ex.seq_indptr, seq_indptr)
    np.testing.assert_array_equal(ex.seq_indices, seq_indices)


# ------------------------------------------------------------ decode parity
SMALL_CASES = {
    "tiny": lambda: make_config("tiny"),
    "h16_ps1": lambda: small(71, [1, 2, 31, 32, 33, 257], H=16, ps=1),
    "h32_ps16": lambda: small(72, [1, 17, 64, 200, 513], H=32, ps=16),
    "h64_ps64": lambda: small(73, [1, 63, 64, 65, 1000], H=64, ps=64),
    "h128_ps64": lambda: small(74, [1, 33, 100, 700, 2049], H=128, ps=64),
    "h128_ps16": lambda: small(75, [1, 5, 96, 300], H=128, ps=16),
    "h128_ps1": lambda: small(76, [1, 31, 160], H=128, ps=1),
    "h16_ps256": lambda: small(77, [3, 256, 257, 900], H=16, ps=256),
    "h64_ps2_explicit_scale": lambda: small(78, [1, 9, 77, 130], H=64, ps=2, sm_scale=0.11),
    "h128_extra_pages": lambda: small(79, [1, 40, 64, 129], H=128, ps=64, extra=2),
    "h128_ps32": lambda: small(66, [1, 31, 32, 33, 500, 1025], H=128, ps=32),
    "h32_ps8": lambda: small(67, [2, 8, 33, 250], H=32, ps=8),
    "h16_ps32": lambda: small(68, [32, 64, 65, 700], H=16, ps=32),
}


@pytest.mark.parametrize("name", sorted(SMALL_CASES))
def test_decode_small(name):
    inp = SMALL_CASES[name]()
    note(f"decode {name}")
    out, lse = run_gpu(pk.plan_for(inp), Dev(inp))
    ref_o, ref_l = oracle_flat(inp)
    compare(out, lse, ref_o, ref_l, name=name)


@pytest.mark.parametrize("kind", STRESS_KINDS)
@pytest.mark.parametrize("H,ps", [(16, 16), (128, 64), (64, 1)])
def test_decode_stress(kind, H, ps):
    base = small(80 + H + ps, [1, 17, 64, 200, 777], H=H, ps=ps)
    inp = stress_variant(base, kind)
    note(f"stress {kind} H{H} ps{ps}")
    out, lse = run_gpu(pk.plan_for(inp), Dev(inp))
    ref_o, ref_l = oracle_flat(inp)
    compare(out, lse, ref_o, ref_l, name=f"{kind}/H{H}/ps{ps}")


@pytest.mark.parametrize("H,ps", [(16, 16), (128, 64), (32, 1)])
def test_poison_permutation_and_determinism(H, ps):
    inp = small(90 + H, [1, 15, 64, 333], H=H, ps=ps, extra=1)
    note(f"invariants H{H} ps{ps}")
    d = Dev(inp)
    plan = pk.plan_for(inp)
    o1, l1 = run_gpu(plan, d)
    o1, l1 = bits_of(o1), l1.cpu().numpy().copy()
    # run to run: bitwise identical, every output written (NaN-prefilled buffers)
    out = torch.full((inp.batch, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((inp.batch, H), float("nan"), dtype=torch.float32, device="cuda")
    o2, l2 = run_gpu(plan, d, out=out, lse=lse)
    assert np.array_equal(bits_of(o2), o1) and np.array_equal(l2.cpu().numpy(), l1)
    # NaN in every slot no request attends: bitwise identical
    pz = poison_unreferenced(inp)
    o3, l3 = run_gpu(pk.plan_for(pz), Dev(pz))
    assert np.array_equal(bits_of(o3), o1) and np.array_equal(l3.cpu().numpy(), l1)
    # physical page permutation: bitwise identical
    pp = permute_pages(inp, seed=11)
    o4, l4 = run_gpu(pk.plan_for(pp), Dev(pp))
    assert np.array_equal(bits_of(o4), o1) and np.array_equal(l4.cpu().numpy(), l1)


@pytest.mark.parametrize("H", [16, 128])
def test_single_token_is_exact(H):
    """kv_len = 1: the softmax weight is exactly 1, so out is the ckv row bit for bit."""
    inp = small(95, [1, 1, 1, 1], H=H, ps=16, pool=20)
    note(f"single token H{H}")
    out, lse = run_gpu(pk.plan_for(inp), Dev(inp))
    ob = bits_of(out)
    for b in range(inp.batch):
        p = inp.kv_indices[inp.kv_indptr[b]]
        assert np.array_equal(ob[b], np.broadcast_to(inp.ckv[p, 0], ob[b].shape))
    _, ref_l = oracle_flat(inp)
    np.testing.assert_allclose(lse.double().cpu().numpy(), ref_l, atol=1e-5, rtol=0)


def test_cascade_small():
    cas = make_cascade("cs", 96, 6, 64, 16, [32, 48], [1, 20, 0, 33, 5, 300], groups=2)
    note("cascade small")
    out, lse = run_gpu(pk.plan_for(cas), Dev(cas))
    ref_o, ref_l = oracle_cascade(cas)
    compare(out, lse, ref_o, ref_l, name="cascade small")
    fo, fl = run_gpu(pk.plan_for(cas.flat_view()), Dev(cas))
    compare(out, lse, *oracle_flat(cas.flat_view()), name="cascade vs flat oracle")
    # cascade and flat plans on the GPU agree within the same bar
    compare(out, lse, fo.float().double().cpu().numpy(), fl.double().cpu().numpy(),
            name="cascade vs flat gpu")


# Several groups, empty suffixes, prefixes that end inside a page (and one
# group whose prefix is empty), at every head count.
CASCADE_CASES = {
    "h16_ps16_unaligned": lambda: make_cascade("c16", 101, 7, 16, 16, [37, 0, 5],
                                               [1, 0, 40, 2, 17, 3, 0], groups=3),
    "h32_ps8_unaligned": lambda: make_cascade("c32", 102, 6, 32, 8, [61, 100],
                                              [0, 9, 0, 33, 250, 1], groups=2),
    "h128_ps64_unaligned": lambda: make_cascade("c128", 103, 5, 128, 64, [700, 64],
                                                [0, 1, 65, 0, 300], groups=2),
    "h128_ps1": lambda: make_cascade("c128p1", 104, 4, 128, 1, [45], [0, 3, 70, 1], groups=1),
    "h64_ps32_many_groups": lambda: make_cascade("c64", 105, 8, 64, 32, [33, 96, 1, 250],
                                                 [0, 5, 0, 77, 1, 0, 31, 32], groups=4),
}


@pytest.mark.parametrize("name", sorted(CASCADE_CASES))
def test_cascade_cases(name):
    cas = CASCADE_CASES[name]()
    note(f"cascade {name}")
    out, lse = run_gpu(pk.plan_for(cas), Dev(cas))
    ref_o, ref_l = oracle_cascade(cas)
    compare(out, lse, ref_o, ref_l, name=f"cascade {name}")


@pytest.mark.parametrize("kind", STRESS_KINDS)
@pytest.mark.parametrize("H,ps", [(128, 64), (16, 1), (32, 16)])
def test_cascade_stress(kind, H, ps):
    prefix = {64: [256, 70], 1: [90, 33], 16: [160, 45]}[ps]
    base = make_cascade(f"cst{H}", 110 + H + ps, 6, H, ps, prefix, [0, 40, 300, 1, 77, 129],
                        groups=2)
    cas = stress_variant_cascade(base, kind)
    note(f"cascade stress {kind} H{H} ps{ps}")
    out, lse = run_gpu(pk.plan_for(cas), Dev(cas))
    ref_o, ref_l = oracle_cascade(cas)
    compare(out, lse, ref_o, ref_l, name=f"cascade {kind}/H{H}/ps{ps}")


@pytest.mark.parametrize("H,ps", [(128, 64), (16, 16)])
def test_cascade_poison_permutation_and_determinism(H, ps):
    cas = make_cascade(f"cpp{H}", 120 + H, 5, H, ps, [100, 3 * ps], [0, 9, 70, 1, 200],
                       groups=2)
    note(f"cascade invariants H{H} ps{ps}")
    plan = pk.plan_for(cas)
    d = Dev(cas)
    o1, l1 = run_gpu(plan, d)
    o1, l1 = bits_of(o1), l1.cpu().numpy().copy()
    o2, l2 = run_gpu(plan, d)
    assert np.array_equal(bits_of(o2), o1) and np.array_equal(l2.cpu().numpy(), l1)
    pz = poison_unreferenced(cas)
    o3, l3 = run_gpu(pk.plan_for(pz), Dev(pz))
    assert np.array_equal(bits_of(o3), o1) and np.array_equal(l3.cpu().numpy(), l1)
    pp = permute_pages(cas, seed=12)
    o4, l4 = run_gpu(pk.plan_for(pp), Dev(pp))
    assert np.array_equal(bits_of(o4), o1) and np.array_equal(l4.cpu().numpy(), l1)
    ref_o, ref_l = oracle_cascade(cas)
    compare(torch.from_numpy(o1.view(np.int16)).view(torch.bfloat16), torch.from_numpy(l1),
            ref_o, ref_l, name=f"cascade invariants H{H}")


# ------------------------------------------------------------- full sizes
@pytest.mark.parametrize("name", ["deepseek", "long", "ragged"])
def test_full_size_flat(name):
    """Every request of the full-size workload against the oracle."""
    inp = make_config(name)
    note(f"full {name}: B={inp.batch} H={inp.num_heads} tokens={inp.total_tokens}")
    out, lse = run_gpu(pk.plan_for(inp), Dev(inp))
    ref_o, ref_l = oracle_flat(inp)
    st = compare(out, lse, ref_o, ref_l, name=name)
    note(f"full {name} stats {st}")


def test_full_size_cascade():
    """Every request of the full-size cascade workload against the oracle."""
    cas = make_config("cascade")
    note(f"full cascade: B={cas.batch} attended={cas.attended_tokens()}")
    out, lse = run_gpu(pk.plan_for(cas), Dev(cas))
    ref_o, ref_l = oracle_cascade(cas)
    st = compare(out, lse, ref_o, ref_l, name="cascade")
    note(f"full cascade stats {st}")


# ---------------------------------------- one combined [P, ps, 576] cache
@pytest.mark.parametrize("H,ps", [(128, 64), (128, 32), (64, 16), (16, 1)])
def test_combined_cache_views(H, ps):
    """The ckv and kpe views of one [pages, page_size, 576] cache (row stride
    576 for both) give the same bits as two packed caches, and match the
    oracle."""
    lens = {1: [1, 31, 70, 200], 16: [1, 17, 300, 513]}.get(ps, [1, 33, 100, 700, 2049])
    inp = small(90 + ps, lens, H=H, ps=ps)
    note(f"combined cache H={H} ps={ps}")
    dev = Dev(inp)
    plan = pk.plan_for(inp)
    o1, l1 = run_gpu(plan, dev)
    comb = torch.cat([dev.ckv, dev.kpe], dim=2).contiguous()
    o2, l2 = plan.run(dev.q_nope, dev.q_pe, comb[..., :512], comb[..., 512:])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ref_o, ref_l = oracle_flat(inp)
    compare(o2, l2, ref_o, ref_l, name=f"combined H{H} ps{ps}")


def test_combined_cache_cascade_and_bad_strides():
    cas = make_cascade("cc", 95, 6, 64, 16, [32, 48], [1, 20, 0, 33, 5, 7], groups=2)
    dev = Dev(cas)
    plan = pk.plan_for(cas)
    o1, l1 = run_gpu(plan, dev)
    comb = torch.cat([dev.ckv, dev.kpe], dim=2).contiguous()
    o2, l2 = plan.run(dev.q_nope, dev.q_pe, comb[..., :512], comb[..., 512:])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    out = torch.empty_like(o1)
    lse = torch.empty_like(l1)
    s = int(torch.cuda.current_stream().cuda_stream)
    for cs, ks in [(500, 64), (512, 60), (516, 64), (576, 1 << 21)]:
        rc = pk._lib.pkvmla_run_strided(plan._h, dev.q_nope.data_ptr(), dev.q_pe.data_ptr(),
                                        dev.ckv.data_ptr(), dev.kpe.data_ptr(), cs, ks,
                                        out.data_ptr(), lse.data_ptr(), s)
        assert rc == pk.EINVAL, (cs, ks)


# ------------------------------------------------------- extreme shapes
def test_one_request_over_every_lane():
    """One 131072-token request: the schedule splits it over every lane, so
    the merge combines the largest number of partial states (one per lane)."""
    inp = small(97, [131072], H=128, ps=64)
    ex = pk.plan_for(inp).export()
    n_split = int(ex.merges[0, 2])
    note(f"one request, {n_split} partial states")
    assert ex.merges.shape[0] == 1 and n_split == ex.grid >= 64
    out, lse = run_gpu(pk.plan_for(inp), Dev(inp))
    ref_o, ref_l = oracle_flat(inp)
    compare(out, lse, ref_o, ref_l, name="one request")


@pytest.mark.parametrize("H", [16, 128])
def test_many_tiny_requests(H):
    """2048 requests of 1..8 tokens at page size 1: many units per lane (more
    than the four whose bounds the kernel's prologue loads together, so the
    tile count also takes its per-unit loop), no splits, every request
    written by the decode kernel directly."""
    rng = np.random.default_rng(98)
    lens = rng.integers(1, 9, size=2048).tolist()
    inp = small(98, lens, H=H, ps=1)
    ex = pk.plan_for(inp).export()
    per_lane = np.diff(ex.wg_indptr)
    note(f"2048 tiny requests H{H}: {ex.units.shape[0]} units on {ex.grid} lanes, "
         f"up to {per_lane.max()} per lane")
    assert ex.merges.shape[0] == 0
    assert per_lane.max() > 4
    out, lse = run_gpu(pk.plan_for(inp), Dev(inp))
    ref_o, ref_l = oracle_flat(inp)
    compare(out, lse, ref_o, ref_l, name=f"tiny requests H{H}")


def lane_tiles(ex):
    """Tiles each workgroup of a plan walks (its units' 32-token tiles)."""
    wg, u = ex.wg_indptr, ex.units
    return [int(sum((u[k, 3] - u[k, 2] + 31) // 32 for k in range(wg[l], wg[l + 1])))
            for l in range(len(wg) - 1) if wg[l + 1] > wg[l]]


# (requests, lengths drawn from [1, hi), page size): together their
# workgroups walk every tile count from 1 to 8, around the 4-stage ring
PROGRESS_CASES = [(100, 300, 1), (300, 100, 16), (120, 600, 64), (100, 900, 16), (64, 2000, 1)]


@pytest.mark.parametrize("H", [16, 32])
def test_progress_counters_short_workgroups(H):
    """At 16 and 32 heads the roles of a workgroup synchronise through LDS
    progress counters; workgroups with 1..8 tiles exercise the copy waves'
    first refills of the 4-stage ring and the end of every wait."""
    seen = set()
    for i, (n, hi, ps) in enumerate(PROGRESS_CASES):
        rng = np.random.default_rng(4000 + 10 * H + i)
        lens = rng.integers(1, hi, size=n).tolist()
        inp = small(4000 + 10 * H + i, lens, H=H, ps=ps)
        plan = pk.plan_for(inp)
        g = lane_tiles(plan.export())
        seen.update(g)
        note(f"counters H{H} case {i}: {n} requests ps{ps}, tiles per workgroup {min(g)}..{max(g)}")
        out, lse = run_gpu(plan, Dev(inp))
        ref_o, ref_l = oracle_flat(inp)
        compare(out, lse, ref_o, ref_l, name=f"counters H{H} case {i}")
    assert set(range(1, 9)) <= seen, sorted(seen)


@pytest.mark.parametrize("H", [16, 32, 128])
def test_wait_limit_failure_path(H):
    """The failure path of the progress counters, forced from the host: with a
    wait limit of 0 polls every counter wait gives up at once and marks its
    workgroup, so every output of the 16- and 32-head kernels reads NaN (all
    accesses stay in bounds and the launch ends normally); the 128-head kernel
    keeps its barrier and ignores the limit; at the default limit the results
    match the oracle again."""
    inp = small(4100 + H, [1, 40, 300, 900, 2000, 77], H=H, ps=16)
    plan = pk.plan_for(inp)
    dev = Dev(inp)
    with pytest.raises(pk.PkvmlaError):
        plan.set_wait_limit(-1)
    plan.set_wait_limit(0)
    note(f"wait limit 0, H{H}")
    out, lse = run_gpu(plan, dev)
    ref_o, ref_l = oracle_flat(inp)
    if H < 64:
        assert bool(torch.isnan(out.float()).all()) and bool(torch.isnan(lse).all())
    else:
        compare(out, lse, ref_o, ref_l, name=f"wait limit 0, H{H}")
    plan.set_wait_limit()
    out, lse = run_gpu(plan, dev)
    compare(out, lse, ref_o, ref_l, name=f"default wait limit, H{H}")


# ------------------------------------- several new query tokens per request
QO_CASES = {
    "h16_qo2_ps16": lambda: make_qo("q1", 131, 5, 16, 16, [2, 17, 64, 200, 777], [2] * 5),
    "h16_qo4_ps1": lambda: make_qo("q2", 132, 4, 16, 1, [4, 31, 33, 300], [4] * 4),
    "h128_qo2_ps64": lambda: make_qo("q3", 133, 4, 128, 64, [2, 65, 700, 2049], [2] * 4),
    "h128_qo4_ps64": lambda: make_qo("q4", 134, 4, 128, 64, [4, 100, 1025, 3000], [4] * 4),
    "h32_mixed_ps8": lambda: make_qo("q5", 135, 6, 32, 8, [1, 5, 40, 9, 250, 16], [1, 5, 3, 2, 4, 16]),
    "h64_mixed_ps16": lambda: make_qo("q6", 136, 5, 64, 16, [3, 48, 513, 7, 90], [3, 1, 4, 7, 2]),
}


@pytest.mark.parametrize("name", sorted(QO_CASES))
def test_qo_decode(name):
    inp = QO_CASES[name]()
    note(f"qo {name}: {int(inp.qo_indptr[-1])} query rows")
    out, lse = run_gpu(pk.plan_for(inp), Dev(inp))
    ref_o, ref_l = oracle_qo(inp)
    compare(out, lse, ref_o, ref_l, name=f"qo {name}")


@pytest.mark.parametrize("H,ps", [(16, 16), (128, 64)])
def test_qo_stress_and_export(H, ps):
    inp = stress_variant(make_qo("qs", 137 + H, 4, H, ps, [4, 70, 300, 1500], [4, 2, 3, 4]), "qx8")
    note(f"qo stress H{H} ps{ps}")
    plan = pk.plan_for(inp, qo_layout=pk.QO_TOKENS)
    out, lse = run_gpu(plan, Dev(inp))
    compare(out, lse, *oracle_qo(inp), name=f"qo qx8 H{H}")
    # the uploaded schedule is the rule's, one item per query row
    ex = plan.export()
    kc = kernel_config(H)
    lanes = max(1, ex.num_cu * kc["wg_per_cu"] // kc["head_groups"])
    wg, units, merges = schedule_ref(qo_items(inp.qo_indptr, inp.kv_lens), int(inp.qo_indptr[-1]),
                                     lanes, kc["tile"], kc["fixed_cost"])
    units = unit_page_fields(units, inp.kv_indptr, inp.kv_indices, ps)
    assert int(ex.header[26]) == 1 and int(ex.header[27]) == inp.batch
    np.testing.assert_array_equal(ex.wg_indptr, wg)
    np.testing.assert_array_equal(ex.units, units)
    np.testing.assert_array_equal(ex.merges, merges)


# Row blocks of query tokens (16 and 32 heads): each case runs in both
# layouts, each checked against the oracle; the row-block plan's tables are
# checked against the oracle's schedule re-derivation bit for bit.
QO_ROW_CASES = {
    "h16_qo4_ps1": lambda: make_qo("r1", 141, 4, 16, 1, [4, 31, 33, 300], [4] * 4),
    "h16_qo3_ps16": lambda: make_qo("r2", 142, 5, 16, 16, [3, 17, 64, 200, 777], [3] * 5),
    "h32_mixed_ps8": QO_CASES["h32_mixed_ps8"],
    "h32_qo2_ps64": lambda: make_qo("r3", 143, 3, 32, 64, [2, 700, 2049], [2, 2, 2]),
    # one request's 40 tokens (10 blocks) over 101 positions, split in
    # 32-token pieces: a block's last piece can start past its first tokens'
    # reach, so they see no token of it at all
    "h16_masked_pieces_ps16": lambda: make_qo("r4", 144, 3, 16, 16, [101, 100, 90], [40, 1, 6]),
    # a prefill (every token new) beside decodes: early blocks stop early
    "h16_prefill_mix_ps16": lambda: make_qo("r7", 150, 4, 16, 16, [512, 300, 90, 700],
                                            [512, 1, 6, 1]),
    "h32_masked_pieces_ps1": lambda: make_qo("r5", 145, 2, 32, 1, [400, 33], [36, 2]),
    # partial blocks: 5 tokens at 16 heads (80 rows), 3 at 32 (96 rows)
    "h16_h32_tails": lambda: make_qo("r6", 146, 4, 16, 32, [5, 900, 63, 64], [5, 5, 2, 7]),
}


def qo_row_tables_ref(inp, num_cu):
    from oracle.schedule_ref import qo_rows_ref
    return qo_rows_ref(inp.qo_indptr, inp.kv_lens, inp.num_heads, num_cu,
                       pages=(inp.kv_indptr, inp.kv_indices, inp.page_size))


def fully_masked_waves(units, H):
    """Waves (16 rows of one token) of row-block units that see no token of
    their piece."""
    n = 0
    for r0, c, k0, k1, _, r1, _, _ in units.tolist():
        for w in range(4):
            row = r0 + 16 * w
            if row < r1 and (row // H) + c <= k0:
                n += 1
    return n


@pytest.mark.parametrize("name", sorted(QO_ROW_CASES))
def test_qo_row_blocks(name):
    from oracle.schedule_ref import QO_ROWS_DIRECT
    inp = QO_ROW_CASES[name]()
    H = inp.num_heads
    note(f"qo rows {name}: {int(inp.qo_indptr[-1])} query tokens, H{H}")
    d = Dev(inp)
    ref_o, ref_l = oracle_qo(inp)
    plan = pk.plan_for(inp, qo_layout=pk.QO_ROW_BLOCKS)
    ex = plan.export()
    assert int(ex.header[26]) == 2 and int(ex.header[27]) == inp.batch
    wg, units, merges, slot_list, n_slots = qo_row_tables_ref(inp, ex.num_cu)
    np.testing.assert_array_equal(ex.wg_indptr0, wg)
    np.testing.assert_array_equal(ex.units0, units)
    np.testing.assert_array_equal(ex.merges, merges)
    np.testing.assert_array_equal(ex.slot_list, slot_list)
    assert ex.units.shape[0] == 0 and int(ex.header[15]) == n_slots
    if "masked" in name:
        assert fully_masked_waves(units, H) > 0
        assert (units[:, 4] != QO_ROWS_DIRECT).any()
    out, lse = run_gpu(plan, d)
    compare(out, lse, ref_o, ref_l, name=f"qo rows {name}")
    # the same inputs one item per token
    out2, lse2 = run_gpu(pk.plan_for(inp, qo_layout=pk.QO_TOKENS), d)
    compare(out2, lse2, ref_o, ref_l, name=f"qo tokens {name}")


@pytest.mark.parametrize("kind", STRESS_KINDS)
def test_qo_row_blocks_stress(kind):
    inp = stress_variant(make_qo("rs", 147, 4, 16, 16, [4, 70, 300, 1500], [4, 9, 3, 16]), kind)
    note(f"qo rows stress {kind}")
    plan = pk.plan_for(inp, qo_layout=pk.QO_ROW_BLOCKS)
    out, lse = run_gpu(plan, Dev(inp))
    compare(out, lse, *oracle_qo(inp), name=f"qo rows {kind}")


def test_qo_row_blocks_poison_permutation_bit_identity():
    """Pages no table names hold NaN and the pool is permuted: the outputs
    are bit-identical to the plain layout's."""
    base = make_qo("rp", 148, 3, 32, 16, [64, 500, 333], [3, 8, 2])
    note("qo rows poison + permutation")
    o1, l1 = run_gpu(pk.plan_for(base, qo_layout=pk.QO_ROW_BLOCKS), Dev(base))
    alt = poison_unreferenced(permute_pages(base, 5))
    o2, l2 = run_gpu(pk.plan_for(alt, qo_layout=pk.QO_ROW_BLOCKS), Dev(alt))
    assert np.array_equal(bits_of(o1), bits_of(o2))
    assert torch.equal(l1, l2)


def test_qo_row_blocks_full_size():
    """64 requests of 4 new tokens at 16 heads, kv_len uniform in
    [1024, 4096], page size 64: every query row against the oracle."""
    rng = np.random.default_rng(149)
    lens = rng.integers(1024, 4096, size=64, endpoint=True)
    inp = make_qo("rf", 149, 64, 16, 64, lens.tolist(), [4] * 64)
    note("qo rows full size B64 H16 qo4")
    plan = pk.plan_for(inp)
    assert int(plan.export().header[26]) == 2        # the rule picks row blocks
    out, lse = run_gpu(plan, Dev(inp))
    compare(out, lse, *oracle_qo(inp), name="qo rows full size")
