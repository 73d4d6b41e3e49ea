"""HIP-graph capture of the decode and in-place page-table updates.

A plan built with a page-id capacity keeps its device tables, split workspace
and launch shapes across `Plan.update`, so one HIP graph captured around
`Plan.run` serves successive page tables.  The graph-capture failure of the
MLA decode path is the recurring problem on the vLLM pull-request page
"[WIP][Kernel] Flashinfer MLA support".

Every replay is checked bit for bit against an eager run of the same plan
state (and of a fresh ordinary plan for the same tables), with the program's
own eager work and synchronisations between replays, and the updated tables'
results against the fp64 oracle.
"""

import numpy as np
import pytest
import torch

from mla_workloads import make_flat
from gpu_helpers import Dev, oracle_flat, compare, dev_bf16

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


POOL = 160


def tables(seed, lens, H, ps):
    return make_flat(f"g{seed}", seed, len(lens), H, ps, list(lens), pool_pages=POOL)


def load_into(dev: Dev, inp) -> None:
    """Copy another bundle's tensors into the captured tensors (same shapes)."""
    dev.q_nope.copy_(dev_bf16(inp.q_nope))
    dev.q_pe.copy_(dev_bf16(inp.q_pe))
    dev.ckv.copy_(dev_bf16(inp.ckv))
    dev.kpe.copy_(dev_bf16(inp.kpe))


def eager(plan, dev, out, lse, stream):
    with torch.cuda.stream(stream):
        plan.run(dev.q_nope, dev.q_pe, dev.ckv, dev.kpe, out=out, lse=lse, stream=stream)
    torch.cuda.synchronize()
    return out.clone(), lse.clone()


@pytest.mark.parametrize("H,ps", [(128, 64), (16, 1), (64, 16)])
def test_graph_replay_and_update(H, ps):
    # three page tables of one batch: different lengths, page counts and
    # split patterns (the long request splits across lanes, the others not)
    specs = [[1, 40, 333, 1000, 64], [700, 3, 129, 64, 1200], [5, 5, 5, 5, 5]]
    if ps == 1:
        specs = [[1, 20, 33, 50, 4], [30, 3, 9, 64, 40], [5, 5, 5, 5, 5]]
    bundles = [tables(200 + i, s, H, ps) for i, s in enumerate(specs)]
    cap = max(len(b.kv_indices) for b in bundles) + 7
    A = bundles[0]
    note(f"graph H={H} ps={ps} cap={cap}")
    plan = pk.plan(A.kv_indptr, A.kv_indices, A.kv_lens, H, ps, POOL, index_capacity=cap)
    assert plan.export().header[24] == 1
    dev = Dev(A)
    out = torch.empty((A.batch, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((A.batch, H), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    ref_o, ref_l = eager(plan, dev, out, lse, side)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        plan.run(dev.q_nope, dev.q_pe, dev.ckv, dev.kpe, out=out, lse=lse, stream=side)
    torch.cuda.synchronize()

    for step, inp in enumerate(bundles + [A]):
        if step > 0:
            plan.update(inp.kv_indptr, inp.kv_indices, inp.kv_lens, stream=side)
            load_into(dev, inp)
            torch.cuda.synchronize()
            ref_o, ref_l = eager(plan, dev, out, lse, side)
            # a fresh ordinary plan (exact launch shapes) gives the same bits
            fresh = pk.plan(inp.kv_indptr, inp.kv_indices, inp.kv_lens, H, ps, POOL)
            fo, fl = eager(fresh, dev, torch.empty_like(out), torch.empty_like(lse), side)
            assert torch.equal(fo, ref_o) and torch.equal(fl, ref_l)
            o64, l64 = oracle_flat(inp)
            compare(ref_o, ref_l, o64, l64, name=f"update {step}")
        for rep in range(3):
            out.fill_(7.0)          # eager work between replays
            lse.fill_(-1.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o), (step, rep)
            assert torch.equal(lse, ref_l), (step, rep)
        note(f"graph step {step}: 3 replays bit-identical")


def test_update_rejects_and_keeps_tables():
    A = tables(210, [10, 200, 31], 32, 16)
    B = tables(211, [300, 300, 300], 32, 16)
    plan = pk.plan(A.kv_indptr, A.kv_indices, A.kv_lens, 32, 16, POOL,
                   index_capacity=len(A.kv_indices))
    before = plan.export()
    with pytest.raises(pk.PkvmlaError) as e:
        plan.update(B.kv_indptr, B.kv_indices, B.kv_lens)
    assert e.value.code == pk.EINVAL and "capacity" in str(e.value)
    bad = A.kv_indices.copy()
    bad[0] = POOL                          # page id outside the pool
    with pytest.raises(pk.PkvmlaError) as e:
        plan.update(A.kv_indptr, bad, A.kv_lens)
    assert e.value.code == pk.EINVAL
    after = plan.export()
    for f in ("wg_indptr", "units", "merges", "seq_indptr", "seq_lens", "seq_indices"):
        assert np.array_equal(getattr(before, f), getattr(after, f)), f
    # an ordinary plan accepts updates within its first table's page count
    plain = pk.plan(B.kv_indptr, B.kv_indices, B.kv_lens, 32, 16, POOL)
    assert plain.export().header[24] == 0
    plain.update(A.kv_indptr, A.kv_indices, A.kv_lens)
    dev = Dev(A)
    o, l = plain.run(dev.q_nope, dev.q_pe, dev.ckv, dev.kpe)
    torch.cuda.synchronize()
    o64, l64 = oracle_flat(A)
    compare(o, l, o64, l64, name="plain update")


def test_update_of_cascade_plan_needs_the_cascade_call():
    from mla_workloads import make_cascade
    cas = make_cascade("gu", 212, 4, 16, 16, [32], [3, 0, 20, 7])
    plan = pk.plan_for(cas)
    with pytest.raises(pk.PkvmlaError) as e:
        plan.update(cas.kv_indptr, cas.kv_indices, np.maximum(cas.kv_lens, 1))
    assert e.value.code == pk.EINVAL and "cascade" in str(e.value)
    flat = tables(213, [10, 20], 16, 16)
    fplan = pk.plan(flat.kv_indptr, flat.kv_indices, flat.kv_lens, 16, 16, POOL)
    fplan.num_groups = 1
    with pytest.raises(pk.PkvmlaError) as e:
        fplan.update_cascade([0, 2], [0, 2], cas.prefix_indices[:2], [32], flat.kv_indptr,
                             flat.kv_indices, flat.kv_lens)
    assert e.value.code == pk.EINVAL


@pytest.mark.parametrize("H,ps", [(128, 64), (16, 16), (32, 1)])
def test_graph_replay_and_update_cascade(H, ps):
    """A captured cascade run (level 0, level 1, merge) across in-place
    updates of groups' prefixes and requests' suffixes."""
    from mla_workloads import make_cascade
    from gpu_helpers import oracle_cascade
    specs = [([500, 64], [1, 40, 0, 300, 7, 64]), ([0, 1000], [30, 3, 9, 64, 1, 5]),
             ([33, 33], [5, 5, 5, 5, 5, 5])]
    if ps == 1:
        specs = [([50, 20], [1, 4, 0, 30, 7, 6]), ([0, 100], [3, 3, 9, 6, 1, 5]),
                 ([33, 33], [5, 5, 5, 5, 5, 5])]
    bundles = [make_cascade(f"gc{i}", 220 + i, 6, H, ps, pre, suf, groups=2, pool_pages=POOL)
               for i, (pre, suf) in enumerate(specs)]
    cap = max(len(b.prefix_indices) + len(b.kv_indices) for b in bundles) + 7
    A = bundles[0]
    note(f"graph cascade H={H} ps={ps} cap={cap}")

    def args(c):
        return (c.group_req_indptr, c.prefix_indptr, c.prefix_indices, c.prefix_lens,
                c.kv_indptr, c.kv_indices, c.kv_lens)

    plan = pk.plan_cascade(*args(A), H, ps, POOL, index_capacity=cap)
    assert plan.export().header[24] == 1
    dev = Dev(A)
    out = torch.empty((A.batch, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((A.batch, H), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    ref_o, ref_l = eager(plan, dev, out, lse, side)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        plan.run(dev.q_nope, dev.q_pe, dev.ckv, dev.kpe, out=out, lse=lse, stream=side)
    torch.cuda.synchronize()

    for step, inp in enumerate(bundles + [A]):
        if step > 0:
            plan.update_cascade(*args(inp), stream=side)
            load_into(dev, inp)
            torch.cuda.synchronize()
            ref_o, ref_l = eager(plan, dev, out, lse, side)
            fresh = pk.plan_cascade(*args(inp), H, ps, POOL)
            fo, fl = eager(fresh, dev, torch.empty_like(out), torch.empty_like(lse), side)
            o64, l64 = oracle_cascade(inp)
            compare(ref_o, ref_l, o64, l64, name=f"cascade update {step}")
            if fresh.export().header[31] == 0:
                # the same two-level layout: the same bits
                assert torch.equal(fo, ref_o) and torch.equal(fl, ref_l)
            else:
                # an ordinary plan may run the cascade in one launch (chained
                # suffixes): other rounding, the same attention
                compare(fo, fl, o64, l64, name=f"cascade fresh one-launch {step}")
        for rep in range(3):
            out.fill_(7.0)
            lse.fill_(-1.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o), (step, rep)
            assert torch.equal(lse, ref_l), (step, rep)
        note(f"graph cascade step {step}: 3 replays bit-identical")


@pytest.mark.parametrize("H,ps,layout", [(16, 16, "rows"), (32, 1, "rows"), (128, 64, "tokens"),
                                         (16, 64, "tokens")])
def test_graph_replay_and_update_qo(H, ps, layout):
    """Several query tokens per request: one captured run serves new page
    tables and new splits of the same 12 tokens over the same 4 requests."""
    from mla_workloads import make_qo
    from gpu_helpers import oracle_qo
    lay = pk.QO_ROW_BLOCKS if layout == "rows" else pk.QO_TOKENS
    specs = [([40, 333, 1000, 64], [3, 3, 3, 3]), ([700, 5, 129, 64], [1, 5, 2, 4]),
             ([9, 64, 6, 1200], [6, 1, 1, 4])]
    if ps == 1:
        specs = [([40, 33, 100, 64], [3, 3, 3, 3]), ([70, 5, 29, 64], [1, 5, 2, 4]),
                 ([9, 64, 6, 120], [6, 1, 1, 4])]
    pool = 400                  # pages of every bundle's pool (same tensor shapes)
    bundles = [make_qo(f"gq{i}", 220 + i, 4, H, ps, lens, qo, pool_pages=pool)
               for i, (lens, qo) in enumerate(specs)]
    cap = max(len(b.kv_indices) for b in bundles) + 7
    A = bundles[0]
    note(f"graph qo H={H} ps={ps} {layout} cap={cap}")
    plan = pk.plan_qo(A.qo_indptr, A.kv_indptr, A.kv_indices, A.kv_lens, H, ps, pool,
                      layout=lay, index_capacity=cap)
    hdr = plan.export().header
    assert hdr[24] == 1 and hdr[26] == (2 if layout == "rows" else 1)
    dev = Dev(A)
    T = int(A.qo_indptr[-1])
    out = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    ref_o, ref_l = eager(plan, dev, out, lse, side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        plan.run(dev.q_nope, dev.q_pe, dev.ckv, dev.kpe, out=out, lse=lse, stream=side)
    torch.cuda.synchronize()
    for step, inp in enumerate(bundles + [A]):
        if step > 0:
            plan.update_qo(inp.qo_indptr, inp.kv_indptr, inp.kv_indices, inp.kv_lens, stream=side)
            load_into(dev, inp)
            torch.cuda.synchronize()
            ref_o, ref_l = eager(plan, dev, out, lse, side)
            fresh = pk.plan_qo(inp.qo_indptr, inp.kv_indptr, inp.kv_indices, inp.kv_lens, H, ps,
                               pool, layout=lay)
            fo, fl = eager(fresh, dev, torch.empty_like(out), torch.empty_like(lse), side)
            assert torch.equal(fo, ref_o) and torch.equal(fl, ref_l)
        compare(ref_o, ref_l, *oracle_qo(inp), name=f"qo update {step}")
        for rep in range(3):
            out.fill_(7.0)
            lse.fill_(-1.0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_o), (step, rep)
            assert torch.equal(lse, ref_l), (step, rep)
        note(f"graph qo step {step}: 3 replays bit-identical")


def test_update_qo_rejects():
    from mla_workloads import make_qo
    A = make_qo("gr", 230, 3, 16, 16, [50, 60, 70], [2, 3, 4], pool_pages=POOL)
    plan = pk.plan_qo(A.qo_indptr, A.kv_indptr, A.kv_indices, A.kv_lens, 16, 16, POOL,
                      index_capacity=len(A.kv_indices) + 4)
    before = plan.export()
    with pytest.raises(ValueError, match="query tokens"):
        plan.update_qo([0, 2, 3, 5], A.kv_indptr, A.kv_indices, A.kv_lens)   # 5 tokens, not 9
    lens = A.kv_lens.copy()
    lens[2] = 3                                        # 4 tokens but kv_len 3
    with pytest.raises(pk.PkvmlaError) as e:
        plan.update_qo(A.qo_indptr, A.kv_indptr, A.kv_indices, lens)
    assert e.value.code == pk.EINVAL
    # the flat update refuses the plan
    ip, ix, ln = (np.ascontiguousarray(x, dtype=np.int32)
                  for x in (A.kv_indptr, A.kv_indices, A.kv_lens))
    assert pk._lib.pkvmla_plan_update(plan._h, pk._ptr(ip), pk._ptr(ix), pk._ptr(ln), None) == pk.EINVAL
    after = plan.export()
    for f in ("wg_indptr0", "units0", "merges", "slot_list", "seq_lens", "seq_indices"):
        assert np.array_equal(getattr(before, f), getattr(after, f)), f
