"""GPU: the allocation-free run (pkvmla_run_noalloc, split workspace in the
library's static per-device scratch) against pkvmla_run of the same plan.

Two calls in a row, the second with a smaller input: bitwise equal to the
ordinary run and within the oracle's bar.  A plan whose partial states exceed
the scratch is refused before any launch.
"""

import numpy as np
import pytest
import torch

# a plain import: a library that fails to build or load fails this suite
import paged_kv_mla_amd as pk
from mla_workloads import make_flat
from gpu_helpers import Dev, oracle_flat, compare, bits_of

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield


def _both(inp):
    plan = pk.plan_for(inp)
    d = Dev(inp)
    B, H = inp.batch, inp.num_heads
    o1, l1 = plan.run(d.q_nope, d.q_pe, d.ckv, d.kpe)
    o2 = torch.full((B, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
    l2 = torch.full((B, H), float("nan"), dtype=torch.float32, device="cuda")
    plan.run_noalloc_ptrs(d.q_nope.data_ptr(), d.q_pe.data_ptr(), d.ckv.data_ptr(),
                          d.kpe.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                          int(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return plan, (o1, l1), (o2, l2)


def test_noalloc_matches_run_twice_second_smaller():
    big = make_flat("na1", 301, 6, 128, 64, [3000, 100, 2500, 700, 4000, 1])
    small = make_flat("na2", 302, 3, 16, 16, [5, 300, 40])
    for inp in (big, small):
        plan, (o1, l1), (o2, l2) = _both(inp)
        ex = plan.export()
        note(f"noalloc {inp.name}: {ex.units.shape[0]} units, {ex.merges.shape[0]} merged requests")
        assert ex.merges.shape[0] > 0          # the merge reads the static workspace too
        assert np.array_equal(bits_of(o1), bits_of(o2))
        assert torch.equal(l1, l2)
        ref_o, ref_l = oracle_flat(inp)
        compare(o2, l2, ref_o, ref_l, name=f"noalloc {inp.name}")


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    B = 500
    indptr = np.arange(B + 1, dtype=np.int32)
    indices = np.arange(B, dtype=np.int32)
    lens = np.ones(B, np.int32)
    # a capacity plan sizes its workspace for batch + lanes slots of 128 heads
    plan = pk.plan(indptr, indices, lens, 128, 64, B, index_capacity=2 * B)
    z = torch.zeros(1, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(pk.PkvmlaError) as e:
        plan.run_noalloc_ptrs(z.data_ptr(), z.data_ptr(), z.data_ptr(), z.data_ptr(),
                              z.data_ptr(), z.data_ptr(), 0)
    assert e.value.code == pk.EUNSUPPORTED and "scratch" in str(e.value)


def test_noalloc_row_blocks_of_query_tokens():
    """A row-block plan of several query tokens per request (partial rows at
    an offset from each block's first row, per-token merges over slot lists)
    through the static scratch: bitwise equal to the ordinary run."""
    from mla_workloads import make_qo
    from gpu_helpers import oracle_qo
    inp = make_qo("na3", 303, 4, 16, 16, [101, 900, 64, 2000], [40, 3, 1, 6])
    plan = pk.plan_for(inp, qo_layout=pk.QO_ROW_BLOCKS)
    ex = plan.export()
    assert int(ex.header[26]) == 2 and ex.merges.shape[0] > 0
    d = Dev(inp)
    T, H = int(inp.qo_indptr[-1]), inp.num_heads
    o1, l1 = plan.run(d.q_nope, d.q_pe, d.ckv, d.kpe)
    for rep in range(2):
        o2 = torch.full((T, H, 512), float("nan"), dtype=torch.bfloat16, device="cuda")
        l2 = torch.full((T, H), float("nan"), dtype=torch.float32, device="cuda")
        plan.run_noalloc_ptrs(d.q_nope.data_ptr(), d.q_pe.data_ptr(), d.ckv.data_ptr(),
                              d.kpe.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                              int(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        note(f"noalloc qo rows, call {rep}")
        assert np.array_equal(bits_of(o1), bits_of(o2))
        assert torch.equal(l1, l2)
    compare(o2, l2, *oracle_qo(inp), name="noalloc qo rows")
