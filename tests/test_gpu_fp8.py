"""fp8 (OCP E4M3) KV caches with bf16 queries on the GPU, against the fp64
oracle's E4M3 path.

Reading (the pages give none): one scale per cache tensor, a token's value
being scale * code value, dequantized before the dot products.  The vLLM
page "[V1][Core] FlashInfer attention backend for V1" lists a KV-cache dtype
other than the query dtype as the limitation of its cascade path; here flat
and cascade plans both take fp8 caches."""

import numpy as np
import pytest
import torch

from mla_workloads import (make_flat, make_cascade, make_config, make_qo, stress_variant,
                           quantize_kv_fp8, poison_unreferenced, permute_pages)
from gpu_helpers import Dev, run_gpu, oracle_flat, oracle_cascade, oracle_qo, compare, bits_of

pytestmark = pytest.mark.gpu

import paged_kv_mla_amd as pk  # noqa: E402


def note(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.init()
    yield


def q8(inp, **kw):
    return quantize_kv_fp8(inp, **kw)


FLAT = {
    "tiny": lambda: q8(make_config("tiny")),
    "h16_ps1": lambda: q8(make_flat("e1", 601, 6, 16, 1, [1, 2, 31, 32, 33, 257])),
    "h32_ps16": lambda: q8(make_flat("e2", 602, 5, 32, 16, [1, 17, 64, 200, 513])),
    "h64_ps64": lambda: q8(make_flat("e3", 603, 5, 64, 64, [1, 63, 64, 65, 1000])),
    "h128_ps64_split": lambda: q8(make_flat("e4", 604, 4, 128, 64, [3, 700, 4096, 9000])),
    "h128_ps8": lambda: q8(make_flat("e5", 605, 4, 128, 8, [9, 40, 161, 333])),
    "h16_unequal_scales": lambda: q8(make_flat("e6", 606, 3, 16, 16, [5, 77, 300]),
                                     ckv_scale=3.0 / 448, kpe_scale=7.0 / 448),
}


@pytest.mark.parametrize("name", sorted(FLAT))
def test_fp8_flat(name):
    inp = FLAT[name]()
    note(f"fp8 {name} scales {inp.ckv_scale:.4g} {inp.kpe_scale:.4g}")
    out, lse = run_gpu(pk.plan_for(inp), Dev(inp, fp8=True))
    compare(out, lse, *oracle_flat(inp, fp8=True), name=f"fp8 {name}")


@pytest.mark.parametrize("kind", ["qx8", "needle", "increasing", "negative"])
def test_fp8_stress(kind):
    inp = q8(stress_variant(make_flat("e7", 607, 4, 128, 64, [33, 300, 1500, 64]), kind))
    note(f"fp8 stress {kind}")
    out, lse = run_gpu(pk.plan_for(inp), Dev(inp, fp8=True))
    compare(out, lse, *oracle_flat(inp, fp8=True), name=f"fp8 stress {kind}")


@pytest.mark.parametrize("H,ps", [(16, 16), (128, 64), (32, 1)])
def test_fp8_poison_permutation_and_determinism(H, ps):
    base = make_flat(f"e8{H}", 608 + H, 4, H, ps, [1, 15, 64, 333], extra_pages=1)
    inp = q8(base)
    sc = dict(ckv_scale=inp.ckv_scale, kpe_scale=inp.kpe_scale)
    note(f"fp8 invariants H{H} ps{ps}")
    plan = pk.plan_for(inp)
    o1, l1 = run_gpu(plan, Dev(inp, fp8=True))
    o1, l1 = bits_of(o1), l1.cpu().numpy().copy()
    o2, l2 = run_gpu(plan, Dev(inp, fp8=True))
    assert np.array_equal(bits_of(o2), o1) and np.array_equal(l2.cpu().numpy(), l1)
    pz = q8(poison_unreferenced(base), **sc)          # NaN codes in every unattended slot
    assert ((pz.ckv8 & 0x7F) == 0x7F).any()
    assert np.array_equal(np.isin(pz.ckv8, [0x7F, 0xFF]), ~np.isin(inp.ckv8, [0x7F, 0xFF]) & np.isin(pz.ckv8, [0x7F, 0xFF]))
    o3, l3 = run_gpu(pk.plan_for(pz), Dev(pz, fp8=True))
    assert np.array_equal(bits_of(o3), o1) and np.array_equal(l3.cpu().numpy(), l1)
    pp = q8(permute_pages(base, seed=13), **sc)
    o4, l4 = run_gpu(pk.plan_for(pp), Dev(pp, fp8=True))
    assert np.array_equal(bits_of(o4), o1) and np.array_equal(l4.cpu().numpy(), l1)


@pytest.mark.parametrize("H,ps", [(128, 64), (16, 1)])
def test_fp8_combined_cache_views(H, ps):
    """The two views of one uint8 [pages, page_size, 576] cache (row stride
    576 bytes) give the same bits as two packed fp8 caches."""
    inp = q8(make_flat(f"e9{H}", 609 + ps, 4, H, ps, [1, 31, 70, 200] if ps == 1 else
                       [1, 33, 100, 2049]))
    note(f"fp8 combined H{H} ps{ps}")
    d = Dev(inp, fp8=True)
    plan = pk.plan_for(inp)
    o1, l1 = run_gpu(plan, d)
    comb = torch.cat([d.ckv, d.kpe], dim=2).contiguous()
    o2, l2 = plan.run(d.q_nope, d.q_pe, comb[..., :512], comb[..., 512:], kv_scales=d.kv_scales)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("H", [16, 128])
def test_fp8_cascade(H):
    cas = q8(make_cascade(f"ec{H}", 610 + H, 6, H, 16, [40, 300], [1, 20, 0, 33, 5, 300],
                          groups=2))
    note(f"fp8 cascade H{H}")
    out, lse = run_gpu(pk.plan_for(cas), Dev(cas, fp8=True))
    compare(out, lse, *oracle_cascade(cas, fp8=True), name=f"fp8 cascade H{H}")


def test_fp8_full_size_deepseek():
    """Every request of the DeepSeek-shaped workload with fp8 caches."""
    inp = q8(make_config("deepseek"))
    note(f"fp8 full deepseek tokens={inp.total_tokens}")
    out, lse = run_gpu(pk.plan_for(inp), Dev(inp, fp8=True))
    st = compare(out, lse, *oracle_flat(inp, fp8=True), name="fp8 deepseek")
    note(f"fp8 deepseek stats {st}")


def test_fp8_rejects():
    inp = q8(make_flat("er", 620, 2, 16, 16, [5, 9]))
    d = Dev(inp, fp8=True)
    plan = pk.plan_for(inp)
    for bad in ((0.0, 1.0), (1.0, float("nan")), (-1.0, 1.0), (float("inf"), 1.0)):
        with pytest.raises(pk.PkvmlaError) as e:
            plan.run(d.q_nope, d.q_pe, d.ckv, d.kpe, kv_scales=bad)
        assert e.value.code == pk.EINVAL
    b = Dev(inp)                                     # bf16 caches with fp8 scales
    with pytest.raises(ValueError):
        plan.run(b.q_nope, b.q_pe, b.ckv, b.kpe, kv_scales=(1.0, 1.0))
    with pytest.raises(ValueError):                  # fp8 caches without scales
        plan.run(d.q_nope, d.q_pe, d.ckv, d.kpe)


@pytest.mark.parametrize("layout", ["tokens", "rows"])
def test_fp8_several_query_tokens(layout):
    """fp8 caches under a plan with several query tokens per request, in both
    layouts (row blocks include pieces some tokens see nothing of)."""
    inp = q8(make_qo("e8", 611, 3, 16, 16, [101, 100, 90], [40, 1, 6]))
    note(f"fp8 qo {layout}")
    lay = pk.QO_ROW_BLOCKS if layout == "rows" else pk.QO_TOKENS
    out, lse = run_gpu(pk.plan_for(inp, qo_layout=lay), Dev(inp, fp8=True))
    compare(out, lse, *oracle_qo(inp, fp8=True), name=f"fp8 qo {layout}")
