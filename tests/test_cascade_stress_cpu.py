"""CPU: the cascade stress inputs do what they claim, and the oracle's
two-level result still equals flat attention on them (the V1 FlashInfer
backend page requires cascade and normal attention to agree)."""

import numpy as np
import pytest

import oracle
from mla_workloads import make_cascade, stress_variant_cascade, poison_unreferenced, STRESS_KINDS


def _cascade(cas):
    return oracle.attend_cascade(cas.q_nope, cas.q_pe, cas.ckv, cas.kpe, cas.page_size,
                                 cas.group_req_indptr, cas.prefix_indptr, cas.prefix_indices,
                                 cas.prefix_lens, cas.kv_indptr, cas.kv_indices, cas.kv_lens,
                                 sm_scale=cas.sm_scale)


def _flat(f):
    return oracle.attend_flat(f.q_nope, f.q_pe, f.ckv, f.kpe, f.kv_indptr, f.kv_indices,
                              f.kv_lens, f.page_size, sm_scale=f.sm_scale)


@pytest.mark.parametrize("kind", STRESS_KINDS)
def test_cascade_stress_equals_flat(kind):
    base = make_cascade("p", 7, 5, 16, 16, [64, 32], [0, 9, 40, 1, 17], groups=2)
    cas = stress_variant_cascade(base, kind)
    o, l = _cascade(cas)
    fo, fl = _flat(cas.flat_view())
    np.testing.assert_allclose(o, fo, atol=1e-12, rtol=0)
    np.testing.assert_allclose(l, fl, atol=1e-11, rtol=0)
    if kind == "negative":
        assert l.max() < -50            # every logit near -80
    if kind == "qx8":
        assert np.all(np.isfinite(o))


def test_cascade_needle_dominates():
    base = make_cascade("n", 8, 4, 16, 16, [48], [5, 9, 30, 2], groups=1)
    cas = stress_variant_cascade(base, "needle")
    o, l = _cascade(cas)
    for b in range(cas.batch):
        h = b % cas.num_heads
        # the planted suffix row carries nearly all of head h's probability mass
        rows = cas.ckv[cas.kv_indices[cas.kv_indptr[b]:cas.kv_indptr[b + 1]]].reshape(-1, 512)
        rows = oracle.bf16_to_f64(rows[:cas.kv_lens[b]])
        best = np.abs(rows - o[b, h]).max(axis=1).min()
        assert best < 0.05 * np.abs(o[b, h]).max(), (b, best)


def test_cascade_poison_leaves_result_unchanged():
    cas = make_cascade("q", 9, 4, 16, 16, [37], [0, 5, 17, 1], groups=1)
    o1, l1 = _cascade(cas)
    o2, l2 = _cascade(poison_unreferenced(cas))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert np.isnan(oracle.bf16_to_f64(poison_unreferenced(cas).ckv)).any()
