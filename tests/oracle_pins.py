"""Pins that tie the fp64 oracle to something other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
the pinned fact.  ``test_oracle_pins.py`` runs them as tests and
``test_oracle_mutations.py`` plants mistakes in the oracle to show that every
planted mistake is caught by at least one pin.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle
import oracle.mla_decode as od
from mla_workloads import make_flat, make_cascade, f32_to_bf16_bits, permute_pages, poison_unreferenced

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_derived_decode.json")


def small_flat(seed=5, lens=(1, 17, 64, 200), heads=16, ps=16, pool=64, extra=0):
    return make_flat("pin", seed, len(lens), heads, ps, list(lens), pool_pages=pool, extra_pages=extra)


def run_flat(inp, **kw):
    return oracle.attend_flat(inp.q_nope, inp.q_pe, inp.ckv, inp.kpe, inp.kv_indptr,
                              inp.kv_indices, inp.kv_lens, inp.page_size,
                              sm_scale=kw.get("sm_scale", inp.sm_scale))


def _bits_to_f64(bits):
    # independent of the oracle's own widening: via torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------- library pin
def pin_sdpa(inp=None):
    """torch fp64 scaled_dot_product_attention, the H heads as H query rows of a
    single head, K = [ckv | kpe] and V = ckv gathered by a page walk written
    with explicit per-page loops."""
    inp = inp or small_flat()
    out, lse = run_flat(inp)
    scale = 1.0 / math.sqrt(512 + 64) if inp.sm_scale is None else inp.sm_scale
    ps = inp.page_size
    for b in range(inp.batch):
        L = int(inp.kv_lens[b])
        rows_c, rows_r = [], []
        for j, page in enumerate(inp.kv_indices[inp.kv_indptr[b]:inp.kv_indptr[b + 1]]):
            for slot in range(ps):
                if j * ps + slot < L:
                    rows_c.append(inp.ckv[page, slot])
                    rows_r.append(inp.kpe[page, slot])
        c = torch.from_numpy(_bits_to_f64(np.stack(rows_c)))
        r = torch.from_numpy(_bits_to_f64(np.stack(rows_r)))
        q = torch.cat([torch.from_numpy(_bits_to_f64(inp.q_nope[b])),
                       torch.from_numpy(_bits_to_f64(inp.q_pe[b]))], dim=1)
        k = torch.cat([c, r], dim=1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            q[None, None], k[None, None], c[None, None], scale=scale)[0, 0]
        ref_lse = torch.logsumexp(scale * (q @ k.T), dim=1)
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[b], ref_lse.numpy(), rtol=0, atol=1e-12)


# -------------------------------------------------- non-absorbed brute force
def pin_nonabsorbed(seed=3, H=4, L=9, d=32, dv=48):
    """Absorbed attention (one shared latent row per token) equals ordinary
    multi-head attention with per-head up-projections: keys [W_UK c_t | r_t],
    values W_UV c_t, queries [q_orig | q_pe], when q_nope = W_UK^T q_orig and the
    output is mapped back through W_UV."""
    rng = np.random.default_rng(seed)
    c = rng.standard_normal((L, 512)) * 0.5
    r = rng.standard_normal((L, 64)) * 0.5
    W_UK = rng.standard_normal((H, d, 512)) * 0.05
    W_UV = rng.standard_normal((H, dv, 512)) * 0.05
    q_orig = rng.standard_normal((H, d))
    q_pe = rng.standard_normal((H, 64))
    scale = 1.0 / math.sqrt(512 + 64)
    q_nope = np.einsum("hdk,hd->hk", W_UK, q_orig)
    out_abs, lse_abs = oracle.attend_rows(np.concatenate([q_nope, q_pe], 1),
                                          np.concatenate([c, r], 1), c, scale)
    for h in range(H):
        keys = np.concatenate([c @ W_UK[h].T, r], 1)            # [L, d+64]
        vals = c @ W_UV[h].T                                    # [L, dv]
        qh = np.concatenate([q_orig[h], q_pe[h]])
        s = [scale * math.fsum(qh * keys[t]) for t in range(L)]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        z = math.fsum(w)
        ref = np.array([math.fsum(w[t] * vals[t, j] for t in range(L)) / z for j in range(dv)])
        np.testing.assert_allclose(W_UV[h] @ out_abs[h], ref, rtol=0, atol=1e-10)
        assert abs(lse_abs[h] - (m + math.log(z))) < 1e-10


# --------------------------------------------------- python-float brute force
def pin_fsum(inp=None, heads=(0, 7, 15)):
    """Pure-python loops with math.fsum on the small workload."""
    inp = inp or small_flat()
    out, lse = run_flat(inp)
    scale = 1.0 / math.sqrt(512 + 64) if inp.sm_scale is None else inp.sm_scale
    ps = inp.page_size
    C = _bits_to_f64(inp.ckv)
    R = _bits_to_f64(inp.kpe)
    QN = _bits_to_f64(inp.q_nope)
    QP = _bits_to_f64(inp.q_pe)
    for b in range(inp.batch):
        L = int(inp.kv_lens[b])
        toks = []
        for j in range(int(inp.kv_indptr[b + 1] - inp.kv_indptr[b])):
            for slot in range(ps):
                if len(toks) < L:
                    toks.append((int(inp.kv_indices[inp.kv_indptr[b] + j]), slot))
        for h in heads:
            qn = QN[b, h].tolist()
            qp = QP[b, h].tolist()
            s = []
            for (p, sl) in toks:
                s.append(scale * math.fsum([a * x for a, x in zip(qn, C[p, sl].tolist())] +
                                           [a * x for a, x in zip(qp, R[p, sl].tolist())]))
            m = max(s)
            w = [math.exp(x - m) for x in s]
            z = math.fsum(w)
            assert abs(lse[b, h] - (m + math.log(z))) < 1e-12
            for dim in (0, 1, 255, 511):
                ref = math.fsum(w[i] * C[p, sl, dim] for i, (p, sl) in enumerate(toks)) / z
                assert abs(out[b, h, dim] - ref) < 1e-12


# ------------------------------------------------------------- closed forms
def pin_closed_forms():
    # L = 1: the output is exactly the single ckv row, lse the single scaled logit
    inp = small_flat(seed=11, lens=(1, 1, 1), heads=16, ps=16, pool=8)
    out, lse = run_flat(inp)
    for b in range(3):
        p = inp.kv_indices[inp.kv_indptr[b]]
        c = _bits_to_f64(inp.ckv[p, 0])
        assert np.array_equal(out[b], np.broadcast_to(c, out[b].shape))
        q = np.concatenate([_bits_to_f64(inp.q_nope[b]), _bits_to_f64(inp.q_pe[b])], 1)
        k = np.concatenate([c, _bits_to_f64(inp.kpe[p, 0])])
        np.testing.assert_allclose(lse[b], (q @ k) / 24.0, rtol=0, atol=1e-13)
    # all ckv rows equal: out equals that row whatever the weights
    inp = small_flat(seed=12, lens=(40, 7), heads=16, ps=16, pool=8)
    ckv = inp.ckv.copy()
    ckv[:] = inp.ckv[0, 0]
    out, _ = run_flat(inp.replace(ckv=ckv))
    np.testing.assert_allclose(out, np.broadcast_to(_bits_to_f64(inp.ckv[0, 0]), out.shape),
                               rtol=1e-14, atol=1e-15)
    # q = 0: uniform weights, out = mean of the rows, lse = ln L
    inp = small_flat(seed=13, lens=(33, 5), heads=16, ps=16, pool=8)
    z = inp.replace(q_nope=np.zeros_like(inp.q_nope), q_pe=np.zeros_like(inp.q_pe))
    out, lse = run_flat(z)
    for b in range(2):
        L = int(inp.kv_lens[b])
        rows = [_bits_to_f64(inp.ckv[inp.kv_indices[inp.kv_indptr[b] + t // 16], t % 16])
                for t in range(L)]
        np.testing.assert_allclose(out[b, 3], np.mean(rows, axis=0), rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse[b], math.log(L), rtol=0, atol=1e-14)


# -------------------------------------------------------------- golden file
def _golden_inputs(case, ckv_dim, kpe_dim):
    H, ps, P = case["num_heads"], case["page_size"], case["num_pages"]
    qn = np.zeros((1, H, ckv_dim), np.float32)
    qp = np.zeros((1, H, kpe_dim), np.float32)
    ckv = np.zeros((P, ps, ckv_dim), np.float32)
    kpe = np.zeros((P, ps, kpe_dim), np.float32)
    for h, d, v in case["q_nope"]:
        qn[0, h, d] = v
    for h, d, v in case["q_pe"]:
        qp[0, h, d] = v
    for p, s, d, v in case["ckv"]:
        ckv[p, s, d] = v
    for p, s, d, v in case["kpe"]:
        kpe[p, s, d] = v
    idx = np.asarray(case["kv_indices"], np.int32)
    return dict(q_nope=f32_to_bf16_bits(qn), q_pe=f32_to_bf16_bits(qp),
                ckv=f32_to_bf16_bits(ckv), kpe=f32_to_bf16_bits(kpe),
                kv_indptr=np.asarray([0, len(idx)], np.int32), kv_indices=idx,
                kv_lens=np.asarray([case["kv_len"]], np.int32), page_size=ps,
                sm_scale=case["sm_scale"])


def golden_cases():
    with open(GOLDEN) as f:
        g = json.load(f)
    return [(c, _golden_inputs(c, g["ckv_dim"], g["kpe_dim"])) for c in g["cases"]]


def pin_golden():
    for case, a in golden_cases():
        out, lse = oracle.attend_flat(**a)
        exp = np.zeros_like(out[0])
        for h, d, v in case["out"]:
            exp[h, d] = v
        np.testing.assert_allclose(out[0], exp, rtol=0, atol=1e-14, err_msg=case["name"])
        np.testing.assert_allclose(lse[0], case["lse"], rtol=0, atol=1e-14, err_msg=case["name"])


# --------------------------------------------------------------- invariants
def pin_invariants():
    inp = small_flat(seed=21)
    out, lse = run_flat(inp)
    # physical page permutation changes nothing (same values, same order)
    o2, l2 = run_flat(permute_pages(inp, seed=5))
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)
    # NaN in every slot no request attends changes nothing
    o3, l3 = run_flat(poison_unreferenced(inp))
    assert np.array_equal(out, o3) and np.array_equal(lse, l3)
    # head permutation equivariance
    perm = np.random.default_rng(0).permutation(inp.num_heads)
    o4, l4 = run_flat(inp.replace(q_nope=inp.q_nope[:, perm], q_pe=inp.q_pe[:, perm]))
    assert np.array_equal(o4, out[:, perm]) and np.array_equal(l4, lse[:, perm])
    # extra trailing pages in a request's list are never read
    ext = small_flat(seed=21, extra=2)
    o5, l5 = run_flat(poison_unreferenced(ext))
    assert np.all(np.isfinite(o5)) and np.all(np.isfinite(l5))


def pin_split_merge():
    inp = small_flat(seed=31)
    out, lse = run_flat(inp)
    rng = np.random.default_rng(1)
    splits = []
    for L in inp.kv_lens:
        k = min(int(L) - 1, 3)
        splits.append(sorted(rng.choice(np.arange(1, int(L)), size=k, replace=False)) if k > 0 else [])
    o2, l2 = oracle.attend_flat_split(inp.q_nope, inp.q_pe, inp.ckv, inp.kpe, inp.kv_indptr,
                                      inp.kv_indices, inp.kv_lens, inp.page_size, splits)
    np.testing.assert_allclose(o2, out, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2, lse, rtol=0, atol=1e-12)
    # the empty state is the identity of the merge
    o = np.random.default_rng(2).standard_normal((3, 512))
    l = np.array([0.3, -2.0, 5.0])
    mo, ml = oracle.merge_states([(o, l), (np.zeros_like(o), np.full(3, -np.inf))])
    np.testing.assert_allclose(mo, o, rtol=0, atol=1e-15)
    np.testing.assert_allclose(ml, l, rtol=0, atol=1e-15)


def pin_cascade_equals_flat():
    for groups, prefix, suffix in ((1, 64, [3, 0, 40, 17]), (2, [32, 48], [1, 20, 0, 33, 5])):
        cas = make_cascade("pin", 41 + groups, len(suffix), 16, 16, prefix, suffix, groups=groups)
        out, lse = oracle.attend_cascade(cas.q_nope, cas.q_pe, cas.ckv, cas.kpe, cas.page_size,
                                         cas.group_req_indptr, cas.prefix_indptr,
                                         cas.prefix_indices, cas.prefix_lens, cas.kv_indptr,
                                         cas.kv_indices, cas.kv_lens)
        fo, fl = run_flat(cas.flat_view())
        np.testing.assert_allclose(out, fo, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, fl, rtol=0, atol=1e-12)


def pin_gather():
    inp = small_flat(seed=51)
    rows = oracle.gather_ref(inp.ckv, inp.kpe, inp.kv_indptr, inp.kv_indices, inp.kv_lens,
                             inp.page_size)
    ps = inp.page_size
    i = 0
    for b in range(inp.batch):
        pages = inp.kv_indices[inp.kv_indptr[b]:inp.kv_indptr[b + 1]]
        for t in range(int(inp.kv_lens[b])):
            p = pages[t // ps]
            assert np.array_equal(rows[i, :512], inp.ckv[p, t % ps])
            assert np.array_equal(rows[i, 512:], inp.kpe[p, t % ps])
            i += 1
    assert i == rows.shape[0]


ALL_PINS = [pin_sdpa, pin_nonabsorbed, pin_fsum, pin_closed_forms, pin_golden,
            pin_invariants, pin_split_merge, pin_cascade_equals_flat, pin_gather]
