"""CPU pins of the oracle for several new query tokens per request (causal
among them): the vLLM "[V1][Core] FlashInfer attention backend for V1" page
runs prefill and decode requests through one batched wrapper; a request's new
tokens are its last ones, and each attends every earlier token and itself."""

import math

import numpy as np
import pytest
import torch

import oracle
from mla_workloads import make_qo, make_flat, permute_pages


def _qo(inp):
    return oracle.attend_qo(inp.q_nope, inp.q_pe, inp.ckv, inp.kpe, inp.qo_indptr, inp.kv_indptr,
                            inp.kv_indices, inp.kv_lens, inp.page_size, sm_scale=inp.sm_scale)


def _rows(inp, b):
    """Key rows [L, 576] and value rows [L, 512] of request b, fp64."""
    L = int(inp.kv_lens[b])
    t = np.arange(L)
    pages = inp.kv_indices[inp.kv_indptr[b] + t // inp.page_size]
    slots = t % inp.page_size
    c = oracle.bf16_to_f64(inp.ckv[pages, slots])
    r = oracle.bf16_to_f64(inp.kpe[pages, slots])
    return np.concatenate([c, r], axis=1), c


def test_matches_torch_sdpa_with_position_mask():
    """Library pin: torch fp64 SDPA, all query rows of a request at once with a
    boolean mask built from token positions (row of token j may attend key t
    iff t <= L - n + j)."""
    inp = make_qo("p", 31, 3, 16, 16, [9, 40, 77], [2, 4, 3])
    out, lse = _qo(inp)
    scale = 1.0 / math.sqrt(576)
    for b in range(inp.batch):
        n = int(inp.qo_indptr[b + 1] - inp.qo_indptr[b])
        L = int(inp.kv_lens[b])
        k, v = _rows(inp, b)
        rows = slice(int(inp.qo_indptr[b]), int(inp.qo_indptr[b + 1]))
        q = np.concatenate([oracle.bf16_to_f64(inp.q_nope[rows]), oracle.bf16_to_f64(inp.q_pe[rows])],
                           axis=2).reshape(n * 16, 576)
        pos = np.repeat(L - n + np.arange(n), 16)                       # position of each row
        mask = torch.from_numpy(np.arange(L)[None, :] <= pos[:, None])
        qt, kt, vt = (torch.from_numpy(x)[None, None] for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                               scale=scale)[0, 0].numpy()
        s = scale * (torch.from_numpy(q) @ torch.from_numpy(k).T)
        ref_lse = torch.logsumexp(s.masked_fill(~mask, float("-inf")), dim=1).numpy()
        np.testing.assert_allclose(out[rows].reshape(n * 16, 512), ref, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse[rows].reshape(n * 16), ref_lse, atol=1e-12, rtol=0)


def test_fsum_brute_force():
    inp = make_qo("f", 32, 2, 2, 4, [6, 3], [3, 2])
    out, lse = _qo(inp)
    scale = 1.0 / math.sqrt(576)
    for b in range(inp.batch):
        n = int(inp.qo_indptr[b + 1] - inp.qo_indptr[b])
        L = int(inp.kv_lens[b])
        k, v = _rows(inp, b)
        for j in range(n):
            row = int(inp.qo_indptr[b]) + j
            for h in range(2):
                q = list(oracle.bf16_to_f64(inp.q_nope[row, h])) + list(oracle.bf16_to_f64(inp.q_pe[row, h]))
                vis = range(L - n + j + 1)
                s = [scale * math.fsum(qi * ki for qi, ki in zip(q, k[t])) for t in vis]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                z = math.fsum(w)
                assert abs(lse[row, h] - (mx + math.log(z))) < 1e-12
                for d in (0, 7, 511):
                    o = math.fsum(wi * v[t, d] for wi, t in zip(w, vis)) / z
                    assert abs(out[row, h, d] - o) < 1e-12


def test_one_query_token_is_flat_decode():
    inp = make_qo("o", 33, 4, 16, 16, [1, 17, 64, 200], [1, 1, 1, 1])
    out, lse = _qo(inp)
    fo, fl = oracle.attend_flat(inp.q_nope, inp.q_pe, inp.ckv, inp.kpe, inp.kv_indptr,
                                inp.kv_indices, inp.kv_lens, inp.page_size)
    np.testing.assert_allclose(out, fo, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse, fl, atol=1e-13, rtol=0)


def test_last_token_sees_everything_and_first_sees_prefix():
    inp = make_qo("l", 34, 2, 16, 8, [30, 12], [4, 12])
    out, lse = _qo(inp)
    for b in range(2):
        n = int(inp.qo_indptr[b + 1] - inp.qo_indptr[b])
        L = int(inp.kv_lens[b])
        for j, length in ((n - 1, L), (0, L - n + 1)):
            row = int(inp.qo_indptr[b]) + j
            one = make_flat("x", 0, 1, 16, 8, [length], pool_pages=inp.num_pages)
            ip = np.array([0, inp.kv_indptr[b + 1] - inp.kv_indptr[b]], np.int32)
            fo, fl = oracle.attend_flat(inp.q_nope[row:row + 1], inp.q_pe[row:row + 1], inp.ckv,
                                        inp.kpe, ip, inp.kv_indices[inp.kv_indptr[b]:inp.kv_indptr[b + 1]],
                                        np.array([length], np.int32), inp.page_size)
            np.testing.assert_allclose(out[row], fo[0], atol=1e-13, rtol=0)
            np.testing.assert_allclose(lse[row], fl[0], atol=1e-13, rtol=0)


def test_causal_boundary_matters():
    """Moving the boundary by one token changes the result (the masked
    positions are not dead inputs)."""
    inp = make_qo("c", 35, 1, 16, 16, [50], [3])        # 4 pages hold 64 slots
    out, _ = _qo(inp)
    o2, _ = _qo(inp.replace(kv_lens=inp.kv_lens + 1))
    assert np.abs(o2 - out).max() > 1e-6


def test_page_permutation_invariance():
    inp = make_qo("pp", 36, 3, 16, 16, [20, 33, 64], [2, 5, 1])
    out, lse = _qo(inp)
    o2, l2 = _qo(permute_pages(inp, seed=5))
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)


def test_fp8_caches_reduce_to_flat_fp8_at_each_causal_length():
    """With E4M3 caches, query token j of request b equals the flat oracle's
    fp8 decode of that token's query over the first kv_len - n + 1 + j tokens
    of b's pages (the flat fp8 path has its own pins)."""
    from mla_workloads import quantize_kv_fp8
    inp = quantize_kv_fp8(make_qo("q8", 35, 3, 16, 8, [7, 40, 65], [3, 4, 2]), 0.02, 0.03)
    sc = (inp.ckv_scale, inp.kpe_scale)
    out, lse = oracle.attend_qo(inp.q_nope, inp.q_pe, inp.ckv8, inp.kpe8, inp.qo_indptr,
                                inp.kv_indptr, inp.kv_indices, inp.kv_lens, inp.page_size,
                                kv_scales=sc)
    ref_b, _ = oracle.attend_qo(inp.q_nope, inp.q_pe, inp.ckv, inp.kpe, inp.qo_indptr,
                                inp.kv_indptr, inp.kv_indices, inp.kv_lens, inp.page_size)
    assert not np.allclose(out, ref_b, atol=1e-9)       # the codes, not the bf16 values
    for b in range(inp.batch):
        n = int(inp.qo_indptr[b + 1] - inp.qo_indptr[b])
        for j in range(n):
            row = int(inp.qo_indptr[b]) + j
            L = int(inp.kv_lens[b]) - n + 1 + j
            o, l = oracle.attend_flat(inp.q_nope[row:row + 1], inp.q_pe[row:row + 1], inp.ckv8,
                                      inp.kpe8, np.array([0, inp.kv_indptr[b + 1] - inp.kv_indptr[b]]),
                                      inp.kv_indices[inp.kv_indptr[b]:inp.kv_indptr[b + 1]],
                                      np.array([L]), inp.page_size, kv_scales=sc)
            np.testing.assert_allclose(out[row], o[0], atol=1e-12, rtol=0)
            np.testing.assert_allclose(lse[row], l[0], atol=1e-12, rtol=0)
