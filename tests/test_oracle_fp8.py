"""Pins of the oracle's fp8 (OCP E4M3) KV-cache path, CPU only.

The pages only name the limitation (the V1 FlashInfer backend page: the KV
cache dtype cannot differ from the query dtype in cascade mode); the reading
here is per-tensor scales with dequantization before the dot products, bf16
queries.  The E4M3 values are fixed by the OCP OFP8 format."""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from mla_workloads import make_flat, make_cascade, quantize_kv_fp8

GOLD = os.path.join(os.path.dirname(__file__), "golden", "e4m3_ocp_values.json")


def test_e4m3_hand_listed_values():
    cases = json.load(open(GOLD))["cases"]
    codes = np.array([int(c["code"], 16) for c in cases], np.uint8)
    got = oracle.e4m3_to_f64(codes)
    for c, g in zip(cases, got):
        want = float(c["value"])
        if math.isnan(want):
            assert math.isnan(g), c
        else:
            assert g == want and math.copysign(1.0, g) == math.copysign(1.0, want), c


def test_e4m3_all_codes_match_torch_widening():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert nan.sum() == 2                                  # 0x7f and 0xff only


def test_e4m3_order_and_sign():
    v = oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)                          # positive codes increase
    neg = oracle.e4m3_to_f64(np.arange(0x80, 0xFF, dtype=np.uint8))
    assert np.array_equal(neg, -v)


def _bf16_bits(x):
    b = np.asarray(x, np.float32).view(np.uint32)
    assert np.all(b & 0xFFFF == 0)                         # exactly a bf16 value
    return (b >> 16).astype(np.uint16)


def test_power_of_two_scales_reduce_to_the_bf16_oracle():
    """With scales 2^-5 and 2^-3, every dequantized value is exactly a bf16
    value, so the fp8 oracle equals the bf16 oracle on those values."""
    inp = quantize_kv_fp8(make_flat("f8a", 501, 3, 16, 16, [1, 37, 300]), 2.0 ** -5, 2.0 ** -3)
    deq_c = 2.0 ** -5 * oracle.e4m3_to_f64(inp.ckv8)
    deq_k = 2.0 ** -3 * oracle.e4m3_to_f64(inp.kpe8)
    o8, l8 = oracle.attend_flat(inp.q_nope, inp.q_pe, inp.ckv8, inp.kpe8, inp.kv_indptr,
                                inp.kv_indices, inp.kv_lens, inp.page_size,
                                kv_scales=(inp.ckv_scale, inp.kpe_scale))
    ob, lb = oracle.attend_flat(inp.q_nope, inp.q_pe, _bf16_bits(deq_c), _bf16_bits(deq_k),
                                inp.kv_indptr, inp.kv_indices, inp.kv_lens, inp.page_size)
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)


def test_fp8_matches_torch_sdpa_on_dequantized_rows():
    inp = quantize_kv_fp8(make_flat("f8b", 502, 2, 16, 8, [5, 77]))
    o8, l8 = oracle.attend_flat(inp.q_nope, inp.q_pe, inp.ckv8, inp.kpe8, inp.kv_indptr,
                                inp.kv_indices, inp.kv_lens, inp.page_size,
                                kv_scales=(inp.ckv_scale, inp.kpe_scale))
    scale = 1.0 / math.sqrt(576)
    for b in range(inp.batch):
        pages, slots = oracle.token_pages(inp.kv_indptr, inp.kv_indices, inp.kv_lens[b], b,
                                          inp.page_size)
        c = inp.ckv_scale * oracle.e4m3_to_f64(inp.ckv8[pages, slots])
        k = np.concatenate([c, inp.kpe_scale * oracle.e4m3_to_f64(inp.kpe8[pages, slots])], 1)
        q = np.concatenate([oracle.bf16_to_f64(inp.q_nope[b]), oracle.bf16_to_f64(inp.q_pe[b])], 1)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(c)[None],
            scale=scale)[0].numpy()
        np.testing.assert_allclose(o8[b], ref, rtol=0, atol=1e-12)
        s = scale * (q @ k.T)
        np.testing.assert_allclose(l8[b], np.log(np.exp(s).sum(1)), rtol=0, atol=1e-12)


def test_fp8_cascade_equals_flat():
    cas = quantize_kv_fp8(make_cascade("f8c", 503, 4, 32, 16, [48, 64], [3, 0, 25, 9], groups=2))
    sc = (cas.ckv_scale, cas.kpe_scale)
    oc, lc = oracle.attend_cascade(cas.q_nope, cas.q_pe, cas.ckv8, cas.kpe8, cas.page_size,
                                   cas.group_req_indptr, cas.prefix_indptr, cas.prefix_indices,
                                   cas.prefix_lens, cas.kv_indptr, cas.kv_indices, cas.kv_lens,
                                   kv_scales=sc)
    flat = cas.flat_view()
    q8 = quantize_kv_fp8(flat, *sc)
    of, lf = oracle.attend_flat(q8.q_nope, q8.q_pe, q8.ckv8, q8.kpe8, q8.kv_indptr,
                                q8.kv_indices, q8.kv_lens, q8.page_size, kv_scales=sc)
    np.testing.assert_allclose(oc, of, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lc, lf, rtol=0, atol=1e-12)


def test_quantizer_rounds_to_nearest_even_and_keeps_nan():
    inp = make_flat("f8d", 504, 1, 16, 16, [10])
    q = quantize_kv_fp8(inp, 1.0, 1.0)
    vals = (inp.ckv.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    dec = oracle.e4m3_to_f64(q.ckv8)
    # nearest: no representable E4M3 value is closer than the chosen one
    grid = oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    grid = np.concatenate([-grid[::-1], grid])
    err = np.abs(dec - vals)
    best = np.min(np.abs(vals.reshape(-1, 1) - grid.reshape(1, -1)), axis=1).reshape(vals.shape)
    assert np.all(err <= best)
