"""CPU: plant plausible mistakes in the oracle and check that the pins catch
every one of them (a pin suite that passes a broken oracle pins nothing)."""

import math

import numpy as np
import pytest

import oracle
import oracle.mla_decode as od
from oracle_pins import ALL_PINS


def _drop_kpe(q_nope, q_pe, ckv, kpe, kv_indptr, kv_indices, kv_len, b, page_size, t0=0, t1=None,
              kv_scales=None):
    q, k, c = _orig_qkv(q_nope, q_pe, ckv, kpe, kv_indptr, kv_indices, kv_len, b, page_size, t0, t1,
                        kv_scales=kv_scales)
    k = k.copy()
    k[:, 512:] = 0.0
    return q, k, c


def _value_includes_kpe(q_nope, q_pe, ckv, kpe, kv_indptr, kv_indices, kv_len, b, page_size, t0=0,
                        t1=None, kv_scales=None):
    q, k, c = _orig_qkv(q_nope, q_pe, ckv, kpe, kv_indptr, kv_indices, kv_len, b, page_size, t0, t1,
                        kv_scales=kv_scales)
    c = c + np.pad(k[:, 512:], ((0, 0), (0, 448)))
    return q, k, c


def _swapped_walk(kv_indptr, kv_indices, kv_len, b, page_size):
    t = np.arange(int(kv_len), dtype=np.int64)
    idx = np.asarray(kv_indices, dtype=np.int64)
    n = int(kv_indptr[b + 1] - kv_indptr[b]) if b + 1 < len(kv_indptr) else 1
    pages = idx[int(kv_indptr[b]) + (t % max(n, 1))]
    return pages, (t // max(n, 1)) % page_size


def _lse_without_max(q, k, v, sm_scale):
    out, lse = _orig_rows(q, k, v, sm_scale)
    if k.shape[0] == 0:
        return out, lse
    s = sm_scale * (q @ k.T)
    return out, np.log(np.exp(s - s.max(axis=1)[:, None]).sum(axis=1))


def _unnormalised(q, k, v, sm_scale):
    if k.shape[0] == 0:
        return _orig_rows(q, k, v, sm_scale)
    s = sm_scale * (q @ k.T)
    e = np.exp(s - s.max(axis=1)[:, None])
    return e @ v, s.max(axis=1) + np.log(e.sum(axis=1))


def _scale_sqrt512(q, k, v, sm_scale):
    return _orig_rows(q, k, v, 1.0 / math.sqrt(512))


def _transposed_heads(q, k, v, sm_scale):
    out, lse = _orig_rows(q, k, v, sm_scale)
    return out[::-1].copy(), lse[::-1].copy()


def _merge_plain_average(states):
    o = np.mean([s[0] for s in states], axis=0)
    l = np.logaddexp.reduce([s[1] for s in states], axis=0)
    return o, l


def _off_by_one_len(kv_indptr, kv_indices, kv_len, b, page_size):
    return _orig_walk(kv_indptr, kv_indices, max(int(kv_len) - 1, 1), b, page_size)


_orig_qkv = od._request_qkv
_orig_rows = od.attend_rows
_orig_walk = od.token_pages

MUTANTS = {
    "drop_rope_term": ("_request_qkv", _drop_kpe),
    "value_includes_rope": ("_request_qkv", _value_includes_kpe),
    "swapped_page_walk": ("token_pages", _swapped_walk),
    "drops_last_token": ("token_pages", _off_by_one_len),
    "lse_missing_max": ("attend_rows", _lse_without_max),
    "unnormalised_softmax": ("attend_rows", _unnormalised),
    "wrong_scale": ("attend_rows", _scale_sqrt512),
    "heads_reversed": ("attend_rows", _transposed_heads),
    "merge_ignores_lse": ("merge_states", _merge_plain_average),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(od, attr, fn)
    if hasattr(oracle, attr):
        monkeypatch.setattr(oracle, attr, fn)
    caught = []
    for pin in ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
