"""Plain fp64 definition of absorbed-form MLA paged decode.

Test infrastructure only (see the package docstring).  No tiling, no online
softmax, no blocking: each function is the textbook definition written out.
"""

from __future__ import annotations

import math

import numpy as np

EMPTY_LSE = -math.inf


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of raw bfloat16 bit patterns (uint16) to float64."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Exact value of OCP 8-bit floating point E4M3 codes (uint8), float64.

    The format (OCP "8-bit Floating Point Specification (OFP8)", E4M3): sign
    bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0 is
    subnormal, (-1)^s * 2^-6 * m/8; otherwise (-1)^s * 2^(e-7) * (1 + m/8).
    There is no infinity: exponent field 15 with mantissa 7 is NaN, so the
    largest finite magnitude is 1.75 * 2^8 = 448."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def default_sm_scale(ckv_dim: int, kpe_dim: int) -> float:
    """Softmax scale the flashinfer_mla plan review asks for:
    1/sqrt(kv_lora_rank + qk_rope_head_dim)  (1/24 for 512 + 64)."""
    return 1.0 / math.sqrt(ckv_dim + kpe_dim)


def token_pages(kv_indptr, kv_indices, kv_len: int, b: int, page_size: int):
    """Page-table walk for request b: token t lives in page
    kv_indices[kv_indptr[b] + t // page_size] at slot t % page_size.
    Only the first kv_len tokens exist (no last_page_len descriptor for MLA)."""
    t = np.arange(int(kv_len), dtype=np.int64)
    pages = np.asarray(kv_indices, dtype=np.int64)[int(kv_indptr[b]) + t // page_size]
    slots = t % page_size
    return pages, slots


def gather_ref(ckv_bits, kpe_bits, kv_indptr, kv_indices, kv_lens, page_size):
    """Raw bf16 rows [sum(kv_lens), ckv_dim + kpe_dim] in (request, token) order:
    the ckv row followed by the kpe row of every attended token, bit for bit."""
    rows = []
    for b in range(len(kv_lens)):
        pages, slots = token_pages(kv_indptr, kv_indices, kv_lens[b], b, page_size)
        rows.append(np.concatenate([ckv_bits[pages, slots], kpe_bits[pages, slots]], axis=1))
    if not rows:
        return np.zeros((0, ckv_bits.shape[-1] + kpe_bits.shape[-1]), dtype=np.uint16)
    return np.concatenate(rows, axis=0)


def attend_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, sm_scale: float):
    """Softmax attention of H query rows over L key/value rows, fp64.

    q [H, D], k [L, D], v [L, Dv].  Returns out [H, Dv] and lse [H] where
    s = sm_scale * q k^T, lse = ln sum_t exp(s_t) (natural log of the *scaled*
    logits) and out = sum_t exp(s_t - lse) v_t.  L = 0 gives the empty state
    (out = 0, lse = -inf), the identity of merge_states.
    """
    H = q.shape[0]
    if k.shape[0] == 0:
        return np.zeros((H, v.shape[1])), np.full(H, EMPTY_LSE)
    s = sm_scale * (q @ k.T)                    # [H, L]
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    z = e.sum(axis=1)
    out = (e @ v) / z[:, None]
    lse = m + np.log(z)
    return out, lse


def _request_qkv(q_nope, q_pe, ckv, kpe, kv_indptr, kv_indices, kv_len, b, page_size,
                 t0=0, t1=None, kv_scales=None):
    """Absorbed-form operands of request b over tokens [t0, t1):
    query [q_nope | q_pe] (H x 576), key [ckv | kpe] (L x 576), value ckv (L x 512).
    All H heads share the one latent KV row per token.  kv_scales None: the
    caches hold bf16 bits; (ckv_scale, kpe_scale): they hold E4M3 codes and a
    row's value is its scale times the code's value."""
    pages, slots = token_pages(kv_indptr, kv_indices, kv_len, b, page_size)
    t1 = int(kv_len) if t1 is None else t1
    pages, slots = pages[t0:t1], slots[t0:t1]
    if kv_scales is None:
        c = bf16_to_f64(ckv[pages, slots])
        r = bf16_to_f64(kpe[pages, slots])
    else:
        c = float(kv_scales[0]) * e4m3_to_f64(ckv[pages, slots])
        r = float(kv_scales[1]) * e4m3_to_f64(kpe[pages, slots])
    q = np.concatenate([bf16_to_f64(q_nope[b]), bf16_to_f64(q_pe[b])], axis=1)
    k = np.concatenate([c, r], axis=1)
    return q, k, c


def attend_flat(q_nope, q_pe, ckv, kpe, kv_indptr, kv_indices, kv_lens, page_size,
                sm_scale=None, kv_scales=None):
    """Batched decode: for every request b and head h,
    score_t = sm_scale (q_nope[b,h].ckv_t + q_pe[b,h].kpe_t) over the kv_lens[b]
    tokens of b's pages (non-causal, one query token), out = softmax . ckv.
    kv_scales (ckv_scale, kpe_scale): ckv and kpe hold E4M3 codes, dequantized
    to scale * value before the products (bf16 queries, as in the fp8 KV-cache
    limitation the V1 FlashInfer backend page lists for cascade).
    Returns out float64 [B, H, ckv_dim] and lse float64 [B, H]."""
    B, H, dc = q_nope.shape
    dr = q_pe.shape[2]
    scale = default_sm_scale(dc, dr) if sm_scale is None else float(sm_scale)
    out = np.zeros((B, H, dc))
    lse = np.zeros((B, H))
    for b in range(B):
        q, k, v = _request_qkv(q_nope, q_pe, ckv, kpe, kv_indptr, kv_indices,
                               kv_lens[b], b, page_size, kv_scales=kv_scales)
        out[b], lse[b] = attend_rows(q, k, v, scale)
    return out, lse


def merge_states(states):
    """Combine attention states over disjoint token sets.

    states: list of (out [..., Dv], lse [...]).  Softmax over a disjoint union:
    lse = ln sum_i exp(lse_i); out = sum_i exp(lse_i - lse) out_i.
    Empty states (lse = -inf) contribute nothing."""
    lses = np.stack([np.asarray(s[1], dtype=np.float64) for s in states])   # [n, ...]
    outs = np.stack([np.asarray(s[0], dtype=np.float64) for s in states])   # [n, ..., Dv]
    m = lses.max(axis=0)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(lses - m_safe)                                                # 0 for empty
    tot = w.sum(axis=0)
    lse = np.where(tot > 0, m_safe + np.log(np.where(tot > 0, tot, 1.0)), EMPTY_LSE)
    wn = np.where(tot > 0, w / np.where(tot > 0, tot, 1.0), 0.0)
    out = (wn[..., None] * outs).sum(axis=0)
    return out, lse


def attend_flat_split(q_nope, q_pe, ckv, kpe, kv_indptr, kv_indices, kv_lens, page_size,
                      splits, sm_scale=None):
    """attend_flat computed as partial states over token ranges, then merged.

    splits[b] is a list of cut points inside (0, kv_lens[b]); each range
    yields a partial state, merged with merge_states."""
    B, H, dc = q_nope.shape
    dr = q_pe.shape[2]
    scale = default_sm_scale(dc, dr) if sm_scale is None else float(sm_scale)
    out = np.zeros((B, H, dc))
    lse = np.zeros((B, H))
    for b in range(B):
        L = int(kv_lens[b])
        cuts = [0] + sorted(int(c) for c in splits[b]) + [L]
        parts = []
        for t0, t1 in zip(cuts[:-1], cuts[1:]):
            q, k, v = _request_qkv(q_nope, q_pe, ckv, kpe, kv_indptr, kv_indices,
                                   L, b, page_size, t0, t1)
            parts.append(attend_rows(q, k, v, scale))
        out[b], lse[b] = merge_states(parts)
    return out, lse


def attend_cascade(q_nope, q_pe, ckv, kpe, page_size,
                   group_req_indptr, prefix_indptr, prefix_indices, prefix_lens,
                   kv_indptr, kv_indices, kv_lens, sm_scale=None, kv_scales=None):
    """Two-level (cascade) attention: level 0 attends every request of group g to
    the group's shared prefix pages, level 1 attends request b to its own suffix
    pages, and the two states are merged by log-sum-exp.  Equals flat attention
    over prefix-then-suffix tokens (the V1 FlashInfer backend discussion requires
    cascade and normal attention to agree)."""
    B, H, dc = q_nope.shape
    dr = q_pe.shape[2]
    scale = default_sm_scale(dc, dr) if sm_scale is None else float(sm_scale)
    out = np.zeros((B, H, dc))
    lse = np.zeros((B, H))
    G = len(prefix_lens)
    for g in range(G):
        for b in range(int(group_req_indptr[g]), int(group_req_indptr[g + 1])):
            # level 0: shared prefix of group g (its own page list)
            q, k, v = _request_qkv(q_nope, q_pe, ckv, kpe, prefix_indptr, prefix_indices,
                                   prefix_lens[g], g, page_size, kv_scales=kv_scales)
            q = np.concatenate([bf16_to_f64(q_nope[b]), bf16_to_f64(q_pe[b])], axis=1)
            s0 = attend_rows(q, k, v, scale)
            # level 1: request b's suffix
            q, k, v = _request_qkv(q_nope, q_pe, ckv, kpe, kv_indptr, kv_indices,
                                   kv_lens[b], b, page_size, kv_scales=kv_scales)
            s1 = attend_rows(q, k, v, scale)
            out[b], lse[b] = merge_states([s0, s1])
    return out, lse


def attend_qo(q_nope, q_pe, ckv, kpe, qo_indptr, kv_indptr, kv_indices, kv_lens, page_size,
              sm_scale=None, kv_scales=None):
    """Several new query tokens per request, causal among them.

    Request b brings n_b = qo_indptr[b+1] - qo_indptr[b] new query tokens; they
    are the last n_b of its kv_lens[b] tokens.  Query row qo_indptr[b] + j sits
    at position kv_lens[b] - n_b + j and attends exactly the tokens at positions
    0 .. that position (scores of later positions masked to -inf before the
    softmax).  q_nope [T, H, ckv_dim], q_pe [T, H, kpe_dim] with
    T = qo_indptr[B].  kv_scales as in attend_flat.  Returns out float64
    [T, H, ckv_dim] and lse [T, H]."""
    T, H, dc = q_nope.shape
    dr = q_pe.shape[2]
    scale = default_sm_scale(dc, dr) if sm_scale is None else float(sm_scale)
    out = np.zeros((T, H, dc))
    lse = np.zeros((T, H))
    for b in range(len(kv_lens)):
        n = int(qo_indptr[b + 1]) - int(qo_indptr[b])
        L = int(kv_lens[b])
        pages, slots = token_pages(kv_indptr, kv_indices, L, b, page_size)
        if kv_scales is None:
            c = bf16_to_f64(ckv[pages, slots])
            r = bf16_to_f64(kpe[pages, slots])
        else:
            c = float(kv_scales[0]) * e4m3_to_f64(ckv[pages, slots])
            r = float(kv_scales[1]) * e4m3_to_f64(kpe[pages, slots])
        k = np.concatenate([c, r], axis=1)                                 # [L, 576]
        positions = np.arange(L)
        for j in range(n):
            row = int(qo_indptr[b]) + j
            q = np.concatenate([bf16_to_f64(q_nope[row]), bf16_to_f64(q_pe[row])], axis=1)
            s = scale * (q @ k.T)                                           # [H, L]
            s = np.where(positions[None, :] <= L - n + j, s, -np.inf)
            m = s.max(axis=1)
            e = np.exp(s - m[:, None])
            z = e.sum(axis=1)
            out[row] = (e @ c) / z[:, None]
            lse[row] = m + np.log(z)
    return out, lse
