"""Seeded input generators (no attention arithmetic in here).

Draw order for every workload: kv_lens -> page permutation -> q_nope, q_pe,
ckv pool, kpe pool.  All bf16 tensors are raw uint16 bit patterns.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

CKV_DIM = 512  # head_dim_ckv = kv_lora_rank
KPE_DIM = 64   # head_dim_kpe = qk_rope_head_dim
VALUE_STD = 0.5

# Workloads, described by what they are.  "tiny" is small enough for the
# oracle to finish in well under a second; the others are full-size shapes.
CONFIGS = {
    "tiny": dict(kind="flat", batch=4, num_heads=16, page_size=16,
                 lens=("fixed", [1, 17, 64, 200]), pool_pages=64),
    "deepseek": dict(kind="flat", batch=64, num_heads=128, page_size=64,
                     lens=("uniform", 1024, 4096), pool_pages=None),
    "long": dict(kind="flat", batch=8, num_heads=128, page_size=64,
                 lens=("fixed", [32768] * 8), pool_pages=None),
    "ragged": dict(kind="flat", batch=256, num_heads=16, page_size=1,
                   lens=("lognormal", 1024.0, 1.0, 1, 16384), pool_pages=None),
    "cascade": dict(kind="cascade", batch=128, num_heads=128, page_size=64,
                    prefix_len=8192, suffix=(64, 1024)),
    # several new tokens per request (e.g. speculative decode with 3 draft
    # tokens) on a 16-head share: 4 query tokens each, causal among them
    "qo": dict(kind="qo", batch=64, num_heads=16, page_size=64,
               lens=("uniform", 1024, 4096), pool_pages=None, qo_len=4),
}
CONFIG_SEEDS = {"tiny": 0, "deepseek": 1, "long": 2, "ragged": 3, "cascade": 4, "qo": 5}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even) -> uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def _bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    # exact widening used only to build structured stress inputs
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal_bf16(rng: np.random.Generator, shape, std=VALUE_STD) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    step = 1 << 24
    for s in range(0, n, step):
        e = min(n, s + step)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal(e - s, dtype=np.float32) * np.float32(std))
    return out.reshape(shape)


@dataclasses.dataclass
class FlatInputs:
    name: str
    seed: int
    batch: int
    num_heads: int
    page_size: int
    num_pages: int
    kv_lens: np.ndarray      # int32 [B]
    kv_indptr: np.ndarray    # int32 [B+1]
    kv_indices: np.ndarray   # int32 [indptr[B]]
    q_nope: np.ndarray       # uint16 (bf16 bits) [B, H, 512]
    q_pe: np.ndarray         # uint16 [B, H, 64]
    ckv: np.ndarray          # uint16 [P, ps, 512]
    kpe: np.ndarray          # uint16 [P, ps, 64]
    sm_scale: Optional[float] = None  # None -> 1/sqrt(512 + 64)
    ckv_dim: int = CKV_DIM
    kpe_dim: int = KPE_DIM
    # several new query tokens per request: q rows qo_indptr[b] .. qo_indptr[b+1]
    qo_indptr: Optional[np.ndarray] = None
    # fp8 KV caches (quantize_kv_fp8): E4M3 codes and per-tensor scales
    ckv8: Optional[np.ndarray] = None   # uint8 [P, ps, 512]
    kpe8: Optional[np.ndarray] = None   # uint8 [P, ps, 64]
    ckv_scale: Optional[float] = None
    kpe_scale: Optional[float] = None

    @property
    def total_tokens(self) -> int:
        return int(self.kv_lens.astype(np.int64).sum())

    def replace(self, **kw) -> "FlatInputs":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass
class CascadeInputs:
    """Two-level layout: per group a shared prefix page list, per request a suffix list.

    Groups partition the requests contiguously (group_req_indptr).  The prefix of
    group g is prefix_lens[g] tokens in pages prefix_indices[prefix_indptr[g]:...].
    Request b additionally owns suffix_lens[b] tokens (may be 0).
    """
    name: str
    seed: int
    batch: int
    num_heads: int
    page_size: int
    num_pages: int
    group_req_indptr: np.ndarray  # int32 [G+1]
    prefix_indptr: np.ndarray     # int32 [G+1]
    prefix_indices: np.ndarray    # int32
    prefix_lens: np.ndarray       # int32 [G]
    kv_indptr: np.ndarray         # suffix page CSR, int32 [B+1]
    kv_indices: np.ndarray
    kv_lens: np.ndarray           # suffix lengths, int32 [B]
    q_nope: np.ndarray
    q_pe: np.ndarray
    ckv: np.ndarray
    kpe: np.ndarray
    sm_scale: Optional[float] = None
    ckv8: Optional[np.ndarray] = None   # fp8 KV caches (quantize_kv_fp8)
    kpe8: Optional[np.ndarray] = None
    ckv_scale: Optional[float] = None
    kpe_scale: Optional[float] = None
    ckv_dim: int = CKV_DIM
    kpe_dim: int = KPE_DIM

    @property
    def num_groups(self) -> int:
        return int(self.prefix_lens.shape[0])

    def group_of(self, b: int) -> int:
        return int(np.searchsorted(self.group_req_indptr, b, side="right") - 1)

    def attended_tokens(self) -> int:
        tot = int(self.kv_lens.astype(np.int64).sum())
        for g in range(self.num_groups):
            nreq = int(self.group_req_indptr[g + 1] - self.group_req_indptr[g])
            tot += nreq * int(self.prefix_lens[g])
        return tot

    def unique_tokens(self) -> int:
        return int(self.kv_lens.astype(np.int64).sum() + self.prefix_lens.astype(np.int64).sum())

    def flat_view(self) -> FlatInputs:
        """The same attention written as one flat page list per request
        (prefix pages then suffix pages).  Needs every prefix_len % page_size == 0."""
        ps = self.page_size
        indptr = [0]
        idx = []
        lens = []
        for b in range(self.batch):
            g = self.group_of(b)
            pl = int(self.prefix_lens[g])
            if pl % ps:
                raise ValueError("flat view needs prefix_len to be a multiple of page_size")
            pp = self.prefix_indices[self.prefix_indptr[g]:self.prefix_indptr[g] + pl // ps]
            sp = self.kv_indices[self.kv_indptr[b]:self.kv_indptr[b + 1]]
            idx.append(pp)
            idx.append(sp)
            lens.append(pl + int(self.kv_lens[b]))
            indptr.append(indptr[-1] + len(pp) + len(sp))
        return FlatInputs(
            name=self.name + "/flat", seed=self.seed, batch=self.batch,
            num_heads=self.num_heads, page_size=ps, num_pages=self.num_pages,
            kv_lens=np.asarray(lens, dtype=np.int32),
            kv_indptr=np.asarray(indptr, dtype=np.int32),
            kv_indices=np.concatenate(idx).astype(np.int32),
            q_nope=self.q_nope, q_pe=self.q_pe, ckv=self.ckv, kpe=self.kpe,
            sm_scale=self.sm_scale)


def _draw_lens(rng, batch, spec) -> np.ndarray:
    kind = spec[0]
    if kind == "fixed":
        lens = np.asarray(spec[1], dtype=np.int64)
        assert lens.shape[0] == batch
    elif kind == "uniform":
        lens = rng.integers(spec[1], spec[2], size=batch, endpoint=True)
    elif kind == "lognormal":
        median, sigma, lo, hi = spec[1:]
        lens = np.clip(np.rint(np.exp(rng.normal(math.log(median), sigma, size=batch))), lo, hi)
    else:
        raise ValueError(kind)
    return lens.astype(np.int32)


def make_flat(name: str, seed: int, batch: int, num_heads: int, page_size: int,
              lens, pool_pages: Optional[int] = None, extra_pages: int = 0,
              sm_scale: Optional[float] = None) -> FlatInputs:
    """Flat paged decode batch.  ``lens`` is a spec tuple or an explicit list.

    Request b owns the next ceil(L_b/ps) (+extra_pages) entries of a seeded
    permutation of the page pool, so pages are scattered over the pool.
    """
    rng = np.random.default_rng(seed)
    if isinstance(lens, (list, np.ndarray)):
        kv_lens = np.asarray(lens, dtype=np.int32)
    else:
        kv_lens = _draw_lens(rng, batch, lens)
    assert kv_lens.shape == (batch,)
    npages_b = (kv_lens.astype(np.int64) + page_size - 1) // page_size + extra_pages
    need = int(npages_b.sum())
    num_pages = need if pool_pages is None else int(pool_pages)
    if num_pages < need:
        raise ValueError(f"pool of {num_pages} pages is smaller than the {need} needed")
    perm = rng.permutation(num_pages).astype(np.int32)
    indptr = np.zeros(batch + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(npages_b)
    indices = perm[:need].copy()
    q_nope = _normal_bf16(rng, (batch, num_heads, CKV_DIM))
    q_pe = _normal_bf16(rng, (batch, num_heads, KPE_DIM))
    ckv = _normal_bf16(rng, (num_pages, page_size, CKV_DIM))
    kpe = _normal_bf16(rng, (num_pages, page_size, KPE_DIM))
    return FlatInputs(name=name, seed=seed, batch=batch, num_heads=num_heads,
                      page_size=page_size, num_pages=num_pages, kv_lens=kv_lens,
                      kv_indptr=indptr, kv_indices=indices, q_nope=q_nope, q_pe=q_pe,
                      ckv=ckv, kpe=kpe, sm_scale=sm_scale)


def make_qo(name: str, seed: int, batch: int, num_heads: int, page_size: int, lens,
            qo_lens, pool_pages: Optional[int] = None,
            sm_scale: Optional[float] = None) -> FlatInputs:
    """Flat paged batch whose request b brings qo_lens[b] new query tokens
    (its last qo_lens[b] tokens); q_nope/q_pe hold one row per query token."""
    base = make_flat(name, seed, batch, num_heads, page_size, lens, pool_pages=pool_pages,
                     sm_scale=sm_scale)
    qo = np.asarray(qo_lens, dtype=np.int32)
    assert qo.shape == (batch,) and np.all(qo >= 1) and np.all(qo <= base.kv_lens)
    qo_indptr = np.zeros(batch + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo)
    rng = np.random.default_rng(seed + 7919)
    T = int(qo_indptr[-1])
    q_nope = _normal_bf16(rng, (T, num_heads, CKV_DIM))
    q_pe = _normal_bf16(rng, (T, num_heads, KPE_DIM))
    return base.replace(q_nope=q_nope, q_pe=q_pe, qo_indptr=qo_indptr)


def make_cascade(name: str, seed: int, batch: int, num_heads: int, page_size: int,
                 prefix_len, suffix, groups: int = 1,
                 sm_scale: Optional[float] = None,
                 pool_pages: Optional[int] = None) -> CascadeInputs:
    """Shared-prefix batch.  ``prefix_len`` is an int (same for all groups) or a list;
    ``suffix`` is (lo, hi) for uniform suffix lengths or an explicit list.
    ``pool_pages`` fixes the pool size (at least the pages needed; the tables
    take the first pages of a permutation of the whole pool)."""
    rng = np.random.default_rng(seed)
    if isinstance(suffix, tuple):
        kv_lens = rng.integers(suffix[0], suffix[1], size=batch, endpoint=True).astype(np.int32)
    else:
        kv_lens = np.asarray(suffix, dtype=np.int32)
    if isinstance(prefix_len, int):
        prefix_lens = np.full(groups, prefix_len, dtype=np.int32)
    else:
        prefix_lens = np.asarray(prefix_len, dtype=np.int32)
    groups = int(prefix_lens.shape[0])
    # contiguous, near-equal request groups
    group_req_indptr = np.asarray([(g * batch) // groups for g in range(groups + 1)], dtype=np.int32)
    ppages = (prefix_lens.astype(np.int64) + page_size - 1) // page_size
    spages = (kv_lens.astype(np.int64) + page_size - 1) // page_size
    num_pages = int(ppages.sum() + spages.sum())
    if pool_pages is not None:
        if pool_pages < num_pages:
            raise ValueError(f"pool of {pool_pages} pages is below the {num_pages} needed")
        num_pages = int(pool_pages)
    perm = rng.permutation(num_pages).astype(np.int32)
    prefix_indptr = np.zeros(groups + 1, dtype=np.int32)
    prefix_indptr[1:] = np.cumsum(ppages)
    prefix_indices = perm[:prefix_indptr[-1]].copy()
    indptr = np.zeros(batch + 1, dtype=np.int32)
    indptr[1:] = np.cumsum(spages)
    indices = perm[prefix_indptr[-1]:prefix_indptr[-1] + indptr[-1]].copy()
    q_nope = _normal_bf16(rng, (batch, num_heads, CKV_DIM))
    q_pe = _normal_bf16(rng, (batch, num_heads, KPE_DIM))
    ckv = _normal_bf16(rng, (num_pages, page_size, CKV_DIM))
    kpe = _normal_bf16(rng, (num_pages, page_size, KPE_DIM))
    return CascadeInputs(name=name, seed=seed, batch=batch, num_heads=num_heads,
                         page_size=page_size, num_pages=num_pages,
                         group_req_indptr=group_req_indptr, prefix_indptr=prefix_indptr,
                         prefix_indices=prefix_indices, prefix_lens=prefix_lens,
                         kv_indptr=indptr, kv_indices=indices, kv_lens=kv_lens,
                         q_nope=q_nope, q_pe=q_pe, ckv=ckv, kpe=kpe, sm_scale=sm_scale)


def make_config(name: str, seed: Optional[int] = None):
    """Build one of the named workloads with its default seed."""
    cfg = dict(CONFIGS[name])
    seed = CONFIG_SEEDS[name] if seed is None else seed
    kind = cfg.pop("kind")
    if kind == "flat":
        return make_flat(name, seed, cfg["batch"], cfg["num_heads"], cfg["page_size"],
                         cfg["lens"], cfg["pool_pages"])
    if kind == "qo":
        return make_qo(name, seed, cfg["batch"], cfg["num_heads"], cfg["page_size"],
                       cfg["lens"], [cfg["qo_len"]] * cfg["batch"], cfg["pool_pages"])
    return make_cascade(name, seed, cfg["batch"], cfg["num_heads"], cfg["page_size"],
                        cfg["prefix_len"], cfg["suffix"])


def config_lens(name: str, seed: Optional[int] = None):
    """Only the length draw of a named workload (the first thing its generator
    draws, so the values equal those of make_config).  Flat workloads return
    kv_lens; the cascade workload returns (prefix_len, suffix_lens)."""
    cfg = CONFIGS[name]
    seed = CONFIG_SEEDS[name] if seed is None else seed
    rng = np.random.default_rng(seed)
    if cfg["kind"] in ("flat", "qo"):
        return _draw_lens(rng, cfg["batch"], cfg["lens"])
    lo, hi = cfg["suffix"]
    return cfg["prefix_len"], rng.integers(lo, hi, size=cfg["batch"], endpoint=True).astype(np.int32)


# ---------------------------------------------------------------------------
# Stress variants: structured values that force the online softmax to work.
# ---------------------------------------------------------------------------
STRESS_KINDS = ("qx8", "needle", "increasing", "negative")


def _token_rows(inp: FlatInputs, b: int):
    """(page, slot) of every valid token of request b (page-table walk)."""
    ps = inp.page_size
    L = int(inp.kv_lens[b])
    base = int(inp.kv_indptr[b])
    t = np.arange(L)
    return inp.kv_indices[base + t // ps], t % ps


def stress_variant(inp: FlatInputs, kind: str, seed: int = 1234) -> FlatInputs:
    """Return a copy of ``inp`` whose values stress the running-max logic.

    qx8        q scaled by 8 (exact in bf16): logit std ~2 instead of ~0.25.
    needle     per request one token whose ckv/kpe row is a scaled copy of one
               head's query, giving that head a logit near +20.
    increasing q_pe shares a per-request direction w and kpe rows grow along t,
               so the largest logit moves forward with every tile.
    negative   kpe rows ~ -30*w, every logit near -80.
    Requires pages not shared between requests (true for make_flat).
    """
    rng = np.random.default_rng(seed)
    scale = inp.sm_scale if inp.sm_scale is not None else 1.0 / math.sqrt(inp.ckv_dim + inp.kpe_dim)
    q_nope = inp.q_nope.copy()
    q_pe = inp.q_pe.copy()
    ckv = inp.ckv.copy()
    kpe = inp.kpe.copy()
    if kind == "qx8":
        q_nope = f32_to_bf16_bits(_bf16_bits_to_f32(q_nope) * np.float32(8))
        q_pe = f32_to_bf16_bits(_bf16_bits_to_f32(q_pe) * np.float32(8))
    elif kind == "needle":
        for b in range(inp.batch):
            h = b % inp.num_heads
            pages, slots = _token_rows(inp, b)
            j = int(rng.integers(0, len(pages)))
            qn = _bf16_bits_to_f32(q_nope[b, h]).astype(np.float64)
            qp = _bf16_bits_to_f32(q_pe[b, h]).astype(np.float64)
            beta = 20.0 / (scale * (qn @ qn + qp @ qp))
            ckv[pages[j], slots[j]] = f32_to_bf16_bits((beta * qn).astype(np.float32))
            kpe[pages[j], slots[j]] = f32_to_bf16_bits((beta * qp).astype(np.float32))
    elif kind in ("increasing", "negative"):
        for b in range(inp.batch):
            w = rng.standard_normal(inp.kpe_dim).astype(np.float32)
            noise = rng.standard_normal((inp.num_heads, inp.kpe_dim)).astype(np.float32) * 0.05
            q_pe[b] = f32_to_bf16_bits(w[None, :] + noise)
            pages, slots = _token_rows(inp, b)
            L = len(pages)
            if kind == "increasing":
                gamma = 30.0 / (scale * float(w @ w))
                coef = gamma * (np.arange(L, dtype=np.float32) / max(L, 1))
            else:
                coef = np.full(L, -80.0 / (scale * float(w @ w)), dtype=np.float32)
            rows = coef[:, None] * w[None, :] + rng.standard_normal((L, inp.kpe_dim)).astype(np.float32) * 0.1
            kpe[pages, slots] = f32_to_bf16_bits(rows.astype(np.float32))
    else:
        raise ValueError(kind)
    return inp.replace(name=f"{inp.name}/{kind}", q_nope=q_nope, q_pe=q_pe, ckv=ckv, kpe=kpe)


def _csr_rows(indptr, indices, length: int, i: int, page_size: int):
    """(page, slot) of the first ``length`` tokens of page list i of a CSR table."""
    t = np.arange(int(length))
    return indices[int(indptr[i]) + t // page_size], t % page_size


def _cascade_rows(cas: "CascadeInputs", b: int):
    """(page, slot) of request b's tokens: its group's prefix, then its suffix."""
    g = cas.group_of(b)
    pp, ps_ = _csr_rows(cas.prefix_indptr, cas.prefix_indices, cas.prefix_lens[g], g,
                        cas.page_size)
    sp, ss = _csr_rows(cas.kv_indptr, cas.kv_indices, cas.kv_lens[b], b, cas.page_size)
    return np.concatenate([pp, sp]), np.concatenate([ps_, ss])


def poison_unreferenced(inp):
    """Copy of ``inp`` (flat or cascade) where every pool slot that no request
    attends holds NaN bits: unused pages, the tail slots of each last page and
    any extra trailing pages."""
    used = np.zeros((inp.num_pages, inp.page_size), dtype=bool)
    for b in range(inp.batch):
        if isinstance(inp, CascadeInputs):
            pages, slots = _cascade_rows(inp, b)
        else:
            pages, slots = _token_rows(inp, b)
        used[pages, slots] = True
    ckv = inp.ckv.copy()
    kpe = inp.kpe.copy()
    ckv[~used] = 0x7FC0
    kpe[~used] = 0x7FC0
    return dataclasses.replace(inp, name=inp.name + "/poison", ckv=ckv, kpe=kpe)


def permute_pages(inp, seed: int = 99):
    """Re-scatter the page pool by a random physical permutation and remap the
    page tables (flat or cascade inputs); attention is unchanged by construction."""
    rng = np.random.default_rng(seed)
    pi = rng.permutation(inp.num_pages).astype(np.int32)
    ckv = np.empty_like(inp.ckv)
    kpe = np.empty_like(inp.kpe)
    ckv[pi] = inp.ckv
    kpe[pi] = inp.kpe
    kw = dict(ckv=ckv, kpe=kpe, kv_indices=pi[inp.kv_indices], name=inp.name + "/perm")
    if isinstance(inp, CascadeInputs):
        kw["prefix_indices"] = pi[inp.prefix_indices]
    return dataclasses.replace(inp, **kw)


def stress_variant_cascade(cas: CascadeInputs, kind: str, seed: int = 4321) -> CascadeInputs:
    """Cascade counterpart of :func:`stress_variant`.  The prefix pages are
    shared by a group's requests, so the structured rows follow the group:

    qx8        q scaled by 8 (exact in bf16).
    needle     request b (non-empty suffix) gets one suffix token whose rows are
               a scaled copy of head b % H's query (logit near +20); each
               group's prefix gets one such token for its first request.
    increasing every request of group g shares a q_pe direction w_g; kpe rows
               grow along the position (prefix, then suffix), so the largest
               logit moves forward with every tile of both levels.
    negative   kpe rows ~ -30 w_g everywhere: logits near -80.
    """
    rng = np.random.default_rng(seed)
    scale = cas.sm_scale if cas.sm_scale is not None else 1.0 / math.sqrt(cas.ckv_dim + cas.kpe_dim)
    q_nope, q_pe = cas.q_nope.copy(), cas.q_pe.copy()
    ckv, kpe = cas.ckv.copy(), cas.kpe.copy()
    ps = cas.page_size
    G = cas.num_groups
    if kind == "qx8":
        q_nope = f32_to_bf16_bits(_bf16_bits_to_f32(q_nope) * np.float32(8))
        q_pe = f32_to_bf16_bits(_bf16_bits_to_f32(q_pe) * np.float32(8))
    elif kind == "needle":
        def plant(b, h, page, slot):
            qn = _bf16_bits_to_f32(q_nope[b, h]).astype(np.float64)
            qp = _bf16_bits_to_f32(q_pe[b, h]).astype(np.float64)
            beta = 20.0 / (scale * (qn @ qn + qp @ qp))
            ckv[page, slot] = f32_to_bf16_bits((beta * qn).astype(np.float32))
            kpe[page, slot] = f32_to_bf16_bits((beta * qp).astype(np.float32))
        for g in range(G):
            b0 = int(cas.group_req_indptr[g])
            if cas.prefix_lens[g] > 0 and b0 < int(cas.group_req_indptr[g + 1]):
                pp, sl = _csr_rows(cas.prefix_indptr, cas.prefix_indices, cas.prefix_lens[g], g, ps)
                j = int(rng.integers(0, len(pp)))
                plant(b0, 0, pp[j], sl[j])
        for b in range(cas.batch):
            if cas.kv_lens[b] > 0:
                sp, sl = _csr_rows(cas.kv_indptr, cas.kv_indices, cas.kv_lens[b], b, ps)
                j = int(rng.integers(0, len(sp)))
                plant(b, b % cas.num_heads, sp[j], sl[j])
    elif kind in ("increasing", "negative"):
        for g in range(G):
            w = rng.standard_normal(cas.kpe_dim).astype(np.float32)
            reqs = range(int(cas.group_req_indptr[g]), int(cas.group_req_indptr[g + 1]))
            P = int(cas.prefix_lens[g])
            span = P + max([int(cas.kv_lens[b]) for b in reqs] or [0])

            def rows_for(pos):
                if kind == "increasing":
                    coef = (30.0 / (scale * float(w @ w))) * (pos.astype(np.float32) / max(span, 1))
                else:
                    coef = np.full(len(pos), -80.0 / (scale * float(w @ w)), dtype=np.float32)
                r = coef[:, None] * w[None, :] + rng.standard_normal((len(pos), cas.kpe_dim)).astype(np.float32) * 0.1
                return f32_to_bf16_bits(r.astype(np.float32))
            for b in reqs:
                noise = rng.standard_normal((cas.num_heads, cas.kpe_dim)).astype(np.float32) * 0.05
                q_pe[b] = f32_to_bf16_bits(w[None, :] + noise)
                if cas.kv_lens[b] > 0:
                    sp, sl = _csr_rows(cas.kv_indptr, cas.kv_indices, cas.kv_lens[b], b, ps)
                    kpe[sp, sl] = rows_for(P + np.arange(len(sp)))
            if P > 0:
                pp, sl = _csr_rows(cas.prefix_indptr, cas.prefix_indices, P, g, ps)
                kpe[pp, sl] = rows_for(np.arange(P))
    else:
        raise ValueError(kind)
    return dataclasses.replace(cas, name=f"{cas.name}/{kind}", q_nope=q_nope, q_pe=q_pe,
                               ckv=ckv, kpe=kpe)


def _e4m3_codes(x: np.ndarray) -> np.ndarray:
    """float32 values (|x| <= 448 or NaN) to OCP E4M3 codes, round to nearest
    even (PyTorch's float8_e4m3fn cast on the CPU)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()


def quantize_kv_fp8(inp, ckv_scale: Optional[float] = None, kpe_scale: Optional[float] = None):
    """The same bundle with E4M3 copies of its KV caches: code = RNE(value /
    scale), one scale per cache (default: its largest finite magnitude / 448,
    so no value overflows; NaN poison stays NaN).  Input preparation only: the
    attention side decodes the codes itself."""
    def f32(bits):
        return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
    c, k = f32(inp.ckv), f32(inp.kpe)

    def auto(x):
        m = float(np.nanmax(np.abs(x))) if np.isfinite(x).any() else 1.0
        return np.float32(m / 448.0) if m > 0 else np.float32(1.0)
    sc = np.float32(ckv_scale) if ckv_scale is not None else auto(c)
    sk = np.float32(kpe_scale) if kpe_scale is not None else auto(k)
    codes = []
    for name, x, s in (("ckv", c, sc), ("kpe", k, sk)):
        q = _e4m3_codes(x / s)
        if np.any(np.isfinite(x) & ((q & 0x7F) == 0x7F)):     # a finite value overflowed
            raise ValueError(f"{name} scale {s} lets values pass the E4M3 maximum 448")
        codes.append(q)
    return dataclasses.replace(inp, ckv8=codes[0], kpe8=codes[1], ckv_scale=float(sc),
                               kpe_scale=float(sk))
