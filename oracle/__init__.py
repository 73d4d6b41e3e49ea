"""fp64 CPU oracle for batched paged-KV MLA decode (absorbed form).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check
(``__graft_entry__.smoke``) and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library (``paged_kv_mla_amd``); both are fed from
the seeded generators in ``mla_workloads``, which hold no attention arithmetic.

Sources (web pages this follows; no line numbers, the pages are cited by title
and comment):
  * vLLM-metax pull request "[WIP] support flashinfer_mla", review of the
    ``decode_wrapper.plan`` call: the compressed-KV width head_dim_ckv is
    kv_lora_rank (not the single KV head count), head_dim_kpe is
    qk_rope_head_dim, causal is off and the softmax scale is
    1/sqrt(kv_lora_rank + qk_rope_head_dim) instead of a dummy 1.0.
  * same review, metadata slicing comment: the paged-KV descriptors are an
    indptr of B+1 entries and a per-request length array of B entries, held on
    the host; MLA needs no last_page_len.
  * vLLM pull request "[V1][Core] FlashInfer attention backend for V1": cascade
    (multi-level) attention must give the same output as normal attention.

Parity pins (all in tests/test_oracle_*.py, CPU only):
  attend_rows / attend_flat : torch fp64 SDPA (library), non-absorbed MHA brute
                              force, python-float fsum brute force, closed forms
                              (L=1, equal rows, q=0), golden hand-derived values.
  merge_states              : split-then-merge equals unsplit; identity state.
  attend_cascade            : equals attend_flat on the concatenated page list.
  attend_qo                 : torch fp64 SDPA with an explicit position mask,
                              python-float fsum brute force, reduces to
                              attend_flat for one query token, last query
                              token equals full (unmasked) attention.
  e4m3_to_f64               : hand-listed OCP E4M3 values (tests/golden), all 256
                              codes against torch's float8_e4m3fn widening,
                              monotone positive codes, sign symmetry.
  kv_scales (fp8 caches)    : power-of-two scales reduce to the bf16 oracle
                              on the same values; torch fp64 SDPA on the
                              dequantized rows; cascade = flat.
  gather_ref                : closed-form address walk vs an independent index
                              construction; permutation invariance.
  schedule_ref              : coverage/uniqueness invariants and hand-worked
                              small cases (the rule is this library's own design,
                              the pages describe no scheduler).
"""

from .mla_decode import (  # noqa: F401
    bf16_to_f64,
    e4m3_to_f64,
    default_sm_scale,
    token_pages,
    gather_ref,
    attend_rows,
    attend_flat,
    attend_flat_split,
    merge_states,
    attend_cascade,
    attend_qo,
    EMPTY_LSE,
)
from .schedule_ref import schedule_ref, kernel_config, PLAN_TILE  # noqa: F401
