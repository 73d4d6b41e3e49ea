"""Seeded synthetic inputs for batched paged-KV MLA decode.

This module only *draws* inputs: sequence lengths, page tables and bf16 value
pools.  It holds none of the attention arithmetic, so both the fp64 oracle
(``oracle/``) and the HIP path (``paged_kv_mla_amd``) can be fed from it without
sharing any of the method's code.

Values are drawn as float32 N(0,1)*0.5 with ``numpy.random.default_rng(seed)``
and rounded to bfloat16 with round-to-nearest-even on the bit pattern; every
bf16 tensor is returned as its raw ``uint16`` bits.

Workload shapes follow the absorbed-form MLA decode setting discussed in the
vLLM-metax "support flashinfer_mla" review (head_dim_ckv = kv_lora_rank = 512,
head_dim_kpe = qk_rope_head_dim = 64, one query token per request, causal off).
"""

from .generate import (  # noqa: F401
    CONFIGS,
    FlatInputs,
    CascadeInputs,
    f32_to_bf16_bits,
    make_flat,
    make_cascade,
    make_qo,
    make_config,
    config_lens,
    stress_variant,
    stress_variant_cascade,
    poison_unreferenced,
    permute_pages,
    STRESS_KINDS,
    quantize_kv_fp8,
)
