"""CPU oracle for UniPrefill's token-selection path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library and its
Python binding) imports, links or calls this package.  It may be used by
`tests/`, by `__graft_entry__.smoke()` and by the `cpu_baseline` leg of
`bench.py`, and by nothing else.

It is a plain, slow and obviously correct restatement of what the UniPrefill
paper (arXiv 2605.06221, "UniPrefill: Universal Long-Context Prefill
Acceleration via Block-wise Dynamic Sparsification") defines, in NumPy float64.
It shares no code with the GPU path.
"""
from .uniprefill_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    token_importance,
    block_scores,
    request_block_scores,
    phi,
    pack_keys,
    top_p_select,
    expand_mask,
    select,
    compact,
    scatter_back,
    update_metadata,
    seqused_eq17,
    MetadataState,
    retained_positions,
    slot_mapping,
    write_kv_cache,
    silu,
    ffn_hidden,
    ffn_swiglu,
)
