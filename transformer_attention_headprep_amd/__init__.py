"""HeadPrep + scaled-dot-product attention for AMD MI355X (gfx950).

The compute lives in ``libattn.so`` (hand-written HIP kernels behind a C ABI, declared
in ``include/attn.h``); this package is its thin Python binding.  Build the library
with ``python -m transformer_attention_headprep_amd.build``.
"""
from .attn import (  # noqa: F401
    AttnError,
    HeadPrep,
    QuantCache,
    LIB_PATH,
    EXPORTS,
    attn_decode,
    attn_decode_paged,
    attn_decode_static,
    attn_decode_q,
    attn_decode_q_paged,
    attn_kv_quantize,
    attn_prefill,
    attn_prefill_chunk,
    attn_prefill_chunk_paged,
    attn_prep,
    attn_row_norm_rope,
    attn_rows,
    attn_rows8,
    attn_rows8_attend,
    attn_rows8_quantize,
    rows8_layout,
    attn_supported,
    decode_default_splits,
    decode_q_default_splits,
    decode_static_scratch_bytes,
    decode_workspace_size,
    key_bound,
    load_library,
)
