"""Plain f64 CPU oracle for HeadPrep and attention.

TEST INFRASTRUCTURE ONLY.  This package is the checker the GPU library is compared
against.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it; the GPU library never does, and this package never
imports the GPU library.

The arithmetic lives in ``oracle.c`` (f64, plain loops).  This module only marshals
numpy arrays into it and composes the steps the way the attention path does (prefill,
chunked prefill against a KV cache, decode):

* HeadPrep -- gizml:netops reference page, "Types > HeadPrep" (split halves, and
  FLUX.3's adjacent pairs).
* the whole-row norm and rotary -- same page, "Functions > rowNormRopeInto".
* attention and its causal mask -- same page, "Functions > attention" and
  "Functions > causalMask"; packed rows with block-diagonal groups -- same page,
  "Functions > attentionRows" and "Functions > attendedRows".
* the quantised KV cache's coding -- compute guide "Tensors, GPU kernels and AI models",
  "Step 5: Run a language model" (8, 4 or 2 bits, least-squared-error range per head).
* the paged KV pool the engine's slots read their keys and values from (a page table
  mapping each sequence's rows to pool pages) -- compute guide, Step 5.
* headPrepInPlace's position rule (the table row of a token is its sequence row,
  ``row0`` being the row of the first) -- same page, "Functions > headPrepInPlace".
"""
from .oracle import (  # noqa: F401
    build,
    library_path,
    headprep,
    row_norm_rope,
    attention,
    attention_rows,
    paged_rows,
    gather_paged,
    decode_paged,
    prefill,
    prefill_chunk,
    prefill_chunk_ragged,
    attended_rows,
    attended_rows8,
    rows8_operands,
    int8_code,
    e4m3_code,
    KEY_TILE,
    decode,
    decode_q,
    kv_quantize,
    kv_dequantize,
    kv_pack,
    kv_unpack,
    threads,
)
