"""int8 / int4 / 2-bit / Q4_0 KV-cache decode attention for AMD Instinct MI355X (gfx950).

The compute lives in the HIP library ``libkvq8.so`` (C ABI in
``include/kvq8.h``); :mod:`decode_attention_int8_amd.kvq8` is its thin ctypes
binding.  Importing this package does not load the library; the first call
does, and raises if the library has not been built.
"""
from .kvq8 import (  # noqa: F401
    KVQ8Error,
    alloc_workspace,
    kvq2_decode_attn,
    kvq2_decode_chunk_tokens,
    kvq2_decode_workspace_size,
    kvq2_quantize_append,
    kvq2_requantize_q4,
    kvq4_0_decode_attn,
    kvq4_0_decode_chunk_tokens,
    kvq4_0_decode_workspace_size,
    kvq4_0_quantize_append,
    kvq4_decode_attn,
    kvq4_decode_chunk_tokens,
    kvq4_decode_workspace_size,
    kvq4_quantize_append,
    kvq4_requantize_q8,
    kvq8_append_decode_attn,
    kvq8_decode_attn,
    kvq8_decode_attn_noalloc,
    kvq8_decode_chunk_tokens,
    kvq8_decode_workspace_size,
    kvq8_qk_partials,
    kvq8_quantize_append,
    kvq8_quantize_q,
    kvq8_status_string,
    kvq8_version,
    lib,
)
