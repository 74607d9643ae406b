"""Diagonal-aware sparse attention for autoregressive image generation on
MI355X (gfx950): HIP kernels behind the C ABI in include/diagattn.h, with a
thin torch binding for device memory and streams.
"""
from ._native import DiagAttnError, load  # noqa: F401
from .api import (  # noqa: F401
    BAND,
    DENSE,
    ROWDIAG,
    band_prefill_attn,
    decode_schedule,
    decode_workspace,
    decode_workspace_bytes,
    gather_read_probe,
    hbm_read_probe,
    keep_cap,
    keep_count,
    keepset_build,
    keepset_tiles,
    kept_row_offsets,
    kv_cache,
    mask,
    prefill_tiles_build,
    ring_block_table,
    ring_pages,
    sparse_decode_attn,
    sparse_decode_attn_masked,
    sparse_decode_attn_masked_noalloc,
    decode_scratch_bytes,
)
