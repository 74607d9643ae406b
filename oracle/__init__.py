"""CPU oracle for diagonal-aware sparse attention.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or call anything in this package.  It shares no code with the
HIP library (``ar_image_generation_amd``) and never imports it.
"""
from .reference import (  # noqa: F401
    BAND,
    DENSE,
    ROWDIAG,
    attend,
    decode_attention,
    keep,
    keep_row,
    keepset,
    keepset_loop,
    mask_matrix,
    prefill_attention,
    prefill_kept_pairs,
    runs,
    sparsity,
    speedup,
    tiles,
)
