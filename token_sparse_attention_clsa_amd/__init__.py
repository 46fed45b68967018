"""Token-level sparse attention with a cross-layer shared index, for MI355X.

The computation lives in hand-written gfx950 HIP kernels behind the C ABI of
``libclsa.so`` (declared in ``include/clsa.h``); this package is the thin
Python binding over it plus the seeded input generators.
"""

from .binding import (  # noqa: F401
    BF16,
    F32,
    FP8_E4M3FN,
    ClsaError,
    DecodeStep,
    block_paged_attn,
    block_union_build,
    cache_append,
    decode_step,
    declared_symbols,
    index_score,
    load,
    sparse_attn,
    topk,
    topk_margin,
    workspace_bytes,
)
