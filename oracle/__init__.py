"""CPU oracle for the CLSA hot path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``. The product library never
imports, links or runs anything here, and nothing here imports the product.
"""

from .oracle import (  # noqa: F401
    BF16,
    F32,
    FP8_E4M3FN,
    block_attn,
    block_union,
    build,
    cache_append,
    decode,
    decode_step,
    index_score,
    sparse_attn,
    topk,
    topk_margin,
)
