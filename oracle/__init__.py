"""Float64 CPU oracle -- test infrastructure only.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  Nothing in the product path imports it.
"""
from .msa_oracle import (  # noqa: F401
    block_max_scores,
    decode_bf16,
    decode_e4m3fn,
    dequant,
    select_topk,
    sparse_decode,
)
