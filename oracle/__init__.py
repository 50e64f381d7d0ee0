"""CPU oracle of the KPool DSA indexer -- test infrastructure only.

Only tests/, `__graft_entry__.smoke()` and the CPU-baseline leg of bench.py may
import it. The HIP library never imports, links or calls anything here, and
this package imports nothing from the library.
"""
from .kpool_oracle import (  # noqa: F401
    bf16_round,
    causal_pools,
    compress,
    cu_pools_of,
    doc_of,
    e4m3_decode_table,
    e4m3_encode,
    expand_row,
    fp8_quantize_rows,
    fwht128,
    indexer_projections,
    indexer_topk,
    layer_norm,
    linear_bf16,
    pow2_row_exponent,
    row_scores,
    select_pools,
    sparse_mla_forward,
)
