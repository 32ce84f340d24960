"""CPU oracle for HySparse2's inner-level KV Reuse path (test infrastructure).

This package is the slow, plain, obviously-correct reference that the HIP
library is checked against.  It is test infrastructure only: the tests, the
smoke check and the CPU-baseline leg of the benchmark may call it; the product
path never does.  It shares no code with the HIP library and imports nothing
from it.  See ``oracle/hs2_oracle.py`` for the definitions and citations.
"""

from .hs2_oracle import (  # noqa: F401
    attention_probs,
    bf16_round,
    block_scores,
    bridge_kv,
    bridge_kv_decode,
    dense_attention,
    dequant_kv,
    fp8_e4m3_value,
    full_attn_scores,
    query_positions,
    round_to_f32,
    pool_end,
    select_topk_blocks,
    select_topk_window,
    selection_set,
    sparse_attention,
    swa_attention,
)
