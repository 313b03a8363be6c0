"""Float64 CPU oracle for the SpargeAttention2 hot path (test infrastructure only).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import this
package. The GPU library never imports, links or calls it, and the two share no code.
"""
from .spa2_oracle import (  # noqa: F401
    n_blocks,
    block_range,
    pool_blocks,
    pooled_probs,
    topk_count,
    select_row,
    block_mask_head,
    block_mask,
    attn_fwd_head,
    attn_fwd,
    error_terms_head,
    attn_bwd_head,
    attn_bwd,
)
