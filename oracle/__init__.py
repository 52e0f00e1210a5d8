"""fp64 CPU oracle (test infrastructure only; see attention.py)."""
from .attention import (  # noqa: F401
    aggregate_scores,
    attend,
    block_positions,
    block_sums,
    collected_logits,
    default_scale,
    kvgroup_sum,
    select_blocks,
    select_blocks_batch,
    select_topk,
    select_topk_batch,
    select_topk_hybrid,
    select_topk_hybrid_batch,
    sparse_attention,
    verify_attention,
    widen_bf16,
)
