"""CPU oracle for the fused attention forward and its gradient (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  It shares no code with
the HIP path: it is the plain definition of the operator, in float64 numpy,
against which the GPU kernels are checked.
"""
from .attention import (attention_head, attn_fwd, attn_fwd_block, attn_fwd_blocksparse, merge_lse,
                        merge_states, output_stage, scores_stage, softmax_stage, token_mask_block_sparse,
                        token_mask_dense, token_mask_offsets)
from .backward import (attention_head_bwd, attn_bwd, attn_bwd_blocksparse, probabilities_from_lse,
                       row_scalar_d, score_gradient)
from .blockmask import canonical_blockmask
from .gqa import attn_bwd_gqa, attn_fwd_gqa, expand_kv, expand_lists
from .selector import block_means, meanpool_scores, meanpool_select, select_topk

__all__ = [
    "attention_head", "attn_fwd", "attn_fwd_blocksparse", "merge_states", "output_stage",
    "scores_stage", "softmax_stage", "token_mask_block_sparse", "token_mask_dense",
    "canonical_blockmask", "attention_head_bwd", "attn_bwd", "attn_bwd_blocksparse",
    "probabilities_from_lse", "row_scalar_d", "score_gradient", "attn_fwd_block", "merge_lse",
    "token_mask_offsets", "attn_fwd_gqa", "attn_bwd_gqa", "expand_kv", "expand_lists",
    "block_means", "meanpool_scores", "meanpool_select", "select_topk",
]
