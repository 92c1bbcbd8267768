"""BlockRank hot path on MI355X (gfx950): block-sparse prefill attention, attention-mass
document scores and per-prompt ranking, behind the C ABI of include/blockrank.h.

The Python layer only marshals arguments to libblockrank.so; all computation runs in its
hand-written HIP kernels.
"""
from ._lib import (BlockRankError, BrDims, EXPORTED, LIB_PATH, NOALLOC_SCRATCH_BYTES, attn_bwd, attn_bwd_workspace_bytes, attn_fwd,
                   attn_fwd_noalloc, attn_fwd_rope, attn_fwd_rope_workspace_bytes, attn_fwd_sink,
                   attn_plan_items, attn_plan_schedule,
                   attn_routed, attn_routed_workspace_bytes,
                   attn_workspace_bytes, doc_scores, doc_scores_bwd, doc_scores_bwd_workspace_bytes, doc_scores_workspace_bytes,
                   infonce, load_library,
                   make_dims, query_attn, query_attn_workspace_bytes, rank_step, rank_workspace_bytes, rope, rope_positions, rope_signal,
                   rope_workspace_bytes, sort_docs, ssmax_scale, version)

__all__ = ["BlockRankError", "BrDims", "EXPORTED", "LIB_PATH", "NOALLOC_SCRATCH_BYTES", "attn_bwd", "attn_bwd_workspace_bytes",
           "attn_fwd", "attn_fwd_noalloc", "attn_fwd_rope", "attn_fwd_rope_workspace_bytes", "attn_fwd_sink", "attn_plan_items", "attn_plan_schedule",
           "attn_routed", "attn_routed_workspace_bytes",
           "attn_workspace_bytes", "doc_scores", "doc_scores_bwd", "doc_scores_bwd_workspace_bytes",
           "doc_scores_workspace_bytes", "infonce", "load_library",
           "make_dims", "query_attn", "query_attn_workspace_bytes", "rank_step", "rank_workspace_bytes", "rope", "rope_positions", "rope_signal",
           "rope_workspace_bytes", "sort_docs", "ssmax_scale", "version", "rank_prompts"]


def rank_prompts(Q, K, V, Q_S, segment_offsets, seg_ptr, doc_offsets, doc_ptr, softmax_scale=0.0,
                 out=None, scores=None, order=None, attn_workspace=None, score_workspace=None, stream=None):
    """One pass of the hot path on one layer: attention output, document scores, order."""
    out = attn_fwd(Q, K, V, segment_offsets, seg_ptr, out=out, softmax_scale=softmax_scale,
                   workspace=attn_workspace, stream=stream)
    scores = doc_scores(Q_S, K, doc_offsets, doc_ptr, softmax_scale=softmax_scale, scores=scores,
                        workspace=score_workspace, stream=stream)
    order = sort_docs(scores, doc_ptr, order=order, stream=stream)
    return out, scores, order
