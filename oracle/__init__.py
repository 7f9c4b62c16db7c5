"""CPU fp64 oracle for exact attention (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg use this package.
"""
from .attention_ref import (NEG_INF, allowed_mask, attend_rows, attention_bh,  # noqa: F401
                            attention_bwd_bh, attention_bwd_ref, attention_ref, attention_varlen_bwd_ref, attention_varlen_ref, combine_ref, kvcache_append_ref,
                            paged_gather_ref, prob_weighted_abs_ref, scores_ref, softmax_rows, split_bounds,
                            splitkv_append_ref, splitkv_ref, visible_span)
