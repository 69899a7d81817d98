"""fp64 CPU oracle for exact attention, forward and backward (test
infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg use it; the
product path never does.
"""
from .attention import (ROW_CHUNK, attention_bwd_picked, attention_bwd_ref, attention_fp8_ref,
                        attention_head, attention_head_bwd, attention_picked,
                        attention_ref, bias_of, e4m3_value, kv_head_of, scores,
                        softmax_rows, softmax_rows_bwd, visible_mask)

__all__ = ["ROW_CHUNK", "attention_bwd_picked", "attention_bwd_ref", "attention_fp8_ref",
           "attention_head", "attention_head_bwd", "attention_picked", "attention_ref", "bias_of",
           "e4m3_value", "kv_head_of", "scores", "softmax_rows", "softmax_rows_bwd",
           "visible_mask"]
