"""fp64 CPU oracle for exact attention forward (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg use it; the
product path never does.
"""
from .attention import (ROW_CHUNK, attention_head, attention_picked,
                        attention_ref, kv_head_of, scores, softmax_rows,
                        visible_mask)

__all__ = ["ROW_CHUNK", "attention_head", "attention_picked", "attention_ref",
           "kv_head_of", "scores", "softmax_rows", "visible_mask"]
