"""fp64 CPU oracle for the attention forward pass -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package. The product path never does.
"""
from .attention import (attention_bwd_ref, attention_ref, block_summary, decode_ref, merge_lse,
                        merge_summaries, paged_decode_ref, paged_rows, split_decode_ref,
                        stream_attention, varlen_ref)

from .fp8 import e4m3_round, fp8_attention_ref, hadamard, quantize, rotate_f32

__all__ = ["e4m3_round", "hadamard", "rotate_f32", "quantize", "fp8_attention_ref", "attention_ref", "attention_bwd_ref", "stream_attention", "block_summary", "merge_summaries",
           "merge_lse", "decode_ref", "split_decode_ref", "paged_rows", "paged_decode_ref",
           "varlen_ref"]
