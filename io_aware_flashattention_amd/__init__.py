"""MI355X (gfx950) FlashAttention: prefill, its backward, and split-KV decode.

The compute path is the C-ABI library ``libfa.so`` built from ``csrc/``;
``fwd``, ``fwd_varlen``, ``bwd``, ``fp8_quantize``, ``fwd_fp8``, ``decode``,
``decode_noalloc`` and ``decode_paged`` marshal torch tensors into it and raise
if it is missing or refuses a call.
"""
from ._lib import (FaError, bwd, decode, decode_noalloc, decode_paged, decode_workspace_bytes, fp8_quantize, fwd,
                   fwd_fp8, fwd_varlen, load)

__all__ = ["fwd", "fwd_varlen", "bwd", "fp8_quantize", "fwd_fp8", "decode", "decode_noalloc", "decode_paged",
           "decode_workspace_bytes", "load", "FaError"]
