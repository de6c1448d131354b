"""MI355X (gfx950) FlashAttention forward pass: prefill and split-KV decode.

The compute path is the C-ABI library ``libfa.so`` built from ``csrc/``;
``fwd`` and ``decode`` marshal torch tensors into it.
"""
