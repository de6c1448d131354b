"""fa_decode_noalloc (through the C ABI) against fa_decode.

The no-alloc entry point runs fa_decode's kernels with the partials in the
library's static scratch instead of a caller's workspace, so on the same
inputs it must return fa_decode's bits. Two calls in a row, the second with a
smaller input, show that the scratch's leftover contents from the first call
do not leak into the second (nothing in it has to start at zero). Both are
also held to the oracle bar.
"""
import numpy as np
import pytest
import torch

from io_aware_flashattention_amd import workloads as W
from oracle import decode_ref
from tests.parity import check, say, to_dev

pytestmark = pytest.mark.gpu


def fa():
    import io_aware_flashattention_amd as m
    return m


def _inputs(cfg):
    q, kc, vc, lens = W.make_decode_inputs(cfg, pad="nan")
    o_ref, l_ref = decode_ref(W.to_f64(q), W.to_f64(kc), W.to_f64(vc), lens, cfg.scale)
    dev = (to_dev(q), to_dev(kc), to_dev(vc), torch.from_numpy(lens).to("cuda"))
    return dev, (o_ref, l_ref)


def test_noalloc_matches_decode_on_two_calls_in_a_row():
    big = W.DecodeConfig("noalloc_big", 16, 64, 8, 1024, 8192, 128, 6101)
    small = W.DecodeConfig("noalloc_small", 3, 16, 2, 1, 700, 64, 6102)
    for cfg, split in ((big, 0), (small, 64)):
        (q, k, v, lens), (o_ref, l_ref) = _inputs(cfg)
        B, Hq = cfg.batch, cfg.heads_q
        say(f"case decode_noalloc {cfg.name} d={cfg.head_dim} split={split} "
            f"workspace {fa().decode_workspace_bytes(B, Hq, cfg.heads_kv, cfg.max_len, cfg.head_dim, split)} B")
        o_n = torch.empty(B, Hq, cfg.head_dim, dtype=torch.float32, device="cuda")
        l_n = torch.empty(B, Hq, dtype=torch.float32, device="cuda")
        fa().decode_noalloc(q, k, v, lens, o_n, l_n, scale=cfg.scale, split_tokens=split)
        o_w, l_w = fa().decode(q, k, v, lens, scale=cfg.scale, split_tokens=split, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o_n, o_w) and torch.equal(l_n, l_w), f"{cfg.name}: noalloc != decode"
        check(o_n, l_n, o_ref, l_ref, f"decode_noalloc {cfg.name}")


def test_noalloc_rejects_sizes_past_its_scratch():
    """A request whose partials need more than the static 16 MiB fails before
    any launch, with the reason in the message."""
    lib = fa().load()
    need = fa().decode_workspace_bytes(4096, 64, 8, 1024, 128, 0)
    assert need > fa()._lib.DECODE_SCRATCH_BYTES
    q = torch.zeros(4096, 64, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(4096, 8, 16, 128, dtype=torch.bfloat16, device="cuda")
    lens = torch.ones(4096, dtype=torch.int32, device="cuda")
    out = torch.empty(4096, 64, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fa().FaError, match="static scratch"):
        fa().decode_noalloc(q, kc, kc, lens, out)
    assert "static scratch" in lib.fa_last_error_message().decode()
