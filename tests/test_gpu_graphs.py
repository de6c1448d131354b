"""The entry points under HIP-graph capture. Each allocates nothing on its own
and only enqueues kernels on the caller's stream, so a captured sequence of
calls must replay to the eager launches' bits. Every replay runs after eager
work and a synchronisation, into outputs poisoned with NaN first, and is
compared element for element with the eager result."""
import numpy as np
import pytest
import torch

import io_aware_flashattention_amd as fa
from io_aware_flashattention_amd import workloads as W
from tests.parity import say, to_dev

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.contiguous().view(torch.uint8)


def _same(a, b):
    return a.shape == b.shape and a.dtype == b.dtype and torch.equal(_bits(a), _bits(b))


def test_entry_points_replay_to_the_eager_bits():
    dev = torch.device("cuda", 0)
    say("graph capture: prefill, packed prefill, backward, decode, FP8")
    q, k, v = (to_dev(x) for x in W.make_random_prefill(1, 8, 2, 300, 300, 128, seed=11, heavy_frac=0.01))
    g = to_dev(W.make_random_prefill(1, 8, 2, 300, 300, 128, seed=12)[0])
    lens = np.array([120, 0, 181], dtype=np.int64)
    vq, vk, vv, vcu = W.make_varlen_inputs(8, 2, 128, lens, seed=13)
    vq, vk, vv, vcu = to_dev(vq), to_dev(vk), to_dev(vv), torch.from_numpy(vcu).to(dev)
    dcfg = W.DecodeConfig("graph", batch=4, heads_q=8, heads_kv=2, head_dim=128, min_len=1, max_len=700, seed=14)
    dq, dk, dv, dlen = W.make_decode_inputs(dcfg, pad="zero")
    dq, dk, dv, dlen = to_dev(dq), to_dev(dk), to_dev(dv), torch.from_numpy(dlen).to(dev)
    signs = torch.from_numpy(np.random.default_rng(15).choice([-1.0, 1.0], 128).astype(np.float32)).to(dev)

    outs = dict(o=torch.empty_like(q, dtype=torch.float32), lse=torch.empty(1, 8, 300, device=dev),
                vo=torch.empty_like(vq), vlse=torch.empty(8, int(lens.sum()), device=dev),
                gq=torch.empty_like(q), gk=torch.empty_like(k), gv=torch.empty_like(v),
                do=torch.empty(4, 8, 128, dtype=torch.bfloat16, device=dev), dl=torch.empty(4, 8, device=dev),
                o8=torch.empty_like(q), l8=torch.empty(1, 8, 300, device=dev))
    ws_b = torch.empty(fa.load().fa_bwd_workspace_bytes(1, 8, 300), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(fa.decode_workspace_bytes(4, 8, 2, 700, 128, 0), dtype=torch.uint8, device=dev)
    held = {}

    def calls():
        fa.fwd(q, k, v, causal=True, out=outs["o"], lse=outs["lse"])
        fa.fwd_varlen(vq, vk, vv, vcu, int(lens.max()), causal=True, window=64, out=outs["vo"], lse=outs["vlse"])
        fa.bwd(q, k, v, outs["o"], g, outs["lse"], causal=True, dq=outs["gq"], dk=outs["gk"], dv=outs["gv"],
               workspace=ws_b)
        fa.decode(dq, dk, dv, dlen, out=outs["do"], lse=outs["dl"], workspace=ws_d)
        held["quant"] = fa.fp8_quantize(q, k, v, signs)
        fa.fwd_fp8(held["quant"], causal=True, out=outs["o8"], lse=outs["l8"])

    calls()
    torch.cuda.synchronize()
    want = {n: t.clone() for n, t in outs.items()}
    want.update({f"quant.{n}": t.clone() for n, t in held["quant"].items()})

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    other = torch.empty_like(q, dtype=torch.float32)
    for rep in range(3):
        for t in list(outs.values()) + [t for t in held["quant"].values() if t.is_floating_point()]:
            if t.is_floating_point() and t.dtype not in (torch.float8_e4m3fn,):
                t.fill_(float("nan"))
        fa.fwd(q, k, v, causal=False, out=other)           # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = dict(outs)
        got.update({f"quant.{n}": t for n, t in held["quant"].items()})
        bad = [n for n in want if not _same(got[n], want[n])]
        say(f"  replay {rep}: {'all equal' if not bad else 'differ: ' + ', '.join(bad)}")
        assert not bad, f"replay {rep}: {bad}"
