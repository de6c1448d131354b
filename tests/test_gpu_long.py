"""Long contexts against the fp64 oracle: a 131,072-token causal GQA prefill
and a packed batch holding a 131,072-token sequence under a 4,096-token
window, on sampled rows, and decode over caches of up to 131,072 tokens in
full, contiguous and paged (the paged form bit for bit the contiguous one).
Offsets, tile counters and the decode's token ranges all grow with the
length, so these are the sizes where an index kept in too narrow a type
would show."""
import numpy as np
import pytest
import torch

import io_aware_flashattention_amd as fa
from io_aware_flashattention_amd import workloads as W
from oracle import attention_ref, varlen_ref
from tests.parity import check, say, to_dev

pytestmark = pytest.mark.gpu

N = 131072


def test_prefill_128k_causal_sampled_rows():
    say(f"case prefill B1 Hq8 Hkv1 N{N} d128 causal (1% of K rows x8)")
    q, k, v = W.make_random_prefill(1, 8, 1, N, N, 128, seed=21, heavy_frac=0.01)
    scale = 1 / np.sqrt(128)
    o, lse = fa.fwd(to_dev(q), to_dev(k), to_dev(v), causal=True, scale=scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    k64, v64 = W.to_f64(k), W.to_f64(v)
    rng = np.random.default_rng(21)
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for h in range(8):
        r = {0, 1, 63, 64, 255, 256, N // 2, N - 257, N - 256, N - 65, N - 64, N - 2, N - 1}
        r |= set(rng.integers(0, N, 24).tolist())
        r = np.array(sorted(r))
        ro, rl = attention_ref(W.to_f64(q[:, h:h + 1, r]), k64, v64, scale, causal=True, q_positions=r)
        got_o.append(o[0, h, r]); got_l.append(lse[0, h, r]); ref_o.append(ro[0, 0]); ref_l.append(rl[0, 0])
    check(np.concatenate(got_o), np.concatenate(got_l), np.concatenate(ref_o), np.concatenate(ref_l),
          f"prefill N{N} [{sum(len(x) for x in got_o)} sampled rows]")


def test_decode_128k_caches():
    lens = np.array([N, 5, 70001], dtype=np.int32)
    cfg = W.DecodeConfig("long", 3, 16, 2, 1, N, 128, 22)
    say(f"case decode B3 Hq16 Hkv2 lengths {lens.tolist()} (NaN padding)")
    q, kc, vc, _ = W.make_decode_inputs(cfg, pad="nan", lengths=lens)
    o, l = fa.decode(to_dev(q), to_dev(kc), to_dev(vc), torch.from_numpy(lens).to("cuda"), scale=cfg.scale,
                     out_dtype=torch.float32)
    torch.cuda.synchronize()
    o, l = o.cpu().numpy(), l.cpu().numpy()
    for b in range(3):
        n = int(lens[b])
        ro, rl = attention_ref(W.to_f64(q[b])[None, :, None, :], W.to_f64(kc[b:b + 1, :, :n]),
                               W.to_f64(vc[b:b + 1, :, :n]), cfg.scale)
        check(o[b], l[b], ro[0, :, 0], rl[0, :, 0], f"decode b={b} L={n}")


def test_packed_128k_window_sampled_rows():
    lens = np.array([3000, N, 1], dtype=np.int64)
    W_ = 4096
    say(f"case packed lengths {lens.tolist()} Hq8 Hkv1 d128 causal window {W_}")
    q, k, v, cu = W.make_varlen_inputs(8, 1, 128, lens, seed=23)
    o, lse = fa.fwd_varlen(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(cu).to("cuda"), int(lens.max()),
                           causal=True, window=W_, out_dtype=torch.float32)
    torch.cuda.synchronize()
    s0 = int(cu[1])
    rng = np.random.default_rng(23)
    local = {0, 1, W_ - 1, W_, W_ + 1, W_ + 63, W_ + 64, N // 2, N - 65, N - 64, N - 1}
    local |= set(rng.integers(0, N, 24).tolist())
    rows = [0, 1, 2999] + [s0 + r for r in sorted(local)] + [int(cu[2])]
    o_ref, l_ref = varlen_ref(q, k, v, cu, 1 / np.sqrt(128), causal=True, window=W_, rows=rows, values=W.to_f64)
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    check(o[rows], lse[:, rows], o_ref[rows], l_ref[:, rows], f"packed N{N} window {W_} [{len(rows)} sampled rows]")


def test_paged_decode_128k_equals_contiguous():
    lens = np.array([N, 5, 70001], dtype=np.int32)
    cfg = W.DecodeConfig("long", 3, 16, 2, 1, N, 128, 22)
    say(f"case paged decode B3 Hq16 Hkv2 lengths {lens.tolist()}, 16-token token-major pages")
    q, kc, vc, _ = W.make_decode_inputs(cfg, pad="nan", lengths=lens)
    dev_lens = torch.from_numpy(lens).to("cuda")
    o_c, l_c = fa.decode(to_dev(q), to_dev(kc), to_dev(vc), dev_lens, scale=cfg.scale, out_dtype=torch.float32)
    del kc, vc
    q2, kp, vp, table, _ = W.make_paged_decode_inputs(cfg, 16, layout="token", pad="nan", lengths=lens)
    assert np.array_equal(q2, q)
    o_p, l_p = fa.decode_paged(to_dev(q), to_dev(kp).transpose(1, 2), to_dev(vp).transpose(1, 2),
                               torch.from_numpy(table).to("cuda"), dev_lens, scale=cfg.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_c) and torch.equal(l_p, l_c)
