"""GPU parity of fa_fwd_varlen (through the C ABI): packed variable-length
prefill and the sliding-window mask, against the fp64 oracle, plus exact
agreement with fa_fwd where the two describe the same computation."""
import numpy as np
import pytest
import torch

from io_aware_flashattention_amd import workloads as W
from oracle import varlen_ref
from tests.parity import check, say, to_dev

pytestmark = pytest.mark.gpu

SMALL_LENS = [1, 63, 64, 65, 0, 255, 256, 257, 700, 1000]


def fa():
    import io_aware_flashattention_amd as m
    return m


def _run(q, k, v, cu, max_len, causal, window, out_dtype=torch.float32):
    o, lse = fa().fwd_varlen(q, k, v, cu, max_len, causal=causal, window=window, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return o, lse


@pytest.fixture(scope="module", params=[64, 128])
def small(request):
    d = request.param
    q, k, v, cu = W.make_varlen_inputs(8, 2, d, SMALL_LENS, seed=600 + d)
    dev = dict(q=to_dev(q), k=to_dev(k), v=to_dev(v), cu=torch.from_numpy(cu).to("cuda"))
    return d, (W.to_f64(q), W.to_f64(k), W.to_f64(v), cu), dev


@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, 0), (True, 1), (True, 63),
                                           (True, 64), (True, 100), (True, 1000)])
def test_varlen_small(small, causal, window):
    d, (q, k, v, cu), dev = small
    say(f"case varlen d={d} lens={SMALL_LENS} causal={causal} window={window}")
    o, lse = _run(dev["q"], dev["k"], dev["v"], dev["cu"], max(SMALL_LENS), causal, window)
    o_ref, l_ref = varlen_ref(q, k, v, cu, 1.0 / np.sqrt(d), causal=causal, window=window)
    check(o, lse, o_ref, l_ref, f"varlen d={d} causal={causal} window={window}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_uniform_varlen_is_dense(d, causal):
    """Equal lengths on a token-major layout: the same memory seen as a dense
    [B, H, N, d] strided view gives identical bits through fa_fwd."""
    B, N, Hq, Hkv = 3, 777, 8, 2
    say(f"case varlen == dense d={d} causal={causal}")
    q, k, v, cu = W.make_varlen_inputs(Hq, Hkv, d, [N] * B, seed=700 + d)
    qd, kd, vd, cud = to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(cu).to("cuda")
    o_v, l_v = _run(qd, kd, vd, cud, N, causal, None)
    view = lambda t: t.view(B, N, t.shape[1], d).transpose(1, 2)
    o_d = torch.empty(B * N, Hq, d, dtype=torch.float32, device="cuda")
    _, l_d = fa().fwd(view(qd), view(kd), view(vd), causal=causal, out=view(o_d))
    torch.cuda.synchronize()
    assert torch.equal(o_v, o_d)
    assert torch.equal(l_v, l_d.permute(1, 0, 2).reshape(Hq, B * N))


@pytest.mark.parametrize("d", [64, 128])
def test_window_covering_the_sequence_is_causal(d):
    lens = [300, 513]
    say(f"case window >= length is causal d={d}")
    q, k, v, cu = W.make_varlen_inputs(4, 4, d, lens, seed=800 + d)
    qd, kd, vd, cud = to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(cu).to("cuda")
    o_c, l_c = _run(qd, kd, vd, cud, 513, True, None)
    o_w, l_w = _run(qd, kd, vd, cud, 513, True, 512)
    assert torch.equal(o_c, o_w) and torch.equal(l_c, l_w)


def _sampled_rows(cu, extra):
    rows = set()
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        for r in [0, 1, 31, 32, 63, 64, 255, 256] + list(extra) + [s1 - s0 - 1, (s1 - s0) // 2]:
            if 0 <= r < s1 - s0:
                rows.add(s0 + r)
    return sorted(rows)


def test_window_8k():
    cfg = W.VARLEN_CONFIGS["c7_window_8k"]
    lens = W.varlen_lengths(cfg)
    say(f"case {cfg.name}: N={int(lens[0])} Hq={cfg.heads_q} Hkv={cfg.heads_kv} window={cfg.window}")
    q, k, v, cu = W.make_varlen_inputs(cfg.heads_q, cfg.heads_kv, cfg.head_dim, lens, seed=cfg.seed)
    o, lse = _run(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(cu).to("cuda"), int(lens.max()), True,
                  cfg.window)
    rows = _sampled_rows(cu, [1023, 1024, 1025, 1087, 1088, 1089, 4095, 4096, 8000])
    o_ref, l_ref = varlen_ref(q, k, v, cu, cfg.scale, causal=True, window=cfg.window, rows=rows, values=W.to_f64)
    check(o[rows], lse[:, rows], o_ref[rows], l_ref[:, rows], f"{cfg.name} (sampled rows {len(rows)})")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()


@pytest.mark.parametrize("causal,window", [(True, None), (False, None), (True, 200)])
def test_one_sequence_with_overstated_max_len(causal, window):
    """A packed batch of one sequence runs on the persistent grid. The
    caller's longest length (1500) overstates the sequence (700), so half the
    query-tile positions (6 per head, 3 real) lie past its end and are
    skipped, the heavy causal ones first. Hq64 Hkv8 d128: 384 positions on
    256 workgroups. Every 7th row of every head, and the tile edges."""
    lens = np.array([700])
    q, k, v, cu = W.make_varlen_inputs(64, 8, 128, lens, seed=777)
    say(f"case one sequence of 700 (max_len 1500) causal={causal} window={window}")
    o, lse = _run(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(cu).to("cuda"), 1500, causal, window)
    rows = sorted(set(range(0, 700, 7)) | {255, 256, 511, 512, 699})
    o_ref, l_ref = varlen_ref(q, k, v, cu, 1.0 / np.sqrt(128), causal=causal, window=window, rows=rows,
                              values=W.to_f64)
    check(o[rows], lse[:, rows], o_ref[rows], l_ref[:, rows], f"one sequence causal={causal} window={window}")


def test_varlen_mixed_lengths_gqa():
    cfg = W.VARLEN_CONFIGS["c6_varlen_causal"]
    lens = W.varlen_lengths(cfg)
    say(f"case {cfg.name}: {cfg.n_seqs} sequences, total {int(lens.sum())}, max {int(lens.max())}")
    q, k, v, cu = W.make_varlen_inputs(cfg.heads_q, cfg.heads_kv, cfg.head_dim, lens, seed=cfg.seed)
    dev = (to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(cu).to("cuda"))
    o, lse = _run(*dev, int(lens.max()), True, None)
    rows = _sampled_rows(cu, [])
    o_ref, l_ref = varlen_ref(q, k, v, cu, cfg.scale, causal=True, rows=rows, values=W.to_f64)
    check(o[rows], lse[:, rows], o_ref[rows], l_ref[:, rows], f"{cfg.name} (sampled rows {len(rows)})")
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    # bf16 output: the same arithmetic rounded once (short sequences have |O| up to ~4, where bf16
    # storage alone moves a value by up to 2^-7, so the oracle gate runs on the float32 output)
    o16, _ = _run(*dev, int(lens.max()), True, None, out_dtype=torch.bfloat16)
    assert torch.equal(o16, o.to(torch.bfloat16))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, 100)])
def test_varlen_kv_heads_per_xcd(d, causal, window):
    """Eight kv heads (a multiple of 8): each XCD takes one kv head of every
    sequence, the sequences one after another. Lengths include an empty and
    a one-token sequence, ragged tiles and a long tail."""
    lens = [300, 0, 1, 129, 64, 777, 31]
    say(f"case varlen kv heads per XCD d={d} lens={lens} causal={causal} window={window}")
    q, k, v, cu = W.make_varlen_inputs(16, 8, d, lens, seed=800 + d)
    dev = dict(q=to_dev(q), k=to_dev(k), v=to_dev(v), cu=torch.from_numpy(cu).to("cuda"))
    o, lse = _run(dev["q"], dev["k"], dev["v"], dev["cu"], max(lens), causal, window)
    o_ref, l_ref = varlen_ref(W.to_f64(q), W.to_f64(k), W.to_f64(v), cu, 1.0 / np.sqrt(d), causal=causal,
                              window=window)
    check(o, lse, o_ref, l_ref, f"varlen kv/XCD d={d} causal={causal} window={window}")
