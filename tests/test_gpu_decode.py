"""GPU parity of fa_decode (through the C ABI) against the fp64 oracle.

The cache rows past every sequence's length hold NaN, so any read beyond a
length poisons the output and fails the comparison.
"""
import numpy as np
import pytest
import torch

from io_aware_flashattention_amd import workloads as W
from oracle import attention_ref, decode_ref
from tests.parity import check, say, to_dev

pytestmark = pytest.mark.gpu


def fa():
    import io_aware_flashattention_amd as m
    return m


@pytest.fixture(scope="module")
def c5():
    cfg = W.DECODE_CONFIGS["c5_decode"]
    say(f"generating {cfg.name} inputs (NaN padding)")
    q, kc, vc, lens = W.make_decode_inputs(cfg, pad="nan")
    dev = dict(q=to_dev(q), k=to_dev(kc), v=to_dev(vc), lens=torch.from_numpy(lens).to("cuda"))
    say("computing oracle")
    o_ref, l_ref = _oracle(cfg, q, kc, vc, lens)
    return cfg, (q, kc, vc, lens), dev, (o_ref, l_ref)


def _oracle(cfg, q, kc, vc, lens):
    # per sequence, upcasting only the valid rows (the padding is never read)
    B = cfg.batch
    O = np.zeros((B, cfg.heads_q, cfg.head_dim))
    L = np.zeros((B, cfg.heads_q))
    for b in range(B):
        n = int(lens[b])
        o, l = decode_ref(W.to_f64(q[b:b + 1]), W.to_f64(kc[b:b + 1, :, :n]), W.to_f64(vc[b:b + 1, :, :n]),
                          np.array([n]), cfg.scale)
        O[b], L[b] = o[0], l[0]
    return O, L


def test_c5_decode_full(c5):
    cfg, host, dev, (o_ref, l_ref) = c5
    say(f"case {cfg.name}: B={cfg.batch} Hq={cfg.heads_q} Hkv={cfg.heads_kv} sum(L)={int(host[3].sum())}")
    o32, lse = fa().decode(dev["q"], dev["k"], dev["v"], dev["lens"], scale=cfg.scale, out_dtype=torch.float32)
    o16, lse16 = fa().decode(dev["q"], dev["k"], dev["v"], dev["lens"], scale=cfg.scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check(o32, lse, o_ref, l_ref, cfg.name)
    check(o16, lse16, o_ref, l_ref, cfg.name + " [bf16 out]")
    assert torch.equal(o16, o32.to(torch.bfloat16))


@pytest.mark.parametrize("split", [64, 256, 4096, 32768])
def test_split_size_invariance(c5, split):
    """Every split size meets the oracle bar. LSE is built from float32 sums and
    agrees across split sizes to float32 rounding; O moves slightly more,
    because each split rounds its probabilities to bf16 relative to its own
    running maximum before the P V product."""
    cfg, host, dev, (o_ref, l_ref) = c5
    say(f"case split={split}")
    o_a, l_a = fa().decode(dev["q"], dev["k"], dev["v"], dev["lens"], scale=cfg.scale, out_dtype=torch.float32)
    o_b, l_b = fa().decode(dev["q"], dev["k"], dev["v"], dev["lens"], scale=cfg.scale, out_dtype=torch.float32,
                           split_tokens=split)
    torch.cuda.synchronize()
    check(o_b, l_b, o_ref, l_ref, f"{cfg.name} split={split}")
    assert (l_a - l_b).abs().max().item() <= 1e-5
    assert (o_a - o_b).abs().max().item() <= 2e-3


def test_decode_equals_prefill_single_row(c5):
    cfg, host, dev, (o_ref, _) = c5
    o_dec, l_dec = fa().decode(dev["q"], dev["k"], dev["v"], dev["lens"], scale=cfg.scale, out_dtype=torch.float32)
    for b in (0, 17, 63):
        n = int(host[3][b])
        say(f"case decode vs prefill row b={b} L={n}")
        qb = dev["q"][b][None, :, None, :]
        o_p, l_p = fa().fwd(qb, dev["k"][b:b + 1, :, :n], dev["v"][b:b + 1, :, :n], causal=False,
                            scale=cfg.scale, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert (o_p[0, :, 0] - o_dec[b]).abs().max().item() <= 2e-3
        assert (l_p[0, :, 0] - l_dec[b]).abs().max().item() <= 1e-5


def test_small_lengths_and_edges():
    cfg = W.DecodeConfig("edges", 9, 16, 2, 1, 700, 128, 77)
    lens = np.array([0, 1, 63, 64, 65, 127, 500, 700, 900], dtype=np.int32)   # 900 > max: clamped to 700
    q, kc, vc, _ = W.make_decode_inputs(cfg, pad="nan", lengths=np.minimum(lens, 700))
    dev_lens = torch.from_numpy(lens).to("cuda")
    for split in (64, 128, 0):
        say(f"case decode edges split={split}")
        o, l = fa().decode(to_dev(q), to_dev(kc), to_dev(vc), dev_lens, scale=cfg.scale, split_tokens=split,
                           out_dtype=torch.float32)
        torch.cuda.synchronize()
        o, l = o.cpu().numpy(), l.cpu().numpy()
        assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))          # empty sequence
        eff = np.minimum(lens, 700)
        for b in range(1, 9):
            n = int(eff[b])
            ro, rl = attention_ref(W.to_f64(q[b])[None, :, None, :], W.to_f64(kc[b:b + 1, :, :n]),
                                   W.to_f64(vc[b:b + 1, :, :n]), cfg.scale)
            check(o[b], l[b], ro[0, :, 0], rl[0, :, 0], f"edges b={b} L={n} split={split}")


def test_huge_row_stride_takes_the_general_path():
    """Whole blocks load from one base plus 32-bit per-lane offsets over 32
    rows; a row (or page-slot) stride of 2^25 elements is past what those
    offsets hold, so these calls must take the clamped general path and still
    match the oracle. (About 12 GB of strided cache.)"""
    import gc
    d, L, stride = 128, 45, 1 << 25
    cfg = W.DecodeConfig("huge_stride", 1, 8, 1, 1, L, d, 79)
    q, kc, vc, _ = W.make_decode_inputs(cfg, pad="zero", lengths=np.array([L], dtype=np.int32))
    ro, rl = attention_ref(W.to_f64(q[0])[None, :, None, :], W.to_f64(kc), W.to_f64(vc), cfg.scale)
    lens = torch.tensor([L], dtype=torch.int32, device="cuda")
    say(f"case decode row stride {stride} elements, L={L}")
    bufs = []
    for x in (kc, vc):
        buf = torch.zeros((L, stride), dtype=torch.bfloat16, device="cuda")
        buf[:, :d] = to_dev(x)[0, 0]
        bufs.append(buf)
    k, v = (b.as_strided((1, 1, L, d), (L * stride, L * stride, stride, 1)) for b in bufs)
    o, l = fa().decode(to_dev(q), k, v, lens, scale=cfg.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check(o.cpu().numpy()[0], l.cpu().numpy()[0], ro[0, :, 0], rl[0, :, 0], "decode, huge row stride")
    del k, v, bufs
    gc.collect()
    torch.cuda.empty_cache()

    say(f"case paged decode slot stride {stride} elements, 16-slot pages")
    ps = 16
    npg = -(-L // ps)
    pools = []
    for x in (kc, vc):
        pool = torch.zeros((npg * ps, stride), dtype=torch.bfloat16, device="cuda")   # page p, slot s at row p*ps+s
        pool[:L, :d] = to_dev(x)[0, 0]
        pools.append(pool.as_strided((npg, 1, ps, d), (ps * stride, ps * stride, stride, 1)))
    table = torch.arange(npg, dtype=torch.int32, device="cuda")[None]
    o, l = fa().decode_paged(to_dev(q), pools[0], pools[1], table, lens, scale=cfg.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check(o.cpu().numpy()[0], l.cpu().numpy()[0], ro[0, :, 0], rl[0, :, 0], "paged decode, huge slot stride")
    del pools
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("B,Hq,Hkv,lo,hi", [(8, 12, 12, 1, 1024), (16, 32, 4, 100, 5000)],
                         ids=["gpt2_small_12x64", "gqa_32x4"])
def test_decode_head_dim_64(B, Hq, Hkv, lo, hi):
    """Decode at head_dim 64: GPT-2-small's heads (12 of 64, one kv head each,
    contexts of 1..1024 tokens, the pages' GPT-2 workload shape) and a GQA mix.
    Full oracle comparison for several split sizes; the paged form of the same
    cache (16-token pages, token-major, shuffled table) returns the same bits;
    NaN sits past every length in both."""
    cfg = W.DecodeConfig(f"d64_B{B}_Hq{Hq}_Hkv{Hkv}", B, Hq, Hkv, lo, hi, 64, 5100 + Hq)
    q, kc, vc, lens = W.make_decode_inputs(cfg, pad="nan")
    o_ref, l_ref = decode_ref(W.to_f64(q), W.to_f64(kc), W.to_f64(vc), lens, cfg.scale)
    qd, kd, vd, ld = to_dev(q), to_dev(kc), to_dev(vc), torch.from_numpy(lens).to("cuda")
    _, kp, vp, table, _ = W.make_paged_decode_inputs(cfg, 16, layout="token", pad="nan", lengths=lens)
    kpd, vpd, tab = to_dev(kp).transpose(1, 2), to_dev(vp).transpose(1, 2), torch.from_numpy(table).to("cuda")
    for split in (0, 64, 1000):
        say(f"case {cfg.name} split={split} sum(L)={int(lens.sum())}")
        o32, l32 = fa().decode(qd, kd, vd, ld, scale=cfg.scale, split_tokens=split, out_dtype=torch.float32)
        o16, _ = fa().decode(qd, kd, vd, ld, scale=cfg.scale, split_tokens=split, out_dtype=torch.bfloat16)
        op, lp = fa().decode_paged(qd, kpd, vpd, tab, ld, scale=cfg.scale, split_tokens=split,
                                   out_dtype=torch.float32)
        torch.cuda.synchronize()
        check(o32, l32, o_ref, l_ref, f"{cfg.name} split={split}")
        assert torch.equal(o16, o32.to(torch.bfloat16))
        assert torch.equal(op, o32) and torch.equal(lp, l32), "paged and contiguous decode differ"
