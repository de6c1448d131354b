"""GPU parity of fa_decode_paged (through the C ABI).

Against the fp64 oracle, which reads the pool through the block table, and
bit-identical to fa_decode on a contiguous cache holding the same values (the
split, the arithmetic and the merge are shared; only the addresses differ).
Pool slots past a sequence's length, the pad page that every unused table
entry names, and the contiguous cache's padding all hold NaN, so a stray read
fails the comparison.
"""
import numpy as np
import pytest
import torch

from io_aware_flashattention_amd import workloads as W
from oracle import decode_ref, paged_decode_ref
from tests.parity import check, say, to_dev

pytestmark = pytest.mark.gpu

EDGE_LENS = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 500, 699, 700]


def fa():
    import io_aware_flashattention_amd as m
    return m


def _pool_view(t: torch.Tensor, layout: str) -> torch.Tensor:
    """Pools are passed indexed [page, kv head, slot, d]."""
    return t if layout == "head" else t.transpose(1, 2)


@pytest.fixture(scope="module")
def edges():
    cfg = W.DecodeConfig("paged_edges", len(EDGE_LENS), 32, 4, 1, 700, 128, 91)
    lens = np.array(EDGE_LENS, dtype=np.int32)
    say("generating paged-edge inputs")
    q, kc, vc, _ = W.make_decode_inputs(cfg, pad="nan", lengths=lens)
    o_ref, l_ref = decode_ref(W.to_f64(q), W.to_f64(kc), W.to_f64(vc), lens, cfg.scale)
    dev = dict(q=to_dev(q), k=to_dev(kc), v=to_dev(vc), lens=torch.from_numpy(lens).to("cuda"))
    return cfg, lens, dev, (o_ref, l_ref)


@pytest.mark.parametrize("layout", ["head", "token"])
@pytest.mark.parametrize("ps", [16, 24, 32, 48, 64, 128, 256])
def test_paged_edges(edges, ps, layout):
    cfg, lens, dev, (o_ref, l_ref) = edges
    _, kp, vp, table, _ = W.make_paged_decode_inputs(cfg, ps, layout=layout, pad="nan", lengths=lens)
    kpd, vpd = _pool_view(to_dev(kp), layout), _pool_view(to_dev(vp), layout)
    tab = torch.from_numpy(table).to("cuda")
    for split in (0, 64, 200):
        say(f"case paged edges page_size={ps} layout={layout} split={split}")
        o_p, l_p = fa().decode_paged(dev["q"], kpd, vpd, tab, dev["lens"], scale=cfg.scale, split_tokens=split,
                                     out_dtype=torch.float32)
        o_c, l_c = fa().decode(dev["q"], dev["k"], dev["v"], dev["lens"], scale=cfg.scale, split_tokens=split,
                               out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o_p, o_c) and torch.equal(l_p, l_c), "paged and contiguous decode differ"
        o, l = o_p.cpu().numpy(), l_p.cpu().numpy()
        assert np.all(o[0] == 0) and np.all(np.isneginf(l[0]))          # empty sequence
        check(o[1:], l[1:], o_ref[1:], l_ref[1:], f"paged edges ps={ps} {layout} split={split}")


def test_paged_length_clamped_to_table_capacity():
    """A length above max_blocks * page_size reads the whole table and no more."""
    ps = 48
    cfg = W.DecodeConfig("paged_clamp", 3, 16, 2, 1, 700, 128, 93)
    cap = -(-cfg.max_len // ps) * ps                                   # 720
    lens = np.array([cap, 5, 300], dtype=np.int32)
    q, kp, vp, table, _ = W.make_paged_decode_inputs(cfg, ps, layout="head", pad="nan", lengths=lens)
    assert table.shape[1] * ps == cap
    say(f"case paged clamp page_size={ps} capacity={cap}")
    dev_lens = torch.tensor([cap + 1000, 5, 300], dtype=torch.int32, device="cuda")
    o, l = fa().decode_paged(to_dev(q), to_dev(kp), to_dev(vp), torch.from_numpy(table).to("cuda"), dev_lens,
                             scale=cfg.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, l_ref = paged_decode_ref(W.to_f64(q), W.to_f64(kp), W.to_f64(vp), table, lens, cfg.scale)
    check(o, l, o_ref, l_ref, "paged clamp")


SAMPLED = (0, 1, 2, 31, 62, 63)      # sequences the fp64 oracle computes at full size


@pytest.fixture(scope="module")
def c5_paged():
    cfg = W.DECODE_CONFIGS["c5_decode"]
    say(f"generating {cfg.name} inputs as a token-major pool of 16-token pages (NaN padding)")
    q, kp, vp, table, lens = W.make_paged_decode_inputs(cfg, 16, layout="token", pad="nan")
    say(f"computing oracle through the block table for sequences {SAMPLED}")
    # [page, slot, head, d] storage read as [page, head, slot, d]; rows widened per sequence
    o_ref, l_ref = paged_decode_ref(W.to_f64(q), kp.transpose(0, 2, 1, 3), vp.transpose(0, 2, 1, 3), table, lens,
                                    cfg.scale, batches=SAMPLED, values=W.to_f64)
    dev = dict(q=to_dev(q), k=to_dev(kp).transpose(1, 2), v=to_dev(vp).transpose(1, 2),
               table=torch.from_numpy(table).to("cuda"), lens=torch.from_numpy(lens).to("cuda"))
    return cfg, lens, dev, (o_ref, l_ref)


def test_c5_paged_full(c5_paged):
    cfg, lens, dev, (o_ref, l_ref) = c5_paged
    say(f"case {cfg.name} paged: B={cfg.batch} Hq={cfg.heads_q} Hkv={cfg.heads_kv} page_size=16 sum(L)={int(lens.sum())}")
    o32, l32 = fa().decode_paged(dev["q"], dev["k"], dev["v"], dev["table"], dev["lens"], scale=cfg.scale,
                                 out_dtype=torch.float32)
    o16, l16 = fa().decode_paged(dev["q"], dev["k"], dev["v"], dev["table"], dev["lens"], scale=cfg.scale,
                                 out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    idx = list(SAMPLED)
    check(o32[idx], l32[idx], o_ref[idx], l_ref[idx], cfg.name + " paged (sampled sequences)")
    check(o16[idx], l16[idx], o_ref[idx], l_ref[idx], cfg.name + " paged [bf16 out] (sampled sequences)")
    assert torch.equal(o16, o32.to(torch.bfloat16))
    assert torch.isfinite(o32).all() and torch.isfinite(l32).all()

    say("case c5 paged vs contiguous: the same values copied into a padded contiguous cache")
    B, Hkv, d = cfg.batch, cfg.heads_kv, cfg.head_dim
    kc = torch.full((B, Hkv, cfg.max_len, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    for b in range(B):
        t = torch.arange(int(lens[b]), device="cuda")
        pages = dev["table"][b, t // 16].long()
        kc[b, :, :len(t)] = dev["k"][pages, :, t % 16].transpose(0, 1)
        vc[b, :, :len(t)] = dev["v"][pages, :, t % 16].transpose(0, 1)
    o_c, l_c = fa().decode(dev["q"], kc, vc, dev["lens"], scale=cfg.scale, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o32, o_c) and torch.equal(l32, l_c), "paged and contiguous decode differ"
