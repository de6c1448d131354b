"""GPU parity of fa_fwd (through the C ABI) against the fp64 oracle.

Small and ragged shapes are checked element by element in full, and so is
the long-context GQA workload at 8192 tokens (all 524,288 rows). The others
are checked in full where the oracle finishes in seconds and otherwise on
sampled rows of every head: first, last, tile-boundary and heavy-key rows,
and at least one row of every 32-row block of every head, so of every work
item (the persistent kernel streams K/V tiles and query rows across items,
so a fault tied to one ring position would show only on the rows of the
items it hits).
"""
import numpy as np
import pytest
import torch

from io_aware_flashattention_amd import workloads as W
from oracle import attention_ref
from tests.parity import check, say, to_dev

pytestmark = pytest.mark.gpu


def fa():
    import io_aware_flashattention_amd as m
    return m


def run_and_check(q, k, v, causal, scale, what, rows=None, heads=None, bf16_direct=False):
    """Run fa_fwd with fp32 output (and bf16 output), compare with the oracle.

    The bar is applied to the float32 output everywhere; the bf16 output must
    be that result rounded once to nearest even, bit for bit. ``bf16_direct``
    also applies the bar to the bf16 output itself (the mid-length workload,
    whose output is bf16 by definition and stays below 4 in magnitude, so its
    storage rounding is at most 2^-8)."""
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    say(f"case {what}: q{tuple(q.shape)} k{tuple(k.shape)} causal={causal}")
    o32, lse = fa().fwd(qd, kd, vd, causal=causal, scale=scale, out_dtype=torch.float32)
    o16, lse16 = fa().fwd(qd, kd, vd, causal=causal, scale=scale, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # the bf16 output is the float32 result rounded once, to nearest even
    assert torch.equal(o16, o32.to(torch.bfloat16)), f"{what}: bf16 out != RNE(fp32 out)"
    assert torch.equal(lse16, lse)
    q64, k64, v64 = W.to_f64(q), W.to_f64(k), W.to_f64(v)
    if rows is None:
        o_ref, l_ref = attention_ref(q64, k64, v64, scale, causal=causal)
        check(o32, lse, o_ref, l_ref, what)
        if bf16_direct:
            check(o16, lse16, o_ref, l_ref, what + " [bf16 out]")
        else:
            e = np.abs(o16.float().cpu().numpy() - o_ref)
            say(f"  {what} [bf16 out, reported]: O max {e.max():.3e} mean {e.mean():.3e}")
        return
    o_h = o32.cpu().numpy()
    l_h = lse.cpu().numpy()
    B, Hq = q.shape[:2]
    G = Hq // k.shape[1]
    errs = []
    for b in range(B):
        for h in (range(Hq) if heads is None else heads):
            r = rows(b, h)
            o_ref, l_ref = attention_ref(q64[b:b + 1, h:h + 1, r], k64[b:b + 1, h // G:h // G + 1],
                                         v64[b:b + 1, h // G:h // G + 1], scale, causal=causal, q_positions=r)
            errs.append((o_h[b, h, r], l_h[b, h, r], o_ref[0, 0], l_ref[0, 0]))
    o_g = np.concatenate([e[0] for e in errs])
    l_g = np.concatenate([e[1] for e in errs])
    o_r = np.concatenate([e[2] for e in errs])
    l_r = np.concatenate([e[3] for e in errs])
    check(o_g, l_g, o_r, l_r, what + f" [{len(o_g)} sampled rows]")


SMALL = [
    # B, Hq, Hkv, Nq, Nk, d, causal, dtype
    (1, 1, 1, 1, 1, 64, False, "bf16"),
    (1, 1, 1, 1, 1, 128, True, "bf16"),
    (1, 2, 1, 37, 37, 64, True, "bf16"),
    (2, 4, 2, 100, 100, 128, True, "bf16"),
    (1, 2, 2, 129, 129, 128, False, "bf16"),
    (1, 8, 2, 200, 200, 128, True, "bf16"),
    (2, 3, 1, 255, 255, 64, True, "bf16"),
    (1, 2, 1, 300, 300, 128, False, "bf16"),
    (1, 2, 2, 50, 333, 128, False, "bf16"),
    (1, 2, 1, 64, 1, 128, False, "bf16"),
    (1, 1, 1, 513, 513, 64, True, "bf16"),
    (1, 2, 1, 77, 77, 64, True, "fp32"),
    (1, 2, 2, 130, 130, 128, False, "fp32"),
    (1, 4, 1, 640, 640, 128, True, "bf16"),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s[:6])) + ("c" if s[6] else "n") + s[7])
def test_small_and_ragged(shape):
    B, Hq, Hkv, Nq, Nk, d, causal, dtype = shape
    q, k, v = W.make_random_prefill(B, Hq, Hkv, Nq, Nk, d, dtype, seed=101 + Nq, heavy_frac=0.02)
    run_and_check(q, k, v, causal, 1.0 / np.sqrt(d), f"small {shape}")


def test_c1_single_head_fp32():
    cfg = W.CONFIGS["c1_single_head_fp32"]
    q, k, v = W.make_prefill_inputs(cfg)
    run_and_check(q, k, v, cfg.causal, cfg.scale, cfg.name)


def test_c2_gpt2_causal():
    cfg = W.CONFIGS["c2_gpt2_causal"]
    q, k, v = W.make_prefill_inputs(cfg)
    run_and_check(q, k, v, cfg.causal, cfg.scale, cfg.name)


def _per_item_rows(n, seed):
    """One row inside every 32-row block, at a seeded offset: a work item
    holds 256 rows of one head, or under the causal mask 256 / h rows of h
    heads that share a kv head (h up to 8), so every item of every head is
    sampled."""
    rng = np.random.default_rng([seed, 32])
    return {min(n - 1, i + int(rng.integers(0, 32))) for i in range(0, n, 32)}


def _sample_rows(n, seed, extra=()):
    rng = np.random.default_rng(seed)
    base = {0, 1, 63, 64, 127, 128, 129, n // 2, n - 129, n - 128, n - 2, n - 1}
    base |= set(rng.integers(0, n, 12).tolist()) | set(int(x) for x in extra if 0 <= x < n)
    base |= _per_item_rows(n, seed)
    return np.array(sorted(base))


@pytest.mark.parametrize("name", ["c3_mid_causal", "c3_mid_none"])
def test_c3_mid_length(name):
    cfg = W.CONFIGS[name]
    q, k, v = W.make_prefill_inputs(cfg)
    run_and_check(q, k, v, cfg.causal, cfg.scale, name,
                  rows=lambda b, h: _sample_rows(cfg.seqlen, 1000 * b + h), bf16_direct=False)
    # two heads in full, bf16 output checked directly as well
    for b, h in [(0, 0), (3, 31)]:
        run_and_check(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], cfg.causal, cfg.scale,
                      f"{name} head ({b},{h}) full", bf16_direct=True)


def test_c4a_long_context_gqa_full():
    """The headline workload (B1 Hq64 Hkv8 N8192 d128, causal, 1% of K rows
    x8) compared in full: every element of O (float32 out) and every LSE
    against the fp64 oracle (about 30 s of oracle on 16 host cores); the bf16
    output equals RNE(float32 output) bit for bit."""
    cfg = W.CONFIGS["c4a_gqa_8k"]
    q, k, v = W.make_prefill_inputs(cfg)
    run_and_check(q, k, v, cfg.causal, cfg.scale, cfg.name + " [all rows]")


def test_c4b_long_context_gqa_sampled():
    cfg = W.CONFIGS["c4b_gqa_16k"]
    q, k, v = W.make_prefill_inputs(cfg)

    def rows(b, h):
        heavy = W.heavy_rows(cfg, b, h // cfg.group)
        return _sample_rows(cfg.seqlen, 7 * h + 1, extra=list(heavy[:4]) + list(heavy[:4] + 1) + list(heavy[-3:]))
    run_and_check(q, k, v, cfg.causal, cfg.scale, cfg.name, rows=rows)


@pytest.mark.parametrize("B,causal", [(2, True), (3, False)])
def test_persistent_items_with_ragged_tiles(B, causal):
    """More work items than workgroups, so every workgroup of the persistent
    grid takes two or three, with a ragged last key tile: B x Hq64 Hkv8
    N1000 d128 (4 query tiles per head; 512 or 768 items). K/V tiles and query
    rows then stream across item boundaries, and items start in every stage
    of the ring (16 key tiles per non-causal item; 4..16 under the mask).
    Sampled rows of every head: first and last, tile edges, and one more."""
    q, k, v = W.make_random_prefill(B, 64, 8, 1000, 1000, 128, seed=4242 + B, heavy_frac=0.01)
    base = [0, 1, 63, 64, 255, 256, 257, 511, 512, 767, 768, 960, 998, 999]

    def rows(b, h):
        return np.array(sorted(set(base) | {(37 * h + 11 * b) % 1000}))
    run_and_check(q, k, v, causal, 1 / np.sqrt(128), f"persistent B{B} N1000 causal={causal}", rows=rows)


# (B, Hq, Hkv, N, causal): 1 to 5 items per workgroup of the persistent grid,
# kv groups of 1, 2, 4, 8 and 16 (under the causal mask: items of 1, 2, 4 and
# 8 heads, and two 8-head items per kv head), ragged and whole last key tiles
SWEEP = [(1, 128, 128, 700, True), (2, 96, 48, 517, False), (4, 64, 8, 384, True), (1, 256, 32, 1100, True),
         (3, 40, 5, 830, False), (2, 160, 20, 960, True), (2, 32, 16, 900, True), (1, 64, 16, 777, True),
         (1, 64, 4, 1000, True)]


@pytest.mark.parametrize("shape", SWEEP, ids=lambda s: "x".join(map(str, s[:4])) + ("c" if s[4] else "n"))
def test_persistent_shape_sweep(shape):
    """Seeded shapes whose item counts give the persistent workgroups one to
    five items each; sampled rows of every head (edges, tile boundaries, a
    head-dependent row, and one row inside every 32-row block)."""
    B, Hq, Hkv, N, causal = shape
    q, k, v = W.make_random_prefill(B, Hq, Hkv, N, N, 128, seed=900 + N, heavy_frac=0.02)
    edges = [0, 1, 63, 64, 255, 256, N // 2, N - 65, N - 64, N - 2, N - 1]

    def rows(b, h):
        return np.array(sorted({r for r in edges if 0 <= r < N} | {(53 * h + 17 * b) % N}
                               | _per_item_rows(N, 1000 * b + h)))
    run_and_check(q, k, v, causal, 1 / np.sqrt(128), f"sweep B{B} Hq{Hq} Hkv{Hkv} N{N} causal={causal}", rows=rows)


def test_gqa_bit_identical_to_replicated_kv():
    q, k, v = W.make_random_prefill(2, 8, 2, 300, 300, 128, seed=5, heavy_frac=0.01)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    kr = kd.repeat_interleave(4, dim=1).contiguous()
    vr = vd.repeat_interleave(4, dim=1).contiguous()
    for causal in (False, True):
        say(f"case gqa vs replicated causal={causal}")
        o1, l1 = fa().fwd(qd, kd, vd, causal=causal, out_dtype=torch.float32)
        o2, l2 = fa().fwd(qd, kr, vr, causal=causal, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_strided_views_and_no_lse():
    """q/k/v/o given as [B, N, H, d] storage viewed as [B, H, N, d]."""
    B, H, N, d = 2, 4, 200, 128
    q, k, v = W.make_random_prefill(B, H, H, N, N, d, seed=9)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    qs, ks, vs = (t.transpose(1, 2).contiguous().transpose(1, 2) for t in (qd, kd, vd))
    assert not qs.is_contiguous()
    say("case strided views")
    o_ref, l_ref = fa().fwd(qd, kd, vd, causal=True, out_dtype=torch.float32)
    o_store = torch.empty(B, N, H, d, device="cuda", dtype=torch.float32)
    o_s, none = fa().fwd(qs, ks, vs, causal=True, out=o_store.transpose(1, 2), lse=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(o_s, o_ref)


def test_repeat_runs_bit_identical():
    q, k, v = W.make_random_prefill(1, 8, 1, 1000, 1000, 128, seed=3)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    say("case determinism")
    o1, l1 = fa().fwd(qd, kd, vd, causal=True)
    o2, l2 = fa().fwd(qd, kd, vd, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_unsupported_raises_not_falls_back():
    q = torch.zeros(1, 1, 16, 96, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(fa().FaError):
        fa().fwd(q, q, q)
    q = torch.zeros(1, 1, 16, 64, device="cuda", dtype=torch.float16)
    with pytest.raises(ValueError):
        fa().fwd(q, q, q)
