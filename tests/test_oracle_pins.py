"""Pins for the fp64 oracle against facts fixed outside it: the pages' worked
examples, closed forms, a pure-Python brute force, scipy's softmax and
logsumexp, and invariants of softmax attention. CPU only."""
import math

import numpy as np
import pytest
import scipy.special
from hypothesis import given, settings
from hypothesis import strategies as st

from oracle import (attention_bwd_ref, attention_ref, block_summary, decode_ref, merge_lse, merge_summaries,
                    paged_decode_ref, paged_rows, split_decode_ref, stream_attention, varlen_ref)
from tests.conftest import golden


def _close(x, spec):
    return abs(x - spec["value"]) <= spec["tol"]


def _row_problem(scores, values):
    """One query row whose scores (scale 1) are exactly ``scores``: q = e0, k_j = s_j e0."""
    n = len(scores)
    values = np.asarray(values, dtype=np.float64).reshape(n, -1)
    q = np.zeros((1, 1, 1, 2))
    q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, n, 2))
    k[0, 0, :, 0] = scores
    return q, k, values[None, None]


# ------------------------------------------------------------ page examples --

def test_t1_four_scores_direct():
    g = golden("t1_four_scores.json")
    q, k, v = _row_problem(g["scores"], g["values"])
    O, L = attention_ref(q, k, v, scale=1.0)
    assert _close(O[0, 0, 0, 0], g["final"]["output"])
    assert _close(L[0, 0, 0], g["lse_derived"])
    assert _close(math.exp(L[0, 0, 0]), g["exp_sum_no_shift"])
    # with V = I the output row is the probability row itself
    P, _ = attention_ref(q, k, np.eye(4)[None, None], scale=1.0)
    for p, want in zip(P[0, 0, 0], g["probabilities"]["value"]):
        assert abs(p - want) <= g["probabilities"]["tol"]
    # l relative to the global max 3 is exp(LSE - 3)
    assert _close(math.exp(L[0, 0, 0] - 3.0), g["final"]["l"])


def test_t1_four_scores_streaming_states():
    g = golden("t1_four_scores.json")
    q, k, v = _row_problem(g["scores"], g["values"])
    states = []
    O, L = stream_attention(q, k, v, 1.0, causal=False, Br=1, Bc=g["tile"],
                            trace=lambda b, h, i, j, m, l, a, al: states.append((m[0], l[0], a[0, 0], al[0])))
    assert len(states) == 2
    m, l, a, _ = states[0]
    assert m == g["after_tile_A"]["m"]
    assert _close(l, g["after_tile_A"]["l"]) and _close(a, g["after_tile_A"]["o_unnormalised"])
    m, l, a, alpha = states[1]
    assert m == g["final"]["m"]
    assert _close(alpha, g["correction_factor"])
    assert _close(l, g["final"]["l"]) and _close(a, g["final"]["o_unnormalised"])
    assert _close(O[0, 0, 0, 0], g["final"]["output"])
    assert _close(L[0, 0, 0], g["lse_derived"])


def test_t2_block_merge():
    g = golden("t2_block_merge.json")
    (m1, l1), (m2, l2) = (block_summary(b) for b in g["blocks"])
    assert m1 == g["summary_1"]["m"] and _close(l1, g["summary_1"]["l"])
    assert m2 == g["summary_2"]["m"] and _close(l2, g["summary_2"]["l"])
    m, l = merge_summaries(m1, l1, m2, l2)
    assert m == g["merged"]["m"] and _close(l, g["merged"]["l"])
    assert _close(math.exp(m2 - m) * l2, g["shrink_factor_block_2"])
    md, ld = block_summary(sum(g["blocks"], []))
    assert md == m and abs(ld - l) < 1e-14


def test_t3_two_tile_trace():
    g = golden("t3_two_tile_trace.json")
    q, k, v = _row_problem(g["scores"], g["values"])
    O, L = attention_ref(q, k, v, scale=1.0)
    for o, want in zip(O[0, 0, 0], g["output"]["value"]):
        assert abs(o - want) <= g["output"]["tol"]
    assert _close(L[0, 0, 0], g["lse_derived"])
    W, _ = attention_ref(q, k, np.eye(4)[None, None], scale=1.0)
    for w, want in zip(W[0, 0, 0], g["weights"]["value"]):
        assert abs(w - want) <= g["weights"]["tol"]
    states = []
    O2, _ = stream_attention(q, k, v, 1.0, causal=False, Br=1, Bc=g["tile"],
                             trace=lambda b, h, i, j, m, l, a, al: states.append((m[0], l[0], a[0].copy(), al[0])))
    (m1, l1, a1, _), (m2, l2, a2, al2) = states
    assert m1 == g["tile_1"]["m"] and _close(l1, g["tile_1"]["l"])
    assert all(abs(x - w) <= g["tile_1"]["a"]["tol"] for x, w in zip(a1, g["tile_1"]["a"]["value"]))
    assert m2 == g["tile_2"]["m"] and _close(al2, g["tile_2"]["alpha"]) and _close(l2, g["tile_2"]["l"])
    assert all(abs(x - w) <= g["tile_2"]["a"]["tol"] for x, w in zip(a2, g["tile_2"]["a"]["value"]))
    assert np.allclose(O2, O, rtol=0, atol=1e-14)


def test_t4_causal_tile_behaviour_in_streaming_reference():
    """Query tile 5 (1-based) at Br=128, Bc=64: loads tiles 1..10, and tile 10
    leaves rows 513..576 untouched; dropping the mask changes the answer."""
    g = golden("t4_causal_tiles.json")
    Br, Bc = g["Br"], g["Bc"]
    n = g["rows"][1]                      # rows up to 640 reproduce tile 5's geometry
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((1, 1, n, 4)) for _ in range(3))
    seen = {}

    def tr(b, h, i, j, m, l, a, al):
        if i == g["query_tile"] - 1:
            seen[j] = (l.copy(), al.copy())
    O, L = stream_attention(q, k, v, 0.5, causal=True, Br=Br, Bc=Bc, trace=tr)
    assert sorted(seen) == list(range(g["loaded_tiles"][0] - 1, g["loaded_tiles"][1]))
    lo, hi = g["tile_10_silent_rows"][0] - 1 - (g["query_tile"] - 1) * Br, g["tile_10_silent_rows"][1] - (g["query_tile"] - 1) * Br
    l9, _ = seen[8]
    l10, al10 = seen[9]
    assert np.array_equal(l10[lo:hi], l9[lo:hi]) and np.all(al10[lo:hi] == 1.0)
    Oref, Lref = attention_ref(q, k, v, 0.5, causal=True)
    assert np.abs(O - Oref).max() < 1e-12 and np.abs(L - Lref).max() < 1e-12
    Onm, _ = stream_attention(q, k, v, 0.5, causal=True, Br=Br, Bc=Bc, apply_mask=False)
    rows = slice((g["query_tile"] - 1) * Br, n)
    assert np.abs(Onm[0, 0, rows] - Oref[0, 0, rows]).max() > 1e-2


# -------------------------------------------------------------- brute force --

def _brute(q, k, v, scale, causal):
    """Scalar loops with math.exp / math.fsum, no arrays, no max shift beyond
    what the exponent range needs (inputs are kept small)."""
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    O = np.zeros((B, Hq, Nq, v.shape[3]))
    L = np.zeros((B, Hq, Nq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for r in range(Nq):
                cols = [c for c in range(Nk) if not (causal and c > r)]
                s = [scale * math.fsum(float(q[b, h, r, t]) * float(k[b, g, c, t]) for t in range(d)) for c in cols]
                e = [math.exp(x) for x in s]
                z = math.fsum(e)
                L[b, h, r] = math.log(z)
                for t in range(v.shape[3]):
                    O[b, h, r, t] = math.fsum(e[i] * float(v[b, g, c, t]) for i, c in enumerate(cols)) / z
    return O, L


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 3), (1, 2, 1, 5, 3), (2, 4, 2, 7, 4), (1, 3, 3, 6, 2)])
def test_brute_force_tiny(shape, causal):
    B, Hq, Hkv, N, d = shape
    rng = np.random.default_rng(hash((shape, causal)) % 2**32)
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d + 1))
    O, L = attention_ref(q, k, v, 0.7, causal=causal)
    Ob, Lb = _brute(q, k, v, 0.7, causal)
    assert np.abs(O - Ob).max() < 1e-12
    assert np.abs(L - Lb).max() < 1e-12


def test_against_scipy_softmax_and_logsumexp():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 37, 16))
    k = rng.standard_normal((1, 1, 53, 16))
    v = rng.standard_normal((1, 1, 53, 16))
    O, L = attention_ref(q, k, v, 0.25)
    S = 0.25 * np.einsum("id,jd->ij", q[0, 0], k[0, 0])
    assert np.abs(L[0, 0] - scipy.special.logsumexp(S, axis=1)).max() < 1e-12
    assert np.abs(O[0, 0] - scipy.special.softmax(S, axis=1) @ v[0, 0]).max() < 1e-12
    # causal: each row's logsumexp over its visible prefix
    q2 = rng.standard_normal((1, 1, 40, 8))
    k2 = rng.standard_normal((1, 1, 40, 8))
    v2 = rng.standard_normal((1, 1, 40, 8))
    O2, L2 = attention_ref(q2, k2, v2, 0.5, causal=True)
    for r in range(40):
        s = 0.5 * k2[0, 0, :r + 1] @ q2[0, 0, r]
        assert abs(L2[0, 0, r] - scipy.special.logsumexp(s)) < 1e-12
        assert np.abs(O2[0, 0, r] - scipy.special.softmax(s) @ v2[0, 0, :r + 1]).max() < 1e-12


# ------------------------------------------------------------- closed forms --

def test_closed_form_causal_first_row():
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((2, 3, 33, 8)) for _ in range(3))
    O, L = attention_ref(q, k, v, 0.3, causal=True)
    assert np.abs(O[:, :, 0] - v[:, :, 0]).max() < 1e-14
    assert np.abs(L[:, :, 0] - 0.3 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0])).max() < 1e-13


def test_closed_form_zero_query_is_mean():
    rng = np.random.default_rng(12)
    q = np.zeros((1, 2, 20, 8))
    k, v = (rng.standard_normal((1, 2, 20, 8)) for _ in range(2))
    O, L = attention_ref(q, k, v, 1.0)
    assert np.abs(O - v.mean(axis=2, keepdims=True)).max() < 1e-14
    assert np.abs(L - math.log(20)).max() < 1e-14
    Oc, Lc = attention_ref(q, k, v, 1.0, causal=True)
    prefix = np.cumsum(v, axis=2) / np.arange(1, 21)[None, None, :, None]
    assert np.abs(Oc - prefix).max() < 1e-13
    assert np.abs(Lc - np.log(np.arange(1, 21))[None, None]).max() < 1e-14


def test_closed_form_single_key_and_dominant_key():
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((1, 1, 1, 8)) for _ in range(3))
    O, L = attention_ref(q, k, v, 0.9)
    assert np.abs(O - v).max() < 1e-15 and abs(L[0, 0, 0] - 0.9 * float(q[0, 0, 0] @ k[0, 0, 0])) < 1e-14
    # one key 200 above every other score: its value row wins to ~1e-80
    k = np.zeros((1, 1, 6, 2))
    k[0, 0, :, 0] = [0, 1, 2, 202, -3, 1]
    qq = np.array([[[[1.0, 0.0]]]])
    vv = rng.standard_normal((1, 1, 6, 3))
    O, L = attention_ref(qq, k, vv, 1.0)
    assert np.abs(O[0, 0, 0] - vv[0, 0, 3]).max() < 1e-12 and abs(L[0, 0, 0] - 202.0) < 1e-12


def test_large_scores_do_not_overflow():
    q = np.full((1, 1, 3, 1), 100.0)
    k = np.array([[[[10.0], [9.0], [8.0]]]])
    v = np.array([[[[1.0], [2.0], [3.0]]]])
    O, L = attention_ref(q, k, v, 1.0)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    w = np.exp(np.array([0.0, -100.0, -200.0]))
    assert abs(O[0, 0, 0, 0] - (w @ [1, 2, 3]) / w.sum()) < 1e-12
    assert abs(L[0, 0, 0] - 1000.0 - math.log(w.sum())) < 1e-9


# --------------------------------------------------------------- invariants --

@settings(max_examples=25, deadline=None)
@given(n=st.integers(1, 40), d=st.sampled_from([1, 3, 8]), causal=st.booleans(),
       seed=st.integers(0, 2**31 - 1))
def test_invariants(n, d, causal, seed):
    rng = np.random.default_rng(seed)
    q, k, v = (rng.standard_normal((1, 1, n, d)) for _ in range(3))
    O, L = attention_ref(q, k, v, 0.8, causal=causal)
    S = 0.8 * q[0, 0] @ k[0, 0].T
    for r in range(n):
        vis = slice(0, r + 1) if causal else slice(0, n)
        cnt = (r + 1) if causal else n
        smax = S[r, vis].max()
        assert smax - 1e-12 <= L[0, 0, r] <= smax + math.log(cnt) + 1e-12
        lo, hi = v[0, 0, vis].min(axis=0), v[0, 0, vis].max(axis=0)
        assert np.all(O[0, 0, r] >= lo - 1e-12) and np.all(O[0, 0, r] <= hi + 1e-12)
    # adding a constant to every value row shifts O by that constant
    O2, _ = attention_ref(q, k, v + 1.5, 0.8, causal=causal)
    assert np.abs(O2 - O - 1.5).max() < 1e-12


def test_key_permutation_invariance_unmasked():
    rng = np.random.default_rng(21)
    q, k, v = (rng.standard_normal((1, 2, 30, 8)) for _ in range(3))
    perm = rng.permutation(30)
    O, L = attention_ref(q, k, v, 0.4)
    O2, L2 = attention_ref(q, k[:, :, perm], v[:, :, perm], 0.4)
    assert np.abs(O - O2).max() < 1e-13 and np.abs(L - L2).max() < 1e-13


def test_gqa_equals_explicitly_replicated_heads():
    """Query head h reads kv head h // G: same as repeating each kv head G times."""
    rng = np.random.default_rng(22)
    G, Hkv = 4, 2
    q = rng.standard_normal((2, G * Hkv, 17, 8))
    k, v = (rng.standard_normal((2, Hkv, 17, 8)) for _ in range(2))
    for causal in (False, True):
        O, L = attention_ref(q, k, v, 0.5, causal=causal)
        Or, Lr = attention_ref(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), 0.5, causal=causal)
        assert np.array_equal(O, Or) and np.array_equal(L, Lr)
        # and the mapping is not the interleaved one
        Oi, _ = attention_ref(q, np.tile(k, (1, G, 1, 1)), np.tile(v, (1, G, 1, 1)), 0.5, causal=causal)
        assert np.abs(Oi - O).max() > 1e-3


def test_row_subset_matches_full():
    rng = np.random.default_rng(23)
    q, k, v = (rng.standard_normal((1, 2, 50, 8)) for _ in range(3))
    O, L = attention_ref(q, k, v, 0.5, causal=True)
    rows = np.array([0, 7, 31, 49])
    Os, Ls = attention_ref(q[:, :, rows], k, v, 0.5, causal=True, q_positions=rows)
    assert np.abs(Os - O[:, :, rows]).max() < 1e-14 and np.abs(Ls - L[:, :, rows]).max() < 1e-14


def test_row_blocking_does_not_change_result():
    rng = np.random.default_rng(24)
    q, k, v = (rng.standard_normal((1, 1, 70, 8)) for _ in range(3))
    O, L = attention_ref(q, k, v, 0.5, causal=True)
    O2, L2 = attention_ref(q, k, v, 0.5, causal=True, row_block=16)
    assert np.abs(O - O2).max() < 1e-15 and np.abs(L - L2).max() < 1e-15


@settings(max_examples=20, deadline=None)
@given(n=st.integers(1, 70), Br=st.sampled_from([1, 4, 16, 32]), Bc=st.sampled_from([1, 3, 8, 16]),
       causal=st.booleans(), seed=st.integers(0, 2**31 - 1))
def test_streaming_recurrence_equals_materialised(n, Br, Bc, causal, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 2, n, 4))
    k, v = (rng.standard_normal((1, 1, n, 4)) for _ in range(2))
    k[0, 0, rng.integers(0, n)] *= 8.0
    O, L = stream_attention(q, k, v, 0.6, causal=causal, Br=Br, Bc=Bc)
    Or, Lr = attention_ref(q, k, v, 0.6, causal=causal)
    assert np.abs(O - Or).max() < 1e-12 and np.abs(L - Lr).max() < 1e-12


# ---------------------------------------------------------- merge / decode --

@settings(max_examples=20, deadline=None)
@given(n=st.integers(1, 60), split=st.integers(1, 64), seed=st.integers(0, 2**31 - 1))
def test_split_merge_identity(n, split, seed):
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, d, Lmax = 2, 4, 2, 4, 64
    q = rng.standard_normal((B, Hq, d))
    kc = rng.standard_normal((B, Hkv, Lmax, d))
    vc = rng.standard_normal((B, Hkv, Lmax, d))
    lens = np.array([n, max(1, n // 2)])
    O, L = decode_ref(q, kc, vc, lens, 0.5)
    O2, L2 = split_decode_ref(q, kc, vc, lens, 0.5, split)
    assert np.abs(O - O2).max() < 1e-12 and np.abs(L - L2).max() < 1e-12


def test_decode_ignores_padding_and_matches_prefill_row():
    rng = np.random.default_rng(31)
    B, Hq, Hkv, d, Lmax = 3, 4, 2, 8, 40
    q = rng.standard_normal((B, Hq, d))
    kc = rng.standard_normal((B, Hkv, Lmax, d))
    vc = rng.standard_normal((B, Hkv, Lmax, d))
    lens = np.array([40, 1, 17])
    for b in range(B):
        kc[b, :, lens[b]:] = np.nan
        vc[b, :, lens[b]:] = np.nan
    O, L = decode_ref(q, kc, vc, lens, 0.35)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    for b in range(B):
        n = lens[b]
        Op, Lp = attention_ref(q[b][None, :, None], kc[b:b + 1, :, :n], vc[b:b + 1, :, :n], 0.35)
        assert np.abs(Op[0, :, 0] - O[b]).max() < 1e-15
    # a length-1 sequence returns its only value row
    assert np.abs(O[1] - np.repeat(vc[1, :, 0], Hq // Hkv, axis=0)).max() < 1e-15


def test_no_key_gives_zero_output_and_minus_inf_lse():
    rng = np.random.default_rng(43)
    q = rng.standard_normal((1, 2, 3, 4))
    O, L = attention_ref(q, np.zeros((1, 1, 0, 4)), np.zeros((1, 1, 0, 5)), 0.5)
    assert O.shape == (1, 2, 3, 5) and np.all(O == 0) and np.all(np.isneginf(L))
    kc = rng.standard_normal((2, 1, 6, 4))
    O, L = decode_ref(q[0, :, 0][None].repeat(2, 0), kc, kc, np.array([0, 6]), 0.5)
    assert np.all(O[0] == 0) and np.all(np.isneginf(L[0])) and np.all(np.isfinite(L[1]))


def test_merge_lse_edge_cases():
    rng = np.random.default_rng(41)
    o = rng.standard_normal((3, 4))
    lse = rng.standard_normal(3)
    o1, l1 = merge_lse([(o, lse)])
    assert np.abs(o1 - o).max() < 1e-15 and np.abs(l1 - lse).max() < 1e-15
    o2, l2 = merge_lse([(o, lse), (np.zeros((3, 4)), np.full(3, -np.inf))])
    assert np.abs(o2 - o).max() < 1e-15 and np.abs(l2 - lse).max() < 1e-15
    o3, l3 = merge_lse([(o, lse), (o, lse)])
    assert np.abs(o3 - o).max() < 1e-15 and np.abs(l3 - lse - math.log(2)).max() < 1e-14


# ------------------------------------------------------------- paged cache --

def test_paged_rows_hand_example():
    """Page size 4, table [2, 0, 1]: tokens 0-3 live in page 2, 4-7 in page 0,
    8 in page 1 (slot = token mod 4). Entry values encode page, head and slot."""
    P, H, ps, d = 3, 2, 4, 1
    pool = np.zeros((P, H, ps, d))
    for pg in range(P):
        for h in range(H):
            for sl in range(ps):
                pool[pg, h, sl, 0] = 1000 * pg + 100 * h + sl
    table = np.array([[2, 0, 1, 77]])          # the last entry is past the 9 tokens: never read
    rows = paged_rows(pool, table, 0, 9)
    assert rows.shape == (H, 9, d)
    assert rows[1, :, 0].tolist() == [2100, 2101, 2102, 2103, 100, 101, 102, 103, 1100]
    assert rows[0, :, 0].tolist() == [2000, 2001, 2002, 2003, 0, 1, 2, 3, 1000]
    assert paged_rows(pool, table, 0, 0).shape == (H, 0, d)


@pytest.mark.parametrize("ps", [4, 16, 24])
@pytest.mark.parametrize("token_major", [False, True])
def test_paged_decode_equals_contiguous(ps, token_major):
    """A contiguous cache copied page by page into a shuffled pool gives the
    identical decode result; slots past a length hold NaN and table entries
    past the last block are out of range, so any stray read fails."""
    rng = np.random.default_rng(51 + ps)
    B, Hq, Hkv, d, Lmax = 3, 4, 2, 8, 70
    q = rng.standard_normal((B, Hq, d))
    kc = rng.standard_normal((B, Hkv, Lmax, d))
    vc = rng.standard_normal((B, Hkv, Lmax, d))
    lens = np.array([70, 1, 33])
    nblk = [-(-int(n) // ps) for n in lens]
    P = sum(nblk)
    order = rng.permutation(P)
    table = np.full((B, -(-Lmax // ps)), 10 ** 9, dtype=np.int64)
    kpool = np.full((P, Hkv, ps, d), np.nan)
    vpool = np.full((P, Hkv, ps, d), np.nan)
    nxt = 0
    for b in range(B):
        for j in range(nblk[b]):
            pg = order[nxt]
            nxt += 1
            table[b, j] = pg
            for sl in range(ps):
                t = j * ps + sl
                if t < lens[b]:
                    kpool[pg, :, sl] = kc[b, :, t]
                    vpool[pg, :, sl] = vc[b, :, t]
    if token_major:    # same values stored [page, slot, head, d], read through a strided view
        kpool = np.ascontiguousarray(kpool.transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)
        vpool = np.ascontiguousarray(vpool.transpose(0, 2, 1, 3)).transpose(0, 2, 1, 3)
    O, L = decode_ref(q, kc, vc, lens, 0.3)
    Op, Lp = paged_decode_ref(q, kpool, vpool, table, lens, 0.3)
    assert np.array_equal(O, Op) and np.array_equal(L, Lp)


@pytest.mark.parametrize("ps,layout", [(16, "head"), (24, "token"), (64, "token")])
def test_paged_workload_holds_the_decode_values(ps, layout):
    from io_aware_flashattention_amd import workloads as W
    cfg = W.DecodeConfig("paged_pin", 3, 8, 2, 1, 200, 128, 777)
    lens = np.array([200, 1, 77], dtype=np.int32)
    q, kc, vc, _ = W.make_decode_inputs(cfg, lengths=lens)
    q2, kp, vp, table, lens2 = W.make_paged_decode_inputs(cfg, ps, layout=layout, lengths=lens)
    assert np.array_equal(q, q2) and np.array_equal(lens, lens2)
    view = (lambda x: x) if layout == "head" else (lambda x: x.transpose(0, 2, 1, 3))
    for b in range(cfg.batch):
        n = int(lens[b])
        assert np.array_equal(paged_rows(view(kp), table, b, n), kc[b, :, :n])
        assert np.array_equal(paged_rows(view(vp), table, b, n), vc[b, :, :n])
    nblk = [-(-int(n) // ps) for n in lens]
    used = np.concatenate([table[b, :nblk[b]] for b in range(cfg.batch)])
    assert len(set(used.tolist())) == len(used) == kp.shape[0] - 1     # distinct pages plus one pad page
    pad_page = (set(range(kp.shape[0])) - set(used.tolist())).pop()
    assert np.all(kp[pad_page] == W.BF16_NAN)
    for b in range(cfg.batch):
        assert np.all(table[b, nblk[b]:] == pad_page)


# ---------------------------------------------------------- sliding window --

@pytest.mark.parametrize("W", [0, 1, 5, 17, 100])
def test_window_closed_form_with_zero_query(W):
    """q = 0 gives equal weights over the visible keys: with V[c] = c the output
    of row r is the mean of lo..r, lo = max(0, r - W), and LSE = ln(r - lo + 1)."""
    N = 40
    q = np.zeros((1, 1, N, 4))
    k = np.random.default_rng(W).standard_normal((1, 1, N, 4))
    v = np.arange(N, dtype=np.float64).reshape(1, 1, N, 1)
    O, L = attention_ref(q, k, v, 0.7, causal=True, window=W)
    for r in range(N):
        lo = max(0, r - W)
        assert abs(O[0, 0, r, 0] - (lo + r) / 2) < 1e-12
        assert abs(L[0, 0, r] - math.log(r - lo + 1)) < 1e-12


def test_window_brute_force():
    rng = np.random.default_rng(61)
    N, d, W, scale = 13, 3, 4, 0.6
    q = rng.standard_normal((N, d))
    k = rng.standard_normal((N, d))
    v = rng.standard_normal((N, 2))
    O, L = attention_ref(q[None, None], k[None, None], v[None, None], scale, causal=True, window=W)
    for r in range(N):
        vis = [c for c in range(N) if c <= r and r - c <= W]
        sc = [scale * sum(q[r, i] * k[c, i] for i in range(d)) for c in vis]
        mx = max(sc)
        w = [math.exp(x - mx) for x in sc]
        tot = sum(w)
        for j in range(2):
            assert abs(O[0, 0, r, j] - sum(wi * v[c, j] for wi, c in zip(w, vis)) / tot) < 1e-12
        assert abs(L[0, 0, r] - (mx + math.log(tot))) < 1e-12


def test_window_limits():
    rng = np.random.default_rng(62)
    q, k, v = (rng.standard_normal((1, 2, 30, 8)) for _ in range(3))
    Oc, Lc = attention_ref(q, k, v, 0.3, causal=True)
    Ow, Lw = attention_ref(q, k, v, 0.3, causal=True, window=29)
    assert np.array_equal(Oc, Ow) and np.array_equal(Lc, Lw)          # a window as long as the sequence
    O0, L0 = attention_ref(q, k, v, 0.3, causal=True, window=0)     # each row sees only itself
    assert np.array_equal(O0, v)
    assert np.allclose(L0, 0.3 * np.einsum("bhnd,bhnd->bhn", q, k), rtol=0, atol=1e-13)
    with pytest.raises(AssertionError):
        attention_ref(q, k, v, 0.3, causal=False, window=4)


# ------------------------------------------------------ packed sequences ----

def _packed(rng, lens, Hq=4, Hkv=2, d=8):
    total = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return (rng.standard_normal((total, Hq, d)), rng.standard_normal((total, Hkv, d)),
            rng.standard_normal((total, Hkv, d)), cu)


@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, 3)])
def test_varlen_brute_force(causal, window):
    """Every packed row attends to the keys of its own sequence only: the rule is
    written over global token indices with a sequence-id array."""
    rng = np.random.default_rng(71)
    lens = [5, 0, 1, 7]
    q, k, v, cu = _packed(rng, lens, Hq=2, Hkv=1, d=3)
    O, L = varlen_ref(q, k, v, cu, 0.8, causal=causal, window=window)
    seq = np.repeat(np.arange(len(lens)), lens)
    start = cu[seq]
    for r in range(len(seq)):
        for h in range(2):
            vis = [c for c in range(len(seq)) if seq[c] == seq[r]
                   and (not causal or c <= r) and (window is None or r - c <= window)]
            sc = [0.8 * sum(q[r, h, i] * k[c, 0, i] for i in range(3)) for c in vis]
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = sum(w)
            for j in range(3):
                assert abs(O[r, h, j] - sum(wi * v[c, 0, j] for wi, c in zip(w, vis)) / tot) < 1e-12
            assert abs(L[h, r] - (mx + math.log(tot))) < 1e-12
    assert np.all(start <= np.arange(len(seq)))


def test_varlen_sequences_are_isolated_and_order_free():
    rng = np.random.default_rng(72)
    lens = [9, 4, 12]
    q, k, v, cu = _packed(rng, lens)
    O, L = varlen_ref(q, k, v, cu, 0.5, causal=True)
    k2, v2 = k.copy(), v.copy()
    k2[cu[1]:cu[2]] += 3.0                      # change only sequence 1
    v2[cu[1]:cu[2]] -= 1.0
    O2, L2 = varlen_ref(q, k2, v2, cu, 0.5, causal=True)
    for b in (0, 2):
        sl = slice(cu[b], cu[b + 1])
        assert np.array_equal(O[sl], O2[sl]) and np.array_equal(L[:, sl], L2[:, sl])
    assert not np.allclose(O[cu[1]:cu[2]], O2[cu[1]:cu[2]])
    order = [2, 0, 1]                           # pack the same sequences in another order
    idx = np.concatenate([np.arange(cu[b], cu[b + 1]) for b in order])
    cu3 = np.concatenate([[0], np.cumsum([lens[b] for b in order])])
    O3, L3 = varlen_ref(q[idx], k[idx], v[idx], cu3, 0.5, causal=True)
    assert np.array_equal(O3, O[idx]) and np.array_equal(L3, L[:, idx])


def test_varlen_single_sequence_is_dense_and_rows_subset():
    rng = np.random.default_rng(73)
    q, k, v, cu = _packed(rng, [33], Hq=4, Hkv=2, d=8)
    O, L = varlen_ref(q, k, v, cu, 0.4, causal=True, window=7)
    Od, Ld = attention_ref(q.transpose(1, 0, 2)[None], k.transpose(1, 0, 2)[None], v.transpose(1, 0, 2)[None],
                           0.4, causal=True, window=7)
    assert np.array_equal(O, Od[0].transpose(1, 0, 2)) and np.array_equal(L, Ld[0])
    rows = [0, 5, 32]
    Os, Ls = varlen_ref(q, k, v, cu, 0.4, causal=True, window=7, rows=rows)
    assert np.array_equal(Os[rows], O[rows]) and np.array_equal(Ls[:, rows], L[:, rows])
    others = [r for r in range(33) if r not in rows]
    assert np.all(Os[others] == 0) and np.all(np.isneginf(Ls[:, others]))


# ---------------------------------------------------------------- backward --

def _loss_grad_fd(q, k, v, w, scale, causal, window, which, idx, eps=1e-6):
    """Central difference of L = sum(O * w) with respect to one input entry."""
    args = {"q": q.copy(), "k": k.copy(), "v": v.copy()}
    vals = []
    for sgn in (1, -1):
        a = {n: x.copy() for n, x in args.items()}
        a[which][idx] += sgn * eps
        O, _ = attention_ref(a["q"], a["k"], a["v"], scale, causal=causal, window=window)
        vals.append(float((O * w).sum()))
    return (vals[0] - vals[1]) / (2 * eps)


@pytest.mark.parametrize("causal,window", [(False, None), (True, None), (True, 2)])
def test_backward_matches_finite_differences(causal, window):
    rng = np.random.default_rng(81)
    B, Hq, Hkv, N, d, scale = 1, 4, 2, 7, 3, 0.7
    q = rng.standard_normal((B, Hq, N, d))
    k = rng.standard_normal((B, Hkv, N, d))
    v = rng.standard_normal((B, Hkv, N, d))
    w = rng.standard_normal((B, Hq, N, d))                  # dO = dL/dO for L = sum(O * w)
    dq, dk, dv, _ = attention_bwd_ref(q, k, v, w, scale, causal=causal, window=window)
    for which, grad, shape in (("q", dq, q.shape), ("k", dk, k.shape), ("v", dv, v.shape)):
        for flat in rng.choice(int(np.prod(shape)), size=12, replace=False):
            idx = np.unravel_index(int(flat), shape)
            fd = _loss_grad_fd(q, k, v, w, scale, causal, window, which, idx)
            assert abs(fd - grad[idx]) < 1e-7, (which, idx, fd, grad[idx])


def test_backward_matches_torch_autograd_fp64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(82)
    B, Hq, Hkv, N, d, scale = 2, 4, 2, 9, 5, 0.45
    q, do = rng.standard_normal((B, Hq, N, d)), rng.standard_normal((B, Hq, N, d))
    k, v = rng.standard_normal((B, Hkv, N, d)), rng.standard_normal((B, Hkv, N, d))
    for causal in (False, True):
        tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
        kk = tk.repeat_interleave(Hq // Hkv, dim=1)
        vv = tv.repeat_interleave(Hq // Hkv, dim=1)
        s = scale * torch.matmul(tq, kk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
        o = torch.matmul(torch.softmax(s, dim=-1), vv)
        o.backward(torch.tensor(do))
        dq, dk, dv, _ = attention_bwd_ref(q, k, v, do, scale, causal=causal)
        assert np.abs(dq - tq.grad.numpy()).max() < 1e-12
        assert np.abs(dk - tk.grad.numpy()).max() < 1e-12
        assert np.abs(dv - tv.grad.numpy()).max() < 1e-12


def test_backward_row_term_identity_and_invariants():
    """D is rowsum(dO * O); softmax ignores a shift added to every key, so the
    key gradients sum to zero; with dO = 1 each row of P sums to one, so the
    value gradients sum to the number of rows."""
    rng = np.random.default_rng(83)
    B, H, N, d, scale = 1, 2, 11, 4, 0.6
    q, k, v, do = (rng.standard_normal((B, H, N, d)) for _ in range(4))
    dq, dk, dv, D = attention_bwd_ref(q, k, v, do, scale, causal=True)
    O, _ = attention_ref(q, k, v, scale, causal=True)
    assert np.abs(D - (do * O).sum(axis=3)).max() < 1e-13
    # softmax is invariant to adding the same vector to every key: sum_j dK_j = 0
    assert np.abs(dk.sum(axis=2)).max() < 1e-12
    # dV sums P^T dO: with dO = 1 everywhere, every row of P sums to one, so sum_j dV_j = N per column
    _, _, dv1, _ = attention_bwd_ref(q, k, v, np.ones_like(do), scale, causal=True)
    assert np.abs(dv1.sum(axis=2) - N).max() < 1e-12
