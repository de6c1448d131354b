"""Plain fp64 CPU oracle for exact softmax attention.

TEST INFRASTRUCTURE ONLY. Nothing in the product path imports, links or runs
this module; only the tests, the smoke check and the benchmark's CPU-baseline
leg may call it. It shares no code with the HIP path: the one common input is
the seeded generator in ``io_aware_flashattention_amd.workloads``, which holds
no attention arithmetic and is not imported here (callers pass arrays in).

What it computes, and where the pages define it:

* ``attention_ref`` -- materialising attention, S = scale * Q K^T, the causal
  mask added before the softmax, P = softmax(S) with the row maximum
  subtracted, O = P V, and the per-row log-sum-exp L = m + ln(l).
  ("How FlashAttention Reduces HBM Traffic Exactly", section "The performance
  problem is data movement, not the attention formula"; "FlashAttention and
  GPU Data Movement" section 1, the three-kernel baseline; "FlashAttention
  Explained: IO-Aware Attention, Tiling, Online Softmax and FP8 on Hopper",
  sections "Safe softmax, then online softmax" and "Why the statistics are
  cheap to store".)  Library matmul is the only primitive used.
* ``stream_attention`` -- the FlashAttention-2 tile recurrence (query tiles
  outer, key/value tiles inner, running max m, running sum l, unnormalised
  accumulator a, one division at the end), with the causal skip bound and the
  diagonal mask kept as two separate steps.  ("FlashAttention and GPU Data
  Movement" sections 2, 2.1 and 3.1; "FlashAttention Explained" section "The
  tile recurrence".)  It exists to reproduce the pages' intermediate states;
  it is not the oracle's definition of the result.
* ``merge_summaries`` / ``merge_lse`` -- combining two block summaries
  (max, sum) and combining split partials by their log-sum-exp.
  ("FlashAttention, annotated" section 3.1 "Softmax in pieces"; "How
  FlashAttention Reduces HBM Traffic Exactly" section "Why softmax does not
  prevent tiling"; "FlashAttention Explained" section "Decoding, Paged and
  Split-KV Variants".)
* ``attention_ref(..., window=W)`` -- the sliding-window mask on top of the
  causal one: row r sees keys r - W .. r (the pages' example keeps a key when
  q_idx >= kv_idx and q_idx - kv_idx <= W; "FlashAttention Explained",
  section "FlexAttention"; "FlashAttention and Why Attention Is a
  Memory-Traffic Problem": windows skip every block outside them).
* ``varlen_ref`` -- packed variable-length batches: sequences concatenated on
  the token axis with cumulative offsets cu_seqlens, each attending only to
  itself ("FlashAttention Explained", section "Trade-offs, Gotchas, and What
  Goes Wrong": varlen kernels skip pad tokens given cumulative lengths).
* ``attention_bwd_ref`` -- gradients of the forward pass for an incoming dO:
  dV = P^T dO, dP = dO V^T, D = rowsum(dO * O), dS = P * (dP - D),
  dQ = scale dS K, dK = scale dS^T Q, with P recomputed from the scores
  ("FlashAttention Explained", section "Backward Pass: Recomputation Beats
  Storage"; "How FlashAttention Reduces HBM Traffic Exactly", section
  "Training: recomputation replaces saved attention probabilities"). Under
  GQA a kv head's dK and dV sum the contributions of its query heads.
* ``decode_ref`` -- single-token decode: the same attention for one query row
  per head over the first L_b cached keys of each sequence.
* ``paged_rows`` / ``paged_decode_ref`` -- the same decode over a paged cache:
  fixed-size pages addressed through a per-sequence block table, token t of
  a sequence in slot t mod page_size of the page that the table names for
  logical block floor(t / page_size). ("FlashAttention Explained" section
  "Decoding, Paged and Split-KV Variants": the cache lives in non-contiguous
  fixed-size blocks found through a block table.)

Readings where the pages are silent (each listed in the design notes):
GQA maps query head h to kv head h // (Hq / Hkv); key c is visible to query
row r under the causal mask iff c <= r (same length for queries and keys, or
an explicit absolute position per query row); the log-sum-exp is natural-log
over the scaled, masked scores; a row with no visible key has O = 0 and
L = -inf.
"""
from __future__ import annotations

import math

import numpy as np

_ROW_BLOCK = 1024


def _as64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _softmax_rows(S: np.ndarray):
    """Safe softmax of each row of S (entries may be -inf).

    Returns (P, m, l): P = exp(S - m) / l with m the row max and l the row sum
    of exp(S - m). Rows whose entries are all -inf, or that have no entries
    (no key at all), get P = 0, m = -inf, l = 0.
    """
    m = S.max(axis=1, initial=-np.inf)
    live = np.isfinite(m)
    shift = np.where(live, m, 0.0)
    E = np.exp(S - shift[:, None])          # exp(-inf) = 0 for masked entries
    l = E.sum(axis=1)
    P = np.zeros_like(E)
    P[live] = E[live] / l[live, None]
    if live.any():
        err = np.abs(P[live].sum(axis=1) - 1.0).max()
        assert err <= 1e-12, f"softmax rows do not sum to 1 (err {err})"
    return P, m, l


def attention_ref(q, k, v, scale: float, causal: bool = False, q_positions=None,
                  row_block: int = _ROW_BLOCK, window=None):
    """Materialising attention in fp64.

    q: [B, Hq, Nq, d]; k: [B, Hkv, Nk, d]; v: [B, Hkv, Nk, dv]; Hq % Hkv == 0.
    q_positions: absolute key-axis position of each query row (default 0..Nq-1),
    used only by the masks, so a subset of rows can be checked alone.
    window: sliding-window size W (with ``causal``): key c is also masked when
    it lies more than W positions behind the row, so a row sees keys
    [row - W, row].
    Returns O [B, Hq, Nq, dv] and LSE [B, Hq, Nq], both fp64.
    """
    assert window is None or (causal and window >= 0), "a window is defined on top of the causal mask"
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nk, dk = k.shape
    assert Bk == B and dk == d and v.shape[:3] == k.shape[:3]
    assert Hq % Hkv == 0, "query heads must be a multiple of kv heads"
    G = Hq // Hkv
    pos = np.arange(Nq) if q_positions is None else np.asarray(q_positions, dtype=np.int64)
    assert pos.shape == (Nq,)
    cols = np.arange(Nk)
    O = np.zeros((B, Hq, Nq, v.shape[3]))
    L = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            K = k[b, h // G]
            V = v[b, h // G]
            for r0 in range(0, Nq, row_block):
                r1 = min(Nq, r0 + row_block)
                S = scale * (q[b, h, r0:r1] @ K.T)
                if causal:
                    S[cols[None, :] > pos[r0:r1, None]] = -np.inf
                if window is not None:
                    S[cols[None, :] < pos[r0:r1, None] - window] = -np.inf
                P, m, l = _softmax_rows(S)
                O[b, h, r0:r1] = P @ V
                live = l > 0
                L[b, h, r0:r1][live] = m[live] + np.log(l[live])
    return O, L


def attention_bwd_ref(q, k, v, do, scale: float, causal: bool = False, window=None, row_block: int = _ROW_BLOCK):
    """Gradients of attention_ref's O with respect to q, k and v, given dO.

    q, do: [B, Hq, N, d]; k, v: [B, Hkv, N, d]. Returns dQ, dK, dV (shapes of
    q, k, v) and D = rowsum(dO * O) [B, Hq, N], all fp64. P is recomputed per
    block of rows from the scores and the row statistics, never stored whole.
    """
    q, k, v, do = _as64(q), _as64(k), _as64(v), _as64(do)
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    O, _ = attention_ref(q, k, v, scale, causal=causal, window=window, row_block=row_block)
    D = (do * O).sum(axis=3)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    rows, cols = np.arange(Nq), np.arange(Nk)
    for b in range(B):
        for h in range(Hq):
            K, V = k[b, h // G], v[b, h // G]
            for r0 in range(0, Nq, row_block):
                r1 = min(Nq, r0 + row_block)
                S = scale * (q[b, h, r0:r1] @ K.T)
                if causal:
                    S[cols[None, :] > rows[r0:r1, None]] = -np.inf
                if window is not None:
                    S[cols[None, :] < rows[r0:r1, None] - window] = -np.inf
                P, _, _ = _softmax_rows(S)
                dO = do[b, h, r0:r1]
                dv[b, h // G] += P.T @ dO
                dP = dO @ V.T
                dS = P * (dP - D[b, h, r0:r1, None])
                dq[b, h, r0:r1] = scale * (dS @ K)
                dk[b, h // G] += scale * (dS.T @ q[b, h, r0:r1])
    return dq, dk, dv, D


def varlen_ref(q, k, v, cu_seqlens, scale: float, causal: bool = False, window=None, rows=None, values=None):
    """Attention over packed sequences.

    q: [total, Hq, d]; k, v: [total, Hkv, d] (token-major, all sequences
    concatenated); cu_seqlens: [batch + 1] offsets, sequence b owning tokens
    cu_seqlens[b] .. cu_seqlens[b+1]-1 of q, k and v alike, with positions
    counted from its own start. ``rows`` optionally restricts the work to a
    list of packed token indices (others stay O = 0, LSE = -inf). ``values``
    maps stored entries to numbers (for bfloat16 bit patterns), applied to the
    slices a sequence uses.
    Returns O [total, Hq, dv] and LSE [Hq, total] in fp64.
    """
    conv = values if values is not None else (lambda x: x)
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    total, Hq, d = q.shape
    cu = [int(x) for x in cu_seqlens]
    O = np.zeros((total, Hq, v.shape[2]))
    L = np.full((Hq, total), -np.inf)
    want = None if rows is None else set(int(r) for r in rows)
    for b in range(len(cu) - 1):
        s0, s1 = cu[b], cu[b + 1]
        if s1 <= s0:
            continue
        local = np.arange(s1 - s0) if want is None else np.array([r - s0 for r in range(s0, s1) if r in want])
        if local.size == 0:
            continue
        qb = _as64(conv(q[s0 + local])).transpose(1, 0, 2)[None]   # [1, Hq, n_rows, d]
        kb = _as64(conv(k[s0:s1])).transpose(1, 0, 2)[None]
        vb = _as64(conv(v[s0:s1])).transpose(1, 0, 2)[None]
        ob, lb = attention_ref(qb, kb, vb, scale, causal=causal, q_positions=local, window=window)
        O[s0 + local] = ob[0].transpose(1, 0, 2)
        L[:, s0 + local] = lb[0]
    return O, L


def stream_attention(q, k, v, scale: float, causal: bool, Br: int, Bc: int,
                     apply_mask: bool = True, trace=None):
    """FlashAttention-2 forward recurrence in fp64 with tile sizes Br x Bc.

    For each query tile i (rows i*Br ...), state m = -inf, l = 0, a = 0; for
    each key/value tile j allowed by the skip bound (all tiles unmasked; under
    the causal mask only tiles that hold some column <= the tile's last row):
        S   = scale * Q_i K_j^T, then -inf where column > row (diagonal mask)
        m'  = max(m, rowmax S);  alpha = exp(m - m');  Pt = exp(S - m')
        l   = alpha * l + rowsum Pt;  a = alpha * a + Pt V_j;  m = m'
    and finally O_i = a / l, LSE_i = m + ln l.  ``apply_mask=False`` keeps the
    skip bound but drops the diagonal mask (the mistake the pages warn of).
    ``trace(b, h, i, j, m, l, a, alpha)`` sees the state after every tile.
    """
    q, k, v = _as64(q), _as64(k), _as64(v)
    B, Hq, Nq, d = q.shape
    _, Hkv, Nk, _ = k.shape
    G = Hq // Hkv
    if causal:
        assert Nq == Nk, "causal streaming reference is defined for Nq == Nk"
    O = np.zeros((B, Hq, Nq, v.shape[3]))
    LSE = np.full((B, Hq, Nq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            K, V = k[b, h // G], v[b, h // G]
            for i in range(-(-Nq // Br)):
                r0, r1 = i * Br, min(Nq, (i + 1) * Br)
                rows = np.arange(r0, r1)
                Qi = q[b, h, r0:r1]
                m = np.full(r1 - r0, -np.inf)
                l = np.zeros(r1 - r0)
                a = np.zeros((r1 - r0, v.shape[3]))
                last_col = min(Nk, r1) if causal else Nk     # skip bound
                for j in range(-(-last_col // Bc)):
                    c0, c1 = j * Bc, min(Nk, (j + 1) * Bc)
                    S = scale * (Qi @ K[c0:c1].T)
                    if causal and apply_mask:
                        S[np.arange(c0, c1)[None, :] > rows[:, None]] = -np.inf
                    m_new = np.maximum(m, S.max(axis=1))
                    # rows that have seen no visible key keep a neutral base
                    base = np.where(np.isfinite(m_new), m_new, 0.0)
                    alpha = np.where(np.isfinite(m), np.exp(m - base), 0.0)
                    Pt = np.exp(S - base[:, None])
                    l = alpha * l + Pt.sum(axis=1)
                    a = alpha[:, None] * a + Pt @ V[c0:c1]
                    m = m_new
                    if trace is not None:
                        trace(b, h, i, j, m.copy(), l.copy(), a.copy(), alpha.copy())
                live = l > 0
                O[b, h, r0:r1][live] = a[live] / l[live, None]
                LSE[b, h, r0:r1][live] = m[live] + np.log(l[live])
    return O, LSE


def block_summary(x):
    """(max, sum of exp(x - max)) of one block of scores."""
    x = _as64(x)
    m = x.max()
    return m, float(np.exp(x - m).sum())


def merge_summaries(m1, l1, m2, l2):
    """Merge two block summaries: the larger max, each sum shrunk onto it."""
    m = max(m1, m2)
    return m, math.exp(m1 - m) * l1 + math.exp(m2 - m) * l2


def merge_lse(partials):
    """Combine split partials [(o_s, lse_s), ...] of the same query rows.

    o_s is each split's normalised output [rows, dv], lse_s its log-sum-exp
    [rows]. Result: LSE = log(sum_s exp(lse_s)), O = sum_s exp(lse_s - LSE) o_s.
    Splits with lse_s = -inf (no visible key) contribute nothing.
    """
    lses = np.stack([_as64(s) for _, s in partials])          # [S, rows]
    outs = np.stack([_as64(o) for o, _ in partials])          # [S, rows, dv]
    top = lses.max(axis=0)
    live = np.isfinite(top)
    base = np.where(live, top, 0.0)
    w = np.exp(lses - base[None, :])                          # [S, rows]
    tot = w.sum(axis=0)
    lse = np.full(top.shape, -np.inf)
    lse[live] = base[live] + np.log(tot[live])
    o = np.zeros(outs.shape[1:])
    o[live] = (w[:, live, None] * outs[:, live]).sum(axis=0) / tot[live, None]
    return o, lse


def decode_ref(q, k_cache, v_cache, seqlens, scale: float, batches=None):
    """Single-token decode: q [B, Hq, d]; caches [B, Hkv, Lmax, d]; seqlens [B].

    Each sequence b attends over its first seqlens[b] cached keys only; rows at
    or beyond that length are never read. ``batches`` restricts the work to a
    subset of sequences (others are left as O = 0, LSE = -inf).
    Returns O [B, Hq, dv] and LSE [B, Hq] in fp64.
    """
    B, Hq, d = np.shape(q)
    O = np.zeros((B, Hq, np.shape(v_cache)[3]))
    L = np.full((B, Hq), -np.inf)
    for b in (range(B) if batches is None else batches):
        n = int(seqlens[b])
        ob, lb = attention_ref(_as64(q[b])[None, :, None, :],
                               _as64(k_cache[b, :, :n])[None],
                               _as64(v_cache[b, :, :n])[None], scale)
        O[b] = ob[0, :, 0]
        L[b] = lb[0, :, 0]
    return O, L


def split_decode_ref(q, k_cache, v_cache, seqlens, scale: float, split: int, batches=None):
    """Decode computed per key chunk of ``split`` tokens, then merged by LSE.

    Each chunk's (O_s, LSE_s) is plain attention over that chunk; ``merge_lse``
    combines them. Equal to ``decode_ref`` up to rounding, by associativity of
    the merge.
    """
    B, Hq, d = np.shape(q)
    O = np.zeros((B, Hq, np.shape(v_cache)[3]))
    L = np.full((B, Hq), -np.inf)
    for b in (range(B) if batches is None else batches):
        n = int(seqlens[b])
        parts = []
        for c0 in range(0, n, split):
            c1 = min(n, c0 + split)
            ob, lb = attention_ref(_as64(q[b])[None, :, None, :],
                                   _as64(k_cache[b, :, c0:c1])[None],
                                   _as64(v_cache[b, :, c0:c1])[None], scale)
            parts.append((ob[0, :, 0], lb[0, :, 0]))
        O[b], L[b] = merge_lse(parts)
    return O, L


def paged_rows(pool, block_table, b: int, n: int):
    """Rows 0..n-1 of every kv head of sequence b, read through the block table.

    pool is indexed [page, kv head, slot, d] (any strides); returns [Hkv, n, d].
    Only table entries of blocks that hold one of the n tokens are read.
    """
    pool = np.asarray(pool)
    ps = pool.shape[2]
    t = np.arange(n)
    pages = np.asarray(block_table)[b, t // ps]               # [n]
    return pool[pages, :, t % ps].transpose(1, 0, 2)         # [n, H, d] -> [H, n, d]


def paged_decode_ref(q, k_pool, v_pool, block_table, seqlens, scale: float, batches=None, values=None):
    """decode_ref over a paged cache: q [B, Hq, d]; pools [page, Hkv, slot, d];
    block_table [B, max_blocks]; seqlens [B]. Returns O [B, Hq, dv], LSE [B, Hq].

    ``values`` maps gathered pool entries to numbers (for pools stored as
    bfloat16 bit patterns), so that only the rows a sequence uses are widened.
    """
    B, Hq, d = np.shape(q)
    O = np.zeros((B, Hq, np.shape(v_pool)[3]))
    L = np.full((B, Hq), -np.inf)
    conv = values if values is not None else (lambda x: x)
    for b in (range(B) if batches is None else batches):
        n = int(seqlens[b])
        kb = _as64(conv(paged_rows(k_pool, block_table, b, n)))
        vb = _as64(conv(paged_rows(v_pool, block_table, b, n)))
        ob, lb = attention_ref(_as64(q[b])[None, :, None, :], kb[None], vb[None], scale)
        O[b] = ob[0, :, 0]
        L[b] = lb[0, :, 0]
    return O, L
