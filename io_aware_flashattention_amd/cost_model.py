"""FLOP and logical-byte counts for attention, used to turn kernel times into
roofline fractions.

Conventions (all from the pages):

* FLOPs: the two matmuls cost 4 * Nq * Nk * d per head; a causal mask is
  counted as half of that, not N(N+1)/2 ("FlashAttention and Why Attention Is
  a Memory-Traffic Problem", section "The bottleneck is traffic"; "FlashAttention
  Explained: IO-Aware Attention, Tiling, Online Softmax and FP8 on Hopper",
  section "Worked arithmetic: standard attention on one head" and the SDPA
  walk-through's causal FLOP count).
* Logical HBM traffic of the three-kernel materialising baseline and of the
  FlashAttention-2 loop: cold cache, exact bytes, no sector padding, Q read
  once, O written once, each K/V tile read once per query tile that the skip
  bound lets through ("FlashAttention and GPU Data Movement", sections 1.1,
  2.2 and 4).
* Decode reads every cached K and V row once per step: 2 * Hkv * d * elem
  bytes per (sequence, token) ("FlashAttention Explained", section "Worked
  decode example").
"""
from __future__ import annotations

from typing import Iterable


def attention_flops(batch: int, heads_q: int, seqlen_q: int, seqlen_k: int, head_dim: int,
                    causal: bool) -> float:
    """Algorithmic FLOPs of the forward pass (matmuls only)."""
    f = 4.0 * batch * heads_q * seqlen_q * seqlen_k * head_dim
    return f / 2.0 if causal else f


def backward_flops(batch: int, heads_q: int, seqlen_q: int, seqlen_k: int, head_dim: int, causal: bool) -> float:
    """Algorithmic FLOPs of the backward pass: five matmuls (QK^T recomputed, dV,
    dP, dQ, dK) against the forward's two, so 2.5x attention_flops ("FlashAttention
    Explained", section "Backward Pass: Recomputation Beats Storage")."""
    return 2.5 * attention_flops(batch, heads_q, seqlen_q, seqlen_k, head_dim, causal)


def window_flops(heads_q: int, seqlen: int, head_dim: int, window: int) -> float:
    """Algorithmic FLOPs of one sequence under a sliding window W on top of the
    causal mask: 4 * d per visible (row, key) pair, counted exactly (row r sees
    min(r, W) + 1 keys), since the halved-square convention of the plain
    causal mask has no analogue for a band."""
    n, w = int(seqlen), int(window)
    full = max(0, n - w)                       # rows r >= W see W + 1 keys
    ramp = min(n, w)                           # rows r < W see r + 1 keys
    pairs = full * (w + 1) + ramp * (ramp + 1) // 2
    return 4.0 * heads_q * head_dim * pairs


def varlen_flops(lengths: Iterable[int], heads_q: int, head_dim: int, causal: bool) -> float:
    """Sum over packed sequences of attention_flops(1, Hq, L, L, d, causal)."""
    return sum(attention_flops(1, heads_q, int(n), int(n), head_dim, causal) for n in lengths)


def causal_kv_tiles(i: int, Br: int, Bc: int, seqlen: int) -> int:
    """Number of K/V tiles query tile i (0-based) loads under the causal skip bound.

    Tile j holds columns j*Bc .. j*Bc+Bc-1; the query tile's last row is
    min(N, (i+1)*Br) - 1, so tiles 0 .. ceil(min(N, (i+1)*Br) / Bc) - 1 are loaded.
    """
    last = min(seqlen, (i + 1) * Br)
    return -(-last // Bc)


def causal_diagonal_tiles(i: int, Br: int, Bc: int, seqlen: int) -> range:
    """K/V tiles of query tile i (0-based) that straddle the diagonal and need the mask.

    A loaded tile needs masking when its last column lies past the tile's
    first row, i.e. some (row, column) pair in it has column > row.
    """
    first_row = i * Br
    n = causal_kv_tiles(i, Br, Bc, seqlen)
    masked = [j for j in range(n) if min(seqlen, (j + 1) * Bc) - 1 > first_row]
    return range(masked[0], n) if masked else range(n, n)


def naive_traffic(seqlen: int, head_dim: int, elem_bytes: int = 2, causal: bool = False):
    """(reads, writes) in bytes of the three-kernel baseline, one head.

    GEMM1 reads Q, K and writes S; softmax reads S and writes P; GEMM2 reads
    P, V and writes O. The causal variant is the idealised lower-triangular
    kernel that stores exactly half of S and P.
    """
    nd = seqlen * head_dim * elem_bytes
    nn = seqlen * seqlen * elem_bytes
    if causal:
        nn = nn // 2
    return 3 * nd + 2 * nn, 2 * nn + nd


def fa2_traffic(seqlen: int, head_dim: int, Br: int, Bc: int, elem_bytes: int = 2,
                causal: bool = False, lse: bool = False):
    """(reads, writes) in bytes of the FlashAttention-2 loop for one head.

    Q is read once, O written once (plus 4 bytes per row of log-sum-exp when
    ``lse``), and every K/V tile is read once per query tile that loads it.
    """
    row = head_dim * elem_bytes
    n_q_tiles = -(-seqlen // Br)
    n_kv_tiles = -(-seqlen // Bc)
    kv_rows = 0
    for i in range(n_q_tiles):
        n = causal_kv_tiles(i, Br, Bc, seqlen) if causal else n_kv_tiles
        kv_rows += min(seqlen, n * Bc)
    reads = seqlen * row + 2 * kv_rows * row
    writes = seqlen * row + (4 * seqlen if lse else 0)
    return reads, writes


def kv_passes(seqlen: int, Br: int, Bc: int, causal: bool) -> float:
    """Complete passes over K/V made by all query tiles of one head."""
    n_q_tiles = -(-seqlen // Br)
    n_kv_tiles = -(-seqlen // Bc)
    if not causal:
        return float(n_q_tiles)
    return sum(causal_kv_tiles(i, Br, Bc, seqlen) for i in range(n_q_tiles)) / n_kv_tiles


def compulsory_bytes(batch: int, heads_q: int, heads_kv: int, seqlen: int, head_dim: int,
                     in_bytes: int = 2, out_bytes: int = 2, lse: bool = True) -> int:
    """Q, K, V read once and O (plus LSE) written once: the fused kernel's floor."""
    q = batch * heads_q * seqlen * head_dim * in_bytes
    kv = 2 * batch * heads_kv * seqlen * head_dim * in_bytes
    o = batch * heads_q * seqlen * head_dim * out_bytes
    return q + kv + o + (4 * batch * heads_q * seqlen if lse else 0)


def decode_kv_bytes(lengths: Iterable[int], heads_kv: int, head_dim: int, elem_bytes: int = 2) -> int:
    """Cache bytes one decode step must read: K and V of every valid token."""
    return int(sum(int(x) for x in lengths)) * 2 * heads_kv * head_dim * elem_bytes


def decode_flops(lengths: Iterable[int], heads_q: int, head_dim: int) -> float:
    """Matmul FLOPs of one decode step: 4 * Hq * d per cached token."""
    return 4.0 * heads_q * head_dim * float(sum(int(x) for x in lengths))
