"""CPU oracle for FP8 (e4m3) attention with incoherent processing.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py). Shares no code with the
HIP path.

The method ("FlashAttention Explained: IO-Aware Attention, Tiling, Online
Softmax and FP8 on Hopper", section "FP8 Attention and Incoherent
Processing"): Q and K are multiplied by the same random orthogonal matrix
M = diag(s) H / sqrt(d) (H the Sylvester Hadamard matrix, s random signs)
before quantization, which leaves Q K^T unchanged and spreads outlier
channels; the operands are stored as e4m3 with one scale per block of rows;
the softmax statistics stay in float32.

Readings where the pages stop (each listed in the design notes):
* e4m3 is the OCP format (bias 7, largest finite 448, no infinities);
  rounding is to nearest, ties to even, after clamping to +-448.
* Blocks: one scale per 128 query rows of a head, per 64 keys of a kv head,
  and per kv head for V; scale = amax / 448 and codes = e4m3(x * (448 /
  amax)), both in float32 (a quantised code is decided in float32 on both
  sides); an all-zero block has scale 1.
* The rotation runs as the fast Walsh-Hadamard transform in float32
  (butterflies of distance 1, 2, 4, ... within each row, then one multiply
  by the float32 value of 1/sqrt(d)), so the codes it feeds are the ones the
  GPU quantiser produces.
* Both products run in fp8: the probabilities are quantised too, as
  P8 = 2^-8 e4m3(2^8 * 2^(x - B)) with x = S log2(e) and B = ceil(max x) the
  row's base, so a weight keeps its relative precision down to 2^-14 of the
  largest; O = sum P8 V / sum P8 (the weights that enter the product
  normalise it), and LSE is the exact log-sum-exp of the dequantised scores.
"""
from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0


def e4m3_round(x) -> np.ndarray:
    """Nearest e4m3 value (ties to even) after clamping to +-448, in fp64."""
    x = np.clip(np.asarray(x, dtype=np.float64), -E4M3_MAX, E4M3_MAX)
    a = np.abs(x)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)                        # below 2^-6 the spacing is fixed (subnormals)
    step = np.exp2(e - 3.0)                        # three mantissa bits
    r = np.round(a / step) * step                  # numpy rounds halves to even
    return np.copysign(r, x)


def hadamard(d: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order d (a power of two), entries +-1."""
    assert d > 0 and d & (d - 1) == 0
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def rotate_f32(x, signs) -> np.ndarray:
    """x diag(s) H / sqrt(d) along the last axis, as float32 butterflies."""
    y = (np.asarray(x, dtype=np.float32) * np.asarray(signs, dtype=np.float32)).astype(np.float32)
    d = y.shape[-1]
    h = 1
    while h < d:
        y = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(y.shape[:-3] + (d,))
        h *= 2
    return (y * np.float32(1.0 / math.sqrt(d))).astype(np.float32)


def quantize_rows(x, block: int):
    """Block quantisation along the row axis (axis -2) of float32 values.

    Returns (codes as fp64 e4m3 values, scales [.., n_blocks] float32).
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[-2]
    nb = -(-n // block)
    codes = np.empty(x.shape, dtype=np.float64)
    scales = np.empty(x.shape[:-2] + (nb,), dtype=np.float32)
    for i in range(nb):
        blk = x[..., i * block:(i + 1) * block, :]
        amax = np.abs(blk).max(axis=(-2, -1)).astype(np.float32)
        safe = np.where(amax > 0, amax, np.float32(448.0))
        inv = (np.float32(448.0) / safe).astype(np.float32)
        scales[..., i] = (safe / np.float32(448.0)).astype(np.float32)
        codes[..., i * block:(i + 1) * block, :] = e4m3_round((blk * inv[..., None, None]).astype(np.float32))
    return codes, scales


def quantize(q, k, v, signs, q_block: int = 128, k_block: int = 64, rotate: bool = True):
    """The quantiser: rotated Q and K, and V, as e4m3 codes with their scales.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (input values, e.g. bf16 as float).
    ``rotate=False`` skips the incoherent processing (plain block quantisation).
    Returns dict(q8, sq, k8, sk, v8, sv) with sv shaped [B, Hkv, 1].
    """
    rot = (lambda x: rotate_f32(x, signs)) if rotate else (lambda x: np.asarray(x, dtype=np.float32))
    q8, sq = quantize_rows(rot(q), q_block)
    k8, sk = quantize_rows(rot(k), k_block)
    n = np.shape(v)[-2]
    v8, sv = quantize_rows(np.asarray(v, dtype=np.float32), n)
    return dict(q8=q8, sq=sq, k8=k8, sk=sk, v8=v8, sv=sv)


def fp8_attention_ref(quant, scale: float, causal: bool = False, q_block: int = 128, k_block: int = 64,
                      rows=None):
    """Attention on the quantised operands (fp64 arithmetic on the codes).

    Returns O [B, Hq, N, d] and LSE [B, Hq, N]. ``rows`` restricts the work to
    a list of query rows (others stay O = 0, LSE = -inf).
    """
    q8, sq, k8, sk, v8, sv = (quant[n] for n in ("q8", "sq", "k8", "sk", "v8", "sv"))
    B, Hq, N, d = q8.shape
    Hkv = k8.shape[1]
    G = Hq // Hkv
    rsel = np.arange(N) if rows is None else np.asarray(rows)
    qd = q8 * np.repeat(sq.astype(np.float64), q_block, axis=-1)[..., :N, None]
    kd = k8 * np.repeat(sk.astype(np.float64), k_block, axis=-1)[..., :N, None]
    vd = v8 * sv.astype(np.float64)[..., None]
    O = np.zeros((B, Hq, N, d))
    L = np.full((B, Hq, N), -np.inf)
    cols = np.arange(N)
    for b in range(B):
        for h in range(Hq):
            S = scale * (qd[b, h, rsel] @ kd[b, h // G].T)
            if causal:
                S[cols[None, :] > rsel[:, None]] = -np.inf
            x = S * (1.0 / math.log(2.0))
            base = np.ceil(x.max(axis=1))
            w = np.exp2(x - base[:, None])
            p8 = e4m3_round(w * 256.0) / 256.0
            O[b, h, rsel] = (p8 @ vd[b, h // G]) / p8.sum(axis=1)[:, None]
            m = S.max(axis=1)
            L[b, h, rsel] = m + np.log(np.exp(S - m[:, None]).sum(axis=1))
    return O, L
