"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and lays them out. It holds none of the
attention arithmetic, and it is the one thing the CPU oracle and the GPU path
share: both receive exactly the bit patterns produced here.

Recipe (the pages give shapes and "drawn from N(0,1)" but no generator):

* every (tensor, batch, head) slice has its own NumPy PCG64 stream keyed
  ``[seed, tag, b, h]`` (tag: Q=1, K=2, V=3, heavy-row choice=4, lengths=5),
  so slices are independent of draw order, can be generated in parallel, and
  any single slice can be regenerated alone for a sampled oracle check;
* values are float32 standard normals rounded to bfloat16 with
  round-to-nearest-even (the fp32 workload keeps the float32 values);
* the long-context GQA workload multiplies round(1% * N) distinct K rows of
  every (b, kv-head) by 8 (exact in bfloat16) to stress the running-max
  rescale;
* the decode workload draws each sequence's KV length uniformly from
  [1024, 32768] inclusive; cache rows past a sequence's length are filled
  with a pad value (NaN in tests, so over-reads poison the result; zero in
  the benchmark);
* packed (varlen) prefill inputs draw each sequence's length uniformly from
  the config's [min, max] (stream ``[seed, tag=5]``) and store every
  sequence's heads token-major at its cumulative offset;
* the paged form of a decode workload holds the same token values in a pool
  of fixed-size pages: every sequence gets ceil(L_b / page_size) pages, the
  pages of all sequences are a random permutation of the pool (stream
  ``[seed, tag=6]``), one extra pool page is filled with the pad value and
  every unused block-table entry names it, and slots past L_b in a
  sequence's last page hold the pad value too.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

TAG_Q, TAG_K, TAG_V, TAG_HEAVY, TAG_LENS, TAG_PAGES = 1, 2, 3, 4, 5, 6
BF16_NAN = np.uint16(0x7FC0)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    t = u >> 16
    t &= 1
    t += 0x7FFF
    t += u
    t >>= 16
    out = t.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(seed: int, tag: int, b: int, h: int, shape) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64([seed, tag, b, h]))
    return f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))


def _normal_f32(seed: int, tag: int, b: int, h: int, shape) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64([seed, tag, b, h]))
    return rng.standard_normal(shape, dtype=np.float32)


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen: int
    head_dim: int
    causal: bool
    dtype: str  # "bf16" or "fp32" (input values)
    seed: int
    heavy_frac: float = 0.0  # fraction of K rows scaled by 8 per (b, kv-head)

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    min_len: int
    max_len: int
    head_dim: int
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def group(self) -> int:
        return self.heads_q // self.heads_kv


# The five workloads: one fp32 single head, GPT-2-small-shaped causal prefill,
# a mid-length prefill run causal and unmasked, long-context GQA causal
# prefill at two lengths, and split-KV decode over a GQA cache.
CONFIGS = {
    "c1_single_head_fp32": PrefillConfig("c1_single_head_fp32", 1, 1, 1, 256, 64, False, "fp32", 20260001),
    "c2_gpt2_causal": PrefillConfig("c2_gpt2_causal", 8, 12, 12, 1024, 64, True, "bf16", 20260002),
    "c3_mid_causal": PrefillConfig("c3_mid_causal", 4, 32, 32, 4096, 128, True, "bf16", 20260003),
    "c3_mid_none": PrefillConfig("c3_mid_none", 4, 32, 32, 4096, 128, False, "bf16", 20260003),
    "c4a_gqa_8k": PrefillConfig("c4a_gqa_8k", 1, 64, 8, 8192, 128, True, "bf16", 20260004, 0.01),
    "c4b_gqa_16k": PrefillConfig("c4b_gqa_16k", 1, 64, 8, 16384, 128, True, "bf16", 20260004, 0.01),
}
DECODE_CONFIGS = {
    "c5_decode": DecodeConfig("c5_decode", 64, 64, 8, 1024, 32768, 128, 20260005),
}


# ---------------------------------------------------------------- prefill ---

def heavy_rows(cfg: PrefillConfig, b: int, kvh: int) -> np.ndarray:
    """Sorted K row indices of (b, kvh) that are scaled by 8."""
    n = int(round(cfg.heavy_frac * cfg.seqlen))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64([cfg.seed, TAG_HEAVY, b, kvh]))
    return np.sort(rng.choice(cfg.seqlen, size=n, replace=False))


def prefill_slice(cfg: PrefillConfig, which: str, b: int, h: int) -> np.ndarray:
    """One head of Q, K or V: [N, d] uint16 bf16 bits, or float32 for fp32 configs."""
    tag = {"q": TAG_Q, "k": TAG_K, "v": TAG_V}[which]
    shape = (cfg.seqlen, cfg.head_dim)
    if cfg.dtype == "fp32":
        x = _normal_f32(cfg.seed, tag, b, h, shape)
        if which == "k" and cfg.heavy_frac:
            x[heavy_rows(cfg, b, h)] *= np.float32(8.0)
        return x
    x = _normal_bf16(cfg.seed, tag, b, h, shape)
    if which == "k" and cfg.heavy_frac:
        rows = heavy_rows(cfg, b, h)
        # scaling by 8 is exact in bfloat16: add 3 to the exponent field
        # (N(0,1) draws never come near overflow or the subnormal range)
        f = bf16_bits_to_f32(x[rows]) * np.float32(8.0)
        x[rows] = f32_to_bf16_bits(f)
    return x


def make_prefill_inputs(cfg: PrefillConfig):
    """Full Q [B,Hq,N,d], K and V [B,Hkv,N,d] (uint16 bf16 bits or float32)."""
    dt = np.float32 if cfg.dtype == "fp32" else np.uint16
    q = np.empty((cfg.batch, cfg.heads_q, cfg.seqlen, cfg.head_dim), dtype=dt)
    k = np.empty((cfg.batch, cfg.heads_kv, cfg.seqlen, cfg.head_dim), dtype=dt)
    v = np.empty_like(k)
    jobs = [("q", b, h) for b in range(cfg.batch) for h in range(cfg.heads_q)]
    jobs += [(w, b, h) for w in ("k", "v") for b in range(cfg.batch) for h in range(cfg.heads_kv)]
    dst = {"q": q, "k": k, "v": v}

    def run(job):
        w, b, h = job
        dst[w][b, h] = prefill_slice(cfg, w, b, h)

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(run, jobs))
    return q, k, v


# ----------------------------------------------------------------- decode ---

def decode_lengths(cfg: DecodeConfig) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64([cfg.seed, TAG_LENS]))
    return rng.integers(cfg.min_len, cfg.max_len, size=cfg.batch, endpoint=True).astype(np.int32)


def decode_query(cfg: DecodeConfig, b: int) -> np.ndarray:
    """Query token of sequence b: [Hq, d] bf16 bits."""
    return _normal_bf16(cfg.seed, TAG_Q, b, 0, (cfg.heads_q, cfg.head_dim))


def decode_kv_slice(cfg: DecodeConfig, which: str, b: int, kvh: int, length: int) -> np.ndarray:
    """Valid cache rows [length, d] of K or V for (b, kvh): bf16 bits."""
    tag = {"k": TAG_K, "v": TAG_V}[which]
    return _normal_bf16(cfg.seed, tag, b, kvh, (length, cfg.head_dim))


def make_decode_inputs(cfg: DecodeConfig, pad: str = "nan", lengths=None):
    """q [B,Hq,d], k_cache/v_cache [B,Hkv,max_len,d] bf16 bits, lengths [B] int32.

    ``pad`` fills cache rows at or past each sequence's length: "nan" or "zero".
    """
    lens = decode_lengths(cfg) if lengths is None else np.asarray(lengths, dtype=np.int32)
    q = np.stack([decode_query(cfg, b) for b in range(cfg.batch)])
    padv = BF16_NAN if pad == "nan" else np.uint16(0)
    kc = np.empty((cfg.batch, cfg.heads_kv, cfg.max_len, cfg.head_dim), dtype=np.uint16)
    vc = np.empty_like(kc)

    def run(job):
        w, b, h = job
        dst = kc if w == "k" else vc
        L = int(lens[b])
        dst[b, h, :L] = decode_kv_slice(cfg, w, b, h, L)
        dst[b, h, L:] = padv

    jobs = [(w, b, h) for w in ("k", "v") for b in range(cfg.batch) for h in range(cfg.heads_kv)]
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(run, jobs))
    return q, kc, vc, lens


def make_paged_decode_inputs(cfg: DecodeConfig, page_size: int, layout: str = "head", pad: str = "nan",
                             lengths=None):
    """Paged cache holding the same values as ``make_decode_inputs``.

    Returns q [B,Hq,d], k_pool/v_pool, block_table [B, ceil(max_len/page_size)]
    int32, lengths [B] int32. layout "head": pools are [P, Hkv, page_size, d];
    layout "token": [P, page_size, Hkv, d] (vLLM-style). Token t of (b, kv head)
    is stored in page block_table[b, t // page_size], slot t % page_size.
    """
    if layout not in ("head", "token"):
        raise ValueError(layout)
    lens = decode_lengths(cfg) if lengths is None else np.asarray(lengths, dtype=np.int32)
    B, Hkv, d, ps = cfg.batch, cfg.heads_kv, cfg.head_dim, page_size
    q = np.stack([decode_query(cfg, b) for b in range(B)])
    nblk = [-(-int(L) // ps) for L in lens]
    max_blocks = -(-cfg.max_len // ps)
    n_pages = sum(nblk) + 1
    rng = np.random.Generator(np.random.PCG64([cfg.seed, TAG_PAGES]))
    perm = rng.permutation(n_pages).astype(np.int32)
    poison = int(perm[-1])
    table = np.full((B, max_blocks), poison, dtype=np.int32)
    used = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[used:used + nblk[b]]
        used += nblk[b]
    padv = BF16_NAN if pad == "nan" else np.uint16(0)
    shape = (n_pages, Hkv, ps, d) if layout == "head" else (n_pages, ps, Hkv, d)
    kp = np.full(shape, padv, dtype=np.uint16)
    vp = np.full(shape, padv, dtype=np.uint16)

    def run(job):
        w, b, h = job
        dst = kp if w == "k" else vp
        L, n = int(lens[b]), nblk[b]
        rows = np.full((n * ps, d), padv, dtype=np.uint16)
        rows[:L] = decode_kv_slice(cfg, w, b, h, L)
        if layout == "head":
            dst[table[b, :n], h] = rows.reshape(n, ps, d)
        else:
            dst[table[b, :n], :, h] = rows.reshape(n, ps, d)

    jobs = [(w, b, h) for w in ("k", "v") for b in range(B) for h in range(Hkv)]
    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(run, jobs))
    return q, kp, vp, table, lens


@dataclass(frozen=True)
class VarlenConfig:
    """Packed prefill: sequences concatenated on the token axis (cu_seqlens)."""
    name: str
    n_seqs: int
    heads_q: int
    heads_kv: int
    min_len: int
    max_len: int
    head_dim: int
    causal: bool
    window: int          # sliding window W (row r sees keys r-W..r), -1 for none
    seed: int

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


# Packed-batch and sliding-window prefill on the GQA shape of the decode and
# long-context workloads: a mix of lengths, and the pages' window example
# (8192 tokens, keys at most 1024 positions behind the row).
VARLEN_CONFIGS = {
    "c6_varlen_causal": VarlenConfig("c6_varlen_causal", 16, 64, 8, 1, 8192, 128, True, -1, 20260006),
    "c7_window_8k": VarlenConfig("c7_window_8k", 1, 64, 8, 8192, 8192, 128, True, 1024, 20260007),
}


def varlen_lengths(cfg: VarlenConfig) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64([cfg.seed, TAG_LENS]))
    return rng.integers(cfg.min_len, cfg.max_len, size=cfg.n_seqs, endpoint=True).astype(np.int32)


def make_varlen_inputs(heads_q: int, heads_kv: int, head_dim: int, lengths, seed: int, dtype: str = "bf16"):
    """Packed q [total, Hq, d], k/v [total, Hkv, d] (bf16 bits) and cu_seqlens [n+1] int32.

    Sequence b's head h is the slice keyed [seed, tag, b, h], as for the dense
    workloads, laid out token-major.
    """
    lens = np.asarray(lengths, dtype=np.int64)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    total = int(cu[-1])
    conv = (lambda x: x) if dtype == "fp32" else f32_to_bf16_bits
    dt = np.float32 if dtype == "fp32" else np.uint16
    q = np.empty((total, heads_q, head_dim), dtype=dt)
    k = np.empty((total, heads_kv, head_dim), dtype=dt)
    v = np.empty_like(k)
    jobs = [("q", b, h) for b in range(len(lens)) for h in range(heads_q)]
    jobs += [(w, b, h) for w in ("k", "v") for b in range(len(lens)) for h in range(heads_kv)]
    dst = {"q": q, "k": k, "v": v}
    tags = {"q": TAG_Q, "k": TAG_K, "v": TAG_V}

    def run(job):
        w, b, h = job
        n = int(lens[b])
        dst[w][cu[b]:cu[b] + n, h] = conv(_normal_f32(seed, tags[w], b, h, (n, head_dim)))

    with ThreadPoolExecutor(_workers()) as ex:
        list(ex.map(run, jobs))
    return q, k, v, cu


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact fp64 values of generated inputs (bf16 bits or float32)."""
    if x.dtype == np.uint16:
        return bf16_bits_to_f32(x).astype(np.float64)
    return np.asarray(x, dtype=np.float64)


def make_random_prefill(batch: int, heads_q: int, heads_kv: int, seqlen_q: int, seqlen_k: int,
                        head_dim: int, dtype: str = "bf16", seed: int = 0, heavy_frac: float = 0.0):
    """Q [B,Hq,Nq,d], K/V [B,Hkv,Nk,d] for arbitrary (ragged, small) test shapes.

    Same recipe as the named workloads: per-slice PCG64 streams, N(0,1)
    float32 rounded to bf16 (kept as float32 for dtype="fp32"), and an
    optional fraction of K rows per (b, kv head) multiplied by 8.
    """
    conv = (lambda x: x) if dtype == "fp32" else f32_to_bf16_bits
    q = np.stack([np.stack([conv(_normal_f32(seed, TAG_Q, b, h, (seqlen_q, head_dim))) for h in range(heads_q)])
                  for b in range(batch)])
    ks, vs = [], []
    for b in range(batch):
        kb, vb = [], []
        for h in range(heads_kv):
            kf = _normal_f32(seed, TAG_K, b, h, (seqlen_k, head_dim))
            n = int(round(heavy_frac * seqlen_k))
            if n:
                rng = np.random.Generator(np.random.PCG64([seed, TAG_HEAVY, b, h]))
                kf[rng.choice(seqlen_k, size=n, replace=False)] *= np.float32(8.0)
            kb.append(conv(kf))
            vb.append(conv(_normal_f32(seed, TAG_V, b, h, (seqlen_k, head_dim))))
        ks.append(np.stack(kb))
        vs.append(np.stack(vb))
    return q, np.stack(ks), np.stack(vs)
