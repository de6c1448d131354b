"""The seeded input generator: determinism, slice independence, rounding. CPU only."""
import numpy as np
import torch

from io_aware_flashattention_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10 ** rng.uniform(-30, 30, 100000).astype(np.float32),
                        np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, 1e-40, 1.00390625, 1.01171875], dtype=np.float32)])
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert W.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))[0] == 0x7FC0
    back = W.bf16_bits_to_f32(ours)
    assert np.array_equal(back[np.isfinite(back)], torch.from_numpy(x).to(torch.bfloat16).float().numpy()[np.isfinite(back)])


def test_prefill_deterministic_and_slices_regenerate():
    cfg = W.CONFIGS["c2_gpt2_causal"]
    q1, k1, v1 = W.make_prefill_inputs(cfg)
    q2, k2, v2 = W.make_prefill_inputs(cfg)
    assert np.array_equal(q1, q2) and np.array_equal(k1, k2) and np.array_equal(v1, v2)
    assert np.array_equal(W.prefill_slice(cfg, "q", 3, 7), q1[3, 7])
    assert np.array_equal(W.prefill_slice(cfg, "v", 5, 11), v1[5, 11])
    assert not np.array_equal(q1[0, 0], k1[0, 0])
    x = W.bf16_bits_to_f32(q1)
    assert abs(float(x.mean())) < 0.01 and abs(float(x.std()) - 1.0) < 0.01


def test_fp32_config_keeps_float32_values():
    cfg = W.CONFIGS["c1_single_head_fp32"]
    q, k, v = W.make_prefill_inputs(cfg)
    assert q.dtype == np.float32 and q.shape == (1, 1, 256, 64)
    assert not np.array_equal(W.bf16_bits_to_f32(W.f32_to_bf16_bits(q)), q)


def test_heavy_rows_scaled_by_eight():
    cfg = W.CONFIGS["c4a_gqa_8k"]
    rows = W.heavy_rows(cfg, 0, 3)
    assert len(rows) == 82 and len(set(rows.tolist())) == 82
    k = W.prefill_slice(cfg, "k", 0, 3)
    raw = W._normal_bf16(cfg.seed, W.TAG_K, 0, 3, (cfg.seqlen, cfg.head_dim))
    assert np.array_equal(W.bf16_bits_to_f32(k[rows]), 8 * W.bf16_bits_to_f32(raw[rows]))
    mask = np.ones(cfg.seqlen, bool)
    mask[rows] = False
    assert np.array_equal(k[mask], raw[mask])
    assert len(W.heavy_rows(W.CONFIGS["c4b_gqa_16k"], 0, 0)) == 164


def test_decode_lengths_and_padding():
    cfg = W.DecodeConfig("small", 4, 8, 2, 5, 40, 16, 99)
    q, kc, vc, lens = W.make_decode_inputs(cfg, pad="nan")
    assert q.shape == (4, 8, 16) and kc.shape == (4, 2, 40, 16)
    assert np.all((lens >= 5) & (lens <= 40))
    for b in range(4):
        assert np.all(np.isnan(W.bf16_bits_to_f32(kc[b, :, lens[b]:])))
        assert np.all(np.isfinite(W.bf16_bits_to_f32(vc[b, :, :lens[b]])))
        assert np.array_equal(W.decode_kv_slice(cfg, "k", b, 1, int(lens[b])), kc[b, 1, :lens[b]])
    L = W.decode_lengths(W.DECODE_CONFIGS["c5_decode"])
    assert L.shape == (64,) and L.min() >= 1024 and L.max() <= 32768
