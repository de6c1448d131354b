"""Pins for the FP8 oracle (oracle/fp8.py) against the e4m3 format's bit-level
definition, SciPy's Hadamard matrix, orthogonality, closed forms and the
pages' claim that incoherent processing shrinks quantisation error on inputs
with outlier channels. CPU only."""
import math

import numpy as np
import pytest
import scipy.linalg

from oracle import attention_ref, e4m3_round, fp8_attention_ref, hadamard, quantize, rotate_f32


def decode_e4m3(code: int) -> float:
    """Value of an OCP e4m3 byte from its bit fields (sign, 4-bit exponent with
    bias 7, 3-bit mantissa; exponent 0 is subnormal; S.1111.111 is NaN)."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


FINITE = sorted({decode_e4m3(c): c for c in range(256) if not math.isnan(decode_e4m3(c)) and c < 128}.items())


def test_e4m3_every_code_is_fixed_and_range():
    vals = [v for v, _ in FINITE]
    assert len(vals) == 127 and vals[0] == 0.0 and vals[-1] == 448.0 and vals[1] == 2.0 ** -9
    for v in vals:
        assert e4m3_round(v) == v and e4m3_round(-v) == -v


def test_e4m3_ties_go_to_even_codes_and_nearest_otherwise():
    for (a, ca), (b, cb) in zip(FINITE[:-1], FINITE[1:]):
        mid = (a + b) / 2
        want = a if ca % 2 == 0 else b
        assert e4m3_round(mid) == want, (a, b)
    rng = np.random.default_rng(5)
    vals = np.array([v for v, _ in FINITE])
    for x in rng.uniform(-450, 450, 2000):
        r = e4m3_round(x)
        best = np.abs(vals - abs(x)).min()
        assert abs(abs(r) - abs(x)) == best
    assert e4m3_round(1000.0) == 448.0 and e4m3_round(-1e9) == -448.0 and e4m3_round(464.0) == 448.0


def test_hadamard_matches_scipy_and_is_orthogonal():
    for d in (1, 2, 8, 64, 128):
        h = hadamard(d)
        assert np.array_equal(h, scipy.linalg.hadamard(d))
        assert np.array_equal(h @ h.T, d * np.eye(d))


def test_rotation_is_the_orthogonal_product_and_keeps_scores():
    rng = np.random.default_rng(6)
    d = 128
    s = rng.choice([-1.0, 1.0], d)
    x = rng.standard_normal((5, d)).astype(np.float32)
    y = rng.standard_normal((7, d)).astype(np.float32)
    m = np.diag(s) @ hadamard(d) / math.sqrt(d)
    assert np.allclose(m @ m.T, np.eye(d), atol=1e-12)
    xr, yr = rotate_f32(x, s), rotate_f32(y, s)
    assert np.abs(xr - x.astype(np.float64) @ m).max() < 1e-5
    assert np.abs(xr.astype(np.float64) @ yr.T - x.astype(np.float64) @ y.T).max() < 1e-4


def test_block_quantisation_codes_and_scales():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 2, 300, 128)).astype(np.float32)
    k = rng.standard_normal((1, 1, 300, 128)).astype(np.float32)
    k[0, 0, 70:140] = 0.0                                   # an all-zero key block gets scale 1
    quant = quantize(q, k, k, np.ones(128))
    assert quant["sq"].shape == (1, 2, 3) and quant["sk"].shape == (1, 1, 5) and quant["sv"].shape == (1, 1, 1)
    for key in ("q8", "k8", "v8"):
        c = quant[key]
        assert np.array_equal(e4m3_round(c), c) and np.abs(c).max() == 448.0
    assert quant["sk"][0, 0, 1] == pytest.approx(np.abs(rotate_f32(k, np.ones(128))[0, 0, 64:128]).max() / 448)
    assert quant["sk"][0, 0, 2] == np.float32(1.0) or np.all(quant["k8"][0, 0, 128:140] == 0)
    # dequantised values are within half a code step of the rotated inputs
    xr = rotate_f32(q, np.ones(128)).astype(np.float64)
    deq = quant["q8"] * np.repeat(quant["sq"], 128, axis=-1)[..., :300, None]
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(quant["q8"]), 2.0 ** -6))) - 3)
    assert np.all(np.abs(deq - xr) <= 0.5 * step * np.repeat(quant["sq"], 128, axis=-1)[..., :300, None] * 1.0001)


def test_fp8_attention_closed_form_zero_query():
    """q = 0: every visible score is 0, every weight is 1 (exact in e4m3), so O is
    the mean of the dequantised V rows and LSE the log of the count."""
    rng = np.random.default_rng(8)
    N, d = 70, 128
    q = np.zeros((1, 1, N, d))
    k = rng.standard_normal((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    quant = quantize(q, k, v, rng.choice([-1.0, 1.0], d))
    O, L = fp8_attention_ref(quant, 0.1, causal=True)
    vd = quant["v8"][0, 0] * float(quant["sv"][0, 0, 0])
    for r in (0, 1, 33, 69):
        assert np.abs(O[0, 0, r] - vd[:r + 1].mean(axis=0)).max() < 1e-12
        assert abs(L[0, 0, r] - math.log(r + 1)) < 1e-12


def test_fp8_attention_is_close_to_exact_and_rows_subset():
    rng = np.random.default_rng(9)
    B, Hq, Hkv, N, d = 1, 4, 2, 200, 128
    q, k, v = (rng.standard_normal(s) for s in ((B, Hq, N, d), (B, Hkv, N, d), (B, Hkv, N, d)))
    quant = quantize(q, k, v, rng.choice([-1.0, 1.0], d))
    O, L = fp8_attention_ref(quant, 1 / math.sqrt(d), causal=True)
    Oe, Le = attention_ref(q, k, v, 1 / math.sqrt(d), causal=True)
    # e4m3 keeps three mantissa bits: about 1% mean error on O, a few hundredths on LSE
    assert np.abs(O - Oe).mean() < 0.02 and np.abs(L - Le).max() < 0.1
    rows = [0, 57, 199]
    Os, Ls = fp8_attention_ref(quant, 1 / math.sqrt(d), causal=True, rows=rows)
    assert np.abs(Os[:, :, rows] - O[:, :, rows]).max() < 1e-12 and np.abs(Ls[:, :, rows] - L[:, :, rows]).max() < 1e-12


def test_rotation_spreads_an_outlier_channel_over_every_channel():
    """The rotation moves a single hot channel's energy evenly into all d
    channels (every entry of a rotated one-hot row is +-1/sqrt(d)), which is what
    lets one block scale serve rows with outlier channels."""
    d = 128
    rng = np.random.default_rng(10)
    s = rng.choice([-1.0, 1.0], d)
    for i in (0, 5, 127):
        e = np.zeros((1, d), dtype=np.float32)
        e[0, i] = 50.0
        r = rotate_f32(e, s)
        assert np.allclose(np.abs(r), 50.0 / math.sqrt(d), rtol=1e-6)
        assert abs(float((r.astype(np.float64) ** 2).sum()) - 2500.0) < 1e-3
