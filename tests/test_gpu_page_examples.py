"""The pages' worked numeric examples run through the GPU kernels.

T1 ("FlashAttention and Why Attention Is a Memory-Traffic Problem", section
"Tiling and online softmax: exact attention without ever holding all the
scores"; "FlashAttention Explained: IO-Aware Attention, Tiling, Online Softmax
and FP8 on Hopper", section "Worked numeric example"): one query, scores
2, 1, 3, 0, values 1, 2, 3, 4, two tiles of two keys; output 2.4712.

T3 ("FlashAttention and GPU Data Movement", section 3.2 "A two-tile trace,
worked"): one query, scores 8, 6, 10, 7, two-dimensional values (1,2), (3,4),
(5,6), (7,8); output (4.6025, 5.6025).

Both are scalar examples; they are embedded at head_dim 64 with scale 1 by
q = e0, key j = s_j e0 and value j = (v_j, 0, ..., 0), so q . k_j = s_j
exactly (every number is exact in bf16). The pages' two tiles are kept as two
of the kernel's 64-key tiles: the example's first two keys sit at positions 0
and 1, its last two at 64 and 65, so the second tile raises the running
maximum exactly as in the pages' trace. Every other key scores -100 (key
-100 e0) against a zero value, so its weight (below e^-100 of the largest)
rounds away in float32 and the exact answer is the pages' to far below the
printed digits.

Gate: the parity bar against the printed values (O within 1e-2, LSE within
1e-3 of the log of the printed sum), plus exact zeros in the value
components the example does not use. The kernels round the weights to bf16
for the P V product, so the printed 4-5 digits are not reached exactly.
"""
import math

import numpy as np
import pytest
import torch

from tests.conftest import golden
from tests.parity import LSE_MAX, O_MAX, say

pytestmark = pytest.mark.gpu

D, NK = 64, 128
POS = [0, 1, 64, 65]          # the example's keys: two in key tile 0, two in key tile 1


def fa():
    import io_aware_flashattention_amd as m
    return m


def _embed(scores, values):
    """q [1,1,1,D], k/v [1,1,NK,D] bf16 on the GPU for one query row."""
    vals = np.asarray(values, dtype=np.float32)
    if vals.ndim == 1:
        vals = vals[:, None]
    q = torch.zeros(1, 1, 1, D)
    q[0, 0, 0, 0] = 1.0
    k = torch.zeros(1, 1, NK, D)
    k[0, 0, :, 0] = -100.0
    v = torch.zeros(1, 1, NK, D)
    for j, p in enumerate(POS):
        k[0, 0, p, 0] = float(scores[j])
        v[0, 0, p, :vals.shape[1]] = torch.from_numpy(vals[j])
    to = lambda t: t.to(torch.bfloat16).cuda()
    return to(q), to(k), to(v), vals.shape[1]


def _check_row(o_row, lse, want_o, want_lse, used, what):
    o_row = np.asarray(o_row, dtype=np.float64)
    err = np.abs(o_row[:used] - np.asarray(want_o, dtype=np.float64))
    lerr = abs(float(lse) - want_lse)
    say(f"  {what}: O {o_row[:used]} (printed {want_o}), max err {err.max():.2e}; "
        f"LSE {float(lse):.6f} (from the printed sum {want_lse:.5f}), err {lerr:.2e}")
    assert err.max() <= O_MAX, what
    assert np.all(o_row[used:] == 0.0), what
    assert lerr <= LSE_MAX, what


@pytest.mark.parametrize("example", ["t1", "t3"])
def test_page_example_through_fa_fwd(example):
    if example == "t1":
        g = golden("t1_four_scores.json")
        want_o, want_lse = [g["final"]["output"]["value"]], g["lse_derived"]["value"]
    else:
        g = golden("t3_two_tile_trace.json")
        want_o, want_lse = g["output"]["value"], g["lse_derived"]["value"]
    q, k, v, used = _embed(g["scores"], g["values"])
    say(f"case page example {example} through fa_fwd (d={D}, keys at {POS} of {NK})")
    for out_dtype in (torch.float32, torch.bfloat16):
        o, lse = fa().fwd(q, k, v, causal=False, scale=1.0, out_dtype=out_dtype)
        torch.cuda.synchronize()
        _check_row(o[0, 0, 0].float().cpu().numpy(), lse[0, 0, 0].item(), want_o, want_lse, used,
                   f"{example} fa_fwd out={out_dtype}")


@pytest.mark.parametrize("example", ["t1", "t3"])
def test_page_example_through_fa_decode(example):
    """The same row as a single-token decode over a 128-token cache, split
    into ranges of 64 keys (each of the example's tiles in its own split, so
    the log-sum-exp merge joins them)."""
    if example == "t1":
        g = golden("t1_four_scores.json")
        want_o, want_lse = [g["final"]["output"]["value"]], g["lse_derived"]["value"]
    else:
        g = golden("t3_two_tile_trace.json")
        want_o, want_lse = g["output"]["value"], g["lse_derived"]["value"]
    q, k, v, used = _embed(g["scores"], g["values"])
    lens = torch.tensor([NK], dtype=torch.int32, device="cuda")
    for split in (0, 64):
        say(f"case page example {example} through fa_decode split={split}")
        o, lse = fa().decode(q[:, :, 0].contiguous(), k, v, lens, scale=1.0, split_tokens=split,
                             out_dtype=torch.float32)
        torch.cuda.synchronize()
        _check_row(o[0, 0].cpu().numpy(), lse[0, 0].item(), want_o, want_lse, used,
                   f"{example} fa_decode split={split}")


def test_exp_sum_of_t1_from_the_gpu_lse():
    """T1 also prints the plain exponential sum 31.193 (no maximum
    subtracted); exp of the GPU's LSE must give it to the parity bar's
    relative accuracy."""
    g = golden("t1_four_scores.json")
    q, k, v, _ = _embed(g["scores"], g["values"])
    _, lse = fa().fwd(q, k, v, causal=False, scale=1.0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    s = math.exp(lse[0, 0, 0].item())
    say(f"  t1 exp sum from the GPU LSE: {s:.4f} (printed {g['exp_sum_no_shift']['value']})")
    assert abs(s / g["exp_sum_no_shift"]["value"] - 1.0) <= LSE_MAX
