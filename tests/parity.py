"""Shared helpers of the GPU parity tests: device upload of generated bits and
the comparison bar (O: max-abs <= 1e-2 and mean-abs <= 1e-3; LSE: max-abs
<= 1e-3, all against the fp64 oracle)."""
import sys

import numpy as np
import torch

O_MAX, O_MEAN, LSE_MAX = 1e-2, 1e-3, 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray) -> torch.Tensor:
    """Upload generated inputs: uint16 bf16 bits -> bfloat16, float32 -> float32."""
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to("cuda")


def check(o_gpu, lse_gpu, o_ref, lse_ref, what: str, o_max=O_MAX, o_mean=O_MEAN, lse_max=LSE_MAX):
    o = o_gpu.detach().float().cpu().numpy().astype(np.float64) if isinstance(o_gpu, torch.Tensor) else o_gpu
    ln = lse_gpu.detach().cpu().numpy().astype(np.float64) if isinstance(lse_gpu, torch.Tensor) else lse_gpu
    assert o.shape == o_ref.shape, (o.shape, o_ref.shape)
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    err = np.abs(o - o_ref)
    lerr = np.abs(ln - lse_ref)
    stats = dict(o_max=float(err.max()), o_mean=float(err.mean()), lse_max=float(lerr.max()))
    say(f"  {what}: O max {stats['o_max']:.3e} mean {stats['o_mean']:.3e}  LSE max {stats['lse_max']:.3e}")
    assert stats["o_max"] <= o_max and stats["o_mean"] <= o_mean, f"{what}: O {stats}"
    assert stats["lse_max"] <= lse_max, f"{what}: LSE {stats}"
    return stats
