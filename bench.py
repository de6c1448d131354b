#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic inputs:
  1. causal GQA prefill, batch 1, 64 query heads over 8 kv heads, N = 8192,
     d = 128, bf16 (fa_fwd), and
  2. split-KV decode, 64 sequences, 64 query heads over 8 kv heads, d = 128,
     kv lengths uniform in [1024, 32768], bf16 cache (fa_decode: split kernel
     and merge kernel).
After the timed steps, more paths are timed on their own (not part of the
step): the same decode against a paged cache (fa_decode_paged: 16-token
pages in a token-major pool, shuffled block table) as ``decode_paged``, and
through fa_fwd_varlen the 8192-token sliding-window-1024 prefill
(``prefill_window``) and a packed batch of 16 causal sequences of 1..8192
tokens (``prefill_varlen``), and the backward of the step's prefill through
fa_bwd (``backward``, 2.5x the forward FLOPs), and the FP8 prefill of the
step's workload (``prefill_fp8``: fa_fwd_fp8, with fa_fp8_quantize timed
apart). Then every other prefill configuration (``configs``: the fp32 single
head, GPT-2-shaped causal prefill, the mid-length prefill causal and
unmasked, and the 16384-token GQA prefill), each with its own algorithmic
TFLOP/s, fraction of peak, HBM counter bytes when the committed counter
summary matches the kernel sources, and the fp64 oracle timed on a bounded
sample of the same configuration.
Every phase's inputs are generated and uploaded before the first timed
region, so the phases then run back to back: the shader clock drops while the
GPU idles (as it does while the host generates inputs) and needs a few tens of
milliseconds of load to come back up. Each phase runs W untimed warm-up
launches (default 100: about 0.18 s of the step), then exactly K timed ones
between two device synchronisations. Times come from HIP events recorded on
the stream the kernels run on: around each kernel of the step and of the
paged decode, and around the K back-to-back launches of every later phase
(per launch: the span / K).

Prints one JSON line. ``value`` is the prefill throughput in algorithmic
TFLOP/s (4*B*Hq*N^2*d, halved for the causal mask); the decode bandwidth in
algorithmic KV GB/s (every cached K/V byte of every valid token, read once)
is reported alongside. ``roofline`` / ``roofline_decode`` put both against
MI355X peaks; ``cpu_baseline`` times the fp64 oracle on a sample of the same
prefill workload on the host cores. ``clock`` records the shader clock the
chip ran at under the prefill (read from the SMU after the timed regions;
clocks are not pinned) and the prefill's fraction of the matrix peak at that
clock, beside the fraction of the published 2.4 GHz peak that ``roofline``
reports.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline] [--no-clock]
    python bench.py --summarize-trace DIR --out FILE [--steps K --warmup W]   (rocprofv3 kernel trace -> text)
    python bench.py --summarize-pmc FETCH_DIR WRITE_DIR --out FILE [--steps K --warmup W]  (HBM bytes per launch)
  (--steps/--warmup: those of the profiled run, so its dispatches can be split into the bench's phases)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 matrix peak: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_FP8_TFLOPS = 5033.2      # MI355X dense fp8 matrix peak (twice bf16)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E peak
PEAK_CLOCK_MHZ = 2400.0       # the shader clock the published matrix peaks assume
PREFILL_CFG = "c4a_gqa_8k"
DECODE_CFG = "c5_decode"
PAGE_SIZE = 16                # tokens per page of the paged-decode measurement
PMC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_pmc.json")
KERNEL_SOURCES = ["io_aware_flashattention_amd/csrc/" + f for f in
                  ("fa_fwd.hip", "fa_fwd_f32.hip", "fa_decode.hip", "fa_bwd.hip", "fa_fp8.hip", "fa_device.h",
                   "fa_launch.h")]
# prefill configurations timed after the step, in launch order (labels of the profile summaries)
CONFIG_PHASES = ("c1_single_head_fp32", "c2_gpt2_causal", "c3_mid_causal", "c3_mid_none", "c4b_gqa_16k")
# Extra warm-up launches of a configuration phase. The GPT-2-shaped launch
# (~28 us) follows the launch-bound fp32 single head, during which the GPU
# idles most of the time and its clock falls; W of its own launches are only
# a few milliseconds of load, too few to bring the clock back up.
CONFIG_EXTRA_WARMUP = {"c2_gpt2_causal": 1500}
ORACLE_SECONDS = {"c1_single_head_fp32": 1.0, "c2_gpt2_causal": 2.0, "c3_mid_causal": 3.0, "c3_mid_none": 3.0,
                  "c4b_gqa_16k": 6.0, "c5_decode": 2.0}
COPY_BYTES = 1 << 30          # calibration copy: 1 GiB read + 1 GiB written


def sources_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# --------------------------------------------------------------- the bench --

def run(args):
    import numpy as np
    import torch

    import io_aware_flashattention_amd as fa
    from io_aware_flashattention_amd import cost_model as cm
    from io_aware_flashattention_amd import workloads as W

    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    fa.load()

    pc = W.CONFIGS[PREFILL_CFG]
    dc = W.DECODE_CONFIGS[DECODE_CFG]
    t0 = time.time()
    print(f"[bench] generating {pc.name} and {dc.name} inputs", file=sys.stderr, flush=True)
    qh, kh, vh = W.make_prefill_inputs(pc)
    to_dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).view(torch.int16).view(torch.bfloat16).to(dev)
    q, k, v = to_dev(qh), to_dev(kh), to_dev(vh)
    o = torch.empty_like(q)
    lse = torch.empty(pc.batch, pc.heads_q, pc.seqlen, dtype=torch.float32, device=dev)
    dq, dk, dv, lens = W.make_decode_inputs(dc, pad="zero")
    dq_d, dk_d, dv_d = to_dev(dq), to_dev(dk), to_dev(dv)
    del dk, dv
    lens_d = torch.from_numpy(lens).to(dev)
    do = torch.empty(dc.batch, dc.heads_q, dc.head_dim, dtype=torch.bfloat16, device=dev)
    dlse = torch.empty(dc.batch, dc.heads_q, dtype=torch.float32, device=dev)
    ws = torch.empty(fa.decode_workspace_bytes(dc.batch, dc.heads_q, dc.heads_kv, dc.max_len, dc.head_dim, 0),
                     dtype=torch.uint8, device=dev)
    # calibration copy of known size (its FETCH/WRITE counters scale the HBM byte counters)
    csrc = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    cdst = torch.empty_like(csrc)
    cdst.copy_(csrc)
    torch.cuda.synchronize()
    del csrc, cdst
    # the later phases' inputs, generated now so the timed phases run back to back
    print(f"[bench] generating the paged form of {dc.name} (page size {PAGE_SIZE}, token-major)",
          file=sys.stderr, flush=True)
    _, pk, pv, ptab, plens = W.make_paged_decode_inputs(dc, PAGE_SIZE, layout="token", pad="zero")
    assert np.array_equal(plens, lens)
    pk_d, pv_d = to_dev(pk).transpose(1, 2), to_dev(pv).transpose(1, 2)   # indexed [page, kv head, slot, d]
    del pk, pv
    ptab_d = torch.from_numpy(ptab).to(dev)
    varlen_in = {}
    for name in ("c7_window_8k", "c6_varlen_causal"):
        vc = W.VARLEN_CONFIGS[name]
        vl = W.varlen_lengths(vc)
        vq, vk, vv, vcu = W.make_varlen_inputs(vc.heads_q, vc.heads_kv, vc.head_dim, vl, seed=vc.seed)
        varlen_in[name] = (vc, vl, to_dev(vq), to_dev(vk), to_dev(vv), torch.from_numpy(vcu).to(dev))
        del vq, vk, vv
    gh, _, _ = W.make_random_prefill(pc.batch, pc.heads_q, pc.heads_kv, pc.seqlen, pc.seqlen, pc.head_dim,
                                     seed=pc.seed + 100)
    dout = to_dev(gh)                        # dO of the backward
    del gh
    config_in = config_inputs(W, to_dev, dev)
    torch.cuda.synchronize()
    print(f"[bench] inputs ready in {time.time() - t0:.1f}s; warmup {args.warmup}, steps {args.steps}",
          file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fwd(q, k, v, causal=True, scale=pc.scale, out=o, lse=lse)
        if ev is not None:
            ev[1].record(stream)
        fa.decode(dq_d, dk_d, dv_d, lens_d, scale=dc.scale, out=do, lse=dlse, workspace=ws)
        if ev is not None:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    pre_ms = [e[0].elapsed_time(e[1]) for e in events]
    dec_ms = [e[1].elapsed_time(e[2]) for e in events]
    step_ms = [e[0].elapsed_time(e[2]) for e in events]
    print(f"[bench] timed {args.steps} steps in {wall * 1e3:.2f} ms wall", file=sys.stderr, flush=True)

    # paged-KV decode of the same workload, timed on its own after the steps
    def paged():
        fa.decode_paged(dq_d, pk_d, pv_d, ptab_d, lens_d, scale=dc.scale, out=do, lse=dlse, workspace=ws)

    for _ in range(args.warmup):
        paged()
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        pev[i][0].record(stream)
        paged()
        pev[i][1].record(stream)
    torch.cuda.synchronize()
    pag_ms = [e[0].elapsed_time(e[1]) for e in pev]
    del pk_d, pv_d

    def time_launches(fn, extra_warmup=0):
        """ms per launch: K launches back to back between two HIP events, after
        the warm-up (a pair of events around every launch would add the
        events' own cost, ~3 us, to each of the short ones)."""
        for _ in range(args.warmup + extra_warmup):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    # packed prefill: sliding window and mixed lengths, each timed on its own
    extra = {}
    for key, name in (("prefill_window", "c7_window_8k"), ("prefill_varlen", "c6_varlen_causal")):
        vc, vl, vq, vk, vv, vcu = varlen_in.pop(name)
        vo = torch.empty_like(vq)
        vlse = torch.empty(vc.heads_q, int(vl.sum()), dtype=torch.float32, device=dev)
        win = vc.window if vc.window >= 0 else None
        ms = time_launches(lambda: fa.fwd_varlen(vq, vk, vv, vcu, int(vl.max()), causal=vc.causal, window=win,
                                                 scale=vc.scale, out=vo, lse=vlse))
        if win is not None:
            fl = sum(cm.window_flops(vc.heads_q, int(n), vc.head_dim, win) for n in vl)
        else:
            fl = cm.varlen_flops(vl, vc.heads_q, vc.head_dim, vc.causal)
        tf = fl / (ms * 1e-3) / 1e12
        extra[key] = {"ms": round(ms, 4), "value": round(tf, 2), "unit": "TFLOP/s",
                      "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "flops_per_launch": fl,
                      "workload": f"{vc.n_seqs} sequence(s), lengths {int(vl.min())}..{int(vl.max())} "
                                  f"(total {int(vl.sum())}), Hq{vc.heads_q} Hkv{vc.heads_kv} d{vc.head_dim}, "
                                  + (f"causal window {win}" if win is not None else "causal"),
                      "kernel": "fa_fwd_varlen"}
        del vq, vk, vv, vo
    # FP8 prefill of the step's workload: quantiser and attention timed separately
    signs = torch.from_numpy(np.random.default_rng([pc.seed, 7]).choice([-1.0, 1.0], pc.head_dim)
                             .astype(np.float32)).to(dev)
    quant = fa.fp8_quantize(q, k, v, signs)
    o8 = torch.empty_like(q)
    ms_q = time_launches(lambda: fa.fp8_quantize(q, k, v, signs))
    ms_a = time_launches(lambda: fa.fwd_fp8(quant, causal=True, scale=pc.scale, out=o8, lse=lse))
    fl = cm.attention_flops(pc.batch, pc.heads_q, pc.seqlen, pc.seqlen, pc.head_dim, True)
    extra["prefill_fp8"] = {"ms": round(ms_a, 4), "value": round(fl / (ms_a * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                            "frac_fp8_peak": round(fl / (ms_a * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
                            "quantize_ms": round(ms_q, 4), "flops_per_launch": fl,
                            "workload": "causal GQA B1 Hq64 Hkv8 N8192 d128, e4m3 with random-sign Hadamard",
                            "kernel": "fa_fwd_fp8 (fa_fp8_quantize timed apart)"}
    del quant, o8
    # backward of the step's prefill (same inputs, its O and LSE, a seeded dO)
    fa.fwd(q, k, v, causal=True, scale=pc.scale, out=o, lse=lse)
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(fa.load().fa_bwd_workspace_bytes(pc.batch, pc.heads_q, pc.seqlen), dtype=torch.uint8,
                      device=dev)
    ms = time_launches(lambda: fa.bwd(q, k, v, o, dout, lse, causal=True, scale=pc.scale, dq=gq, dk=gk, dv=gv,
                                      workspace=bws))
    fl = cm.backward_flops(pc.batch, pc.heads_q, pc.seqlen, pc.seqlen, pc.head_dim, True)
    extra["backward"] = {"ms": round(ms, 4), "value": round(fl / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s",
                         "frac_bf16_peak": round(fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                         "flops_per_launch": fl, "workload": "causal GQA B1 Hq64 Hkv8 N8192 d128, bf16 gradients",
                         "kernel": "fa_bwd (pre-pass + dK/dV + dQ)"}
    del dout, gq, gk, gv, bws

    configs = config_phases(config_in, fa, W, cm, time_launches, dev)
    clock = None if args.no_clock else observed_clock(
        lambda: fa.fwd(q, k, v, causal=True, scale=pc.scale, out=o, lse=lse), sum(pre_ms) / len(pre_ms))

    pre_flops = cm.attention_flops(pc.batch, pc.heads_q, pc.seqlen, pc.seqlen, pc.head_dim, causal=True)
    kv_bytes = cm.decode_kv_bytes(lens, dc.heads_kv, dc.head_dim)
    pre_avg = sum(pre_ms) / len(pre_ms)
    dec_avg = sum(dec_ms) / len(dec_ms)
    pre_tflops = pre_flops / (pre_avg * 1e-3) / 1e12
    dec_gbs = kv_bytes / (dec_avg * 1e-3) / 1e9
    pag_avg = sum(pag_ms) / len(pag_ms)
    pag_gbs = kv_bytes / (pag_avg * 1e-3) / 1e9
    ms_per_step = wall * 1e3 / args.steps

    traffic, traffic_dec, per_phase = load_traffic()
    for name, c in configs.items():
        c["traffic"] = per_phase.get(f"prefill {name}") if per_phase else None
    result = {
        "metric": "prefill attention TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% HBM peak)",
        "value": round(pre_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) bf16, 1% of K rows x8 in the prefill, uniform kv lengths in the decode",
        "config": {
            "workload": "causal GQA prefill B1 Hq64 Hkv8 N8192 d128 + split-KV decode B64 Hq64 Hkv8 L~U[1024,32768] d128",
            "prefill": {"batch": pc.batch, "heads_q": pc.heads_q, "heads_kv": pc.heads_kv, "seq_len": pc.seqlen,
                        "head_dim": pc.head_dim, "mask": "causal", "flops_per_launch": pre_flops},
            "decode": {"batch": dc.batch, "heads_q": dc.heads_q, "heads_kv": dc.heads_kv, "head_dim": dc.head_dim,
                       "sum_kv_len": int(lens.sum()), "kv_bytes_per_launch": kv_bytes,
                       "split_tokens": 0},
        },
        "prefill_ms": round(pre_avg, 4),
        "decode_ms": round(dec_avg, 4),
        "decode_value": {"value": round(dec_gbs, 1), "unit": "GB/s", "frac_hbm_peak": round(dec_gbs / PEAK_HBM_GBS, 4)},
        "decode_paged": {"ms": round(pag_avg, 4), "value": round(pag_gbs, 1), "unit": "GB/s",
                         "frac_hbm_peak": round(pag_gbs / PEAK_HBM_GBS, 4), "page_size": PAGE_SIZE,
                         "pool": "token-major [page, slot, kv head, d], shuffled block table",
                         "kernel": "fa_decode_paged (split + merge)"},
        "roofline": {"bound": "mfma", "achieved": round(pre_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(pre_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "fa_fwd (causal, d=128, bf16)"},
        "roofline_decode": {"bound": "hbm", "achieved": round(dec_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(dec_gbs / PEAK_HBM_GBS, 4), "traffic": traffic_dec,
                            "kernel": "fa_decode (split + merge)"},
        **extra,
        "configs": configs,
        "kernel_sources": sources_hash(),
    }
    if clock is not None:
        if clock.get("mhz_mean"):
            peak_clk = PEAK_BF16_TFLOPS * clock["mhz_mean"] / PEAK_CLOCK_MHZ
            clock["bf16_peak_at_this_clock"] = round(peak_clk, 1)
            clock["prefill_frac_at_this_clock"] = round(pre_tflops / peak_clk, 4)
        result["clock"] = clock
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(pc, args.cpu_seconds)
        result["cpu_baseline"]["host"] = host_info()
        for name, c in configs.items():
            c["oracle"] = oracle_timing(W.CONFIGS[name], ORACLE_SECONDS[name], c["ms"])
        result["decode_value"]["oracle"] = oracle_decode_timing(dc, lens, ORACLE_SECONDS["c5_decode"], dec_avg)
        result["cpu_baseline"]["oracle_per_config"] = {n: c["oracle"] for n, c in configs.items()}
        result["cpu_baseline"]["oracle_per_config"][DECODE_CFG] = result["decode_value"]["oracle"]
    print(json.dumps(result), flush=True)


def observed_clock(launch, launch_ms: float, seconds: float = 2.5, settle: float = 1.5):
    """The shader (GFX) clock the chip runs at under the prefill: `launch` runs
    back to back for `seconds`, and after `settle` seconds of that load the
    per-XCD current clocks are read from the SMU metrics (amdsmi), which
    refresh about once a second with roughly one-second averages. The bench
    does not pin clocks; this records what it observed. It runs after every
    timed region, so it perturbs none of them."""
    import torch
    try:
        import amdsmi
    except Exception as e:                   # noqa: BLE001 - reported, not fatal
        return {"source": None, "error": f"amdsmi not importable: {e}"}
    try:
        amdsmi.amdsmi_init()
    except Exception as e:                   # noqa: BLE001
        return {"source": None, "error": f"amdsmi_init failed: {e}"}
    try:
        handles = amdsmi.amdsmi_get_processor_handles()
        if len(handles) != 1:
            return {"source": None, "error": f"{len(handles)} GPUs visible to amdsmi; the bench's one is ambiguous"}
        chunk = max(1, int(100.0 / max(launch_ms, 1e-3)))       # about 0.1 s of GPU work
        t0 = time.time()
        reads = []
        while time.time() - t0 < seconds:
            for _ in range(chunk):
                launch()
            torch.cuda.synchronize()
            if time.time() - t0 >= settle:
                m = amdsmi.amdsmi_get_gpu_metrics_info(handles[0])
                clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 65535]
                if not clks and isinstance(m.get("current_gfxclk"), (int, float)):
                    clks = [m["current_gfxclk"]]
                if clks:
                    reads.append(clks)
        if not reads:
            return {"source": None, "error": "no current GFX clock in the SMU metrics"}
        k = len(reads[-1])
        rows = [r for r in reads if len(r) == k]
        mean_x = [round(sum(r[i] for r in rows) / len(rows), 1) for i in range(k)]
        return {"source": "amdsmi GPU metrics, current_gfxclks (per XCD, ~1 s averages)",
                "under": f"fa_fwd c4a back to back for {seconds:g} s, read after {settle:g} s",
                "reads": len(rows), "mhz_per_xcd": mean_x, "mhz_mean": round(sum(mean_x) / len(mean_x), 1),
                "peak_assumes_mhz": PEAK_CLOCK_MHZ}
    except Exception as e:                   # noqa: BLE001
        torch.cuda.synchronize()
        return {"source": None, "error": f"amdsmi query failed: {e}"}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:                    # noqa: BLE001
            pass


def config_inputs(W, to_dev, dev):
    """Device inputs of every configuration in CONFIG_PHASES (generated before
    the first timed region)."""
    import numpy as np
    import torch
    out = {}
    for name in CONFIG_PHASES:
        c = W.CONFIGS[name]
        qh, kh, vh = W.make_prefill_inputs(c)
        up = (lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(dev)) if c.dtype == "fp32" else to_dev
        out[name] = (up(qh), up(kh), up(vh))
        del qh, kh, vh
    return out


def config_phases(config_in, fa, W, cm, time_launches, dev):
    """Every other prefill configuration, timed on its own with HIP events:
    algorithmic TFLOP/s (4 B Hq N^2 d, halved for causal), fraction of the bf16
    peak. The fp32 single head is launch-bound (its bar is parity)."""
    import torch
    out = {}
    for name in CONFIG_PHASES:
        c = W.CONFIGS[name]
        t0 = time.time()
        q, k, v = config_in.pop(name)
        o = torch.empty(q.shape, dtype=torch.bfloat16 if c.dtype == "bf16" else torch.float32, device=dev)
        lse = torch.empty(c.batch, c.heads_q, c.seqlen, dtype=torch.float32, device=dev)
        ms = time_launches(lambda: fa.fwd(q, k, v, causal=c.causal, scale=c.scale, out=o, lse=lse),
                           CONFIG_EXTRA_WARMUP.get(name, 0))
        fl = cm.attention_flops(c.batch, c.heads_q, c.seqlen, c.seqlen, c.head_dim, c.causal)
        tf = fl / (ms * 1e-3) / 1e12
        out[name] = {"ms": round(ms, 4), "value": round(tf, 2), "unit": "TFLOP/s",
                     "frac_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4), "flops_per_launch": fl,
                     "workload": f"B{c.batch} Hq{c.heads_q} Hkv{c.heads_kv} N{c.seqlen} d{c.head_dim} "
                                 f"{'causal' if c.causal else 'no mask'}, {c.dtype} in, {o.dtype} out".replace(
                                     "torch.", ""),
                     "kernel": "fa_fwd"}
        print(f"[bench] {name}: {ms:.4f} ms, {tf:.1f} TFLOP/s ({time.time() - t0:.2f}s)",
              file=sys.stderr, flush=True)
        del q, k, v, o, lse
    return out


def host_info():
    """CPU model, core counts and NumPy's BLAS build of the host the oracle ran on."""
    import numpy as np
    import threadpoolctl
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = [{k: i.get(k) for k in ("internal_api", "version", "num_threads", "architecture")}
            for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cores": len(os.sched_getaffinity(0)),
            "numpy": np.__version__, "blas": blas}


def oracle_timing(c, seconds: float, gpu_ms: float):
    """The fp64 oracle on whole query heads of a prefill configuration (spread
    over the kv groups) until about ``seconds`` of work: seconds per head,
    executed fp64 GFLOP/s (the oracle materialises every score, so 4 Nq Nk d
    per head even under the causal mask), the whole configuration's projected
    oracle time and the GPU's speedup over it (context only)."""
    from io_aware_flashattention_amd import workloads as W
    from oracle import attention_ref
    heads, elapsed = [], 0.0
    units = [(b, h) for h in [(9 * i) % c.heads_q for i in range(c.heads_q)] for b in range(c.batch)]
    for b, h in units:
        kvh = h // c.group
        q = W.to_f64(W.prefill_slice(c, "q", b, h))[None, None]
        k = W.to_f64(W.prefill_slice(c, "k", b, kvh))[None, None]
        v = W.to_f64(W.prefill_slice(c, "v", b, kvh))[None, None]
        ts = time.perf_counter()
        attention_ref(q, k, v, c.scale, causal=c.causal)
        elapsed += time.perf_counter() - ts
        heads.append((b, h))
        if elapsed >= seconds:
            break
    per_head = elapsed / len(heads)
    whole = per_head * c.batch * c.heads_q
    return {"heads_timed": len(heads), "seconds": round(elapsed, 3), "seconds_per_head": round(per_head, 4),
            "executed_fp64_gflops": round(4.0 * c.seqlen * c.seqlen * c.head_dim * len(heads) / elapsed / 1e9, 2),
            "projected_config_seconds": round(whole, 2), "gpu_speedup": round(whole / (gpu_ms * 1e-3), 1)}


def oracle_decode_timing(dc, lens, seconds: float, gpu_ms: float):
    """The fp64 oracle on whole sequences of the decode workload until about
    ``seconds`` of work, projected to all sequences."""
    import numpy as np

    from io_aware_flashattention_amd import workloads as W
    from oracle import decode_ref
    done, toks, elapsed = 0, 0, 0.0
    for b in range(dc.batch):
        n = int(lens[b])
        q = W.to_f64(W.decode_query(dc, b))[None]
        k = np.stack([W.to_f64(W.decode_kv_slice(dc, "k", b, h, n)) for h in range(dc.heads_kv)])[None]
        v = np.stack([W.to_f64(W.decode_kv_slice(dc, "v", b, h, n)) for h in range(dc.heads_kv)])[None]
        ts = time.perf_counter()
        decode_ref(q, k, v, np.array([n]), dc.scale)
        elapsed += time.perf_counter() - ts
        done += 1
        toks += n
        if elapsed >= seconds:
            break
    whole = elapsed * float(lens.sum()) / toks
    return {"sequences_timed": done, "seconds": round(elapsed, 3), "projected_config_seconds": round(whole, 2),
            "gpu_speedup": round(whole / (gpu_ms * 1e-3), 1)}


def load_traffic():
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources (else null)."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None, None, None
    if d.get("kernel_sources") != sources_hash():
        return None, None, None
    per = {k: v["fetch"] + v["write"] for k, v in d.get("per_phase_bytes", {}).items()}
    return d.get("prefill_bytes_per_launch"), d.get("decode_bytes_per_launch"), per


def cpu_baseline(pc, seconds: float):
    """The fp64 oracle, as it stands, on whole query heads of the prefill
    workload until about ``seconds`` of CPU work; scaled to TFLOP/s with the
    same algorithmic causal FLOP count as the GPU figure."""
    import threadpoolctl

    from io_aware_flashattention_amd import cost_model as cm
    from io_aware_flashattention_amd import workloads as W
    from oracle import attention_ref

    threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"),
                  default=1)
    heads = []
    t0 = time.perf_counter()
    elapsed = 0.0
    for h in [(9 * i) % pc.heads_q for i in range(pc.heads_q)]:   # spread over kv groups
        kvh = h // pc.group
        q = W.to_f64(W.prefill_slice(pc, "q", 0, h))[None, None]
        k = W.to_f64(W.prefill_slice(pc, "k", 0, kvh))[None, None]
        v = W.to_f64(W.prefill_slice(pc, "v", 0, kvh))[None, None]
        ts = time.perf_counter()
        attention_ref(q, k, v, pc.scale, causal=True)
        elapsed += time.perf_counter() - ts
        heads.append(h)
        if elapsed >= seconds:
            break
    flops = cm.attention_flops(1, len(heads), pc.seqlen, pc.seqlen, pc.head_dim, causal=True)
    print(f"[bench] cpu baseline: {len(heads)} heads in {elapsed:.1f}s ({time.perf_counter() - t0:.1f}s with input "
          f"generation)", file=sys.stderr, flush=True)
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"fp64 oracle on {len(heads)} whole query heads {heads} of the causal B1 Hq64 Hkv8 N8192 d128 "
                      f"prefill ({elapsed:.1f} s); host os.cpu_count()={os.cpu_count()}"}


# ------------------------------------------------------ profile summaries --

def _read_csv(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _dispatch_labels(rows, name_key: str, n_launch: int):
    """Label per-dispatch rows (sorted by Dispatch_Id) with the bench phase
    they belong to. The bench launches, in this order: n_launch steps of
    (prefill, decode split, decode merge); n_launch paged decodes (paged split,
    merge); n_launch window prefills; n_launch packed prefills; the fp8
    quantiser and prefill (their own kernels); one prefill for the backward's
    inputs, then n_launch backward passes; then n_launch prefills of each
    configuration in CONFIG_PHASES (plus its CONFIG_EXTRA_WARMUP). One prefill
    kernel serves several phases, so the phase comes from the dispatch order."""
    rows = sorted(rows, key=lambda r: int(r["Dispatch_Id"]))
    seen = {"fwd": 0, "merge": 0}
    fwd_phases = [("prefill c4a (step)", n_launch), ("prefill window c7", n_launch),
                  ("prefill varlen c6", n_launch), ("prefill c4a (backward inputs)", 1)]
    fwd_phases += [(f"prefill {c}", n_launch + CONFIG_EXTRA_WARMUP.get(c, 0)) for c in CONFIG_PHASES]

    def fwd_label(i):
        for label, n in fwd_phases:
            if i < n:
                return label
            i -= n
        return None
    out = []
    for r in rows:
        name = r.get(name_key, "")
        if "fp8" in name:
            label = "fp8 " + re.sub(r".*((?:fwd|fp8)_\w*?_kernel).*", r"\1", name)
        elif re.search(r"fwd_\w*kernel", name):
            i = seen["fwd"]
            seen["fwd"] += 1
            label = fwd_label(i)
        elif "bwd_" in name:
            label = "backward " + re.sub(r".*(bwd_\w+?_kernel).*", r"\1", name)
        elif "decode_split" in name:            # contiguous: template flag false (mangled "Lb0E")
            label = "decode split (step)" if ("Lb0E" in name or "false" in name) else "paged decode split"
        elif "decode_merge" in name:
            i = seen["merge"]
            seen["merge"] += 1
            label = "decode merge (step)" if i < n_launch else "paged decode merge"
        else:
            label = None
        out.append((label, r))
    return out


def summarize_trace(d: str, out: str, cmd: str, n_launch: int, n_timed: int):
    """rocprofv3 --kernel-trace --stats output directory -> short text tables:
    per bench phase from the per-dispatch trace, then rocprofv3's own stats."""
    stats = sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True))
    trace = sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True))
    if not stats or not trace:
        sys.exit(f"no kernel_stats.csv / kernel_trace.csv under {d}")
    lines = [f"# rocprofv3 kernel statistics", "", f"command: `{cmd}`", "",
             f"kernel sources: {sources_hash()}", "",
             f"Per bench phase (per-dispatch trace; {n_launch} launches per phase: the warm-up, then the "
             f"{n_timed} timed ones; extra warm-up launches: {CONFIG_EXTRA_WARMUP}):", "",
             f"| phase | kernel | dispatches | avg us (all) | avg us (last {n_timed}) | min us | max us |",
             "|---|---|---|---|---|---|---|"]
    groups = {}
    for label, r in _dispatch_labels(_read_csv(trace[0]), "Kernel_Name", n_launch):
        if label is None:
            continue
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault((label, r["Kernel_Name"]), []).append(dur)
    for (label, name), ds in groups.items():
        short = name if len(name) < 70 else name[:67] + "..."
        tail = ds[-n_timed:]
        lines.append(f"| {label} | `{short}` | {len(ds)} | {sum(ds) / len(ds):.2f} | {sum(tail) / len(tail):.2f} | "
                     f"{min(ds):.2f} | {max(ds):.2f} |")
    lines += ["", "rocprofv3 --stats (per kernel name; the prefill kernel's row mixes its three phases):", "",
              "| kernel | calls | avg us | min us | max us | total % |", "|---|---|---|---|---|---|"]
    for r in _read_csv(stats[0]):
        name = r.get("Name", "")
        short = name if len(name) < 90 else name[:87] + "..."
        avg = float(r.get("AverageNs", 0)) / 1e3
        lines.append(f"| `{short}` | {r.get('Calls')} | {avg:.2f} | {float(r.get('MinNs', 0)) / 1e3:.2f} | "
                     f"{float(r.get('MaxNs', 0)) / 1e3:.2f} | {float(r.get('Percentage', 0)):.2f} |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_pmc(fetch_dir: str, write_dir: str, out: str, cmd_fetch: str, cmd_write: str, n_launch: int):
    """Two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of this bench -> HBM
    bytes per launch of each kernel of the step, scaled by what the counters
    read for the calibration copy of known size."""
    def per_phase(dd, counter):
        files = sorted(glob.glob(os.path.join(dd, "**", "*counter_collection.csv"), recursive=True))
        if not files:
            sys.exit(f"no counter_collection.csv under {dd}")
        rows = [r for r in _read_csv(files[0]) if r.get("Counter_Name") == counter]
        acc, copy = {}, []
        for label, r in _dispatch_labels(rows, "Kernel_Name", n_launch):
            v = float(r.get("Counter_Value", 0)) * 1024.0          # KiB -> bytes
            if label is not None:
                acc.setdefault(label, []).append(v)
            elif "copy" in r["Kernel_Name"].lower() or "elementwise" in r["Kernel_Name"].lower():
                copy.append(v)
        return {k: sum(v) / len(v) for k, v in acc.items()}, (max(copy) if copy else None)

    fetch, copy_fetch = per_phase(fetch_dir, "FETCH_SIZE")
    write, copy_write = per_phase(write_dir, "WRITE_SIZE")
    sf = COPY_BYTES / copy_fetch if copy_fetch else 1.0
    sw = COPY_BYTES / copy_write if copy_write else 1.0
    g = lambda acc, k: acc.get(k, 0.0)
    d = {
        "kernel_sources": sources_hash(),
        "command_fetch": cmd_fetch, "command_write": cmd_write,
        "copy_calibration": {"bytes": COPY_BYTES, "fetch_counter_bytes": copy_fetch, "write_counter_bytes": copy_write,
                             "fetch_scale": sf, "write_scale": sw},
        "per_phase_bytes": {k: {"fetch": g(fetch, k) * sf, "write": g(write, k) * sw}
                            for k in sorted(set(fetch) | set(write))},
        "prefill_fetch_bytes": g(fetch, "prefill c4a (step)") * sf,
        "prefill_write_bytes": g(write, "prefill c4a (step)") * sw,
        "decode_fetch_bytes": (g(fetch, "decode split (step)") + g(fetch, "decode merge (step)")) * sf,
        "decode_write_bytes": (g(write, "decode split (step)") + g(write, "decode merge (step)")) * sw,
    }
    d["prefill_bytes_per_launch"] = d["prefill_fetch_bytes"] + d["prefill_write_bytes"]
    d["decode_bytes_per_launch"] = d["decode_fetch_bytes"] + d["decode_write_bytes"]
    with open(out, "w") as f:
        json.dump(d, f, indent=2)
    print(json.dumps(d, indent=2))


MOPS_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_F6F4")
MOPS_FLOPS = 512              # FLOPs per unit of the SQ_INSTS_VALU_MFMA_MOPS_* counters


def phase_flops():
    """Algorithmic FLOPs per launch of each bench phase that runs on the
    matrix cores, counted as in the bench line (4 d per visible pair; the
    backward's five products). Decode, priced in bytes, is listed as 4 Hq d
    per cached token for the counter cross-check."""
    from io_aware_flashattention_amd import cost_model as cm
    from io_aware_flashattention_amd import workloads as W
    pc = W.CONFIGS["c4a_gqa_8k"]
    pre = cm.attention_flops(pc.batch, pc.heads_q, pc.seqlen, pc.seqlen, pc.head_dim, True)
    out = {"prefill c4a (step)": pre, "prefill c4a (backward inputs)": pre, "fp8 fwd_fp8_kernel": pre,
           "backward (dK/dV + dQ)": cm.backward_flops(pc.batch, pc.heads_q, pc.seqlen, pc.seqlen, pc.head_dim, True)}
    for name in CONFIG_PHASES:
        c = W.CONFIGS[name]
        out[f"prefill {name}"] = cm.attention_flops(c.batch, c.heads_q, c.seqlen, c.seqlen, c.head_dim, c.causal)
    for label, name in (("prefill window c7", "c7_window_8k"), ("prefill varlen c6", "c6_varlen_causal")):
        vc = W.VARLEN_CONFIGS[name]
        vl = W.varlen_lengths(vc)
        if vc.window >= 0:
            out[label] = sum(cm.window_flops(vc.heads_q, int(n), vc.head_dim, vc.window) for n in vl)
        else:
            out[label] = cm.varlen_flops(vl, vc.heads_q, vc.head_dim, vc.causal)
    dc = W.DECODE_CONFIGS["c5_decode"]
    dec = 4 * dc.heads_q * dc.head_dim * int(W.decode_lengths(dc).sum())   # q K^T and P V per cached token
    out["decode split (step)"] = out["paged decode split"] = dec
    return out


def summarize_mops(d: str, out: str, cmd: str, n_launch: int):
    """rocprofv3 --pmc run of this bench with the MFMA-op counters -> FLOPs the
    matrix cores executed per launch of each phase, beside the algorithmic
    count. Executed >= algorithmic; the excess is masked work on diagonal and
    ragged tiles, the weight-sum products, (backward) S and dP computed in
    both kernels, and (decode) the 24 of 32 matrix columns that one kv head's
    8 query rows leave empty."""
    files = sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True))
    if not files:
        sys.exit(f"no counter_collection.csv under {d}")
    rows = _read_csv(files[0])
    flops = {}
    for counter in MOPS_COUNTERS:               # one row per dispatch and counter: label each counter apart
        per = {}
        for label, r in _dispatch_labels([r for r in rows if r.get("Counter_Name") == counter], "Kernel_Name",
                                         n_launch):
            if label is None:
                continue
            key = "backward (dK/dV + dQ)" if label.startswith(("backward bwd_dkdv", "backward bwd_dq")) else label
            per.setdefault(key, {}).setdefault(label, []).append(float(r["Counter_Value"]))
        for key, parts in per.items():           # average over launches, summed over a phase's kernels
            flops.setdefault(key, {})[counter] = sum(sum(x) / len(x) for x in parts.values()) * MOPS_FLOPS
    alg = phase_flops()
    lines = ["# MFMA work executed per launch (rocprofv3 counters)", "", f"command: `{cmd}`", "",
             f"kernel sources: {sources_hash()}", "",
             f"FLOPs = counter x {MOPS_FLOPS}, averaged over a phase's launches; algorithmic FLOPs as in the bench line.",
             "", "| phase | bf16 MFMA FLOPs | fp8 MFMA FLOPs | fp4 MFMA FLOPs | algorithmic FLOPs | executed / algorithmic |",
             "|---|---|---|---|---|---|"]
    for label in sorted(flops):
        f = flops[label]
        ex = sum(f.values())
        a = alg.get(label)
        ratio = f"{ex / a:.3f}" if a else "—"
        lines.append(f"| {label} | {f.get(MOPS_COUNTERS[0], 0):.4g} | {f.get(MOPS_COUNTERS[1], 0):.4g} | "
                     f"{f.get(MOPS_COUNTERS[2], 0):.4g} | {a:.4g} | {ratio} |" if a else
                     f"| {label} | {f.get(MOPS_COUNTERS[0], 0):.4g} | {f.get(MOPS_COUNTERS[1], 0):.4g} | "
                     f"{f.get(MOPS_COUNTERS[2], 0):.4g} | — | — |")
    with open(out, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-clock", action="store_true", help="skip sampling the shader clock after the timed regions")
    ap.add_argument("--summarize-trace", metavar="DIR")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--summarize-mops", metavar="DIR")
    ap.add_argument("--cmd", nargs="*", default=[], help="commands recorded in a summary")
    ap.add_argument("--out")
    args = ap.parse_args()
    n_launch = args.warmup + args.steps       # launches per bench phase of the profiled run
    if args.summarize_trace:
        return summarize_trace(args.summarize_trace, args.out, " ".join(args.cmd), n_launch, args.steps)
    if args.summarize_mops:
        return summarize_mops(args.summarize_mops, args.out, " ".join(args.cmd), n_launch)
    if args.summarize_pmc:
        cmds = args.cmd + ["", ""]
        return summarize_pmc(*args.summarize_pmc, args.out, cmds[0], cmds[1], n_launch)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        sys.exit("bench.py measures one GPU (--gpus 1): the attention path runs on a single MI355X "
                 "and has no multi-GPU mode")
    run(args)


if __name__ == "__main__":
    main()
