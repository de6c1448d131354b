"""Host logic of bench.py's profile summaries, on synthetic rocprofv3 CSVs.

The summaries label each dispatch with the bench phase it belongs to from the
dispatch order alone (the bf16 prefill kernel is one instantiation in four
phases), so the order the bench launches in is written out here once and
every summary is checked against it.
"""
import csv
import json

import bench

FWD = "_ZN2fa6detail13fwd_pp_kernelILi128ELb1EDF16bLi3EEEvNS_9FwdParamsE"
SPLIT = "_ZN2fa6detail19decode_split_kernelIDF16bLb0EEEvNS_12DecodeParamsE"
PAGED = "void fa::detail::decode_split_kernel<bool _Accum, bool, E>(fa::DecodeParams)"
MERGE = "_ZN2fa6detail19decode_merge_kernelIDF16bEEvNS_12DecodeParamsE"
FP8 = [("void fa::detail::fp8_quant_qk_kernel<128>(fa::Fp8QuantParams, int)", "fp8 fp8_quant_qk_kernel"),
       ("void fa::detail::fp8_quant_qk_kernel<64>(fa::Fp8QuantParams, int)", "fp8 fp8_quant_qk_kernel"),
       ("fa::detail::fp8_v_amax_kernel(fa::Fp8QuantParams)", "fp8 fp8_v_amax_kernel"),
       ("fa::detail::fp8_quant_v_kernel(fa::Fp8QuantParams)", "fp8 fp8_quant_v_kernel"),
       ("fa::detail::fp8_v_scale_kernel(fa::Fp8QuantParams)", "fp8 fp8_v_scale_kernel")]
FWD8 = "_ZN2fa6detail14fwd_fp8_kernelIDF16bEEvNS_12Fp8FwdParamsE"
BWD = [("void fa::detail::bwd_pre_kernel<128>(fa::BwdParams)", "backward bwd_pre_kernel"),
       ("_ZN2fa6detail15bwd_dkdv_kernelILi128ELb1EDF16bEEvNS_9BwdParamsE", "backward bwd_dkdv_kernel"),
       ("_ZN2fa6detail13bwd_dq_kernelILi128ELb1EDF16bEEvNS_9BwdParamsE", "backward bwd_dq_kernel")]
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float>>"
F32 = "_ZN2fa6detail14fwd_f32_kernelILi64ELb0EfEEvNS_9FwdParamsE"
FWD64 = "_ZN2fa6detail15fwd_bf16_kernelILi64ELb1EDF16bLi4ELi1ELi3EEEvNS_9FwdParamsE"
FWD_NONE = "_ZN2fa6detail13fwd_pp_kernelILi128ELb0EDF16bLi3EEEvNS_9FwdParamsE"


def bench_dispatches(n):
    """(kernel, expected label) in the order bench.py launches them, n launches per phase."""
    seq = [(COPY, None)]
    for _ in range(n):
        seq += [(FWD, "prefill c4a (step)"), (SPLIT, "decode split (step)"), (MERGE, "decode merge (step)")]
    for _ in range(n):
        seq += [(PAGED, "paged decode split"), (MERGE, "paged decode merge")]
    seq += [(FWD, "prefill window c7")] * n
    seq += [(FWD, "prefill varlen c6")] * n
    for _ in range(n):
        seq += FP8
    seq += [(FWD8, "fp8 fwd_fp8_kernel")] * n
    seq += [(FWD, "prefill c4a (backward inputs)")]
    for _ in range(n):
        seq += BWD
    for cfg, kern in zip(bench.CONFIG_PHASES, (F32, FWD64, FWD, FWD_NONE, FWD)):
        seq += [(kern, f"prefill {cfg}")] * (n + bench.CONFIG_EXTRA_WARMUP.get(cfg, 0))
    return seq


def test_dispatch_labels_follow_the_bench_order():
    n = 3
    seq = bench_dispatches(n)
    rows = [{"Dispatch_Id": str(i + 1), "Kernel_Name": k} for i, (k, _) in enumerate(seq)]
    got = [label for label, _ in bench._dispatch_labels(rows[::-1], "Kernel_Name", n)]   # any row order
    assert got == [lab for _, lab in seq]


def write_counters(path, seq, values):
    """One row per (dispatch, counter): values(kernel, label) -> [(counter, value), ...]."""
    path.mkdir(parents=True, exist_ok=True)
    with open(path / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (k, lab) in enumerate(seq):
            for c, v in values(k, lab):
                w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_mops_summary_labels_each_counter_apart(tmp_path):
    """Three counters per dispatch must not shift the phase labels."""
    n = 2
    seq = bench_dispatches(n)
    units = {"prefill c4a (step)": 10.0, "prefill window c7": 3.0, "prefill varlen c6": 7.0,
             "prefill c4a (backward inputs)": 10.0, "backward bwd_dkdv_kernel": 5.0, "backward bwd_dq_kernel": 4.0,
             "decode split (step)": 1.0, "paged decode split": 1.0}

    def values(k, lab):
        bf = units.get(lab, 0.0)
        f8 = 11.0 if lab == "fp8 fwd_fp8_kernel" else 0.0
        return [("SQ_INSTS_VALU_MFMA_MOPS_BF16", bf), ("SQ_INSTS_VALU_MFMA_MOPS_F8", f8),
                ("SQ_INSTS_VALU_MFMA_MOPS_F6F4", 0.0)]

    write_counters(tmp_path / "mops", seq, values)
    out = tmp_path / "m.md"
    bench.summarize_mops(str(tmp_path / "mops"), str(out), "cmd", n)
    rows = {}
    for line in out.read_text().splitlines():
        cells = [c.strip() for c in line.strip("|").split("|")]
        if len(cells) == 6 and cells[0] not in ("phase", "---"):
            rows[cells[0]] = cells
    u = bench.MOPS_FLOPS
    assert float(rows["prefill c4a (step)"][1]) == 10.0 * u
    assert float(rows["prefill window c7"][1]) == 3.0 * u
    assert float(rows["prefill varlen c6"][1]) == 7.0 * u
    assert float(rows["backward (dK/dV + dQ)"][1]) == 9.0 * u       # both kernels of one backward pass
    assert float(rows["fp8 fwd_fp8_kernel"][2]) == 11.0 * u
    alg = bench.phase_flops()
    assert float(rows["prefill c4a (step)"][5]) == round(10.0 * u / alg["prefill c4a (step)"], 3)


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path):
    n = 2
    seq = bench_dispatches(n)

    def kib(counter, k, lab, on_copy):
        if k == COPY:
            return [(counter, on_copy)]
        return [(counter, {"prefill c4a (step)": 100.0, "decode split (step)": 1000.0,
                           "decode merge (step)": 2.0}.get(lab, 1.0))]

    write_counters(tmp_path / "f", seq, lambda k, lab: kib("FETCH_SIZE", k, lab, bench.COPY_BYTES / 2 / 1024))
    write_counters(tmp_path / "w", seq, lambda k, lab: kib("WRITE_SIZE", k, lab, bench.COPY_BYTES / 1024))
    out = tmp_path / "t.json"
    bench.summarize_pmc(str(tmp_path / "f"), str(tmp_path / "w"), str(out), "cf", "cw", n)
    d = json.loads(out.read_text())
    assert d["copy_calibration"]["fetch_scale"] == 2.0 and d["copy_calibration"]["write_scale"] == 1.0
    assert d["prefill_fetch_bytes"] == 100.0 * 1024 * 2.0
    assert d["prefill_write_bytes"] == 100.0 * 1024
    assert d["decode_fetch_bytes"] == (1000.0 + 2.0) * 1024 * 2.0
    assert d["kernel_sources"] == bench.sources_hash()
