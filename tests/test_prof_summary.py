"""Host logic of the rocprofv3 summaries (no GPU): symbol -> step mapping,
copy-kernel calibration of the HBM counters, and the source-hash stamp."""
import csv

from chunked_top_kl_amd.prof_summary import (kernel_sources_hash, read_summary_json, step_of,
                                             summarize_trace, summarize_traffic)

PMC_FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]


def _pmc_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=PMC_FIELDS)
        w.writeheader()
        for i, (name, val) in enumerate(rows):
            w.writerow(dict(Dispatch_Id=i, Kernel_Name=name, Counter_Name=counter,
                            Counter_Value=val))


def test_step_names():
    assert step_of("kd_bwd_dw_bf16") == "bwd_dw"
    assert step_of("kd_fwd_lse_gather_rows_bf16") == "fwd_lse_gather"
    assert step_of("kd_bwd_grad_tile_f32") == "bwd_grad_tile"
    assert step_of("kd::dh_reduce_kernel(kd::DhReduceArgs, int)") == "bwd_dhidden_reduce"
    assert step_of("kd_bwd_dhidden_bf16") == "bwd_dhidden"
    assert step_of("__amd_rocclr_copyBuffer") == "device_copy"
    assert step_of("something_else") == "other"


def test_traffic_calibration(tmp_path):
    # a 4 MiB copy that FETCH_SIZE counts at half and WRITE_SIZE at full size
    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    _pmc_csv(f, "FETCH_SIZE", [("__amd_rocclr_copyBuffer", 2048.0), ("__amd_rocclr_copyBuffer", 1.0),
                               ("kd_bwd_dw_bf16", 100.0), ("kd_bwd_dw_bf16", 300.0)])
    _pmc_csv(w, "WRITE_SIZE", [("__amd_rocclr_copyBuffer", 4096.0),
                               ("kd_bwd_dw_bf16", 50.0), ("kd_bwd_dw_bf16", 50.0)])
    text = summarize_traffic(str(f), str(w), 4, ["cmd"], "wl")
    out = tmp_path / "s.md"
    out.write_text(text)
    js = read_summary_json(str(out))
    assert js["kernel_sources_sha256"] == kernel_sources_hash()
    assert abs(js["calibration"]["fetch_factor"] - 2.0) < 1e-12
    assert abs(js["calibration"]["write_factor"] - 1.0) < 1e-12
    dw = js["steps"]["bwd_dw"]
    assert dw["launches"] == 2
    assert dw["read_bytes"] == 200 * 1024 * 2          # mean 200 KiB, x2
    assert dw["write_bytes"] == 50 * 1024
    assert dw["traffic_bytes"] == dw["read_bytes"] + dw["write_bytes"]


def test_trace_summary(tmp_path):
    p = tmp_path / "k.csv"
    with open(p, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Name", "Calls", "TotalDurationNs", "AverageNs"])
        w.writeheader()
        w.writerow(dict(Name="kd_bwd_dw_bf16", Calls=4, TotalDurationNs=4e6, AverageNs=1e6))
        w.writerow(dict(Name="kd_fwd_lse_gather_bf16", Calls=1, TotalDurationNs=3e6, AverageNs=3e6))
        w.writerow(dict(Name="kd_fwd_lse_gather_rows_bf16", Calls=1, TotalDurationNs=1e6,
                        AverageNs=1e6))
    out = tmp_path / "t.md"
    out.write_text(summarize_trace(str(p), ["cmd"], "wl", 1))
    js = read_summary_json(str(out))
    assert js["steps"]["bwd_dw"]["avg_ms"] == 1.0
    assert js["steps"]["fwd_lse_gather"]["launches"] == 2
    assert js["steps"]["fwd_lse_gather"]["avg_ms"] == 2.0


def _kernel_names():
    """Names of every __global__ kernel defined in the library's sources."""
    import os
    import re
    from chunked_top_kl_amd.prof_summary import CSRC
    names = set()
    for fn in sorted(os.listdir(CSRC)):
        if not fn.endswith(".hip"):
            continue
        text = open(os.path.join(CSRC, fn)).read()
        for m in re.finditer(r"__global__\s+(?:__launch_bounds__\([^)]*\)\s*)?void\s+"
                             r"([A-Za-z_][A-Za-z_0-9]*)\s*\(", text):
            names.add(m.group(1))
        # kernels stamped out by a macro: KD_SWEEP_KERNEL(name, ...)
        for m in re.finditer(r"^KD_SWEEP_KERNEL\(([A-Za-z_0-9]+),", text, re.M):
            names.add(m.group(1))
    names.discard("NAME")
    return names


def test_every_kernel_maps_to_a_step():
    names = _kernel_names()
    assert "prepass_reg_kernel" in names and "kd_bwd_dw_bf16" in names and len(names) > 50
    unmapped = sorted(n for n in names if step_of(n) == "other")
    assert not unmapped, unmapped
    assert step_of("void kd::prepass_reg_kernel<64>(kd::PrepassArgs)") == "prepass"
    assert step_of("kd::grad_teacher_kernel<__bf16>(kd::GradTeacherArgs)") == "bwd_grad_teacher"
    assert step_of("teacher_gather_kernel") == "teacher_gather"
    assert step_of("kd_sample_draw_tiles_bf16") == "sample_draw"
    assert step_of("kd::draw_tile_fill_kernel(int const*, int, int, int const*, int*, int*)") == "sample_draw"
    assert step_of("kd::sample_refined_entropy_kernel(kd::SelectWs, int, int, double*)") == \
        "select_refine_fp64"


def test_counter_summary(tmp_path):
    from chunked_top_kl_amd.prof_summary import summarize_counters
    a = tmp_path / "a.csv"
    b = tmp_path / "b.csv"
    _pmc_csv(a, "MfmaUtil", [("kd_bwd_dw_bf16", 60.0), ("kd_bwd_dw_bf16", 50.0)])
    with open(b, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=PMC_FIELDS)
        w.writeheader()
        for i, (c, v) in enumerate((("TCC_HIT_sum", 90.0), ("TCC_MISS_sum", 10.0),
                                    ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 2.0))):
            w.writerow(dict(Dispatch_Id=0, Kernel_Name="kd_bwd_dw_bf16", Counter_Name=c,
                            Counter_Value=v))
    out = tmp_path / "c.md"
    out.write_text(summarize_counters([str(a), str(b)], ["cmd"], "wl"))
    js = read_summary_json(str(out))
    d = js["steps"]["bwd_dw"]["derived"]
    assert d["mfma_util_pct"] == 55.0
    assert abs(d["l2_hit_rate"] - 0.9) < 1e-12
    assert d["bf16_mfma_flop"] == 1024.0
