"""Short text summaries of rocprofv3 output for the top-K KL kernels.

Two summaries are produced from rocprofv3's CSV output:

* ``trace``: per-step kernel durations from ``--kernel-trace --stats``
  (``*_kernel_stats.csv``), one row per path step.
* ``traffic``: HBM bytes per launch from two ``--pmc`` runs (``FETCH_SIZE``,
  then ``WRITE_SIZE``, each reported in KiB per dispatch). Each counter is
  scaled by what it reads for a device-to-device copy of a known size (run in
  the same process: ``bench.py --calib-copy-mib``), since these counters need
  not count every byte once.

Every summary records the SHA-256 of the kernel sources (``csrc/``) it was
measured with; ``bench.py`` reports the traffic figure only while the sources
still hash to that value.

Usage::

    python -m chunked_top_kl_amd.prof_summary trace --stats X_kernel_stats.csv \\
        --out profiles/kernel_trace_<workload>.md --command "<command that made X>"
    python -m chunked_top_kl_amd.prof_summary traffic --fetch F.csv --write W.csv \\
        --calib-mib 1024 --out profiles/hbm_traffic_<workload>.md \\
        --command "<FETCH command>" --command "<WRITE command>"
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import re

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")

# kernel symbol (mangled or demangled) -> path step, as named by the library's
# profiling scopes; the first matching pattern wins
STEP_PATTERNS = [
    ("kd_fwd_lse_gather_keep", "fwd_lse_gather_keep"),
    ("kd_fwd_lse_gather", "fwd_lse_gather"),
    ("kd_grad_tile_from_logits", "grad_tile_from_logits"),
    ("kd_bwd_grad_tile", "bwd_grad_tile"),
    ("kd_entropy_sweep", "entropy_sweep"),
    ("kd_bwd_dhidden", "bwd_dhidden"),
    ("kd_bwd_dw", "bwd_dw"),
    ("dh_reduce_kernel", "bwd_dhidden_reduce"),
    ("grad_teacher_kernel", "bwd_grad_teacher"),
    ("fwd_combine_kernel", "fwd_combine"),
    ("fwd_combine_chunk_kernel", "fwd_combine"),
    ("fwd_finish_kernel", "fwd_finish"),
    ("loss_final_kernel", "fwd_combine"),
    ("ent_combine_kernel", "entropy_combine"),
    ("prepass", "prepass"),                      # prepass_kernel, prepass_reg_kernel
    ("compact_kernel", "compact"),
    ("zero_rows_kernel", "zero_rows"),
    ("gather_rows_t", "gather_rows_t"),
    ("transpose_w", "transpose_w"),
    ("signals_kernel", "position_signals"),
    ("seg_band_final", "select_segments_final"),
    ("select_segments", "select_segments"),
    ("seg_band_", "select_segments"),
    ("fill_u8_kernel", "select_segments"),
    ("select_above", "select_above"),
    ("select_threshold", "select_threshold"),
    ("refine_kernel", "select_refine_fp64"),
    ("refine_mfma_kernel", "select_refine_fp64"),
    ("band_rows_f64", "select_refine_fp64"),
    ("sample_refined_entropy", "select_refine_fp64"),
    ("probe_list_kernel", "select_error_probe"),
    ("max_abs_diff_kernel", "select_error_probe"),
    ("select_final", "select_final"),
    ("sample_mean_kernel", "sample_means"),
    ("sample_mark_kernel", "select_refine_fp64"),
    ("sample_band_mean", "sample_final"),
    ("sample_final", "sample_final"),
    ("sample_zero_flag", "offsets_check"),
    ("sample_offsets_check", "offsets_check"),
    ("kd_teacher_pilot", "teacher_pilot"),
    ("kd_teacher_emit", "teacher_emit"),
    ("teacher_threshold_kernel", "teacher_threshold"),
    ("teacher_gather_kernel", "teacher_gather"),
    ("teacher_final", "teacher_final"),          # teacher_final_kernel, teacher_final_big_kernel
    ("teacher_wnorm", "teacher_wnorm"),
    ("kd_sample_mass", "sample_mass"),
    ("kd_sample_draw", "sample_draw"),
    ("draw_tile", "sample_draw"),
    ("draw_cumsum", "sample_assign"),
    ("draw_assign", "sample_assign"),
    ("draw_zero_flag", "uniforms_check"),
    ("draw_check", "uniforms_check"),
    ("validate_order", "validate_order"),
    ("validate_kernel", "validate"),
    ("zero_u64_kernel", "validate"),
    ("kd_cmp_logits", "cmp_logits"),
    ("cmp_kl_", "cmp_rows"),
    ("cmp_dense_grid", "cmp_rows"),
    ("cmp_loss_blocks", "cmp_loss"),
    ("cmp_grad_kernel", "cmp_grad"),
    ("scale_kernel", "scale_grads"),
    ("copyBuffer", "device_copy"),
]


def kernel_sources_hash() -> str:
    """SHA-256 over the kernel sources (file names and contents, sorted by name)."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".hip", ".hpp", ".h")):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def step_of(kernel_name: str) -> str:
    for pat, step in STEP_PATTERNS:
        if pat in kernel_name:
            return step
    return "other"


def _json_block(obj) -> str:
    return "```json\n" + json.dumps(obj, indent=1, sort_keys=True) + "\n```\n"


def read_summary_json(path: str):
    """The JSON block of a summary written by this module, or None."""
    try:
        with open(path) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"```json\n(.*?)\n```", text, re.S)
    return json.loads(m.group(1)) if m else None


# ---------------------------------------------------------------------------
# kernel trace
# ---------------------------------------------------------------------------
def summarize_trace(stats_csv: str, commands, workload: str, steps: int) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    agg = collections.OrderedDict()
    for r in rows:
        step = step_of(r["Name"])
        calls = int(r["Calls"])
        tot = float(r["TotalDurationNs"])
        a = agg.setdefault(step, dict(calls=0, total_ns=0.0, kernels=set()))
        a["calls"] += calls
        a["total_ns"] += tot
        a["kernels"].add(r["Name"] if len(r["Name"]) < 60 else r["Name"][:57] + "...")
    total = sum(a["total_ns"] for a in agg.values())
    out = [f"# Kernel trace: {workload}\n",
           "rocprofv3 `--kernel-trace --stats`, durations per path step (all launches in the run,",
           f"{steps} timed steps plus warm-up).\n",
           "Commands (from the repository root):\n"]
    out += [f"    {c}" for c in commands]
    out += ["", "| step | launches | total ms | avg ms per launch | share |",
            "|:--|--:|--:|--:|--:|"]
    data = {}
    for step, a in sorted(agg.items(), key=lambda kv: -kv[1]["total_ns"]):
        avg = a["total_ns"] / max(a["calls"], 1) / 1e6
        out.append(f"| {step} | {a['calls']} | {a['total_ns'] / 1e6:.3f} | {avg:.5f} | "
                   f"{100.0 * a['total_ns'] / max(total, 1):.1f}% |")
        data[step] = dict(launches=a["calls"], total_ms=round(a["total_ns"] / 1e6, 4),
                          avg_ms=round(avg, 6), kernels=sorted(a["kernels"]))
    out += ["", "Machine-readable copy:", "",
            _json_block(dict(kind="kernel_trace", workload=workload,
                             kernel_sources_sha256=kernel_sources_hash(), steps=data))]
    return "\n".join(out)


# ---------------------------------------------------------------------------
# HBM traffic
# ---------------------------------------------------------------------------
def _counter_rows(path, counter):
    per = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        per[step_of(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return per


def summarize_traffic(fetch_csv: str, write_csv: str, calib_mib: int, commands,
                      workload: str) -> str:
    fetch = _counter_rows(fetch_csv, "FETCH_SIZE")
    write = _counter_rows(write_csv, "WRITE_SIZE")
    calib_kib = calib_mib * 1024.0
    if not fetch.get("device_copy") or not write.get("device_copy"):
        raise SystemExit("no device copy dispatch in the counter dumps: run bench.py with "
                         "--calib-copy-mib")
    # the calibration copy is the largest copy dispatch of the run
    f_cal = max(fetch["device_copy"])
    w_cal = max(write["device_copy"])
    f_fac = calib_kib / f_cal
    w_fac = calib_kib / w_cal
    out = [f"# HBM traffic per launch: {workload}\n",
           "rocprofv3 `--pmc FETCH_SIZE` and `--pmc WRITE_SIZE` (KiB per dispatch), each in a run",
           "of its own, averaged over all launches of a step's kernels. Calibration: a",
           f"device-to-device copy of {calib_mib} MiB in the same process read FETCH_SIZE =",
           f"{f_cal:.0f} KiB and WRITE_SIZE = {w_cal:.0f} KiB, so the counters are scaled by",
           f"{f_fac:.3f} (reads) and {w_fac:.3f} (writes).\n",
           "Commands (from the repository root):\n"]
    out += [f"    {c}" for c in commands]
    out += ["", "| step | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | read GB | written GB | "
            "total GB per launch |", "|:--|--:|--:|--:|--:|--:|--:|"]
    data = {}
    for step in sorted(set(fetch) | set(write)):
        if step == "device_copy" or step not in fetch or step not in write:
            continue
        fv, wv = fetch[step], write[step]
        fk = sum(fv) / len(fv)
        wk = sum(wv) / len(wv)
        rb = fk * 1024.0 * f_fac
        wb = wk * 1024.0 * w_fac
        out.append(f"| {step} | {len(fv)} | {fk:.0f} | {wk:.0f} | {rb / 1e9:.3f} | {wb / 1e9:.3f} | "
                   f"{(rb + wb) / 1e9:.3f} |")
        data[step] = dict(launches=len(fv), fetch_kib=round(fk, 1), write_kib=round(wk, 1),
                          read_bytes=round(rb), write_bytes=round(wb),
                          traffic_bytes=round(rb + wb))
    out += ["", "Machine-readable copy:", "",
            _json_block(dict(kind="hbm_traffic", workload=workload,
                             kernel_sources_sha256=kernel_sources_hash(),
                             calibration=dict(copy_mib=calib_mib, fetch_kib=f_cal,
                                              write_kib=w_cal, fetch_factor=f_fac,
                                              write_factor=w_fac),
                             steps=data))]
    return "\n".join(out)


# ---------------------------------------------------------------------------
# hardware counters (MFMA utilisation, instruction mix, L2, texture path)
# ---------------------------------------------------------------------------
def _pmc_means(paths):
    """{step: {counter: mean per dispatch}} over one or more --pmc CSV dumps
    (each pass a run of its own); also {step: dispatches}."""
    sums = collections.defaultdict(lambda: collections.defaultdict(float))
    cnts = collections.defaultdict(lambda: collections.defaultdict(int))
    for path in paths:
        for r in csv.DictReader(open(path)):
            step = step_of(r["Kernel_Name"])
            sums[step][r["Counter_Name"]] += float(r["Counter_Value"])
            cnts[step][r["Counter_Name"]] += 1
    means = {st: {c: sums[st][c] / cnts[st][c] for c in sums[st]} for st in sums}
    disp = {st: max(cnts[st].values()) for st in cnts}
    return means, disp


def _derived(m, avg_ns=None, xcc=8, cus=256):
    """Ratios of the mean counters of one step. With the step's mean duration
    from a kernel trace: the shader clock (GRBM_GUI_ACTIVE is summed over the
    XCCs) and the TD / TA busy fraction per CU-cycle (summed over the CUs)."""
    d = {}
    g = m.get("GRBM_GUI_ACTIVE")
    if g:
        cyc = g / xcc
        if avg_ns:
            d["clock_ghz"] = cyc / avg_ns
        for c, k in (("TD_TD_BUSY_sum", "td_busy_per_cu_cycle"), ("TA_TA_BUSY_sum", "ta_busy_per_cu_cycle")):
            if c in m:
                d[k] = m[c] / (cyc * cus)
    if "MfmaUtil" in m:
        d["mfma_util_pct"] = m["MfmaUtil"]
    if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m:
        d["bf16_mfma_flop"] = m["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
    h, mi = m.get("TCC_HIT_sum"), m.get("TCC_MISS_sum")
    if h is not None and mi is not None and h + mi > 0:
        d["l2_hit_rate"] = h / (h + mi)
    if m.get("SQ_INSTS_LDS"):
        if "SQ_LDS_BANK_CONFLICT" in m:
            d["lds_bank_conflict_cycles_per_lds_inst"] = m["SQ_LDS_BANK_CONFLICT"] / m["SQ_INSTS_LDS"]
    if m.get("SQ_INSTS_MFMA"):
        for c, k in (("SQ_INSTS_VALU", "valu_inst_per_mfma_inst"), ("SQ_INSTS_LDS", "lds_inst_per_mfma_inst")):
            if c in m:
                d[k] = m[c] / m["SQ_INSTS_MFMA"]
    if m.get("TCP_TCC_READ_REQ_sum") and "TCP_TCC_READ_REQ_LATENCY_sum" in m:
        d["l2_read_latency_cycles"] = m["TCP_TCC_READ_REQ_LATENCY_sum"] / m["TCP_TCC_READ_REQ_sum"]
    return d


def summarize_counters(paths, commands, workload: str, steps_of_interest=None,
                       trace_stats=None) -> str:
    means, disp = _pmc_means(paths)
    avg_ns = {}
    if trace_stats:
        tot = collections.defaultdict(float)
        cnt = collections.defaultdict(int)
        for r in csv.DictReader(open(trace_stats)):
            st = step_of(r["Name"])
            tot[st] += float(r["TotalDurationNs"])
            cnt[st] += int(r["Calls"])
        avg_ns = {st: tot[st] / cnt[st] for st in tot if cnt[st]}
    names = sorted(means, key=lambda st: -means[st].get("GRBM_GUI_ACTIVE", 0.0) * disp[st])
    if steps_of_interest:
        names = [n for n in names if n in steps_of_interest]
    out = [f"# Hardware counters per launch: {workload}\n",
           "rocprofv3 `--pmc`, one pass per counter set (each a run of its own), mean per",
           "dispatch of each path step. `MfmaUtil` is rocprofv3's derived metric:",
           "SQ_VALU_MFMA_BUSY_CYCLES summed over SIMDs / (GRBM_GUI_ACTIVE x SIMDs), in percent.",
           "bf16 MFMA flop = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512. L2 hit rate = TCC_HIT /",
           "(TCC_HIT + TCC_MISS). L2 read latency = TCP_TCC_READ_REQ_LATENCY / TCP_TCC_READ_REQ",
           "(cycles per request, as seen from the vector L1). Clock = GRBM_GUI_ACTIVE / 8 XCCs",
           "over the step's mean duration in the kernel trace of the same sources; TD and TA",
           "busy = TD_TD_BUSY / TA_TA_BUSY summed over the CUs, per CU-cycle (256 CUs).\n",
           "Commands (from the repository root):\n"]
    out += [f"    {c}" for c in commands]
    out += ["", "| step | launches | MfmaUtil % | clock GHz | bf16 MFMA TFLOP per launch | "
            "VALU / MFMA inst | LDS / MFMA inst | LDS bank-conflict cycles / LDS inst | L2 hit | "
            "L2 read latency | TD busy | TA busy |",
            "|:--|--:|--:|--:|--:|--:|--:|--:|--:|--:|--:|--:|"]

    def f(x, fmt):
        return "" if x is None else format(x, fmt)

    data = {}
    for st in names:
        d = _derived(means[st], avg_ns.get(st))
        out.append(f"| {st} | {disp[st]} | {f(d.get('mfma_util_pct'), '.1f')} | "
                   f"{f(d.get('clock_ghz'), '.2f')} | "
                   f"{f(d.get('bf16_mfma_flop', 0) / 1e12 if 'bf16_mfma_flop' in d else None, '.3f')} | "
                   f"{f(d.get('valu_inst_per_mfma_inst'), '.3f')} | "
                   f"{f(d.get('lds_inst_per_mfma_inst'), '.3f')} | "
                   f"{f(d.get('lds_bank_conflict_cycles_per_lds_inst'), '.3f')} | "
                   f"{f(d.get('l2_hit_rate'), '.3f')} | {f(d.get('l2_read_latency_cycles'), '.0f')} | "
                   f"{f(d.get('td_busy_per_cu_cycle'), '.2f')} | {f(d.get('ta_busy_per_cu_cycle'), '.2f')} |")
        data[st] = dict(launches=disp[st], derived={k: round(v, 6) for k, v in d.items()},
                        counters={k: round(v, 3) for k, v in sorted(means[st].items())})
    out += ["", "Machine-readable copy (mean counter values per dispatch):", "",
            _json_block(dict(kind="hw_counters", workload=workload,
                             kernel_sources_sha256=kernel_sources_hash(), steps=data))]
    return "\n".join(out)


def main(argv=None):
    ap = argparse.ArgumentParser(description="summaries of rocprofv3 output")
    sub = ap.add_subparsers(dest="what", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--stats", required=True)
    t.add_argument("--steps", type=int, default=0)
    c = sub.add_parser("counters")
    c.add_argument("--pmc", action="append", required=True, help="a --pmc CSV dump (repeatable)")
    c.add_argument("--steps-of-interest", default="")
    c.add_argument("--trace-stats", default=None,
                   help="kernel-trace stats CSV of the same sources (for the clock)")
    m = sub.add_parser("traffic")
    m.add_argument("--fetch", required=True)
    m.add_argument("--write", required=True)
    m.add_argument("--calib-mib", type=int, required=True)
    for p in (t, m, c):
        p.add_argument("--out", required=True)
        p.add_argument("--workload", required=True)
        p.add_argument("--command", action="append", default=[])
    a = ap.parse_args(argv)
    if a.what == "trace":
        text = summarize_trace(a.stats, a.command, a.workload, a.steps)
    elif a.what == "counters":
        soi = [x for x in a.steps_of_interest.split(",") if x]
        text = summarize_counters(a.pmc, a.command, a.workload, soi or None, a.trace_stats)
    else:
        text = summarize_traffic(a.fetch, a.write, a.calib_mib, a.command, a.workload)
    with open(a.out, "w") as f:
        f.write(text)
    print(f"wrote {a.out}")


if __name__ == "__main__":
    main()
