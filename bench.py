#!/usr/bin/env python3
"""Benchmark of the fused chunked top-K KL loss (forward + backward) on one MI355X.

One step = the whole hot path over one batch: teacher prepass, fused projection
with online log-sum-exp and id gather, combine and loss, then per chunk the
recomputed gradient tile, dHidden and dW contractions.

Default workload (the 32K-context, large-vocabulary configuration):
  S=32768, H=2880, V=201088, K=100, T=1.0, chunk=2048, bf16 hidden/W, bf16
  teacher logits, int32 ids; synthetic inputs from kd_synth (seed 1003).

Prints ONE JSON line. Besides tokens/s it reports the achieved MFMA fraction
(counting 4 contractions of 2*S*H*V FLOP per step), per-kernel HIP-event
timings over the timed region, the roofline of the dominant kernel, peak
device memory against S for the 256K-context configuration shapes, and the
fp64 CPU oracle timed on a bounded sample of rows. Beside the step it times
the forward and backward in one call (kd_topk_kl_fwd_bwd: each chunk's logits
kept, no second projection; the `one_call` objects), the loss's comparator
forms, the chunk sizes, the teacher cache writer and the selection policies.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0

WORKLOADS = {
    "c2": dict(S=8192, H=3072, V=128256, K=100, T=1.0, chunk=1024, seed=1002, slug="8k_context",
               name="8K context: S=8192 H=3072 V=128256 K=100 T=1.0 chunk=1024 bf16"),
    "c3": dict(S=32768, H=2880, V=201088, K=100, T=1.0, chunk=2048, seed=1003, slug="32k_context",
               name="32K context, large vocab: S=32768 H=2880 V=201088 K=100 T=1.0 chunk=2048 bf16"),
    "c4": dict(S=262144, H=3072, V=128256, K=100, T=2.0, chunk=2048, seed=1004, slug="256k_context",
               name="256K context: S=262144 H=3072 V=128256 K=100 T=2.0 chunk=2048 bf16"),
    "c5": dict(S=32768, H=2048, V=151936, K=100, T=1.0, chunk=1024, seed=1005,
               slug="entropy_selective_32k",
               name="entropy-selective: S=32768 H=2048 V=151936 K=100 top 20% by entropy, chunk=1024 bf16"),
}

METRIC = "fwd+bwd tokens/s at S=32K,V=201088 + MFMA % of peak + peak GiB vs S"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev(p, torch):
    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    return bf(p.hidden_bits), bf(p.W_bits), torch.from_numpy(p.ids).cuda(), bf(p.tl_bits)


def kernel_flops(name, wl, C_rows, S_rows):
    """Algorithmic FLOPs of one launch of a projection kernel."""
    H, V = wl["H"], wl["V"]
    if name in ("fwd_lse_gather", "entropy_sweep"):
        return 2.0 * S_rows * H * V
    if name in ("bwd_grad_tile", "bwd_dhidden", "bwd_dw", "fwd_lse_gather_keep"):
        return 2.0 * C_rows * H * V
    return None


def teacher_profile_name(wl):
    """The workload name the teacher cache writer's counter summaries carry."""
    return (f"teacher top-K cache writer at the 32K context shapes: S={wl['S']} H={wl['H']} "
            f"V={wl['V']} K={wl['K']} chunk={wl['chunk']} bf16")


def measured_traffic(wl, step, slug=None, name=None):
    """HBM bytes per launch of `step` from the committed counter summary of this
    workload (named `name`, else the workload's own name), or None when there
    is none or the kernel sources changed since."""
    from chunked_top_kl_amd.prof_summary import kernel_sources_hash, read_summary_json
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{slug or wl['slug']}.md")
    js = read_summary_json(path)
    if not js or js.get("workload") != (name or wl["name"]):
        return None
    if js.get("kernel_sources_sha256") != kernel_sources_hash():
        log(f"[bench] {os.path.relpath(path, ROOT)} was measured on other kernel sources: traffic null")
        return None
    st = js.get("steps", {}).get(step)
    if not st:
        return None
    return dict(bytes=st["traffic_bytes"], read_bytes=st["read_bytes"],
                write_bytes=st["write_bytes"], source=os.path.relpath(path, ROOT))


def run_step(kd, torch, wl, t, ws, mask=None):
    hidden, W, ids, tl = t
    out = kd.kd_topk_kl_fwd(hidden, W, ids, tl, wl["T"], wl["chunk"], mask, workspace=ws)
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    dh, dW = kd.kd_topk_kl_bwd(hidden, W, ids, tl, out["lse"], g, wl["T"], wl["chunk"], mask,
                               workspace=ws)
    return out, dh, dW


def run_c5_step(kd, torch, wl, t, ws):
    hidden, W, ids, tl = t
    ent = kd.kd_student_entropy(hidden, W, workspace=ws)
    mask, idx, cnt = kd.kd_select_top_fraction(ent, hidden, W, 20, 100, workspace=ws)
    return run_step(kd, torch, wl, t, ws, mask=mask), cnt


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(p, wl, rows):
    """fp64 oracle forward+backward on the first `rows` positions of the same workload.
    `cores` is the number of BLAS threads the oracle's products ran on; the
    host's logical CPU count is given beside it."""
    from oracle import oracle_loss_grads
    threads = blas_threads()
    t0 = time.perf_counter()
    oracle_loss_grads(p.hidden[:rows], p.W, p.ids[:rows], p.tlogits[:rows], T=wl["T"], chunk=128)
    dt = time.perf_counter() - t0
    return dict(value=rows / dt, unit="tokens/s", cores=int(threads), kind="oracle",
                host_cpu_count=os.cpu_count(), blas_threads=int(threads),
                sample=f"first {rows} positions of the workload (full H and V): fp64 loss, "
                       f"dHidden and the dW contribution of those rows, row blocks of 128; {dt:.1f} s")


def kernel_table(prof, wl, C, N_rows, steps):
    """Per-step launches, time and achieved TFLOP/s of each profiled step."""
    S, H, V = wl["S"], wl["H"], wl["V"]
    kernels = {}
    for name, (n, tot) in prof.items():
        per = tot / max(n, 1)
        f = kernel_flops(name, wl, C, N_rows if name == "fwd_lse_gather" else S)
        if name in ("bwd_grad_tile", "bwd_dhidden", "bwd_dw"):
            f = 8.0 * N_rows * H * V / 4.0 / max(n / steps, 1)   # per launch, averaged over chunks
        kernels[name] = dict(launches_per_step=round(n / steps, 2), ms_per_step=round(tot / steps, 4),
                             avg_ms=round(per, 5),
                             tflops=(round(f / (per / 1000.0) / 1e12, 1) if f else None))
    if "prepass" in kernels:
        # teacher prepass: ids (4 B) and logits read, (id, p, k) (12 B) per entry and
        # 5 B per row written; an HBM-bound step, reported against 8 TB/s
        tl_b = 2 if wl.get("tl_dtype", "bf16") == "bf16" else 4
        pb = S * wl["K"] * (4 + tl_b) + S * wl["K"] * 12 + 5 * S
        gbs = pb / (kernels["prepass"]["avg_ms"] / 1000.0) / 1e9
        kernels["prepass"].update(bytes=pb, gb_per_s=round(gbs, 1), hbm_frac=round(gbs / 8000.0, 4))
    return kernels


def time_workload(kd, torch, key, p=None, steps=3, warmup=1, comparators=False):
    """fwd+bwd of another configuration at its full size (the entropy-selective
    one with its entropy sweep and selection): ms per step, tokens/s, the MFMA
    fraction of the counted work, peak device memory and the per-step kernels."""
    from kd_synth import make_problem
    wl = dict(WORKLOADS[key])
    S, H, V, K, C = wl["S"], wl["H"], wl["V"], wl["K"], wl["chunk"]
    if p is None:
        log(f"[bench] generating inputs: {wl['name']}")
        p = make_problem(S, H, V, K, T=wl["T"], chunk=C, seed=wl["seed"])
    t = to_dev(p, torch)
    prob = kd.make_problem(S, H, V, K, C, wl["T"], kd.KD_BF16, kd.KD_BF16)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated() - sum(x.numel() * x.element_size() for x in t)
    ws = torch.empty(kd.kd_topk_kl_workspace_bytes(prob), dtype=torch.uint8, device="cuda")
    step = (lambda: run_c5_step(kd, torch, wl, t, ws)) if key == "c5" else \
        (lambda: run_step(kd, torch, wl, t, ws))
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    kd.kd_profile_reset()
    kd.kd_profile_enable(True)
    t0 = time.perf_counter()
    res = None
    for _ in range(steps):
        res = None          # the previous step's outputs are freed before the next step
        res = step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / steps
    kd.kd_profile_enable(False)
    prof = kd.kd_profile_read()
    kd.kd_profile_reset()
    peak = (torch.cuda.max_memory_allocated() - base) / 2**30
    N_rows = int(res[1]) if key == "c5" else S
    flops = 2.0 * S * H * V + 8.0 * N_rows * H * V if key == "c5" else 8.0 * S * H * V
    loss = float(res[0][0]["loss"][0]) if key == "c5" else float(res[0]["loss"][0])
    out = dict(workload=wl["name"], steps=steps, warmup=warmup, ms_per_step=round(ms, 3),
               tokens_per_s=round(S / (ms / 1000.0), 1),
               mfma_frac=round(flops / (ms / 1000.0) / (PEAK_BF16_TFLOPS * 1e12), 4),
               counted_tflop_per_step=round(flops / 1e12, 3), rows_in_loss=N_rows,
               peak_gib=round(peak, 3), loss=loss,
               kernels=kernel_table(prof, wl, C, N_rows, steps))
    log(f"[bench] {key}: {ms:.2f} ms/step, {out['tokens_per_s']:.0f} tokens/s, "
        f"MFMA {100 * out['mfma_frac']:.1f}%, peak {out['peak_gib']} GiB")
    del ws, res
    out["one_call"] = one_call_leg(kd, torch, wl, t, steps=steps, warmup=warmup,
                                   two_call_ms=ms, select=(key == "c5"))
    if comparators:
        out["comparators"] = comparator_leg(kd, torch, wl, t)
    del t
    torch.cuda.empty_cache()
    return out


def comparator_leg(kd, torch, wl, t, steps=3, warmup=1):
    """The dense and forward-chunked loss forms ("what chunked KL loss does")
    at the workload's shapes: fwd+bwd ms per step, tokens/s and peak device
    memory (inputs, outputs, the workspace with its stored grids), beside the
    fused form's numbers from the main timing. Same counted FLOP: the
    comparators project once (no recompute), so their MFMA work is
    6*S*H*V, while 8*S*H*V is what the fused form runs."""
    S, H, V, K, C = wl["S"], wl["H"], wl["V"], wl["K"], wl["chunk"]
    hidden, W, ids, tl = t
    in_bytes = sum(x.numel() * x.element_size() for x in t)
    out = {}
    for name, form in (("forward_chunked", kd.KD_FORM_FORWARD_CHUNKED), ("dense", kd.KD_FORM_DENSE)):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        prob = kd.make_problem(S, H, V, K, C, wl["T"], kd.KD_BF16, kd.KD_BF16)
        need = kd.lib.kd_kl_comparator_workspace_bytes(ctypes.byref(prob), form)
        free, _ = torch.cuda.mem_get_info()
        if need + (4 << 30) > free:
            out[name] = dict(skipped=f"workspace {need / 2**30:.1f} GiB does not fit")
            continue
        base = torch.cuda.memory_allocated() - in_bytes
        torch.cuda.reset_peak_memory_stats()
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        g = torch.ones(1, dtype=torch.float32, device="cuda")

        def step():
            o = kd.kd_kl_comparator_fwd(hidden, W, ids, tl, form, wl["T"], C, workspace=ws)
            dh, dW = kd.kd_kl_comparator_bwd(hidden, W, ids, tl, o["lse"], g, form, ws, wl["T"], C)
            return o, dh, dW

        for _ in range(warmup):
            res = step()
            del res
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        res = None
        for _ in range(steps):
            res = None
            res = step()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1000.0 / steps
        peak = (torch.cuda.max_memory_allocated() - base) / 2**30
        out[name] = dict(ms_per_step=round(ms, 3), tokens_per_s=round(S / (ms / 1000.0), 1),
                         peak_gib=round(peak, 3), workspace_gib=round(need / 2**30, 3),
                         loss=float(res[0]["loss"][0]),
                         mfma_frac_of_its_6SHV=round(6.0 * S * H * V / (ms / 1000.0)
                                                     / (PEAK_BF16_TFLOPS * 1e12), 4))
        log(f"[bench] {name} form: {ms:.2f} ms/step, peak {peak:.2f} GiB")
        del ws, res
    torch.cuda.empty_cache()
    return out


def one_call_leg(kd, torch, wl, t, steps=5, warmup=2, two_call_ms=None, select=False):
    """The forward and backward in one call (kd_topk_kl_fwd_bwd: each chunk's
    logits kept, its gradient tile formed from them, no second projection) at
    the workload's shapes: ms per step, tokens/s, peak device memory (inputs,
    outputs, workspace), the per-step kernels, and the MFMA fraction of the
    6*S*H*V it projects (the counted 8*S*H*V over its time as well, for
    comparison with the two calls). select: the entropy-selective step (entropy
    sweep, top-20% selection, then the one call on the kept rows; the MFMA
    fractions then count the rows in the loss)."""
    S, H, V, K, C = wl["S"], wl["H"], wl["V"], wl["K"], wl["chunk"]
    hidden, W, ids, tl = t
    in_bytes = sum(x.numel() * x.element_size() for x in t)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated() - in_bytes
    torch.cuda.reset_peak_memory_stats()
    need = kd.kd_topk_kl_fwd_bwd_workspace_bytes(hidden, W, ids, tl, wl["T"], C)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    g = torch.ones(1, dtype=torch.float32, device="cuda")

    def step():
        if not select:
            return kd.kd_topk_kl_fwd_bwd(hidden, W, ids, tl, g, wl["T"], C, workspace=ws)
        # entropy-selective: the entropy sweep and the selection first (the
        # one-call workspace holds theirs), then the one call on the kept rows
        ent = kd.kd_student_entropy(hidden, W, workspace=ws)
        mask, _, _ = kd.kd_select_top_fraction(ent, hidden, W, 20, 100, workspace=ws)
        return kd.kd_topk_kl_fwd_bwd(hidden, W, ids, tl, g, wl["T"], C, mask, workspace=ws)

    for _ in range(warmup):
        res = step()
        del res
    torch.cuda.synchronize()
    kd.kd_profile_reset()
    kd.kd_profile_enable(True)
    t0 = time.perf_counter()
    res = None
    for _ in range(steps):
        res = None
        res = step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1000.0 / steps
    kd.kd_profile_enable(False)
    prof = kd.kd_profile_read()
    kd.kd_profile_reset()
    peak = (torch.cuda.max_memory_allocated() - base) / 2**30
    N = (20 * S) // 100 if select else S
    pre = 2.0 * S * H * V if select else 0.0     # the entropy sweep
    out = dict(ms_per_step=round(ms, 3), tokens_per_s=round(S / (ms / 1000.0), 1),
               peak_gib=round(peak, 3), workspace_gib=round(need / 2**30, 3),
               loss=float(res["loss"][0]),
               mfma_frac_of_its_6SHV=round((pre + 6.0 * N * H * V) / (ms / 1000.0)
                                           / (PEAK_BF16_TFLOPS * 1e12), 4),
               counted_8SHV_frac=round((pre + 8.0 * N * H * V) / (ms / 1000.0)
                                       / (PEAK_BF16_TFLOPS * 1e12), 4),
               kernels=kernel_table(prof, wl, C, N, steps))
    if two_call_ms:
        out["speedup_vs_two_calls"] = round(two_call_ms / ms, 3)
    gp = out["kernels"].get("grad_tile_from_logits")
    if gp and not select:
        # the gradient tile from the kept logits: HBM-bound, 4 bytes of logit
        # read and 2 bytes of gradient written per (row, vocabulary entry) of a
        # chunk (the padding to whole tiles and 8 columns left out)
        b = (4.0 + 2.0) * min(C, S) * V
        gbs = b / (gp["avg_ms"] / 1000.0) / 1e9
        tr = measured_traffic(wl, "grad_tile_from_logits")
        out["roofline_grad_tile_from_logits"] = dict(
            bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
            frac=round(gbs / PEAK_HBM_GBS, 4), bytes_per_launch=b,
            traffic=tr["bytes"] if tr else None, avg_ms=gp["avg_ms"])
    log(f"[bench] one call: {ms:.2f} ms/step, {out['tokens_per_s']:.0f} tokens/s, "
        f"peak {peak:.2f} GiB")
    del ws, res
    torch.cuda.empty_cache()
    return out


def chunk_sweep(kd, torch, wl, t, chunks, steps=3, warmup=1):
    """fwd+bwd time and peak device memory of the workload at several chunk sizes."""
    S, H, V, K = wl["S"], wl["H"], wl["V"], wl["K"]
    hidden, W, ids, tl = t
    out = {}
    for C in chunks:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        prob = kd.make_problem(S, H, V, K, C, wl["T"], kd.KD_BF16, kd.KD_BF16)
        ws = torch.empty(kd.kd_topk_kl_workspace_bytes(prob), dtype=torch.uint8, device="cuda")
        wlc = dict(wl, chunk=C)
        for _ in range(warmup):
            run_step(kd, torch, wlc, t, ws)
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        t0 = time.perf_counter()
        for _ in range(steps):
            run_step(kd, torch, wlc, t, ws)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1000.0 / steps
        out[str(C)] = dict(ms_per_step=round(ms, 3), tokens_per_s=round(S / (ms / 1000.0), 1),
                           peak_gib=round(torch.cuda.max_memory_allocated() / 2**30, 3),
                           workspace_gib=round(ws.numel() / 2**30, 3))
        log(f"[bench] chunk {C}: {ms:.2f} ms/step, peak {out[str(C)]['peak_gib']} GiB")
        del ws
    return out


def teacher_leg(kd, torch, wl, t, p, steps=3, warmup=1, cpu_rows=64, cpu=True):
    """Teacher top-K cache writer at the workload's shapes: the workload's
    hidden rows and W stand in for the teacher's. Counted work: 2*S*H*V FLOP,
    the emit pass over the whole vocabulary (the pilot pass over its first
    16384 rows is extra work and not counted)."""
    S, H, V, K, C = wl["S"], wl["H"], wl["V"], wl["K"], wl["chunk"]
    hidden, W = t[0], t[1]
    prob = kd.make_problem(S, H, V, K, C, 1.0, kd.KD_BF16, kd.KD_BF16)
    ws = torch.empty(kd.kd_teacher_topk_workspace_bytes(prob), dtype=torch.uint8, device="cuda")
    for _ in range(warmup):
        kd.kd_teacher_topk(hidden, W, K, chunk=C, workspace=ws)
    torch.cuda.synchronize()
    kd.kd_profile_reset()
    kd.kd_profile_enable(True)
    t0 = time.perf_counter()
    for _ in range(steps):
        ids, logits = kd.kd_teacher_topk(hidden, W, K, chunk=C, workspace=ws)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    kd.kd_profile_enable(False)
    prof = kd.kd_profile_read()
    kd.kd_profile_reset()
    ms = dt * 1000.0 / steps
    P = min(V, 16384)
    kernels = {}
    for name, (n, tot) in prof.items():
        per = tot / max(n, 1)
        f = None
        if name == "teacher_pilot":
            f = 2.0 * S * H * P / (n / steps)
        elif name == "teacher_emit":
            f = 2.0 * S * H * V / (n / steps)
        kernels[name] = dict(launches_per_step=round(n / steps, 2), ms_per_step=round(tot / steps, 4),
                             avg_ms=round(per, 5),
                             tflops=(round(f / (per / 1000.0) / 1e12, 1) if f else None))
    em = kernels.get("teacher_emit")
    roofline = None
    if em:
        f = 2.0 * S * H * V / em["launches_per_step"]
        a = f / (em["avg_ms"] / 1000.0) / 1e12
        tr = measured_traffic(wl, "teacher_emit", slug="teacher_topk_" + wl["slug"],
                              name=teacher_profile_name(wl))
        roofline = dict(kernel="teacher_emit", bound="mfma", achieved=round(a, 1),
                        peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", frac=round(a / PEAK_BF16_TFLOPS, 4),
                        traffic=tr["bytes"] if tr else None, traffic_detail=tr,
                        flops_per_launch=f, avg_ms=em["avg_ms"])
    out = dict(workload=f"teacher cache writer at {wl['name']} (synthetic teacher = the workload's hidden and W)",
               ms=round(ms, 3), tokens_per_s=round(S / (ms / 1000.0), 1),
               mfma_frac=round(2.0 * S * H * V / (ms / 1000.0) / (PEAK_BF16_TFLOPS * 1e12), 4),
               workspace_gib=round(ws.numel() / 2**30, 3), roofline=roofline, kernels=kernels)
    log(f"[bench] teacher cache writer: {ms:.2f} ms, {out['tokens_per_s']:.0f} tokens/s")
    del ws, ids, logits
    torch.cuda.empty_cache()
    if cpu:
        from oracle import oracle_teacher_topk
        t0 = time.perf_counter()
        oracle_teacher_topk(p.hidden[:cpu_rows], p.W, K, out_dtype="bf16")
        d = time.perf_counter() - t0
        out["cpu_baseline"] = dict(value=cpu_rows / d, unit="tokens/s", cores=blas_threads(),
                                   kind="oracle", host_cpu_count=os.cpu_count(),
                                   sample=f"first {cpu_rows} positions (full H and V): fp64 logits and "
                                          f"the sorted top-{K}; {d:.1f} s")
    return out


def selection_leg(kd, torch, wl, t, steps=3, warmup=1, n_seq=32, seed=77):
    """Position signals and selection policies at the workload's shapes: all S
    positions as n_seq sequences of equal length, labels drawn uniformly. Times
    kd_position_signals (one entropy sweep at T = 1, counted as 2*S*H*V FLOP,
    plus the label dot products and teacher rows), per-sequence SE-KD
    selection (20%), per-sequence top 20% by cross-entropy, sample selection
    by mean entropy (20%), a global threshold, and sampled teacher targets
    (K ids per position drawn from softmax(z/T) of the same projection: two
    vocabulary sweeps, counted as 2*2*S*H*V FLOP)."""
    S, H, V = wl["S"], wl["H"], wl["V"]
    hidden, W, ids, tl = t
    rng = np.random.default_rng(seed)
    labels = torch.from_numpy(rng.integers(0, V, size=S).astype(np.int32)).cuda()
    off = torch.from_numpy((np.arange(n_seq + 1, dtype=np.int64) * S) // n_seq).cuda()
    prob = kd.make_problem(S, H, V, wl["K"], wl["chunk"], wl["T"], kd.KD_BF16, kd.KD_BF16)
    ws = torch.empty(kd.kd_topk_kl_workspace_bytes(prob), dtype=torch.uint8, device="cuda")

    def timed(fn):
        for _ in range(warmup):
            r = fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            r = fn()
        torch.cuda.synchronize()
        return r, (time.perf_counter() - t0) * 1000.0 / steps

    kd.kd_profile_reset()
    kd.kd_profile_enable(True)
    sig, t_sig = timed(lambda: kd.kd_position_signals(hidden, W, ids, tl, labels, T=wl["T"],
                                                      workspace=ws))
    ent, ce = sig["entropy"], sig["ce"]
    (_, _, k_seq), t_seq = timed(lambda: kd.kd_select_top_fraction_segments(
        ent, off, hidden, W, 20, 100, workspace=ws))
    (_, _, k_ce, thr), t_ce = timed(lambda: kd.kd_select_by_signal(ce, off, 20, 100, workspace=ws))
    (_, _, k_smp), t_smp = timed(lambda: kd.kd_select_samples(ent, off, hidden, W, 20, 100,
                                                              workspace=ws))
    tau = float(torch.quantile(ce[: min(S, 1 << 20)].float(), 0.8))
    (_, _, k_thr), t_thr = timed(lambda: kd.kd_select_above(ce, tau, workspace=ws))
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    u = torch.sort(torch.rand(S, wl["K"], dtype=torch.float64, device="cuda", generator=gen),
                   dim=1).values.contiguous()
    sprob = kd.make_problem(S, H, V, wl["K"], wl["chunk"], wl["T"], kd.KD_BF16, kd.KD_F32)
    sws = torch.empty(kd.kd_teacher_sample_workspace_bytes(sprob), dtype=torch.uint8, device="cuda")
    sids, t_tsm = timed(lambda: kd.kd_teacher_sample(hidden, W, u, T=wl["T"], chunk=wl["chunk"],
                                                     workspace=sws))
    kd.kd_profile_enable(False)
    prof = kd.kd_profile_read()
    kd.kd_profile_reset()
    calls = steps + warmup
    kernels = {name: dict(launches_per_call=round(n / calls, 2), avg_ms=round(tot / max(n, 1), 5))
               for name, (n, tot) in prof.items()}
    es = kernels.get("entropy_sweep")
    sweep_tf = None
    if es:
        sweep_tf = round(2.0 * S * H * V / (es["avg_ms"] / 1000.0) / 1e12, 1)
    out = dict(workload=f"{wl['name']}; {n_seq} sequences of {S // n_seq} positions",
               signals_ms=round(t_sig, 3), entropy_sweep_tflops=sweep_tf,
               entropy_sweep_roofline_frac=(round(sweep_tf / PEAK_BF16_TFLOPS, 4) if sweep_tf else None),
               per_sequence_sekd_ms=round(t_seq, 3), per_sequence_sekd_kept=int(k_seq),
               per_sequence_ce_ms=round(t_ce, 3), per_sequence_ce_kept=int(k_ce),
               sample_select_ms=round(t_smp, 3), samples_kept=int(k_smp),
               threshold_ms=round(t_thr, 3), threshold_kept=int(k_thr),
               teacher_sample_ms=round(t_tsm, 3),
               # one projection sweep counted (the mass sweep); the draw pass
               # recomputes only the drawn-in tiles and is not counted
               teacher_sample_tflops=round(2.0 * S * H * V / (t_tsm / 1000.0) / 1e12, 1),
               teacher_sample_ids_in_range=bool(int(sids.min()) >= 0 and int(sids.max()) < V),
               kernels=kernels)
    log(f"[bench] selection leg: signals {t_sig:.2f} ms, per-sequence SE-KD {t_seq:.2f} ms, "
        f"sampled targets {t_tsm:.2f} ms")
    del ws, sws, u, sids
    torch.cuda.empty_cache()
    return out


def mem_sweep(kd, torch, sizes, p):
    """Peak device memory of one fwd+bwd at the 256K-context shapes for several S
    (the first S rows of the 256K-context inputs `p`)."""
    H, V, K, T, C = 3072, 128256, 100, 2.0, 2048
    assert (p.H, p.V, p.K) == (H, V, K) and p.S >= max(sizes)
    out = {}
    for S in sorted(sizes):
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        torch.cuda.reset_peak_memory_stats()
        base = torch.cuda.memory_allocated()
        hidden = torch.from_numpy(p.hidden_bits[:S].view(np.int16)).view(torch.bfloat16).cuda()
        W = torch.from_numpy(p.W_bits.view(np.int16)).view(torch.bfloat16).cuda()
        ids = torch.from_numpy(p.ids[:S]).cuda()
        tl = torch.from_numpy(p.tl_bits[:S].view(np.int16)).view(torch.bfloat16).cuda()
        fo = kd.kd_topk_kl_fwd(hidden, W, ids, tl, T, C)
        g = torch.ones(1, dtype=torch.float32, device="cuda")
        dh, dW = kd.kd_topk_kl_bwd(hidden, W, ids, tl, fo["lse"], g, T, C)
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        out[S] = peak / 2**30
        log(f"[bench] mem S={S}: peak {out[S]:.3f} GiB (loss {float(fo['loss'][0]):.4f})")
        del hidden, W, ids, tl, fo, dh, dW, g
    xs = np.array(sorted(out), dtype=np.float64)
    ys = np.array([out[s] for s in sorted(out)])
    A = np.stack([np.ones_like(xs), xs], axis=1)
    coef, *_ = np.linalg.lstsq(A, ys, rcond=None)
    pred = A @ coef
    r2 = 1.0 - float(np.sum((ys - pred) ** 2)) / max(float(np.sum((ys - ys.mean()) ** 2)), 1e-30)
    return dict(shapes="H=3072 V=128256 K=100 T=2 chunk=2048 bf16",
                peak_gib={str(int(k)): round(v, 4) for k, v in out.items()},
                fit_intercept_gib=round(float(coef[0]), 4),
                fit_kib_per_token=round(float(coef[1]) * 2**20, 3), r2=round(r2, 6))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="c3", choices=sorted(WORKLOADS))
    ap.add_argument("--chunk", type=int, default=None)
    ap.add_argument("--cpu-rows", type=int, default=2048)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-mem-sweep", action="store_true")
    ap.add_argument("--mem-sizes", default="16384,32768,65536,131072,262144")
    ap.add_argument("--no-chunk-sweep", action="store_true",
                    help="skip the fwd+bwd timing and peak memory at chunks 512/1024/2048")
    ap.add_argument("--no-teacher", action="store_true",
                    help="skip the teacher top-K cache writer leg")
    ap.add_argument("--no-selection", action="store_true",
                    help="skip the position-signal and selection-policy leg")
    ap.add_argument("--teacher-only", action="store_true",
                    help="time only the teacher top-K cache writer (steps / warmup calls) and "
                         "print its line")
    ap.add_argument("--no-one-call", action="store_true",
                    help="skip the forward and backward in one call (kd_topk_kl_fwd_bwd)")
    ap.add_argument("--no-comparators", action="store_true",
                    help="skip the dense and forward-chunked loss forms (8K and 32K contexts)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the timed fwd+bwd of the other configurations (8K, 256K, "
                         "entropy-selective) at full size")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a device copy of this many MiB (HBM counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the loss shards by positions; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import chunked_top_kl_amd as kd
    from kd_synth import make_problem

    wl = dict(WORKLOADS[args.workload])
    if args.chunk:
        wl["chunk"] = args.chunk
        wl["name"] = wl["name"].replace(f"chunk={WORKLOADS[args.workload]['chunk']}",
                                        f"chunk={args.chunk}")
    S, H, V, K, C = wl["S"], wl["H"], wl["V"], wl["K"], wl["chunk"]
    log(f"[bench] generating inputs: {wl['name']}")
    t0 = time.perf_counter()
    p = make_problem(S, H, V, K, T=wl["T"], chunk=C, seed=wl["seed"])
    log(f"[bench] inputs ready in {time.perf_counter() - t0:.1f} s; uploading")
    t = to_dev(p, torch)
    prob = kd.make_problem(S, H, V, K, C, wl["T"], kd.KD_BF16, kd.KD_BF16)
    ws = torch.empty(kd.kd_topk_kl_workspace_bytes(prob), dtype=torch.uint8, device="cuda")

    if args.calib_copy_mib:
        n = args.calib_copy_mib * 2**20 // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy of {args.calib_copy_mib} MiB done")
        del a, b

    if args.teacher_only:
        del ws
        torch.cuda.empty_cache()
        r = teacher_leg(kd, torch, wl, t, p, steps=args.steps, warmup=args.warmup,
                        cpu=not args.no_cpu_baseline)
        r.update(metric="teacher top-K cache writer tokens/s", value=r["tokens_per_s"],
                 unit="tokens/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
                 higher_is_better=True, dtype="bf16", data="synthetic")
        print(json.dumps(r), flush=True)
        return
    step = (lambda: run_c5_step(kd, torch, wl, t, ws)) if args.workload == "c5" else \
        (lambda: run_step(kd, torch, wl, t, ws))
    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"[bench] warmup {i + 1}/{args.warmup} done")

    torch.cuda.reset_peak_memory_stats()
    kd.kd_profile_reset()
    kd.kd_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res = None
    for _ in range(args.steps):
        res = None          # the previous step's outputs are freed before the next step
        res = step()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    kd.kd_profile_enable(False)
    prof = kd.kd_profile_read()
    kd.kd_profile_reset()
    peak_gib = torch.cuda.max_memory_allocated() / 2**30
    ms = dt * 1000.0 / args.steps
    log(f"[bench] {args.steps} steps in {dt:.3f} s: {ms:.2f} ms/step")

    N_rows = S
    if args.workload == "c5":
        N_rows = int(res[1])
    # counted MFMA work of one step
    if args.workload == "c5":
        flops = 2.0 * S * H * V + 8.0 * N_rows * H * V
    else:
        flops = 8.0 * S * H * V
    mfma_frac = flops / (ms / 1000.0) / (PEAK_BF16_TFLOPS * 1e12)

    kernels = kernel_table(prof, wl, C, N_rows, args.steps)
    dom = max(kernels.items(), key=lambda kv: kv[1]["ms_per_step"])
    dom_name, dom_v = dom
    # the forward runs over the rows in the loss, the entropy sweep over all S
    dom_flops = kernel_flops(dom_name, wl, C, S if dom_name == "entropy_sweep" else N_rows)
    if dom_name in ("bwd_grad_tile", "bwd_dhidden", "bwd_dw"):
        dom_flops = 8.0 * N_rows * H * V / 4.0 / max(dom_v["launches_per_step"], 1)
    achieved = dom_flops / (dom_v["avg_ms"] / 1000.0) / 1e12 if dom_flops else None
    tr = measured_traffic(wl, dom_name)
    roofline = dict(kernel=dom_name, bound="mfma", achieved=round(achieved, 1) if achieved else None,
                    peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved / PEAK_BF16_TFLOPS, 4) if achieved else None,
                    traffic=tr["bytes"] if tr else None,
                    traffic_unit="bytes per launch past L2 (calibrated FETCH_SIZE + WRITE_SIZE: "
                                 "L2 misses, served by the MALL or by HBM)",
                    traffic_detail=tr,
                    flops_per_launch=dom_flops, avg_ms=dom_v["avg_ms"])

    result = {
        "metric": METRIC,
        "value": round(S / (ms / 1000.0), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl["name"], "S": S, "H": H, "V": V, "K": K, "T": wl["T"],
                   "chunk": C, "rows_in_loss": N_rows},
        "mfma_frac": round(mfma_frac, 4),
        "counted_tflop_per_step": round(flops / 1e12, 3),
        "peak_gib": round(peak_gib, 3),
        "loss": float(res[0][0]["loss"][0]) if args.workload == "c5" else float(res[0]["loss"][0]),
        "roofline": roofline,
        "kernels": kernels,
    }
    del ws
    torch.cuda.empty_cache()
    if not args.no_one_call:
        result["one_call"] = one_call_leg(kd, torch, wl, t, two_call_ms=ms,
                                          select=(args.workload == "c5"))
    if not args.no_chunk_sweep and args.workload == "c3":
        result["chunk_sweep"] = chunk_sweep(kd, torch, wl, t, [512, 1024, 2048])
    if not args.no_comparators and args.workload in ("c2", "c3"):
        result["comparators"] = comparator_leg(kd, torch, wl, t)
    if not args.no_teacher and args.workload == "c3":
        result["teacher_topk"] = teacher_leg(kd, torch, wl, t, p, cpu=not args.no_cpu_baseline)
    if not args.no_selection:
        result["selection"] = selection_leg(kd, torch, wl, t)
    del t
    torch.cuda.empty_cache()
    if not args.no_workloads:
        # the other configurations at full size, beside the headline one
        result["workloads"] = {}
        for key in ("c2", "c5"):
            if key != args.workload:
                result["workloads"][key] = time_workload(
                    kd, torch, key, comparators=(key == "c2" and not args.no_comparators))
    p4 = None
    if not args.no_mem_sweep or (not args.no_workloads and args.workload != "c4"):
        c4 = WORKLOADS["c4"]
        log("[bench] generating the 256K-context inputs")
        p4 = make_problem(c4["S"], c4["H"], c4["V"], c4["K"], T=c4["T"], chunk=c4["chunk"],
                          seed=c4["seed"])
    if not args.no_mem_sweep:
        sizes = [int(x) for x in args.mem_sizes.split(",") if x]
        result["peak_gib_vs_S"] = mem_sweep(kd, torch, sizes, p4)
    if not args.no_workloads and args.workload != "c4":
        result["workloads"]["c4"] = time_workload(kd, torch, "c4", p=p4)
    del p4
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_rows} rows")
        result["cpu_baseline"] = cpu_baseline(p, wl, args.cpu_rows)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
