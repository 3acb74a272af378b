#!/usr/bin/env python
"""Benchmark of the MLA forward on one MI355X.

One step = one DeepSeek-V3-shaped prefill (B=1, S=4096, bf16, interleaved
RoPE) followed by one absorbed decode step (B=64 sequences, latent cache
capacity 8193, lengths uniform in [1024, 8192], bf16).  Inputs are seeded
synthetic tensors already resident in HBM when timing starts.

Printed: one JSON line.  `value` is the prefill throughput in algorithmic
TFLOP/s (2 B S sum(params) + 2 B H S(S+1)/2 (d_n + d_r + d_v); the masked
upper triangle is not counted).  The decode result (latent-cache GB/s of the
attention kernel, algorithmic bytes = sum_b (L_b + 1) (r_kv + d_r) 2) sits in
"decode".  Kernel times come from HIP events the library records at its
stage boundaries on the launch stream.  Each recorded event costs the stream
a few microseconds, so the timed steps mark only the ends of each call and
the two kernels the roofline lines name (the prefill's dominant stage and the
latent attention); the per-stage breakdown comes from a separate pass of the
same steps with every boundary marked.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MI355X_BF16_TFLOPS = 2516.6   # dense MFMA bf16 peak
MI355X_HBM_GBS = 8000.0       # HBM3E peak

# HBM traffic per launch of the kernels a roofline line can name, from two
# rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE; KiB per
# dispatch, mean over the dispatches of that kernel), each scaled by what the
# same counter reads for a plain 1 GiB device copy (--copy-calibration):
# FETCH_SIZE reports half of the bytes the copy reads, WRITE_SIZE all it
# writes.  An entry holds only for the kernel sources it was measured on
# (SHA-256 over the listed files); otherwise the traffic is null.
COUNTER_SCALE = {"FETCH_SIZE": 2.0, "WRITE_SIZE": 1.0}
KERNEL_SOURCES = {
    "attention": ["attn_prefill.hip", "common.h", "internal.h"],
    "out_proj": ["gemm.hip", "common.h", "internal.h"],
    "latent_attention": ["decode.hip", "common.h", "internal.h"],
    "fp8_out_proj": ["gemm_fp8.hip", "common.h", "internal.h"],
}
TRAFFIC = {
    "attention": {
        "sha256": "a75e34605cb7e18bf5230a138275282c9c872140e0170178a4c3d2c5c67205a6",
        "FETCH_SIZE_KiB": 338164.8, "WRITE_SIZE_KiB": 132023.0},
    "out_proj": {
        "sha256": "1ce4fccadccf01107b93d0dad80251b2de984b467591e5025d7eb45a6ab40511",
        "FETCH_SIZE_KiB": 1481169.8, "WRITE_SIZE_KiB": 57344.0},
    "latent_attention": {
        "sha256": "5141dfedf8eddf2bfb5d071cb0d96d3dd0c523d724a8b3c07b2caf60f1727ef4",
        "FETCH_SIZE_KiB": 181457.15, "WRITE_SIZE_KiB": 38571.0},
    "fp8_out_proj": {
        "sha256": "d12584c8d003b594e35e2010205f90def85093e1799b289684299359a2e9cca4",
        "FETCH_SIZE_KiB": 380295.3, "WRITE_SIZE_KiB": 57792.0},
}
METRIC = "MLA prefill TFLOP/s + absorbed-decode latent-cache GB/s, V3 shapes, 1 MI355X"


def prefill_flops(c, B, S):
    D, H = c["hidden_size"], c["num_attention_heads"]
    rq, rkv = c["q_lora_rank"], c["kv_lora_rank"]
    dn, dr, dv = c["qk_nope_head_dim"], c["qk_rope_head_dim"], c["v_head_dim"]
    params = (rq * D + H * dn * rq + H * dr * rq + rkv * D + dr * D + H * dn * rkv
              + H * dv * rkv + D * H * dv)
    proj = 2.0 * B * S * params
    attn = 2.0 * B * H * (S * (S + 1) / 2.0) * (dn + dr + dv)
    return proj, attn, {
        "down_proj": 2.0 * B * S * (rq + rkv + dr) * D,
        "q_up_proj": 2.0 * B * S * H * (dn + dr) * rq,
        "kv_up_proj": 2.0 * B * S * H * (dn + dv) * rkv,
        "attention": attn,
        "out_proj": 2.0 * B * S * D * H * dv,
    }


def kernel_sha(stage):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[stage]:
        with open(os.path.join(ROOT, "head_latent_attention_08_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_bytes(stage):
    """Measured HBM bytes per launch of a stage's kernel, or None."""
    t = TRAFFIC.get(stage)
    if not t or t["sha256"] != kernel_sha(stage):
        return None
    return (t["FETCH_SIZE_KiB"] * COUNTER_SCALE["FETCH_SIZE"]
            + t["WRITE_SIZE_KiB"] * COUNTER_SCALE["WRITE_SIZE"]) * 1024.0


def decode_bytes(c, lens):
    w = c["kv_lora_rank"] + c["qk_rope_head_dim"]
    return float(sum(int(L) + 1 for L in lens) * w * 2)


def decode_flops(c, lens):
    H, r, dr = c["num_attention_heads"], c["kv_lora_rank"], c["qk_rope_head_dim"]
    return float(sum(int(L) + 1 for L in lens) * H * (2 * (r + dr) + 2 * r))


def multi_token_bytes_flops(c, lens, T):
    """Cache bytes (each row of a sequence read once for all its new tokens)
    and FLOPs of a multi-token decode step with T new tokens per sequence."""
    H, r, dr = c["num_attention_heads"], c["kv_lora_rank"], c["qk_rope_head_dim"]
    rows = sum(int(L) + T for L in lens)
    seen = sum(int(L) + t + 1 for L in lens for t in range(T))
    return float(rows * (r + dr) * 2), float(seen * H * (2 * (r + dr) + 2 * r))


def chunk_flops(c, L, T):
    """Algorithmic FLOPs of an expanded-form chunk of T tokens after L cached
    rows (one sequence): projections of the new tokens, the up-projection of
    all L + T key rows, the causal attention and the output projection."""
    D, H = c["hidden_size"], c["num_attention_heads"]
    rq, rkv = c["q_lora_rank"], c["kv_lora_rank"]
    dn, dr, dv = c["qk_nope_head_dim"], c["qk_rope_head_dim"], c["v_head_dim"]
    proj = 2 * T * (D * (rq + rkv + dr) + rq * H * (dn + dr) + H * dv * D)
    kv = 2 * (L + T) * rkv * H * (dn + dv)
    pairs = sum(L + t + 1 for t in range(T))
    return float(proj + kv + pairs * H * 2 * (dn + dr + dv))


def cpu_baseline(c_pre, x, w, c_dec, xd, wd, lens, cache, seconds_hint=True):
    """The float64 oracle, untuned, on bounded samples of the same workloads."""
    import numpy as np

    import oracle as orc
    from tests.helpers import oracle_cfg
    blas = "unknown"
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        bl = [i for i in info if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in bl] or [1])
        if bl:
            blas = f"{bl[0].get('internal_api', '?')} {bl[0].get('version', '')}".strip()
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    s_sample = x.shape[1]  # the whole S=4096 prefill: about 10 s of float64 work
    t0 = time.perf_counter()
    orc.mla_prefill(oracle_cfg(c_pre), w, x[:, :s_sample])
    t_pre = time.perf_counter() - t0
    proj, attn, _ = prefill_flops(c_pre, 1, s_sample)
    n_seq = len(lens)  # all 64 sequences
    t0 = time.perf_counter()
    orc.mla_decode_absorbed(oracle_cfg(c_dec), wd, xd[:n_seq], cache[:n_seq], lens[:n_seq])
    t_dec = time.perf_counter() - t0
    return {
        "value": (proj + attn) / t_pre / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"the full prefill workload (B=1, S={s_sample}; {(proj + attn) / 1e9:.1f} GFLOP "
                  f"in {t_pre:.2f} s, float64 NumPy)",
        "decode": {
            "value": decode_bytes(c_dec, lens[:n_seq]) / t_dec / 1e9,
            "unit": "GB/s",
            "sample": f"absorbed decode of all {n_seq} sequences ({t_dec:.2f} s)",
        },
        "blas": blas,
        "host_cpus": os.cpu_count(),
        "affinity_cpus": len(os.sched_getaffinity(0)),
    }


MI355X_FP8_TFLOPS = 2 * MI355X_BF16_TFLOPS  # dense E4M3 matrix-core peak


def fp8_projections(m, S, log, reps=20):
    """Block-scaled FP8 products at the prefill projection shapes (S tokens):
    activation quantisation (1 x 128 tiles) plus the product, per projection,
    timed with HIP events on the stream both run on.  Operands are seeded
    device draws (activations N(0, 1), weights N(0, 0.006^2)); the weights
    are quantised once, outside the timed region (they are static).  A
    context line: the headline value stays the bf16 path."""
    import torch
    D, rq, rkv, dr, H, dn, dv = 7168, 1536, 512, 64, 128, 128, 128
    shapes = {"down_proj": (S, rq + rkv + dr, D), "q_up_proj": (S, H * (dn + dr), rq),
              "kv_up_proj": (S, H * (dn + dv), rkv), "out_proj": (S, D, H * dv)}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9000)
    res, ops = {}, {}
    for name, (M, N, K) in shapes.items():
        x = torch.randn(M, K, device="cuda", dtype=torch.float32, generator=gen).to(torch.bfloat16)
        w = (torch.randn(N, K, device="cuda", dtype=torch.float32, generator=gen) * 0.006).to(torch.bfloat16)
        qb, sb = m.mla_fp8_quantize_blocks(w)
        del w
        qa, sa = m.mla_fp8_quantize_rows(x)
        ops[name] = (x, qa, sa, qb, sb, torch.empty(M, N, device="cuda", dtype=torch.bfloat16))
    st = torch.cuda.current_stream()
    for _ in range(3):
        for name in shapes:
            x, qa, sa, qb, sb, c = ops[name]
            m.mla_fp8_gemm(qa, sa, qb, sb, c=c)
    torch.cuda.synchronize()
    tot_q = tot_g = 0.0
    for name, (M, N, K) in shapes.items():
        x, qa, sa, qb, sb, c = ops[name]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(st)
        for _ in range(reps):
            m.mla_fp8_quantize_rows(x)
        ev[1].record(st)
        for _ in range(reps):
            m.mla_fp8_gemm(qa, sa, qb, sb, c=c)
        ev[2].record(st)
        torch.cuda.synchronize()
        q_ms, g_ms = ev[0].elapsed_time(ev[1]) / reps, ev[1].elapsed_time(ev[2]) / reps
        fl = 2.0 * M * N * K
        res[name] = {"M": M, "N": N, "K": K, "quant_ms": q_ms, "gemm_ms": g_ms,
                     "gemm_tflops": fl / (g_ms * 1e-3) / 1e12,
                     "frac_of_fp8_peak": fl / (g_ms * 1e-3) / 1e12 / MI355X_FP8_TFLOPS}
        tot_q += q_ms
        tot_g += g_ms
        log(f"bench: fp8 {name} {M}x{N}x{K}: quant {q_ms * 1e3:.1f} us, product {g_ms * 1e3:.1f} us, "
            f"{res[name]['gemm_tflops']:.0f} TFLOP/s")
    o = ops["out_proj"]
    M, N, K = shapes["out_proj"]
    res["roofline"] = {"bound": "mfma", "kernel": "fp8_gemm_kernel (out_proj)",
                       "achieved": res["out_proj"]["gemm_tflops"], "peak": MI355X_FP8_TFLOPS,
                       "unit": "TFLOP/s", "frac": res["out_proj"]["frac_of_fp8_peak"],
                       "traffic": traffic_bytes("fp8_out_proj"),
                       "flops_per_launch": 2.0 * M * N * K, "ms_per_launch": res["out_proj"]["gemm_ms"]}
    res["total_ms"] = {"quant": tot_q, "gemm": tot_g}
    del ops, o
    torch.cuda.empty_cache()
    return res


def long_context_line(m, log, reps=3):
    """Long-context V3 prefill with YaRN RoPE: B=1, S=32768, factor 40 over
    an original 4096 context, beta 32/1, mscale 1/1 (the configuration whose
    260 sampled rows the GPU tests check against the oracle, same seeded
    inputs).  Per-stage times from the library's stage events; the roofline
    entry is for its dominant kernel (attention: 78% of the FLOPs)."""
    import torch
    import synth_inputs as si
    from tests.gpu_util import mla_cfg, to_dev, weights_to_dev
    c = si.CONFIGS["v3_yarn"]
    B, S = c["batch"], c["seq"]
    log(f"bench: generating long-context inputs (B={B}, S={S}, seed {c['seed']})")
    x, w = si.make_inputs(c)
    xd, wd = to_dev(x, "bf16"), weights_to_dev(w, "bf16")
    del x, w
    cfg = mla_cfg(c)
    y = torch.empty((B, S, c["hidden_size"]), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(m.mla_prefill_workspace_size(cfg, B, S), dtype=torch.uint8, device="cuda")
    n_ev = len(m.PREFILL_STAGES) + 1
    m.mla_prefill_forward(cfg, wd, xd, y=y, workspace=ws)
    torch.cuda.synchronize()
    evs = []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        for ev in e:
            ev.record()
        evs.append(e)
    torch.cuda.synchronize()
    for e in evs:
        m.mla_set_stage_events([ev.cuda_event for ev in e])
        m.mla_prefill_forward(cfg, wd, xd, y=y, workspace=ws)
        m.mla_set_stage_events(None)
    torch.cuda.synchronize()
    import statistics
    stage = {n: statistics.median(e[k].elapsed_time(e[k + 1]) for e in evs)
             for k, n in enumerate(m.PREFILL_STAGES)}
    whole = [e[0].elapsed_time(e[-1]) for e in evs]
    proj, attn, per = prefill_flops(c, B, S)
    ms = statistics.median(whole)
    tf = (proj + attn) / (ms * 1e-3) / 1e12
    stage_tf = {k: per[k] / (stage[k] * 1e-3) / 1e12 for k in per}
    log(f"bench: long-context prefill S={S} YaRN: {ms:.2f} ms, {tf:.0f} TFLOP/s "
        f"(attention {stage['attention']:.2f} ms, {stage_tf['attention']:.0f} TFLOP/s)")
    del xd, wd, y, ws
    torch.cuda.empty_cache()
    return {"workload": "v3_yarn_prefill_b1_s32768", "batch": B, "seq_len": S,
            "rope": "interleaved, YaRN factor 40, original 4096, beta 32/1, mscale 1/1",
            "gflop": (proj + attn) / 1e9, "ms": ms, "ms_min": min(whole), "tflops": tf,
            "frac_of_bf16_peak": tf / MI355X_BF16_TFLOPS, "stage_ms": stage, "stage_tflops": stage_tf,
            "roofline": {"bound": "mfma", "kernel": "attention", "achieved": stage_tf["attention"],
                         "peak": MI355X_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": stage_tf["attention"] / MI355X_BF16_TFLOPS,
                         "flops_per_launch": per["attention"], "ms_per_launch": stage["attention"]}}


def fp8_prefill_line(m, cfg_pre, wd_pre, xd_pre, bf16_ms, log, reps=20):
    """The V3 prefill (B=1, S=4096) with its four projection products on
    block-scaled FP8 and attention in bf16 (mla_prefill_forward_fp8), same
    inputs as the headline; weights quantised once outside the timed region.
    Per-stage medians from the stage events; FLOPs counted as for the bf16
    prefill."""
    import statistics
    import torch
    B, S = xd_pre.shape[0], xd_pre.shape[1]
    buf, w8 = m.mla_fp8_prepare_weights(cfg_pre, wd_pre)
    y = torch.empty_like(xd_pre)
    ws = torch.empty(m.mla_prefill_fp8_workspace_size(cfg_pre, B, S), dtype=torch.uint8, device="cuda")
    for _ in range(5):
        m.mla_prefill_forward_fp8(cfg_pre, wd_pre, w8, xd_pre, y=y, workspace=ws)
    n_ev = len(m.PREFILL_STAGES) + 1
    evs = []
    for _ in range(reps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(n_ev)]
        for ev in e:
            ev.record()
        evs.append(e)
    torch.cuda.synchronize()
    for e in evs:
        m.mla_set_stage_events([ev.cuda_event for ev in e])
        m.mla_prefill_forward_fp8(cfg_pre, wd_pre, w8, xd_pre, y=y, workspace=ws)
        m.mla_set_stage_events(None)
    torch.cuda.synchronize()
    stage = {n: statistics.median(e[k].elapsed_time(e[k + 1]) for e in evs)
             for k, n in enumerate(m.PREFILL_STAGES)}
    ms = statistics.median(e[0].elapsed_time(e[-1]) for e in evs)
    import synth_inputs as si
    proj, attn, _ = prefill_flops(si.CONFIGS["v3_prefill"], B, S)
    tf = (proj + attn) / (ms * 1e-3) / 1e12
    log(f"bench: fp8 prefill S={S}: {ms:.3f} ms, {tf:.0f} TFLOP/s (bf16 prefill {bf16_ms:.3f} ms)")
    del buf, y, ws
    torch.cuda.empty_cache()
    return {"workload": "v3_prefill_b1_s4096, projections block-scaled fp8 (e4m3), attention bf16",
            "ms": ms, "tflops": tf, "speedup_vs_bf16": bf16_ms / ms, "stage_ms": stage}


def attention_backward_line(m, S, log, reps=2):
    """Causal attention backward (dQ, dK, dV) at the V3 prefill attention
    shape: 128 heads, S tokens, d_qk 192, d_v 128, bf16, seeded device draws
    (N(0, 1) q, k, v, dout; o a stand-in of the same shape: it only enters
    through rowsum(dout * o)).  Algorithmic work: the five causal products
    (Q K^T, dO V^T, P^T dO, dS K, dS^T Q) over the S(S+1)/2 visible pairs."""
    import torch
    H, dqk, dv = 128, 192, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(9500)
    mk = lambda d: torch.randn((H, S, d), device="cuda", generator=gen).to(torch.bfloat16)
    q, k, v, o, do = mk(dqk), mk(dqk), mk(dv), mk(dv), mk(dv)
    scale = dqk ** -0.5
    m.mla_attention_backward(q, k, v, o, do, scale)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(reps):
        m.mla_attention_backward(q, k, v, o, do, scale)
    e1.record(st)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    fl = 2.0 * H * (S * (S + 1) / 2.0) * (3 * dqk + 2 * dv)
    tf = fl / (ms * 1e-3) / 1e12
    log(f"bench: attention backward H={H} S={S}: {ms:.2f} ms, {tf:.1f} TFLOP/s")
    del q, k, v, o, do
    torch.cuda.empty_cache()
    # the whole MLA backward (forward recomputed, every gradient) on the V3
    # prefill's inputs with a seeded upstream gradient
    import synth_inputs as si
    from tests.gpu_util import mla_cfg, to_dev, weights_to_dev
    c = si.CONFIGS["v3_prefill"]
    x, w = si.make_inputs(c, seq=S)
    xd, wd = to_dev(x, "bf16"), weights_to_dev(w, "bf16")
    dy = torch.randn(xd.shape, device="cuda", generator=gen).to(torch.bfloat16)
    cfg = mla_cfg(c)
    ws = torch.empty(m.mla_backward_workspace_size(cfg, 1, S), dtype=torch.uint8, device="cuda")
    m.mla_backward(cfg, wd, xd, dy, workspace=ws)
    torch.cuda.synchronize()
    e0.record(st)
    m.mla_backward(cfg, wd, xd, dy, workspace=ws)
    e1.record(st)
    torch.cuda.synchronize()
    full_ms = e0.elapsed_time(e1)
    log(f"bench: MLA backward (forward recomputed, all gradients) S={S}: {full_ms:.2f} ms")
    del xd, wd, dy, ws
    torch.cuda.empty_cache()
    return {"heads": H, "seq_len": S, "d_qk": dqk, "d_v": dv, "dtype": "bf16", "ms": ms,
            "gflop": fl / 1e9, "tflops": tf, "frac_of_bf16_peak": tf / MI355X_BF16_TFLOPS,
            "note": "bf16 32x32x16 MFMA kernels: row statistics, dK/dV per key block, dQ per query block (no atomics)",
            "mla_backward_ms": full_ms,
            "mla_backward_note": "mla_backward at V3 sizes, B=1: forward recomputed, dx and every weight gradient"}


def _read_csv(path):
    import csv
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def _short_name(name):
    """Kernel name without namespaces and arguments.  rocprofv3 prints some
    names mangled; those in this library's namespace are decoded here (the
    kernel name and its type / integer template arguments), since the
    system demangler does not know the bf16 type's code."""
    import re
    m = re.match(r"_ZN3mla12_GLOBAL__N_1(\d+)", name)
    if m:
        n = int(m.group(1))
        rest = name[m.end():]
        base, rest = rest[:n], rest[n:]
        args = []
        if rest.startswith("I"):
            rest = rest[1:]
            while rest and not rest.startswith("E"):
                t = re.match(r"DF16b|f|L[ib]\d+E|Li-?\d+E", rest)
                if not t:
                    break
                tok = t.group(0)
                args.append({"DF16b": "bf16", "f": "float"}.get(
                    tok, tok[2:-1] if tok.startswith("Li") else ("true" if tok == "Lb1E" else "false")))
                rest = rest[t.end():]
        return base + (f"<{', '.join(args)}>" if args else "")
    n = name.replace("(anonymous namespace)::", "").replace("void ", "").replace("mla::", "")
    return n.split("(")[0][:96]


def summarize_trace(path):
    """Markdown table of a rocprofv3 kernel trace (kernel_trace.csv): one row
    per (kernel, grid size), with the launch count and the mean, median and
    min duration.  Separate rows per grid keep the projection GEMMs apart."""
    import statistics
    rows = _read_csv(path)
    groups = {}
    for r in rows:
        key = (_short_name(r["Kernel_Name"]),
               int(r.get("Grid_Size_X", r.get("Grid_Size", 0)) or 0)
               * int(r.get("Grid_Size_Y", 1) or 1) * int(r.get("Grid_Size_Z", 1) or 1),
               int(r.get("Workgroup_Size_X", r.get("Workgroup_Size", 0)) or 0))
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault(key, []).append(d)
    out = ["| kernel | grid (threads) | workgroups | launches | mean us | median us | min us | total us |",
           "|---|---|---|---|---|---|---|---|"]
    for (name, grid, wg), ds in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        out.append(f"| `{name}` | {grid} | {grid // wg if wg else '-'} | {len(ds)} | "
                   f"{statistics.mean(ds):.1f} | {statistics.median(ds):.1f} | {min(ds):.1f} | "
                   f"{sum(ds):.1f} |")
    return "\n".join(out)


def summarize_counters(path):
    """Markdown table of a rocprofv3 --pmc run (counter_collection.csv): per
    (kernel, grid size), the mean of each counter over its dispatches, plus
    what the counters give directly.  GRBM_GUI_ACTIVE is summed over the
    eight XCDs, so GRBM_GUI_ACTIVE / 8 / duration is the clock; the SQ cycle
    counters are summed over the SIMDs (1024) or CUs (256) they name:
      clock MHz   = GRBM_GUI_ACTIVE / 8 / duration
      MFMA busy   = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024)
      bf16 MFMA TFLOP/s executed = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 / duration
      LDS busy    = SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE / 8 x 256)
      LDS conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
    (MFMA busy cycles count 1024 bf16 FLOPs each: one SIMD's dense rate.)"""
    rows = _read_csv(path)
    groups = {}
    for r in rows:
        key = (_short_name(r["Kernel_Name"]), int(r.get("Grid_Size", 0) or 0))
        g = groups.setdefault(key, {"dispatch": {}, "dur": {}})
        did = r.get("Dispatch_Id") or r.get("Correlation_Id")
        g["dispatch"].setdefault(did, {})
        g["dispatch"][did][r["Counter_Name"]] = g["dispatch"][did].get(r["Counter_Name"], 0.0) + \
            float(r["Counter_Value"])
        if r.get("Start_Timestamp") and r.get("End_Timestamp"):
            g["dur"][did] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    names = sorted({c for g in groups.values() for d in g["dispatch"].values() for c in d})
    head = "| kernel | grid | dispatches | mean us | " + " | ".join(names)
    extra = []
    has = lambda *cs: all(c in names for c in cs)
    if has("GRBM_GUI_ACTIVE"):
        extra.append("clock MHz")
    if has("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"):
        extra.append("MFMA busy")
    if has("SQ_INSTS_VALU_MFMA_MOPS_BF16"):
        extra.append("bf16 MFMA TFLOP/s")
    if has("SQ_LDS_IDX_ACTIVE", "GRBM_GUI_ACTIVE"):
        extra.append("LDS busy")
    if has("SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT"):
        extra.append("LDS conflict share")
    out = [head + "".join(f" | {e}" for e in extra) + " |",
           "|" + "---|" * (4 + len(names) + len(extra))]
    for (name, grid), g in sorted(groups.items()):
        ds = list(g["dispatch"].values())
        mean = {c: sum(d.get(c, 0.0) for d in ds) / len(ds) for c in names}
        dur = sum(g["dur"].values()) / len(g["dur"]) if g["dur"] else float("nan")
        cells = [f"`{name}`", str(grid), str(len(ds)), f"{dur:.1f}"] + [f"{mean[c]:.4g}" for c in names]
        cyc = mean.get("GRBM_GUI_ACTIVE", 0.0) / 8.0
        if "clock MHz" in extra:
            cells.append(f"{cyc / dur:.0f}")
        if "MFMA busy" in extra:
            cells.append(f"{mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (cyc * 1024.0):.3f}" if cyc else "-")
        if "bf16 MFMA TFLOP/s" in extra:
            cells.append(f"{512.0 * mean['SQ_INSTS_VALU_MFMA_MOPS_BF16'] / (dur * 1e-6) / 1e12:.1f}")
        if "LDS busy" in extra:
            cells.append(f"{mean['SQ_LDS_IDX_ACTIVE'] / (cyc * 256.0):.3f}" if cyc else "-")
        if "LDS conflict share" in extra:
            a = mean["SQ_LDS_IDX_ACTIVE"]
            cells.append(f"{mean['SQ_LDS_BANK_CONFLICT'] / a:.3f}" if a else "-")
        out.append("| " + " | ".join(cells) + " |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the GPU's clocks settle over the first second or so of load: the
    # default warm-up runs ~1.5 s of the same full steps
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the causal attention backward (context line)")
    ap.add_argument("--no-long-context", action="store_true",
                    help="skip the S=32768 YaRN prefill (context line)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the block-scaled FP8 projection products (context line)")
    ap.add_argument("--no-multi-token", action="store_true",
                    help="skip the multi-token decode lines (q_len 2 and 4)")
    ap.add_argument("--only", choices=["prefill", "decode", "backward"], default=None,
                    help="time one of the two workloads, or the backward context line, only "
                         "(profiling aid; no JSON line)")
    ap.add_argument("--replicas", type=int, default=3,
                    help="decode cache replicas rotated per step (defeats the 256 MB MALL)")
    ap.add_argument("--kernel-sha", action="store_true",
                    help="print the source hashes the traffic table is keyed on and exit")
    ap.add_argument("--summarize-trace", metavar="KERNEL_TRACE_CSV",
                    help="print a per-(kernel, grid) markdown table of a rocprofv3 kernel "
                         "trace and exit (no GPU)")
    ap.add_argument("--summarize-counters", metavar="COUNTER_COLLECTION_CSV",
                    help="print a per-(kernel, grid) markdown table of a rocprofv3 --pmc "
                         "run and exit (no GPU)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy three times: the known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    if args.kernel_sha:
        print(json.dumps({k: kernel_sha(k) for k in KERNEL_SOURCES}))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return

    import numpy as np
    import torch

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"read_bytes": n, "write_bytes": n, "launches": 3}}),
              flush=True)
        return

    import head_latent_attention_08_amd as m
    import synth_inputs as si
    from tests.gpu_util import mla_cfg, to_dev, weights_to_dev

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    if args.only == "backward":
        torch.cuda.set_device(0)
        r = attention_backward_line(m, si.CONFIGS["v3_prefill"]["seq"], log)
        log(f"bench: backward only: attention {r['ms']:.2f} ms, MLA backward {r['mla_backward_ms']:.2f} ms")
        return

    torch.cuda.set_device(0)
    c_pre = si.CONFIGS["v3_prefill"]
    c_dec = si.CONFIGS["v3_decode"]
    cfg_pre = mla_cfg(c_pre)
    B, S = c_pre["batch"], c_pre["seq"]
    if args.only != "decode":
        log("bench: generating V3 prefill inputs (seed 3000)")
        x, w = si.make_inputs(c_pre)
        xd_pre = to_dev(x, "bf16")
        wd_pre = weights_to_dev(w, "bf16")
        y_pre = torch.empty((B, S, c_pre["hidden_size"]), dtype=torch.bfloat16, device="cuda")
        lat_pre = torch.empty((B, S, 576), dtype=torch.bfloat16, device="cuda")
        ws_pre = torch.empty(m.mla_prefill_workspace_size(cfg_pre, B, S), dtype=torch.uint8,
                             device="cuda")

    log("bench: generating V3 decode inputs (seed 4000)")
    xdec, wdec, lens, cache = si.make_decode_inputs(c_dec)
    cfg_dec = mla_cfg(c_dec)
    caches = [to_dev(cache, "bf16")]
    for _ in range(args.replicas - 1):
        caches.append(caches[0].clone())
    lens_d = torch.from_numpy(lens).cuda()
    xdec_d = to_dev(xdec, "bf16")
    wdec_d = weights_to_dev(wdec, "bf16")
    Bd = xdec.shape[0]
    y_dec = torch.empty((Bd, c_dec["hidden_size"]), dtype=torch.bfloat16, device="cuda")
    ws_dec = torch.empty(m.mla_decode_workspace_size(cfg_dec, Bd, caches[0].shape[1]),
                         dtype=torch.uint8, device="cuda")

    n_pe = len(m.PREFILL_STAGES) + 1
    n_de = len(m.DECODE_STAGES) + 1

    def new_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record()  # creates the underlying hipEvent_t
        return evs

    def step(i, pe=None, de=None):
        if args.only != "decode":
            m.mla_set_stage_events([e.cuda_event if e is not None else None for e in pe]
                                   if pe else None)
            m.mla_prefill_forward(cfg_pre, wd_pre, xd_pre, y=y_pre, latent_out=lat_pre,
                                  workspace=ws_pre)
        if args.only != "prefill":
            m.mla_set_stage_events([e.cuda_event if e is not None else None for e in de]
                                   if de else None)
            m.mla_decode_absorbed(cfg_dec, wdec_d, xdec_d, caches[i % len(caches)], lens_d,
                                  y=y_dec, workspace=ws_dec)
        m.mla_set_stage_events(None)

    log(f"bench: warmup {args.warmup} steps")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # per-stage breakdown: the same steps with every stage boundary marked
    pev = [new_events(n_pe) for _ in range(args.steps)]
    dev_ = [new_events(n_de) for _ in range(args.steps)]
    torch.cuda.synchronize()
    log(f"bench: stage breakdown over {args.steps} steps")
    for i in range(args.steps):
        step(i, pev[i], dev_[i])
    torch.cuda.synchronize()
    if args.only:
        total_ms = sum(e[0].elapsed_time(e[-1]) for e in (pev if args.only == "prefill" else dev_))
        log(f"bench: {args.only} only, {total_ms / args.steps:.3f} ms per step")
        evs, names = (pev, m.PREFILL_STAGES) if args.only == "prefill" else (dev_, m.DECODE_STAGES)
        for k, n in enumerate(names):
            t = sum(e[k].elapsed_time(e[k + 1]) for e in evs) / len(evs)
            log(f"bench:   {n:18s} {t * 1e3:9.1f} us")
        return

    def stage_ms(evs, names):
        per = {n: [] for n in names}
        whole = []
        for e in evs:
            for k, n in enumerate(names):
                per[n].append(e[k].elapsed_time(e[k + 1]))
            whole.append(e[0].elapsed_time(e[-1]))
        return {n: float(np.median(v)) for n, v in per.items()}, float(np.median(whole)), \
            float(np.min(whole))

    pst, _, _ = stage_ms(pev, m.PREFILL_STAGES)
    dst, _, _ = stage_ms(dev_, m.DECODE_STAGES)
    proj, attn, per_flops = prefill_flops(c_pre, B, S)
    stage_tf = {k: per_flops[k] / (pst[k] * 1e-3) / 1e12 for k in per_flops}
    dom = max(per_flops, key=lambda k: pst[k])

    # timed steps: events at the ends of each call and around the prefill's
    # dominant stage and the decode's latent attention only
    k_dom = m.PREFILL_STAGES.index(dom)
    k_lat = m.DECODE_STAGES.index("latent_attention")
    keep_p = {0, k_dom, k_dom + 1, n_pe - 1}
    keep_d = {0, k_lat, k_lat + 1, n_de - 1}
    tpe = [[e if j in keep_p else None for j, e in enumerate(new_events(n_pe))]
           for _ in range(args.steps)]
    tde = [[e if j in keep_d else None for j, e in enumerate(new_events(n_de))]
           for _ in range(args.steps)]
    log(f"bench: timing {args.steps} steps")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for i in range(args.steps):
        step(i, tpe[i], tde[i])
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)

    def span(evs, a, b):
        return [e[a].elapsed_time(e[b]) for e in evs]

    pre_all, dec_all = span(tpe, 0, n_pe - 1), span(tde, 0, n_de - 1)
    pre_ms, pre_min = float(np.median(pre_all)), float(np.min(pre_all))
    dec_ms, dec_min = float(np.median(dec_all)), float(np.min(dec_all))
    dom_ms = float(np.median(span(tpe, k_dom, k_dom + 1)))
    pre_tflops = (proj + attn) / (pre_ms * 1e-3) / 1e12
    kv_bytes = decode_bytes(c_dec, lens)
    att_ms = float(np.median(span(tde, k_lat, k_lat + 1)))
    att_merge_ms = dst["latent_attention"] + dst["split_merge"]
    dec_gbs = kv_bytes / (att_ms * 1e-3) / 1e9

    dom_tf = per_flops[dom] / (dom_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "kernel": dom, "achieved": dom_tf,
                "peak": MI355X_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": dom_tf / MI355X_BF16_TFLOPS, "traffic": traffic_bytes(dom),
                "flops_per_launch": per_flops[dom], "ms_per_launch": dom_ms}
    decode_roofline = {"bound": "hbm", "kernel": "latent_attention", "achieved": dec_gbs,
                       "peak": MI355X_HBM_GBS, "unit": "GB/s", "frac": dec_gbs / MI355X_HBM_GBS,
                       "traffic": traffic_bytes("latent_attention"),
                       "bytes_per_launch": kv_bytes, "ms_per_launch": att_ms}

    out = {
        "metric": METRIC,
        "value": pre_tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": total_ms / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations and cache, N(0,0.006^2) weights)",
        "config": {"workload": "v3_prefill_b1_s4096 + v3_decode_b64_cap8193",
                   "prefill": {"batch": B, "seq_len": S, "rope": "interleaved",
                               "gflop": (proj + attn) / 1e9},
                   "decode": {"batch": Bd, "cache_capacity": int(caches[0].shape[1]),
                              "lens": "U{1024..8192} seed 4001",
                              "latent_bytes": kv_bytes, "replicas": len(caches)}},
        "prefill": {"ms": pre_ms, "ms_min": pre_min, "tflops": pre_tflops,
                    "frac_of_bf16_peak": pre_tflops / MI355X_BF16_TFLOPS,
                    "stage_ms": pst, "stage_tflops": stage_tf,
                    "stage_note": "stage_ms from a separate pass with every stage boundary marked; "
                                  "ms from steps marked at the ends and around the dominant stage"},
        "decode": {"value": dec_gbs, "unit": "GB/s", "attention_ms": att_ms,
                   "attention_plus_merge_ms": att_merge_ms,
                   "attention_plus_merge_gbs": kv_bytes / (att_merge_ms * 1e-3) / 1e9,
                   "attention_tflops": decode_flops(c_dec, lens) / (att_ms * 1e-3) / 1e12,
                   "step_ms": dec_ms, "step_ms_min": dec_min, "stage_ms": dst},
        "roofline": roofline,
        "decode_roofline": decode_roofline,
    }
    if not args.no_multi_token:
        # Multi-token absorbed decode (q_len new tokens per sequence) on the
        # first sequences of the same cache, 64 token rows per step; not part
        # of the headline value
        lines = []
        for Bm, T in ((32, 2), (16, 4)):
            lm = np.minimum(lens[:Bm], caches[0].shape[1] - T).astype(np.int32)
            xm = torch.randn((Bm, T, c_dec["hidden_size"]), dtype=torch.float32,
                             generator=torch.Generator().manual_seed(4300 + T)).to(
                                 "cuda", torch.bfloat16)
            ym = torch.empty_like(xm)
            wsm = torch.empty(m.mla_decode_multi_workspace_size(cfg_dec, Bm, T, caches[0].shape[1]),
                              dtype=torch.uint8, device="cuda")
            lmd = torch.from_numpy(lm).cuda()
            evm = [new_events(n_de) for _ in range(8)]
            for i in range(8):
                m.mla_set_stage_events([e.cuda_event for e in evm[i]])
                m.mla_decode_absorbed_multi(cfg_dec, wdec_d, xm, caches[i % len(caches)][:Bm], lmd,
                                            y=ym, workspace=wsm)
                m.mla_set_stage_events(None)
            torch.cuda.synchronize()
            mst, m_ms, _ = stage_ms(evm[3:], m.DECODE_STAGES)
            mb, mf = multi_token_bytes_flops(c_dec, lm, T)
            a_ms = mst["latent_attention"]
            lines.append({"q_len": T, "batch": Bm, "attention_ms": a_ms,
                          "cache_gbs": mb / (a_ms * 1e-3) / 1e9,
                          "attention_tflops": mf / (a_ms * 1e-3) / 1e12,
                          "step_ms": m_ms, "cache_bytes": mb})
            log(f"bench: multi-token decode q_len={T} B={Bm}: attention {a_ms * 1e3:.1f} us, "
                f"{mb / (a_ms * 1e-3) / 1e9:.0f} GB/s, step {m_ms * 1e3:.1f} us")
        out["decode_multi_token"] = lines
        # Chunked prefill against a latent cache, expanded form: one sequence,
        # 3072 cached rows (a copy of a decode sequence's cache), 1024 new
        # tokens; context only
        Lc, Tc = 3072, 1024
        cache_c = caches[0][:1].clone()
        lens_c = torch.tensor([Lc], dtype=torch.int32, device="cuda")
        xc = torch.randn((1, Tc, c_dec["hidden_size"]), dtype=torch.float32,
                         generator=torch.Generator().manual_seed(4400)).to("cuda", torch.bfloat16)
        yc = torch.empty_like(xc)
        wsc = torch.empty(m.mla_prefill_chunk_workspace_size(cfg_dec, 1, Tc, cache_c.shape[1], Lc + Tc),
                          dtype=torch.uint8, device="cuda")
        for _ in range(3):
            m.mla_prefill_chunk(cfg_dec, wdec_d, xc, cache_c, lens_c, Lc + Tc, y=yc, workspace=wsc)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            m.mla_prefill_chunk(cfg_dec, wdec_d, xc, cache_c, lens_c, Lc + Tc, y=yc, workspace=wsc)
        e1.record()
        torch.cuda.synchronize()
        c_ms = e0.elapsed_time(e1) / 5
        c_fl = chunk_flops(c_dec, Lc, Tc)
        out["prefill_chunk"] = {"cached_rows": Lc, "q_len": Tc, "ms": c_ms,
                                "tflops": c_fl / (c_ms * 1e-3) / 1e12, "gflop": c_fl / 1e9}
        log(f"bench: prefill chunk {Tc} tokens after {Lc} cached rows: {c_ms:.3f} ms, "
            f"{c_fl / (c_ms * 1e-3) / 1e12:.0f} TFLOP/s")
    if not args.no_fp8:
        out["fp8_prefill"] = fp8_prefill_line(m, cfg_pre, wd_pre, xd_pre, pre_ms, log)
    if not args.no_long_context:
        out["long_context"] = long_context_line(m, log)
    if not args.no_fp8:
        out["fp8_projections"] = fp8_projections(m, S, log)
    if not args.no_backward:
        out["attention_backward"] = attention_backward_line(m, S, log)
    if not args.no_cpu_baseline:
        log("bench: timing the float64 oracle on bounded samples")
        out["cpu_baseline"] = cpu_baseline(c_pre, x, w, c_dec, xdec, wdec, lens, cache)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
