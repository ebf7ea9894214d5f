#!/usr/bin/env python3
"""Benchmark of the CSA2 layer hot path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
  compress (write the new token's KV row)  ->  index FULL (lightning-indexer scan +
  top-k)  ->  sparse shared-KV attention (selected entries + window).

Default workload: the decoder Full layer at decode (32 queries, each over 65,536 cached
entries, m = 1, bf16 cache, 64 indexer heads x 128, top-512 + 128-token window,
64 heads x 512).  Inputs are resident in HBM before the timed region; two independent
input instances alternate so the gathered rows of one step are not cache-resident from
the step before.

Prints one JSON line.  `value` = decode queries per second of the whole step.  The
roofline block is for the dominant kernel (the indexer scan), with per-launch durations
from HIP events recorded around every kernel on its stream (a second timed pass; the
first pass, without per-kernel events, gives `value`).

    python bench.py [--steps K] [--warmup W] [--config 2|3|4|5] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "decode queries/s + indexer scores/s at 64K-1M ctx; % of HBM / MFMA peak"
HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=2, choices=[2, 3, 4, 5])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="bound of the oracle sample")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (calibrates the HBM byte counters)")
    return p.parse_args()


# ---------------------------------------------------------------------------- workloads
def make_decode(torch, W, wl, seed, fp4=False):
    """One instance of a decode workload on the device (seeded generator)."""
    g = W.rng(seed, device="cuda")
    B, L, c, H = wl.B, wl.L, wl.c, wl.H
    d = {}
    if fp4:
        d.update(W.indexer_inputs(g, B, 1, L, wl.H_I, wl.d_I, wl.w_values, k_format="mxfp4"))
        a = W.attn_inputs(g, B, 1, L, H, c, Lw=wl.window, kv_format="fp4")
    else:
        d.update(W.indexer_inputs(g, B, 1, L, wl.H_I, wl.d_I, wl.w_values))
        a = W.attn_inputs(g, B, 1, L, H, c, Lw=wl.window)
    d.update(a)
    d["q_pos"] = torch.full((B, 1), L, dtype=torch.int32, device="cuda")
    d["win_pos0"] = torch.full((B,), L - wl.window + 1, dtype=torch.int32, device="cuda")
    # the new token's projected KV and gate logits (m = 1 compress input)
    d["c_new"] = g.normal((B, 1, c), dtype="bf16")
    d["z_new"] = g.normal((B, 1, c), dtype="bf16")
    return d


def decode_step(C, torch, wl, d, ws, out_idx, out, fp4=False):
    B, c = wl.B, wl.c
    # 1. compress: the new token's row (m = 1: RMSNorm + RoPE at position L) into the
    #    last slot of the window buffer
    win = d["win"]
    C.csa2_compress(d["c_new"], d["z_new"], 1, pos0=d["q_pos"][:, 0], rope_dims=wl.rope_dims,
                    out=win[:, wl.window - 1:, :])
    # 2. indexer scan + top-k over all L visible entries
    kw = (dict(k_codes=d["k_codes"], k_scales=d["k_scales"]) if fp4 else dict(k_idx=d["k_idx"]))
    C.csa2_index_topk(C.CSA2_MODE_FULL, d["q_pos"], wl.k, q_idx=d["q_idx"], w=d["w"], m=1,
                      out_idx=out_idx, workspace=ws["index"], **kw)
    # 3. sparse attention over the selected entries + the window
    kvkw = (dict(kv_codes=d["kv_codes"], kv_scales=d["kv_scales"]) if fp4 else dict(kv=d["kv"]))
    C.csa2_sparse_attn(d["q"], d["q_pos"], out_idx, win=win, win_pos0=d["win_pos0"], n_win=wl.window,
                       sink=d["sink"], rope_dims=wl.rope_dims, out=out, workspace=ws["attn"], **kvkw)


# ---------------------------------------------------------------------------- timing
def time_steps(torch, step, steps, warmup):
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def per_kernel(C, torch, step, steps):
    C.csa2_profile_enable(True)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    recs = C.csa2_profile_collect(1 << 16)
    C.csa2_profile_enable(False)
    agg = {}
    for name, ms in recs:
        agg.setdefault(name, []).append(ms)
    return {k: {"launches": len(v), "avg_ms": float(np.mean(v))} for k, v in agg.items()}


def load_traffic(kernel, workload):
    """HBM traffic per launch measured with rocprofv3 counters, from the committed summary
    profiles/<kernel>_<workload>_traffic.txt, if it was taken on the current kernel source."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_traffic.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = (s.strip() for s in line.split("=", 1))
            vals[k] = v
    import hashlib

    h = hashlib.sha256()
    for name in vals.get("source", "").split(","):
        src = os.path.join(ROOT, "compressed_sparse_attention_gated_amd", "csrc", name.strip())
        if not name.strip() or not os.path.exists(src):
            return None
        h.update(open(src, "rb").read())
    if h.hexdigest()[:16] != vals.get("source_sha256_16"):
        return None
    try:
        return float(vals["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------------------- CPU baseline
def cpu_baseline_decode(torch, wl, d, budget_s, fp4=False):
    """The oracle, as it stands, on a bounded sample of the same decode workload: whole
    queries (scan + top-k + attention) until about `budget_s` seconds of oracle work."""
    sys.path.insert(0, ROOT)
    import oracle as O
    from oracle import formats as F

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    done, spent = 0, 0.0
    b = 0
    while spent < budget_s and b < wl.B:
        # host copies of one sequence (not timed)
        qi = d["q_idx"][b:b + 1].float().cpu().numpy().astype(np.float64)
        w = d["w"][b:b + 1].cpu().numpy().astype(np.float64)
        if fp4:
            ki = F.mxfp4_decode(d["k_codes"][b:b + 1].cpu().numpy(), d["k_scales"][b:b + 1].cpu().numpy())
        else:
            ki = d["k_idx"][b:b + 1].float().cpu().numpy().astype(np.float64)
        q = d["q"][b:b + 1].float().cpu().numpy().astype(np.float64)
        win = d["win"][b:b + 1].float().cpu().numpy().astype(np.float64)
        qp = d["q_pos"][b:b + 1].cpu().numpy()
        wp0 = d["win_pos0"][b:b + 1].cpu().numpy()
        sink = d["sink"].cpu().numpy().astype(np.float64)
        if fp4:
            kv_all = (d["kv_codes"][b:b + 1].cpu().numpy(), d["kv_scales"][b:b + 1].cpu().numpy())
        else:
            kv_all = d["kv"][b:b + 1].float().cpu().numpy()
        t0 = time.perf_counter()
        idx = O.index_topk_full(qi, w, ki, qp, 1, wl.k)
        sel = idx[0, 0][idx[0, 0] >= 0]
        kv_rows = (F.fp4_main_decode(kv_all[0][0, sel], kv_all[1][0, sel]) if fp4
                   else kv_all[0, sel].astype(np.float64))
        O.sparse_attn(q, qp, kv_rows[None], np.arange(len(sel))[None, None], win, wp0, wl.window, sink,
                      rope_dims=wl.rope_dims)
        spent += time.perf_counter() - t0
        done += 1
        b += 1
    return {"value": done / spent, "unit": "queries/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} of the {wl.B} decode queries (full scan of {wl.L} entries, top-{wl.k}, "
                      f"attention) by the fp64 numpy oracle, {spent:.1f} s"}


def copy_probe(torch, mib):
    """A plain device-to-device copy of known size: the scale for FETCH_SIZE / WRITE_SIZE."""
    torch.cuda.set_device(0)
    n = mib << 20
    x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(4):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 4}), flush=True)


# ---------------------------------------------------------------------------- main
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the hot path is measured on a single MI355X).", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_probe:
        copy_probe(torch, args.copy_probe)
        return
    sys.path.insert(0, ROOT)
    from compressed_sparse_attention_gated_amd import csa2 as C
    from compressed_sparse_attention_gated_amd import workloads as W

    C.lib()
    torch.cuda.set_device(0)
    wl = W.WORKLOADS[args.config]
    if args.config not in (2, 5):
        print("bench.py: only the decode workloads (--config 2, 5) are wired into the step yet",
              file=sys.stderr)
        sys.exit(2)
    fp4 = args.config == 5
    insts = [make_decode(torch, W, wl, 2000 + 17 * i, fp4=fp4) for i in range(2)]
    out_idx = torch.empty((wl.B, 1, wl.k), dtype=torch.int32, device="cuda")
    out = torch.empty((wl.B, 1, wl.H, wl.c), dtype=torch.bfloat16, device="cuda")
    d0 = insts[0]
    kw = (dict(k_codes=d0["k_codes"], k_scales=d0["k_scales"]) if fp4 else dict(k_idx=d0["k_idx"]))
    ws_idx = C.csa2_index_workspace_bytes(C.CSA2_MODE_FULL, d0["q_pos"], wl.k, q_idx=d0["q_idx"], w=d0["w"],
                                          m=1, out_idx=out_idx, **kw)
    kvkw = (dict(kv_codes=d0["kv_codes"], kv_scales=d0["kv_scales"]) if fp4 else dict(kv=d0["kv"]))
    ws_attn = C.csa2_attn_workspace_bytes(d0["q"], d0["q_pos"], out_idx, win=d0["win"], win_pos0=d0["win_pos0"],
                                          n_win=wl.window, sink=d0["sink"], rope_dims=wl.rope_dims, out=out, **kvkw)
    ws = {"index": torch.empty(max(ws_idx, 1), dtype=torch.uint8, device="cuda"),
          "attn": torch.empty(max(ws_attn, 1), dtype=torch.uint8, device="cuda")}

    def step(i):
        decode_step(C, torch, wl, insts[i % 2], ws, out_idx, out, fp4=fp4)

    ms = time_steps(torch, step, args.steps, args.warmup)
    kern = per_kernel(C, torch, step, args.steps)

    scan_name = next((n for n in kern if n.startswith("index_scan")), "index_scan_decode")
    attn_name = "attn_mfma_fp4" if fp4 else "attn_mfma"
    k_bytes = wl.d_I // 2 + wl.d_I // 32 if fp4 else wl.d_I * 2
    row_bytes = 288 if fp4 else wl.c * 2
    scan_bytes = wl.B * wl.L * k_bytes + wl.B * (wl.H_I * wl.d_I * 2 + wl.H_I * 4)
    attn_bytes = wl.B * (wl.k * row_bytes + wl.window * wl.c * 2 + 2 * wl.H * wl.c * 2 + wl.k * 4)
    scan_ms = kern.get(scan_name, {}).get("avg_ms", float("nan"))
    attn_ms = sum(v["avg_ms"] for k, v in kern.items() if k.startswith("attn_"))
    achieved = scan_bytes / (scan_ms * 1e-3) / 1e9
    workload_tag = "decode_full_b32_l65536" if not fp4 else "decode_fp4_b64_l262144"
    traffic = load_traffic(scan_name, workload_tag)
    stages = {k: {**v} for k, v in kern.items()}
    stages.setdefault(scan_name, {})["algorithmic_bytes"] = scan_bytes
    stages[scan_name]["GB_per_s"] = achieved
    stages[scan_name]["frac_hbm"] = achieved / HBM_PEAK_GBS
    if attn_name in stages:
        a_gbs = attn_bytes / (attn_ms * 1e-3) / 1e9
        stages[attn_name]["algorithmic_bytes"] = attn_bytes
        stages[attn_name]["GB_per_s_incl_combine"] = a_gbs
        stages[attn_name]["frac_hbm_incl_combine"] = a_gbs / HBM_PEAK_GBS
    value = wl.B / (ms * 1e-3)
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded on-device generator; random-init, no trained weights)",
        "config": {"workload": wl.name, "batch_queries": wl.B, "context_entries": wl.L, "m": wl.m,
                   "indexer": f"{wl.H_I}x{wl.d_I}", "top_k": wl.k, "window": wl.window,
                   "heads": wl.H, "head_dim": wl.c, "kv_cache": "fp4+e4m3" if fp4 else "bf16",
                   "indexer_k": "mxfp4" if fp4 else "bf16"},
        "scores_per_s": wl.B * wl.L / (scan_ms * 1e-3),
        "roofline": {"bound": "hbm", "kernel": scan_name, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic},
        "stages": stages,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_decode(torch, wl, insts[0], args.cpu_seconds, fp4=fp4)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
