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

  --config 3  the 32,768-token prefill (value in tokens/s; the scan's roofline is bf16 MFMA)
  --config 4  the hierarchical decoder group at 1M context (Full + pool + Reindex + 3 Reuse)
  --config 5  the FP4 / MXFP4 cache decode
  --config 6  the pages' HCA variant at decode (32 x 1,048,576 tokens -> 8,192 entries of
              m' = 128, dense attention; not one of the five reference workloads)
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
FP4_MFMA_PEAK_TFLOPS = 10100.0  # dense FP4 (and FP6) MFMA
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=2, choices=[2, 3, 4, 5, 6])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="bound of the oracle sample")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB (calibrates the HBM byte counters)")
    return p.parse_args()


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


def step_distribution(torch, step, reps):
    """Each of `reps` steps timed on its own between two events on the current stream:
    median, p10 and p90 in ms (the value itself comes from the back-to-back timing)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        step(i)
        b.record()
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return {"reps": reps, "median_ms": float(np.median(t)), "p10_ms": float(np.percentile(t, 10)),
            "p90_ms": float(np.percentile(t, 90))}


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
def _cores():
    try:
        from threadpoolctl import threadpool_info

        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def host_cpu():
    """The host the oracle runs on: logical CPUs this process may use, their total, the
    CPU model from /proc/cpuinfo."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:  # pragma: no cover
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count()
    return {"nproc": usable, "cpu_count": os.cpu_count(), "cpu_model": model}


def _h(t):
    return t.float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def _bf16_bits_to_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def cpu_baseline(torch, wl, d, budget_s):
    """The oracle on the host with numpy's BLAS threads as they are, then the same sample
    kind again with one BLAS thread (a shorter budget), reported as `single_thread`."""
    res = _cpu_baseline(torch, wl, d, budget_s)
    res.update(host_cpu())
    try:
        from threadpoolctl import threadpool_limits

        with threadpool_limits(limits=1):
            one = _cpu_baseline(torch, wl, d, max(budget_s / 3, min(2.0, budget_s)))
        res["single_thread"] = {"value": one["value"], "unit": one["unit"], "cores": 1, "sample": one["sample"]}
    except Exception as e:  # pragma: no cover
        res["single_thread"] = {"error": str(e)}
    return res


def _cpu_baseline(torch, wl, d, budget_s):
    """The oracle, as it stands, on a bounded sample of the same workload: whole queries
    (scan + top-k + attention; the whole layer group for the hierarchical workload) until
    about `budget_s` seconds of oracle work.  Host copies of the inputs are not timed."""
    sys.path.insert(0, ROOT)
    import oracle as O
    from oracle import formats as F

    if wl.kind == "prefill" and "e_oracle" not in d:
        # not timed: the oracle's own compressor output for the whole sequence (entries and
        # the projected indexer K, as the step's scan reads them), used by the sampled
        # tokens' scan and attention
        e, k = O.compress(_h(d["ca"][0]), _h(d["za"][0]), wl.m, rope_dims=wl.rope_dims, w_ik=_h(d["w_ik"]))
        d = dict(d, e_oracle=e, k_oracle=torch.from_numpy(k))
    done, spent = 0, 0.0
    kind = wl.kind
    # decode batches are short: the sample cycles over the batch's queries until the budget
    # is spent (each pass over a query repeats the same work)
    n_units = wl.n_tokens if kind == "prefill" else 64 * wl.B
    rs = np.random.default_rng(0)
    while spent < budget_s and done < n_units:
        if kind == "prefill":
            # one query token at a random position over the compressed entries (the
            # compressor's share, one entry per m tokens, is timed with it)
            t = int(rs.integers(wl.n_tokens // 2, wl.n_tokens))
            qi, w, q = _h(d["q_idx"][0, t]), _h(d["w"][0, t]), _h(d["q"][0, t])
            blk = slice(wl.m * (t // wl.m), wl.m * (t // wl.m) + wl.m)
            ca, za, w_ik = _h(d["ca"][0, blk]), _h(d["za"][0, blk]), _h(d["w_ik"])
            kidx = _h(d["k_oracle"]) if "k_oracle" in d else None
            win_src = _h(d["win_src"][0, max(0, t - wl.window + 1):t + 1])
            sink = _h(d["sink"])
            entries = d.get("e_oracle")
            t0 = time.perf_counter()
            O.compress(ca, za, wl.m, rope_dims=wl.rope_dims, pos0=blk.start, w_ik=w_ik)
            wr, _ = O.compress(win_src, win_src, 1, rope_dims=wl.rope_dims, pos0=max(0, t - wl.window + 1))
            nv = O.n_visible(t, wl.n_tokens // wl.m, wl.m)
            idx = O.topk_indices(O.indexer_scores(qi, w, kidx, nv), wl.k)
            sel = idx[idx >= 0]
            O.sparse_attn(q[None, None], np.array([[t]]), entries[sel][None], np.arange(len(sel))[None, None],
                          wr[None], [max(0, t - wl.window + 1)], wl.window, sink, rope_dims=wl.rope_dims)
        elif kind == "hca_decode":
            b = done % wl.B
            q, win, sink = _h(d["q"][b, 0]), _h(d["win"][b]), _h(d["sink"])
            kv_h = d["kv"][b].view(torch.int16).cpu().numpy().view(np.uint16)  # raw bits, not timed
            L = wl.L
            t0 = time.perf_counter()
            rows = _bf16_bits_to_f64(kv_h)
            O.dense_attn(q[None, None], np.array([[L]]), rows[None], wl.m, win=win[None], win_pos0=[L - wl.window + 1],
                         window=wl.window, sink=sink, rope_dims=wl.rope_dims)
        else:
            b = done % wl.B
            hier = kind == "hier"
            layers = d["layers"] if hier else [d]
            fp4 = kind == "decode_fp4"
            if fp4:
                ki = F.mxfp4_decode(_h(d["k_codes"][b]), _h(d["k_scales"][b]))
            else:
                ki = _h(d["k_idx"][b])
            qs = [(_h(e["q_idx"][b, 0]) if "q_idx" in e else None, _h(e["w"][b, 0]) if "w" in e else None,
                   _h(e["q"][b, 0]), _h(e["win"][b]), _h(e["sink"])) for e in layers]
            # this query's cache rows as raw bits on the host (not timed); the oracle's gather
            # and decode of the selected rows run on the host inside the timed region
            if fp4:
                kv_h = (d["kv_codes"][b].cpu().numpy(), d["kv_scales"][b].cpu().numpy())
            else:
                kv_h = d["kv"][b].view(torch.int16).cpu().numpy().view(np.uint16)
            L = wl.L
            t0 = time.perf_counter()
            s = O.indexer_scores(qs[0][0], qs[0][1], ki, L)
            sels = [O.topk_indices(s, wl.k)]
            if hier:
                pool = O.hier_candidates(O.block_max(s, wl.block), L, n_keep=wl.n_keep_blocks, block=wl.block)
                sels.append(O.reindex_topk(qs[1][0], qs[1][1], ki, pool, wl.k))
                sels += [sels[1]] * (len(layers) - 2)
            for (qi, w, q, win, sink), idx in zip(qs, sels):
                sel = idx[idx >= 0]
                if fp4:
                    rows = F.fp4_main_decode(kv_h[0][sel], kv_h[1][sel])
                else:
                    rows = _bf16_bits_to_f64(kv_h[sel])
                O.sparse_attn(q[None, None], np.array([[L]]), rows[None], np.arange(len(sel))[None, None],
                              win[None], [L - wl.window + 1], wl.window, sink, rope_dims=wl.rope_dims)
        spent += time.perf_counter() - t0
        done += 1
    unit = "tokens/s" if kind == "prefill" else "queries/s"
    what = {"prefill": f"{done} query tokens of the {wl.n_tokens}-token prefill (their compressor block and "
                       f"window rows, causal scan, top-{wl.k}, attention)",
            "hca_decode": f"{done} query passes over the batch's {wl.B} queries (dense attention over "
                          f"{wl.L // wl.m} entries plus the window)",
            "hier": f"{done} query passes over the batch's {wl.B} queries, each through the whole 5-layer group "
                    f"(full scan of {wl.L}, pool, Reindex, 5 attentions)",
            }.get(kind, f"{done} query passes over the batch's {wl.B} decode queries (full scan of {wl.L} entries, "
                        f"top-{wl.k}, attention)")
    return {"value": done / spent, "unit": unit, "cores": int(_cores()), "kind": "oracle",
            "sample": f"{what} by the fp64 numpy oracle on the host, {spent:.1f} s; each query's inputs are "
                      "copied to the host before its timed region"}


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
TAGS = {2: "decode_full_b32_l65536", 3: "prefill_n32768", 4: "hier_b8_l1048576", 5: "decode_fp4_b64_l262144",
        6: "hca_decode_b32_l1048576"}


def scan_work(wl):
    """Algorithmic bytes and flops of one indexer-scan launch (the Full layer's)."""
    fp4 = wl.kind == "decode_fp4"
    k_bytes = wl.d_I // 2 + wl.d_I // 32 if fp4 else wl.d_I * 2
    q_bytes = wl.H_I * wl.d_I * 2 + wl.H_I * 4
    if wl.kind == "prefill":
        ne = wl.n_tokens // wl.m
        pairs = sum(min(ne, t // wl.m) for t in range(wl.n_tokens))
        return ne * k_bytes + wl.n_tokens * (q_bytes + wl.k * 4), 2.0 * wl.H_I * wl.d_I * pairs, pairs
    pairs = wl.B * wl.L
    return pairs * k_bytes + wl.B * q_bytes, 2.0 * wl.H_I * wl.d_I * pairs, pairs


def attn_bytes(wl):
    row_bytes = 288 if wl.kind == "decode_fp4" else wl.c * 2
    queries = wl.n_tokens if wl.kind == "prefill" else wl.B
    if wl.kind == "hca_decode":  # every visible entry, no index list
        return queries * ((wl.L // wl.m) * row_bytes + wl.window * wl.c * 2 + 2 * wl.H * wl.c * 2)
    return queries * (wl.k * row_bytes + wl.window * wl.c * 2 + 2 * wl.H * wl.c * 2 + wl.k * 4)


def _mxfp4_exact(torch, x):
    """Integer values in [-3, 3] as MXFP4 planes with scale byte 127 (exact: 0, 1, 2, 3 are
    E2M1 codes 0, 2, 4, 5), or None if x holds anything else."""
    x = x.float()
    if not bool(((x == x.round()) & (x.abs() <= 3)).all()):
        return None
    lut = torch.tensor([0, 2, 4, 5], dtype=torch.uint8, device=x.device)
    code = lut[x.abs().long()] | ((x < 0).to(torch.uint8) << 3)
    codes = (code[..., 0::2] | (code[..., 1::2] << 4)).contiguous()  # dim 2i in the low nibble
    scales = torch.full((*x.shape[:-1], x.shape[-1] // 32), 127, dtype=torch.uint8, device=x.device)
    return codes, scales


def mxfp4_query_stage(torch, C, wl, d, idx_ref, reps=20, keys_too=False):
    """The Full layer's index call with q_I in MXFP4 as well (the indexer QK path in FP4 on
    both sides, scaled FP4 x FP4 MFMA); with keys_too the bf16 K_I is encoded as MXFP4 too.
    The workloads' integer q_I and K_I values are exact in E2M1 (scale byte 127), so the call
    must return the step's own indices; its scan and merge are timed per launch like the
    step's."""
    qe = _mxfp4_exact(torch, d["q_idx"])
    if qe is None:
        return {"skipped": "q_I is not exactly representable in E2M1"}
    if keys_too:
        ke = _mxfp4_exact(torch, d["k_idx"])
        if ke is None:
            return {"skipped": "K_I is not exactly representable in E2M1"}
    else:
        ke = (d["k_codes"], d["k_scales"])
    out = torch.empty_like(idx_ref)
    kw = dict(q_idx=qe[0], q_scales=qe[1], w=d["w"], m=wl.m, k_codes=ke[0], k_scales=ke[1], out_idx=out)
    ws = torch.empty(max(1, C.csa2_index_workspace_bytes(C.CSA2_MODE_FULL, d["q_pos"], wl.k, **kw)),
                     dtype=torch.uint8, device=out.device)

    def call(_i):
        C.csa2_index_topk(C.CSA2_MODE_FULL, d["q_pos"], wl.k, workspace=ws, **kw)

    call(0)
    torch.cuda.synchronize()
    same = bool(torch.equal(out, idx_ref))
    kern = per_kernel(C, torch, call, reps)
    scan_ms = kern["index_scan_select"]["avg_ms"]
    merge_ms = kern.get("topk_merge", {"avg_ms": 0.0})["avg_ms"]
    sbytes = wl.B * wl.L * (wl.d_I // 2 + wl.d_I // 32) + wl.B * wl.H_I * (wl.d_I // 2 + wl.d_I // 32 + 4)
    flops = 2.0 * wl.H_I * wl.d_I * wl.B * wl.L
    what = ("index FULL with the step's q_I and K_I stored as MXFP4 (exact for its integers; "
            "scaled FP4 x FP4 MFMA)" if keys_too else "index FULL with MXFP4 q_I and K_I (scaled FP4 x FP4 MFMA)")
    return {"what": what, "same_indices": same,
            "scan_us": scan_ms * 1e3, "merge_us": merge_ms * 1e3, "algorithmic_bytes": sbytes,
            "frac_hbm": sbytes / (scan_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "flops": flops,
            "frac_fp4_mfma": flops / (scan_ms * 1e-3) / 1e12 / FP4_MFMA_PEAK_TFLOPS}


def write_path_stage(torch, C, wl, d, reps=20):
    """The write path into the 4-bit decode cache (csa2_compress with FP4 entry planes and
    the MXFP4 indexer-K projection), timed with HIP events per launch.  Decode workloads
    append one entry per sequence (m = 1: the new token); the prefill writes every entry of
    its sequence (m = 2).  Not part of the step: the step's cache is generated directly."""
    dev = d["q"].device
    g = torch.Generator(device=dev)
    g.manual_seed(99)
    d_I = 128
    w_ik = (torch.randn((wl.c, d_I), generator=g, device=dev) * wl.c ** -0.5).to(torch.bfloat16)
    if wl.kind == "prefill":
        ca, za, m, pos0 = d["ca"], d["za"], wl.m, None
        what = f"all {wl.n_tokens // wl.m} entries of the {wl.n_tokens}-token sequence (m={wl.m})"
    else:
        ca, za, m, pos0 = d["c_new"], d["z_new"], 1, d["q_pos"][:, 0]
        what = f"one new entry for each of the {wl.B} sequences (m=1), at its cache row"
    B, n, c = ca.shape
    ne = n // m
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8, device=dev)  # noqa: E731
    planes = dict(out_codes=u8(B, ne, c // 2), out_scales=u8(B, ne, c // 16), ik_codes=u8(B, ne, d_I // 2),
                  ik_scales=u8(B, ne, d_I // 32))

    def run():
        C.csa2_compress(ca, za, m, pos0=pos0, rope_dims=wl.rope_dims, w_ik=w_ik, plain_out=False, **planes)

    run()
    torch.cuda.synchronize()
    C.csa2_profile_enable(True)
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    recs = C.csa2_profile_collect(1 << 12)
    C.csa2_profile_enable(False)
    us = float(np.mean([ms for _, ms in recs])) * 1e3
    nbytes = B * n * c * 2 * 2 + c * d_I * 2 + B * ne * (c // 2 + c // 16 + d_I // 2 + d_I // 32)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": "compress", "what": what + ": RMSNorm, RoPE, K_I projection, FP4 + MXFP4 planes",
            "avg_us": us, "algorithmic_bytes": nbytes, "GB_per_s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS}


def out_proj_stage(torch, C, wl, reps=10):
    """The grouped output projection after the attention (csa2_out_proj), at the pages'
    V4-Flash shape (64 heads x 512 -> 8 groups of 1,024 -> 4,096), for the step's query
    tokens; random bf16 weights.  Not part of the step (the pages put it after the path)."""
    dev = "cuda"
    M = wl.n_tokens if wl.kind == "prefill" else wl.B
    g_, d_g, d = 8, 1024, 4096
    kg = wl.H * wl.c // g_
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    o = torch.randn((M, wl.H, wl.c), generator=gen, device=dev).to(torch.bfloat16)
    w1 = (torch.randn((g_, d_g, kg), generator=gen, device=dev) * kg ** -0.5).to(torch.bfloat16)
    w2 = (torch.randn((d, g_ * d_g), generator=gen, device=dev) * (g_ * d_g) ** -0.5).to(torch.bfloat16)
    mid = torch.empty((M, g_ * d_g), dtype=torch.bfloat16, device=dev)
    out = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    C.csa2_out_proj(o, w1, w2, mid=mid, out=out)
    torch.cuda.synchronize()
    C.csa2_profile_enable(True)
    for _ in range(reps):
        C.csa2_out_proj(o, w1, w2, mid=mid, out=out)
    torch.cuda.synchronize()
    recs = C.csa2_profile_collect(1 << 12)
    C.csa2_profile_enable(False)
    per = {}
    for n, ms in recs:
        per.setdefault(n, []).append(ms)
    us = sum(float(np.mean(v)) for v in per.values()) * 1e3
    flops = 2.0 * M * (wl.H * wl.c * d_g + g_ * d_g * d)
    nbytes = 2 * (w1.numel() + w2.numel() + o.numel() + 2 * mid.numel() + out.numel())
    res = {"kernels": {k: float(np.mean(v)) * 1e3 for k, v in per.items()}, "tokens": M,
           "shape": f"{wl.H}x{wl.c} -> {g_} groups x {d_g} -> {d}", "avg_us": us, "flops": flops,
           "algorithmic_bytes": nbytes, "TFLOP_per_s": flops / (us * 1e-6) / 1e12,
           "GB_per_s": nbytes / (us * 1e-6) / 1e9}
    if wl.kind == "prefill":
        res["frac_mfma"] = res["TFLOP_per_s"] / BF16_MFMA_PEAK_TFLOPS
    else:
        res["frac_hbm"] = res["GB_per_s"] / HBM_PEAK_GBS
    return res


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
    from compressed_sparse_attention_gated_amd import steps as S
    from compressed_sparse_attention_gated_amd import workloads as W

    C.lib()
    torch.cuda.set_device(0)
    wl = W.WORKLOADS[args.config]
    make, Step = {"decode": (W.decode_inputs, S.DecodeStep), "decode_fp4": (W.decode_inputs, S.DecodeStep),
                  "hier": (W.hier_inputs, S.HierStep), "prefill": (W.prefill_inputs, S.PrefillStep),
                  "hca_decode": (W.hca_inputs, S.HcaDecodeStep)}[wl.kind]
    # two independent input instances alternate, so no step finds its rows cache-resident
    n_inst = 2
    insts = [make(wl, 2000 + 17 * i) for i in range(n_inst)]
    if wl.kind == "decode_fp4":
        # the 4-bit cache as the write path stores it: N(0,1) source rows through csa2_compress
        # (RMSNorm, RoPE, FP4 + E4M3 planes) and integer K_I as MXFP4, tiled over the context
        for i, d in enumerate(insts):
            d["kv_codes"], d["kv_scales"], d["k_codes"], d["k_scales"] = S.written_fp4_cache(wl, 5000 + i)
    runner = Step(wl, insts[0])

    def step(i):
        runner.run(insts[i % n_inst])

    ms = time_steps(torch, step, args.steps, args.warmup)
    dist = step_distribution(torch, step, max(args.steps, 50))
    kern = per_kernel(C, torch, step, args.steps)
    launches_per_step = {k: v["launches"] / args.steps for k, v in kern.items()}

    stages = {k: dict(v) for k, v in kern.items()}
    hca = wl.kind == "hca_decode"
    if not hca:
        # the Full layer's scan: the fused scan + chunk top-k at decode, the shared-tile scan at prefill
        scan_name = "index_scan_prefill" if wl.kind == "prefill" else "index_scan_select"
        if scan_name not in kern:
            scan_name = next(n for n in kern if n.startswith("index_scan"))
        sb, sf, pairs = scan_work(wl)
        scan_ms = kern[scan_name]["avg_ms"]
    if hca:
        # no indexer: the dense attention is the path; its row-reading kernel is the roofline
        ab_in = wl.B * ((wl.L // wl.m) * wl.c * 2 + wl.window * wl.c * 2 + wl.H * wl.c * 2)
        a_ms = kern["attn_mfma"]["avg_ms"]
        achieved = ab_in / (a_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "attn_mfma", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic("attn_mfma", TAGS[args.config]),
                "bytes_per_launch": ab_in}
    elif wl.kind == "prefill":
        achieved = sf / (scan_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": scan_name, "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS,
                "traffic": load_traffic(scan_name, TAGS[args.config]),
                "flops_per_launch": sf}
    else:
        achieved = sb / (scan_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": scan_name, "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": load_traffic(scan_name, TAGS[args.config]),
                "bytes_per_launch": sb}
    attn_ms = sum(v["avg_ms"] * launches_per_step[k] for k, v in kern.items() if k.startswith("attn_"))
    n_attn = 5 if wl.kind == "hier" else 1
    ab = attn_bytes(wl) * n_attn
    if wl.kind in ("decode", "decode_fp4", "hier"):
        # the whole step against HBM: the Full layer's scan and every attention (top-k keeps
        # its scores on chip; its index lists are counted with the attention)
        stages["step_total"] = {"algorithmic_bytes": sb + ab, "ms_per_step": ms,
                                "frac_hbm": (sb + ab) / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    stages["attention_total"] = {"ms_per_step": attn_ms, "algorithmic_bytes": ab,
                                 "GB_per_s": ab / (attn_ms * 1e-3) / 1e9,
                                 "frac_hbm": ab / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    # the two stated targets beside what this run measured: decode sparse attention at
    # >= 60 % of HBM, the prefill indexer scan at >= 50 % of bf16 MFMA
    if wl.kind == "prefill":
        roof["target"] = {"what": "prefill indexer scan, fraction of bf16 MFMA peak", "frac": roof["frac"],
                          "target_frac": 0.5, "met": roof["frac"] >= 0.5}
    elif not hca:
        fa = stages["attention_total"]["frac_hbm"]
        roof["target"] = {"what": "decode sparse attention (all attention launches of the step), fraction of HBM "
                                  "peak", "frac": fa, "target_frac": 0.6, "met": fa >= 0.6,
                          "us_per_attention": attn_ms * 1e3 / n_attn}
    if wl.kind in ("decode", "decode_fp4"):
        # FP4 on the indexer QK path where the inputs allow it: MXFP4 queries against the FP4
        # cache's MXFP4 keys; for the bf16-key decode, its integer keys and queries as MXFP4
        # (a context figure beside the step, which keeps its bf16 keys)
        runner.run(insts[0])
        torch.cuda.synchronize()
        name = "mxfp4_query" if wl.kind == "decode_fp4" else "mxfp4_indexer"
        stages[name] = mxfp4_query_stage(torch, C, wl, insts[0], runner.idx.clone(), keys_too=wl.kind == "decode")
    if wl.kind not in ("hier", "hca_decode"):
        stages["write_path"] = write_path_stage(torch, C, wl, insts[0])
    if wl.kind != "hier":
        stages["out_proj"] = out_proj_stage(torch, C, wl)
    prefill = wl.kind == "prefill"
    units = wl.n_tokens if prefill else wl.B
    value = units / (ms * 1e-3)
    cfg = {"workload": wl.name}
    if prefill:
        cfg.update({"tokens": wl.n_tokens, "m": wl.m, "entries": wl.n_tokens // wl.m})
    elif hca:
        cfg.update({"batch_queries": wl.B, "context_tokens": wl.L, "m_prime": wl.m, "entries": wl.L // wl.m})
    else:
        cfg.update({"batch_queries": wl.B, "context_entries": wl.L, "m": wl.m})
    if hca:
        cfg.update({"window": wl.window, "heads": wl.H, "head_dim": wl.c, "kv_cache": "bf16",
                    "attention": "dense over every visible entry (no indexer)"})
    else:
        cfg.update({"indexer": f"{wl.H_I}x{wl.d_I}", "top_k": wl.k, "window": wl.window, "heads": wl.H,
                    "head_dim": wl.c, "kv_cache": "fp4+e4m3" if wl.kind == "decode_fp4" else "bf16",
                    "indexer_k": "mxfp4" if wl.kind == "decode_fp4" else "bf16"})
    if wl.kind == "hier":
        cfg["layers"] = "Full (scan, top-512, block max) + pool (2048 blocks) + Reindex + 3 Reuse"
    res = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s" if prefill else "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded on-device generator; random-init, no trained weights)",
        "config": cfg,
        "step_ms": dist,
        "scores_per_s": None if hca else pairs / (scan_ms * 1e-3),
        "roofline": roof,
        "stages": stages,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(torch, wl, insts[0], args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
