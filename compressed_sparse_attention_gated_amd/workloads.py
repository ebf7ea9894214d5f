"""Seeded synthetic inputs for the CSA2 hot path.

This module only draws random numbers in the shapes, dtypes and value
distributions of the five workloads; it holds none of the method's arithmetic
(no pooling, scoring, selection, attention or quantisation).  Both the tests'
oracle side and the HIP side consume the tensors it returns.

Two backends with the same call signature:
  * ``device=None``  -> numpy ``PCG64(seed)`` arrays (small cases, CPU oracle runs);
  * ``device="cuda"`` -> torch tensors drawn on the device by a seeded
    ``torch.Generator`` (full-size workloads, which would take minutes on the host).

Integer-valued indexer inputs and power-of-two head weights keep every index
score exact in fp32, so top-k indices can be compared bit for bit.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# ----------------------------------------------------------------- workloads
@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "prefill" | "decode" | "hier" | "decode_fp4"
    B: int = 1
    n_tokens: int = 0  # prefill: tokens of the sequence
    L: int = 0  # decode: cached entries per sequence (query position t = L)
    c: int = 512
    m: int = 1
    overlap: bool = False
    H_I: int = 64
    d_I: int = 128
    w_values: tuple = (1.0, -1.0, 0.5, -0.5, 0.25, -0.25)
    k: int = 512
    window: int = 128
    H: int = 64
    rope_dims: int = 64
    io_dtype: str = "bf16"
    sink_std: float = 1.0  # 0 -> sink logit fixed at 0
    n_keep_blocks: int = 2048
    block: int = 8
    extra: dict = field(default_factory=dict)


WORKLOADS = {
    1: Workload("tiny CSA prefill, n=256, c=64, m=2 overlap, 4x32 indexer, top-16, 8 heads",
                "prefill", B=1, n_tokens=256, c=64, m=2, overlap=True, H_I=4, d_I=32,
                w_values=(1.0, -1.0, 0.5, -0.5), k=16, window=16, H=8, rope_dims=16,
                io_dtype="f32", sink_std=0.0, extra={"bias_std": 0.1}),
    2: Workload("decoder Full layer decode, B=32 x 65,536 ctx, m=1, bf16 cache",
                "decode", B=32, L=65536, c=512, m=1),
    3: Workload("encoder Full layer prefill, 32,768 tokens, m=2 -> 16,384 entries",
                "prefill", B=1, n_tokens=32768, c=512, m=2, extra={"w_ik": True}),
    4: Workload("hierarchical decoder group, B=8 x 1,048,576 ctx, L20 Full + L24 Reindex + L25-27 Reuse",
                "hier", B=8, L=1048576, c=512, m=1),
    5: Workload("FP4 cache decode, B=64 x 262,144 ctx, FP4 main KV + MXFP4 indexer K",
                "decode_fp4", B=64, L=262144, c=512, m=1),
    # the pages' HCA variant (not one of the five workloads above): m' = 128 entries read
    # densely, no indexer; L counts tokens, so each query sees L / 128 entries
    6: Workload("HCA decode layer, B=32 x 1,048,576 ctx, m'=128 -> 8,192 entries, dense attention",
                "hca_decode", B=32, L=1048576, c=512, m=128),
}


# ----------------------------------------------------------------- RNG backends
class _NumpyRNG:
    def __init__(self, seed):
        self.g = np.random.Generator(np.random.PCG64(seed))

    def normal(self, shape, std=1.0, dtype="f32"):
        x = self.g.standard_normal(shape) * std
        return _to_np_dtype(x, dtype)

    def ints(self, shape, lo, hi, dtype="bf16"):
        return _to_np_dtype(self.g.integers(lo, hi + 1, size=shape).astype(np.float64), dtype)

    def choice(self, shape, values, dtype="f32"):
        v = np.asarray(values, dtype=np.float64)
        return _to_np_dtype(v[self.g.integers(0, len(v), size=shape)], dtype)

    def bytes(self, shape, lo=0, hi=255):
        return self.g.integers(lo, hi + 1, size=shape).astype(np.uint8)

    def byte_choice(self, shape, values):
        v = np.asarray(values, dtype=np.uint8)
        return v[self.g.integers(0, len(v), size=shape)]

    def sorted_sample(self, n, k):
        """k distinct ascending integers from [0, n) (k <= n)."""
        return np.sort(self.g.choice(n, size=k, replace=False)).astype(np.int32)


class _TorchRNG:
    def __init__(self, seed, device):
        import torch

        self.torch = torch
        self.device = device
        self.g = torch.Generator(device=device)
        self.g.manual_seed(seed)

    def _dt(self, dtype):
        t = self.torch
        return {"f32": t.float32, "bf16": t.bfloat16, "f64": t.float64}[dtype]

    def normal(self, shape, std=1.0, dtype="f32"):
        t = self.torch
        x = t.randn(shape, generator=self.g, device=self.device, dtype=t.float32)
        if std != 1.0:
            x.mul_(std)
        return x.to(self._dt(dtype))

    def ints(self, shape, lo, hi, dtype="bf16"):
        t = self.torch
        x = t.randint(lo, hi + 1, shape, generator=self.g, device=self.device, dtype=t.int32)
        return x.to(self._dt(dtype))

    def choice(self, shape, values, dtype="f32"):
        t = self.torch
        v = t.tensor(values, dtype=t.float32, device=self.device)
        i = t.randint(0, len(values), shape, generator=self.g, device=self.device)
        return v[i].to(self._dt(dtype))

    def bytes(self, shape, lo=0, hi=255):
        t = self.torch
        return t.randint(lo, hi + 1, shape, generator=self.g, device=self.device,
                         dtype=t.int32).to(t.uint8)

    def byte_choice(self, shape, values):
        t = self.torch
        v = t.tensor(values, dtype=t.uint8, device=self.device)
        i = t.randint(0, len(values), shape, generator=self.g, device=self.device)
        return v[i]

    def sorted_sample(self, n, k):
        t = self.torch
        p = t.randperm(n, generator=self.g, device=self.device)[:k]
        return t.sort(p).values.to(t.int32)


def rng(seed, device=None):
    return _NumpyRNG(seed) if device is None else _TorchRNG(seed, device)


def _to_np_dtype(x, dtype):
    if dtype == "f32":
        return x.astype(np.float32)
    if dtype == "f64":
        return x.astype(np.float64)
    if dtype == "bf16":
        # stored as float32 holding a bf16-representable value (truncate-free:
        # round to nearest even on the top 16 bits); callers move it to torch.bfloat16
        f = x.astype(np.float32)
        u = f.view(np.uint32).astype(np.uint64)
        u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
        return u.astype(np.uint32).view(np.float32)
    raise ValueError(dtype)


# ----------------------------------------------------------------- stage inputs
# E4M3 scale bytes in [2^-4, 1] (exponent fields 3..7) - the range amax/6 of
# 16 N(0,1) values falls in - and E8M0 bytes 126/127 (scales 1/2 and 1).
FP4_SCALE_BYTES = tuple(range(0x18, 0x39))
MX_SCALE_BYTES = (126, 127)


def compress_inputs(g, n, c, m, *, overlap=False, dtype="bf16", bias_std=0.0,
                    d_I=0, B=1):
    """C^a, Z^a (and C^b, Z^b if overlap) ~ N(0,1) [B, n, c]; position biases
    ~ N(0, bias_std^2) [m, c] when bias_std > 0; W_ik ~ N(0, 1/c) [c, d_I] if d_I."""
    d = {"ca": g.normal((B, n, c), dtype=dtype), "za": g.normal((B, n, c), dtype=dtype)}
    if overlap:
        d["cb"] = g.normal((B, n, c), dtype=dtype)
        d["zb"] = g.normal((B, n, c), dtype=dtype)
    if bias_std > 0:
        d["ba"] = g.normal((m, c), std=bias_std, dtype="f32")
        if overlap:
            d["bb"] = g.normal((m, c), std=bias_std, dtype="f32")
    if d_I:
        d["w_ik"] = g.normal((c, d_I), std=float(c) ** -0.5, dtype=dtype)
    return d


def indexer_inputs(g, B, T, N, H_I, d_I, w_values, *, k_format="bf16", q_format="bf16", lo=-3, hi=3):
    """q_I ints U{lo..hi} [B, T, H_I, d_I] (bf16), or with q_format "mxfp4" the planes
    q_codes [B, T, H_I, d_I/2] (uniform random bytes) and q_scales [B, T, H_I, d_I/32] in
    {126, 127}; w from w_values [B, T, H_I] (f32); K_I ints U{lo..hi} [B, N, d_I] (bf16),
    or MXFP4 planes: codes [B, N, d_I/2] uniform random bytes, scales [B, N, d_I/32] in
    {126, 127}."""
    if q_format == "bf16":
        d = {"q_idx": g.ints((B, T, H_I, d_I), lo, hi, dtype="bf16")}
    else:
        d = {"q_codes": g.bytes((B, T, H_I, d_I // 2)),
             "q_scales": g.byte_choice((B, T, H_I, d_I // 32), MX_SCALE_BYTES)}
    d["w"] = g.choice((B, T, H_I), w_values, dtype="f32")
    if k_format == "bf16":
        d["k_idx"] = g.ints((B, N, d_I), lo, hi, dtype="bf16")
    else:
        d["k_codes"] = g.bytes((B, N, d_I // 2))
        d["k_scales"] = g.byte_choice((B, N, d_I // 32), MX_SCALE_BYTES)
    return d


def attn_inputs(g, B, T, N, H, c, *, Lw=128, io_dtype="bf16", kv_format="bf16",
                sink_std=1.0):
    """q ~ N(0,1) [B, T, H, c]; main KV rows ~ N(0,1) [B, N, c] (or FP4 planes:
    codes [B, N, c/2] random bytes, E4M3 scales [B, N, c/16] in [2^-4, 1]);
    window rows ~ N(0,1) [B, Lw, c]; sink ~ N(0, sink_std^2) [H] (0 if sink_std == 0)."""
    d = {"q": g.normal((B, T, H, c), dtype=io_dtype)}
    if kv_format == "fp4":
        d["kv_codes"] = g.bytes((B, N, c // 2))
        d["kv_scales"] = g.byte_choice((B, N, c // 16), FP4_SCALE_BYTES)
    else:
        d["kv"] = g.normal((B, N, c), dtype=io_dtype)
    d["win"] = g.normal((B, Lw, c), dtype=io_dtype)
    d["sink"] = (g.normal((H,), std=sink_std, dtype="f32") if sink_std > 0
                 else g.normal((H,), dtype="f32") * 0)
    return d


def random_topk_lists(g, B, T, n_vis, k):
    """Synthetic index lists: for each query, min(k, n_vis) distinct ascending entry
    ids from [0, n_vis), -1 padded to k.  n_vis is an int or an array [B, T]."""
    nv = np.broadcast_to(np.asarray(n_vis), (B, T))
    out = np.full((B, T, k), -1, dtype=np.int32)
    for b in range(B):
        for t in range(T):
            kk = int(min(k, nv[b, t]))
            if kk:
                s = g.sorted_sample(int(nv[b, t]), kk)
                out[b, t, :kk] = np.asarray(s.cpu() if hasattr(s, "cpu") else s)
    return out


# ----------------------------------------------------------------- whole-step inputs
def decode_inputs(wl, seed, device="cuda"):
    """One instance of a decode workload (indexer + attention inputs, the new token's
    compressor input, positions) for a step of `wl` (kind "decode" or "decode_fp4").
    Every query sits at position t = L, so all L cached entries are visible."""
    import torch

    g = rng(seed, device=device)
    B, L, c, H = wl.B, wl.L, wl.c, wl.H
    fp4 = wl.kind == "decode_fp4"
    d = dict(indexer_inputs(g, B, 1, L, wl.H_I, wl.d_I, wl.w_values, k_format="mxfp4" if fp4 else "bf16"))
    d.update(attn_inputs(g, B, 1, L, H, c, Lw=wl.window, kv_format="fp4" if fp4 else "bf16"))
    d["q_pos"] = torch.full((B, 1), L, dtype=torch.int32, device=device)
    d["win_pos0"] = torch.full((B,), L - wl.window + 1, dtype=torch.int32, device=device)
    d["c_new"] = g.normal((B, 1, c), dtype="bf16")
    d["z_new"] = g.normal((B, 1, c), dtype="bf16")
    return d


def hca_inputs(wl, seed, device="cuda"):
    """One HCA decode instance: the compressed cache [B, L/m', c] ~ N(0,1) (bf16), the query
    ~ N(0,1), the 128-token window, the sink, the new token's compressor input; every query
    sits at t = L, so all L/m' entries are visible."""
    import torch

    g = rng(seed, device=device)
    B, L, c, H = wl.B, wl.L, wl.c, wl.H
    d = dict(attn_inputs(g, B, 1, L // wl.m, H, c, Lw=wl.window))
    d["q_pos"] = torch.full((B, 1), L, dtype=torch.int32, device=device)
    d["win_pos0"] = torch.full((B,), L - wl.window + 1, dtype=torch.int32, device=device)
    d["c_new"] = g.normal((B, 1, c), dtype="bf16")
    d["z_new"] = g.normal((B, 1, c), dtype="bf16")
    return d


def hier_inputs(wl, seed, device="cuda", n_layers=5):
    """The hierarchical decoder group: one shared main KV and indexer K, then per layer
    (Full, Reindex, Reuse x3) its own indexer query and weights (the first two layers),
    attention query, 128-token window and sink.  Queries sit at t = L."""
    import torch

    g = rng(seed, device=device)
    B, L, c, H = wl.B, wl.L, wl.c, wl.H
    d = {"kv": g.normal((B, L, c), dtype="bf16"),
         "k_idx": g.ints((B, L, wl.d_I), -3, 3, dtype="bf16")}
    d["layers"] = []
    for layer in range(n_layers):
        e = {}
        if layer < 2:
            e["q_idx"] = g.ints((B, 1, wl.H_I, wl.d_I), -3, 3, dtype="bf16")
            e["w"] = g.choice((B, 1, wl.H_I), wl.w_values, dtype="f32")
        e["q"] = g.normal((B, 1, H, c), dtype="bf16")
        e["win"] = g.normal((B, wl.window, c), dtype="bf16")
        e["sink"] = g.normal((H,), dtype="f32")
        d["layers"].append(e)
    d["q_pos"] = torch.full((B, 1), L, dtype=torch.int32, device=device)
    d["win_pos0"] = torch.full((B,), L - wl.window + 1, dtype=torch.int32, device=device)
    return d


def prefill_inputs(wl, seed, device="cuda"):
    """One prefill sequence: compressor input C, Z [1, n, c] ~ N(0,1), W_IK ~ N(0, 1/c),
    the per-token window source [1, n, c] ~ N(0,1), indexer queries (integers) and head
    weights, attention queries ~ N(0,1) and sink ~ N(0,1); query t sits at position t."""
    import torch

    g = rng(seed, device=device)
    n, c, H = wl.n_tokens, wl.c, wl.H
    d = compress_inputs(g, n, c, wl.m, dtype="bf16", d_I=wl.d_I)
    d["win_src"] = g.normal((1, n, c), dtype="bf16")
    d["q_idx"] = g.ints((1, n, wl.H_I, wl.d_I), -3, 3, dtype="bf16")
    d["w"] = g.choice((1, n, wl.H_I), wl.w_values, dtype="f32")
    d["q"] = g.normal((1, n, H, c), dtype="bf16")
    d["sink"] = g.normal((H,), dtype="f32")
    d["q_pos"] = torch.arange(n, dtype=torch.int32, device=device)[None]
    return d
