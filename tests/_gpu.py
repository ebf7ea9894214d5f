"""Helpers for the GPU parity tests: move generator arrays to the device and back."""
import sys

import numpy as np
import torch

from oracle import formats as F

DEV = "cuda"


def banner(msg):
    """Name the case before a GPU step (so a failing run says which case it was)."""
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def dev(x, dtype=None):
    """numpy -> device tensor.  bf16 arrays from the generators hold bf16-exact fp32."""
    if isinstance(x, torch.Tensor):
        return x.to(DEV)
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def bf16(x):
    return dev(np.asarray(x, np.float32), torch.bfloat16)


def f32(x):
    return dev(np.asarray(x, np.float32), torch.float32)


def i32(x):
    return dev(np.asarray(x, np.int32))


def u8(x):
    return dev(np.asarray(x, np.uint8))


def host(t):
    """device tensor -> float64 / int64 numpy (exact for bf16 and fp32)."""
    t = t.detach().cpu()
    if t.dtype in (torch.bfloat16, torch.float16, torch.float32):
        return t.to(torch.float64).numpy()
    return t.numpy()


def assert_close(got, want, atol, rtol, what=""):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.abs(got - want) > atol + rtol * np.abs(want)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside atol={atol} rtol={rtol}; "
                             f"first at {tuple(i)}: got {got[tuple(i)]} want {want[tuple(i)]}; "
                             f"max abs err {np.abs(got - want).max():.3g}")


def plant_high_scores(g, q, kv, ids_gammas, aligned=256, fp4=False):
    """Give every head of each query one sign pattern s on the first `aligned` channels
    (|q| kept), and set each listed key row to gamma * s there and N(0, 1) elsewhere: its
    score is then about 0.82 * gamma * aligned * scale * log2(e) for every head, a sum of
    like-signed terms (small relative rounding), while the N(0, 1) part decides how rows
    of one level share the softmax.  With fp4 the planted rows are replaced by their
    decoded FP4 quantisation.  q [B, 1, H, c] and kv [B, N, c] (fp64) are changed in
    place; ids_gammas[b] lists (entry id, gamma)."""
    B, c = q.shape[0], q.shape[-1]
    for b in range(B):
        s = np.where(g.normal((aligned,), dtype="f32") >= 0, 1.0, -1.0)
        q[b, 0, :, :aligned] = np.abs(q[b, 0, :, :aligned]) * s
        for e, gamma in ids_gammas[b]:
            row = np.asarray(g.normal((c,), dtype="bf16"), np.float64)
            row[:aligned] = gamma * s
            if fp4:
                row = F.fp4_main_decode(*F.quantize_fp4_main(row[None]))[0]
            kv[b, e] = row


def oracle_quantised_cache(B, L, seed, pool_rows=32768, c=512, d_I=128, rope_dims=64):
    """A decode cache of B x L entries in the 4-bit formats, quantised by the oracle: main
    KV rows are N(0,1) source rows after the write path's RMSNorm and RoPE (at the pool
    index), stored as FP4 E2M1 with E4M3 scales per 16; indexer-K rows are integers
    U{-3..3} stored as MXFP4 (exact).  `pool_rows` distinct rows of each are quantised on
    the host and tiled over the cache by seeded random indices drawn on the device.
    Returns device tensors (kv_codes, kv_scales, k_codes, k_scales)."""
    import oracle as O

    r = np.random.Generator(np.random.PCG64(seed))
    src = r.standard_normal((pool_rows, c))
    rows = O.rope(O.rms_norm(src), np.arange(pool_rows), rope_dims)
    kv_codes, kv_scales = F.quantize_fp4_main(rows)
    ki = r.integers(-3, 4, size=(pool_rows, d_I)).astype(np.float64)
    k_codes, k_scales = F.quantize_mxfp4(ki)
    assert np.array_equal(F.mxfp4_decode(k_codes, k_scales), ki)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    pick_kv = torch.randint(0, pool_rows, (B, L), generator=g, device=DEV)
    pick_k = torch.randint(0, pool_rows, (B, L), generator=g, device=DEV)
    out = []
    for pool, pick in ((kv_codes, pick_kv), (kv_scales, pick_kv), (k_codes, pick_k), (k_scales, pick_k)):
        out.append(u8(pool)[pick].contiguous())
    return tuple(out)
