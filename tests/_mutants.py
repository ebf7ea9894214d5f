"""Planted mistakes in the oracle, to show that the pins catch them.

Each mutant replaces one oracle function, in memory only, by a plausible wrong version
(a dropped term, a wrong sign, index or slice, a transposed pairing, a reversed tie rule).
`tests/test_oracle_mutations.py` runs the pin suite once per mutant in a child process
(environment variable CSA2_ORACLE_MUTANT, applied by conftest.py) and requires that at
least one pin fails.  Nothing here runs on a GPU or touches the HIP library.
"""
from __future__ import annotations

import math

import numpy as np


def _set(name, fn, module=None):
    import oracle
    import oracle.csa2_oracle as M

    mod = module or M
    setattr(mod, name, fn)
    if module is None and hasattr(oracle, name):
        setattr(oracle, name, fn)


def _orig(name):
    import oracle.csa2_oracle as M

    return getattr(M, name)


# ------------------------------------------------------------------ compressor
def pool_drop_history():
    f = _orig("gated_pool")
    _set("gated_pool", lambda c_a, z_a, m, **kw: f(c_a, z_a, m, b_a=kw.get("b_a")))


def pool_history_wrong_block():
    f = _orig("gated_pool")

    def g(c_a, z_a, m, *, c_b=None, z_b=None, **kw):
        if c_b is not None:  # history taken from the current block instead of the previous one
            c_b, z_b = np.roll(np.asarray(c_b), -m, axis=0), np.roll(np.asarray(z_b), -m, axis=0)
        return f(c_a, z_a, m, c_b=c_b, z_b=z_b, **kw)
    _set("gated_pool", g)


def pool_ignore_bias():
    f = _orig("gated_pool")
    _set("gated_pool", lambda c_a, z_a, m, *, b_a=None, b_b=None, **kw: f(c_a, z_a, m, **kw))


def rms_sum_not_mean():
    _set("rms_norm", lambda x, eps=1e-6: np.asarray(x, np.float64) / np.sqrt(
        np.sum(np.asarray(x, np.float64) ** 2, axis=-1, keepdims=True) + eps))


def rope_sign_flip():
    f = _orig("rope")
    _set("rope", lambda x, pos, r, theta=10000.0, inverse=False: f(x, pos, r, theta, not inverse))


def rope_half_split_pairs():
    def g(x, pos, r, theta=10000.0, inverse=False):
        x = np.array(x, np.float64, copy=True)
        if r == 0:
            return x
        c = x.shape[-1]
        u = np.arange(r // 2, dtype=np.float64)
        ang = np.asarray(pos, np.float64)[..., None] * theta ** (-2.0 * u / r)
        ang = -ang if inverse else ang
        a, b = x[..., c - r:c - r // 2].copy(), x[..., c - r // 2:].copy()
        x[..., c - r:c - r // 2] = a * np.cos(ang) - b * np.sin(ang)
        x[..., c - r // 2:] = a * np.sin(ang) + b * np.cos(ang)
        return x
    _set("rope", g)


def compress_position_i_not_mi():
    f = _orig("compress")

    def g(c_a, z_a, m, *, pos0=0, rope_dims=0, theta=10000.0, **kw):
        out, k = f(c_a, z_a, m, rope_dims=0, **kw)
        pos = pos0 + np.arange(out.shape[0])
        return (_orig("rope")(out, pos, rope_dims, theta) if rope_dims else out), k
    _set("compress", g)


def kproj_after_rope():
    f = _orig("compress")

    def g(c_a, z_a, m, *, w_ik=None, **kw):
        out, _ = f(c_a, z_a, m, **kw)
        return out, (None if w_ik is None else out @ np.asarray(w_ik, np.float64))
    _set("compress", g)


def packed_positions_continue():
    f = _orig("compress_packed")

    def g(c_a, z_a, m, cu_seqlens, *, c_b=None, z_b=None, **kw):
        # positions carried on from the stream instead of restarting per sample
        cu = [int(x) for x in cu_seqlens]
        outs, iks, cu_e = [], [], [0]
        for s in range(len(cu) - 1):
            sl = slice(cu[s], cu[s + 1])
            extra = dict(kw, pos0=cu[s])
            if c_b is not None:
                extra.update(c_b=np.asarray(c_b)[sl], z_b=np.asarray(z_b)[sl], overlap=True)
            e, k = _orig("compress")(np.asarray(c_a)[sl], np.asarray(z_a)[sl], m, **extra)
            outs.append(e)
            iks.append(k)
            cu_e.append(cu_e[-1] + e.shape[0])
        ent = np.concatenate(outs, axis=0)
        kix = None if kw.get("w_ik") is None else np.concatenate(iks, axis=0)
        return ent, kix, np.array(cu_e, dtype=np.int64)
    _set("compress_packed", g)


def packed_share_window():
    def g(c_a, z_a, m, cu_seqlens, *, c_b=None, z_b=None, **kw):
        # the whole stream compressed as one sequence: windows straddle sample boundaries
        extra = dict(kw)
        if c_b is not None:
            extra.update(c_b=c_b, z_b=z_b, overlap=True)
        e, k = _orig("compress")(c_a, z_a, m, **extra)
        cu = [int(x) for x in cu_seqlens]
        cu_e = [0]
        for s in range(len(cu) - 1):
            cu_e.append(cu_e[-1] + (cu[s + 1] - cu[s]) // m)
        n = cu_e[-1]
        return e[:n], (None if k is None else k[:n]), np.array(cu_e, dtype=np.int64)
    _set("compress_packed", g)


# ------------------------------------------------------------------ indexer, top-k, pool
def visibility_off_by_one():
    _set("n_visible", lambda t, n_entries, m: int(max(0, min(n_entries, t // m + 1))))


def indexer_no_relu():
    def g(q_idx, w, k_idx, n_vis=None):
        k = np.asarray(k_idx, np.float64)[:n_vis] if n_vis is not None else np.asarray(k_idx, np.float64)
        return (np.asarray(w, np.float64)[:, None] * (np.asarray(q_idx, np.float64) @ k.T)).sum(axis=0)
    _set("indexer_scores", g)


def indexer_abs_not_relu():
    def g(q_idx, w, k_idx, n_vis=None):
        k = np.asarray(k_idx, np.float64)[:n_vis] if n_vis is not None else np.asarray(k_idx, np.float64)
        return (np.asarray(w, np.float64)[:, None] * np.abs(np.asarray(q_idx, np.float64) @ k.T)).sum(axis=0)
    _set("indexer_scores", g)


def topk_ties_to_higher_index():
    def g(scores, k):
        s = np.asarray(scores, np.float64)
        n = s.shape[0]
        order = np.lexsort((-np.arange(n), -s))
        out = np.full(k, -1, dtype=np.int64)
        ch = np.sort(order[:min(k, n)])
        out[:ch.shape[0]] = ch
        return out
    _set("topk_indices", g)


def topk_score_order():
    def g(scores, k):
        s = np.asarray(scores, np.float64)
        n = s.shape[0]
        order = np.lexsort((np.arange(n), -s))[:min(k, n)]
        out = np.full(k, -1, dtype=np.int64)
        out[:order.shape[0]] = order
        return out
    _set("topk_indices", g)


def block_mean_not_max():
    def g(scores, block=8):
        s = np.asarray(scores, np.float64)
        nb = -(-s.shape[0] // block)
        return np.array([s[block * b:block * b + block].mean() for b in range(nb)])
    _set("block_max", g)


def hier_latest_not_forced():
    def g(block_scores, n_vis, n_keep=2048, block=8):
        bs = np.asarray(block_scores, np.float64)
        nb = bs.shape[0]
        idx = np.arange(nb)
        chosen = np.sort(idx[np.lexsort((idx, -bs))][:n_keep])
        pos = (chosen[:, None] * block + np.arange(block)[None, :]).reshape(-1)
        return pos[pos < n_vis]
    _set("hier_candidates", g)


def reindex_returns_slots():
    def g(q_idx, w, k_idx, cand, k):
        cand = np.asarray(cand, np.int64)
        return _orig("topk_indices")(_orig("indexer_scores")(q_idx, w, np.asarray(k_idx)[cand]), k)
    _set("reindex_topk", g)


# ------------------------------------------------------------------ attention
def attn_drop_sink():
    f = _orig("attend_one")
    _set("attend_one", lambda q, rows, sink, scale: f(q, rows, None, scale))


def attn_scale_one_over_c():
    f = _orig("attend_one")
    _set("attend_one", lambda q, rows, sink, scale: f(q, rows, sink, scale / math.sqrt(q.shape[-1])))


def attn_no_inverse_rotation():
    f = _orig("rope")
    _set("rope", lambda x, pos, r, theta=10000.0, inverse=False: (
        np.array(x, np.float64, copy=True) if inverse else f(x, pos, r, theta)))


def window_excludes_current_token():
    def g(t, win_pos0, n_win_rows, window):
        lo = max(t - window, win_pos0)
        hi = min(t - 1, win_pos0 + n_win_rows - 1)
        return np.arange(lo - win_pos0, hi - win_pos0 + 1) if hi >= lo else np.zeros(0, np.int64)
    _set("window_rows", g)


def out_proj_interleaved_groups():
    def g(o, w1, w2):
        o = np.asarray(o, np.float64)
        w1 = np.asarray(w1, np.float64)
        w2 = np.asarray(w2, np.float64)
        M, n_h, c = o.shape
        gg = w1.shape[0]
        x = o.reshape(M, n_h // gg, gg, c).transpose(0, 2, 1, 3).reshape(M, gg, -1)  # heads j, j+g, ..
        mid = np.concatenate([x[:, j] @ w1[j].T for j in range(gg)], axis=1)
        return mid, mid @ w2.T
    _set("grouped_out_proj", g)


def packed_window_crosses_samples():
    _set("packed_window_rows", lambda t, cu_seqlens, window: np.arange(max(0, int(t) - window + 1), int(t) + 1))


def packed_visibility_stream_position():
    def g(t, cu_seqlens, cu_entries, m):
        s = _orig("packed_sample_of")(t, cu_seqlens)
        n_s = int(cu_entries[s + 1]) - int(cu_entries[s])
        return int(cu_entries[s]) + np.arange(_orig("n_visible")(int(t), n_s, m))  # t, not t - cu[s]
    _set("packed_visible_entries", g)


# ------------------------------------------------------------------ cache formats
def fp4_ties_away_from_zero():
    import oracle.formats as F

    def enc(x):
        x = np.asarray(x, np.float64)
        a = np.abs(x)
        grid = F.E2M1_MAGNITUDES
        d = np.abs(a[..., None] - grid)
        best = d.min(axis=-1, keepdims=True)
        field = (np.where(d == best, np.arange(8), -1)).max(axis=-1)  # ties go up
        field = np.where(a >= grid[-1], 7, field)
        sign = (x < 0) & (field != 0)
        return (field | np.where(sign, 8, 0)).astype(np.uint8)
    _set("e2m1_encode", enc, F)


def mxfp4_exponent_off_by_one():
    import oracle.formats as F
    f = F.quantize_mxfp4

    def g(x):
        codes, sc = f(np.asarray(x, np.float64) * 0.5)  # e one lower than the rule's
        return codes, (sc.astype(np.int64) + 1).clip(0, 254).astype(np.uint8)
    _set("quantize_mxfp4", g, F)


def e4m3_bias_eight():
    import oracle.formats as F
    tab = np.array([F.e4m3_decode_scalar(b) for b in range(256)]) * 0.5
    _set("e4m3_decode", lambda codes: tab[np.asarray(codes, dtype=np.int64)], F)


MUTANTS = {f.__name__: f for f in [
    pool_drop_history, pool_history_wrong_block, pool_ignore_bias, rms_sum_not_mean, rope_sign_flip,
    rope_half_split_pairs, compress_position_i_not_mi, kproj_after_rope, packed_positions_continue,
    packed_share_window, visibility_off_by_one, indexer_no_relu, indexer_abs_not_relu,
    topk_ties_to_higher_index, topk_score_order, block_mean_not_max, hier_latest_not_forced,
    reindex_returns_slots, attn_drop_sink, attn_scale_one_over_c, attn_no_inverse_rotation,
    window_excludes_current_token, out_proj_interleaved_groups, fp4_ties_away_from_zero,
    packed_window_crosses_samples, packed_visibility_stream_position,
    mxfp4_exponent_off_by_one, e4m3_bias_eight,
]}


def apply(name: str) -> None:
    MUTANTS[name]()
