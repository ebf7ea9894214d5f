"""Plain fp64 CPU oracle of the CSA2 layer hot path.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import or call this module.  It shares no code, table
or helper with the HIP library.  Every function is the definition on the pages
written out directly in numpy fp64: no blocking, fusion or reordering beyond
what the definition states.  Python loops appear where the definition is a loop
(blocks of the compressor, queries of the attention); sizes in the tests keep
them short.

Pages (cited by title and section / equation):
  [CSA2 column]  daiw.org "CSA2：跨层共享的压缩稀疏注意力" (DeepSeek V4.1 Flash column):
                 sections "保留了 CSA 的骨架" (skeleton), "三种模式：谁算、谁复用" (modes table),
                 "解码器里的分层索引" (hierarchical indexer), "890 字节是怎么来的" (cache budget).
  [Evolution blog] 0xnullpath "DeepSeek 的 Attention 演进 -【DSA、CSA、CSA2】":
                 §2.2 (lightning indexer), §3.1 (gated pooling and overlap transform),
                 §3.2 (sliding window), §4.1 (CSA2 compressor), §4.3 (sharing modes),
                 §4.4 (hierarchical indexer).
  [DSA-to-CSA notes] wineandchord "从 DSA 到 CSA/HCA：先压缩时间轴，再决定怎样寻址":
                 eq. (9)-(12) overlapped compressor and its worked example, eq. (16)-(17)
                 indexer and top-k, eq. (18)-(19) shared-KV MQA with its worked example,
                 section "因果边界与短滑窗" (causal rule, window), eq. (27) sink,
                 section "怎样验证" (checklist).

Readings where the pages leave a step open (each also listed in the design notes):
  * RoPE: theta = 10000, adjacent pairs (c-r+2u, c-r+2u+1), frequency theta^(-2u/r).
  * Position of compressed entry i is pos0 + m*i (the first token of its block).
  * RMSNorm: gamma = 1, eps = 1e-6, x / sqrt(mean(x^2) + eps).
  * KV RMSNorm and RoPE happen when an entry is written; attention normalises and
    rotates only the query, and inverse-rotates the output.
  * Window rows for query t: positions [t-W+1, t] that the window buffer holds; no
    de-duplication against selected entries.
  * Top-k ties go to the lower index; -0 equals +0; output ascending, -1 padded.
  * Hierarchical pool: the latest visible block is always selected, the other
    n_keep-1 blocks by (score desc, block asc).
"""

from __future__ import annotations

import math

import numpy as np

# ============================================================ compressor
def _logsumexp(terms):
    """log(sum_j exp(terms[j])) over axis 0, per channel; -inf terms contribute nothing."""
    t = np.asarray(terms, np.float64)
    top = t.max(axis=0)
    safe = np.where(np.isfinite(top), top, 0.0)
    with np.errstate(divide="ignore"):  # all terms -inf: log 0 = -inf
        return safe + np.log(np.exp(t - safe).sum(axis=0))


def gated_pool(c_a, z_a, m, *, b_a=None, c_b=None, z_b=None, b_b=None, overlap=False):
    """Gated per-channel softmax pooling over blocks of m tokens.

    Non-overlap (CSA2, [Evolution blog] §4.1, and HCA eq. (22)-(23) of
    [DSA-to-CSA notes]): entry i pools tokens [m*i, m*i+m).  For channel ch the gate
    logit of token j is Z[j,ch] + B[j-m*i, ch], and entry i is the weighted sum of
    C[j,ch] with weights exp(logit_j - LSE), where LSE = log sum_j exp(logit_j): a
    softmax over the block's positions, separately for every channel.

    Overlap (CSA, [DSA-to-CSA notes] eq. (11)-(12)): the candidates of entry i are the
    current block (values C^a, logits Z^a + B^a) and the previous block (values C^b,
    logits Z^b + B^b).  Both sets share one normaliser LSE over all 2m logits, and the
    entry is the current-block sum plus the history sum.  Block 0 has no previous block:
    the pages give its history logits -inf (and values 0), so its history weights are 0
    and only the current block enters its normaliser and its sum.

    Only complete blocks are pooled; a ragged tail of n % m tokens is ignored.
    Inputs are [n, c]; biases are [m, c] or None (= 0).  Returns [n // m, c] fp64.
    """
    c_a = np.asarray(c_a, np.float64)
    z_a = np.asarray(z_a, np.float64)
    n, c = c_a.shape
    ba = np.zeros((m, c)) if b_a is None else np.asarray(b_a, np.float64)
    bb = np.zeros((m, c)) if b_b is None else np.asarray(b_b, np.float64)
    out = np.zeros((n // m, c))
    for i in range(n // m):
        cur_logit = z_a[m * i:m * i + m] + ba          # [m, c]
        cur_value = c_a[m * i:m * i + m]
        has_history = overlap and i > 0
        if has_history:
            hist_logit = np.asarray(z_b, np.float64)[m * (i - 1):m * i] + bb
            hist_value = np.asarray(c_b, np.float64)[m * (i - 1):m * i]
            lse = _logsumexp(np.concatenate([_logsumexp(cur_logit)[None], _logsumexp(hist_logit)[None]]))
        else:
            lse = _logsumexp(cur_logit)
        y = (np.exp(cur_logit - lse) * cur_value).sum(axis=0)
        if has_history:
            y = y + (np.exp(hist_logit - lse) * hist_value).sum(axis=0)
        out[i] = y
    return out


def gated_pool_weights(z_a, m, *, b_a=None, z_b=None, b_b=None, overlap=False):
    """The softmax weights of `gated_pool`, [n//m, m or 2m, c]; the history half
    (overlap) is the second m rows.  Used by the tests that check zero history mass."""
    z_a = np.asarray(z_a, np.float64)
    n, c = z_a.shape
    ba = np.zeros((m, c)) if b_a is None else np.asarray(b_a, np.float64)
    bb = np.zeros((m, c)) if b_b is None else np.asarray(b_b, np.float64)
    out = []
    for i in range(n // m):
        lg = [z_a[m * i:m * i + m] + ba]
        if overlap:
            lg.append(np.full((m, c), -np.inf) if i == 0 else np.asarray(z_b, np.float64)[m * (i - 1):m * i] + bb)
        lg = np.concatenate(lg, axis=0)
        p = np.exp(lg - lg.max(axis=0))
        out.append(p / p.sum(axis=0))
    return np.stack(out) if out else np.zeros((0, 2 * m if overlap else m, c))


def rms_norm(x, eps=1e-6):
    """RMSNorm with unit gain over the last axis: x / sqrt(mean(x^2) + eps)
    ([Evolution blog] §4.1 kv_norm; [DSA-to-CSA notes] §Shared-KV MQA, per-head norm)."""
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope_angles(pos, r, theta=10000.0):
    """Angles [..., r/2] = pos * theta^(-2u/r) for u = 0..r/2-1."""
    u = np.arange(r // 2, dtype=np.float64)
    freq = theta ** (-2.0 * u / r)
    return np.asarray(pos, np.float64)[..., None] * freq


def rope(x, pos, r, theta=10000.0, inverse=False):
    """Rotate the last r channels of x ([..., c]) in adjacent pairs by angle pos*freq_u
    (by -pos*freq_u if inverse).  `pos` broadcasts against x's leading axes.
    [DSA-to-CSA notes] §Shared-KV MQA: RoPE only on the last 64 dims, and the
    output's last dims are rotated back by the query position."""
    x = np.array(x, np.float64, copy=True)
    if r == 0:
        return x
    c = x.shape[-1]
    ang = rope_angles(pos, r, theta)
    if inverse:
        ang = -ang
    cos, sin = np.cos(ang), np.sin(ang)
    x0 = x[..., c - r::2].copy()
    x1 = x[..., c - r + 1::2].copy()
    x[..., c - r::2] = x0 * cos - x1 * sin
    x[..., c - r + 1::2] = x0 * sin + x1 * cos
    return x


def compress(c_a, z_a, m, *, b_a=None, c_b=None, z_b=None, b_b=None, overlap=False,
             norm=True, eps=1e-6, rope_dims=0, theta=10000.0, pos0=0, w_ik=None):
    """The compressor with its write-path epilogue ([Evolution blog] §4.1):
    pool -> RMSNorm (kv_norm) -> optional indexer-K projection of the normalised,
    not yet rotated entry -> RoPE of the main entry at position pos0 + m*i.
    Returns (entries [n//m, c], k_index [n//m, d_I] or None)."""
    y = gated_pool(c_a, z_a, m, b_a=b_a, c_b=c_b, z_b=z_b, b_b=b_b, overlap=overlap)
    xh = rms_norm(y, eps) if norm else y
    k_index = None if w_ik is None else xh @ np.asarray(w_ik, np.float64)
    pos = pos0 + m * np.arange(xh.shape[0])
    out = rope(xh, pos, rope_dims, theta) if rope_dims else xh
    return out, k_index


def compress_packed(c_a, z_a, m, cu_seqlens, *, c_b=None, z_b=None, **kw):
    """The compressor over packed samples ([DSA-to-CSA notes], the note after the minimal
    compressor code and the checklist "怎样验证"): samples that share one token stream must not
    share a compression window, and a sample's tail shorter than m is not completed by the
    next sample.  Sample s holds tokens [cu[s], cu[s+1]); it is compressed on its own
    (positions from 0, no history for its first entry) and its floor(len/m) entries follow
    those of the samples before it.  Returns (entries, k_index or None, cu_entries)."""
    cu = [int(x) for x in cu_seqlens]
    outs, iks, cu_e = [], [], [0]
    for s in range(len(cu) - 1):
        sl = slice(cu[s], cu[s + 1])
        extra = dict(kw)
        if c_b is not None:
            extra.update(c_b=np.asarray(c_b)[sl], z_b=np.asarray(z_b)[sl], overlap=True)
        e, k = compress(np.asarray(c_a)[sl], np.asarray(z_a)[sl], m, **extra)
        outs.append(e)
        iks.append(k)
        cu_e.append(cu_e[-1] + e.shape[0])
    c = np.asarray(c_a).shape[-1]
    ent = np.concatenate(outs, axis=0) if outs else np.zeros((0, c))
    kix = None if kw.get("w_ik") is None else np.concatenate(iks, axis=0)
    return ent, kix, np.array(cu_e, dtype=np.int64)


def write_cache(entries, k_index, dst_row, n_rows):
    """The write path into a decode cache: [CSA2 column] "890 字节是怎么来的" stores each
    main-KV entry in 4 bits (E2M1 codes, one E4M3 scale per 16 channels) and the indexer
    key in MXFP4 (E2M1 codes, one E8M0 scale per 32 dims); [Evolution blog] §4.1 writes
    an entry after its norm and position encoding, then quantises it.  `entries` [ne, c]
    and `k_index` [ne, d] (or None) are what `compress` returns; entry i lands in cache
    row dst_row + i, rows outside [0, n_rows) are dropped, untouched rows stay zero.
    The rounding rule (nearest, ties to the even code) is the one in `formats`.
    Returns (codes [n_rows, c/2], scales [n_rows, c/16], ik_codes [n_rows, d/2] or None,
    ik_scales [n_rows, d/32] or None)."""
    from . import formats as F

    e = np.asarray(entries, np.float64)
    ne, c = e.shape
    codes = np.zeros((n_rows, c // 2), np.uint8)
    scales = np.zeros((n_rows, c // F.MAIN_KV_GROUP), np.uint8)
    ik_codes = ik_scales = None
    if k_index is not None:
        d = np.asarray(k_index).shape[1]
        ik_codes = np.zeros((n_rows, d // 2), np.uint8)
        ik_scales = np.zeros((n_rows, d // F.MX_GROUP), np.uint8)
    for i in range(ne):
        r = dst_row + i
        if not 0 <= r < n_rows:
            continue
        codes[r], scales[r] = F.quantize_fp4_main(e[i])
        if k_index is not None:
            ik_codes[r], ik_scales[r] = F.quantize_mxfp4(np.asarray(k_index[i], np.float64))
    return codes, scales, ik_codes, ik_scales


# ============================================================ causal rule
def n_visible(t, n_entries, m):
    """Compressed entry j (tokens [m*j, m*j+m)) is visible to query position t iff
    t >= m*(j+1) ([DSA-to-CSA notes] §因果边界与短滑窗).  Returns min(N, floor(t/m))."""
    return int(max(0, min(n_entries, t // m)))


# ============================================================ lightning indexer
def indexer_scores(q_idx, w, k_idx, n_vis=None):
    """I[s] = sum_h w[h] * ReLU(q_I[h] . K_I[s]) ([DSA-to-CSA notes] eq. (16);
    [Evolution blog] §2.2: ReLU and a signed head weight instead of a softmax).
    q_idx [H_I, d_I], w [H_I], k_idx [N, d_I] -> scores [n_vis]."""
    k = np.asarray(k_idx, np.float64)
    if n_vis is not None:
        k = k[:n_vis]
    sim = np.asarray(q_idx, np.float64) @ k.T  # [H_I, n]
    return (np.asarray(w, np.float64)[:, None] * np.maximum(sim, 0.0)).sum(axis=0)


def topk_indices(scores, k):
    """TopK of eq. (17), [DSA-to-CSA notes]: the min(k, n) largest scores, ties to the
    lower index, returned as indices in ascending order and padded with -1 to k.
    Done as a full stable sort by (-score, index)."""
    s = np.asarray(scores, np.float64)
    n = s.shape[0]
    order = np.lexsort((np.arange(n), -s))  # primary -s, secondary index
    chosen = np.sort(order[:min(k, n)])
    out = np.full(k, -1, dtype=np.int64)
    out[:chosen.shape[0]] = chosen
    return out


def index_topk_full(q_idx, w, k_idx, q_pos, m, k):
    """FULL mode for a batch: q_idx [B, T, H_I, d_I], w [B, T, H_I], k_idx [B, N, d_I],
    q_pos [B, T] -> idx [B, T, k]."""
    B, T = np.asarray(q_pos).shape
    N = np.asarray(k_idx).shape[1]
    out = np.full((B, T, k), -1, dtype=np.int64)
    for b in range(B):
        for t in range(T):
            nv = n_visible(int(q_pos[b, t]), N, m)
            out[b, t] = topk_indices(indexer_scores(q_idx[b, t], w[b, t], k_idx[b], nv), k)
    return out


# ============================================================ hierarchical pool
def block_max(scores, block=8):
    """Block score = max over the visible positions [block*b, block*b+block)
    ([CSA2 column] §解码器里的分层索引; [Evolution blog] §4.4)."""
    s = np.asarray(scores, np.float64)
    nb = -(-s.shape[0] // block)
    return np.array([s[block * b:block * b + block].max() for b in range(nb)])


def hier_candidates(block_scores, n_vis, n_keep=2048, block=8):
    """Candidate pool: at most n_keep blocks, the latest visible block always kept
    ([Evolution blog] §4.4), the others by (score desc, block asc); returns the
    ascending visible positions of the chosen blocks."""
    bs = np.asarray(block_scores, np.float64)
    nb = bs.shape[0]
    if nb == 0:
        return np.zeros(0, dtype=np.int64)
    last = nb - 1
    others = np.arange(nb - 1)
    order = others[np.lexsort((others, -bs[:nb - 1]))]
    chosen = np.sort(np.concatenate([[last], order[:max(0, n_keep - 1)]]))
    pos = (chosen[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    return pos[pos < n_vis]


def reindex_topk(q_idx, w, k_idx, cand, k):
    """REINDEX ([CSA2 column] modes table; [Evolution blog] §4.4): score only the
    candidate positions with this layer's indexer query, keep the top k by
    (score desc, position asc); returns positions ascending, -1 padded."""
    cand = np.asarray(cand, np.int64)
    s = indexer_scores(q_idx, w, np.asarray(k_idx)[cand])
    sel = topk_indices(s, k)
    return np.where(sel >= 0, cand[np.maximum(sel, 0)], -1)


def reindex_topk_masked(q_idx, w, k_idx, cand, n_vis, k):
    """The same selection written as the pages describe the reference code: full
    scores over all visible positions, non-candidates set to -inf, then top-k
    ([Evolution blog] §4.4).  Only positions with a finite score may be returned."""
    s = indexer_scores(q_idx, w, k_idx, n_vis)
    masked = np.full_like(s, -np.inf)
    cand = np.asarray(cand, np.int64)
    masked[cand] = s[cand]
    sel = topk_indices(masked, min(k, cand.shape[0]))
    out = np.full(k, -1, dtype=np.int64)
    out[:sel.shape[0]] = sel
    return out


def reuse(src_idx):
    """REUSE: the indices of the upstream Full/Reindex layer, unchanged
    ([CSA2 column] modes table)."""
    return np.array(src_idx, copy=True)


# ============================================================ sparse shared-KV MQA
def window_rows(t, win_pos0, n_win_rows, window):
    """Window buffer row numbers whose positions lie in [t-window+1, t]
    ([CSA2 column] §保留了 CSA 的骨架: the latest 128 tokens of this layer)."""
    lo = max(t - window + 1, win_pos0)
    hi = min(t, win_pos0 + n_win_rows - 1)
    return np.arange(lo - win_pos0, hi - win_pos0 + 1) if hi >= lo else np.zeros(0, np.int64)


def attend_one(q, rows, sink, scale):
    """Softmax over the rows plus a value-less sink logit ([DSA-to-CSA notes]
    eq. (27)); rows are both keys and values (eq. (19)).  q [c], rows [R, c].
    Returns (output [c], real mass)."""
    rows = np.asarray(rows, np.float64)
    if rows.shape[0] == 0:
        return np.zeros(q.shape[-1]), 0.0
    z = rows @ q * scale
    mx = z.max() if sink is None or sink == -np.inf else max(z.max(), sink)
    e = np.exp(z - mx)
    den = e.sum() + (0.0 if sink is None or sink == -np.inf else math.exp(sink - mx))
    p = e / den
    return p @ rows, float(p.sum())


def sparse_attn(q, q_pos, kv, idx, win=None, win_pos0=None, window=128, sink=None,
                rope_dims=64, theta=10000.0, eps=1e-6, scale=None, q_norm=True):
    """Shared-KV sparse MQA for a batch ([DSA-to-CSA notes] eq. (18)-(19), (27) and
    §Shared-KV MQA).  For query t and head h:
        q_hat = RoPE_t(RMSNorm(q_h))                      (norm optional)
        rows  = kv[idx != -1]  ++  window rows at positions [t-W+1, t]
        p_j   = exp(q_hat.row_j * scale) / (sum_j exp(...) + exp(sink_h))
        o     = sum_j p_j row_j;  o's last r dims rotated by -t.
    q [B, T, H, c]; kv [B, N, c]; idx [B, T, k]; win [B, Lw, c] or None;
    win_pos0 [B]; sink [H] or None (no sink).  scale defaults to 1/sqrt(c).
    Returns (out [B, T, H, c], mass [B, T, H])."""
    q = np.asarray(q, np.float64)
    kv = np.asarray(kv, np.float64)
    B, T, H, c = q.shape
    scale = 1.0 / math.sqrt(c) if not scale else scale
    out = np.zeros((B, T, H, c))
    mass = np.zeros((B, T, H))
    for b in range(B):
        for t in range(T):
            pos = int(q_pos[b, t])
            sel = [int(j) for j in idx[b, t] if j >= 0]
            rows = [kv[b, sel]]
            if win is not None and window > 0:
                wr = window_rows(pos, int(win_pos0[b]), win.shape[1], window)
                rows.append(np.asarray(win[b], np.float64)[wr])
            rows = np.concatenate(rows, axis=0)
            for h in range(H):
                qh = rms_norm(q[b, t, h], eps) if q_norm else q[b, t, h]
                qh = rope(qh, pos, rope_dims, theta) if rope_dims else qh
                sk = None if sink is None else float(sink[h])
                o, ms = attend_one(qh, rows, sk, scale)
                out[b, t, h] = rope(o, pos, rope_dims, theta, inverse=True) if rope_dims else o
                mass[b, t, h] = ms
    return out, mass


def dense_attn(q, q_pos, kv, m_prime, win=None, win_pos0=None, window=128, sink=None,
               rope_dims=64, theta=10000.0, eps=1e-6, scale=None, q_norm=True):
    """HCA's attention ([DSA-to-CSA notes] eq. (20)-(26)): no indexer; every compressed
    entry the query may see is both key and value, CoreAttn(q, C^Comp, C^Comp).  Entry j
    pools tokens [m'j, m'j+m') and is visible from position m'(j+1) on (section
    "因果边界与短滑窗", with m replaced by m'); the latest n_win uncompressed rows are joined
    as in CSA, and the sink logit of eq. (27) applies alike.  That is the shared-KV
    attention above with the index list 0 .. n_vis-1.  Returns (out, mass)."""
    B, T = np.asarray(q).shape[:2]
    N = np.asarray(kv).shape[1]
    idx = np.full((B, T, max(N, 1)), -1, dtype=np.int64)
    for b in range(B):
        for t in range(T):
            nv = n_visible(int(q_pos[b, t]), N, m_prime)
            idx[b, t, :nv] = np.arange(nv)
    return sparse_attn(q, q_pos, kv, idx, win=win, win_pos0=win_pos0, window=window, sink=sink,
                       rope_dims=rope_dims, theta=theta, eps=eps, scale=scale, q_norm=q_norm)


# ============================================================ packed samples
def packed_sample_of(t, cu_seqlens):
    """The sample holding stream token t: s with cu[s] <= t < cu[s+1]."""
    cu = np.asarray(cu_seqlens, np.int64)
    return int(np.searchsorted(cu, t, side="right") - 1)


def packed_visible_entries(t, cu_seqlens, cu_entries, m):
    """Stream entry ids the indexer of stream token t may score ([DSA-to-CSA notes], checklist
    "怎样验证": the indexer mask must not cross a sample boundary).  t is token p of its sample
    s, which owns entries cu_e[s] .. cu_e[s+1]-1 (compress_packed's offsets); the causal rule
    applies within the sample: cu_e[s] + [0, n_visible(p))."""
    s = packed_sample_of(t, cu_seqlens)
    p = int(t) - int(cu_seqlens[s])
    n_s = int(cu_entries[s + 1]) - int(cu_entries[s])
    return int(cu_entries[s]) + np.arange(n_visible(p, n_s, m))


def packed_window_rows(t, cu_seqlens, window):
    """Stream rows in the sliding window of token t: the latest `window` tokens of its own
    sample up to and including t (the window must not cross a sample boundary either)."""
    s = packed_sample_of(t, cu_seqlens)
    return np.arange(max(int(cu_seqlens[s]), int(t) - window + 1), int(t) + 1)


def index_topk_packed(q_idx, w, k_idx, cu_seqlens, cu_entries, m, k):
    """FULL mode over a packed stream: q_idx [T, H_I, d_I], w [T, H_I] for every token,
    k_idx [N, d_I] the stream's entries.  Each token scores only its sample's visible
    entries; returns stream entry ids [T, k] (ascending, -1 padded)."""
    T = np.asarray(q_idx).shape[0]
    out = np.full((T, k), -1, dtype=np.int64)
    for t in range(T):
        ids = packed_visible_entries(t, cu_seqlens, cu_entries, m)
        s = indexer_scores(q_idx[t], w[t], np.asarray(k_idx)[ids])
        sel = topk_indices(s, k)
        out[t] = np.where(sel >= 0, ids[np.maximum(sel, 0)] if len(ids) else -1, -1)
    return out


def sparse_attn_packed(q, kv, idx, win, cu_seqlens, window=128, sink=None, rope_dims=64,
                       theta=10000.0, eps=1e-6, scale=None, q_norm=True, tokens=None):
    """Shared-KV sparse MQA over a packed stream: q [T, H, c] for every token, kv [N, c] the
    stream's entries, idx [T, k] stream entry ids, win [T, c] the stream's per-token rows.
    Token t (position p in its sample) attends to its selected entries and the window rows
    of its own sample; RoPE and the inverse rotation use p.  `tokens` (optional) limits the
    work to those tokens (the others stay zero).  Returns (out [T, H, c], mass [T, H])."""
    q = np.asarray(q, np.float64)
    T, H, c = q.shape
    out = np.zeros((T, H, c))
    mass = np.zeros((T, H))
    for t in (range(T) if tokens is None else tokens):
        s = packed_sample_of(t, cu_seqlens)
        p = t - int(cu_seqlens[s])
        rows = packed_window_rows(t, cu_seqlens, window)
        # the window buffer of the query is its own sample's rows, position 0 at row cu[s]
        o, ms = sparse_attn(q[t][None, None], np.array([[p]]), np.asarray(kv, np.float64)[None],
                            np.asarray(idx)[t][None, None], np.asarray(win, np.float64)[rows][None],
                            [p - len(rows) + 1], window, sink, rope_dims=rope_dims, theta=theta,
                            eps=eps, scale=scale, q_norm=q_norm)
        out[t], mass[t] = o[0, 0], ms[0, 0]
    return out, mass


def grouped_out_proj(o, w1, w2):
    """Grouped output projection after the core attention ([DSA-to-CSA notes] section
    "Grouped output projection"): the n_h heads' outputs are split into g groups of n_h/g
    consecutive heads; group j's c*n_h/g values are projected to d_g, the g results are
    concatenated and projected to d.  o [M, n_h, c]; w1 [g, d_g, c*n_h/g] and w2 [d, g*d_g]
    hold each projection as (output, input), so y = x @ w.T.
    Returns (mid [M, g*d_g], out [M, d])."""
    o = np.asarray(o, np.float64)
    w1 = np.asarray(w1, np.float64)
    w2 = np.asarray(w2, np.float64)
    M, n_h, c = o.shape
    g = w1.shape[0]
    x = o.reshape(M, g, (n_h // g) * c)
    mid = np.concatenate([x[:, j] @ w1[j].T for j in range(g)], axis=1)
    return mid, mid @ w2.T


__all__ = [
    "grouped_out_proj",
    "gated_pool", "gated_pool_weights", "rms_norm", "rope_angles", "rope", "compress", "write_cache",
    "compress_packed",
    "dense_attn",
    "n_visible", "indexer_scores", "topk_indices", "index_topk_full", "block_max",
    "hier_candidates", "reindex_topk", "reindex_topk_masked", "reuse", "window_rows",
    "attend_one", "sparse_attn",
    "packed_sample_of", "packed_visible_entries", "packed_window_rows", "index_topk_packed",
    "sparse_attn_packed",
]
