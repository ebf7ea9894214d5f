"""Whole-step GPU parity on the six workloads at their full sizes, through the same call
chains (and so the same kernels and launch shapes) that the benchmark times.

The tiny prefill is checked whole against the oracle.  At full size, the oracle computes
sampled outputs one by one:
  - decode: every query's top-k indices (bit-exact) and attention output;
  - FP4 decode, the hierarchical group and HCA decode: a sample of the sequences;
  - the 32K-token prefill: every compressed entry, indexer-K row and window row, plus a
    sample of the query positions (the earliest ones, block boundaries, the last ones and
    random ones).

Indices are compared bit for bit.  Floating outputs must be within atol = rtol = 2e-2
(bf16 I/O) or 1e-4 (fp32 I/O).  No input of the oracle comes from the GPU side.  Where a
GPU stage writes into a buffer the next stage reads (the new window row), the oracle side
uses its own result for that row."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import formats as F
from compressed_sparse_attention_gated_amd import workloads as W
from compressed_sparse_attention_gated_amd.steps import DecodeStep, HcaDecodeStep, HierStep, PrefillStep
from tests._gpu import assert_close, banner, dev, f32, host, i32, oracle_quantised_cache, u8

pytestmark = pytest.mark.gpu

BF16_TOL = dict(atol=2e-2, rtol=2e-2)
F32_TOL = dict(atol=1e-4, rtol=1e-4)


@pytest.fixture(scope="module")
def C():
    from compressed_sparse_attention_gated_amd import csa2

    csa2.lib()
    return csa2


@pytest.fixture(autouse=True)
def _free_device_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _np(t):
    return host(t)


def _oracle_attn_query(q_bt, t, rows_sel, win_rows, win_pos0, window, sink, rope_dims):
    """Oracle attention for one query: q_bt [H, c]; rows_sel [k', c] the selected entries;
    win_rows [Lw, c] the window buffer starting at position win_pos0."""
    kv = rows_sel[None]
    idx = np.arange(rows_sel.shape[0])[None, None]
    out, mass = O.sparse_attn(q_bt[None, None], np.array([[t]]), kv, idx, win_rows[None], [win_pos0], window,
                              sink, rope_dims=rope_dims)
    return out[0, 0], mass[0, 0]


# =================================================================== tiny prefill, whole
def test_tiny_prefill_end_to_end(C):
    wl = W.WORKLOADS[1]
    banner("tiny prefill end to end: n=256 c=64 m=2 overlap, 4x32 indexer, top-16 + 16 window, fp32")
    g = W.rng(1001)
    n, c = wl.n_tokens, wl.c
    cin = W.compress_inputs(g, n, c, wl.m, overlap=True, dtype="f32", bias_std=wl.extra["bias_std"])
    win_src = g.normal((1, n, c), dtype="f32")
    ind = W.indexer_inputs(g, 1, n, n // wl.m, wl.H_I, wl.d_I, wl.w_values)
    att = W.attn_inputs(g, 1, n, 1, wl.H, c, Lw=1, io_dtype="f32", sink_std=0.0)
    q_pos = np.arange(n, dtype=np.int32)[None]

    entries, _ = C.csa2_compress(f32(cin["ca"]), f32(cin["za"]), wl.m, cb=f32(cin["cb"]), zb=f32(cin["zb"]),
                                 ba=f32(cin["ba"]), bb=f32(cin["bb"]), rope_dims=wl.rope_dims)
    wsrc = f32(win_src)
    win, _ = C.csa2_compress(wsrc, wsrc, 1, rope_dims=wl.rope_dims)
    qp = i32(q_pos)
    idx = C.csa2_index_topk(C.CSA2_MODE_FULL, qp, wl.k, q_idx=dev(ind["q_idx"], torch.bfloat16), w=f32(ind["w"]),
                            m=wl.m, k_idx=dev(ind["k_idx"], torch.bfloat16))
    mass = torch.empty((1, n, wl.H), device="cuda")
    out = C.csa2_sparse_attn(f32(att["q"]), qp, idx, kv=entries, win=win, win_pos0=i32([0]), n_win=wl.window,
                             sink=f32(att["sink"]), rope_dims=wl.rope_dims, out_mass=mass)
    torch.cuda.synchronize()

    e_ref, _ = O.compress(cin["ca"][0], cin["za"][0], wl.m, b_a=cin["ba"], c_b=cin["cb"][0], z_b=cin["zb"][0],
                          b_b=cin["bb"], overlap=True, rope_dims=wl.rope_dims)
    w_ref, _ = O.compress(win_src[0], win_src[0], 1, rope_dims=wl.rope_dims)
    i_ref = O.index_topk_full(ind["q_idx"], ind["w"], ind["k_idx"], q_pos, wl.m, wl.k)
    o_ref, m_ref = O.sparse_attn(att["q"], q_pos, e_ref[None], i_ref, w_ref[None], [0], wl.window, att["sink"],
                                 rope_dims=wl.rope_dims)
    assert_close(_np(entries)[0], e_ref, **F32_TOL, what="entries")
    assert_close(_np(win)[0], w_ref, **F32_TOL, what="window rows")
    np.testing.assert_array_equal(_np(idx), i_ref)
    assert_close(_np(out), o_ref, **F32_TOL, what="attention")
    assert_close(_np(mass), m_ref, **F32_TOL, what="mass")


# =================================================================== decode (bf16 and FP4)
def _check_decode(C, wl, seed, sample, cache=None):
    d = W.decode_inputs(wl, seed)
    if cache is not None:
        d["kv_codes"], d["kv_scales"], d["k_codes"], d["k_scales"] = cache
    step = DecodeStep(wl, d)
    win_before = d["win"].clone()
    idx, out = step.run(d)
    torch.cuda.synchronize()
    gi, go, gw = _np(idx), _np(out), _np(d["win"])
    fp4 = wl.kind == "decode_fp4"
    L, W_ = wl.L, wl.window
    sink = _np(d["sink"])
    for b in sample:
        # the new token's window row (m = 1 compressor at position L)
        new_row, _ = O.compress(_np(d["c_new"][b]), _np(d["z_new"][b]), 1, rope_dims=wl.rope_dims, pos0=L)
        assert_close(gw[b, W_ - 1], new_row[0], **BF16_TOL, what=f"new window row b={b}")
        # FULL: scan of all L entries + top-k
        if fp4:
            kb = F.mxfp4_decode(_np(d["k_codes"][b]), _np(d["k_scales"][b]))
        else:
            kb = _np(d["k_idx"][b])
        s = O.indexer_scores(_np(d["q_idx"][b, 0]), _np(d["w"][b, 0]), kb, O.n_visible(L, L, 1))
        i_ref = O.topk_indices(s, wl.k)
        np.testing.assert_array_equal(gi[b, 0], i_ref, err_msg=f"indices b={b}")
        # attention over the oracle's selection and the oracle's window (its own new row)
        sel = torch.as_tensor(i_ref[i_ref >= 0], device="cuda")
        if fp4:
            rows = F.fp4_main_decode(_np(d["kv_codes"][b].index_select(0, sel)),
                                     _np(d["kv_scales"][b].index_select(0, sel)))
        else:
            rows = _np(d["kv"][b].index_select(0, sel))
        win_ref = _np(win_before[b])
        win_ref[W_ - 1] = new_row[0]
        o_ref, _ = _oracle_attn_query(_np(d["q"][b, 0]), L, rows, win_ref, L - W_ + 1, W_, sink, wl.rope_dims)
        assert_close(go[b, 0], o_ref, **BF16_TOL, what=f"attention b={b}")


def test_full_decode_bf16_b32_l65536(C):
    wl = W.WORKLOADS[2]
    banner("full decode: B=32 L=65536 bf16 cache, every query checked")
    _check_decode(C, wl, 3002, range(wl.B))


def test_full_decode_fp4_b64_l262144(C):
    # the cache as the workload states it: N(0,1) source rows through the write path's
    # RMSNorm and RoPE, quantised by the oracle (FP4 main KV, MXFP4 integer K_I)
    wl = W.WORKLOADS[5]
    banner("full FP4 decode: B=64 L=262144 oracle-quantised FP4 main KV + MXFP4 K_I, 8 queries checked")
    cache = oracle_quantised_cache(wl.B, wl.L, 3015)
    _check_decode(C, wl, 3005, [0, 9, 18, 27, 36, 45, 54, 63], cache=cache)


def test_full_decode_fp4_random_codes(C):
    # every FP4 / MXFP4 code value and a spread of scale bytes (random bytes), fewer queries
    wl = W.WORKLOADS[5]
    banner("full FP4 decode: B=64 L=262144 random code bytes, 3 queries checked")
    _check_decode(C, wl, 3025, [1, 32, 62])


def test_full_index_fp4_query_b64_l262144(C):
    # the indexer QK path in FP4 on both sides: MXFP4 q_I (random code bytes) against the
    # FP4 workload's MXFP4 K_I, through the fused scan at full size
    wl = W.WORKLOADS[5]
    banner("full FP4 index: B=64 L=262144 MXFP4 q_I x MXFP4 K_I, 8 queries checked")
    d = W.decode_inputs(wl, 3035)
    q = W.indexer_inputs(W.rng(3036), wl.B, 1, 1, wl.H_I, wl.d_I, wl.w_values, k_format="mxfp4", q_format="mxfp4")
    idx = C.csa2_index_topk(C.CSA2_MODE_FULL, d["q_pos"], wl.k, q_idx=u8(q["q_codes"]), q_scales=u8(q["q_scales"]),
                            w=f32(q["w"]), m=wl.m, k_codes=d["k_codes"], k_scales=d["k_scales"])
    torch.cuda.synchronize()
    gi = _np(idx)
    qp = _np(d["q_pos"])
    for b in [0, 9, 18, 27, 36, 45, 54, 63]:
        kb = F.mxfp4_decode(_np(d["k_codes"][b]), _np(d["k_scales"][b]))
        qb = F.mxfp4_decode(q["q_codes"][b, 0], q["q_scales"][b, 0])
        s = O.indexer_scores(qb, q["w"][b, 0].astype(np.float64), kb, O.n_visible(int(qp[b, 0]), wl.L, wl.m))
        np.testing.assert_array_equal(gi[b, 0], O.topk_indices(s, wl.k), err_msg=f"indices b={b}")


# =================================================================== hierarchical group
def test_full_hier_group_b8_l1m(C):
    wl = W.WORKLOADS[4]
    banner("full hierarchical group: B=8 L=1048576, Full + pool + Reindex + 3 Reuse, 2 sequences checked")
    d = W.hier_inputs(wl, 3004)
    step = HierStep(wl, d)
    idx_full, cand, count, idx_re, outs = step.run(d)
    torch.cuda.synchronize()
    g_full, g_cand, g_cnt, g_re = _np(idx_full), _np(cand), _np(count), _np(idx_re)
    g_outs = [_np(o) for o in outs]
    L, W_ = wl.L, wl.window
    for b in (0, 5):
        kb = _np(d["k_idx"][b])
        l0, l1 = d["layers"][0], d["layers"][1]
        s = O.indexer_scores(_np(l0["q_idx"][b, 0]), _np(l0["w"][b, 0]), kb, L)
        i_full = O.topk_indices(s, wl.k)
        np.testing.assert_array_equal(g_full[b, 0], i_full, err_msg=f"Full-layer indices b={b}")
        pool = O.hier_candidates(O.block_max(s, wl.block), L, n_keep=wl.n_keep_blocks, block=wl.block)
        assert g_cnt[b, 0] == len(pool) == wl.n_keep_blocks * wl.block
        np.testing.assert_array_equal(g_cand[b, 0, :len(pool)], pool, err_msg=f"candidates b={b}")
        i_re = O.reindex_topk(_np(l1["q_idx"][b, 0]), _np(l1["w"][b, 0]), kb, pool, wl.k)
        np.testing.assert_array_equal(g_re[b, 0], i_re, err_msg=f"Reindex indices b={b}")
        for layer, sel_idx in enumerate([i_full] + [i_re] * (len(outs) - 1)):
            e = d["layers"][layer]
            sel = torch.as_tensor(sel_idx[sel_idx >= 0], device="cuda")
            rows = _np(d["kv"][b].index_select(0, sel))
            o_ref, _ = _oracle_attn_query(_np(e["q"][b, 0]), L, rows, _np(e["win"][b]), L - W_ + 1, W_,
                                          _np(e["sink"]), wl.rope_dims)
            assert_close(g_outs[layer][b, 0], o_ref, **BF16_TOL, what=f"attention layer {layer} b={b}")
    # the same step with its second stream folded into the current one: every output equal,
    # bit for bit (the kernels are deterministic, so a race between the two streams would show)
    step.side = torch.cuda.current_stream()
    seq = step.run(d)
    torch.cuda.synchronize()
    for name, got, ref in (("Full indices", seq[0], g_full), ("candidates", seq[1], g_cand),
                           ("counts", seq[2], g_cnt), ("Reindex indices", seq[3], g_re)):
        np.testing.assert_array_equal(_np(got), ref, err_msg=f"{name}: two-stream and one-stream runs differ")
    for layer, o in enumerate(seq[4]):
        np.testing.assert_array_equal(_np(o), g_outs[layer], err_msg=f"attention layer {layer}: stream order")


# =================================================================== HCA decode
def test_full_hca_decode_b32_l1m(C):
    wl = W.WORKLOADS[6]
    banner("full HCA decode: B=32 L=1048576 m'=128 -> 8192 entries + 128 window, dense, 4 sequences checked")
    d = W.hca_inputs(wl, 3006)
    step = HcaDecodeStep(wl, d)
    win_before = d["win"].clone()
    _, out = step.run(d)
    torch.cuda.synchronize()
    go, gw = _np(out), _np(d["win"])
    L, W_ = wl.L, wl.window
    sink = _np(d["sink"])
    for b in (0, 11, 22, 31):
        new_row, _ = O.compress(_np(d["c_new"][b]), _np(d["z_new"][b]), 1, rope_dims=wl.rope_dims, pos0=L)
        assert_close(gw[b, W_ - 1], new_row[0], **BF16_TOL, what=f"new window row b={b}")
        win_ref = _np(win_before[b])
        win_ref[W_ - 1] = new_row[0]
        want, _ = O.dense_attn(_np(d["q"][b:b + 1]), np.array([[L]]), _np(d["kv"][b:b + 1]), wl.m,
                               win=win_ref[None], win_pos0=[L - W_ + 1], window=W_, sink=sink,
                               rope_dims=wl.rope_dims)
        assert_close(go[b, 0], want[0, 0], **BF16_TOL, what=f"HCA attention b={b}")


# =================================================================== 32K-token prefill
def test_full_prefill_32k(C):
    wl = W.WORKLOADS[3]
    banner("full prefill: 32768 tokens -> 16384 entries (m=2, W_IK), causal top-512 + 128 window, 64 heads")
    d = W.prefill_inputs(wl, 3003)
    step = PrefillStep(wl, d)
    n, m = wl.n_tokens, wl.m
    # oracle write path: entries, indexer K, window rows
    e_ref, k_ref = O.compress(_np(d["ca"][0]), _np(d["za"][0]), m, rope_dims=wl.rope_dims, w_ik=_np(d["w_ik"]))
    ws = _np(d["win_src"][0])
    w_ref, _ = O.compress(ws, ws, 1, rope_dims=wl.rope_dims)
    # the index stage reads integer K_I derived from the oracle's projection, so that every
    # score is exact and the selection can be compared bit for bit
    k_int = np.clip(np.rint(2.0 * k_ref), -3, 3)
    k_int_dev = dev(k_int[None].astype(np.float32), torch.bfloat16)
    entries, k_index, win, idx, out = step.run(d, k_idx=k_int_dev)
    torch.cuda.synchronize()
    assert_close(_np(entries)[0], e_ref, **BF16_TOL, what="entries")
    assert_close(_np(k_index)[0], k_ref, **BF16_TOL, what="indexer K projection")
    assert_close(_np(win)[0], w_ref, **BF16_TOL, what="window rows")
    rs = np.random.default_rng(7)
    ts = sorted({0, 1, 2, 3, 5, 127, 128, 129, 1023, 1024, 1025, 2047, 4096, 8191, 16383, 16384, 20001,
                 32766, 32767, *rs.integers(0, n, 13).tolist()})
    tt = torch.as_tensor(ts, device="cuda")
    gi = _np(idx[0].index_select(0, tt))
    go = _np(out[0].index_select(0, tt))
    qi = _np(d["q_idx"][0].index_select(0, tt))
    wv = _np(d["w"][0].index_select(0, tt))
    qq = _np(d["q"][0].index_select(0, tt))
    sink = _np(d["sink"])
    for j, t in enumerate(ts):
        nv = O.n_visible(t, n // m, m)
        i_ref = O.topk_indices(O.indexer_scores(qi[j], wv[j], k_int, nv), wl.k)
        np.testing.assert_array_equal(gi[j], i_ref, err_msg=f"indices t={t}")
        rows = e_ref[i_ref[i_ref >= 0]]
        o_ref, _ = _oracle_attn_query(qq[j], t, rows, w_ref, 0, wl.window, sink, wl.rope_dims)
        assert_close(go[j], o_ref, **BF16_TOL, what=f"attention t={t}")
    # the same step with its second stream folded into the current one: every index and every
    # output value equal (a race between the window-row stream and the scan would show)
    first = [t.clone() for t in (entries, k_index, win, idx, out)]
    step.side = torch.cuda.current_stream()
    again = step.run(d, k_idx=k_int_dev)
    torch.cuda.synchronize()
    for name, a, b_ in zip(("entries", "indexer K", "window rows", "indices", "attention"), again, first):
        assert torch.equal(a, b_), f"{name}: two-stream and one-stream runs differ"
