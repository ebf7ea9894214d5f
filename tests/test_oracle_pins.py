"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: values the pages
print or that follow by hand from a worked example on the pages (tests/golden),
closed forms, invariants, special cases that reduce to a library routine, or brute
force on tiny inputs.  CPU only.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import expit, softmax

import oracle as O
from oracle import formats as F
from tests import _golden as G


def _rng(seed=0):
    return np.random.Generator(np.random.PCG64(seed))


# =================================================================== compressor
def test_compress_worked_example():
    g = G.load("compress_worked_example.txt")
    m, c = int(g["m"]), int(g["c"])
    ca, cb = G.matrix(g["ca"]), G.matrix(g["cb"])
    z = np.zeros_like(ca)
    y = O.gated_pool(ca, z, m, c_b=cb, z_b=z, b_a=np.zeros((m, c)), b_b=np.zeros((m, c)),
                     overlap=True)
    np.testing.assert_array_equal(y, G.matrix(g["expect"]))


def test_compress_m1_is_identity():
    # checklist of the DSA-to-CSA notes: with m = 1 the compressor degenerates to per-token
    r = _rng(1)
    ca, za = r.standard_normal((17, 8)), r.standard_normal((17, 8)) * 5
    np.testing.assert_array_equal(O.gated_pool(ca, za, 1), ca)


def test_compress_two_token_block_is_logistic():
    # softmax over two logits is the logistic function of their difference
    r = _rng(2)
    ca, za = r.standard_normal((6, 5)), r.standard_normal((6, 5)) * 3
    y = O.gated_pool(ca, za, 2)
    p0 = expit(za[0::2] - za[1::2])
    np.testing.assert_allclose(y, p0 * ca[0::2] + (1 - p0) * ca[1::2], rtol=1e-13, atol=1e-13)


def test_compress_equal_logits_give_mean_and_shift_invariance():
    r = _rng(3)
    ca, cb = r.standard_normal((16, 4)), r.standard_normal((16, 4))
    z = np.full((16, 4), 0.37)
    y = O.gated_pool(ca, z, 4)
    np.testing.assert_allclose(y, ca.reshape(4, 4, 4).mean(axis=1), rtol=1e-13, atol=1e-14)
    # overlap, equal logits: entry i > 0 is the mean of its own block and the previous C^b block
    yo = O.gated_pool(ca, z, 4, c_b=cb, z_b=z, overlap=True)
    np.testing.assert_allclose(yo[0], ca[:4].mean(axis=0), rtol=1e-13)
    np.testing.assert_allclose(yo[2], np.concatenate([ca[8:12], cb[4:8]]).mean(axis=0), rtol=1e-13)
    # adding a per-channel constant to every logit of the block does not change the output
    za = r.standard_normal((16, 4))
    np.testing.assert_allclose(O.gated_pool(ca, za, 4), O.gated_pool(ca, za + 11.0, 4), rtol=1e-12)


def test_compress_block0_history_has_zero_mass():
    # checklist: the first block's history branch must get exactly zero probability
    r = _rng(4)
    n, c, m = 12, 6, 3
    ca, za = r.standard_normal((n, c)), r.standard_normal((n, c))
    cb, zb = r.standard_normal((n, c)) * 1e6, r.standard_normal((n, c)) + 50.0
    w = O.gated_pool_weights(za, m, z_b=zb, overlap=True)
    assert np.all(w[0, m:] == 0.0)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    y = O.gated_pool(ca, za, m, c_b=cb, z_b=zb, overlap=True)
    np.testing.assert_allclose(y[0], O.gated_pool(ca[:m], za[:m], m)[0], rtol=1e-14)
    # a history branch with -inf logits reduces the overlap variant to the plain one
    y_off = O.gated_pool(ca, za, m, c_b=cb, z_b=np.full((n, c), -np.inf), overlap=True)
    np.testing.assert_allclose(y_off, O.gated_pool(ca, za, m), rtol=1e-14)


def test_compress_output_is_convex_combination_and_bias_acts_per_position():
    r = _rng(5)
    n, c, m = 20, 7, 4
    ca, za = r.standard_normal((n, c)), r.standard_normal((n, c))
    y = O.gated_pool(ca, za, m)
    blk = ca.reshape(n // m, m, c)
    assert np.all(y <= blk.max(axis=1) + 1e-12) and np.all(y >= blk.min(axis=1) - 1e-12)
    # a huge bias on in-block position 2 selects that token in every block
    b = np.zeros((m, c))
    b[2] = 1e4
    np.testing.assert_allclose(O.gated_pool(ca, za, m, b_a=b), ca[2::m], rtol=1e-12)


def test_compress_ragged_tail_ignored():
    r = _rng(6)
    ca, za = r.standard_normal((11, 3)), r.standard_normal((11, 3))
    np.testing.assert_array_equal(O.gated_pool(ca, za, 4), O.gated_pool(ca[:8], za[:8], 4))


# =================================================================== epilogue
def test_rms_norm_unit_rms():
    x = _rng(7).standard_normal((9, 64)) * 3
    y = O.rms_norm(x, eps=0.0)
    np.testing.assert_allclose(np.sqrt((y * y).mean(axis=-1)), 1.0, rtol=1e-14)


def test_rope_matches_complex_rotation_and_relative_positions():
    r = _rng(8)
    c, rd = 16, 8
    x = r.standard_normal(c)
    pos = 37
    y = O.rope(x, pos, rd)
    np.testing.assert_array_equal(y[:c - rd], x[:c - rd])
    u = np.arange(rd // 2)
    zc = (x[c - rd::2] + 1j * x[c - rd + 1::2]) * np.exp(1j * pos * 10000.0 ** (-2 * u / rd))
    np.testing.assert_allclose(y[c - rd::2], zc.real, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(y[c - rd + 1::2], zc.imag, rtol=1e-12, atol=1e-13)
    assert np.isclose(np.linalg.norm(y), np.linalg.norm(x), rtol=1e-14)
    np.testing.assert_allclose(O.rope(y, pos, rd, inverse=True), x, rtol=1e-12, atol=1e-13)
    # dot products of rotated vectors depend on the position difference only
    k = r.standard_normal(c)
    a = O.rope(x, 1000, rd) @ O.rope(k, 990, rd)
    b = O.rope(x, 10, rd) @ k
    assert np.isclose(a, b, rtol=1e-10)
    np.testing.assert_array_equal(O.rope(x, 0, rd), x)


def test_compress_epilogue_order():
    # K_I is projected from the normalised entry before RoPE; RoPE acts at position pos0 + m*i
    r = _rng(9)
    n, c, m, dI = 8, 16, 2, 4
    ca, za = r.standard_normal((n, c)), r.standard_normal((n, c))
    w = r.standard_normal((c, dI))
    out, kI = O.compress(ca, za, m, rope_dims=8, pos0=100, w_ik=w)
    xh = O.rms_norm(O.gated_pool(ca, za, m))
    np.testing.assert_allclose(kI, xh @ w, rtol=1e-13)
    for i in range(n // m):
        np.testing.assert_allclose(out[i], O.rope(xh[i], 100 + m * i, 8), rtol=1e-13, atol=1e-14)


# =================================================================== causal rule
def test_causal_visibility_page_example():
    # the page's HCA example (m' = 128): positions 100 and 127 cannot read entry 0, 128 can
    assert O.n_visible(100, 10, 128) == 0
    assert O.n_visible(127, 10, 128) == 0
    assert O.n_visible(128, 10, 128) == 1
    # m = 2: query t sees entries j with t >= 2(j+1)
    assert [O.n_visible(t, 100, 2) for t in range(7)] == [0, 0, 1, 1, 2, 2, 3]
    assert O.n_visible(10 ** 6, 7, 1) == 7


# =================================================================== indexer + top-k
def test_indexer_page_example_scores_and_ids():
    g = G.load("sparse_shared_kv_example.txt")
    s = O.indexer_scores(G.matrix(g["iq"]), G.vector(g["head_weight"]), G.matrix(g["ik"]))
    np.testing.assert_array_equal(s, G.vector(g["scores"]))
    np.testing.assert_array_equal(O.topk_indices(s, int(g["k"])), G.vector(g["ids"]).astype(int))


def test_indexer_relu_sign_and_single_head():
    # ReLU per head before the weighted head sum: a negative head similarity contributes 0
    q = np.array([[1.0, 0.0], [0.0, 1.0]])
    k = np.array([[-1.0, 2.0]])
    assert O.indexer_scores(q, np.array([1.0, 1.0]), k)[0] == 2.0
    assert O.indexer_scores(q, np.array([-0.5, 1.0]), k)[0] == 2.0
    assert O.indexer_scores(-q, np.array([1.0, 1.0]), -k)[0] == 2.0
    r = _rng(10)
    qi, ki = r.integers(-3, 4, (6, 8)).astype(float), r.integers(-3, 4, (30, 8)).astype(float)
    # one head with weight 1 and non-negative similarities is a plain matrix-vector product
    kp = np.abs(ki)
    qp = np.abs(qi)
    w1 = np.zeros(6)
    w1[2] = 1.0
    np.testing.assert_array_equal(O.indexer_scores(qp, w1, kp), kp @ qp[2])
    # negating every head weight negates the scores; heads add up
    w = r.choice([1.0, -1.0, 0.5, -0.5, 0.25], 6)
    np.testing.assert_array_equal(O.indexer_scores(qi, -w, ki), -O.indexer_scores(qi, w, ki))
    wa, wb = w.copy(), w.copy()
    wa[3:] = 0
    wb[:3] = 0
    np.testing.assert_array_equal(O.indexer_scores(qi, w, ki),
                                  O.indexer_scores(qi, wa, ki) + O.indexer_scores(qi, wb, ki))
    # all similarities negative -> every score is exactly 0
    assert np.all(O.indexer_scores(qp, w, -kp - 1) == 0)


def test_indexer_integer_inputs_exact_in_fp32():
    # the generators' integer inputs and power-of-two weights make fp32 scores exact
    r = _rng(11)
    qi = r.integers(-3, 4, (64, 128)).astype(np.float64)
    ki = r.integers(-3, 4, (500, 128)).astype(np.float64)
    w = r.choice([1.0, -1.0, 0.5, -0.5, 0.25, -0.25], 64)
    s64 = O.indexer_scores(qi, w, ki)
    sim32 = qi.astype(np.float32) @ ki.T.astype(np.float32)
    s32 = (w.astype(np.float32)[:, None] * np.maximum(sim32, 0)).sum(axis=0, dtype=np.float32)
    np.testing.assert_array_equal(s32.astype(np.float64), s64)


def _check_topk_set_property(s, k, out):
    n = s.shape[0]
    kk = min(k, n)
    sel = out[:kk]
    assert np.all(out[kk:] == -1)
    assert np.all(np.diff(sel) > 0)
    mask = np.zeros(n, bool)
    mask[sel] = True
    if kk and kk < n:
        lo = s[mask].min()
        assert s[~mask].max() <= lo
        # boundary ties: every unselected entry with the boundary score sits above every
        # selected entry with that score
        tied_sel = np.nonzero(mask & (s == lo))[0]
        tied_un = np.nonzero(~mask & (s == lo))[0]
        if tied_un.size:
            assert tied_sel.max() < tied_un.min()


@pytest.mark.parametrize("seed", range(6))
def test_topk_brute_force_with_ties(seed):
    r = _rng(100 + seed)
    n = int(r.integers(1, 200))
    s = r.integers(-4, 5, n).astype(np.float64) * 0.5  # many ties
    for k in (1, 3, 16, n, n + 5):
        out = O.topk_indices(s, k)
        _check_topk_set_property(s, k, out)
        ref = sorted(range(n), key=lambda j: (-s[j], j))[:min(k, n)]
        np.testing.assert_array_equal(out[:min(k, n)], np.sort(ref))


def test_topk_negative_zero_and_empty():
    np.testing.assert_array_equal(O.topk_indices(np.array([-0.0, 0.0, -1.0]), 1), [0])
    np.testing.assert_array_equal(O.topk_indices(np.array([0.0, -0.0, -1.0]), 1), [0])
    np.testing.assert_array_equal(O.topk_indices(np.zeros(0), 4), [-1, -1, -1, -1])
    np.testing.assert_array_equal(O.topk_indices(np.full(5, 3.0), 3), [0, 1, 2])


# =================================================================== hierarchical pool
def test_hier_hand_case():
    s = np.zeros(40)
    s[3], s[9], s[17], s[30], s[35] = 5, 9, 1, 7, 3  # block maxima 5, 9, 1, 7, 3
    bm = O.block_max(s)
    np.testing.assert_array_equal(bm, [5, 9, 1, 7, 3])
    # keep 2 blocks: the latest block (4) is forced, plus the best other block (1)
    np.testing.assert_array_equal(O.hier_candidates(bm, 40, n_keep=2),
                                  list(range(8, 16)) + list(range(32, 40)))
    # a partial latest block contributes only its visible positions
    bm37 = O.block_max(s[:37])
    np.testing.assert_array_equal(O.hier_candidates(bm37, 37, n_keep=3),
                                  list(range(8, 16)) + list(range(24, 32)) + list(range(32, 37)))
    # fewer blocks than n_keep: every block
    np.testing.assert_array_equal(O.hier_candidates(bm, 40, n_keep=2048), np.arange(40))


@pytest.mark.parametrize("seed", range(4))
def test_hier_forced_block_equals_replace_rule(seed):
    # "take the top n_keep blocks; if the latest is missing, it replaces the n_keep-th"
    r = _rng(200 + seed)
    nb = int(r.integers(3, 60))
    bs = r.integers(-3, 4, nb).astype(float)
    keep = int(r.integers(1, nb))
    top = sorted(range(nb), key=lambda b: (-bs[b], b))[:keep]
    if nb - 1 not in top:
        top[-1] = nb - 1
    want = np.sort(np.concatenate([np.arange(8 * b, 8 * b + 8) for b in top]))
    np.testing.assert_array_equal(O.hier_candidates(bs, 8 * nb, n_keep=keep), want)


@pytest.mark.parametrize("seed", range(4))
def test_reindex_equals_full_scores_then_candidate_mask(seed):
    r = _rng(300 + seed)
    n, dI, HI = 300, 16, 4
    ki = r.integers(-3, 4, (n, dI)).astype(float)
    qi = r.integers(-3, 4, (HI, dI)).astype(float)
    w = r.choice([1.0, -1.0, 0.5, -0.25], HI)
    cand = np.sort(r.choice(n, int(r.integers(1, 120)), replace=False))
    for k in (1, 16, 200):
        np.testing.assert_array_equal(O.reindex_topk(qi, w, ki, cand, k),
                                      O.reindex_topk_masked(qi, w, ki, cand, n, k))


def test_reuse_is_identity():
    idx = _rng(12).integers(-1, 100, (2, 3, 8))
    np.testing.assert_array_equal(O.reuse(idx), idx)


# =================================================================== attention
def test_attention_page_example():
    g = G.load("sparse_shared_kv_example.txt")
    ids = G.vector(g["ids"]).astype(int)
    kv = G.matrix(g["kv"])
    out, mass = O.sparse_attn(G.vector(g["q"]).reshape(1, 1, 1, 2), np.array([[0]]), kv[None],
                              ids.reshape(1, 1, -1), sink=np.array([float(g["sink"])]),
                              rope_dims=0, q_norm=False)
    np.testing.assert_allclose(out[0, 0, 0], G.vector(g["out"]), rtol=1e-14)
    np.testing.assert_allclose(mass[0, 0, 0], float(g["mass"]), rtol=1e-14)
    assert 0 < mass[0, 0, 0] < 1


def _sdpa_with_sink(q, rows, sink, scale):
    """Library softmax attention (torch SDPA, fp64 on CPU) with the sink realised as
    an extra key whose logit equals the sink and whose value is zero."""
    qt = torch.tensor(q)[None, None, None, :]
    ks = q * (sink / (scale * (q @ q)))
    K = torch.tensor(np.concatenate([rows, ks[None]]))[None, None]
    V = torch.tensor(np.concatenate([rows, np.zeros((1, rows.shape[1]))]))[None, None]
    return torch.nn.functional.scaled_dot_product_attention(qt, K, V, scale=scale)[0, 0, 0].numpy()


def test_dense_attention_when_k_covers_all_entries():
    r = _rng(13)
    N, H, c = 12, 3, 16
    q = r.standard_normal((1, 1, H, c))
    kv = r.standard_normal((1, N, c))
    sink = r.standard_normal(H)
    idx = np.arange(N).reshape(1, 1, N)
    out, mass = O.sparse_attn(q, np.array([[N]]), kv, idx, sink=sink, rope_dims=0)
    for h in range(H):
        qh = q[0, 0, h] / np.sqrt((q[0, 0, h] ** 2).mean() + 1e-6)
        want = _sdpa_with_sink(qh, kv[0], sink[h], 1 / math.sqrt(c))
        np.testing.assert_allclose(out[0, 0, h], want, rtol=1e-12, atol=1e-13)
        z = kv[0] @ qh / math.sqrt(c)
        p = softmax(np.concatenate([z, [sink[h]]]))
        assert np.isclose(mass[0, 0, h], p[:-1].sum(), rtol=1e-13)
        assert 0 < mass[0, 0, h] < 1


def test_attention_without_sink_has_unit_mass_and_no_rows_gives_zero():
    r = _rng(14)
    q, kv = r.standard_normal((1, 1, 2, 8)), r.standard_normal((1, 5, 8))
    _, mass = O.sparse_attn(q, np.array([[9]]), kv, np.array([[[0, 3, -1]]]), sink=None, rope_dims=0)
    np.testing.assert_allclose(mass, 1.0, rtol=1e-14)
    out, mass = O.sparse_attn(q, np.array([[9]]), kv, np.array([[[-1, -1]]]), sink=np.zeros(2),
                              rope_dims=4)
    assert np.all(out == 0) and np.all(mass == 0)


def _written_rows(x, pos, rd):
    return O.rope(x, pos, rd)


def test_attention_shift_invariance_and_relative_position_formula():
    # rows stored rotated at their own positions; query rotated at t, output rotated back by t:
    # every term depends on position differences only (checklist of the DSA-to-CSA notes)
    r = _rng(15)
    N, H, c, rd = 10, 2, 16, 8
    x = r.standard_normal((N, c))
    p = np.sort(r.choice(50, N, replace=False))
    q = r.standard_normal((1, 1, H, c))
    t = 60
    idx = np.arange(N).reshape(1, 1, N)
    sink = np.array([0.3, -1.0])
    o1, _ = O.sparse_attn(q, np.array([[t]]), _written_rows(x, p, rd)[None], idx, sink=sink, rope_dims=rd)
    d = 12345
    o2, _ = O.sparse_attn(q, np.array([[t + d]]), _written_rows(x, p + d, rd)[None], idx, sink=sink,
                          rope_dims=rd)
    np.testing.assert_allclose(o1, o2, rtol=1e-9, atol=1e-10)
    # explicit relative form: logits q_n . R_{p_j - t} x_j, output sum_j p_j R_{p_j - t} x_j
    for h in range(H):
        qn = q[0, 0, h] / np.sqrt((q[0, 0, h] ** 2).mean() + 1e-6)
        rel = np.stack([O.rope(x[j], p[j] - t, rd) for j in range(N)])
        z = rel @ qn / math.sqrt(c)
        pr = softmax(np.concatenate([z, [sink[h]]]))[:-1]
        np.testing.assert_allclose(o1[0, 0, h], pr @ rel, rtol=1e-10, atol=1e-12)


def test_attention_index_permutation_and_window_rows():
    r = _rng(16)
    N, H, c = 20, 2, 8
    q, kv = r.standard_normal((1, 1, H, c)), r.standard_normal((1, N, c))
    win = r.standard_normal((1, 10, c))
    idx = np.array([[[3, 7, 11, -1]]])
    perm = np.array([[[11, -1, 3, 7]]])
    a, _ = O.sparse_attn(q, np.array([[12]]), kv, idx, win, np.array([10]), 3, np.zeros(H), rope_dims=4)
    b, _ = O.sparse_attn(q, np.array([[12]]), kv, perm, win, np.array([10]), 3, np.zeros(H), rope_dims=4)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    # window buffer holding positions 10..19, window 3
    np.testing.assert_array_equal(O.window_rows(12, 10, 10, 3), [0, 1, 2])
    np.testing.assert_array_equal(O.window_rows(20, 10, 10, 3), [8, 9])
    np.testing.assert_array_equal(O.window_rows(25, 10, 10, 3), [])
    np.testing.assert_array_equal(O.window_rows(10, 10, 10, 128), [0])


# =================================================================== formats
def test_cache_budget_890():
    g = {k: int(v) for k, v in G.load("cache_budget.txt").items()}
    assert F.main_kv_entry_bytes() == g["main_kv_entry"] == g["main_kv_codes"] + g["main_kv_scales"]
    assert F.indexer_k_entry_bytes() == g["indexer_entry"] == g["indexer_codes"] + g["indexer_scales"]
    assert F.main_kv_entry_bytes() / 2 == g["per_token_m2_main"]
    assert F.indexer_k_entry_bytes() / 2 == g["per_token_m2_index"]
    assert 3 * (F.main_kv_entry_bytes() + F.indexer_k_entry_bytes()) / 2 == g["encoder_three_layers"]
    assert F.global_cache_bytes_per_token() == g["total"]


def test_ocp_spot_values():
    g = G.load("ocp_formats.txt")
    for code, v in G.mapping(g["e2m1"]).items():
        assert F.e2m1_decode(np.array([code]))[0] == v
    for code, v in G.mapping(g["e4m3"]).items():
        assert F.e4m3_decode(np.array([code]))[0] == v
    for tok in g["e4m3_nan"].split():
        assert np.isnan(F.e4m3_decode(np.array([int(tok, 0)]))[0])
    for code, v in G.mapping(g["e8m0"]).items():
        assert F.e8m0_decode(np.array([code]))[0] == v
    assert np.nanmax(np.abs(F.E4M3_TABLE)) == 448.0


def test_fp4_products_are_exact_bf16():
    # every E2M1 value times every finite E4M3 scale is a bf16 number, so dequantising
    # a main-KV entry into bf16 is exact
    vals = F.e2m1_decode(np.arange(16))
    sc = F.E4M3_TABLE[~np.isnan(F.E4M3_TABLE)]
    assert F.is_exact_bf16(np.outer(vals, sc))


def test_mxfp4_roundtrip_integers_and_fp4_error_bound():
    r = _rng(17)
    x = r.integers(-3, 4, (50, 128)).astype(np.float64)
    x[0, :32] = 0
    x[1, :32] = 1
    codes, sc = F.quantize_mxfp4(x)
    assert codes.shape == (50, 64) and sc.shape == (50, 4)
    np.testing.assert_array_equal(F.mxfp4_decode(codes, sc), x)
    y = r.standard_normal((40, 512))
    cm, sm = F.quantize_fp4_main(y)
    assert cm.shape == (40, 256) and sm.shape == (40, 32)
    deq = F.fp4_main_decode(cm, sm)
    step = np.repeat(F.e4m3_decode(sm), 16, axis=-1)
    # E2M1 gaps are at most 2, so the rounding error is at most one scale unit, plus
    # saturation when the rounded scale falls below amax/6
    amax = np.repeat(np.abs(y.reshape(40, 32, 16)).max(-1), 16, axis=-1)
    assert np.all(np.abs(deq - y) <= step * 1.0 + np.maximum(0, amax - 6 * step) + 1e-12)
    assert F.fp4_main_decode(*F.quantize_fp4_main(np.zeros((1, 512)))).max() == 0


def test_generators_are_seeded():
    from compressed_sparse_attention_gated_amd import workloads as W

    a = W.indexer_inputs(W.rng(5), 2, 1, 10, 4, 32, (1.0, -0.5))
    b = W.indexer_inputs(W.rng(5), 2, 1, 10, 4, 32, (1.0, -0.5))
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    assert set(np.unique(a["k_idx"])) <= set(range(-3, 4))


# =================================================================== write path
def test_cache_rounding_hand_values():
    g = G.load("ocp_rounding.txt")
    for tok in g["e2m1_rne"].split():
        x, code = tok.split(":")
        assert F.e2m1_encode(np.array([float(x)]))[0] == int(code), tok
    for tok in g["e4m3_scale"].split():
        a, byte = tok.split(":")
        x = np.zeros(16)
        x[5] = -float(a)  # the sign of the largest value does not matter
        _, sc = F.quantize_fp4_main(x)
        assert sc[0] == int(byte, 0), tok
    for tok in g["mx_scale"].split():
        a, byte = tok.split(":")
        x = np.zeros(32)
        x[7] = float(a)
        _, sc = F.quantize_mxfp4(x)
        assert sc[0] == int(byte), tok
    for key in ("mx_group_amax6", "mx_group_amax3.99"):
        pairs = [t.split(":") for t in g[key].split()]
        x = np.zeros(32)
        x[:len(pairs)] = [float(v) for v, _ in pairs]
        codes, _ = F.quantize_mxfp4(x)
        nib = F.unpack_nibbles(codes)
        assert list(nib[:len(pairs)]) == [int(c) for _, c in pairs], key


@pytest.mark.parametrize("m,overlap", [(1, False), (2, False), (2, True)])
def test_write_cache_streaming_equals_bulk(m, overlap):
    # A decode step appends one entry per completed block at the cache's length; the cache
    # it builds equals the one written from the whole sequence at once (each entry depends
    # only on its block and, with overlap, the block before: [DSA-to-CSA notes] eq. (11)-(12)).
    r = _rng(31 + m + overlap)
    n, c, d = 10, 64, 32
    ca, za, cb, zb = (r.standard_normal((n, c)) for _ in range(4))
    w_ik = r.standard_normal((c, d)) / 8
    kw = dict(norm=True, rope_dims=16, w_ik=w_ik)
    if overlap:
        kw.update(c_b=cb, z_b=zb, overlap=True)
    ent, kix = O.compress(ca, za, m, **kw)
    n_rows = n // m + 2
    bulk = O.write_cache(ent, kix, 0, n_rows)
    stream = [np.zeros_like(p) for p in bulk]
    for i in range(n // m):
        lo = m * max(i - 1, 0)  # the open block plus, with overlap, the block before
        sl = slice(lo, m * (i + 1))
        kwi = dict(kw)
        if overlap:
            kwi.update(c_b=cb[sl], z_b=zb[sl])
        e_i, k_i = O.compress(ca[sl], za[sl], m, pos0=lo, **kwi)
        np.testing.assert_allclose(e_i[-1], ent[i], rtol=0, atol=1e-12)
        part = O.write_cache(e_i[-1:], k_i[-1:], i, n_rows)
        for s_, p_ in zip(stream, part):
            s_[i] = p_[i]
    for s_, b_ in zip(stream, bulk):
        np.testing.assert_array_equal(s_, b_)
    # rows past the entries stay zero; out-of-range destinations are dropped
    assert not bulk[0][n // m:].any() and not bulk[1][n // m:].any()
    tail = O.write_cache(ent, kix, n_rows - 1, n_rows)
    np.testing.assert_array_equal(tail[0][n_rows - 1], bulk[0][0])
    assert not tail[0][:n_rows - 1].any()
    # dequantised rows are within one scale unit of the entries
    deq = F.fp4_main_decode(bulk[0][:n // m], bulk[1][:n // m])
    step = np.repeat(F.e4m3_decode(bulk[1][:n // m]), 16, axis=-1)
    assert np.all(np.abs(deq - ent) <= step + 1e-12)


# =================================================================== HCA (dense over compressed entries)
def test_hca_causal_boundary_page_example():
    # [DSA-to-CSA notes] "因果边界与短滑窗" with m' = 128: the first entry pools positions
    # 0-127; positions 100 and 127 cannot read it, position 128 can.
    r = _rng(41)
    H, c, W = 2, 16, 4
    kv = r.standard_normal((1, 3, c))
    win = r.standard_normal((1, 300, c))
    q = r.standard_normal((1, 1, H, c))
    sink = r.standard_normal(H)
    for t, n_seen in ((100, 0), (127, 0), (128, 1), (255, 1), (256, 2), (10_000, 3)):
        out, _ = O.dense_attn(q, np.array([[t]]), kv, 128, win=win, win_pos0=[0], window=W, sink=sink,
                              rope_dims=0)
        wrows = win[0, t - W + 1:t + 1]
        for h in range(H):
            qh = q[0, 0, h] / np.sqrt((q[0, 0, h] ** 2).mean() + 1e-6)
            rows = np.concatenate([kv[0, :n_seen], wrows])
            want = _sdpa_with_sink(qh, rows, sink[h], 1 / math.sqrt(c))
            np.testing.assert_allclose(out[0, 0, h], want, rtol=1e-12, atol=1e-13, err_msg=f"t={t}")


def test_hca_pipeline_pools_128_token_blocks_with_bias():
    # eq. (22)-(23): per-channel softmax over a non-overlapping block of m' tokens, logits
    # Z + B; equal logits give the block mean, and a bias column shifts weight to its position
    r = _rng(42)
    c, mp = 8, 128
    C = r.standard_normal((2 * mp, c))
    ent, _ = O.compress(C, np.zeros((2 * mp, c)), mp, norm=False)
    np.testing.assert_allclose(ent, C.reshape(2, mp, c).mean(axis=1), rtol=1e-12, atol=1e-14)
    bias = np.zeros((mp, c))
    bias[5] = 50.0  # e^50 dominates the other 127 unit terms
    ent_b, _ = O.compress(C, np.zeros((2 * mp, c)), mp, b_a=bias, norm=False)
    np.testing.assert_allclose(ent_b, C.reshape(2, mp, c)[:, 5], rtol=0, atol=1e-15)


# =================================================================== grouped output projection
def test_grouped_out_proj_hand_example():
    # n_h = 4 heads of c = 1, g = 2 groups, d_g = 1, d = 2: group 0 sees heads 0-1, group 1
    # heads 2-3; worked by hand
    o = np.array([[[1.0], [2.0], [3.0], [4.0]]])
    w1 = np.array([[[1.0, 10.0]], [[100.0, 1000.0]]])  # [g, d_g, 2]
    w2 = np.array([[1.0, 1.0], [2.0, -1.0]])            # [d, g*d_g]
    mid, out = O.grouped_out_proj(o, w1, w2)
    np.testing.assert_array_equal(mid, [[21.0, 4300.0]])
    np.testing.assert_array_equal(out, [[4321.0, 42.0 - 4300.0]])


def test_grouped_out_proj_is_a_block_diagonal_then_dense_product():
    # the two levels equal one product with a block-diagonal first matrix; with g = 1 it is
    # two plain matrix products
    r = _rng(51)
    M, n_h, c, g, dg, d = 5, 8, 4, 4, 3, 6
    o = r.standard_normal((M, n_h, c))
    w1 = r.standard_normal((g, dg, c * n_h // g))
    w2 = r.standard_normal((d, g * dg))
    mid, out = O.grouped_out_proj(o, w1, w2)
    from scipy.linalg import block_diag
    bd = block_diag(*[w1[j].T for j in range(g)])  # [n_h*c, g*dg]
    np.testing.assert_allclose(mid, o.reshape(M, -1) @ bd, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(out, o.reshape(M, -1) @ bd @ w2.T, rtol=1e-12, atol=1e-12)
    w1b = r.standard_normal((1, dg, n_h * c))
    mid1, out1 = O.grouped_out_proj(o, w1b, w2[:, :dg])
    np.testing.assert_allclose(out1, (o.reshape(M, -1) @ w1b[0].T) @ w2[:, :dg].T, rtol=1e-12)


# =================================================================== packed samples
def test_packed_compressor_hand_example():
    # two samples in one stream, m = 2, equal logits (block means): sample A = 1, 2, 3 (its
    # tail token 3 is dropped, not paired with sample B's first token), sample B = 10, 20
    C = np.array([[1.0], [2.0], [3.0], [10.0], [20.0]])
    ent, _, cu_e = O.compress_packed(C, np.zeros_like(C), 2, [0, 3, 5], norm=False)
    np.testing.assert_array_equal(ent, [[1.5], [15.0]])
    np.testing.assert_array_equal(cu_e, [0, 1, 2])
    # the flat stream would have paired 3 with 10
    flat, _ = O.compress(C[:4], np.zeros((4, 1)), 2, norm=False)
    assert flat[1, 0] == 6.5


def test_packed_compressor_overlap_history_stops_at_sample_start():
    # with overlap, a sample's first entry has no history even when another sample precedes
    # it; a sample of fewer than m tokens yields no entry
    r = _rng(61)
    m, c = 2, 4
    lens = [5, 1, 4]
    n = sum(lens)
    ca, za, cb, zb = (r.standard_normal((n, c)) for _ in range(4))
    cu = np.concatenate([[0], np.cumsum(lens)])
    ent, _, cu_e = O.compress_packed(ca, za, m, cu, c_b=cb, z_b=zb, norm=False)
    np.testing.assert_array_equal(cu_e, [0, 2, 2, 4])
    own, _ = O.compress(ca[6:10], za[6:10], m, c_b=cb[6:10], z_b=zb[6:10], overlap=True, norm=False)
    np.testing.assert_allclose(ent[2:4], own, rtol=0, atol=0)
    # the third sample's first entry: no history, so the same as without overlap
    no_hist, _ = O.compress(ca[6:8], za[6:8], m, norm=False)
    np.testing.assert_allclose(ent[2], no_hist[0], rtol=1e-15, atol=1e-15)


def test_packed_compressor_positions_restart_per_sample():
    # m = 1 without norm writes each token rotated by its position; on c = r = 2 the
    # rotation of (1, 0) by angle p * theta^0 is (cos p, sin p).  Every sample's tokens
    # take positions 0, 1, .. of their own sample, not of the stream.
    x = np.tile([[1.0, 0.0]], (5, 1))
    ent, _, cu_e = O.compress_packed(x, np.zeros_like(x), 1, [0, 3, 5], norm=False, rope_dims=2)
    pos = np.array([0, 1, 2, 0, 1], np.float64)
    np.testing.assert_allclose(ent, np.stack([np.cos(pos), np.sin(pos)], axis=1), rtol=0, atol=1e-15)
    np.testing.assert_array_equal(cu_e, [0, 3, 5])


def test_packed_index_and_window_masks_hand_example():
    # a stream of three samples (5, 1 and 4 tokens), m = 2: the samples own entries [0, 2),
    # none (one token is shorter than m) and [2, 4).  Worked by hand: token p of a sample sees
    # the entries of its own sample whose block has ended (p >= 2(j+1)), and a 3-token window
    # of its own sample.
    cu, cu_e, m, W = [0, 5, 6, 10], [0, 2, 2, 4], 2, 3
    want_entries = {0: [], 1: [], 2: [0], 3: [0], 4: [0, 1], 5: [], 6: [], 7: [], 8: [2], 9: [2]}
    want_window = {0: [0], 1: [0, 1], 2: [0, 1, 2], 3: [1, 2, 3], 4: [2, 3, 4], 5: [5], 6: [6],
                   7: [6, 7], 8: [6, 7, 8], 9: [7, 8, 9]}
    for t in range(10):
        assert list(O.packed_visible_entries(t, cu, cu_e, m)) == want_entries[t], t
        assert list(O.packed_window_rows(t, cu, W)) == want_window[t], t
    # the packed top-k keeps every visible entry (k = 4) and nothing of another sample: with
    # scores equal to the entry id + 1 the order is plain, and entry 3 (not yet visible at
    # token 9) must not appear
    q_idx = np.ones((10, 1, 1))
    k_idx = np.arange(1.0, 5.0)[:, None]
    got = O.index_topk_packed(q_idx, np.ones((10, 1)), k_idx, cu, cu_e, m, 4)
    for t in range(10):
        e = want_entries[t]
        assert list(got[t]) == e + [-1] * (4 - len(e)), t
    # attention of token 8 (sample 3, position 2) over its entry 2 and window rows 6, 7, 8:
    # without norm, rope or sink, a softmax over those four rows with scale 1
    r = _rng(71)
    q, kv, win = r.standard_normal((10, 1, 4)), r.standard_normal((4, 4)), r.standard_normal((10, 4))
    idx = np.full((10, 4), -1)
    idx[8, 0] = 2
    out, mass = O.sparse_attn_packed(q, kv, idx, win, cu, window=W, rope_dims=0, q_norm=False, scale=1.0)
    rows = np.stack([kv[2], win[6], win[7], win[8]])
    p = softmax(rows @ q[8, 0])
    np.testing.assert_allclose(out[8, 0], p @ rows, rtol=1e-13)
    assert mass[8, 0] == pytest.approx(1.0)

