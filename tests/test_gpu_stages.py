"""Stage-isolated GPU parity: each libcsa2 call against the fp64 oracle on the same seeded
inputs.  Indices are compared bit for bit; floating outputs within atol = rtol = 2e-2 for
bf16 I/O and 1e-4 for fp32 I/O."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import formats as F
from compressed_sparse_attention_gated_amd import workloads as W
from tests._gpu import assert_close, banner, bf16, dev, f32, host, i32, plant_high_scores, u8

pytestmark = pytest.mark.gpu

BF16_TOL = dict(atol=2e-2, rtol=2e-2)
F32_TOL = dict(atol=1e-4, rtol=1e-4)


@pytest.fixture(scope="module")
def C():
    from compressed_sparse_attention_gated_amd import csa2

    csa2.lib()
    return csa2


# =================================================================== compressor
def _oracle_compress(d, m, overlap, pos0, rope_dims, w_ik=None, norm=True):
    outs, iks = [], []
    for b in range(d["ca"].shape[0]):
        o, k = O.compress(d["ca"][b], d["za"][b], m, b_a=d.get("ba"),
                          c_b=d["cb"][b] if overlap else None, z_b=d["zb"][b] if overlap else None,
                          b_b=d.get("bb"), overlap=overlap, norm=norm, rope_dims=rope_dims,
                          pos0=int(pos0[b]), w_ik=w_ik)
        outs.append(o)
        iks.append(k)
    return np.stack(outs), (np.stack(iks) if w_ik is not None else None)


def test_compress_tiny_prefill_f32_overlap(C):
    banner("compress cfg1: f32 overlap m=2 n=256 c=64 bias rope16")
    g = W.rng(1001)
    d = W.compress_inputs(g, 256, 64, 2, overlap=True, dtype="f32", bias_std=0.1)
    pos0 = np.zeros(1, np.int32)
    out, _ = C.csa2_compress(f32(d["ca"]), f32(d["za"]), 2, cb=f32(d["cb"]), zb=f32(d["zb"]),
                             ba=f32(d["ba"]), bb=f32(d["bb"]), pos0=i32(pos0), rope_dims=16)
    torch.cuda.synchronize()
    want, _ = _oracle_compress(d, 2, True, pos0, 16)
    assert_close(host(out), want, **F32_TOL, what="compress cfg1")


def test_compress_bf16_m2_projection_ragged(C):
    banner("compress bf16 m=2 n=1001 c=512 B=2 w_ik d=128 rope64 pos0")
    g = W.rng(7)
    d = W.compress_inputs(g, 1001, 512, 2, dtype="bf16", d_I=128, B=2)
    pos0 = np.array([0, 37], np.int32)
    out, ik = C.csa2_compress(bf16(d["ca"]), bf16(d["za"]), 2, pos0=i32(pos0), rope_dims=64,
                              w_ik=bf16(d["w_ik"]))
    torch.cuda.synchronize()
    assert out.shape == (2, 500, 512) and ik.shape == (2, 500, 128)
    want, want_ik = _oracle_compress(d, 2, False, pos0, 64, w_ik=d["w_ik"].astype(np.float64))
    assert_close(host(out), want, **BF16_TOL, what="compress out")
    assert_close(host(ik), want_ik, **BF16_TOL, what="compress k_index")


def test_compress_m1_decode_append_large_positions(C):
    banner("compress m=1 B=4 bf16 at positions ~1M")
    g = W.rng(8)
    d = W.compress_inputs(g, 3, 512, 1, dtype="bf16", B=4)
    pos0 = np.array([65536, 1048575, 262143, 5], np.int32)
    out, _ = C.csa2_compress(bf16(d["ca"]), bf16(d["za"]), 1, pos0=i32(pos0), rope_dims=64)
    torch.cuda.synchronize()
    want, _ = _oracle_compress(d, 1, False, pos0, 64)
    assert_close(host(out), want, **BF16_TOL, what="compress m=1")


@pytest.mark.parametrize("c,m", [(16, 4), (128, 3), (512, 8)])
def test_compress_pooling_only_f32(C, c, m):
    banner(f"compress f32 pooling c={c} m={m}")
    g = W.rng(9 + c)
    d = W.compress_inputs(g, 50, c, m, dtype="f32", bias_std=0.5)
    out, _ = C.csa2_compress(f32(d["ca"]), f32(d["za"]), m, ba=f32(d["ba"]), norm=False)
    torch.cuda.synchronize()
    want, _ = _oracle_compress(d, m, False, np.zeros(1), 0, norm=False)
    assert_close(host(out), want, atol=1e-5, rtol=1e-5, what="pooling")


# =================================================================== indexer + top-k
def _oracle_scores(q_idx, w, k_idx, q_pos, m):
    B, T = q_pos.shape
    N = k_idx.shape[1]
    res = []
    for b in range(B):
        for t in range(T):
            nv = O.n_visible(int(q_pos[b, t]), N, m)
            res.append(O.indexer_scores(q_idx[b, t], w[b, t], k_idx[b], nv))
    return res


def _q_args(d):
    """The query arguments of a call and the oracle's dense q_I: bf16 q_I, or MXFP4 codes and
    scales decoded by the oracle's own format decoder."""
    if "q_codes" in d:
        return (dict(q_idx=u8(d["q_codes"]), q_scales=u8(d["q_scales"])),
                F.mxfp4_decode(d["q_codes"], d["q_scales"]))
    return dict(q_idx=bf16(d["q_idx"])), d["q_idx"].astype(np.float64)


def _check_full(C, d, q_pos, m, k, k_dense=None, mx=False, block=8, what=""):
    """Run FULL on the GPU and compare indices, scores and block maxima with the oracle."""
    B, T = q_pos.shape
    N = (d["k_idx"] if not mx else d["k_codes"]).shape[1]
    scores = torch.full((B, T, N), float("nan"), device="cuda")
    nblk = (N + block - 1) // block
    bmax = torch.full((B, T, nblk), float("nan"), device="cuda")
    kw = dict(k_codes=u8(d["k_codes"]), k_scales=u8(d["k_scales"])) if mx else dict(k_idx=bf16(d["k_idx"]))
    qa, qd = _q_args(d)
    idx = C.csa2_index_topk(C.CSA2_MODE_FULL, i32(q_pos), k, w=f32(d["w"]), m=m,
                            out_scores=scores, out_block_max=bmax, block=block, **qa, **kw)
    torch.cuda.synchronize()
    kd = k_dense if k_dense is not None else d["k_idx"].astype(np.float64)
    ref = _oracle_scores(qd, d["w"].astype(np.float64), kd, q_pos, m)
    gi, gs, gb = host(idx), host(scores), host(bmax)
    for r, s in enumerate(ref):
        b, t = divmod(r, T)
        np.testing.assert_array_equal(gs[b, t, :len(s)], s, err_msg=f"{what} scores row {r}")
        np.testing.assert_array_equal(gi[b, t], O.topk_indices(s, k), err_msg=f"{what} idx row {r}")
        if len(s):
            np.testing.assert_array_equal(gb[b, t, :-(-len(s) // block)], O.block_max(s, block),
                                          err_msg=f"{what} block max row {r}")
    return idx, scores, bmax


def test_index_full_tiny_prefill(C):
    banner("index FULL cfg1: T=256 N=128 H_I=4 d_I=32 m=2 k=16 (shared-B path)")
    wl = W.WORKLOADS[1]
    g = W.rng(1001)
    d = W.indexer_inputs(g, 1, 256, 128, 4, 32, wl.w_values)
    _check_full(C, d, np.arange(256, dtype=np.int32)[None], 2, 16, what="cfg1")


@pytest.mark.parametrize("HI,dI", [(64, 128), (32, 64), (48, 32)])
def test_index_full_prefill_shapes(C, HI, dI):
    banner(f"index FULL prefill T=70 N=150 H_I={HI} d_I={dI} m=2 k=64")
    g = W.rng(30 + HI + dI)
    d = W.indexer_inputs(g, 2, 70, 150, HI, dI, (1.0, -1.0, 0.5, -0.25))
    q_pos = np.stack([np.arange(70) * 4 + 3, np.arange(70) + 200]).astype(np.int32)
    _check_full(C, d, q_pos, 2, 64, what=f"prefill {HI}x{dI}")


def test_index_full_decode_ragged(C):
    banner("index FULL decode B=3 N=5000 k=512 (private-B path)")
    g = W.rng(11)
    d = W.indexer_inputs(g, 3, 1, 5000, 64, 128, W.WORKLOADS[2].w_values)
    q_pos = np.array([[5000], [4000], [37]], np.int32)
    _check_full(C, d, q_pos, 1, 512, what="decode")


def test_index_full_decode_two_level(C):
    banner("index FULL decode B=2 N=70000 k=512 (two-level top-k)")
    g = W.rng(12)
    d = W.indexer_inputs(g, 2, 1, 70000, 64, 128, W.WORKLOADS[2].w_values)
    q_pos = np.array([[70000], [50001]], np.int32)
    _check_full(C, d, q_pos, 1, 512, what="two-level")


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
@pytest.mark.parametrize("HI,dI", [(64, 64), (32, 128), (48, 32), (16, 64)])
def test_index_full_decode_shapes(C, HI, dI, fmt):
    banner(f"index FULL decode {fmt} K_I B=3 N=9000 H_I={HI} d_I={dI} k=256 (fused scan + chunk top-k)")
    g = W.rng(40 + HI + dI + (fmt == "mxfp4"))
    mx = fmt == "mxfp4"
    d = W.indexer_inputs(g, 3, 1, 9000, HI, dI, W.WORKLOADS[5 if mx else 2].w_values,
                         k_format="mxfp4" if mx else "bf16")
    kd = F.mxfp4_decode(d["k_codes"], d["k_scales"]) if mx else None
    q_pos = np.array([[9000], [8191], [300]], np.int32)  # full, ragged tail, mostly empty chunks
    _check_full(C, d, q_pos, 1, 256, k_dense=kd, mx=mx, what=f"decode {fmt} {HI}x{dI}")


@pytest.mark.parametrize("HI,dI", [(64, 128), (48, 64), (16, 32)])
def test_index_mxfp4_query(C, HI, dI):
    """FP4 on both sides of the indexer QK product (scaled FP4 x FP4 MFMA): fused decode
    (N > 8192, ragged and mostly-empty rows), private decode, a 40-query prefill and REINDEX,
    against the oracle's scores of the decoded q_I and K_I."""
    banner(f"index MXFP4 q_I x MXFP4 K_I: H_I={HI} d_I={dI}")
    g = W.rng(60 + HI + dI)
    wv = W.WORKLOADS[5].w_values
    d = W.indexer_inputs(g, 3, 1, 9000, HI, dI, wv, k_format="mxfp4", q_format="mxfp4")
    kd = F.mxfp4_decode(d["k_codes"], d["k_scales"])
    _check_full(C, d, np.array([[9000], [8191], [300]], np.int32), 1, 256, k_dense=kd, mx=True,
                what=f"mxfp4 q fused {HI}x{dI}")
    d = W.indexer_inputs(g, 2, 1, 3000, HI, dI, wv, k_format="mxfp4", q_format="mxfp4")
    kd = F.mxfp4_decode(d["k_codes"], d["k_scales"])
    _check_full(C, d, np.array([[3000], [1234]], np.int32), 1, 128, k_dense=kd, mx=True,
                what=f"mxfp4 q private {HI}x{dI}")
    d = W.indexer_inputs(g, 1, 40, 700, HI, dI, wv, k_format="mxfp4", q_format="mxfp4")
    kd = F.mxfp4_decode(d["k_codes"], d["k_scales"])
    _check_full(C, d, (np.arange(40, dtype=np.int32) * 35 + 7)[None], 2, 64, k_dense=kd, mx=True,
                what=f"mxfp4 q prefill {HI}x{dI}")
    # REINDEX: 300 sorted candidates of the visible entries per query
    N, B = 5000, 2
    d = W.indexer_inputs(g, B, 1, N, HI, dI, wv, k_format="mxfp4", q_format="mxfp4")
    kd = F.mxfp4_decode(d["k_codes"], d["k_scales"])
    q_pos = np.array([[N], [4000]], np.int32)
    r = np.random.default_rng(HI + dI)
    cands = [np.sort(r.choice(int(q_pos[b, 0]), 300, replace=False)) for b in range(B)]
    cand = np.full((B, 1, 320), -1, np.int32)
    for b in range(B):
        cand[b, 0, :300] = cands[b]
    qa, qd = _q_args(d)
    idx = C.csa2_index_topk(C.CSA2_MODE_REINDEX, i32(q_pos), 64, w=f32(d["w"]), m=1,
                            k_codes=u8(d["k_codes"]), k_scales=u8(d["k_scales"]), cand=i32(cand),
                            n_cand=i32(np.full((B, 1), 300, np.int32)), **qa)
    torch.cuda.synchronize()
    gi = host(idx)
    for b in range(B):
        want = O.reindex_topk(qd[b, 0], d["w"][b, 0].astype(np.float64), kd[b], cands[b], 64)
        np.testing.assert_array_equal(gi[b, 0], want, err_msg=f"reindex b={b}")


@pytest.mark.parametrize("HI,dI", [(64, 128), (48, 64), (16, 32)])
def test_index_e4m3_query_path(C, HI, dI):
    """bf16 q_I with an MXFP4 K_I in the fused decode scan: a query whose every value is an
    E4M3 value takes the FP8 x FP4 MFMA, any other the bf16 path; one launch holds both kinds
    (integers; E4M3 values over 2^-1 .. 2^3 with three mantissa bits; multiples of 1/32; and
    integers but for one value with six mantissa bits).  Every score is exact in fp32, so both
    paths must give the oracle's scores and indices exactly."""
    banner(f"index bf16 q_I (E4M3-exact and not) x MXFP4 K_I, fused decode: H_I={HI} d_I={dI}")
    g = W.rng(70 + HI + dI)
    r = np.random.default_rng(70 + HI + dI)
    d = W.indexer_inputs(g, 4, 1, 9000, HI, dI, W.WORKLOADS[5].w_values, k_format="mxfp4")
    shape = d["q_idx"].shape[2:]
    e4m3 = np.exp2(r.integers(-1, 3, size=shape)) * (1 + r.integers(0, 8, size=shape) / 8.0)
    d["q_idx"][1, 0] = (e4m3 * r.choice([-1.0, 1.0], size=shape)).astype(np.float32)
    d["q_idx"][2, 0] = (r.integers(-127, 128, size=shape) / 32.0).astype(np.float32)  # bf16, mostly not E4M3
    d["q_idx"][3, 0] = d["q_idx"][0, 0]
    d["q_idx"][3, 0, HI // 2, dI // 2] = 1.0 + 1.0 / 64  # one value with a longer mantissa
    kd = F.mxfp4_decode(d["k_codes"], d["k_scales"])
    _check_full(C, d, np.array([[9000], [9000], [8191], [5000]], np.int32), 1, 256, k_dense=kd, mx=True,
                what=f"e4m3 / bf16 q {HI}x{dI}")


def test_index_full_mxfp4(C):
    banner("index FULL MXFP4 K_I decode B=2 N=3000 k=128 and prefill T=64")
    g = W.rng(13)
    d = W.indexer_inputs(g, 2, 1, 3000, 64, 128, W.WORKLOADS[5].w_values, k_format="mxfp4")
    kd = F.mxfp4_decode(d["k_codes"], d["k_scales"])
    _check_full(C, d, np.array([[3000], [1234]], np.int32), 1, 128, k_dense=kd, mx=True, what="mxfp4 decode")
    d = W.indexer_inputs(g, 1, 64, 300, 64, 128, W.WORKLOADS[5].w_values, k_format="mxfp4")
    kd = F.mxfp4_decode(d["k_codes"], d["k_scales"])
    _check_full(C, d, (np.arange(64, dtype=np.int32) * 5)[None], 1, 32, k_dense=kd, mx=True, what="mxfp4 prefill")


def test_index_ties_and_zeros(C):
    banner("index FULL all-equal scores and all-negative similarities")
    g = W.rng(14)
    d = W.indexer_inputs(g, 2, 1, 3000, 64, 128, (1.0, -0.5))
    d["k_idx"] = np.zeros_like(d["k_idx"])  # every score is 0: lowest ids win
    idx, _, _ = _check_full(C, d, np.array([[3000], [100]], np.int32), 1, 512, what="zeros")
    np.testing.assert_array_equal(host(idx)[0, 0], np.arange(512))
    d = W.indexer_inputs(g, 1, 1, 2000, 64, 128, (1.0, -1.0), lo=0, hi=1)  # heavy ties
    _check_full(C, d, np.array([[2000]], np.int32), 1, 300, what="ties")


def test_index_topk_row_paths(C):
    banner("index FULL top-512 per query: register rows at 16,384 keys, LDS rows past it, short rows")
    g = W.rng(21)
    # 8 queries of one sequence (not the fused decode path): rows of n_vis = t entries
    d = W.indexer_inputs(g, 1, 8, 16400, 64, 128, (1.0, -1.0, 0.5, -0.5))
    q_pos = np.array([[16384, 16385, 16400, 513, 5000, 512, 1, 0]], np.int32)
    _check_full(C, d, q_pos, 1, 512, what="row lengths around the register capacity")
    # heavy ties in a full register row
    d = W.indexer_inputs(g, 1, 8, 16384, 64, 128, (1.0, -1.0), lo=0, hi=1)
    _check_full(C, d, np.full((1, 8), 16384, np.int32), 1, 512, what="ties, 16,384 keys")


def test_index_topk_many_rows(C):
    banner("index FULL top-128 for 256 queries of 3000 entries (many-row register launch)")
    g = W.rng(22)
    d = W.indexer_inputs(g, 1, 256, 3000, 32, 64, (1.0, -0.5))
    q_pos = np.sort(np.random.default_rng(5).integers(0, 3200, size=(1, 256))).astype(np.int32)
    _check_full(C, d, q_pos, 1, 128, what="many rows")


def _shaped_scores_inputs(g, B, T, N, k0, q0, k1=None, q1=0.0):
    """Indexer inputs whose scores are ReLU(q0 * k0[n] + q1 * k1[n]) exactly: head 0 carries
    two dims, every other head and dim is zero (each product and sum is exact in fp32)."""
    H, D = 64, 128
    q = np.zeros((B, T, H, D), np.float32)
    q[:, :, 0, 0] = q0
    q[:, :, 0, 1] = q1
    k = np.zeros((B, N, D), np.float32)
    k[:, :, 0] = k0
    if k1 is not None:
        k[:, :, 1] = k1
    k[:, :, 2:] = g.ints((B, N, D - 2), -3, 3, dtype="f32")  # met only by zero queries
    w = np.ones((B, T, H), np.float32)
    return {"q_idx": q, "w": w, "k_idx": k}


def test_index_topk_score_shapes(C):
    banner("index FULL top-512 on shaped scores: a large offset over a narrow range, and scores over 80 binades")
    g = W.rng(23)
    r = np.random.default_rng(23)
    # 2^22 + 0.5 j, j < 128: 128 distinct values, 2^16 times the range below the offset, so the
    # first pass's key ranges can miss keys of the boundary bin (the exact gather takes over)
    for B, T, N, q_pos, what in ((1, 8, 16400, [[4000, 5000, 6000, 7000, 8000, 3000, 2500, 16384]], "rows"),
                                 (4, 1, 65536, [[65536], [65536], [40000], [30001]], "chunked decode")):
        k1 = r.integers(0, 128, size=(B, N)).astype(np.float32)
        d = _shaped_scores_inputs(g, B, T, N, 2048.0, 2048.0, k1, 0.5)
        _check_full(C, d, np.asarray(q_pos, np.int32), 1, 512, what=f"offset scores, {what}")
    # 2^e (1 + j/128), e in [-40, 40]: the linear first pass puts almost every key in its
    # lowest bin, and the radix passes resolve it
    for B, T, N, q_pos, what in ((1, 8, 16400, [[16384, 9000, 5000, 16400, 700, 12000, 4096, 2048]], "rows"),
                                 (2, 1, 65536, [[65536], [50000]], "chunked decode")):
        e = r.integers(-40, 41, size=(B, N)).astype(np.float64)
        k0 = (np.exp2(e) * (1.0 + r.integers(0, 128, size=(B, N)) / 128.0)).astype(np.float32)
        d = _shaped_scores_inputs(g, B, T, N, k0, 1.0)
        _check_full(C, d, np.asarray(q_pos, np.int32), 1, 512, what=f"wide scores, {what}")


def test_reindex_reuse_and_hier(C):
    banner("hier pool + REINDEX + REUSE: B=2 N=20000, 64 blocks kept, k=128")
    g = W.rng(15)
    N = 20000
    d = W.indexer_inputs(g, 2, 1, N, 64, 128, W.WORKLOADS[4].w_values)
    q_pos = np.array([[N], [12345]], np.int32)
    _, scores, bmax = _check_full(C, d, q_pos, 1, 128, what="L20")
    n_keep = 64
    cand, cnt = C.csa2_hier_candidates(bmax, i32(q_pos), N, n_keep=n_keep)
    torch.cuda.synchronize()
    gc, gn = host(cand), host(cnt)
    kd = d["k_idx"].astype(np.float64)
    d2 = W.indexer_inputs(g, 2, 1, N, 64, 128, W.WORKLOADS[4].w_values)  # this layer's q_I, w
    refs = []
    for b in range(2):
        nv = int(q_pos[b, 0])
        s = O.indexer_scores(d["q_idx"][b, 0].astype(np.float64), d["w"][b, 0], kd[b], nv)
        want = O.hier_candidates(O.block_max(s), nv, n_keep=n_keep)
        assert gn[b, 0] == len(want)
        np.testing.assert_array_equal(gc[b, 0, :len(want)], want)
        assert np.all(gc[b, 0, len(want):] == -1)
        refs.append(want)
    idx = C.csa2_index_topk(C.CSA2_MODE_REINDEX, i32(q_pos), 128, q_idx=bf16(d2["q_idx"]), w=f32(d2["w"]),
                            m=1, k_idx=bf16(d["k_idx"]), cand=cand, n_cand=cnt)
    torch.cuda.synchronize()
    gi = host(idx)
    for b in range(2):
        want = O.reindex_topk(d2["q_idx"][b, 0].astype(np.float64), d2["w"][b, 0], kd[b], refs[b], 128)
        np.testing.assert_array_equal(gi[b, 0], want)
    out = C.csa2_index_topk(C.CSA2_MODE_REUSE, i32(q_pos), 128, src_idx=idx)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), gi)
    same = C.csa2_index_topk(C.CSA2_MODE_REUSE, i32(q_pos), 128, src_idx=idx, out_idx=idx)
    assert same.data_ptr() == idx.data_ptr()


# =================================================================== attention
def _oracle_attn(q, q_pos, kv, idx, win, win_pos0, n_win, sink, rope_dims, q_norm=True):
    return O.sparse_attn(q, q_pos, kv, idx, win, win_pos0, n_win, sink, rope_dims=rope_dims, q_norm=q_norm)


def test_attn_tiny_prefill_f32(C):
    banner("attn cfg1 f32: T=256 H=8 c=64 k=16 window 16 sink 0 (generic kernel)")
    g = W.rng(1001)
    a = W.attn_inputs(g, 1, 256, 128, 8, 64, Lw=256, io_dtype="f32", sink_std=0.0)
    nv = np.array([[O.n_visible(t, 128, 2) for t in range(256)]])
    idx = W.random_topk_lists(g, 1, 256, nv, 16)
    q_pos = np.arange(256, dtype=np.int32)[None]
    mass = torch.empty((1, 256, 8), device="cuda")
    out = C.csa2_sparse_attn(f32(a["q"]), i32(q_pos), i32(idx), kv=f32(a["kv"]), win=f32(a["win"]),
                             win_pos0=i32([0]), n_win=16, sink=f32(a["sink"]), rope_dims=16, out_mass=mass)
    torch.cuda.synchronize()
    want, wm = _oracle_attn(a["q"], q_pos, a["kv"], idx, a["win"], [0], 16, a["sink"], 16)
    assert_close(host(out), want, **F32_TOL, what="attn cfg1")
    assert_close(host(mass), wm, **F32_TOL, what="mass cfg1")


@pytest.mark.parametrize("kv_format", ["bf16", "fp4"])
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_attn_decode_mfma(C, kv_format, splits):
    banner(f"attn decode MFMA B=3 N=3000 H=64 c=512 k=512 kv={kv_format} splits={splits}")
    g = W.rng(20)
    B, N, L = 3, 3000, 3000
    a = W.attn_inputs(g, B, 1, N, 64, 512, Lw=128, kv_format=kv_format)
    idx = W.random_topk_lists(g, B, 1, np.array([[N], [N], [300]]), 512)  # last query: 300 ids, -1 padded
    q_pos = np.array([[L], [L], [L]], np.int32)
    win_pos0 = np.full(B, L - 127, np.int32)
    kvkw = (dict(kv=bf16(a["kv"])) if kv_format == "bf16"
            else dict(kv_codes=u8(a["kv_codes"]), kv_scales=u8(a["kv_scales"])))
    mass = torch.empty((B, 1, 64), device="cuda")
    out = C.csa2_sparse_attn(bf16(a["q"]), i32(q_pos), i32(idx), win=bf16(a["win"]), win_pos0=i32(win_pos0),
                             n_win=128, sink=f32(a["sink"]), out_mass=mass, num_splits=splits, **kvkw)
    torch.cuda.synchronize()
    kvd = a["kv"] if kv_format == "bf16" else F.fp4_main_decode(a["kv_codes"], a["kv_scales"])
    want, wm = _oracle_attn(a["q"], q_pos, kvd, idx, a["win"], win_pos0, 128, a["sink"], 64)
    assert_close(host(out), want, **BF16_TOL, what=f"attn {kv_format}")
    assert_close(host(mass), wm, atol=1e-2, rtol=1e-2, what="mass")


@pytest.mark.parametrize("splits", [1, 3])
def test_attn_nan_head_leaves_other_heads_exact(C, splits):
    # A zero query head with eps = 0 normalises to 0/0 = NaN, so all its scores are NaN.
    # The softmax reference of the workgroup is fixed on a condition shared by every head
    # (a valid row in the tile), so that head's NaN stays in its own output and the other
    # 63 heads of the workgroup (and of the query) match the oracle.
    banner(f"attn NaN head: B=2 N=3000 H=64 c=512 k=512 eps=0, query 0 head 5 zero, splits={splits}")
    g = W.rng(27)
    B, N, L = 2, 3000, 3000
    a = W.attn_inputs(g, B, 1, N, 64, 512, Lw=128)
    idx = W.random_topk_lists(g, B, 1, N, 512)
    q = np.array(a["q"], np.float32)
    q[0, 0, 5] = 0.0
    q_pos = np.full((B, 1), L, np.int32)
    win_pos0 = np.full(B, L - 127, np.int32)
    out = C.csa2_sparse_attn(bf16(q), i32(q_pos), i32(idx), kv=bf16(a["kv"]), win=bf16(a["win"]),
                             win_pos0=i32(win_pos0), n_win=128, sink=f32(a["sink"]), eps=0.0, num_splits=splits)
    torch.cuda.synchronize()
    with np.errstate(invalid="ignore", divide="ignore"):
        want, _ = O.sparse_attn(q, q_pos, a["kv"], idx, a["win"], win_pos0, 128, a["sink"], rope_dims=64, eps=0.0)
    got = host(out)
    assert np.isnan(want[0, 0, 5]).all()
    keep = np.ones((B, 1, 64), bool)
    keep[0, 0, 5] = False
    assert_close(got[keep], want[keep], **BF16_TOL, what="heads other than the NaN head")


@pytest.mark.parametrize("kv_format", ["bf16", "fp4"])
def test_attn_prefill_mfma_varied_windows_and_heads(C, kv_format):
    banner(f"attn prefill MFMA B=1 T=40 H=128 k=64 kv={kv_format}, windows clipped by position, empty rows")
    g = W.rng(21)
    T, N = 40, 500
    a = W.attn_inputs(g, 1, T, N, 128, 512, Lw=201, kv_format=kv_format)
    q_pos = (np.arange(T, dtype=np.int32) * 5)[None]  # 0 .. 195
    nv = np.minimum(q_pos // 2, N)
    idx = W.random_topk_lists(g, 1, T, nv, 64)
    win_pos0 = np.array([3], np.int32)  # queries before position 3 have no window rows
    kvkw = (dict(kv=bf16(a["kv"])) if kv_format == "bf16"
            else dict(kv_codes=u8(a["kv_codes"]), kv_scales=u8(a["kv_scales"])))
    out = C.csa2_sparse_attn(bf16(a["q"]), i32(q_pos), i32(idx), win=bf16(a["win"]),
                             win_pos0=i32(win_pos0), n_win=128, sink=f32(a["sink"]), **kvkw)
    torch.cuda.synchronize()
    kvd = a["kv"] if kv_format == "bf16" else F.fp4_main_decode(a["kv_codes"], a["kv_scales"])
    want, _ = _oracle_attn(a["q"], q_pos, kvd, idx, a["win"], win_pos0, 128, a["sink"], 64)
    got = host(out)
    assert np.all(got[0, 0] == 0)  # position 0: no visible entry, no window row
    assert_close(got, want, **BF16_TOL, what="attn prefill")


def test_attn_splits_agree(C):
    banner("attn split invariance B=2 N=4000")
    g = W.rng(22)
    a = W.attn_inputs(g, 2, 1, 4000, 64, 512, Lw=128)
    idx = W.random_topk_lists(g, 2, 1, 4000, 512)
    q_pos = np.full((2, 1), 4000, np.int32)
    args = (bf16(a["q"]), i32(q_pos), i32(idx))
    kw = dict(kv=bf16(a["kv"]), win=bf16(a["win"]), win_pos0=i32([3873, 3873]), sink=f32(a["sink"]))
    o1 = host(C.csa2_sparse_attn(*args, num_splits=1, **kw))
    o5 = host(C.csa2_sparse_attn(*args, num_splits=5, **kw))
    o5b = host(C.csa2_sparse_attn(*args, num_splits=5, **kw))
    np.testing.assert_array_equal(o5, o5b)  # deterministic
    assert_close(o5, o1, atol=8e-3, rtol=8e-3, what="splits")



@pytest.mark.parametrize("kv_format", ["bf16", "fp4"])
@pytest.mark.parametrize("splits", [1, 3])
def test_attn_reference_restart(C, kv_format, splits):
    """Selected rows scoring hundreds of log2 units above the first tile's maximum, far
    beyond what the kernel's fixed softmax reference allows: the kernel must raise its
    reference and start the split again, and still give the exact softmax.  Query 0: a row
    at ~100 (slot 100), then two rows at ~390 (slots 300 and 500) that share the softmax,
    so a single split restarts twice.  Query 1: a ~390 row in the first tile (slot 20, no
    restart) and another at slot 511."""
    banner(f"attn reference restart B=2 N=3000 H=64 c=512 k=512 kv={kv_format} splits={splits}")
    g = W.rng(23)
    B, N, L, H, c, r = 2, 3000, 3000, 64, 512, 64
    a = W.attn_inputs(g, B, 1, N, H, c, Lw=128, kv_format=kv_format)
    idx = W.random_topk_lists(g, B, 1, N, 512)
    q = np.array(a["q"], np.float64)
    kvd = (np.array(a["kv"], np.float64) if kv_format == "bf16"
           else F.fp4_main_decode(a["kv_codes"], a["kv_scales"]))
    plants = [[(idx[0, 0, 100], 8.0), (idx[0, 0, 300], 30.0), (idx[0, 0, 500], 30.0)],
              [(idx[1, 0, 20], 30.0), (idx[1, 0, 511], 30.0)]]
    plant_high_scores(g, q, kvd, plants, fp4=kv_format == "fp4")
    if kv_format == "fp4":  # re-encode only the planted rows; the random rows keep their planes
        codes, scales = np.array(a["kv_codes"]), np.array(a["kv_scales"])
        for b in range(B):
            ids = [e for e, _ in plants[b]]
            codes[b, ids], scales[b, ids] = F.quantize_fp4_main(kvd[b, ids])
        assert np.array_equal(F.fp4_main_decode(codes, scales), kvd)
        kvkw = dict(kv_codes=u8(codes), kv_scales=u8(scales))
    else:
        kvkw = dict(kv=bf16(kvd))
    q_pos = np.full((B, 1), L, np.int32)
    win_pos0 = np.full(B, L - 127, np.int32)
    mass = torch.empty((B, 1, H), device="cuda")
    out = C.csa2_sparse_attn(bf16(q), i32(q_pos), i32(idx), win=bf16(a["win"]), win_pos0=i32(win_pos0),
                             n_win=128, sink=f32(a["sink"]), out_mass=mass, num_splits=splits, **kvkw)
    torch.cuda.synchronize()
    want, wm = _oracle_attn(q, q_pos, kvd, idx, a["win"], win_pos0, 128, a["sink"], r)
    assert np.abs(want[:, 0, :, 0]).min() > 20  # every head is dominated by the planted rows
    assert_close(host(out), want, **BF16_TOL, what=f"attn restart {kv_format}")
    assert_close(host(mass), wm, atol=1e-2, rtol=1e-2, what="mass restart")


def test_attn_f32_large_score_jumps(C):
    """The generic kernel's running softmax under the same planted rows: scores ~100 and
    ~410 log2 units above the first rows' (fp32 I/O, c = 64, RoPE on the last 16)."""
    banner("attn f32 large score jumps B=3 N=300 H=4 c=64 k=64 window 16")
    g = W.rng(24)
    B, N, H, c, r = 3, 300, 4, 64, 16
    a = W.attn_inputs(g, B, 1, N, H, c, Lw=64, io_dtype="f32")
    idx = W.random_topk_lists(g, B, 1, N, 64)
    q = np.array(a["q"], np.float64)
    kv = np.array(a["kv"], np.float64)
    plant_high_scores(g, q, kv, [[(idx[b, 0, 5], 15.0), (idx[b, 0, 30], 60.0), (idx[b, 0, 60], 60.0)]
                                 for b in range(B)], aligned=c - r)
    q_pos = np.full((B, 1), 400, np.int32)
    win_pos0 = np.full(B, 400 - 63, np.int32)
    mass = torch.empty((B, 1, H), device="cuda")
    out = C.csa2_sparse_attn(f32(q), i32(q_pos), i32(idx), kv=f32(kv), win=f32(a["win"]), win_pos0=i32(win_pos0),
                             n_win=16, sink=f32(a["sink"]), rope_dims=r, out_mass=mass)
    torch.cuda.synchronize()
    want, wm = _oracle_attn(q, q_pos, kv, idx, a["win"], win_pos0, 16, a["sink"], r)
    assert np.abs(want[:, 0, :, 0]).min() > 50
    assert_close(host(out), want, **F32_TOL, what="attn f32 jumps")
    assert_close(host(mass), wm, **F32_TOL, what="mass f32 jumps")
