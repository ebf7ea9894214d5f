"""GPU parity over packed samples (several samples in one token stream): the compressor
(csa2_compress with cu_seqlens) compresses each sample on its own, against the fp64 oracle
and against separate per-sample calls byte for byte; the indexer (ent_base) and the
attention window (win_row0) of a token stay inside its own sample, against the oracle's
packed index and attention."""
import numpy as np
import pytest
import torch

import oracle as O
from compressed_sparse_attention_gated_amd import workloads as W
from tests._gpu import assert_close, banner, bf16, f32, host, i32

pytestmark = pytest.mark.gpu

F32_TOL = dict(atol=1e-4, rtol=1e-4)
BF16_TOL = dict(atol=2e-2, rtol=2e-2)
W_ = W  # the module, where W names a window size below


@pytest.fixture(scope="module")
def C():
    from compressed_sparse_attention_gated_amd import csa2

    csa2.lib()
    return csa2


def test_packed_compress_f32_overlap(C):
    # lengths with tails, a sample shorter than m, an empty one; overlap with bias; rope 16
    banner("packed compress f32 m=2 overlap c=64, 7 samples")
    lens = [37, 1, 0, 64, 9, 2, 33]
    n = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    g = W.rng(81)
    d = W.compress_inputs(g, n, 64, 2, overlap=True, dtype="f32", bias_std=0.1)
    pos0 = np.arange(len(lens), dtype=np.int32) * 1000  # per sample
    cu_e = torch.full((len(lens) + 1,), -7, dtype=torch.int32, device="cuda")
    out, _ = C.csa2_compress(f32(d["ca"]), f32(d["za"]), 2, cb=f32(d["cb"]), zb=f32(d["zb"]), ba=f32(d["ba"]),
                             bb=f32(d["bb"]), pos0=i32(pos0), rope_dims=16, cu_seqlens=i32(cu), out_cu_entries=cu_e)
    torch.cuda.synchronize()
    want_e = []
    for s in range(len(lens)):
        sl = slice(cu[s], cu[s + 1])
        e, _ = O.compress(d["ca"][0, sl], d["za"][0, sl], 2, b_a=d["ba"], c_b=d["cb"][0, sl], z_b=d["zb"][0, sl],
                          b_b=d["bb"], overlap=True, rope_dims=16, pos0=int(pos0[s]))
        want_e.append(e)
    want = np.concatenate(want_e)
    want_cu = np.concatenate([[0], np.cumsum([x // 2 for x in lens])])
    np.testing.assert_array_equal(host(cu_e), want_cu)
    assert_close(host(out)[0, :want.shape[0]], want, **F32_TOL, what="packed entries")
    # the oracle's packed form agrees (its positions start at 0 per sample)
    ent0, _, cu0 = O.compress_packed(d["ca"][0], d["za"][0], 2, cu, c_b=d["cb"][0], z_b=d["zb"][0], b_a=d["ba"],
                                     b_b=d["bb"], rope_dims=0, norm=False)
    np.testing.assert_array_equal(cu0, want_cu)


def test_packed_equals_per_sample_calls(C):
    # bf16, m = 2, projection to MXFP4 and FP4 planes: the packed call writes, row for row,
    # what per-sample calls write
    banner("packed compress bf16 m=2 c=512 d_I=128 planes, 5 samples")
    lens = [300, 5, 128, 1, 77]
    n = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    g = W.rng(82)
    d = W.compress_inputs(g, n, 512, 2, dtype="bf16", d_I=128)
    t = {k: bf16(v) for k, v in d.items()}
    ne = n // 2
    z = lambda *s: torch.zeros(s, dtype=torch.uint8, device="cuda")  # noqa: E731
    planes = dict(out_codes=z(1, ne, 256), out_scales=z(1, ne, 32), ik_codes=z(1, ne, 64), ik_scales=z(1, ne, 4))
    out, ik = C.csa2_compress(t["ca"], t["za"], 2, rope_dims=64, w_ik=t["w_ik"], cu_seqlens=i32(cu), **planes)
    row = 0
    for s in range(len(lens)):
        k = lens[s] // 2
        if k == 0:
            continue
        ca, za = t["ca"][:, cu[s]:cu[s + 1]].contiguous(), t["za"][:, cu[s]:cu[s + 1]].contiguous()
        p1 = dict(out_codes=z(1, k, 256), out_scales=z(1, k, 32), ik_codes=z(1, k, 64), ik_scales=z(1, k, 4))
        o1, k1 = C.csa2_compress(ca, za, 2, rope_dims=64, w_ik=t["w_ik"], **p1)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out)[0, row:row + k], host(o1)[0], err_msg=f"entries of sample {s}")
        np.testing.assert_array_equal(host(ik)[0, row:row + k], host(k1)[0], err_msg=f"K_I of sample {s}")
        for name in p1:
            np.testing.assert_array_equal(host(planes[name])[0, row:row + k], host(p1[name])[0], err_msg=name)
        row += k


# ------------------------------------------------------------------ index + attention over a packed stream
def _packed_meta(lens, m):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu_e = np.concatenate([[0], np.cumsum([L // m for L in lens])]).astype(np.int32)
    n = int(cu[-1])
    sample = np.searchsorted(cu, np.arange(n), side="right") - 1
    pos = (np.arange(n) - cu[sample]).astype(np.int32)
    return cu, cu_e, sample, pos


@pytest.mark.parametrize("case", ["bf16_mfma", "f32_generic"])
def test_packed_stream_compress_index_attention(C, case):
    # Six samples in one token stream (one shorter than m): the compressor writes each
    # sample's entries (positions restarting), the per-token window rows likewise (m = 1);
    # the indexer of a token scores only its sample's visible entries (ent_base), and its
    # window holds only its sample's latest tokens (win_row0).  Indices bit-exact against the
    # oracle's packed top-k; attention against the oracle's own entries and window rows.
    bf = case == "bf16_mfma"
    lens = [300, 1, 257, 130, 64, 181] if bf else [40, 1, 23, 17, 9, 30]
    m = 2
    c, H, HI, dI, k, W, r = (512, 64, 64, 128, 64, 128, 64) if bf else (64, 4, 4, 32, 8, 16, 16)
    banner(f"packed stream {case}: samples {lens} m=2 c={c} H={H} k={k} window {W}")
    g = W_.rng(5301 if bf else 5302)
    cu, cu_e, sample, pos = _packed_meta(lens, m)
    n, ne = int(cu[-1]), int(cu_e[-1])
    dt = "bf16" if bf else "f32"
    cin = W_.compress_inputs(g, n, c, m, dtype=dt, d_I=dI if bf else 0)
    wsrc = g.normal((1, n, c), dtype=dt)
    ind = W_.indexer_inputs(g, 1, n, 1, HI, dI, W_.WORKLOADS[4].w_values)
    att = W_.attn_inputs(g, 1, n, 1, H, c, Lw=1, io_dtype=dt)
    cast = bf16 if bf else f32
    # compressor: entries per sample and the per-token window rows (m = 1), packed
    ent, k_lib = C.csa2_compress(cast(cin["ca"]), cast(cin["za"]), m, rope_dims=r, cu_seqlens=i32(cu),
                                 w_ik=cast(cin["w_ik"]) if bf else None)
    win, _ = C.csa2_compress(cast(wsrc), cast(wsrc), 1, rope_dims=r, cu_seqlens=i32(cu))
    e_ref, k_ref, cu_e_ref = O.compress_packed(cin["ca"][0], cin["za"][0], m, cu, rope_dims=r,
                                               w_ik=cin["w_ik"].astype(np.float64) if bf else None)
    w_ref, _, _ = O.compress_packed(wsrc[0], wsrc[0], 1, cu, rope_dims=r)
    np.testing.assert_array_equal(cu_e_ref, cu_e)
    tol = BF16_TOL if bf else F32_TOL
    assert_close(host(ent)[0, :ne], e_ref, **tol, what="packed entries")
    assert_close(host(win)[0], w_ref, **tol, what="packed window rows")
    # indexer K: integers (bit-exact scores), from the oracle's projection when there is one
    k_int = np.clip(np.rint(2.0 * k_ref), -3, 3) if bf else g.ints((ne, dI), -3, 3, dtype="f32").astype(np.float64)
    qp = i32(pos[None])
    ent_base = i32(cu_e[sample][None])
    idx = C.csa2_index_topk(C.CSA2_MODE_FULL, qp, k, q_idx=bf16(ind["q_idx"]), w=f32(ind["w"]), m=m,
                            k_idx=bf16(k_int[None].astype(np.float32)), ent_base=ent_base)
    win_row0 = i32(cu[sample][None])
    out = C.csa2_sparse_attn(cast(att["q"]), qp, idx, kv=ent[:, :ne].contiguous(), win=win, win_row0=win_row0,
                             n_win=W, sink=f32(att["sink"]), rope_dims=r)
    torch.cuda.synchronize()
    i_ref = O.index_topk_packed(ind["q_idx"][0].astype(np.float64), ind["w"][0], k_int, cu, cu_e, m, k)
    np.testing.assert_array_equal(host(idx)[0], i_ref)
    # every selected id lies in the query's own sample
    gi = host(idx)[0]
    own_lo, own_hi = cu_e[sample][:, None], cu_e[sample + 1][:, None]
    assert np.all((gi == -1) | ((gi >= own_lo) & (gi < own_hi)))
    # attention: the tokens at and around every sample boundary and a random sample of the rest
    rs = np.random.default_rng(3)
    toks = sorted({int(t) for b in cu[:-1] for t in (b, b + 1, b + 2, b + 3) if t < n} |
                  {int(t) for t in (cu[1:] - 1)} | set(rs.integers(0, n, 24 if bf else n).tolist()))
    want, _ = O.sparse_attn_packed(att["q"][0], e_ref, i_ref, w_ref, cu, window=W, sink=att["sink"],
                                   rope_dims=r, tokens=toks)
    got = host(out)[0]
    assert_close(got[toks], want[toks], **tol, what="packed attention")
