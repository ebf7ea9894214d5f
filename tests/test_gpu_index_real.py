"""The indexer on real-valued inputs, where scores are not exact in fp32.

q_I and K_I ~ N(0,1) in bf16 and head weights ~ N(0,1) in fp32: the kernels sum the products
in fp32, the oracle in fp64.  Per score, the difference is bounded by the fp32 accumulation
error of the two sums,
    |s_gpu - s_oracle| <= eps_s = 2^-22 * sum_h |w_h| * (d_I * sum_d |q_hd| |k_d|),
(a deliberately loose form of the textbook bound gamma_n <= n u / (1 - n u) for the d_I-term
dot products and the H_I-term head sum, u = 2^-24).  Where the fp32 rounding may reorder
scores, the selected set is checked for what is unique: with each GPU score anywhere in
[s - eps_s, s + eps_s], every entry that is in all possible top-k sets is selected, every
entry in none is not, and the output is ascending, duplicate-free and -1 padded.  The undecided band
must stay small (under a tenth of k), so the check keeps its force."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import formats as F
from compressed_sparse_attention_gated_amd import workloads as W
from tests._gpu import banner, bf16, f32, host, i32, u8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def C():
    from compressed_sparse_attention_gated_amd import csa2

    csa2.lib()
    return csa2


def _bound(q, w, k):
    """eps_s per entry: q [H_I, d_I], w [H_I], k [n, d_I] (fp64 copies of the inputs)."""
    d_I = q.shape[1]
    return 2.0 ** -22 * d_I * (np.abs(k) @ np.abs(q).T @ np.abs(w))


def _check_row(got_idx, got_scores, s_ref, eps, k, what):
    n = len(s_ref)
    assert np.all(np.abs(got_scores[:n] - s_ref) <= eps), f"{what}: score beyond the fp32 bound"
    sel = got_idx[got_idx >= 0]
    assert len(sel) == min(k, n), what
    assert np.all(np.diff(sel) > 0), f"{what}: not ascending / duplicates"
    assert np.all(got_idx[len(sel):] == -1), what
    if n <= k:
        np.testing.assert_array_equal(sel, np.arange(n), err_msg=what)
        return
    # each GPU score lies in [s - eps, s + eps]: an entry whose lower end is above the
    # (k+1)-th largest upper end is in every possible top-k, one whose upper end is below
    # the k-th largest lower end is in none
    lo, hi = s_ref - eps, s_ref + eps
    must = np.nonzero(lo > np.sort(hi)[::-1][k])[0]
    never = np.nonzero(hi < np.sort(lo)[::-1][k - 1])[0]
    assert n - len(must) - len(never) <= max(k // 10, 4), f"{what}: the undecided band is too wide"
    assert np.isin(must, sel).all(), f"{what}: a clearly-above score was not selected"
    assert not np.isin(never, sel).any(), f"{what}: a clearly-below score was selected"


@pytest.mark.parametrize("kfmt", ["bf16", "mxfp4"])
@pytest.mark.parametrize("B,T,N,k", [(2, 1, 9000, 512), (2, 1, 3000, 256), (1, 24, 2000, 128)])
def test_index_real_valued_scores_and_selection(C, kfmt, B, T, N, k):
    banner(f"index FULL real-valued q_I, w; {kfmt} K_I; B={B} T={T} N={N} k={k}")
    g = W.rng(700 + N + k + T + (kfmt == "mxfp4"))
    H_I, d_I = 64, 128
    q = g.normal((B, T, H_I, d_I), dtype="bf16")
    w = g.normal((B, T, H_I), dtype="f32")
    if kfmt == "bf16":
        kk = g.normal((B, N, d_I), dtype="bf16")
        kw = dict(k_idx=bf16(kk))
        kd = kk.astype(np.float64)
    else:
        codes, scales = g.bytes((B, N, d_I // 2)), g.byte_choice((B, N, d_I // 32), (120, 124, 127, 130))
        kw = dict(k_codes=u8(codes), k_scales=u8(scales))
        kd = F.mxfp4_decode(codes, scales)
    q_pos = (np.arange(T, dtype=np.int32)[None] * (N // max(T, 1)) + N // 2 + 1).astype(np.int32).repeat(B, 0)
    q_pos[:, -1] = N
    scores = torch.full((B, T, N), float("nan"), device="cuda")
    idx = C.csa2_index_topk(C.CSA2_MODE_FULL, i32(q_pos), k, q_idx=bf16(q), w=f32(w), m=1, out_scores=scores, **kw)
    torch.cuda.synchronize()
    gi, gs = host(idx), host(scores)
    qd, wd = q.astype(np.float64), w.astype(np.float64)
    for b in range(B):
        for t in range(T):
            nv = O.n_visible(int(q_pos[b, t]), N, 1)
            s_ref = O.indexer_scores(qd[b, t], wd[b, t], kd[b], nv)
            eps = _bound(qd[b, t], wd[b, t], kd[b, :nv])
            _check_row(gi[b, t], gs[b, t], s_ref, eps, k, f"b={b} t={t}")
