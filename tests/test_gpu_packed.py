"""GPU parity of the compressor over packed samples (csa2_compress with cu_seqlens): each
sample compressed on its own inside one token stream, against the fp64 oracle; and the
packed call against separate per-sample calls, byte for byte (entries, K_I, cache planes)."""
import numpy as np
import pytest
import torch

import oracle as O
from compressed_sparse_attention_gated_amd import workloads as W
from tests._gpu import assert_close, banner, bf16, f32, host, i32

pytestmark = pytest.mark.gpu

F32_TOL = dict(atol=1e-4, rtol=1e-4)


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
