"""The no-allocation index call (csa2_index_topk_noalloc) against csa2_index_topk: the same
indices, bit for bit, on two calls in a row (the second smaller, so it runs on what the
first left in the static scratch), through the C ABI; a call too large for the scratch is
refused before anything is enqueued."""
import numpy as np
import pytest
import torch

import oracle as O
from compressed_sparse_attention_gated_amd import workloads as W
from tests._gpu import banner, bf16, f32, host, i32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def C():
    from compressed_sparse_attention_gated_amd import csa2

    csa2.lib()
    return csa2


def _case(C, seed, B, N, k, what):
    banner(f"no-alloc index FULL {what}: B={B} N={N} k={k}")
    g = W.rng(seed)
    d = W.indexer_inputs(g, B, 1, N, 64, 128, W.WORKLOADS[2].w_values)
    q_pos = np.full((B, 1), N, np.int32)
    args = (C.CSA2_MODE_FULL, i32(q_pos), k)
    kw = dict(q_idx=bf16(d["q_idx"]), w=f32(d["w"]), k_idx=bf16(d["k_idx"]))
    want = C.csa2_index_topk(*args, **kw)
    got = torch.full_like(want, -7)
    C.csa2_index_topk_noalloc(*args, out_idx=got, **kw)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(got), host(want))
    # and the oracle agrees (one query)
    s = O.indexer_scores(d["q_idx"][0, 0], d["w"][0, 0], d["k_idx"][0], N)
    np.testing.assert_array_equal(host(got)[0, 0], O.topk_indices(s, k))


def test_noalloc_matches_workspace_call_twice(C):
    _case(C, 9101, 8, 70000, 512, "first call (two-level top-k, fused scan)")
    _case(C, 9102, 3, 20000, 256, "second, smaller call")


def test_noalloc_refuses_oversize(C):
    banner("no-alloc index FULL oversize request (refused on the host)")
    B, T, N, k = 1, 4096, 16384, 512  # prefill-shaped: a 256 MiB score matrix
    q_pos = i32(np.full((B, T), 2 * N, np.int32))
    out = torch.empty((B, T, k), dtype=torch.int32, device="cuda")
    qi = torch.zeros((B, T, 64, 128), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((B, T, 64), device="cuda")
    ki = torch.zeros((B, N, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(C.Csa2Error, match="static array"):
        C.csa2_index_topk_noalloc(C.CSA2_MODE_FULL, q_pos, k, q_idx=qi, w=w, k_idx=ki, m=2, out_idx=out)
