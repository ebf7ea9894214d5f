"""GPU parity of the grouped output projection (csa2_out_proj) against the fp64 oracle:
level 1 (per-group projections) and level 2 (the concatenation's projection), bf16 I/O."""
import numpy as np
import pytest
import torch

import oracle as O
from compressed_sparse_attention_gated_amd import workloads as W
from tests._gpu import assert_close, banner, bf16, host

pytestmark = pytest.mark.gpu

BF16_TOL = dict(atol=2e-2, rtol=2e-2)


@pytest.fixture(scope="module")
def C():
    from compressed_sparse_attention_gated_amd import csa2

    csa2.lib()
    return csa2


@pytest.mark.parametrize("M,n_h,c,g,d_g,d", [
    (5, 8, 64, 2, 64, 96),          # tiny, d not a multiple of the 64-column wave tile
    (17, 16, 128, 4, 2032, 200),    # few rows: 32-column split-K tiles, last one half full
    (17, 16, 128, 8, 504, 200),     # few rows: 16-column split-K tiles, last one half full
    (32, 64, 512, 8, 1024, 4096),   # V4-Flash shape at decode (one token per sequence)
    (64, 64, 512, 8, 1024, 4096),   # V4-Flash shape, 64 sequences (four 16-row blocks)
    (40, 16, 128, 4, 2032, 200),    # 33..64 rows: 32-column split-K tiles, last one half full
    (33, 16, 128, 8, 504, 200),     # 33..64 rows: 16-column split-K tiles, one row in block 2
    (300, 64, 512, 8, 1024, 4096),  # many tokens, ragged last row tile
])
def test_out_proj(C, M, n_h, c, g, d_g, d):
    banner(f"out_proj M={M} n_h={n_h} c={c} g={g} d_g={d_g} d={d}")
    g_ = W.rng(71 + M)
    kg = c * n_h // g
    o = g_.normal((M, n_h, c), dtype="bf16")
    w1 = g_.normal((g, d_g, kg), std=kg ** -0.5, dtype="bf16")
    w2 = g_.normal((d, g * d_g), std=(g * d_g) ** -0.5, dtype="bf16")
    mid, out = C.csa2_out_proj(bf16(o), bf16(w1), bf16(w2))
    torch.cuda.synchronize()
    want_mid, want_out = O.grouped_out_proj(o, w1, w2)
    assert_close(host(mid), want_mid, **BF16_TOL, what="level 1")
    assert_close(host(out), want_out, **BF16_TOL, what="out")
    # level 2 on its own: the library's bf16 mid through the oracle's second product
    assert_close(host(out), host(mid) @ w2.astype(np.float64).T, atol=1e-2, rtol=1e-2, what="level 2")
