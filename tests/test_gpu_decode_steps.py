"""Consecutive decode steps against the oracle recomputed over the whole sequence.

A decode loop of a CSA layer with the overlapping m = 2 compressor: a prefill of n0 tokens is
compressed in bulk, then each step takes one new token at position p:
  1. its own row (m = 1: RMSNorm, RoPE at p) goes into the window buffer, so the window of
     the next queries slides by one;
  2. the indexer scores the entries visible at p (floor(p / m), [DSA-to-CSA notes] section
     "因果边界与短滑窗") and keeps the top-k; attention runs over them plus the window
     positions [p - W + 1, p];
  3. when p closes an m-block, the block is compressed alone with the previous block's
     C^b, Z^b rows as its history (cb0, zb0) and appended at the cache's length (dst_row), so
     it becomes visible from p + 1 on ([Evolution blog] §4.1: an entry is written once its
     block is complete).
Every step's indices must equal the oracle's bit for bit and its outputs must be within the
bf16 tolerance of the oracle, whose entries, window rows, selection and attention are all
recomputed from the raw token inputs for the sequence up to p.  The indexer keys are integer
rows (exact scores), one per entry; the main KV entries come from the write path above."""
import numpy as np
import pytest
import torch

import oracle as O
from compressed_sparse_attention_gated_amd import workloads as W
from tests._gpu import assert_close, banner, bf16, f32, host, i32

pytestmark = pytest.mark.gpu

BF16_TOL = dict(atol=2e-2, rtol=2e-2)


@pytest.fixture(scope="module")
def C():
    from compressed_sparse_attention_gated_amd import csa2

    csa2.lib()
    return csa2


def test_decode_steps_window_slides_and_blocks_append(C):
    B, n0, steps, c, m, H, HI, dI, k, Wn, r = 2, 1000, 7, 512, 2, 64, 64, 128, 128, 128, 64
    banner(f"decode steps: B={B} prefill {n0} then {steps} steps, m=2 overlap, k={k}, window {Wn}")
    g = W.rng(6101)
    n = n0 + steps
    cin = W.compress_inputs(g, n, c, m, overlap=True, dtype="bf16", B=B)  # every token's C^a, Z^a, C^b, Z^b
    wsrc = g.normal((B, n, c), dtype="bf16")  # every token's window-row input
    cap = n // m + 4
    k_int = g.ints((B, cap, dI), -3, 3, dtype="bf16")  # indexer key of each entry (exact scores)
    t = {key: bf16(v) for key, v in cin.items()}
    ws_t = bf16(wsrc)
    # ---- prefill: the bulk compressor over tokens [0, n0) and the window rows [n0 - Wn, n0)
    cache = torch.zeros((B, cap, c), dtype=torch.bfloat16, device="cuda")
    C.csa2_compress(t["ca"][:, :n0].contiguous(), t["za"][:, :n0].contiguous(), m, cb=t["cb"][:, :n0].contiguous(),
                    zb=t["zb"][:, :n0].contiguous(), rope_dims=r, out=cache)
    win_pos0 = n0 - Wn
    win = torch.zeros((B, Wn + steps, c), dtype=torch.bfloat16, device="cuda")
    C.csa2_compress(ws_t[:, win_pos0:n0].contiguous(), ws_t[:, win_pos0:n0].contiguous(), 1,
                    pos0=i32(np.full(B, win_pos0, np.int32)), rope_dims=r, out=win)
    n_ent = n0 // m
    for step in range(steps):
        p = n0 + step
        q_pos = np.full((B, 1), p, np.int32)
        # 1. the new token's row into the window buffer (row p - win_pos0)
        C.csa2_compress(ws_t[:, p:p + 1].contiguous(), ws_t[:, p:p + 1].contiguous(), 1,
                        pos0=i32(q_pos[:, 0]), rope_dims=r, out=win[:, p - win_pos0:])
        # 2. index + attention of the query at p
        ind = W.indexer_inputs(g, B, 1, 1, HI, dI, W.WORKLOADS[2].w_values)
        att = W.attn_inputs(g, B, 1, 1, H, c, Lw=1)
        idx = C.csa2_index_topk(C.CSA2_MODE_FULL, i32(q_pos), k, q_idx=bf16(ind["q_idx"]), w=f32(ind["w"]), m=m,
                                k_idx=bf16(k_int))
        out = C.csa2_sparse_attn(bf16(att["q"]), i32(q_pos), idx, kv=cache, win=win,
                                 win_pos0=i32(np.full(B, win_pos0, np.int32)), n_win=Wn, sink=f32(att["sink"]),
                                 rope_dims=r)
        # 3. a block closed by p is compressed alone (history: the previous block's b rows)
        #    and appended at the cache's length
        if (p + 1) % m == 0:
            blk = slice(p + 1 - m, p + 1)
            prev = slice(p + 1 - 2 * m, p + 1 - m)
            C.csa2_compress(t["ca"][:, blk].contiguous(), t["za"][:, blk].contiguous(), m,
                            cb=t["cb"][:, blk].contiguous(), zb=t["zb"][:, blk].contiguous(),
                            cb0=t["cb"][:, prev].contiguous(), zb0=t["zb"][:, prev].contiguous(),
                            pos0=i32(np.full(B, p + 1 - m, np.int32)), rope_dims=r, out=cache,
                            dst_row=i32(np.full(B, n_ent, np.int32)))
            n_ent += 1
        torch.cuda.synchronize()
        gi, go = host(idx), host(out)
        for b in range(B):
            # the oracle over the whole sequence up to p, from the raw token inputs
            e_ref, _ = O.compress(cin["ca"][b, :p + 1], cin["za"][b, :p + 1], m, c_b=cin["cb"][b, :p + 1],
                                  z_b=cin["zb"][b, :p + 1], overlap=True, rope_dims=r)
            w_rows = np.arange(p - Wn + 1, p + 1)
            w_ref, _ = O.compress(wsrc[b, w_rows], wsrc[b, w_rows], 1, rope_dims=r, pos0=int(w_rows[0]))
            nv = O.n_visible(p, cap, m)
            assert nv == p // m and e_ref.shape[0] >= nv
            i_ref = O.topk_indices(O.indexer_scores(ind["q_idx"][b, 0], ind["w"][b, 0], k_int[b], nv), k)
            np.testing.assert_array_equal(gi[b, 0], i_ref, err_msg=f"indices step {step} b={b}")
            o_ref, _ = O.sparse_attn(att["q"][b:b + 1], q_pos[b:b + 1], e_ref[None], i_ref[None, None], w_ref[None],
                                     [int(w_rows[0])], Wn, att["sink"], rope_dims=r)
            assert_close(go[b, 0], o_ref[0, 0], **BF16_TOL, what=f"attention step {step} b={b}")
        # the appended entries equal the oracle's, so later steps read the right cache
        assert_close(host(cache)[:, :n_ent], np.stack([O.compress(cin["ca"][b, :p + 1], cin["za"][b, :p + 1], m,
                                                                   c_b=cin["cb"][b, :p + 1], z_b=cin["zb"][b, :p + 1],
                                                                   overlap=True, rope_dims=r)[0][:n_ent]
                                                       for b in range(B)]), **BF16_TOL, what=f"cache after step {step}")
