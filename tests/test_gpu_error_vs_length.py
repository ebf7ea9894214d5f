"""Attention error against the fp64 oracle by context length ([DSA-to-CSA notes], checklist
"数值与 kernel": the BF16 / FP4 paths compared with a higher-precision reference, reported by
sequence length).

For each context length L in 4K, 64K, 256K and 1M entries, and for a bf16 cache and an FP4
cache (N(0,1) source rows through RMSNorm and RoPE, quantised by the oracle), two decode
queries at position L attend to 512 random entries plus the 128-token window, 64 heads x 512.
The selection and the attention work do not grow with L; what does is the position, so the
table shows how the query's and the output's rotation hold up at large positions.  Each
cell must be within atol = rtol = 2e-2; with -s the table is printed (max and mean |error|,
and the max relative to the largest output magnitude)."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import formats as F
from compressed_sparse_attention_gated_amd import workloads as W
from tests._gpu import assert_close, banner, bf16, f32, host, i32

pytestmark = pytest.mark.gpu

LENGTHS = (4096, 65536, 262144, 1048576)


@pytest.fixture(scope="module")
def C():
    from compressed_sparse_attention_gated_amd import csa2

    csa2.lib()
    return csa2


def _cache_rows(r, L, pool, fp4):
    """A cache of L entries tiled from `pool` distinct N(0,1) rows after RMSNorm and RoPE (at
    the pool index); FP4 caches are the oracle's quantisation of them."""
    src = r.standard_normal((pool, 512))
    rows = O.rope(O.rms_norm(src), np.arange(pool), 64)
    pick = r.integers(0, pool, L)
    if fp4:
        codes, scales = F.quantize_fp4_main(rows)
        return pick, (codes, scales), F.fp4_main_decode(codes, scales)
    return pick, None, F.bf16_round(rows)


def test_attention_error_by_context_length(C, capsys):
    B, H, c, k, Wn = 2, 64, 512, 512, 128
    lines = ["| cache | context | max abs err | mean abs err | max err / max abs out |", "|---|---|---|---|---|"]
    for fp4 in (False, True):
        for L in LENGTHS:
            kind = "fp4" if fp4 else "bf16"
            banner(f"error vs length: {kind} cache, L={L}, B={B}, top-{k} + {Wn} window")
            r = np.random.default_rng(8000 + L + fp4)
            pick, planes, rows = _cache_rows(r, L, 4096, fp4)
            g = W.rng(8100 + L + fp4)
            att = W.attn_inputs(g, B, 1, 1, H, c, Lw=Wn)
            idx = np.stack([np.sort(r.choice(L, k, replace=False)) for _ in range(B)]).astype(np.int32)[:, None]
            q_pos = np.full((B, 1), L, np.int32)
            win_pos0 = np.full(B, L - Wn + 1, np.int32)
            pk = torch.as_tensor(pick, device="cuda")
            if fp4:
                kv = dict(kv_codes=torch.as_tensor(planes[0], device="cuda")[pk][None].expand(B, L, 256).contiguous(),
                          kv_scales=torch.as_tensor(planes[1], device="cuda")[pk][None].expand(B, L, 32).contiguous())
            else:
                kv = dict(kv=bf16(rows)[pk][None].expand(B, L, c).contiguous())
            out = C.csa2_sparse_attn(bf16(att["q"]), i32(q_pos), i32(idx), win=bf16(att["win"]), win_pos0=i32(win_pos0),
                                     n_win=Wn, sink=f32(att["sink"]), rope_dims=64, **kv)
            torch.cuda.synchronize()
            got = host(out)
            sel = rows[pick[idx[:, 0]]]  # [B, k, c]: the selected entries' values
            want = np.stack([O.sparse_attn(att["q"][b:b + 1], q_pos[b:b + 1], sel[b][None], np.arange(k)[None, None],
                                           att["win"][b:b + 1], win_pos0[b:b + 1], Wn, att["sink"], rope_dims=64)[0][0]
                             for b in range(B)])
            err = np.abs(got - want)
            lines.append(f"| {kind} | {L:,} | {err.max():.3g} | {err.mean():.3g} | {err.max() / np.abs(want).max():.3g} |")
            assert_close(got, want, atol=2e-2, rtol=2e-2, what=f"{kind} L={L}")
            del kv, out
            torch.cuda.empty_cache()
    with capsys.disabled():
        print("\n" + "\n".join(lines), flush=True)
