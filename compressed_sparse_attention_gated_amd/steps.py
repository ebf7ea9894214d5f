"""The libcsa2 call chains that make up one step of each workload.

Nothing here computes: each class allocates its outputs and workspaces once, then
`run(inputs)` enqueues the library calls of one step on the current stream.  Calls that do
not depend on each other go to a second stream of the same (default) priority and are joined
back before the first call that reads their output, so the step ends on the current stream:
the prefill's window rows beside its entries and index stage, the Full layer's attention
beside the candidate pool and the Reindex scan, and the Reindex / Reuse attentions two at a
time.

  DecodeStep   compress the new token into the window -> index FULL + top-k over every
               cached entry -> sparse attention (bf16 or FP4 main KV, bf16 or MXFP4 K_I).
  HierStep     the decoder group: Full layer (scan, top-k, block max, attention) ->
               candidate pool -> Reindex layer (rescore candidates, top-k, attention) ->
               three Reuse layers (same indices, own query / window / sink).
  PrefillStep  compress a sequence (m = 2, with the indexer-K projection) and its window
               rows (m = 1) -> causal index FULL + top-k per token -> sparse attention.

The layer structure follows [CSA2 column] (modes table, hierarchical indexer) and
[Evolution blog] §4.2-§4.4.
"""
from __future__ import annotations

import torch

from . import csa2 as C


def _ws(nbytes, device):
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _side_stream(device):
    return torch.cuda.Stream(device=device)  # default priority, like the current stream


class DecodeStep:
    def __init__(self, wl, d):
        self.wl = wl
        self.fp4 = wl.kind == "decode_fp4"
        dev = d["q"].device
        B = wl.B
        self.idx = torch.empty((B, 1, wl.k), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, 1, wl.H, wl.c), dtype=torch.bfloat16, device=dev)
        self.ws_index = _ws(C.csa2_index_workspace_bytes(C.CSA2_MODE_FULL, d["q_pos"], wl.k, q_idx=d["q_idx"],
                                                         w=d["w"], m=wl.m, out_idx=self.idx, **self._kidx(d)), dev)
        self.ws_attn = _ws(C.csa2_attn_workspace_bytes(d["q"], d["q_pos"], self.idx, win=d["win"],
                                                       win_pos0=d["win_pos0"], n_win=wl.window, sink=d["sink"],
                                                       rope_dims=wl.rope_dims, out=self.out, **self._kv(d)), dev)

    def _kidx(self, d):
        return dict(k_codes=d["k_codes"], k_scales=d["k_scales"]) if self.fp4 else dict(k_idx=d["k_idx"])

    def _kv(self, d):
        return dict(kv_codes=d["kv_codes"], kv_scales=d["kv_scales"]) if self.fp4 else dict(kv=d["kv"])

    def run(self, d):
        wl = self.wl
        win = d["win"]
        # the new token's row (m = 1: RMSNorm + RoPE at position L) into the window's last slot.
        # (On a second stream beside the scan it gains nothing: the scan holds every CU.)
        C.csa2_compress(d["c_new"], d["z_new"], 1, pos0=d["q_pos"][:, 0], rope_dims=wl.rope_dims,
                        out=win[:, wl.window - 1:, :])
        C.csa2_index_topk(C.CSA2_MODE_FULL, d["q_pos"], wl.k, q_idx=d["q_idx"], w=d["w"], m=wl.m,
                          out_idx=self.idx, workspace=self.ws_index, **self._kidx(d))
        C.csa2_sparse_attn(d["q"], d["q_pos"], self.idx, win=win, win_pos0=d["win_pos0"], n_win=wl.window,
                           sink=d["sink"], rope_dims=wl.rope_dims, out=self.out, workspace=self.ws_attn,
                           **self._kv(d))
        return self.idx, self.out


class HierStep:
    def __init__(self, wl, d):
        self.wl = wl
        dev = d["kv"].device
        B, L = wl.B, wl.L
        nblk = -(-L // wl.block)
        self.bmax = torch.empty((B, 1, nblk), dtype=torch.float32, device=dev)
        self.idx_full = torch.empty((B, 1, wl.k), dtype=torch.int32, device=dev)
        self.idx_re = torch.empty((B, 1, wl.k), dtype=torch.int32, device=dev)
        self.cand = torch.empty((B, 1, wl.n_keep_blocks * wl.block), dtype=torch.int32, device=dev)
        self.count = torch.empty((B, 1), dtype=torch.int32, device=dev)
        self.outs = [torch.empty((B, 1, wl.H, wl.c), dtype=torch.bfloat16, device=dev) for _ in d["layers"]]
        l0, l1 = d["layers"][0], d["layers"][1]
        self.ws_full = _ws(C.csa2_index_workspace_bytes(C.CSA2_MODE_FULL, d["q_pos"], wl.k, q_idx=l0["q_idx"],
                                                        w=l0["w"], k_idx=d["k_idx"], out_idx=self.idx_full,
                                                        out_block_max=self.bmax), dev)
        self.ws_re = _ws(C.csa2_index_workspace_bytes(C.CSA2_MODE_REINDEX, d["q_pos"], wl.k, q_idx=l1["q_idx"],
                                                      w=l1["w"], k_idx=d["k_idx"], cand=self.cand,
                                                      n_cand=self.count, out_idx=self.idx_re), dev)
        self.ws_attn = _ws(C.csa2_attn_workspace_bytes(l0["q"], d["q_pos"], self.idx_full, kv=d["kv"], win=l0["win"],
                                                       win_pos0=d["win_pos0"], n_win=wl.window, sink=l0["sink"],
                                                       rope_dims=wl.rope_dims, out=self.outs[0]), dev)
        self.ws_hier = _ws(C.csa2_hier_workspace_bytes(self.bmax, d["q_pos"], L, block=wl.block,
                                                       n_keep=wl.n_keep_blocks), dev)
        # one attention workspace per stream: attentions on the two streams run at once
        self.ws_attn_side = _ws(self.ws_attn.numel(), dev)
        self.side = _side_stream(dev)

    def _attn(self, d, layer, idx, side=False):
        e = d["layers"][layer]
        wl = self.wl
        C.csa2_sparse_attn(e["q"], d["q_pos"], idx, kv=d["kv"], win=e["win"], win_pos0=d["win_pos0"],
                           n_win=wl.window, sink=e["sink"], rope_dims=wl.rope_dims, out=self.outs[layer],
                           workspace=self.ws_attn_side if side else self.ws_attn,
                           stream=self.side if side else None)

    def run(self, d):
        wl = self.wl
        l0, l1 = d["layers"][0], d["layers"][1]
        main = torch.cuda.current_stream()
        # Full layer: scan every entry, its own top-k, block maxima for the pool
        C.csa2_index_topk(C.CSA2_MODE_FULL, d["q_pos"], wl.k, q_idx=l0["q_idx"], w=l0["w"], k_idx=d["k_idx"],
                          out_idx=self.idx_full, out_block_max=self.bmax, block=wl.block, workspace=self.ws_full)
        # its attention on the second stream, beside the pool and the Reindex scan
        self.side.wait_stream(main)
        self._attn(d, 0, self.idx_full, side=True)
        # candidate pool from the block maxima
        C.csa2_hier_candidates(self.bmax, d["q_pos"], wl.L, block=wl.block, n_keep=wl.n_keep_blocks,
                               out_cand=self.cand, out_count=self.count, workspace=self.ws_hier)
        # Reindex layer: this layer's indexer over the candidates only
        C.csa2_index_topk(C.CSA2_MODE_REINDEX, d["q_pos"], wl.k, q_idx=l1["q_idx"], w=l1["w"], k_idx=d["k_idx"],
                          cand=self.cand, n_cand=self.count, out_idx=self.idx_re, workspace=self.ws_re)
        # Reuse layers: the Reindex layer's indices, in place (no indexer work, no launch)
        for layer in range(2, len(d["layers"])):
            C.csa2_index_topk(C.CSA2_MODE_REUSE, d["q_pos"], wl.k, src_idx=self.idx_re, out_idx=self.idx_re)
        # the Reindex and Reuse attentions read the same indices: alternate the two streams
        self.side.wait_stream(main)
        for layer in range(1, len(d["layers"])):
            self._attn(d, layer, self.idx_re, side=layer % 2 == 0)
        main.wait_stream(self.side)
        return self.idx_full, self.cand, self.count, self.idx_re, self.outs


class HcaDecodeStep:
    """HCA decode ([DSA-to-CSA notes] eq. (20)-(26)): the new token's row into the window,
    then dense attention over every visible m' = 128 entry plus the window.  (The m' = 128
    compressor runs once per 128 tokens, when a block completes; it is not in this step.)"""

    def __init__(self, wl, d):
        self.wl = wl
        dev = d["q"].device
        self.out = torch.empty((wl.B, 1, wl.H, wl.c), dtype=torch.bfloat16, device=dev)
        self.ws_attn = _ws(C.csa2_attn_workspace_bytes(d["q"], d["q_pos"], None, kv=d["kv"], win=d["win"],
                                                       win_pos0=d["win_pos0"], n_win=wl.window, sink=d["sink"],
                                                       rope_dims=wl.rope_dims, out=self.out, dense_m=wl.m), dev)

    def run(self, d):
        wl = self.wl
        win = d["win"]
        C.csa2_compress(d["c_new"], d["z_new"], 1, pos0=d["q_pos"][:, 0], rope_dims=wl.rope_dims,
                        out=win[:, wl.window - 1:, :])
        C.csa2_sparse_attn(d["q"], d["q_pos"], None, kv=d["kv"], win=win, win_pos0=d["win_pos0"],
                           n_win=wl.window, sink=d["sink"], rope_dims=wl.rope_dims, out=self.out,
                           workspace=self.ws_attn, dense_m=wl.m)
        return None, self.out


class PrefillStep:
    def __init__(self, wl, d):
        self.wl = wl
        dev = d["q"].device
        n, c = wl.n_tokens, wl.c
        ne = n // wl.m
        self.entries = torch.empty((1, ne, c), dtype=torch.bfloat16, device=dev)
        self.k_index = torch.empty((1, ne, wl.d_I), dtype=torch.bfloat16, device=dev)
        self.win = torch.empty((1, n, c), dtype=torch.bfloat16, device=dev)
        self.idx = torch.empty((1, n, wl.k), dtype=torch.int32, device=dev)
        self.out = torch.empty((1, n, wl.H, c), dtype=torch.bfloat16, device=dev)
        self.ws_index = _ws(C.csa2_index_workspace_bytes(C.CSA2_MODE_FULL, d["q_pos"], wl.k, q_idx=d["q_idx"],
                                                         w=d["w"], m=wl.m, k_idx=self.k_index,
                                                         out_idx=self.idx), dev)
        self.ws_attn = _ws(C.csa2_attn_workspace_bytes(d["q"], d["q_pos"], self.idx, kv=self.entries, win=self.win,
                                                       win_pos0=self._wp0(dev), n_win=wl.window, sink=d["sink"],
                                                       rope_dims=wl.rope_dims, out=self.out), dev)
        self.wp0 = self._wp0(dev)
        self.side = _side_stream(dev)

    @staticmethod
    def _wp0(dev):
        return torch.zeros(1, dtype=torch.int32, device=dev)

    def run(self, d, k_idx=None):
        """k_idx: the indexer K the index stage reads; default the compressor's projection."""
        wl = self.wl
        main = torch.cuda.current_stream()
        # window rows on the second stream: every token's own row (m = 1 keeps the row; RMSNorm
        # + RoPE at its position); only the attention reads them
        self.side.wait_stream(main)
        C.csa2_compress(d["win_src"], d["win_src"], 1, rope_dims=wl.rope_dims, out=self.win, stream=self.side)
        C.csa2_compress(d["ca"], d["za"], wl.m, rope_dims=wl.rope_dims, out=self.entries, w_ik=d["w_ik"],
                        out_ik=self.k_index)
        C.csa2_index_topk(C.CSA2_MODE_FULL, d["q_pos"], wl.k, q_idx=d["q_idx"], w=d["w"], m=wl.m,
                          k_idx=self.k_index if k_idx is None else k_idx, out_idx=self.idx,
                          workspace=self.ws_index)
        main.wait_stream(self.side)
        C.csa2_sparse_attn(d["q"], d["q_pos"], self.idx, kv=self.entries, win=self.win, win_pos0=self.wp0,
                           n_win=wl.window, sink=d["sink"], rope_dims=wl.rope_dims, out=self.out,
                           workspace=self.ws_attn)
        return self.entries, self.k_index, self.win, self.idx, self.out


def written_fp4_cache(wl, seed, pool_rows=65536):
    """A decode cache of wl.B x wl.L entries written by the library's own write path:
    `pool_rows` source rows ~ N(0,1) go through csa2_compress (m = 1: RMSNorm, RoPE at the
    row's index, FP4 E2M1 codes with E4M3 scales per 16 channels), and as many indexer-K rows
    of integers U{-3..3} through its K_I projection with an identity W_ik and no norm (MXFP4,
    exact for these integers); the pools are tiled over the context by seeded random indices.
    Returns (kv_codes, kv_scales, k_codes, k_scales)."""
    dev = "cuda"
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    c, d_I = wl.c, wl.d_I
    u8 = lambda *s: torch.empty(s, dtype=torch.uint8, device=dev)  # noqa: E731
    src = torch.randn((1, pool_rows, c), generator=g, device=dev).to(torch.bfloat16)
    kv_c, kv_s = u8(1, pool_rows, c // 2), u8(1, pool_rows, c // 16)
    C.csa2_compress(src, src, 1, rope_dims=wl.rope_dims, out_codes=kv_c, out_scales=kv_s, plain_out=False)
    ints = torch.randint(-3, 4, (1, pool_rows, c), generator=g, device=dev).to(torch.bfloat16)
    eye = torch.zeros((c, d_I), dtype=torch.bfloat16, device=dev)
    eye[torch.arange(d_I), torch.arange(d_I)] = 1
    scratch_c, scratch_s = u8(1, pool_rows, c // 2), u8(1, pool_rows, c // 16)
    k_c, k_s = u8(1, pool_rows, d_I // 2), u8(1, pool_rows, d_I // 32)
    C.csa2_compress(ints, ints, 1, norm=False, w_ik=eye, out_codes=scratch_c, out_scales=scratch_s,
                    ik_codes=k_c, ik_scales=k_s, plain_out=False)
    pick_kv = torch.randint(0, pool_rows, (wl.B, wl.L), generator=g, device=dev)
    pick_k = torch.randint(0, pool_rows, (wl.B, wl.L), generator=g, device=dev)
    out = (kv_c[0][pick_kv].contiguous(), kv_s[0][pick_kv].contiguous(), k_c[0][pick_k].contiguous(),
           k_s[0][pick_k].contiguous())
    del pick_kv, pick_k
    return out
