"""Thin Python binding of libcsa2 (ctypes).

Each function has the name of the C entry point it wraps, takes torch tensors that
already live in device memory, fills the C descriptor with their pointers and sizes,
allocates outputs and workspace with torch when the caller does not pass them, and
calls the library on torch's current stream.  No arithmetic of the method happens here.
"""
from __future__ import annotations

import ctypes as C
import os

import torch  # loaded first: libcsa2 then binds to the HIP runtime torch already loaded

_PKG = os.path.dirname(os.path.abspath(__file__))
# CSA2_LIBRARY names another build of the same library (the sanitized host-layer build of
# the CPU checks); by default the in-tree build
LIB_PATH = os.environ.get("CSA2_LIBRARY") or os.path.join(_PKG, "libcsa2.so")

CSA2_OK, CSA2_ERR_INVALID, CSA2_ERR_UNSUPPORTED, CSA2_ERR_HIP, CSA2_ERR_WORKSPACE = 0, -1, -2, -3, -4
CSA2_F32, CSA2_BF16, CSA2_FP4_E4M3, CSA2_MXFP4 = 0, 1, 2, 3
CSA2_MODE_FULL, CSA2_MODE_REINDEX, CSA2_MODE_REUSE = 0, 1, 2

_vp, _i, _f, _i64 = C.c_void_p, C.c_int, C.c_float, C.c_int64


class CompressDesc(C.Structure):
    _fields_ = [("B", _i), ("n", _i), ("c", _i), ("m", _i), ("overlap", _i), ("dtype", _i),
                ("ca", _vp), ("za", _vp), ("cb", _vp), ("zb", _vp), ("ba", _vp), ("bb", _vp),
                ("pos0", _vp), ("norm", _i), ("eps", _f), ("rope_dims", _i), ("rope_theta", _f),
                ("out", _vp), ("out_batch_stride", _i64), ("w_ik", _vp), ("d_index", _i),
                ("out_ik", _vp), ("out_ik_batch_stride", _i64), ("dst_row", _vp),
                ("out_codes", _vp), ("out_scales", _vp), ("ik_codes", _vp), ("ik_scales", _vp),
                ("q_rows", _i64), ("cb0", _vp), ("zb0", _vp), ("cu_seqlens", _vp), ("n_samples", _i),
                ("out_cu_entries", _vp)]


class IndexDesc(C.Structure):
    _fields_ = [("B", _i), ("T", _i), ("H_I", _i), ("d_I", _i), ("N", _i), ("m", _i), ("k", _i),
                ("q_idx", _vp), ("w", _vp), ("q_pos", _vp), ("k_dtype", _i), ("k_idx", _vp),
                ("k_codes", _vp), ("k_scales", _vp), ("cand", _vp), ("n_cand", _vp),
                ("cand_stride", _i), ("src_idx", _vp), ("out_idx", _vp), ("out_block_max", _vp),
                ("block", _i), ("out_scores", _vp), ("ent_base", _vp), ("q_dtype", _i),
                ("q_scales", _vp)]


class HierDesc(C.Structure):
    _fields_ = [("B", _i), ("T", _i), ("N", _i), ("m", _i), ("block", _i), ("n_keep", _i),
                ("q_pos", _vp), ("block_max", _vp), ("out_cand", _vp), ("out_count", _vp)]


class AttnDesc(C.Structure):
    _fields_ = [("B", _i), ("T", _i), ("H", _i), ("c", _i), ("k", _i), ("N", _i),
                ("rope_dims", _i), ("rope_theta", _f), ("eps", _f), ("scale", _f), ("q_norm", _i),
                ("q_dtype", _i), ("q", _vp), ("q_pos", _vp), ("kv_dtype", _i), ("kv", _vp),
                ("kv_codes", _vp), ("kv_scales", _vp), ("idx", _vp), ("win", _vp), ("Lw", _i),
                ("win_pos0", _vp), ("n_win", _i), ("sink", _vp), ("out", _vp), ("out_mass", _vp),
                ("num_splits", _i), ("dense_m", _i), ("win_row0", _vp)]


class OutProjDesc(C.Structure):
    _fields_ = [("M", _i), ("n_h", _i), ("c", _i), ("g", _i), ("d_g", _i), ("d", _i), ("o", _vp),
                ("w1", _vp), ("w2", _vp), ("mid", _vp), ("out", _vp)]


class KernelTime(C.Structure):
    _fields_ = [("name", C.c_char * 48), ("ms", C.c_float)]


EXPORTS = ["csa2_compress", "csa2_index_workspace_bytes", "csa2_index_topk", "csa2_index_topk_noalloc",
           "csa2_hier_workspace_bytes", "csa2_hier_candidates", "csa2_attn_workspace_bytes",
           "csa2_sparse_attn", "csa2_out_proj", "csa2_version", "csa2_last_error", "csa2_profile_enable",
           "csa2_profile_collect"]

_lib = None
# the descriptor layouts below are those of this version of include/csa2.h
ABI_VERSION = 4


def lib():
    """Load libcsa2.so (built in-tree).  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libcsa2.so not found at {LIB_PATH}; build it with "
                           "`python -m compressed_sparse_attention_gated_amd.build`")
    L = C.CDLL(LIB_PATH)
    L.csa2_compress.argtypes = [C.POINTER(CompressDesc), _vp]
    L.csa2_index_workspace_bytes.argtypes = [C.POINTER(IndexDesc), _i]
    L.csa2_index_workspace_bytes.restype = C.c_size_t
    L.csa2_index_topk.argtypes = [C.POINTER(IndexDesc), _i, _vp, C.c_size_t, _vp]
    L.csa2_index_topk_noalloc.argtypes = [C.POINTER(IndexDesc), _i, _vp]
    L.csa2_hier_workspace_bytes.argtypes = [C.POINTER(HierDesc)]
    L.csa2_hier_workspace_bytes.restype = C.c_size_t
    L.csa2_hier_candidates.argtypes = [C.POINTER(HierDesc), _vp, C.c_size_t, _vp]
    L.csa2_attn_workspace_bytes.argtypes = [C.POINTER(AttnDesc)]
    L.csa2_attn_workspace_bytes.restype = C.c_size_t
    L.csa2_sparse_attn.argtypes = [C.POINTER(AttnDesc), _vp, C.c_size_t, _vp]
    L.csa2_out_proj.argtypes = [C.POINTER(OutProjDesc), _vp]
    if L.csa2_version() != ABI_VERSION:  # a library built from other sources: layouts differ
        raise RuntimeError(f"libcsa2.so reports ABI version {L.csa2_version()}, this binding expects "
                           f"{ABI_VERSION}; rebuild it with `python -m compressed_sparse_attention_gated_amd.build`")
    L.csa2_last_error.restype = C.c_char_p
    L.csa2_profile_enable.argtypes = [_i]
    L.csa2_profile_collect.argtypes = [C.POINTER(KernelTime), _i]
    _lib = L
    return L


class Csa2Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"libcsa2 error {code}: {msg}")
        self.code = code


def _check(rc):
    if rc != CSA2_OK:
        raise Csa2Error(rc, lib().csa2_last_error().decode())


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


_I32, _U8, _F32 = (torch.int32,), (torch.uint8,), (torch.float32,)
_DATA = (torch.float32, torch.bfloat16)


def _arg(name, t, dtypes, device, shape=None, rows_view=False):
    """Check one tensor argument before its pointer goes to the library, which reads every
    buffer as dense row-major memory of the stated dtype: it must be on the call's device,
    of one of `dtypes`, contiguous (with rows_view: the last two dims contiguous, any batch
    stride) and, if given, of `shape` (None entries are free).  Raises ValueError."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a torch.Tensor, got {type(t).__name__}")
    if t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
    if rows_view:
        if t.dim() != 3 or t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != t.shape[2]):
            raise ValueError(f"{name}: [B, rows, c] with contiguous rows required (strides {t.stride()})")
    elif not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous (strides {tuple(t.stride())})")
    if shape is not None:
        if t.dim() != len(shape) or any(s is not None and s != d for s, d in zip(shape, t.shape)):
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple('*' if s is None else s for s in shape)}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream)


_DT = {torch.float32: CSA2_F32, torch.bfloat16: CSA2_BF16}


def _ws(nbytes, device):
    return None if nbytes == 0 else torch.empty(nbytes, dtype=torch.uint8, device=device)


def last_error() -> str:
    return lib().csa2_last_error().decode()


def version() -> int:
    return lib().csa2_version()


# ---------------------------------------------------------------------------- compress
def csa2_compress(ca, za, m, *, cb=None, zb=None, ba=None, bb=None, pos0=None, norm=True,
                  eps=1e-6, rope_dims=0, rope_theta=10000.0, out=None, w_ik=None, out_ik=None,
                  dst_row=None, out_codes=None, out_scales=None, ik_codes=None, ik_scales=None,
                  cb0=None, zb0=None, cu_seqlens=None, out_cu_entries=None, plain_out=True, stream=None):
    """ca, za (cb, zb): [B, n, c] fp32/bf16 -> (out [B, n//m, c], out_ik [B, n//m, d_I] or None).

    Write path: out_codes / out_scales [B, rows, c/2] / [B, rows, c/16] (FP4 entries) and
    ik_codes / ik_scales [B, rows, d_I/2] / [B, rows, d_I/32] (MXFP4 K_I), entry i of
    sequence b at row dst_row[b] + i; cb0 / zb0 [B, m, c]: with overlap, the history rows of
    entry 0 (the block before it).  cu_seqlens [S+1] (int32, B = 1): packed samples, each
    compressed on its own; out gets n//m rows (an upper bound), out_cu_entries [S+1] the
    samples' entry offsets.  With plain_out=False and quantised planes given, the
    plain outputs are not allocated (returned as None) unless passed."""
    if not isinstance(ca, torch.Tensor) or ca.dim() != 3:
        raise ValueError("ca: a [B, n, c] tensor is required")
    B, n, c = ca.shape
    ne = n // m
    dv, dt = ca.device, (ca.dtype,)
    _arg("ca", ca, _DATA, dv)
    for name, t in (("za", za), ("cb", cb), ("zb", zb)):
        _arg(name, t, dt, dv, (B, n, c))
    for name, t in (("ba", ba), ("bb", bb)):
        _arg(name, t, _F32, dv, (m, c))
    for name, t in (("cb0", cb0), ("zb0", zb0)):
        _arg(name, t, dt, dv, (B, m, c))
    S = None if cu_seqlens is None else cu_seqlens.numel() - 1
    _arg("pos0", pos0, _I32, dv, (B if S is None else S,))
    _arg("dst_row", dst_row, _I32, dv, (B,))
    _arg("cu_seqlens", cu_seqlens, _I32, dv, (None,))
    _arg("out_cu_entries", out_cu_entries, _I32, dv, (None if S is None else S + 1,))
    _arg("out", out, dt, dv, (B, None, c), rows_view=True)
    d_w = None
    if w_ik is not None:
        _arg("w_ik", w_ik, dt, dv, (c, None))
        d_w = w_ik.shape[1]
    _arg("out_ik", out_ik, dt, dv, (B, None, d_w), rows_view=True)
    # the FP4 and MXFP4 planes share one row count (q_rows bounds both)
    q_rows = 0
    for t in (out_codes, ik_codes):
        if t is not None:
            q_rows = t.shape[1]
    _arg("out_codes", out_codes, _U8, dv, (B, q_rows, c // 2))
    _arg("out_scales", out_scales, _U8, dv, (B, q_rows, c // 16))
    if (ik_codes is not None or ik_scales is not None) and d_w is None:
        raise ValueError("ik_codes / ik_scales need w_ik")
    _arg("ik_codes", ik_codes, _U8, dv, (B, q_rows, None if d_w is None else d_w // 2))
    _arg("ik_scales", ik_scales, _U8, dv, (B, q_rows, None if d_w is None else d_w // 32))
    if out is None and (plain_out or out_codes is None):
        out = torch.empty((B, ne, c), dtype=ca.dtype, device=ca.device)
    d_index = 0
    if w_ik is not None:
        d_index = w_ik.shape[1]
        if out_ik is None and (plain_out or ik_codes is None):
            out_ik = torch.empty((B, ne, d_index), dtype=ca.dtype, device=ca.device)
    d = CompressDesc(B=B, n=n, c=c, m=m, overlap=int(cb is not None), dtype=_DT[ca.dtype],
                     ca=_p(ca), za=_p(za), cb=_p(cb), zb=_p(zb), ba=_p(ba), bb=_p(bb), pos0=_p(pos0),
                     norm=int(norm), eps=eps, rope_dims=rope_dims, rope_theta=rope_theta, out=_p(out),
                     out_batch_stride=out.stride(0) if out is not None and out.dim() == 3 else 0,
                     w_ik=_p(w_ik), d_index=d_index, out_ik=_p(out_ik),
                     out_ik_batch_stride=out_ik.stride(0) if out_ik is not None else 0,
                     dst_row=_p(dst_row), out_codes=_p(out_codes), out_scales=_p(out_scales),
                     ik_codes=_p(ik_codes), ik_scales=_p(ik_scales), q_rows=q_rows, cb0=_p(cb0),
                     zb0=_p(zb0), cu_seqlens=_p(cu_seqlens),
                     n_samples=cu_seqlens.numel() - 1 if cu_seqlens is not None else 0,
                     out_cu_entries=_p(out_cu_entries))
    _check(lib().csa2_compress(C.byref(d), _stream(stream)))
    return out, out_ik


# ---------------------------------------------------------------------------- index + top-k
def _index_desc(q_idx, w, q_pos, k, m, *, k_idx=None, k_codes=None, k_scales=None, N=None,
                cand=None, n_cand=None, src_idx=None, out_idx=None, out_block_max=None, block=8,
                out_scores=None, ent_base=None, q_scales=None):
    if not isinstance(q_pos, torch.Tensor) or q_pos.dim() != 2:
        raise ValueError("q_pos: a [B, T] int32 tensor is required")
    B, T = q_pos.shape
    dv = q_pos.device
    _arg("q_pos", q_pos, _I32, dv, (B, T))
    if q_scales is None:
        _arg("q_idx", q_idx, (torch.bfloat16,), dv, (B, T, None, None))
        H_I, d_I = (q_idx.shape[2], q_idx.shape[3]) if q_idx is not None else (1, 32)
    else:  # MXFP4 q_I: codes [B, T, H_I, d_I/2] and E8M0 scales [B, T, H_I, d_I/32]
        _arg("q_idx", q_idx, _U8, dv, (B, T, None, None))
        if q_idx is None:
            raise ValueError("q_idx: the MXFP4 codes are required with q_scales")
        H_I, d_I = q_idx.shape[2], 2 * q_idx.shape[3]
        _arg("q_scales", q_scales, _U8, dv, (B, T, H_I, d_I // 32))
    _arg("w", w, _F32, dv, (B, T, H_I))
    if N is None:
        N = (k_idx.shape[1] if k_idx is not None else (k_codes.shape[1] if k_codes is not None else 0))
    _arg("k_idx", k_idx, (torch.bfloat16,), dv, (B, N, d_I))
    _arg("k_codes", k_codes, _U8, dv, (B, N, d_I // 2))
    _arg("k_scales", k_scales, _U8, dv, (B, N, d_I // 32))
    _arg("cand", cand, _I32, dv, (B, T, None))
    _arg("n_cand", n_cand, _I32, dv, (B, T))
    _arg("src_idx", src_idx, _I32, dv, (B, T, k))
    _arg("out_idx", out_idx, _I32, dv, (B, T, k))
    _arg("out_block_max", out_block_max, _F32, dv, (B, T, -(-N // block)))
    _arg("out_scores", out_scores, _F32, dv, (B, T, N if cand is None else cand.shape[-1]))
    _arg("ent_base", ent_base, _I32, dv, (B, T))
    return IndexDesc(B=B, T=T, H_I=H_I, d_I=d_I, N=N, m=m, k=k, q_idx=_p(q_idx), w=_p(w),
                     q_pos=_p(q_pos), k_dtype=CSA2_MXFP4 if k_codes is not None else CSA2_BF16,
                     k_idx=_p(k_idx), k_codes=_p(k_codes), k_scales=_p(k_scales), cand=_p(cand),
                     n_cand=_p(n_cand), cand_stride=cand.shape[-1] if cand is not None else 0,
                     src_idx=_p(src_idx), out_idx=_p(out_idx), out_block_max=_p(out_block_max),
                     block=block, out_scores=_p(out_scores), ent_base=_p(ent_base),
                     q_dtype=CSA2_MXFP4 if q_scales is not None else CSA2_BF16, q_scales=_p(q_scales))


def csa2_index_topk(mode, q_pos, k, *, q_idx=None, w=None, m=1, k_idx=None, k_codes=None,
                    k_scales=None, N=None, cand=None, n_cand=None, src_idx=None, out_idx=None,
                    out_block_max=None, block=8, out_scores=None, ent_base=None, q_scales=None,
                    workspace=None, stream=None):
    """FULL / REINDEX / REUSE.  Returns out_idx [B, T, k] int32.  ent_base [B, T] (FULL):
    packed samples, the first entry id of each query's sample (q_pos is sample-local).
    q_scales [B, T, H_I, d_I/32] uint8: q_idx holds MXFP4 codes [B, T, H_I, d_I/2] (with an
    MXFP4 K_I)."""
    B, T = q_pos.shape
    dev = q_pos.device
    if out_idx is None:
        out_idx = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    d = _index_desc(q_idx, w, q_pos, k, m, k_idx=k_idx, k_codes=k_codes, k_scales=k_scales, N=N,
                    cand=cand, n_cand=n_cand, src_idx=src_idx, out_idx=out_idx,
                    out_block_max=out_block_max, block=block, out_scores=out_scores, ent_base=ent_base,
                    q_scales=q_scales)
    nbytes = lib().csa2_index_workspace_bytes(C.byref(d), mode)
    if workspace is None or workspace.numel() < nbytes:
        workspace = _ws(nbytes, dev)
    _check(lib().csa2_index_topk(C.byref(d), mode, _p(workspace), nbytes, _stream(stream)))
    return out_idx


def csa2_index_topk_noalloc(mode, q_pos, k, *, q_idx=None, w=None, m=1, k_idx=None, k_codes=None,
                            k_scales=None, N=None, cand=None, n_cand=None, src_idx=None, out_idx=None,
                            out_block_max=None, block=8, out_scores=None, ent_base=None, q_scales=None,
                            stream=None):
    """csa2_index_topk with the library's static scratch instead of a workspace (for callers
    that cannot allocate).  out_idx must be given: nothing is allocated."""
    if out_idx is None:
        raise ValueError("out_idx is required: the no-allocation call allocates nothing")
    d = _index_desc(q_idx, w, q_pos, k, m, k_idx=k_idx, k_codes=k_codes, k_scales=k_scales, N=N,
                    cand=cand, n_cand=n_cand, src_idx=src_idx, out_idx=out_idx,
                    out_block_max=out_block_max, block=block, out_scores=out_scores, ent_base=ent_base,
                    q_scales=q_scales)
    _check(lib().csa2_index_topk_noalloc(C.byref(d), mode, _stream(stream)))
    return out_idx


def csa2_index_workspace_bytes(mode, q_pos, k, **kw):
    d = _index_desc(kw.get("q_idx"), kw.get("w"), q_pos, k, kw.get("m", 1), k_idx=kw.get("k_idx"),
                    k_codes=kw.get("k_codes"), k_scales=kw.get("k_scales"), N=kw.get("N"),
                    cand=kw.get("cand"), n_cand=kw.get("n_cand"), src_idx=kw.get("src_idx"),
                    out_idx=kw.get("out_idx"), out_block_max=kw.get("out_block_max"),
                    block=kw.get("block", 8), out_scores=kw.get("out_scores"), ent_base=kw.get("ent_base"),
                    q_scales=kw.get("q_scales"))
    return lib().csa2_index_workspace_bytes(C.byref(d), mode)


# ---------------------------------------------------------------------------- hierarchical pool
def csa2_hier_candidates(block_max, q_pos, N, *, m=1, block=8, n_keep=2048, out_cand=None,
                         out_count=None, workspace=None, stream=None):
    """block_max [B, T, ceil(N/block)] -> (cand [B, T, n_keep*block], count [B, T])."""
    B, T = q_pos.shape
    dev = q_pos.device
    _arg("q_pos", q_pos, _I32, dev, (B, T))
    _arg("block_max", block_max, _F32, dev, (B, T, -(-N // block)))
    _arg("out_cand", out_cand, _I32, dev, (B, T, n_keep * block))
    _arg("out_count", out_count, _I32, dev, (B, T))
    if out_cand is None:
        out_cand = torch.empty((B, T, n_keep * block), dtype=torch.int32, device=dev)
    if out_count is None:
        out_count = torch.empty((B, T), dtype=torch.int32, device=dev)
    d = HierDesc(B=B, T=T, N=N, m=m, block=block, n_keep=n_keep, q_pos=_p(q_pos),
                 block_max=_p(block_max), out_cand=_p(out_cand), out_count=_p(out_count))
    nbytes = lib().csa2_hier_workspace_bytes(C.byref(d))
    if workspace is None or workspace.numel() < nbytes:
        workspace = _ws(nbytes, dev)
    _check(lib().csa2_hier_candidates(C.byref(d), _p(workspace), nbytes, _stream(stream)))
    return out_cand, out_count


def csa2_hier_workspace_bytes(block_max, q_pos, N, *, m=1, block=8, n_keep=2048):
    B, T = q_pos.shape
    d = HierDesc(B=B, T=T, N=N, m=m, block=block, n_keep=n_keep, q_pos=_p(q_pos), block_max=_p(block_max),
                 out_cand=None, out_count=None)
    return lib().csa2_hier_workspace_bytes(C.byref(d))


# ---------------------------------------------------------------------------- attention
def _attn_desc(q, q_pos, idx, *, kv=None, kv_codes=None, kv_scales=None, N=None, win=None,
               win_pos0=None, n_win=128, sink=None, rope_dims=64, rope_theta=10000.0, eps=1e-6,
               scale=0.0, q_norm=True, out=None, out_mass=None, num_splits=0, dense_m=0, win_row0=None):
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q: a [B, T, H, c] tensor is required")
    B, T, H, c = q.shape
    dv, dt = q.device, (q.dtype,)
    _arg("q", q, _DATA, dv)
    _arg("q_pos", q_pos, _I32, dv, (B, T))
    _arg("idx", idx, _I32, dv, (B, T, None))
    if N is None:
        N = kv.shape[1] if kv is not None else (kv_codes.shape[1] if kv_codes is not None else 0)
    _arg("kv", kv, dt, dv, (B, N, c))
    _arg("kv_codes", kv_codes, _U8, dv, (B, N, c // 2))
    _arg("kv_scales", kv_scales, _U8, dv, (B, N, c // 16))
    _arg("win", win, dt, dv, (B, None, c))
    _arg("win_pos0", win_pos0, _I32, dv, (B,))
    _arg("sink", sink, _F32, dv, (H,))
    _arg("out", out, dt, dv, (B, T, H, c))
    _arg("out_mass", out_mass, _F32, dv, (B, T, H))
    _arg("win_row0", win_row0, _I32, dv, (B, T))
    kvdt = CSA2_FP4_E4M3 if kv_codes is not None else _DT[q.dtype]
    return AttnDesc(B=B, T=T, H=H, c=c, k=idx.shape[-1] if idx is not None else 0, N=N,
                    rope_dims=rope_dims, rope_theta=rope_theta, eps=eps, scale=scale,
                    q_norm=int(q_norm), q_dtype=_DT[q.dtype], q=_p(q), q_pos=_p(q_pos),
                    kv_dtype=kvdt, kv=_p(kv), kv_codes=_p(kv_codes), kv_scales=_p(kv_scales),
                    idx=_p(idx), win=_p(win), Lw=win.shape[1] if win is not None else 0,
                    win_pos0=_p(win_pos0), n_win=n_win if win is not None else 0, sink=_p(sink),
                    out=_p(out), out_mass=_p(out_mass), num_splits=num_splits, dense_m=dense_m,
                    win_row0=_p(win_row0))


def csa2_sparse_attn(q, q_pos, idx, *, kv=None, kv_codes=None, kv_scales=None, N=None, win=None,
                     win_pos0=None, n_win=128, sink=None, rope_dims=64, rope_theta=10000.0,
                     eps=1e-6, scale=0.0, q_norm=True, out=None, out_mass=None, num_splits=0,
                     dense_m=0, win_row0=None, workspace=None, stream=None):
    """q [B, T, H, c] -> out [B, T, H, c] (dtype of q).  dense_m > 0 (idx None): dense
    attention over every entry visible at the query's position (entries of dense_m tokens).
    win_row0 [B, T]: packed samples, the window row of position 0 of each query's sample."""
    if out is None:
        out = torch.empty_like(q)
    d = _attn_desc(q, q_pos, idx, kv=kv, kv_codes=kv_codes, kv_scales=kv_scales, N=N, win=win,
                   win_pos0=win_pos0, n_win=n_win, sink=sink, rope_dims=rope_dims,
                   rope_theta=rope_theta, eps=eps, scale=scale, q_norm=q_norm, out=out,
                   out_mass=out_mass, num_splits=num_splits, dense_m=dense_m, win_row0=win_row0)
    nbytes = lib().csa2_attn_workspace_bytes(C.byref(d))
    if workspace is None or workspace.numel() < nbytes:
        workspace = _ws(nbytes, q.device)
    _check(lib().csa2_sparse_attn(C.byref(d), _p(workspace), nbytes, _stream(stream)))
    return out


def csa2_attn_workspace_bytes(q, q_pos, idx, **kw):
    d = _attn_desc(q, q_pos, idx, **kw)
    return lib().csa2_attn_workspace_bytes(C.byref(d))


# ---------------------------------------------------------------------------- output projection
def csa2_out_proj(o, w1, w2, *, mid=None, out=None, stream=None):
    """o [..., n_h, c] bf16; w1 [g, d_g, c*n_h/g]; w2 [d, g*d_g] -> (mid [M, g*d_g], out [M, d])."""
    n_h, c = o.shape[-2], o.shape[-1]
    M = o.numel() // (n_h * c)
    g, d_g = w1.shape[0], w1.shape[1]
    dd = w2.shape[0]
    bf, dv = (torch.bfloat16,), o.device
    _arg("o", o, bf, dv)
    _arg("w1", w1, bf, dv, (g, d_g, c * n_h // g))
    _arg("w2", w2, bf, dv, (dd, g * d_g))
    _arg("mid", mid, bf, dv, (M, g * d_g))
    _arg("out", out, bf, dv, (M, dd))
    if mid is None:
        mid = torch.empty((M, g * d_g), dtype=torch.bfloat16, device=o.device)
    if out is None:
        out = torch.empty((M, dd), dtype=torch.bfloat16, device=o.device)
    d = OutProjDesc(M=M, n_h=n_h, c=c, g=g, d_g=d_g, d=dd, o=_p(o), w1=_p(w1), w2=_p(w2), mid=_p(mid),
                    out=_p(out))
    _check(lib().csa2_out_proj(C.byref(d), _stream(stream)))
    return mid, out


# ---------------------------------------------------------------------------- kernel timing
def csa2_profile_enable(on: bool = True):
    _check(lib().csa2_profile_enable(int(on)))


def csa2_profile_collect(max_records: int = 4096):
    """Wait for the recorded events; return [(kernel name, ms)] in launch order."""
    buf = (KernelTime * max_records)()
    n = lib().csa2_profile_collect(buf, max_records)
    if n < 0:
        _check(n)
    return [(buf[i].name.decode(), float(buf[i].ms)) for i in range(n)]
