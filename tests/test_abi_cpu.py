"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol the header declares, the ctypes descriptors match the C layouts, and argument
validation rejects bad calls before anything is launched."""
import ctypes as C
import os
import re
import subprocess

import pytest
import torch  # noqa: F401  (binds libcsa2 to torch's HIP runtime)

from compressed_sparse_attention_gated_amd import csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


@pytest.fixture(scope="module")
def L():
    return csa2.lib()


def header_functions():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"CSA2_API\s+[\w\s\*]*?\b(csa2_\w+)\s*\(", txt)))


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert sorted(csa2.EXPORTS) == names


def test_single_hip_runtime_in_process(L):
    maps = open("/proc/self/maps").read()
    libs = set(re.findall(r"\S*libamdhip64\S*", maps))
    assert len(libs) == 1, libs


def _c_layout():
    """Compile a tiny C program against the header and read sizeof/offsetof."""
    fields = {
        "csa2_compress_desc": [f[0] for f in csa2.CompressDesc._fields_],
        "csa2_index_desc": [f[0] for f in csa2.IndexDesc._fields_],
        "csa2_hier_desc": [f[0] for f in csa2.HierDesc._fields_],
        "csa2_attn_desc": [f[0] for f in csa2.AttnDesc._fields_],
        "csa2_out_proj_desc": [f[0] for f in csa2.OutProjDesc._fields_],
        "csa2_kernel_time": [f[0] for f in csa2.KernelTime._fields_],
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){"]
    for s, fs in fields.items():
        lines.append(f'printf("{s} size %zu\\n", sizeof({s}));')
        for f in fs:
            lines.append(f'printf("{s} {f} %zu\\n", offsetof({s}, {f}));')
    lines.append("return 0;}")
    tmp = os.path.join("/tmp", f"csa2_layout_{os.getpid()}")
    with open(tmp + ".c", "w") as fh:
        fh.write("\n".join(lines))
    subprocess.run(["gcc", "-std=c99", "-o", tmp, tmp + ".c"], check=True)
    out = subprocess.run([tmp], check=True, capture_output=True, text=True).stdout
    return {tuple(l.split()[:2]): int(l.split()[2]) for l in out.splitlines()}


def test_descriptor_layouts_match_header():
    lay = _c_layout()
    for s, cls in [("csa2_compress_desc", csa2.CompressDesc), ("csa2_index_desc", csa2.IndexDesc),
                   ("csa2_hier_desc", csa2.HierDesc), ("csa2_attn_desc", csa2.AttnDesc),
                   ("csa2_out_proj_desc", csa2.OutProjDesc), ("csa2_kernel_time", csa2.KernelTime)]:
        assert lay[(s, "size")] == C.sizeof(cls), s
        for f, _ in cls._fields_:
            assert lay[(s, f)] == getattr(cls, f).offset, (s, f)


FAKE = C.c_void_p(0x1000)  # never dereferenced: validation fails before any launch


def test_version_and_errors(L):
    assert L.csa2_version() == csa2.ABI_VERSION == 4
    assert L.csa2_compress(None, None) == csa2.CSA2_ERR_INVALID
    assert "null" in csa2.last_error()


def test_compress_validation(L):
    base = dict(B=1, n=8, c=64, m=2, dtype=csa2.CSA2_F32, ca=FAKE, za=FAKE, out=FAKE, eps=1e-6)
    cases = [
        (dict(c=48), csa2.CSA2_ERR_UNSUPPORTED),
        (dict(c=1024), csa2.CSA2_ERR_UNSUPPORTED),
        (dict(m=0), csa2.CSA2_ERR_INVALID),
        (dict(dtype=7), csa2.CSA2_ERR_UNSUPPORTED),
        (dict(ca=None), csa2.CSA2_ERR_INVALID),
        (dict(overlap=1), csa2.CSA2_ERR_INVALID),  # no cb / zb
        (dict(rope_dims=3, rope_theta=1e4), csa2.CSA2_ERR_INVALID),
        (dict(rope_dims=128, rope_theta=1e4), csa2.CSA2_ERR_INVALID),
        (dict(w_ik=FAKE, d_index=128), csa2.CSA2_ERR_INVALID),  # no out_ik
        (dict(w_ik=FAKE, out_ik=FAKE, d_index=100), csa2.CSA2_ERR_UNSUPPORTED),
        (dict(c=16, w_ik=FAKE, out_ik=FAKE, d_index=32), csa2.CSA2_ERR_UNSUPPORTED),  # c * d_index < 1024
        (dict(out_batch_stride=5), csa2.CSA2_ERR_INVALID),
        # write path into the quantised cache
        (dict(out=None), csa2.CSA2_ERR_INVALID),  # no output at all
        (dict(out_codes=FAKE), csa2.CSA2_ERR_INVALID),  # codes without scales
        (dict(c=8, out_codes=FAKE, out_scales=FAKE), csa2.CSA2_ERR_UNSUPPORTED),  # c % 16
        (dict(ik_codes=FAKE, ik_scales=FAKE), csa2.CSA2_ERR_INVALID),  # MXFP4 K_I without w_ik
        (dict(w_ik=FAKE, d_index=128, ik_codes=FAKE), csa2.CSA2_ERR_INVALID),  # no ik_scales
        (dict(q_rows=-1, out_codes=FAKE, out_scales=FAKE), csa2.CSA2_ERR_INVALID),
        (dict(cb0=FAKE, zb0=FAKE), csa2.CSA2_ERR_INVALID),  # history without overlap
        (dict(overlap=1, cb=FAKE, zb=FAKE, cb0=FAKE), csa2.CSA2_ERR_INVALID),  # cb0 without zb0
    ]
    for over, code in cases:
        d = csa2.CompressDesc(**{**base, **over})
        assert L.csa2_compress(C.byref(d), None) == code, (over, csa2.last_error())
    # empty work succeeds without touching the device
    for over in (dict(B=0), dict(n=1), dict(n=0, ca=None), dict(n=0, out=None, out_codes=FAKE)):
        d = csa2.CompressDesc(**{**base, **over})
        assert L.csa2_compress(C.byref(d), None) == csa2.CSA2_OK


def _index(**over):
    base = dict(B=2, T=1, H_I=64, d_I=128, N=100, m=1, k=16, q_idx=FAKE, w=FAKE, q_pos=FAKE,
                k_dtype=csa2.CSA2_BF16, k_idx=FAKE, out_idx=FAKE, block=8)
    return csa2.IndexDesc(**{**base, **over})


def test_index_validation(L):
    F, R, U = csa2.CSA2_MODE_FULL, csa2.CSA2_MODE_REINDEX, csa2.CSA2_MODE_REUSE
    cases = [
        (dict(k=0), F, csa2.CSA2_ERR_INVALID),
        (dict(k=5000), F, csa2.CSA2_ERR_UNSUPPORTED),
        (dict(H_I=65), F, csa2.CSA2_ERR_UNSUPPORTED),
        (dict(d_I=48), F, csa2.CSA2_ERR_UNSUPPORTED),
        (dict(k_idx=None), F, csa2.CSA2_ERR_INVALID),
        (dict(k_dtype=csa2.CSA2_MXFP4, k_idx=None), F, csa2.CSA2_ERR_INVALID),
        (dict(out_block_max=FAKE, block=3), F, csa2.CSA2_ERR_UNSUPPORTED),
        (dict(), R, csa2.CSA2_ERR_INVALID),  # REINDEX without candidates
        (dict(src_idx=None), U, csa2.CSA2_ERR_INVALID),
        (dict(m=0), F, csa2.CSA2_ERR_INVALID),
        # MXFP4 q_I: only with an MXFP4 K_I, and its scales are required
        (dict(q_dtype=csa2.CSA2_MXFP4, q_scales=FAKE), F, csa2.CSA2_ERR_UNSUPPORTED),
        (dict(q_dtype=csa2.CSA2_MXFP4, k_dtype=csa2.CSA2_MXFP4, k_idx=None, k_codes=FAKE, k_scales=FAKE), F,
         csa2.CSA2_ERR_INVALID),
        (dict(q_dtype=csa2.CSA2_FP4_E4M3), F, csa2.CSA2_ERR_UNSUPPORTED),
    ]
    for over, mode, code in cases:
        d = _index(**over)
        assert L.csa2_index_topk(C.byref(d), mode, None, 0, None) == code, (over, csa2.last_error())
    assert L.csa2_index_topk(C.byref(_index()), 9, None, 0, None) == csa2.CSA2_ERR_INVALID
    # a FULL call needs the score workspace; without it nothing is launched
    need = L.csa2_index_workspace_bytes(C.byref(_index()), F)
    assert need >= 2 * 100 * 4
    assert L.csa2_index_topk(C.byref(_index()), F, None, 0, None) == csa2.CSA2_ERR_WORKSPACE
    assert L.csa2_index_topk(C.byref(_index()), F, FAKE, need - 1, None) == csa2.CSA2_ERR_WORKSPACE
    # REUSE needs no workspace; B*T == 0 is a no-op
    assert L.csa2_index_workspace_bytes(C.byref(_index(src_idx=FAKE)), U) == 0
    assert L.csa2_index_topk(C.byref(_index(B=0)), F, None, 0, None) == csa2.CSA2_OK
    for over in (dict(B=0), dict(T=0), dict(B=0, N=70000), dict(T=0, N=0)):
        for mode in (F, R):
            assert L.csa2_index_workspace_bytes(C.byref(_index(**over)), mode) == 0, (over, mode)
    # decode rows (one query per sequence) fuse the chunk top-k into the scan: the
    # workspace holds chunk candidates, far less than a score row
    dec = L.csa2_index_workspace_bytes(C.byref(_index(N=70000)), F)
    assert 0 < dec < 2 * 70000 * 4
    # many queries per sequence keep a score row per query, plus the two-level buffers
    # for rows longer than the single-workgroup limit
    pre = L.csa2_index_workspace_bytes(C.byref(_index(B=1, T=16, N=30000)), F)
    pre_long = L.csa2_index_workspace_bytes(C.byref(_index(B=1, T=16, N=70000)), F)
    assert pre == (16 * 30000 * 4 + 255) // 256 * 256 and pre_long > (16 * 70000 * 4 + 255) // 256 * 256


def test_hier_validation(L):
    base = dict(B=1, T=1, N=1000, m=1, block=8, n_keep=16, q_pos=FAKE, block_max=FAKE,
                out_cand=FAKE, out_count=FAKE)
    for over, code in [(dict(block=3), csa2.CSA2_ERR_UNSUPPORTED), (dict(n_keep=0), csa2.CSA2_ERR_UNSUPPORTED),
                       (dict(out_cand=None), csa2.CSA2_ERR_INVALID), (dict(m=0), csa2.CSA2_ERR_INVALID)]:
        d = csa2.HierDesc(**{**base, **over})
        assert L.csa2_hier_candidates(C.byref(d), FAKE, 1 << 30, None) == code, over
    for over in (dict(B=0), dict(T=0)):  # empty calls: no workspace, nothing launched
        d = csa2.HierDesc(**{**base, **over})
        assert L.csa2_hier_workspace_bytes(C.byref(d)) == 0, over
        assert L.csa2_hier_candidates(C.byref(d), None, 0, None) == csa2.CSA2_OK, over
    d = csa2.HierDesc(**base)
    need = L.csa2_hier_workspace_bytes(C.byref(d))
    assert need > 0
    assert L.csa2_hier_candidates(C.byref(d), FAKE, need - 1, None) == csa2.CSA2_ERR_WORKSPACE


def test_attn_validation(L):
    base = dict(B=1, T=1, H=64, c=512, k=16, N=100, rope_dims=64, rope_theta=1e4, eps=1e-6,
                q_norm=1, q_dtype=csa2.CSA2_BF16, q=FAKE, q_pos=FAKE, kv_dtype=csa2.CSA2_BF16,
                kv=FAKE, idx=FAKE, out=FAKE)
    cases = [
        (dict(c=24), csa2.CSA2_ERR_INVALID),
        (dict(c=1024), csa2.CSA2_ERR_UNSUPPORTED),
        (dict(rope_dims=63), csa2.CSA2_ERR_INVALID),
        (dict(q_dtype=csa2.CSA2_F32), csa2.CSA2_ERR_UNSUPPORTED),  # kv bf16 with f32 q
        (dict(q_dtype=csa2.CSA2_F32, kv_dtype=csa2.CSA2_FP4_E4M3), csa2.CSA2_ERR_UNSUPPORTED),
        (dict(kv_dtype=csa2.CSA2_FP4_E4M3), csa2.CSA2_ERR_INVALID),  # no planes
        (dict(idx=None), csa2.CSA2_ERR_INVALID),
        (dict(kv=None), csa2.CSA2_ERR_INVALID),
        (dict(win=FAKE), csa2.CSA2_ERR_INVALID),  # no win_pos0
        (dict(num_splits=-1), csa2.CSA2_ERR_INVALID),
        (dict(dense_m=-1), csa2.CSA2_ERR_INVALID),
        (dict(dense_m=128), csa2.CSA2_ERR_INVALID),  # dense attention takes no index list
    ]
    for over, code in cases:
        d = csa2.AttnDesc(**{**base, **over})
        assert L.csa2_sparse_attn(C.byref(d), None, 0, None) == code, (over, csa2.last_error())
    # zero-sized calls size no workspace and launch nothing (B, T or H = 0; split choice
    # must not divide by the empty workgroup count)
    for over in (dict(B=0), dict(T=0), dict(H=0), dict(B=0, k=512), dict(T=0, num_splits=0)):
        d = csa2.AttnDesc(**{**base, **over})
        assert L.csa2_attn_workspace_bytes(C.byref(d)) == 0, over
        assert L.csa2_sparse_attn(C.byref(d), None, 0, None) == csa2.CSA2_OK, over
    # a decode batch of 2 queries is split over several workgroups per query -> workspace
    d = csa2.AttnDesc(**{**base, "B": 2, "k": 512})
    need = L.csa2_attn_workspace_bytes(C.byref(d))
    assert need > 0
    assert L.csa2_sparse_attn(C.byref(d), None, 0, None) == csa2.CSA2_ERR_WORKSPACE


def test_profile_collect_empty(L):
    assert csa2.csa2_profile_collect() == []


def test_out_proj_validation(L):
    base = dict(M=4, n_h=8, c=64, g=2, d_g=64, d=64, o=FAKE, w1=FAKE, w2=FAKE, mid=FAKE, out=FAKE)
    for over, code in [(dict(g=3), csa2.CSA2_ERR_INVALID), (dict(c=8), csa2.CSA2_ERR_UNSUPPORTED),
                       (dict(d_g=8, g=2), csa2.CSA2_ERR_UNSUPPORTED), (dict(mid=None), csa2.CSA2_ERR_INVALID),
                       (dict(d=0), csa2.CSA2_ERR_INVALID)]:
        d = csa2.OutProjDesc(**{**base, **over})
        assert L.csa2_out_proj(C.byref(d), None) == code, (over, csa2.last_error())
    d = csa2.OutProjDesc(**{**base, "M": 0, "o": None})
    assert L.csa2_out_proj(C.byref(d), None) == csa2.CSA2_OK


def test_compress_packed_validation(L):
    base = dict(B=1, n=8, c=64, m=2, dtype=csa2.CSA2_F32, ca=FAKE, za=FAKE, out=FAKE, eps=1e-6,
                cu_seqlens=FAKE, n_samples=2)
    for over, code in [(dict(B=2), csa2.CSA2_ERR_INVALID), (dict(n_samples=0), csa2.CSA2_ERR_INVALID),
                       (dict(n_samples=csa2.lib() and 4097), csa2.CSA2_ERR_INVALID),
                       (dict(overlap=1, cb=FAKE, zb=FAKE, cb0=FAKE, zb0=FAKE), csa2.CSA2_ERR_INVALID)]:
        d = csa2.CompressDesc(**{**base, **over})
        assert L.csa2_compress(C.byref(d), None) == code, (over, csa2.last_error())


def test_attn_dense_workspace_counts_every_entry(L):
    # dense mode sizes its split partials over all N entries (k is ignored)
    base = dict(B=2, T=1, H=64, c=512, k=0, N=8192, rope_dims=64, rope_theta=1e4, eps=1e-6, q_norm=1,
                q_dtype=csa2.CSA2_BF16, q=FAKE, q_pos=FAKE, kv_dtype=csa2.CSA2_BF16, kv=FAKE, out=FAKE,
                dense_m=128)
    d = csa2.AttnDesc(**base)
    dense = L.csa2_attn_workspace_bytes(C.byref(d))
    d = csa2.AttnDesc(**{**base, "dense_m": 0, "k": 8192, "idx": FAKE})
    assert dense == L.csa2_attn_workspace_bytes(C.byref(d)) > 0


# ---------------------------------------------------------------- binding argument checks
def test_binding_rejects_bad_tensors_before_any_call():
    # the library reads every buffer as dense memory of one dtype: the binding refuses
    # strided views, wrong dtypes and mismatched plane shapes before anything is called
    import torch

    from compressed_sparse_attention_gated_amd import csa2

    B, T, H, c, N, k = 2, 1, 64, 512, 40, 8
    q = torch.zeros((B, T, H, c), dtype=torch.bfloat16)
    q_pos = torch.zeros((B, T), dtype=torch.int32)
    kv = torch.zeros((B, 2 * N, c), dtype=torch.bfloat16)
    idx64 = torch.zeros((B, T, k), dtype=torch.int64)  # torch.topk's index dtype
    idx = torch.zeros((B, T, k), dtype=torch.int32)
    with pytest.raises(ValueError, match="idx: dtype"):
        csa2.csa2_sparse_attn(q, q_pos, idx64, kv=kv)
    with pytest.raises(ValueError, match="kv: must be contiguous"):
        csa2.csa2_sparse_attn(q, q_pos, idx, kv=kv[:, ::2])  # a strided cache view
    with pytest.raises(ValueError, match="q_pos: dtype"):
        csa2.csa2_sparse_attn(q, q_pos.long(), idx, kv=kv)
    ca = torch.zeros((1, 8, 512), dtype=torch.bfloat16)
    w_ik = torch.zeros((512, 128), dtype=torch.bfloat16)
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)  # noqa: E731
    with pytest.raises(ValueError, match="codes: shape"):  # planes with different row counts
        csa2.csa2_compress(ca, ca, 1, w_ik=w_ik, out_codes=u8(1, 8, 256), out_scales=u8(1, 8, 32),
                           ik_codes=u8(1, 4, 64), ik_scales=u8(1, 4, 4))
    with pytest.raises(ValueError, match="za: dtype"):
        csa2.csa2_compress(ca, ca.float(), 1)
    with pytest.raises(ValueError, match="k_idx: dtype"):
        csa2.csa2_index_topk(csa2.CSA2_MODE_FULL, q_pos, k, q_idx=torch.zeros((B, T, 64, 128), dtype=torch.bfloat16),
                             w=torch.zeros((B, T, 64)), k_idx=torch.zeros((B, N, 128)))
