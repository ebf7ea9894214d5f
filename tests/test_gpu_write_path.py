"""GPU parity of the write path into the decode cache: csa2_compress with FP4 entry planes
and MXFP4 indexer-K planes, appended at a per-sequence row.

The quantised bytes are decided from fp32 entry values.  The oracle's quantiser is exact
(fp64) and the kernel's decisions are exact in fp32, so for the same fp32 values the bytes
must agree bit for bit.  The fp32 values are the kernel's own: the same call with plain fp32
outputs (the epilogue computes them once and stores them in both forms).  Those values are
themselves checked against the fp64 compressor, and the dequantised planes against the fp64
entries (within one scale unit, the E2M1 rounding bound)."""
import numpy as np
import pytest
import torch

import oracle as O
from oracle import formats as F
from compressed_sparse_attention_gated_amd import workloads as W
from tests._gpu import assert_close, banner, bf16, f32, host, i32

pytestmark = pytest.mark.gpu

F32_TOL = dict(atol=1e-4, rtol=1e-4)


@pytest.fixture(scope="module")
def C():
    from compressed_sparse_attention_gated_amd import csa2

    csa2.lib()
    return csa2


def _planes(B, rows, c, d):
    z = lambda *s: torch.zeros(s, dtype=torch.uint8, device="cuda")  # noqa: E731
    return dict(out_codes=z(B, rows, c // 2), out_scales=z(B, rows, c // 16),
                ik_codes=z(B, rows, d // 2), ik_scales=z(B, rows, d // 32))


def _expect(ent, kix, dst, rows):
    """oracle write path per sequence, on the kernel's fp32 entries"""
    outs = [O.write_cache(ent[b], kix[b], int(dst[b]), rows) for b in range(ent.shape[0])]
    return [np.stack([o[j] for o in outs]) for j in range(4)]


def _check_planes(got, want, what):
    names = ("out_codes", "out_scales", "ik_codes", "ik_scales")
    for n, w in zip(names, want):
        g = host(got[n])
        bad = np.argwhere(g != w)
        assert bad.size == 0, f"{what} {n}: {len(bad)} bytes differ, first at {tuple(bad[0])}: got {g[tuple(bad[0])]} want {w[tuple(bad[0])]}"


# ---- threshold straddles.  Every byte the write path stores is decided by comparing an
# fp32 value with a threshold (an E2M1 midpoint times the scale, an E4M3 midpoint for
# amax/6, a power of two for the MXFP4 exponent).  The kernel's fp32 entries differ from
# the oracle's fp64 entries by at most the fp32 rounding of the arithmetic that made them,
# so a byte may differ from the oracle's only where the fp64 value lies within that bound
# of the threshold deciding it.  The bounds: main entries (|x| <= 8 after RMSNorm and RoPE)
# carry a few fp32 ulps, 3e-5 absolute; K_I is a 512-term fp32 dot product whose rounding
# is at most 512 * 2^-24 * sum_i |x_i w_i| (the worst-case summation bound).
E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
_E4M3_GRID = F.E4M3_TABLE[:0x7F]
E4M3_MIDS = (_E4M3_GRID[1:] + _E4M3_GRID[:-1]) / 2
ENTRY_EPS = 3e-5


def _near(x, mids, eps):
    return np.min(np.abs(np.abs(x)[..., None] - mids), axis=-1) <= eps


def _straddles_fp4(e64, codes_ref, scales_ref, eps):
    """(code byte allowed to differ [ne, c/2], scale byte allowed to differ [ne, c/16])."""
    ne, c = e64.shape
    g = e64.reshape(ne, c // 16, 16)
    eps_g = np.broadcast_to(eps, e64.shape).reshape(ne, c // 16, 16).max(axis=-1)
    scale_st = _near(np.abs(g).max(axis=-1) / 6.0, E4M3_MIDS, eps_g / 6.0)
    s = np.repeat(F.e4m3_decode(scales_ref), 16, axis=-1)
    safe = np.where(s > 0, s, 1.0)
    code_st = _near(e64 / safe, E2M1_MIDS, np.broadcast_to(eps, e64.shape) / safe) & (s > 0)
    code_ok = np.repeat(scale_st, 8, axis=-1) | code_st[:, 0::2] | code_st[:, 1::2]
    return code_ok, scale_st


def _straddles_mx(k64, codes_ref, scales_ref, eps):
    ne, d = k64.shape
    g = k64.reshape(ne, d // 32, 32)
    amax = np.abs(g).max(axis=-1)
    eps_g = eps.reshape(ne, d // 32, 32).max(axis=-1)
    j = np.round(np.log2(np.where(amax > 0, amax, 1.0)))
    scale_st = (np.abs(amax - np.exp2(j)) <= eps_g) | (amax <= eps_g)
    s = np.repeat(F.e8m0_decode(scales_ref), 32, axis=-1)
    code_st = _near(k64 / s, E2M1_MIDS, eps / s)
    code_ok = np.repeat(scale_st, 16, axis=-1) | code_st[:, 0::2] | code_st[:, 1::2]
    return code_ok, scale_st


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_write_path_planes_vs_oracle_entries(C, dtype):
    # the planes against the oracle's write path applied to the oracle's own fp64 entries:
    # equal byte for byte except where the fp64 value straddles a threshold (above)
    banner(f"write path vs oracle entries {dtype}: m=2 overlap n=301 c=512 B=2 d_I=128")
    g = W.rng(4107)
    B, n, c, dI, m = 2, 301, 512, 128, 2
    d = W.compress_inputs(g, n, c, m, overlap=True, dtype=dtype, bias_std=0.1, d_I=dI, B=B)
    pos0 = np.array([0, 4096], np.int32)
    dst = np.array([3, 17], np.int32)
    ne = n // m
    rows = ne + 20
    cast = bf16 if dtype == "bf16" else f32
    planes = _planes(B, rows, c, dI)
    C.csa2_compress(cast(d["ca"]), cast(d["za"]), m, cb=cast(d["cb"]), zb=cast(d["zb"]), ba=f32(d["ba"]),
                    bb=f32(d["bb"]), pos0=i32(pos0), rope_dims=64, w_ik=cast(d["w_ik"]), dst_row=i32(dst),
                    plain_out=False, **planes)
    torch.cuda.synchronize()
    got = {k: host(v) for k, v in planes.items()}
    n_diff = n_total = 0
    w64 = d["w_ik"].astype(np.float64)
    for b in range(B):
        e64, k64 = O.compress(d["ca"][b], d["za"][b], m, b_a=d["ba"], c_b=d["cb"][b], z_b=d["zb"][b],
                              b_b=d["bb"], overlap=True, rope_dims=64, pos0=int(pos0[b]), w_ik=w64)
        want = O.write_cache(e64, k64, int(dst[b]), rows)
        r = slice(dst[b], dst[b] + ne)
        xh = O.rms_norm(O.gated_pool(d["ca"][b], d["za"][b], m, b_a=d["ba"], c_b=d["cb"][b], z_b=d["zb"][b],
                                     b_b=d["bb"], overlap=True))
        k_eps = 512 * 2.0 ** -24 * (np.abs(xh) @ np.abs(w64))
        code_ok, scale_ok = _straddles_fp4(e64, want[0][r], want[1][r], ENTRY_EPS)
        ik_code_ok, ik_scale_ok = _straddles_mx(k64, want[2][r], want[3][r], k_eps)
        for name, j, ok in (("out_codes", 0, code_ok), ("out_scales", 1, scale_ok), ("ik_codes", 2, ik_code_ok),
                            ("ik_scales", 3, ik_scale_ok)):
            gb, wb = got[name][b], want[j]
            # rows outside the written range stay zero on both sides
            np.testing.assert_array_equal(np.delete(gb, np.s_[r], axis=0), np.delete(wb, np.s_[r], axis=0))
            diff = gb[r] != wb[r]
            bad = diff & ~ok
            assert not bad.any(), (f"{name} b={b}: {bad.sum()} bytes differ with no threshold straddle, first at "
                                   f"{tuple(np.argwhere(bad)[0])}")
            n_diff += int(diff.sum())
            n_total += diff.size
    assert n_diff <= 0.005 * n_total, (n_diff, n_total)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_write_path_planes_bit_exact(C, dtype):
    banner(f"write path {dtype}: m=2 overlap n=301 c=512 B=2 d_I=128 rope64 dst_row")
    g = W.rng(4101)
    B, n, c, dI, m = 2, 301, 512, 128, 2
    d = W.compress_inputs(g, n, c, m, overlap=True, dtype=dtype, bias_std=0.1, d_I=dI, B=B)
    pos0 = np.array([0, 4096], np.int32)
    dst = np.array([3, 17], np.int32)
    ne = n // m
    rows = ne + 20
    # the kernel's fp32 entries: the same computation with plain fp32 outputs (bf16 inputs
    # are exact in fp32, so the f32 path sees the same numbers)
    ref_kw = dict(cb=f32(d["cb"]), zb=f32(d["zb"]), ba=f32(d["ba"]), bb=f32(d["bb"]), pos0=i32(pos0),
                  rope_dims=64, w_ik=f32(d["w_ik"]))
    ent32, ik32 = C.csa2_compress(f32(d["ca"]), f32(d["za"]), m, **ref_kw)
    cast = bf16 if dtype == "bf16" else f32
    planes = _planes(B, rows, c, dI)
    out, ik = C.csa2_compress(cast(d["ca"]), cast(d["za"]), m, cb=cast(d["cb"]), zb=cast(d["zb"]),
                              ba=f32(d["ba"]), bb=f32(d["bb"]), pos0=i32(pos0), rope_dims=64,
                              w_ik=cast(d["w_ik"]), dst_row=i32(dst), plain_out=False, **planes)
    torch.cuda.synchronize()
    assert out is None and ik is None
    e, k = host(ent32), host(ik32)
    _check_planes(planes, _expect(e, k, dst, rows), f"write path {dtype}")
    # the fp32 entries are the compressor's, and the planes decode to within one scale unit
    for b in range(B):
        want, want_ik = O.compress(d["ca"][b], d["za"][b], m, b_a=d["ba"], c_b=d["cb"][b], z_b=d["zb"][b],
                                   b_b=d["bb"], overlap=True, rope_dims=64, pos0=int(pos0[b]),
                                   w_ik=d["w_ik"].astype(np.float64))
        assert_close(e[b], want, **F32_TOL, what="fp32 entries")
        assert_close(k[b], want_ik, **F32_TOL, what="fp32 K_I")
        r = slice(dst[b], dst[b] + ne)
        deq = F.fp4_main_decode(host(planes["out_codes"])[b, r], host(planes["out_scales"])[b, r])
        step = np.repeat(F.e4m3_decode(host(planes["out_scales"])[b, r]), 16, axis=-1)
        assert np.all(np.abs(deq - want) <= step + 1e-4)


def test_write_path_exact_ties(C):
    # m = 1 without norm or rope writes the input itself, so groups can sit exactly on the
    # rounding thresholds: E2M1 midpoints times the scale, E4M3 scale midpoints, zero groups.
    banner("write path ties: m=1 f32 c=512 identity projection")
    c, dI = 512, 128
    r = np.random.Generator(np.random.PCG64(77))
    x = r.standard_normal((1, 6, c)).astype(np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -1.75, -5.0, 0.0, 6.0, -6.0, 3.0, 0.5, 1.0])
    x[0, 0, :16] = mids                      # amax 6 -> scale 1 exactly
    x[0, 0, 16:32] = mids * 0.125            # amax 0.75 -> scale 0.125
    x[0, 1, :16] = 0.0                       # zero group -> scale 0, zero codes
    x[0, 1, 16:32] = np.r_[6.375, np.zeros(15)]        # amax/6 on an E4M3 midpoint -> even byte
    on_ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -1.75, -5.0, 0.0, 0.5, 1.0, 3.0, 1.5])
    x[0, 1, 32:48] = np.r_[-7.125, 1.25 * on_ties]    # amax/6 = 1.1875, a midpoint -> 0x3A (1.25)
    x[0, 2, :32] = np.r_[6.0, 5.0, -2.5, 0.3, np.zeros(28)]     # MXFP4 group, exponent 0
    x[0, 2, 32:64] = np.r_[3.99, 1.25, -0.375, 0.125, np.zeros(28)]  # exponent -1
    x[0, 3, :32] = 0.0                       # all-zero MXFP4 group
    x[0, 4] = x[0, 4] * 1e-3                 # small values, small scales
    z = np.zeros_like(x)
    w_ik = np.zeros((c, dI), np.float32)
    w_ik[np.arange(dI), np.arange(dI)] = 1.0  # K_I = the first 128 channels, exactly
    planes = _planes(1, 6, c, dI)
    out, ik = C.csa2_compress(f32(x), f32(z), 1, norm=False, w_ik=f32(w_ik), **planes)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(out), x)
    np.testing.assert_array_equal(host(ik), x[..., :dI])
    want = [p[None] for p in O.write_cache(x[0].astype(np.float64), x[0, :, :dI].astype(np.float64), 0, 6)]
    _check_planes(planes, want, "ties")
    assert host(planes["out_scales"])[0, 1, 1] == 0x38 and host(planes["out_scales"])[0, 1, 2] == 0x3A
    assert host(planes["ik_scales"])[0, 3, 0] == 127


@pytest.mark.parametrize("m,overlap", [(1, False), (2, True)])
def test_write_path_decode_append_equals_bulk(C, m, overlap):
    # decode: every completed block is compressed alone and appended at the cache's length
    # (with overlap the previous block's b-branch rows come in as cb0 / zb0); the cache equals
    # the one written from the whole sequence in one call
    banner(f"write path append m={m} overlap={overlap} B=3 c=512 bf16")
    g = W.rng(4200 + m)
    B, n, c, dI = 3, 24, 512, 128
    d = W.compress_inputs(g, n, c, m, overlap=overlap, dtype="bf16", d_I=dI, B=B)
    pos0 = np.array([0, 1000, 65536], np.int32)
    ne, rows = n // m, n // m + 4
    t = {k: bf16(v) for k, v in d.items()}
    ov = dict(cb=t["cb"], zb=t["zb"]) if overlap else {}
    bulk = _planes(B, rows, c, dI)
    C.csa2_compress(t["ca"], t["za"], m, pos0=i32(pos0), rope_dims=64, w_ik=t["w_ik"], plain_out=False,
                    **ov, **bulk)
    stream = _planes(B, rows, c, dI)
    for i in range(ne):
        blk = slice(m * i, m * (i + 1))
        kw = {}
        if overlap:
            kw = dict(cb=t["cb"][:, blk].contiguous(), zb=t["zb"][:, blk].contiguous())
            if i > 0:
                prev = slice(m * (i - 1), m * i)
                kw.update(cb0=t["cb"][:, prev].contiguous(), zb0=t["zb"][:, prev].contiguous())
        C.csa2_compress(t["ca"][:, blk].contiguous(), t["za"][:, blk].contiguous(), m,
                        pos0=i32(pos0 + m * i), rope_dims=64, w_ik=t["w_ik"], plain_out=False,
                        dst_row=i32(np.full(B, i, np.int32)), **kw, **stream)
    torch.cuda.synchronize()
    for k in bulk:
        np.testing.assert_array_equal(host(stream[k]), host(bulk[k]), err_msg=k)
    assert not host(bulk["out_scales"])[:, ne:].any()
    # and the bulk planes are the oracle's write path of the oracle's entries, except for
    # bytes whose fp64 value straddles the threshold that decides them
    w64 = d["w_ik"].astype(np.float64)
    for b in range(B):
        ov = dict(c_b=d["cb"][b], z_b=d["zb"][b], overlap=True) if overlap else {}
        e, k = O.compress(d["ca"][b], d["za"][b], m, rope_dims=64, pos0=int(pos0[b]), w_ik=w64, **ov)
        w = O.write_cache(e, k, 0, rows)
        xh = O.rms_norm(O.gated_pool(d["ca"][b], d["za"][b], m, **ov))
        code_ok, scale_ok = _straddles_fp4(e, w[0][:ne], w[1][:ne], ENTRY_EPS)
        ik_code_ok, ik_scale_ok = _straddles_mx(k, w[2][:ne], w[3][:ne], 512 * 2.0 ** -24 * (np.abs(xh) @ np.abs(w64)))
        for name, j, ok in (("out_codes", 0, code_ok), ("out_scales", 1, scale_ok), ("ik_codes", 2, ik_code_ok),
                            ("ik_scales", 3, ik_scale_ok)):
            diff = host(bulk[name])[b, :ne] != w[j][:ne]
            assert not (diff & ~ok).any(), f"{name} b={b}: a byte differs with no threshold straddle"
