"""Storage formats of the CSA2 caches, decoded and (generator-side) encoded in fp64.

Test infrastructure only: imported by tests, the smoke check and the CPU-baseline
leg of the benchmark, never by the HIP library or its binding.

Sources (cited by page title and section):
  [CSA2 column]   daiw.org, "CSA2：跨层共享的压缩稀疏注意力", section "890 字节是怎么来的":
                  a main-KV entry is 512 channels of 4-bit E2M1 plus one 1-byte E4M3 scale
                  per 16 channels (256 + 32 = 288 B); an indexer-K entry is 128 dims in
                  MXFP4, one shared 1-byte scale per 32 values (64 + 4 = 68 B); the global
                  cache is 890 B per token over layers 2/8/14 (m=2) and 20 (m=1).

The element encodings themselves (E2M1, E4M3 "FN", E8M0) are the OCP 8-bit and
microscaling formats; the pages name them but do not spell them out, so the
definitions below are the published OCP ones, written out from their definition.

The pages are silent on how values are rounded into these formats.  The rule
used by `quantize_*` below (round-to-nearest-even, scale = E4M3(amax/6) for the
main KV, shared exponent floor(log2 amax) - 2 for MXFP4) is a generator-side
choice; both the oracle and the GPU consume the same bytes, so it does not
affect parity.
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------- byte budgets
MAIN_KV_CHANNELS = 512
MAIN_KV_GROUP = 16  # one E4M3 scale per 16 channels
INDEXER_DIM = 128
MX_GROUP = 32  # one E8M0 scale per 32 values


def main_kv_entry_bytes(channels: int = MAIN_KV_CHANNELS) -> int:
    """Bytes of one FP4 main-KV entry: 4-bit codes plus one byte per 16 channels."""
    return channels // 2 + channels // MAIN_KV_GROUP


def indexer_k_entry_bytes(dim: int = INDEXER_DIM) -> int:
    """Bytes of one MXFP4 indexer-K entry: 4-bit codes plus one byte per 32 values."""
    return dim // 2 + dim // MX_GROUP


def global_cache_bytes_per_token(layers=((2, 2), (8, 2), (14, 2), (20, 1))) -> float:
    """Global KV bytes per token: each KV-producing layer with compression ratio m
    stores (main entry + indexer entry) / m bytes per token ([CSA2 column], table of
    the 890-byte section)."""
    per_entry = main_kv_entry_bytes() + indexer_k_entry_bytes()
    return sum(per_entry / m for _, m in layers)


# ---------------------------------------------------------------- E2M1 (4 bit)
# Magnitudes of the 3-bit exponent/mantissa field, OCP FP4 E2M1: 1 sign bit,
# 2 exponent bits (bias 1), 1 mantissa bit, subnormal at exponent 0.
def e2m1_magnitude(field3: int) -> float:
    e = (field3 >> 1) & 3
    mbit = field3 & 1
    if e == 0:
        return mbit * 0.5  # subnormal: 0.m * 2^(1-1)
    return (1.0 + 0.5 * mbit) * 2.0 ** (e - 1)


E2M1_MAGNITUDES = np.array([e2m1_magnitude(f) for f in range(8)], dtype=np.float64)


def e2m1_decode(nibbles: np.ndarray) -> np.ndarray:
    """Decode 4-bit E2M1 codes (values 0..15) to fp64."""
    nib = np.asarray(nibbles, dtype=np.int64)
    mag = E2M1_MAGNITUDES[nib & 7]
    return np.where(nib & 8, -mag, mag)


# ---------------------------------------------------------------- E4M3 (OCP "FN")
def e4m3_decode_scalar(b: int) -> float:
    """OCP E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 is
    subnormal; the all-ones code S.1111.111 is NaN; there is no infinity."""
    s = -1.0 if b & 0x80 else 1.0
    e = (b >> 3) & 0xF
    mt = b & 7
    if e == 15 and mt == 7:
        return float("nan")
    if e == 0:
        return s * mt * 2.0 ** -9  # (mt/8) * 2^(1-7)
    return s * (1.0 + mt / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_decode_scalar(b) for b in range(256)], dtype=np.float64)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.int64)]


# ---------------------------------------------------------------- E8M0
def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E8M0 scale: 2^(code-127); code 255 is NaN."""
    c = np.asarray(codes, dtype=np.int64)
    out = np.ldexp(1.0, c - 127).astype(np.float64)
    return np.where(c == 255, np.nan, out)


# ---------------------------------------------------------------- row decoders
def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[..., n/2] uint8 -> [..., n] codes; element 2i is the low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = p & 0x0F
    hi = p >> 4
    return np.stack([lo, hi], axis=-1).reshape(*p.shape[:-1], p.shape[-1] * 2)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8)
    assert c.shape[-1] % 2 == 0
    pairs = c.reshape(*c.shape[:-1], c.shape[-1] // 2, 2)
    return (pairs[..., 0] | (pairs[..., 1] << 4)).astype(np.uint8)


def fp4_main_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Main-KV rows: codes [..., c/2] uint8, scales [..., c/16] E4M3 bytes -> fp64 [..., c].
    value = E2M1(code) * E4M3(scale of its 16-channel group)."""
    vals = e2m1_decode(unpack_nibbles(codes))
    sc = e4m3_decode(scales)
    return vals * np.repeat(sc, MAIN_KV_GROUP, axis=-1)


def mxfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Indexer-K rows: codes [..., d/2] uint8, scales [..., d/32] E8M0 bytes -> fp64 [..., d]."""
    vals = e2m1_decode(unpack_nibbles(codes))
    sc = e8m0_decode(scales)
    return vals * np.repeat(sc, MX_GROUP, axis=-1)


# ---------------------------------------------------------------- generator-side encoders
def _rne_to_grid(x: np.ndarray, grid: np.ndarray, grid_codes: np.ndarray) -> np.ndarray:
    """Round non-negative x to the nearest value of an ascending grid; a tie goes to
    the code with an even low bit (round-half-to-even on the mantissa).  Values
    above the grid's top saturate to it."""
    x = np.asarray(x, dtype=np.float64)
    hi = np.searchsorted(grid, x, side="left").clip(0, len(grid) - 1)
    lo = (hi - 1).clip(0, len(grid) - 1)
    d_lo = np.abs(x - grid[lo])
    d_hi = np.abs(grid[hi] - x)
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    pick_hi = np.where(tie, (grid_codes[hi] & 1) == 0, pick_hi)
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(x >= grid[-1], len(grid) - 1, idx)
    return grid_codes[idx]


_E2M1_GRID = E2M1_MAGNITUDES.copy()  # ascending already
_E2M1_CODES = np.arange(8)
_E4M3_POS_CODES = np.array([b for b in range(0x7F)])  # 0x00..0x7E, finite non-negative
_E4M3_POS_GRID = E4M3_TABLE[_E4M3_POS_CODES]


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    """fp64 -> 4-bit code, RNE, saturating at +-6; magnitude 0 encodes as +0."""
    x = np.asarray(x, dtype=np.float64)
    field = _rne_to_grid(np.abs(x), _E2M1_GRID, _E2M1_CODES)
    sign = (x < 0) & (field != 0)
    return (field | np.where(sign, 8, 0)).astype(np.uint8)


def e4m3_encode_nonneg(x: np.ndarray) -> np.ndarray:
    return _rne_to_grid(x, _E4M3_POS_GRID, _E4M3_POS_CODES).astype(np.uint8)


def quantize_fp4_main(x: np.ndarray):
    """fp64 rows [..., c] -> (codes [..., c/2], scales [..., c/16]).
    scale = RNE_E4M3(amax16 / 6); code = RNE_E2M1(x / scale); scale 0 -> zero codes."""
    x = np.asarray(x, dtype=np.float64)
    c = x.shape[-1]
    g = x.reshape(*x.shape[:-1], c // MAIN_KV_GROUP, MAIN_KV_GROUP)
    amax = np.abs(g).max(axis=-1)
    sbytes = e4m3_encode_nonneg(amax / 6.0)
    sval = E4M3_TABLE[sbytes]
    safe = np.where(sval > 0, sval, 1.0)
    codes = e2m1_encode(g / safe[..., None])
    codes = np.where((sval > 0)[..., None], codes, 0).astype(np.uint8)
    return pack_nibbles(codes.reshape(x.shape)), sbytes


def quantize_mxfp4(x: np.ndarray):
    """fp64 rows [..., d] -> (codes [..., d/2], scales [..., d/32]) per the OCP MX rule:
    shared exponent e = floor(log2 amax32) - 2 (2 = largest E2M1 exponent),
    code = RNE_E2M1(x / 2^e); an all-zero group gets scale byte 127 and zero codes."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    g = x.reshape(*x.shape[:-1], d // MX_GROUP, MX_GROUP)
    amax = np.abs(g).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, 0)
    e = np.clip(e, -127, 127).astype(np.int64)
    codes = e2m1_encode(g / np.ldexp(1.0, e)[..., None])
    codes = np.where((amax > 0)[..., None], codes, 0).astype(np.uint8)
    return pack_nibbles(codes.reshape(x.shape)), (e + 127).astype(np.uint8)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp64 to the nearest bf16 (RNE) and return it as fp64."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def is_exact_bf16(x: np.ndarray) -> bool:
    x = np.asarray(x, dtype=np.float64)
    return bool(np.all(bf16_round(x) == x))


__all__ = [n for n in dir() if not n.startswith("_") and n not in ("annotations", "math", "np")]
