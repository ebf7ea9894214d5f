// Lightning-indexer scan: I[t,s] = sum_h w[t,h] * ReLU(q_I[t,h] . K_I[s])
// ([DSA-to-CSA notes] eq. (16); [Evolution blog] §2.2), over the visible entries
// s < n_vis(t) = min(N, floor(t/m)) ([DSA-to-CSA notes] "因果边界与短滑窗"), or over a
// candidate list (Reindex, [Evolution blog] §4.4).  Optional block maxima over `block`
// consecutive entries ([CSA2 column] "解码器里的分层索引").
//
// The head contraction is a dense GEMM q_I[H_I x d_I] x K_I^T[d_I x 32 entries] on the
// bf16 MFMA v_mfma_f32_32x32x16_bf16: A = 32 heads x 16 dims (held in registers for the
// whole scan), B = 16 dims x 32 entries loaded straight from HBM into registers (lane l
// reads 16 bytes of entry l%32), C = 32x32 fp32.  In C each lane holds 16 head-rows of one
// entry column, so the ReLU, the signed head weight and the head sum are an in-lane
// epilogue plus one swap between the two half-waves.  The decode scans stage no K_I in
// LDS: every K_I byte is read exactly once per query, straight into registers.  MXFP4 rows
// (E2M1 codes + E8M0 scale per 32) are dequantised into the B registers by the hardware's
// scaled FP4 convert (exact in bf16).  When the queries are MXFP4 as well, both operands'
// codes and E8M0 scales go straight to the scaled FP4 MFMA v_mfma_scale_f32_16x16x128_f8f6f4
// (16 heads x 128 dims x 16 entries per instruction; no convert).
//
// Three variants:
//  * scan_select: decode FULL - workgroup (query, chunk of entries); the chunk's keys go to
//    LDS and its exact top-k is selected in the same kernel, so scores never reach HBM.
//  * scan_private: one query per workgroup slice, scores written out; the 4 waves split
//    the entry range.  Used for Reindex and for decode rows too short to chunk.
//  * scan_shared: prefill - a workgroup takes 8 consecutive queries of one sequence (one
//    per wave) and streams the K_I tiles they share through LDS, so each tile is read from
//    L2 once per 8 queries; the causal limit is per query.

#include "common.h"
#include "internal.h"
#include "topk_core.h"

#include <algorithm>
#include <type_traits>

namespace csa2 {
namespace {

constexpr int kWaves = 4;
constexpr int kPrivThreads = 64 * kWaves;

struct Dev {
  int T, H_I, N, m, block, cand_stride, nblk;
  const uint16_t* q_idx;
  const float* w;
  const int32_t* q_pos;
  const uint16_t* k_idx;
  const uint8_t* k_codes;
  const uint8_t* k_scales;
  const int32_t* cand;
  const int32_t* n_cand;
  float* scores;
  int64_t row_stride;
  float* block_max;
  const int32_t* ent_base;  // [rows] or null: packed samples, the query's first entry
  const uint8_t* q_scales;  // MXFP4 q_I: E8M0 bytes [rows, H_I, d_I/32] (q_idx then holds the codes)
};

// Dimension order inside one 16-wide k-step.  For bf16 rows, lane half h holds dims
// 16*ks + 8h .. +7.  For MXFP4 rows lane half h holds dims (DI/2)*h + 8*ks .. +7, so a
// lane's codes are one contiguous run of DI/4 bytes.  A and B use the same order, so the
// dot product is unchanged.
template <int DI, int KF>
__device__ __forceinline__ int dim_of(int ks, int h) {
  return KF == 0 ? 16 * ks + 8 * h : (DI / 2) * h + 8 * ks;
}

// B operand of one 32-entry tile, as loaded from HBM.  The loads of a tile are issued
// well before the tile is used; conversion to the MFMA operand (to_b) happens at use, so
// nothing waits on a load early.
template <int DI, int KF>
struct RawB;
template <int DI>
struct RawB<DI, 0> {
  bf16x8 v[DI / 16];
};
template <int DI>
struct RawB<DI, 1> {
  uint32_t c[DI / 16];  // this lane's DI/4 code bytes: 8 E2M1 codes per word, low nibble first
  uint32_t s;           // the entry's DI/32 E8M0 scale bytes
};

template <int DI, int KF>
__device__ __forceinline__ void load_raw(const Dev& a, int b, int ent, int h, RawB<DI, KF>& r) {
  if constexpr (KF == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(a.k_idx + ((size_t)b * a.N + ent) * DI + 8 * h);
#pragma unroll
    for (int ks = 0; ks < DI / 16; ++ks) r.v[ks] = as_bf16x8(p[2 * ks]);
  } else {
    // codes: DI/4 bytes at (DI/4)*h of the entry's DI/2 code bytes
    const uint8_t* cp = a.k_codes + ((size_t)b * a.N + ent) * (DI / 2) + (DI / 4) * h;
    const uint8_t* sp = a.k_scales + ((size_t)b * a.N + ent) * (DI / 32);
    if constexpr (DI / 4 >= 16) {
#pragma unroll
      for (int q = 0; q < DI / 64; ++q) {
        const uint4 v = reinterpret_cast<const uint4*>(cp)[q];
        r.c[4 * q] = v.x; r.c[4 * q + 1] = v.y; r.c[4 * q + 2] = v.z; r.c[4 * q + 3] = v.w;
      }
    } else {
      const uint2 v = *reinterpret_cast<const uint2*>(cp);
      r.c[0] = v.x; r.c[1] = v.y;
    }
    if constexpr (DI == 128) r.s = *reinterpret_cast<const uint32_t*>(sp);
    else if constexpr (DI == 64) r.s = *reinterpret_cast<const uint16_t*>(sp);
    else r.s = *sp;
  }
}

// MFMA B registers of a loaded tile.  MXFP4: the hardware's scaled FP4 -> bf16 convert
// takes the power of two 2^(e-127) as an fp32 whose exponent field is e (an E8M0 byte is
// exactly that exponent field), two codes per instruction; E2M1 x 2^k is exact in bf16.
template <int DI, int KF>
__device__ __forceinline__ void to_b(const RawB<DI, KF>& r, int h, bf16x8* breg) {
  if constexpr (KF == 0) {
#pragma unroll
    for (int ks = 0; ks < DI / 16; ++ks) breg[ks] = r.v[ks];
  } else {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    // this lane's dims (DI/2)*h .. +DI/2-1 span the scale groups g0 .. g0 + DI/64 - 1; each
    // scale byte is extracted once
    constexpr int kGroups = DI / 64 > 0 ? DI / 64 : 1;
    const int g0 = dim_of<DI, KF>(0, h) / 32;
    float scale[kGroups];
#pragma unroll
    for (int q = 0; q < kGroups; ++q)
      scale[q] = __builtin_bit_cast(float, __builtin_amdgcn_ubfe(r.s, 8 * (g0 + q), 8) << 23);
#pragma unroll
    for (int ks = 0; ks < DI / 16; ++ks) {
      const float sc = scale[ks / 4 < kGroups ? ks / 4 : kGroups - 1];  // 4 k-steps of 8 dims per group
      const uint32_t cw = r.c[ks];
      uint4 v;
      v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 0));
      v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 1));
      v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 2));
      v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 3));
      breg[ks] = as_bf16x8(v);
    }
  }
}

// ReLU of an fp32 as a signed-integer max with 0 on its bit pattern: non-negative floats
// are non-negative integers and every negative float (and -0) maps to +0.  One instruction,
// where fmaxf(x, 0) needs a canonicalising max first.
__device__ __forceinline__ float relu_bits(float x) {
  return __builtin_bit_cast(float, max(__builtin_bit_cast(int, x), 0));
}

// A operand (q_I of one query) and the head weights in the C layout
template <int DI, int KF, int MT>
__device__ __forceinline__ void load_query(const Dev& a, int row, int lane, bf16x8 (*areg)[DI / 16],
                                           float (*wreg)[16]) {
  const int h = lane / 32;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int head = 32 * mt + lane % 32;
#pragma unroll
    for (int ks = 0; ks < DI / 16; ++ks) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (head < a.H_I)
        v = *reinterpret_cast<const uint4*>(a.q_idx + ((size_t)row * a.H_I + head) * DI + dim_of<DI, KF>(ks, h));
      areg[mt][ks] = as_bf16x8(v);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int hr = 32 * mt + 8 * (r / 4) + 4 * h + (r % 4);  // C-layout row of register r
      wreg[mt][r] = hr < a.H_I ? a.w[(size_t)row * a.H_I + hr] : 0.f;
    }
  }
}

template <int DI, int MT>
__device__ __forceinline__ float tile_score(const bf16x8 (*areg)[DI / 16], const bf16x8* breg,
                                            const float (*wreg)[16]) {
  float s = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < DI / 16; ++ks)
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(areg[mt][ks], breg[ks], acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) s += wreg[mt][r] * relu_bits(acc[r]);
  }
  // lanes l and l^32 hold the two halves of the head rows of the same entry
  s = sum_xor32(s);
  return s;
}

// Two 32-entry tiles at once, in two parts that a caller can separate: the MFMAs (into
// two sets of accumulators) and the epilogue (ReLU, signed head weights, head sum).
template <int DI, int MT>
__device__ __forceinline__ void mfma2(const bf16x8 (*areg)[DI / 16], const bf16x8* b0, const bf16x8* b1,
                                     f32x16* acc0, f32x16* acc1) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    acc0[mt] = f32x16{};
    acc1[mt] = f32x16{};
  }
#pragma unroll
  for (int ks = 0; ks < DI / 16; ++ks)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acc0[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(areg[mt][ks], b0[ks], acc0[mt], 0, 0, 0);
      acc1[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(areg[mt][ks], b1[ks], acc1[mt], 0, 0, 0);
    }
}
template <int MT>
__device__ __forceinline__ void epi2(const f32x16* acc0, const f32x16* acc1, const float (*wreg)[16], float* s0,
                                    float* s1) {
  float x0 = 0.f, x1 = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x0 += wreg[mt][r] * relu_bits(acc0[mt][r]);
      x1 += wreg[mt][r] * relu_bits(acc1[mt][r]);
    }
  *s0 = sum_xor32(x0);
  *s1 = sum_xor32(x1);
}

// One 32-entry tile split the same way: MFMAs into acc, then the epilogue.  A wave that
// issues tile t's MFMAs before tile t-1's epilogue keeps the matrix core and the VALU
// busy together; the epilogue never waits on the MFMAs just issued.
template <int DI, int MT>
__device__ __forceinline__ void mfma1(const bf16x8 (*areg)[DI / 16], const bf16x8* b, f32x16* acc) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < DI / 16; ++ks)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
      acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(areg[mt][ks], b[ks], acc[mt], 0, 0, 0);
}
template <int MT>
__device__ __forceinline__ float epi1(const f32x16* acc, const float (*wreg)[16]) {
  float x = 0.f;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 16; ++r) x += wreg[mt][r] * relu_bits(acc[mt][r]);
  return sum_xor32(x);
}

// the first entry id a query may see: 0, or its sample's first entry (packed samples)
__device__ __forceinline__ int entry_base(const Dev& a, int row) {
  return a.ent_base ? min(max(a.ent_base[row], 0), a.N) : 0;
}
__device__ __forceinline__ int n_visible(const Dev& a, int row) {
  const int t = a.q_pos[row];
  const int nv = t >= 0 ? t / a.m : 0;
  const int cap = a.N - entry_base(a, row);
  return nv < cap ? nv : cap;
}

// block maxima of one 32-slot tile: max over aligned groups of `block` lanes (quad swaps,
// then mirrors pair the halves), visible slots only
__device__ __forceinline__ void emit_block_max(const Dev& a, int row, int lane, int slot, int limit, float s) {
  const bool ok = slot < limit;
  float v = ok ? s : -INFINITY;
  if (a.block >= 2) v = fmaxf(v, dpp<kDppXor1>(v));
  if (a.block >= 4) v = fmaxf(v, dpp<kDppXor2>(v));
  if (a.block >= 8) v = fmaxf(v, dpp<kDppHalfMirror>(v));
  if (a.block >= 16) v = fmaxf(v, dpp<kDppMirror>(v));
  if (a.block >= 32) v = fmaxf(v, swz_xor16(v));
  if (lane < 32 && ok && (slot % a.block) == 0) a.block_max[(size_t)row * a.nblk + slot / a.block] = v;
}

// write scores (lanes 0..31) and, optionally, block maxima of one 32-slot tile
template <bool kBlockMax>
__device__ __forceinline__ void emit(const Dev& a, int row, int lane, int slot, int limit, float s) {
  if (lane < 32 && slot < limit) a.scores[(size_t)row * a.row_stride + slot] = s;
  if constexpr (kBlockMax) emit_block_max(a, row, lane, slot, limit, s);
}

// This wave's tiles tb = t0, t0 + stride, ... < c1 through a kDepth-deep register pipeline:
// tile t is consumed while the next kDepth - 1 tiles load.  load(tile, raw) issues one
// tile's loads (a tile past c1 must load something in bounds); consume(raw, tile) uses it.
// The loop body has no early exit: every path back to its head has issued the same loads
// in the same order as the prologue, so the compiler's wait before each use covers only
// the tile being used (an exit inside the body would join the back edge with fewer loads
// and force a wait for all of them).  The last kDepth - 1 tiles drain after the loop.
template <int kDepth, class Raw, class Load, class Consume>
__device__ __forceinline__ void tile_pipeline(int t0, int c1, int stride, Load&& load, Consume&& consume) {
  Raw buf[kDepth];
#pragma unroll
  for (int i = 0; i < kDepth - 1; ++i) {
    load(t0 + i * stride, buf[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  int tb = t0;
  for (; tb + (kDepth - 1) * stride < c1; tb += kDepth * stride) {
#pragma unroll
    for (int i = 0; i < kDepth; ++i) {
      load(tb + (i + kDepth - 1) * stride, buf[(i + kDepth - 1) % kDepth]);
      consume(buf[i], tb + i * stride);
    }
  }
  // buf[i] holds tile tb + i * stride; fewer than kDepth of them are below c1
#pragma unroll
  for (int i = 0; i < kDepth - 1; ++i) {
    if (tb + i * stride >= c1) break;
    consume(buf[i], tb + i * stride);
  }
}

// Pipeline depth of the private scans.  A raw MXFP4 tile is 9 registers (2.2 KB per wave)
// and affords a deeper pipeline than a bf16 tile (32 registers, 8 KB) at equal occupancy.
template <int KF>
constexpr int kPipeDepth = KF == 1 ? 6 : 3;
// Skewed epilogue (a second accumulator set live): MXFP4 scans are bound by issue, not
// by HBM, and have the registers for it; a bf16 scan would spill.
template <int KF>
constexpr bool kSkewEpilogue = KF == 1;

// ---------------------------------------------------------------- MXFP4 q_I x MXFP4 K_I
// Both operands in MXFP4 go to v_mfma_scale_f32_16x16x128_f8f6f4 with E2M1 codes on both
// sides: lane (n = l % 16, g = l / 16) supplies 32 codes (16 bytes, low nibble first) of row
// n at dims 32g .. 32g + 31 and the E8M0 byte of that 32-dim group, which the instruction
// applies to those values; the 16 x 16 result puts rows 4g + j of column n in lane (n, g).
// One instruction covers 128 dims; for d_I < 128 the lanes of groups g >= d_I / 32 feed
// zero codes.  Every product of two E2M1 values and two powers of two is exact, as with
// the bf16 operands of the other scans.  A 32-entry tile is two sub-tiles of 16 entries
// (A: q_I, 16 heads per block; B: K_I, 16 entries).
typedef int i32x8 __attribute__((ext_vector_type(8)));

struct RawF4 {
  uint4 c[2];      // codes of entries tb + n and tb + 16 + n at this lane's 32 dims
  uint32_t s[2];   // their E8M0 bytes
};

// lanes of groups past d_I load group d_I/32 - 1 (in bounds) and are zeroed in f4_mfma
template <int DI>
__device__ __forceinline__ void load_raw_f4(const Dev& a, int b, int e0, int e1, int g, RawF4& r) {
  const int gg = min(g, DI / 32 - 1);
  const int ent[2] = {e0, e1};
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const size_t e = (size_t)b * a.N + ent[sub];
    r.c[sub] = *reinterpret_cast<const uint4*>(a.k_codes + e * (DI / 2) + 16 * gg);
    r.s[sub] = a.k_scales[e * (DI / 32) + gg];
  }
}

template <int DI, int HB>
__device__ __forceinline__ void load_query_f4(const Dev& a, int row, int lane, i32x8* areg, int* sreg,
                                              float (*wreg)[4]) {
  const int n = lane & 15, g = lane >> 4;
  const uint8_t* qc = reinterpret_cast<const uint8_t*>(a.q_idx);
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = 16 * hb + n;
    uint4 v = make_uint4(0, 0, 0, 0);
    int sc = 127;
    if (head < a.H_I && g < DI / 32) {
      const size_t q = (size_t)row * a.H_I + head;
      v = *reinterpret_cast<const uint4*>(qc + q * (DI / 2) + 16 * g);
      sc = a.q_scales[q * (DI / 32) + g];
    }
    areg[hb] = i32x8{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    sreg[hb] = sc;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hr = 16 * hb + 4 * g + j;
      wreg[hb][j] = hr < a.H_I ? a.w[(size_t)row * a.H_I + hr] : 0.f;
    }
  }
}

// the MFMAs of one 32-entry tile (two sub-tiles x HB head blocks)
// The same tile through buffer loads: codes and scales of entries c0 + o0, c0 + o1 from
// descriptors based at the chunk's first entry (one per workgroup, in scalar registers), so
// each load needs only a 32-bit lane offset
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
struct F4Bufs {
  __amdgpu_buffer_rsrc_t codes, scales;
};
template <int DI>
__device__ __forceinline__ F4Bufs f4_bufs(const Dev& a, int b, int c0) {
  const size_t e = (size_t)b * a.N + c0;
  constexpr int kRawDword3 = 0x00020000;  // raw 32-bit data format
  return F4Bufs{__builtin_amdgcn_make_buffer_rsrc((void*)(a.k_codes + e * (DI / 2)), (short)0, -1, kRawDword3),
                __builtin_amdgcn_make_buffer_rsrc((void*)(a.k_scales + e * (DI / 32)), (short)0, -1, kRawDword3)};
}
template <int DI>
__device__ __forceinline__ void load_raw_f4_buf(const F4Bufs& fb, int o0, int o1, int g, RawF4& r) {
  const int gg = min(g, DI / 32 - 1);
  const int off[2] = {o0, o1};
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(fb.codes, off[sub] * (DI / 2) + 16 * gg, 0, 0);
    r.c[sub] = make_uint4(v.x, v.y, v.z, v.w);
    r.s[sub] = __builtin_amdgcn_raw_buffer_load_b8(fb.scales, off[sub] * (DI / 32) + gg, 0, 0);
  }
}

template <int DI, int HB, int AF = 4>
__device__ __forceinline__ void f4_mfma(const i32x8* areg, const int* sreg, const RawF4& r, int g, f32x4 (*acc)[HB]) {
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    uint4 c = r.c[sub];
    if (DI < 128 && g >= DI / 32) c = make_uint4(0, 0, 0, 0);
    const i32x8 bop = {(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
      acc[sub][hb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(areg[hb], bop, f32x4{0.f, 0.f, 0.f, 0.f}, AF, 4,
                                                                      0, sreg[hb], 0, (int)r.s[sub]);
  }
}
// the tile's scores: lane l gets slot tb + l % 32 (lanes 16..31 of each half take the second
// sub-tile); the four lane groups of an entry are summed by two lane swaps
template <int HB>
__device__ __forceinline__ float f4_epilogue(const f32x4 (*acc)[HB], const float (*wreg)[4], int lane) {
  float x[2];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    float v = 0.f;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int j = 0; j < 4; ++j) v += wreg[hb][j] * relu_bits(acc[sub][hb][j]);
    x[sub] = rows_sum(v);
  }
  return (lane & 16) ? x[1] : x[0];
}
// pipeline depth of the MXFP4 x MXFP4 scans (a raw tile is 10 registers)
constexpr int kPipeDepthF4 = 6;

// ---------------------------------------------------------------- bf16 q_I as E4M3 x MXFP4 K_I
// A bf16 q_I whose values are all E4M3 values at unit scale (zero, or |x| in [2^-6, 448]
// with at most three mantissa bits: the integer-valued queries among them) goes to the same
// scaled MFMA with an FP8 A operand (format 0, E8M0 scale 127).  An 8-bit A operand has
// another lane layout than a 4-bit one (checked with a standalone probe): lane (n, g) holds
// dims 16g .. 16g + 15 of row n in bytes 0..15 and dims 64 + 16g .. 64 + 16g + 15 in bytes
// 16..31, against the B operand's dims 32g .. 32g + 31.  Every product is then the same exact
// product as with bf16 operands, so the scores are those of the bf16 path; the per-tile
// conversion of the MXFP4 keys to bf16 disappears.  Any other query takes the bf16 path.

// the E4M3 byte of a bf16 value; clears `exact` when the value has none
__device__ __forceinline__ uint32_t bf16_to_e4m3(uint32_t h, bool& exact) {
  const uint32_t mag = h & 0x7fffu;
  const int e = (int)(mag >> 7) - 127;
  const uint32_t m = mag & 0x7fu;
  const bool ok = mag == 0u || (e >= -6 && e <= 8 && (m & 0xfu) == 0u && !(e == 8 && (m >> 4) == 7u));
  exact = exact && ok;
  return mag == 0u ? 0u : (((h >> 8) & 0x80u) | ((uint32_t)(e + 7) << 3) | (m >> 4));
}

// Wave w < HB converts head block w of the query into the A-operand layout, staged in LDS
// (stage: HB x 64 lanes x 8 words; flags: HB words).  Returns whether every value was exact
// (block-uniform).  All threads must call it (one barrier); the stage is then read by
// read_query_e4m3, and must not be overwritten before a barrier after that.
template <int DI, int HB>
__device__ __forceinline__ bool stage_query_e4m3(const Dev& a, int row, int lane, int wave, uint32_t* stage,
                                                 uint32_t* flags) {
  const int n = lane & 15, g = lane >> 4;
  if (wave < HB) {
    const int head = 16 * wave + n;
    bool exact = true;
    uint32_t wd[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int d0 = 64 * half + 16 * g;  // dims d0 .. d0 + 15 go to bytes 16 half .. + 15
      if (head < a.H_I && d0 < DI) {
        const uint4* src = reinterpret_cast<const uint4*>(a.q_idx + ((size_t)row * a.H_I + head) * DI + d0);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint4 v = src[q];  // dims d0 + 8q .. + 7, two bf16 per word
          const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const uint32_t lo = u[2 * i], hi = u[2 * i + 1];
            wd[4 * half + 2 * q + i] = bf16_to_e4m3(lo & 0xffffu, exact) | (bf16_to_e4m3(lo >> 16, exact) << 8) |
                                       (bf16_to_e4m3(hi & 0xffffu, exact) << 16) |
                                       (bf16_to_e4m3(hi >> 16, exact) << 24);
          }
        }
      }
    }
    uint4* dst = reinterpret_cast<uint4*>(stage + (wave * 64 + lane) * 8);
    dst[0] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
    dst[1] = make_uint4(wd[4], wd[5], wd[6], wd[7]);
    const bool all = __ballot(!exact) == 0ull;
    if (lane == 0) flags[wave] = all ? 1u : 0u;
  }
  __syncthreads();
  bool all = true;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) all = all && flags[hb] != 0u;
  return all;
}
template <int HB>
__device__ __forceinline__ void read_query_e4m3(const uint32_t* stage, int lane, i32x8* areg) {
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const uint4* src = reinterpret_cast<const uint4*>(stage + (hb * 64 + lane) * 8);
    const uint4 x = src[0], y = src[1];
    areg[hb] = i32x8{(int)x.x, (int)x.y, (int)x.z, (int)x.w, (int)y.x, (int)y.y, (int)y.z, (int)y.w};
  }
}

// the head weights of the 16 x 16 result rows held by lane (n, g)
template <int HB>
__device__ __forceinline__ void load_w_f4(const Dev& a, int row, int lane, float (*wreg)[4]) {
  const int g = lane >> 4;
#pragma unroll
  for (int hb = 0; hb < HB; ++hb)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int hr = 16 * hb + 4 * g + j;
      wreg[hb][j] = hr < a.H_I ? a.w[(size_t)row * a.H_I + hr] : 0.f;
    }
}

// ---------------------------------------------------------------- private-B scan
template <int DI, int KF, int MT, bool kCand, bool kBlockMax>
__global__ void __launch_bounds__(kPrivThreads) scan_private(Dev a, int chunk) {
  const int row = blockIdx.x;
  const int b = row / a.T;
  const int lane = threadIdx.x % 64;
  const int wave = wave_index();
  const int limit = kCand ? min(a.n_cand[row], a.cand_stride) : n_visible(a, row);
  const int c0 = blockIdx.y * chunk;
  const int c1 = min(c0 + chunk, limit);
  if (c0 >= c1) return;

  const int eb = kCand ? 0 : entry_base(a, row);
  auto entry_of = [&](int slot) -> int {
    int s = min(slot, c1 - 1);
    if constexpr (kCand) {
      int e = a.cand[(size_t)row * a.cand_stride + s];
      return min(max(e, 0), a.N - 1);
    }
    return eb + s;
  };

  constexpr int kStride = 32 * kWaves;
  const int t0 = c0 + 32 * wave;
  if (t0 >= c1) return;
  auto cand_mask = [&](float s, int tb) {
    if constexpr (kCand) {
      const int slot = tb + lane % 32;
      if (slot < c1) {
        const int e = a.cand[(size_t)row * a.cand_stride + slot];
        if (e < 0 || e >= a.N) s = -INFINITY;
      }
    }
    return s;
  };
  if constexpr (KF == 2) {
    constexpr int HB = 2 * MT;
    i32x8 areg[HB];
    int sreg[HB];
    float wreg[HB][4];
    load_query_f4<DI, HB>(a, row, lane, areg, sreg, wreg);
    const int n16 = lane & 15, g16 = lane >> 4;
    tile_pipeline<kPipeDepthF4, RawF4>(
        t0, c1, kStride,
        [&](int tb, RawF4& raw) { load_raw_f4<DI>(a, b, entry_of(tb + n16), entry_of(tb + 16 + n16), g16, raw); },
        [&](const RawF4& raw, int tb) {
          f32x4 acc[2][HB];
          f4_mfma<DI, HB>(areg, sreg, raw, g16, acc);
          const float s = cand_mask(f4_epilogue<HB>(acc, wreg, lane), tb);
          emit<kBlockMax>(a, row, lane, tb + lane % 32, c1, s);
        });
  } else {
    bf16x8 areg[MT][DI / 16];
    float wreg[MT][16];
    load_query<DI, KF, MT>(a, row, lane, areg, wreg);
    const int h = lane / 32;
    tile_pipeline<kPipeDepth<KF>, RawB<DI, KF>>(
        t0, c1, kStride,
        [&](int tb, RawB<DI, KF>& raw) { load_raw<DI, KF>(a, b, entry_of(tb + lane % 32), h, raw); },
        [&](const RawB<DI, KF>& raw, int tb) {
          bf16x8 breg[DI / 16];
          to_b<DI, KF>(raw, h, breg);
          const float s = cand_mask(tile_score<DI, MT>(areg, breg, wreg), tb);
          emit<kBlockMax>(a, row, lane, tb + lane % 32, c1, s);
        });
  }
}

// the MXFP4-K_I tiles t0, t0 + 128, ... below c1 through the scaled MFMA (A format AF),
// each tile's epilogue one tile late; finish(score, tile) takes the scores
template <int DI, int HB, int AF, class Finish>
__device__ __forceinline__ void scan_tiles_f4(const Dev& a, int b, int c0, int t0, int c1, int lane,
                                              const i32x8* areg, const int* sreg, const float (*wreg)[4],
                                              Finish finish) {
  constexpr int kStride = 32 * kWaves;
  const int n16 = lane & 15, g16 = lane >> 4;
  const F4Bufs fbuf = f4_bufs<DI>(a, b, c0);
  f32x4 pacc[2][HB];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) pacc[sub][hb] = f32x4{0.f, 0.f, 0.f, 0.f};
  int ptb = t0;
  auto load = [&](int tb, RawF4& raw) {
    load_raw_f4_buf<DI>(fbuf, min(tb + n16, c1 - 1) - c0, min(tb + 16 + n16, c1 - 1) - c0, g16, raw);
  };
  tile_pipeline<kPipeDepthF4, RawF4>(t0, c1, kStride, load, [&](const RawF4& raw, int tb) {
    f32x4 cacc[2][HB];
    f4_mfma<DI, HB, AF>(areg, sreg, raw, g16, cacc);
    finish(f4_epilogue<HB>(pacc, wreg, lane), ptb);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) pacc[sub][hb] = cacc[sub][hb];
    ptb = tb;
  });
  finish(f4_epilogue<HB>(pacc, wreg, lane), ptb);
}

// ---------------------------------------------------------------- fused scan + chunk top-k
// Decode: workgroup (query, chunk) scans its chunk like scan_private but keeps the keys of
// its scores in LDS, then selects the chunk's top-k there and writes (key, slot) pairs;
// the chunk union contains the row's top-k, which topk_merge extracts.
constexpr int kSelThreads = 256;
// A chunk is selected from registers when it fits kRows rows of 4 keys per thread, from
// LDS otherwise.  kRows = 8 (8192 keys) keeps the scan at two waves per SIMD; the longest
// chunks (32,768 keys) hold their workgroup alone on a CU for its LDS, so their variant
// spends the registers of one wave per SIMD on 32 rows instead.
constexpr int kRegRowsSmall = 8;
constexpr int kRegRowsLarge = kMaxSelectChunk / (4 * kSelThreads);

template <int DI, int KF, int MT, bool kBlockMax, bool kScores, int kRows>
__global__ void __launch_bounds__(kSelThreads) scan_select(Dev a, int chunk, int k, int nchunks,
                                                           uint32_t* wkeys, int32_t* wslot, uint2* wbound) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  TopkSmem<kSelThreads>& sm = *reinterpret_cast<TopkSmem<kSelThreads>*>(smem_raw);
  uint32_t* skeys = reinterpret_cast<uint32_t*>(smem_raw + ((sizeof(TopkSmem<kSelThreads>) + 15) & ~(size_t)15));
  const int row = blockIdx.x, c = blockIdx.y;
  const int b = row / a.T;
  const int lane = threadIdx.x % 64, wave = wave_index();
  const int limit = n_visible(a, row);
  const int c0 = c * chunk;
  const int c1 = min(c0 + chunk, limit);
  const int len = c1 - c0;
  uint32_t* ok = wkeys + ((size_t)row * nchunks + c) * k;
  int32_t* os = wslot + ((size_t)row * nchunks + c) * k;
  uint2* ob = wbound + (size_t)row * nchunks + c;
  if (len <= 0) {  // uniform: nothing visible in this chunk
    for (int i = threadIdx.x; i < k; i += kSelThreads) { ok[i] = 0u; os[i] = -1; }
    if (threadIdx.x == 0) *ob = make_uint2(0u, 0u);
    return;
  }
  constexpr int kStride = 32 * kWaves;
  const int t0 = c0 + 32 * wave;
  // The key store needs no branch: tiles start at multiples of 32 from c0 and the chunk is a
  // multiple of 32 entries, so every slot of a tile lies inside the chunk's key array, and
  // keys past the visible end are never read.  With the skewed epilogue, tile t's epilogue
  // runs after tile t+1's MFMAs are issued; before the first tile the pending epilogue is a
  // zero tile at t0, which that tile's own epilogue overwrites.
  auto finish = [&](float s, int tb) {  // s: the score of slot tb + lane % 32
    const int slot = tb + lane % 32;
    skeys[slot - c0] = float_key(s);
    if constexpr (kScores) {
      if (lane < 32 && slot < c1) a.scores[(size_t)row * a.row_stride + slot] = s;
    }
    if constexpr (kBlockMax) emit_block_max(a, row, lane, slot, c1, s);
  };
  // bf16 q_I with an MXFP4 K_I: the FP8 x FP4 MFMA when every q_I value is an E4M3 value
  // (the staging uses the key array, before any key is written)
  constexpr int HB8 = 2 * MT;
  constexpr bool kTryF8 = KF == 1 && HB8 <= kWaves;
  bool f8 = false;
  if constexpr (kTryF8) {
    f8 = stage_query_e4m3<DI, HB8>(a, row, lane, wave, skeys, sm.cand);
    if (f8) {  // block-uniform
      i32x8 areg8[HB8];
      read_query_e4m3<HB8>(skeys, lane, areg8);
      __syncthreads();  // the stage is read: keys may overwrite it
      if (t0 < c1) {
        int sreg[HB8];
        float wreg[HB8][4];
#pragma unroll
        for (int hb = 0; hb < HB8; ++hb) sreg[hb] = 127;  // unit scale
        load_w_f4<HB8>(a, row, lane, wreg);
        scan_tiles_f4<DI, HB8, 0>(a, b, c0, t0, c1, lane, areg8, sreg, wreg, finish);
      }
    }
  }
  if (!f8 && t0 < c1) {
    if constexpr (KF == 2) {
      constexpr int HB = 2 * MT;
      i32x8 areg[HB];
      int sreg[HB];
      float wreg[HB][4];
      load_query_f4<DI, HB>(a, row, lane, areg, sreg, wreg);
      scan_tiles_f4<DI, HB, 4>(a, b, c0, t0, c1, lane, areg, sreg, wreg, finish);
    } else {
      bf16x8 areg[MT][DI / 16];
      float wreg[MT][16];
      load_query<DI, KF, MT>(a, row, lane, areg, wreg);
      const int h = lane / 32;
      auto load = [&](int tb, RawB<DI, KF>& raw) { load_raw<DI, KF>(a, b, min(tb + lane % 32, c1 - 1), h, raw); };
      if constexpr (kSkewEpilogue<KF>) {
        f32x16 pacc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) pacc[mt] = f32x16{};
        int ptb = t0;
        tile_pipeline<kPipeDepth<KF>, RawB<DI, KF>>(t0, c1, kStride, load, [&](const RawB<DI, KF>& raw, int tb) {
          bf16x8 breg[DI / 16];
          to_b<DI, KF>(raw, h, breg);
          f32x16 cacc[MT];
          mfma1<DI, MT>(areg, breg, cacc);
          finish(epi1<MT>(pacc, wreg), ptb);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) pacc[mt] = cacc[mt];
          ptb = tb;
        });
        finish(epi1<MT>(pacc, wreg), ptb);
      } else {
        tile_pipeline<kPipeDepth<KF>, RawB<DI, KF>>(t0, c1, kStride, load, [&](const RawB<DI, KF>& raw, int tb) {
          bf16x8 breg[DI / 16];
          to_b<DI, KF>(raw, h, breg);
          f32x16 acc[MT];
          mfma1<DI, MT>(areg, breg, acc);
          finish(epi1<MT>(acc, wreg), tb);
        });
      }
    }
  }
  __syncthreads();
  if (len <= k) {
    for (int i = threadIdx.x; i < k; i += kSelThreads) {
      ok[i] = i < len ? skeys[i] : 0u;
      os[i] = i < len ? c0 + i : -1;
    }
    if (threadIdx.x == 0) *ob = make_uint2(0u, (uint32_t)len);  // every key >= 0
    return;
  }
  // pruning bound for the merge, from the first radix pass
  const int k2 = bound_rank(k, nchunks);
  uint32_t T, take, L2, g2;
  auto direct = [=](uint32_t pos, int i, uint32_t key) {
    ok[pos] = key;
    os[pos] = c0 + i;
  };
  if (len <= 4 * kSelThreads * kRows) {
    // the chunk's keys move into registers: the selection passes read no LDS
    KeyRegs<kSelThreads, kRows> r;
    key_regs_load(r, skeys, len);
    radix_threshold<kSelThreads>(r, len, k, sm, &T, &take, k2, &L2, &g2);
    if (T != 0u && k <= kTopkBins) {
      // selected (key, slot) pairs staged in the histogram space, then stored coalesced
      uint32_t* sk = sm.hist[0];
      uint32_t* ss = sm.hist[1];
      ordered_compact_regs(r, k, T, take, sm, [&](uint32_t pos, int i, uint32_t key) {
        sk[pos] = key;
        ss[pos] = (uint32_t)(c0 + i);
      });
      lds_barrier();
      if ((k & 3) == 0) {
        for (int i = 4 * threadIdx.x; i < k; i += 4 * kSelThreads) {
          *reinterpret_cast<uint4*>(ok + i) = *reinterpret_cast<const uint4*>(sk + i);
          *reinterpret_cast<uint4*>(os + i) = *reinterpret_cast<const uint4*>(ss + i);
        }
      } else {
        for (int i = threadIdx.x; i < k; i += kSelThreads) {
          ok[i] = sk[i];
          os[i] = (int32_t)ss[i];
        }
      }
    } else if (T != 0u) {
      ordered_compact_regs(r, k, T, take, sm, direct);
    } else {  // the zero slots past len could tie with T = 0: compact from LDS, which stops at len
      ordered_compact<kSelThreads>(KeysLds{skeys}, len, k, T, take, sm, direct);
    }
  } else {
    const KeysLds src{skeys};
    radix_threshold<kSelThreads>(src, len, k, sm, &T, &take, k2, &L2, &g2);
    ordered_compact<kSelThreads>(src, len, k, T, take, sm, direct);
  }
  if (threadIdx.x == 0) *ob = make_uint2(L2, g2);
}

// ---------------------------------------------------------------- shared-B scan (prefill)
constexpr int kShWaves = 8;
constexpr int kShThreads = 64 * kShWaves;
constexpr int kShTile = 128;  // entries per LDS stage (two pairs of 32-entry tiles)

template <int DI, int KF, int MT, bool kBlockMax>
__global__ void __launch_bounds__(kShThreads) scan_shared(Dev a) {
  // workgroup -> 8 consecutive query rows of one sequence (one per wave); within a sequence
  // the heavy (late, long causal range) groups come first
  const int groups_per_seq = (a.T + kShWaves - 1) / kShWaves;
  const int gid = blockIdx.x;
  const int b = gid / groups_per_seq;
  const int g = groups_per_seq - 1 - (gid % groups_per_seq);
  const int lane = threadIdx.x % 64;
  const int wave = wave_index();
  const int t = g * kShWaves + wave;
  const bool active = t < a.T;
  const int row = b * a.T + (active ? t : 0);
  const int limit = active ? n_visible(a, row) : 0;
  // the group's scan length: the largest limit of its queries
  __shared__ int s_lim[kShWaves];
  if (lane == 0) s_lim[wave] = limit;
  lds_barrier();
  int glim = 0;
#pragma unroll
  for (int i = 0; i < kShWaves; ++i) glim = max(glim, s_lim[i]);
  if (glim == 0) return;

  // LDS: two stages of kShTile entries x DI bf16, [entry][16-byte chunk], the chunk index
  // XOR-swizzled with the entry so the 32 lanes of an MFMA B read hit distinct banks
  constexpr int kCPR = DI / 8;  // chunks per entry row
  __shared__ uint4 tile[2][kShTile * kCPR];
  bf16x8 areg[MT][DI / 16];
  float wreg[MT][16];
  load_query<DI, KF, MT>(a, row, lane, areg, wreg);
  const int h = lane / 32;

  constexpr int kChunks = kShTile * kCPR;
  constexpr int kPerThread = (kChunks + kShThreads - 1) / kShThreads;
  // global -> registers for the stage starting at `base` (MXFP4: raw codes and scale,
  // converted when committed to LDS, so the loads stay in flight meanwhile)
  uint4 pre[KF == 0 ? kPerThread : 1];
  uint32_t pre_c[KF == 1 ? kPerThread : 1], pre_s[KF == 1 ? kPerThread : 1];
  auto fetch = [&](int base) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int q = threadIdx.x + i * kShThreads;
      if (q < kChunks) {
        const int e = q / kCPR, part = q % kCPR;
        const int ent = min(base + e, glim - 1);
        if constexpr (KF == 0) {
          pre[i] = reinterpret_cast<const uint4*>(a.k_idx + ((size_t)b * a.N + ent) * DI)[part];
        } else {
          // dims 8*part .. 8*part+7 in natural order
          pre_c[i] = *reinterpret_cast<const uint32_t*>(a.k_codes + ((size_t)b * a.N + ent) * (DI / 2) + 4 * part);
          pre_s[i] = a.k_scales[((size_t)b * a.N + ent) * (DI / 32) + (8 * part) / 32];
        }
      }
    }
  };
  auto commit = [&](int st) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int q = threadIdx.x + i * kShThreads;
      if (q < kChunks) {
        const int e = q / kCPR, part = q % kCPR;
        uint4 v;
        if constexpr (KF == 0) {
          v = pre[i];
        } else {
          // E2M1 x 2^(e-127) by the hardware's scaled convert (exact in bf16)
          const float sc = __builtin_bit_cast(float, pre_s[i] << 23);
          v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(pre_c[i], sc, 0));
          v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(pre_c[i], sc, 1));
          v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(pre_c[i], sc, 2));
          v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(pre_c[i], sc, 3));
        }
        tile[st][e * kCPR + (part ^ (e & (kCPR - 1)))] = v;
      }
    }
  };

  // Waves 4..7 run one stage behind in their epilogue: at each stage they first finish the
  // previous stage (VALU) and then issue this stage's MFMAs, while waves 0..3 do MFMAs then
  // epilogue.  Waves w and w + 4 share a SIMD (waves are dealt round-robin to the 4 SIMDs),
  // so the two alternate between the matrix core and the VALU instead of both waiting on
  // the same unit after every workgroup barrier.
  const bool lag = wave >= kShWaves / 2;
  f32x16 acc0[MT], acc1[MT];
  int pending = -1;  // lagging waves: base of the stage whose epilogue is still due
  auto finish = [&](int sbase) {
    float s0, s1;
    epi2<MT>(acc0, acc1, wreg, &s0, &s1);
    emit<kBlockMax>(a, row, lane, sbase + lane % 32, limit, s0);
    emit<kBlockMax>(a, row, lane, sbase + 32 + lane % 32, limit, s1);
  };
  static_assert(kShTile % 64 == 0, "pairs of 32-entry tiles per stage");
  fetch(0);
  commit(0);
  lds_barrier();
  int st = 0;
  for (int base = 0; base < glim; base += kShTile) {
    const bool more = base + kShTile < glim;
    if (more) fetch(base + kShTile);
#pragma unroll
    for (int pr = 0; pr < kShTile / 64; ++pr) {
      const int pbase = base + 64 * pr;
      if (lag && pending >= 0) {
        finish(pending);
        pending = -1;
      }
      if (active && pbase < limit) {
        // both 32-entry tiles of the pair (the second may lie past this query's limit:
        // its scores are then simply not written)
        bf16x8 b0[DI / 16], b1[DI / 16];
        const int e = 64 * pr + lane % 32;
#pragma unroll
        for (int ks = 0; ks < DI / 16; ++ks) {
          // LDS holds natural dim order; read the dims this lane's A registers hold.  Entry
          // e + 32 has the same swizzle as entry e, 32 rows further on.
          const int part = dim_of<DI, KF>(ks, h) / 8;
          const int idx = e * kCPR + (part ^ (e & (kCPR - 1)));
          b0[ks] = as_bf16x8(tile[st][idx]);
          b1[ks] = as_bf16x8(tile[st][idx + 32 * kCPR]);
        }
        mfma2<DI, MT>(areg, b0, b1, acc0, acc1);
        if (lag) pending = pbase;
        else finish(pbase);
      }
    }
    if (more) commit(st ^ 1);
    lds_barrier();
    st ^= 1;
  }
  if (pending >= 0) finish(pending);
}

template <int DI, int KF, int MT>
hipError_t launch3(const ScanArgs& s, const Dev& d, hipStream_t st) {
  const int rows = s.B * s.T;
  const bool cand = s.cand != nullptr;
  const bool bm = s.block_max != nullptr;
  // the shared-tile prefill scan gives 8 consecutive queries one entry range: packed
  // samples (a range per query) take the private scan, as do MXFP4 queries
  if constexpr (KF != 2) if (!cand && s.T >= kShWaves && !s.ent_base) {
    dim3 grid(((s.T + kShWaves - 1) / kShWaves) * s.B);
    if (bm) hipLaunchKernelGGL((scan_shared<DI, KF, MT, true>), grid, dim3(kShThreads), 0, st, d);
    else hipLaunchKernelGGL((scan_shared<DI, KF, MT, false>), grid, dim3(kShThreads), 0, st, d);
    return hipGetLastError();
  }
  const int len = cand ? s.cand_stride : s.N;
  // chunk: a multiple of 128 entries; aim for >= 2048 workgroups in total
  int chunk = 4096;
  while (chunk > 512 && (long long)rows * ((len + chunk - 1) / chunk) < 2048) chunk /= 2;
  dim3 grid(rows, (len + chunk - 1) / chunk);
  if (cand) {
    hipLaunchKernelGGL((scan_private<DI, KF, MT, true, false>), grid, dim3(kPrivThreads), 0, st, d, chunk);
  } else if (bm) {
    hipLaunchKernelGGL((scan_private<DI, KF, MT, false, true>), grid, dim3(kPrivThreads), 0, st, d, chunk);
  } else {
    hipLaunchKernelGGL((scan_private<DI, KF, MT, false, false>), grid, dim3(kPrivThreads), 0, st, d, chunk);
  }
  return hipGetLastError();
}

template <int DI, int KF>
hipError_t launch2(const ScanArgs& s, const Dev& d, hipStream_t st) {
  return s.H_I <= 32 ? launch3<DI, KF, 1>(s, d, st) : launch3<DI, KF, 2>(s, d, st);
}

template <int DI>
hipError_t launch1(const ScanArgs& s, const Dev& d, hipStream_t st) {
  if (s.k_dtype != CSA2_MXFP4) return launch2<DI, 0>(s, d, st);
  return s.q_scales ? launch2<DI, 2>(s, d, st) : launch2<DI, 1>(s, d, st);
}

template <int DI, int KF, int MT, int kRows>
hipError_t launch_sel4(const Dev& d, dim3 grid, size_t lds, bool bm, bool sc, int chunk, int k, int nchunks,
                       uint32_t* keys, int32_t* slots, uint2* bounds, hipStream_t st) {
  const void* fn = bm ? (sc ? (const void*)scan_select<DI, KF, MT, true, true, kRows> : (const void*)scan_select<DI, KF, MT, true, false, kRows>)
                      : (sc ? (const void*)scan_select<DI, KF, MT, false, true, kRows> : (const void*)scan_select<DI, KF, MT, false, false, kRows>);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (bm && sc) hipLaunchKernelGGL((scan_select<DI, KF, MT, true, true, kRows>), grid, dim3(kSelThreads), lds, st, d, chunk, k, nchunks, keys, slots, bounds);
  else if (bm) hipLaunchKernelGGL((scan_select<DI, KF, MT, true, false, kRows>), grid, dim3(kSelThreads), lds, st, d, chunk, k, nchunks, keys, slots, bounds);
  else if (sc) hipLaunchKernelGGL((scan_select<DI, KF, MT, false, true, kRows>), grid, dim3(kSelThreads), lds, st, d, chunk, k, nchunks, keys, slots, bounds);
  else hipLaunchKernelGGL((scan_select<DI, KF, MT, false, false, kRows>), grid, dim3(kSelThreads), lds, st, d, chunk, k, nchunks, keys, slots, bounds);
  return hipGetLastError();
}

template <int DI, int KF, int MT>
hipError_t launch_sel3(const ScanArgs& s, const Dev& d, int k, int chunk, int nchunks, uint32_t* keys,
                       int32_t* slots, uint2* bounds, hipStream_t st) {
  // the key array also stages an E4M3 q_I (2 MT head blocks x 64 lanes x 32 bytes)
  const size_t key_bytes = std::max((size_t)chunk * 4, KF == 1 ? (size_t)(2 * MT) * 64 * 32 : (size_t)0);
  const size_t lds = ((sizeof(TopkSmem<kSelThreads>) + 15) & ~(size_t)15) + key_bytes;
  dim3 grid(s.B * s.T, nchunks);
  const bool bm = s.block_max != nullptr, sc = s.scores != nullptr;
  // the large register variant only for a bf16 K_I with 128 dims and 33..64 heads (the
  // configuration with chunks that long); others select long chunks from LDS
  if constexpr (DI == 128 && KF == 0 && MT == 2) {
    if (chunk > 4 * kSelThreads * kRegRowsSmall)
      return launch_sel4<DI, KF, MT, kRegRowsLarge>(d, grid, lds, bm, sc, chunk, k, nchunks, keys, slots, bounds, st);
  }
  return launch_sel4<DI, KF, MT, kRegRowsSmall>(d, grid, lds, bm, sc, chunk, k, nchunks, keys, slots, bounds, st);
}

Dev make_dev(const ScanArgs& s) {
  Dev d;
  d.T = s.T; d.H_I = s.H_I; d.N = s.N; d.m = s.m; d.block = s.block > 0 ? s.block : 1;
  d.cand_stride = s.cand_stride; d.nblk = s.nblk;
  d.q_idx = (const uint16_t*)s.q_idx; d.w = s.w; d.q_pos = s.q_pos;
  d.k_idx = (const uint16_t*)s.k_idx; d.k_codes = s.k_codes; d.k_scales = s.k_scales;
  d.cand = s.cand; d.n_cand = s.n_cand; d.scores = s.scores; d.row_stride = s.row_stride;
  d.block_max = s.block_max;
  d.ent_base = s.ent_base;
  d.q_scales = s.q_scales;
  return d;
}

}  // namespace

int scan_select_chunk(int rows, int N, int k) {
  // A power of two >= 2048 such that the merge row (nchunks * k) stays <= 16384 keys.
  // Larger chunks (up to 8192) while the grid would exceed about one round of resident
  // workgroups (2 per CU): each workgroup then streams longer before its chunk top-k, and
  // fewer top-k phases leave the memory system idle.
  constexpr long long kOneRound = 2 * 256 + 64;
  int chunk = 2048;
  auto nch = [&](int c) { return (long long)((N + c - 1) / c); };
  while ((nch(chunk) * k > 16384 || (chunk < 8192 && rows * nch(chunk) > kOneRound)) && chunk < (1 << 30))
    chunk *= 2;
  return chunk;
}

hipError_t launch_index_scan_select(const ScanArgs& s, int k, int chunk, int nchunks, uint32_t* keys,
                                    int32_t* slots, uint2* bounds, hipStream_t st) {
  if (s.B * s.T == 0) return hipSuccess;
  if (!s.q_idx || !s.w || !s.q_pos || !keys || !slots || !bounds || s.cand || s.ent_base ||
      (s.N > 0 && s.k_dtype == CSA2_BF16 && !s.k_idx) ||
      (s.N > 0 && s.k_dtype == CSA2_MXFP4 && (!s.k_codes || !s.k_scales)) || chunk % 128 != 0 || k < 1)
    return hipErrorInvalidValue;
  const Dev d = make_dev(s);
  ScopedProf p(st, "index_scan_select");
  auto go = [&](auto di, auto kf) -> hipError_t {
    constexpr int DI = decltype(di)::value, KF = decltype(kf)::value;
    return s.H_I <= 32 ? launch_sel3<DI, KF, 1>(s, d, k, chunk, nchunks, keys, slots, bounds, st)
                       : launch_sel3<DI, KF, 2>(s, d, k, chunk, nchunks, keys, slots, bounds, st);
  };
  // KF: 0 bf16 K_I; 1 MXFP4 K_I with bf16 q_I; 2 MXFP4 K_I and q_I
  const int kf = s.k_dtype != CSA2_MXFP4 ? 0 : (s.q_scales ? 2 : 1);
  auto by_kf = [&](auto di) -> hipError_t {
    if (kf == 0) return go(di, std::integral_constant<int, 0>{});
    if (kf == 1) return go(di, std::integral_constant<int, 1>{});
    return go(di, std::integral_constant<int, 2>{});
  };
  switch (s.d_I) {
    case 32: return by_kf(std::integral_constant<int, 32>{});
    case 64: return by_kf(std::integral_constant<int, 64>{});
    case 128: return by_kf(std::integral_constant<int, 128>{});
  }
  return hipErrorInvalidValue;
}

hipError_t launch_index_scan(const ScanArgs& s, hipStream_t st) {
  if (s.B * s.T == 0) return hipSuccess;
  // every pointer a kernel dereferences must be set
  if (!s.q_idx || !s.w || !s.q_pos || !s.scores || (s.N > 0 && s.k_dtype == CSA2_BF16 && !s.k_idx) ||
      (s.N > 0 && s.k_dtype == CSA2_MXFP4 && (!s.k_codes || !s.k_scales)) ||
      (s.cand && (!s.n_cand || s.cand_stride < 1)))
    return hipErrorInvalidValue;
  const Dev d = make_dev(s);
  ScopedProf p(st, s.cand ? "index_scan_reindex" : (s.T >= kShWaves ? "index_scan_prefill" : "index_scan_decode"));
  switch (s.d_I) {
    case 32: return launch1<32>(s, d, st);
    case 64: return launch1<64>(s, d, st);
    case 128: return launch1<128>(s, d, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace csa2
