// Exact top-k selection inside one workgroup ([DSA-to-CSA notes] eq. (17)): the k largest
// keys of a row, ties to the lower index, reported in index order.
//
// Keys are order-preserving uint32 images of the scores (see float_key).  The threshold
// T (the k-th largest key) is found in two steps.  A first pass histograms the keys into
// 2048 LDS bins laid linearly over the scores between the smallest and the largest finite
// one; the map is monotone (a key never lands below a smaller key's bin), so the bin that
// holds the k-th largest key is exact.  That bin usually holds a few keys: they are
// gathered in LDS and every wave ranks them directly.  A crowded bin (heavy ties, or
// scores spread over many orders of magnitude) goes on with range-adaptive radix passes
// over its own key range [lo, lo+span]: each histograms (key - lo) >> shift into at most
// 2048 bins (shift chosen from the span), keeps the bin holding the k-th largest key and
// narrows the range to it, until the range is a single key.  A pass costs three barriers
// (the histograms are double buffered).  The compaction counts the selected keys of every 256-key segment, scans the
// segment counts once across the block and then places each key at its rank in index
// order: the output is ascending and ties resolve to the lower index.
#pragma once

#include "common.h"

namespace csa2 {

constexpr int kTopkBins = 2048;
constexpr int kSegKeys = 256;  // keys per compaction segment: 4 per lane of one wave
constexpr int kSegMax = 128;   // segments per compaction sweep (32768 keys)

template <int kT>
struct TopkSmem {
  static constexpr int kW = kT / 64;
  uint32_t hist[2][kTopkBins];  // double-buffered: one pass fills one while the other is cleared
  uint32_t seg[kSegMax];        // per segment: (#keys > T) | (#keys == T) << 16, then their prefix
  uint32_t wsum[2][kW];
  uint32_t wlo[kW], whi[kW];
  uint32_t wl2[kW];
  uint32_t sel_bin[2], krem[2];
  uint32_t bound_lo, bound_cnt;
  uint32_t ncand;
  uint32_t cand[64];  // the keys of the first pass's boundary bin, when it holds at most 64
};

// keys of finite scores lie strictly between float_key(-inf) and float_key(+inf)
constexpr uint32_t kKeyNegInf = 0x007fffffu;
constexpr uint32_t kKeyPosInf = 0xff800000u;
constexpr uint32_t kCandMax = 64;

// the score of a key (inverse of float_key)
__device__ __forceinline__ float key_float(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Bins linear in the score: bin = (x - f0) * 2048 / (f1 - f0) for finite scores x in
// [f0, f1], computed as one fused multiply-add and clamped to [0, 2047]; keys below every
// finite score go to bin 0, keys above to bin 2047.  Each step is monotone (a correctly
// rounded fma of a fixed positive slope, the clamps, truncation), so a larger key never
// takes a lower bin, whatever the rounding.  Without two distinct finite scores (or with a
// range too small for a finite slope) every finite key takes the middle bin.
struct LinearBins {
  float a = 0.f, c = 1024.f;
  __device__ __forceinline__ void init(uint32_t flo, uint32_t fhi) {
    if (flo < fhi) {
      const float f0 = key_float(flo), f1 = key_float(fhi);
      const float aa = 1024.f / (0.5f * f1 - 0.5f * f0);  // halves: no overflow of the range
      const float cc = -f0 * aa;
      if (__builtin_isfinite(aa) && __builtin_isfinite(cc)) {
        a = aa;
        c = cc;
      }
    }
  }
  // a key range that holds every key of bin t, and usually little else: the keys of the
  // scores whose ideal bin value lies in [t - 1, t + 2) (each bin's keys are found exactly
  // among them, and a count check catches a range that missed some)
  __device__ __forceinline__ void key_range(uint32_t t, uint32_t* k_lo, uint32_t* k_hi) const {
    *k_lo = t == 0 ? 0u : float_key(((float)t - 1.f - c) / a);
    *k_hi = t >= kTopkBins - 1 ? 0xffffffffu : float_key(((float)t + 2.f - c) / a);
    if (!(a > 0.f)) {  // every finite key in one bin
      *k_lo = t == 0 ? 0u : kKeyNegInf;
      *k_hi = t >= kTopkBins - 1 ? 0xffffffffu : kKeyPosInf;
    }
  }
  // branch-free: -inf, the keys below it (negative NaNs) and any NaN product clamp to 0;
  // +inf, the keys above it (positive NaNs, forced keys) are set to the last bin
  __device__ __forceinline__ uint32_t operator()(uint32_t u) const {
    const float v = fminf(fmaxf(__builtin_fmaf(key_float(u), a, c), 0.f), (float)(kTopkBins - 1));
    return u >= kKeyPosInf ? (uint32_t)(kTopkBins - 1) : (uint32_t)v;
  }
};

template <int kCtrl>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, kCtrl, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t swz16_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, (0x10 << 10) | 0x1F);
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  v = min(v, dpp_u<kDppXor1>(v));
  v = min(v, dpp_u<kDppXor2>(v));
  v = min(v, dpp_u<kDppHalfMirror>(v));
  v = min(v, dpp_u<kDppMirror>(v));
  v = min(v, swz16_u(v));
  return min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 32));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, dpp_u<kDppXor1>(v));
  v = max(v, dpp_u<kDppXor2>(v));
  v = max(v, dpp_u<kDppHalfMirror>(v));
  v = max(v, dpp_u<kDppMirror>(v));
  v = max(v, swz16_u(v));
  return max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 32));
}

// inclusive prefix sum over the 64 lanes of a wave, by DPP: shifts of 1, 2, 4, 8 lanes
// inside each 16-lane row, then the row totals carried by the row broadcasts of lanes 15
// and 31 (lanes without a source add 0)
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_or0(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp_or0<0x111, 0xF>(v);  // row_shr:1
  v += dpp_or0<0x112, 0xF>(v);  // row_shr:2
  v += dpp_or0<0x114, 0xF>(v);  // row_shr:4
  v += dpp_or0<0x118, 0xF>(v);  // row_shr:8
  v += dpp_or0<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_or0<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return v;
}
__device__ __forceinline__ uint32_t wave_total(uint32_t incl) {
  return (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
}

// exclusive prefix over the block of one value per thread, with the total
template <int kT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t a, uint32_t* total, TopkSmem<kT>& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t x = wave_incl_scan(a);
  if (lane == 63) sm.wsum[1][wave] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < TopkSmem<kT>::kW; ++w) {
    const uint32_t u = sm.wsum[1][w];
    if (w < wave) before += u;
    tot += u;
  }
  *total = tot;
  return before + x - a;
}

// every key of src[0:n): thread-strided; with vector sources 4 consecutive keys per step
template <int kT, class Src, class F>
__device__ __forceinline__ void for_keys(const Src& src, int n, F f) {
  if constexpr (Src::kRegs) {
    src.each(f);
  } else if constexpr (Src::kVec) {
    for (int i = 4 * threadIdx.x; i < n; i += 4 * kT) {
      const uint4 v = src.key4(i);
      f(v.x);
      if (i + 1 < n) f(v.y);
      if (i + 2 < n) f(v.z);
      if (i + 3 < n) f(v.w);
    }
  } else {
    for (int i = threadIdx.x; i < n; i += kT) f(src.key(i));
  }
}

// the 4 keys [i, i+4) of a segment lane (keys at or past n are reported invalid)
template <class Src>
__device__ __forceinline__ void keys4(const Src& src, int i, int n, uint32_t (&k)[4]) {
  if constexpr (Src::kVec) {
    if (i < n) {
      const uint4 v = src.key4(i);
      k[0] = v.x; k[1] = v.y; k[2] = v.z; k[3] = v.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) k[j] = i + j < n ? src.key(i + j) : 0u;
  }
}

// Threshold T (the k-th largest key of src.key(0..n-1)) and how many keys equal to T are
// taken.  Requires 1 <= k <= n.  Every thread of the block must call it.
//
// With k2 (1 <= k2 <= k) it also reports a cheap estimate of the k2-th largest key: a key
// L2 at the lower edge of the first pass's bin that holds it, with g2 = the exact number of
// keys >= L2 (as a rule at least k2).  Chunked selection uses such pairs to prune candidates
// before the merge; any pair with an exact count is safe there.
template <int kT, class Src>
__device__ __forceinline__ void radix_threshold(const Src& src, int n, int k, TopkSmem<kT>& sm, uint32_t* T_out,
                                uint32_t* take_out, int k2 = 0, uint32_t* L2_out = nullptr,
                                uint32_t* g2_out = nullptr) {
  constexpr int kW = TopkSmem<kT>::kW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < kTopkBins; i += kT) sm.hist[0][i] = 0;
  if (threadIdx.x == 0) sm.ncand = 0;
  // key range [lo, hi]
  uint32_t lo = 0xffffffffu, hi = 0u;
  for_keys<kT>(src, n, [&](uint32_t kk) {
    lo = min(lo, kk);
    hi = max(hi, kk);
  });
  lo = wave_umin(lo);
  hi = wave_umax(hi);
  if (lane == 0) {
    sm.wlo[wave] = lo;
    sm.whi[wave] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    lo = min(lo, sm.wlo[w]);
    hi = max(hi, sm.whi[w]);
  }
  uint32_t krem = (uint32_t)k;
  if (lo == hi) {  // all keys equal: the bound is that key, held by every key
    if (k2 > 0) {
      *L2_out = lo;
      *g2_out = (uint32_t)n;
    }
    *T_out = lo;
    *take_out = krem;
    return;
  }
  // the range [flo, fhi] of the keys of finite scores (another pass only when some are not)
  uint32_t flo = lo, fhi = hi;
  if (lo <= kKeyNegInf || hi >= kKeyPosInf) {  // block-uniform
    flo = 0xffffffffu;
    fhi = 0u;
    for_keys<kT>(src, n, [&](uint32_t kk) {
      flo = min(flo, kk > kKeyNegInf ? kk : 0xffffffffu);
      fhi = max(fhi, kk < kKeyPosInf ? kk : 0u);
    });
    flo = wave_umin(flo);
    fhi = wave_umax(fhi);
    if (lane == 0) {
      sm.wsum[0][wave] = flo;
      sm.wsum[1][wave] = fhi;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      flo = min(flo, sm.wsum[0][w]);
      fhi = max(fhi, sm.wsum[1][w]);
    }
  }
  constexpr int kPer = kTopkBins / kT;
  // thread t owns bins [2048 - kPer(t+1), 2048 - kPer*t): low t = high bins
  const int hb = kTopkBins - kPer * threadIdx.x - 1;

  // first pass: bins linear in the score; hist[1] is cleared for the radix passes
  LinearBins fb;
  fb.init(flo, fhi);
  for (int i = threadIdx.x; i < kTopkBins; i += kT) sm.hist[1][i] = 0;
  for_keys<kT>(src, n, [&](uint32_t kk) { atomicAdd(&sm.hist[0][fb(kk)], 1u); });
  __syncthreads();
  {
    uint32_t local = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) local += sm.hist[0][hb - j];
    const uint32_t incl = wave_incl_scan(local);
    if (lane == 63) sm.wsum[0][wave] = incl;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w)
      if (w < wave) before += sm.wsum[0][w];
    const uint32_t above = before + incl - local;
    if (above < krem && above + local >= krem) {
      uint32_t cum = above;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const uint32_t c = sm.hist[0][hb - j];
        if (cum + c >= krem) {
          sm.sel_bin[0] = (uint32_t)(hb - j);
          sm.krem[0] = krem - cum;
          break;
        }
        cum += c;
      }
    }
    if (k2 > 0 && above < (uint32_t)k2 && above + local >= (uint32_t)k2) {
      uint32_t cum = above;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const uint32_t c = sm.hist[0][hb - j];
        if (cum + c >= (uint32_t)k2) {
          sm.bound_lo = (uint32_t)(hb - j);  // the bin
          sm.bound_cnt = cum + c;
          break;
        }
        cum += c;
      }
    }
  }
  __syncthreads();
  const uint32_t b = sm.sel_bin[0];
  krem = sm.krem[0];
  const uint32_t cb = (uint32_t)__builtin_amdgcn_readfirstlane((int)sm.hist[0][b]);
  const uint32_t b2 = k2 > 0 ? sm.bound_lo : 0u;
  const bool few = cb <= kCandMax;
  // the boundary bin's keys (when few), found among the keys of a cheap range; the bound:
  // a key L2 at the lower edge of bin b2 (an estimate), with the count of keys >= L2
  uint32_t r_lo, r_hi, L2 = 0u;
  fb.key_range(b, &r_lo, &r_hi);
  if (k2 > 0 && b2 > 0) {  // the key of the ideal value b2: bin b2's lower edge, up to rounding
    L2 = fb.a > 0.f ? float_key(((float)b2 - fb.c) / fb.a) : kKeyNegInf;
  }
  uint32_t g2c = 0;
  if (few || k2 > 0) {
    for_keys<kT>(src, n, [&](uint32_t kk) {
      if (few && kk >= r_lo && kk <= r_hi) {
        if (fb(kk) == b) sm.cand[atomicAdd(&sm.ncand, 1u)] = kk;
      }
      if (k2 > 0) g2c += kk >= L2 ? 1u : 0u;
    });
  }
  if (k2 > 0) {
    g2c = wave_total(wave_incl_scan(g2c));
    if (lane == 0) sm.wl2[wave] = g2c;
  }
  __syncthreads();
  if (k2 > 0) {
    uint32_t g = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) g += sm.wl2[w];
    *L2_out = L2;
    *g2_out = g;
  }
  if (few && sm.ncand != cb) {  // the range missed keys of the bin: gather them exactly
    __syncthreads();  // every wave has read ncand
    if (threadIdx.x == 0) sm.ncand = 0;
    __syncthreads();
    for_keys<kT>(src, n, [&](uint32_t kk) {
      if (fb(kk) == b) sm.cand[atomicAdd(&sm.ncand, 1u)] = kk;
    });
    __syncthreads();
  }
  if (few) {
    // every wave ranks the bin's keys: T is the key with fewer than krem keys of the bin
    // above it and at least krem at or above it
    const uint32_t v = (uint32_t)lane < cb ? sm.cand[lane] : 0u;
    uint32_t gt = 0, ge = 0;
    for (uint32_t j = 0; j < cb; ++j) {
      const uint32_t w = sm.cand[j];
      gt += w > v ? 1u : 0u;
      ge += w >= v ? 1u : 0u;
    }
    const bool hit = (uint32_t)lane < cb && gt < krem && krem <= ge;
    const int src_lane = __builtin_ctzll(__ballot(hit));
    *T_out = (uint32_t)__builtin_amdgcn_readlane((int)v, src_lane);
    *take_out = krem - (uint32_t)__builtin_amdgcn_readlane((int)gt, src_lane);
    return;
  }
  // a crowded bin: its key range
  uint32_t bmin = 0xffffffffu, bmax = 0u;
  for_keys<kT>(src, n, [&](uint32_t kk) {
    const bool in = fb(kk) == b;
    bmin = min(bmin, in ? kk : 0xffffffffu);
    bmax = max(bmax, in ? kk : 0u);
  });
  bmin = wave_umin(bmin);
  bmax = wave_umax(bmax);
  if (lane == 0) {
    sm.wlo[wave] = bmin;
    sm.whi[wave] = bmax;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    bmin = min(bmin, sm.wlo[w]);
    bmax = max(bmax, sm.whi[w]);
  }
  // radix passes over the crowded bin's key range
  lo = bmin;
  uint32_t span = bmax - bmin;
  int cur = 1;
  while (span != 0) {
    const int bits = 32 - __builtin_clz(span);
    const int shift = bits > 11 ? bits - 11 : 0;
    const uint32_t top = lo + span;
    // fill hist[cur] (cleared before the last barrier); clear the other for the next pass
    for (int i = threadIdx.x; i < kTopkBins; i += kT) sm.hist[cur ^ 1][i] = 0;
    for_keys<kT>(src, n, [&](uint32_t kk) {
      if (kk >= lo && kk <= top) atomicAdd(&sm.hist[cur][(kk - lo) >> shift], 1u);
    });
    __syncthreads();
    uint32_t local = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) local += sm.hist[cur][hb - j];
    const uint32_t incl = wave_incl_scan(local);
    if (lane == 63) sm.wsum[0][wave] = incl;
    __syncthreads();
    uint32_t before = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w)
      if (w < wave) before += sm.wsum[0][w];
    const uint32_t above = before + incl - local;
    if (above < krem && above + local >= krem) {
      uint32_t cum = above;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const uint32_t c = sm.hist[cur][hb - j];
        if (cum + c >= krem) {
          sm.sel_bin[cur] = (uint32_t)(hb - j);
          sm.krem[cur] = krem - cum;
          break;
        }
        cum += c;
      }
    }
    __syncthreads();
    const uint32_t bb = sm.sel_bin[cur];
    krem = sm.krem[cur];
    const uint32_t blo = lo + (bb << shift);
    const uint32_t bspan = shift == 0 ? 0u : ((1u << shift) - 1u);
    span = min(bspan, top - blo);
    lo = blo;
    cur ^= 1;
  }
  *T_out = lo;
  *take_out = krem;
}

// Walk src[0:n) in index order and call out(pos, i, key) for the selected keys: key > T,
// or key == T among the first take_eq such keys, pos = the key's rank in index order.
// The row is cut into 256-key segments, one wave each, 4 consecutive keys per lane.  A
// first sweep counts every segment's keys above / equal to T; one block scan over the
// segment counts gives each segment its output offset; a second sweep places the keys
// (a wave scan of the per-lane counts orders them inside the segment).
template <int kT, class Src, class Out>
__device__ __forceinline__ void ordered_compact(const Src& src, int n, int k, uint32_t T, uint32_t take_eq, TopkSmem<kT>& sm,
                                Out out) {
  constexpr int kW = TopkSmem<kT>::kW;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t gt_base = 0, eq_base = 0;  // counts before the current sweep (block-uniform)
  for (int base = 0; base < n; base += kSegKeys * kSegMax) {
    const int nseg = min(kSegMax, (n - base + kSegKeys - 1) / kSegKeys);
    for (int s = wave; s < nseg; s += kW) {
      const int i = base + kSegKeys * s + 4 * lane;
      uint32_t kk[4] = {0u, 0u, 0u, 0u};
      keys4(src, i, n, kk);
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i + j < n) c += kk[j] > T ? 1u : (kk[j] == T ? 0x10000u : 0u);
      const uint32_t tot = wave_total(wave_incl_scan(c));
      if (lane == 0) sm.seg[s] = tot;
    }
    __syncthreads();
    // segment offsets: thread t takes segment t (nseg <= kSegMax <= kT)
    const uint32_t mine = threadIdx.x < nseg ? sm.seg[threadIdx.x] : 0u;
    uint32_t total;
    const uint32_t ex = block_excl_scan<kT>(mine, &total, sm);  // both 16-bit halves at once
    if (threadIdx.x < nseg) sm.seg[threadIdx.x] = ex;
    __syncthreads();
    for (int s = wave; s < nseg; s += kW) {
      const uint32_t sg = sm.seg[s];
      uint32_t g = gt_base + (sg & 0xffffu), e = eq_base + (sg >> 16);
      if (g + min(e, take_eq) >= (uint32_t)k) break;  // wave-uniform; later segments come later
      const int i = base + kSegKeys * s + 4 * lane;
      uint32_t kk[4] = {0u, 0u, 0u, 0u};
      keys4(src, i, n, kk);
      uint32_t c = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i + j < n) c += kk[j] > T ? 1u : (kk[j] == T ? 0x10000u : 0u);
      const uint32_t ex_lane = wave_incl_scan(c) - c;
      g += ex_lane & 0xffffu;
      e += ex_lane >> 16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (i + j >= n) break;
        if (kk[j] > T) {
          const uint32_t pos = g + min(e, take_eq);
          if (pos < (uint32_t)k) out(pos, i + j, kk[j]);  // always true when the threshold is exact
          ++g;
        } else if (kk[j] == T) {
          if (e < take_eq && g + e < (uint32_t)k) out(g + e, i + j, kk[j]);
          ++e;
        }
      }
    }
    gt_base += total & 0xffffu;
    eq_base += total >> 16;
    if (gt_base + min(eq_base, take_eq) >= (uint32_t)k) break;  // block-uniform
    __syncthreads();  // the segment counts are refilled by the next sweep
  }
}

// Rank of the per-chunk pruning bound in chunked selection: ceil(k / (nchunks - 1)), so
// that the full chunks alone (all but possibly the last) hold at least k keys at or above
// their bounds.
__host__ __device__ __forceinline__ int bound_rank(int k, int nchunks) {
  const int d = nchunks > 1 ? nchunks - 1 : 1;
  const int k2 = (k + d - 1) / d;
  return k2 < k ? k2 : k;
}

// key sources
struct KeysLds {
  static constexpr bool kRegs = false;
  static constexpr bool kVec = true;  // 16-byte aligned, readable in groups of 4
  const uint32_t* keys;
  __device__ __forceinline__ uint32_t key(int i) const { return keys[i]; }
  __device__ __forceinline__ uint4 key4(int i) const { return *reinterpret_cast<const uint4*>(keys + i); }
};
struct KeysGlobal {  // keys in global memory, any alignment
  static constexpr bool kRegs = false;
  static constexpr bool kVec = false;
  const uint32_t* keys;
  __device__ __forceinline__ uint32_t key(int i) const { return keys[i]; }
};
struct KeysScores {
  static constexpr bool kRegs = false;
  static constexpr bool kVec = false;
  const float* scores;
  int force;  // index whose key is forced to the maximum, or -1
  __device__ __forceinline__ uint32_t key(int i) const {
    return i == force ? 0xffffffffu : float_key(scores[i]);
  }
};

// ---------------------------------------------------------------- keys held in registers
// A chunk of n <= 4 * kT * kJ keys spread over the block's registers: in row j, thread t
// holds the keys [4t + 4 kT j, +4) - the layout of the compaction segments above, where
// row j of wave w is segment kW j + w.  The selection passes then read no LDS; only the
// histogram counts go there.  Slots at or past n hold 0.
template <int kT, int kJ>
struct KeyRegs {
  static constexpr bool kRegs = true;
  static constexpr bool kVec = false;
  uint4 v[kJ];
  int n, rows;  // rows: the rows that hold keys below n

  // every key below n, in any order
  template <class F>
  __device__ __forceinline__ void each(F f) const {
    const int i0 = 4 * (int)threadIdx.x;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      if (4 * kT * (j + 1) <= n) {  // a full row (block-uniform)
        f(v[j].x); f(v[j].y); f(v[j].z); f(v[j].w);
      } else if (j < rows) {
        const int i = i0 + 4 * kT * j;
        if (i < n) f(v[j].x);
        if (i + 1 < n) f(v[j].y);
        if (i + 2 < n) f(v[j].z);
        if (i + 3 < n) f(v[j].w);
      }
    }
  }
};

// the n keys of an LDS array (16-byte aligned) into registers
template <int kT, int kJ>
__device__ __forceinline__ void key_regs_load(KeyRegs<kT, kJ>& r, const uint32_t* keys, int n) {
  r.n = n;
  r.rows = (n + 4 * kT - 1) / (4 * kT);
  const int i0 = 4 * (int)threadIdx.x;
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    r.v[j] = make_uint4(0u, 0u, 0u, 0u);
    if (j < r.rows) {
      const int i = i0 + 4 * kT * j;
      if (i + 3 < n) {
        r.v[j] = *reinterpret_cast<const uint4*>(keys + i);
      } else if (i < n) {
        r.v[j].x = keys[i];
        if (i + 1 < n) r.v[j].y = keys[i + 1];
        if (i + 2 < n) r.v[j].z = keys[i + 2];
      }
    }
  }
}

// the keys of n fp32 scores in global memory; key index `force` (if >= 0) is forced to
// the maximum
template <int kT, int kJ>
__device__ __forceinline__ void key_regs_load_scores(KeyRegs<kT, kJ>& r, const float* scores, int n, int force) {
  r.n = n;
  r.rows = (n + 4 * kT - 1) / (4 * kT);
  const bool vec = (((uintptr_t)scores) & 15u) == 0;
  const int i0 = 4 * (int)threadIdx.x;
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    r.v[j] = make_uint4(0u, 0u, 0u, 0u);
    if (j < r.rows) {
      const int i = i0 + 4 * kT * j;
      if (vec && i + 3 < n) {
        const float4 f = *reinterpret_cast<const float4*>(scores + i);
        r.v[j] = make_uint4(float_key(f.x), float_key(f.y), float_key(f.z), float_key(f.w));
      } else {
        if (i < n) r.v[j].x = float_key(scores[i]);
        if (i + 1 < n) r.v[j].y = float_key(scores[i + 1]);
        if (i + 2 < n) r.v[j].z = float_key(scores[i + 2]);
        if (i + 3 < n) r.v[j].w = float_key(scores[i + 3]);
      }
      if (force >= i && force < i + 4) {
        if (force == i) r.v[j].x = 0xffffffffu;
        else if (force == i + 1) r.v[j].y = 0xffffffffu;
        else if (force == i + 2) r.v[j].z = 0xffffffffu;
        else r.v[j].w = 0xffffffffu;
      }
    }
  }
}

// ordered_compact over register keys (one sweep, n <= kSegKeys * kSegMax).  Requires
// T > 0, so the zero slots past n are never taken.
template <int kT, int kJ, class Out>
__device__ __forceinline__ void ordered_compact_regs(const KeyRegs<kT, kJ>& r, int k, uint32_t T, uint32_t take_eq,
                                                     TopkSmem<kT>& sm, Out out) {
  constexpr int kW = TopkSmem<kT>::kW;
  static_assert(kW * kJ <= kSegMax, "one compaction sweep");
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto cnt = [&](uint32_t kk) { return kk > T ? 1u : (kk == T ? 0x10000u : 0u); };
  uint32_t exl[kJ];  // this lane's exclusive prefix inside its segment of row j
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    exl[j] = 0u;
    if (j < r.rows) {
      const uint32_t c = cnt(r.v[j].x) + cnt(r.v[j].y) + cnt(r.v[j].z) + cnt(r.v[j].w);
      const uint32_t incl = wave_incl_scan(c);
      exl[j] = incl - c;
      if (lane == 63) sm.seg[kW * j + wave] = incl;
    }
  }
  __syncthreads();
  // Few segments (at most 32): every wave forms the offsets of its own segments from the
  // segment totals, row by row, with a few broadcast reads - no block-wide scan and no second
  // barrier.  More segments: one block scan over them.
  constexpr bool kDirect = kW * kJ <= 32;
  if constexpr (!kDirect) {
    const int nseg = kW * r.rows;
    const uint32_t mine = (int)threadIdx.x < nseg ? sm.seg[threadIdx.x] : 0u;
    uint32_t total;
    const uint32_t ex = block_excl_scan<kT>(mine, &total, sm);
    if ((int)threadIdx.x < nseg) sm.seg[threadIdx.x] = ex;
    __syncthreads();
  }
  const int i0 = 4 * (int)threadIdx.x;
  bool done = false;  // wave-uniform: every later row lies past the k-th selected key
  uint32_t rowbase = 0;  // direct offsets: the totals of the rows before row j
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    if (done || j >= r.rows) continue;
    uint32_t sg;
    if constexpr (kDirect) {
      uint32_t before = 0, rowtot = 0;
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        const uint32_t v = sm.seg[kW * j + w];
        before += w < wave ? v : 0u;
        rowtot += v;
      }
      sg = rowbase + before;
      rowbase += rowtot;
    } else {
      sg = sm.seg[kW * j + wave];
    }
    uint32_t g = sg & 0xffffu, e = sg >> 16;
    if (g + min(e, take_eq) >= (uint32_t)k) {
      done = true;
      continue;
    }
    g += exl[j] & 0xffffu;
    e += exl[j] >> 16;
    const uint32_t kk[4] = {r.v[j].x, r.v[j].y, r.v[j].z, r.v[j].w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (kk[c] > T) {
        const uint32_t pos = g + min(e, take_eq);
        if (pos < (uint32_t)k) out(pos, i0 + 4 * kT * j + c, kk[c]);
        ++g;
      } else if (kk[c] == T) {
        if (e < take_eq && g + e < (uint32_t)k) out(g + e, i0 + 4 * kT * j + c, kk[c]);
        ++e;
      }
    }
  }
}

}  // namespace csa2
