// Exact top-k selection inside one workgroup ([DSA-to-CSA notes] eq. (17)): the k largest
// keys of a row, ties to the lower index, reported in index order.
//
// Keys are order-preserving uint32 images of the scores (see float_key).  The threshold
// T (the k-th largest key) is found by range-adaptive radix passes: the live key range
// [lo, lo+span] starts as [min, max]; each pass histograms (key - lo) >> shift into at most
// 2048 LDS bins (shift chosen from the span), keeps the bin holding the k-th largest key
// and narrows the range to it, until the range is a single key.  Clustered scores (the
// usual case once rows hold only candidates) therefore still spread over many bins, so
// LDS atomics rarely collide.  A final pass walks the row in index order; one ballot per
// wave plus a cross-wave prefix gives every selected key its output slot, so the output
// is ascending and ties resolve to the lower index.
#pragma once

#include "common.h"

namespace csa2 {

constexpr int kTopkBins = 2048;

template <int kT>
struct TopkSmem {
  static constexpr int kW = kT / 64;
  uint32_t hist[kTopkBins];
  uint32_t wsum[kW];
  uint32_t wgt[kW], weq[kW];
  uint32_t wlo[kW], whi[kW];
  uint32_t sel_bin, krem;
};

__device__ __forceinline__ uint64_t lane_lt_mask() {
  const int l = threadIdx.x & 63;
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

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

// exclusive prefix over the block of one value per thread; the total through *total
template <int kT>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, TopkSmem<kT>& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sm.wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < TopkSmem<kT>::kW; ++w) {
    if (w < wave) before += sm.wsum[w];
    tot += sm.wsum[w];
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Threshold T (the k-th largest key of src.key(0..n-1)) and how many keys equal to T are
// taken.  Requires 1 <= k <= n.  Every thread of the block must call it.
template <int kT, class Src>
__device__ void radix_threshold(const Src& src, int n, int k, TopkSmem<kT>& sm, uint32_t* T_out,
                                uint32_t* take_out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // live range [lo, lo + span]
  uint32_t lo = 0xffffffffu, hi = 0u;
  for (int i = threadIdx.x; i < n; i += kT) {
    const uint32_t kk = src.key(i);
    lo = min(lo, kk);
    hi = max(hi, kk);
  }
  lo = wave_umin(lo);
  hi = wave_umax(hi);
  if (lane == 0) { sm.wlo[wave] = lo; sm.whi[wave] = hi; }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < TopkSmem<kT>::kW; ++w) { lo = min(lo, sm.wlo[w]); hi = max(hi, sm.whi[w]); }
  uint32_t span = hi - lo;
  uint32_t krem = (uint32_t)k;
  constexpr int kPer = kTopkBins / kT;
  while (span != 0) {
    const int bits = 32 - __builtin_clz(span);
    const int shift = bits > 11 ? bits - 11 : 0;
    const uint32_t top = lo + span;
    for (int i = threadIdx.x; i < kTopkBins; i += kT) sm.hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kT) {
      const uint32_t kk = src.key(i);
      if (kk >= lo && kk <= top) atomicAdd(&sm.hist[(kk - lo) >> shift], 1u);
    }
    __syncthreads();
    // thread t owns bins [2048 - kPer(t+1), 2048 - kPer*t): low t = high bins
    const int hb = kTopkBins - kPer * threadIdx.x - 1;
    uint32_t local = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) local += sm.hist[hb - j];
    uint32_t tot;
    const uint32_t above = block_excl_scan<kT>(local, &tot, sm);
    if (above < krem && above + local >= krem) {
      uint32_t cum = above;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        const uint32_t c = sm.hist[hb - j];
        if (cum + c >= krem) {
          sm.sel_bin = (uint32_t)(hb - j);
          sm.krem = krem - cum;
          break;
        }
        cum += c;
      }
    }
    __syncthreads();
    const uint32_t b = sm.sel_bin;
    krem = sm.krem;
    __syncthreads();
    const uint32_t blo = lo + (b << shift);
    const uint32_t bspan = shift == 0 ? 0u : ((1u << shift) - 1u);
    span = min(bspan, top - blo);
    lo = blo;
  }
  *T_out = lo;
  *take_out = krem;
}

// Walk src[0:n) in index order and call out(pos, i, key) for the selected keys: key > T,
// or key == T among the first take_eq such keys.  Stops after k selections.
template <int kT, class Src, class Out>
__device__ void ordered_compact(const Src& src, int n, int k, uint32_t T, uint32_t take_eq, TopkSmem<kT>& sm,
                                Out out) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t sel_seen = 0, eq_seen = 0;
  for (int base = 0; base < n; base += kT) {
    const int i = base + threadIdx.x;
    const bool valid = i < n;
    const uint32_t kk = valid ? src.key(i) : 0u;
    const bool gt = valid && kk > T;
    const bool eq = valid && kk == T;
    const uint64_t mgt = __ballot(gt), meq = __ballot(eq);
    if (lane == 0) {
      sm.wgt[wave] = (uint32_t)__popcll(mgt);
      sm.weq[wave] = (uint32_t)__popcll(meq);
    }
    __syncthreads();
    uint32_t sel_before = sel_seen, tot_sel = 0, tot_eq = 0, my_take = 0;
#pragma unroll
    for (int w = 0; w < TopkSmem<kT>::kW; ++w) {
      const uint32_t e_before_w = eq_seen + tot_eq;
      const uint32_t take_w = take_eq > e_before_w ? min(take_eq - e_before_w, sm.weq[w]) : 0u;
      if (w < wave) sel_before += sm.wgt[w] + take_w;
      if (w == wave) my_take = take_w;
      tot_sel += sm.wgt[w] + take_w;
      tot_eq += sm.weq[w];
    }
    const uint64_t lt = lane_lt_mask();
    const uint32_t eq_rank = (uint32_t)__popcll(meq & lt);
    if (gt || (eq && eq_rank < my_take)) {
      const uint32_t pos = sel_before + (uint32_t)__popcll(mgt & lt) + min(eq_rank, my_take);
      if (pos < (uint32_t)k) out(pos, i, kk);  // always true when the threshold is exact
    }
    sel_seen += tot_sel;
    eq_seen += tot_eq;
    __syncthreads();
    if (sel_seen >= (uint32_t)k) break;  // uniform: every thread holds the same counts
  }
}

// key sources
struct KeysLds {
  const uint32_t* keys;
  __device__ __forceinline__ uint32_t key(int i) const { return keys[i]; }
};
struct KeysScores {
  const float* scores;
  int force;  // index whose key is forced to the maximum, or -1
  __device__ __forceinline__ uint32_t key(int i) const {
    return i == force ? 0xffffffffu : float_key(scores[i]);
  }
};

}  // namespace csa2
