// Exact top-k selection ([DSA-to-CSA notes] eq. (17)) by radix select, and the expansion
// of selected blocks into the hierarchical candidate pool ([CSA2 column]
// "解码器里的分层索引"; [Evolution blog] §4.4).
//
// Scores become order-preserving uint32 keys (-0 maps to +0).  Three histogram passes
// over 11/11/10-bit digits (LDS histograms, one workgroup per row or row chunk) find the
// exact k-th largest key T and how many keys equal to T must be taken.  A final pass walks
// the row in index order; one ballot per wave plus a cross-wave prefix in LDS gives every
// selected element its output slot, so the output is ascending and ties go to the lower
// index, deterministically.
//
// Rows longer than kSingleMax use two levels: chunks of a row are reduced to their own
// top-k (exact: the global top-k is contained in the union of the chunks' top-k), written
// as (key, slot) pairs in index order, then a second pass selects from the pairs; slot
// order of the pairs equals index order, so the tie rule carries over.

#include "common.h"
#include "internal.h"

namespace csa2 {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesTk = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kSingleMax = 32768;

struct RowSrc {
  // either fp32 scores or uint32 keys (two-level second pass)
  const float* scores;
  const uint32_t* keys;
  int force;  // slot whose key is forced to the maximum, or -1
  __device__ __forceinline__ uint32_t key(int i) const {
    if (i == force) return 0xffffffffu;
    return scores ? float_key(scores[i]) : keys[i];
  }
};

struct alignas(16) Smem {
  uint32_t hist[kBins];
  uint32_t wsum[kWavesTk];
  uint32_t wgt[kWavesTk], weq[kWavesTk];
  uint32_t sel_digit, krem;
};

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }
__device__ __forceinline__ uint64_t lt_mask() {
  const int l = threadIdx.x % 64;
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// exclusive prefix over the block of one value per thread; also returns the total
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, Smem& sm) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sm.wsum[wave] = x;
  __syncthreads();
  uint32_t before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWavesTk; ++w) {
    if (w < wave) before += sm.wsum[w];
    tot += sm.wsum[w];
  }
  __syncthreads();
  *total = tot;
  return before + x - v;
}

// Finds the threshold key T (k-th largest) of src[0:n) and the number of keys == T to
// take.  Requires 1 <= k <= n.
__device__ void radix_threshold(const RowSrc& src, int n, int k, Smem& sm, uint32_t* T_out,
                                uint32_t* take_eq_out) {
  uint32_t prefix = 0;
  uint32_t krem = (uint32_t)k;
  const int shifts[3] = {21, 10, 0};
  const uint32_t digit_bits[3] = {11, 11, 10};
  for (int pass = 0; pass < 3; ++pass) {
    const int sh = shifts[pass];
    const uint32_t dmask = (1u << digit_bits[pass]) - 1u;
    const int hi_sh = sh + (int)digit_bits[pass];  // bits above this digit must equal prefix
    for (int i = threadIdx.x; i < kBins; i += kThreads) sm.hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kThreads) {
      const uint32_t kk = src.key(i);
      const bool match = hi_sh >= 32 ? true : ((kk >> hi_sh) == (prefix >> hi_sh));
      if (match) atomicAdd(&sm.hist[(kk >> sh) & dmask], 1u);
    }
    __syncthreads();
    // thread t owns the 8 bins [kBins-8(t+1), kBins-8t): low t = high digits
    const int nb = (int)dmask + 1;
    const int per = nb / kThreads;  // 8 (11-bit) or 4 (10-bit)
    const int top = nb - per * threadIdx.x - 1;
    uint32_t local = 0;
    for (int j = 0; j < per; ++j) local += sm.hist[top - j];
    uint32_t tot;
    uint32_t above = block_excl_scan(local, &tot, sm);
    if (above < krem && above + local >= krem) {
      uint32_t cum = above;
      for (int j = 0; j < per; ++j) {
        const uint32_t hcount = sm.hist[top - j];
        if (cum + hcount >= krem) {
          sm.sel_digit = (uint32_t)(top - j);
          sm.krem = krem - cum;
          break;
        }
        cum += hcount;
      }
    }
    __syncthreads();
    prefix |= sm.sel_digit << sh;
    krem = sm.krem;
    __syncthreads();
  }
  *T_out = prefix;
  *take_eq_out = krem;
}

// Walk src[0:n) in index order and call out(pos, i, key) for every selected element:
// key > T, or key == T among the first take_eq such keys.  Stops after k selections.
template <class Out>
__device__ void ordered_compact(const RowSrc& src, int n, int k, uint32_t T, uint32_t take_eq, Smem& sm,
                                Out out) {
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  uint32_t sel_seen = 0, eq_seen = 0;
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + threadIdx.x;
    const bool valid = i < n;
    const uint32_t kk = valid ? src.key(i) : 0u;
    const bool gt = valid && kk > T;
    const bool eq = valid && kk == T;
    const uint64_t mgt = ballot64(gt), meq = ballot64(eq);
    if (lane == 0) {
      sm.wgt[wave] = (uint32_t)__popcll(mgt);
      sm.weq[wave] = (uint32_t)__popcll(meq);
    }
    __syncthreads();
    uint32_t eq_before = eq_seen, sel_before = sel_seen, tot_sel = 0, tot_eq = 0;
    uint32_t my_take = 0;
#pragma unroll
    for (int w = 0; w < kWavesTk; ++w) {
      const uint32_t e_before_w = eq_seen + tot_eq;
      const uint32_t take_w = take_eq > e_before_w ? min(take_eq - e_before_w, sm.weq[w]) : 0u;
      if (w < wave) { sel_before += sm.wgt[w] + take_w; eq_before += sm.weq[w]; }
      if (w == wave) my_take = take_w;
      tot_sel += sm.wgt[w] + take_w;
      tot_eq += sm.weq[w];
    }
    const uint64_t lt = lt_mask();
    const uint32_t eq_rank_in_wave = (uint32_t)__popcll(meq & lt);
    const bool take = gt || (eq && eq_rank_in_wave < my_take);
    if (take) {
      const uint32_t pos = sel_before + (uint32_t)__popcll(mgt & lt) + min(eq_rank_in_wave, my_take);
      if (pos < (uint32_t)k) out(pos, i, kk);  // always true when the threshold is exact
    }
    sel_seen += tot_sel;
    eq_seen += tot_eq;
    __syncthreads();
    (void)eq_before;
    if (sel_seen >= (uint32_t)k) break;  // uniform: every thread holds the same counts
  }
}

struct Params {
  int rows, k;
  const float* scores;
  int64_t row_stride;
  const int32_t* counts;
  const int32_t* q_pos;
  int N, m, len_div;
  int force_last;
  const int32_t* idx_map;
  int64_t idx_map_stride;
  int32_t* out_idx;
  int max_len;  // row lengths are clamped to this (the row stride of the scores)
  // two-level
  int chunk, nchunks;
  uint32_t* ws_keys;  // [rows, nchunks*k]
  int32_t* ws_slot;   // [rows, nchunks*k]
};

__device__ __forceinline__ int row_len(const Params& p, int r) {
  int len;
  if (p.counts) {
    len = p.counts[r];
  } else {
    const int t = p.q_pos[r];
    len = t >= 0 ? t / p.m : 0;
    if (len > p.N) len = p.N;
  }
  if (p.len_div > 1) len = (len + p.len_div - 1) / p.len_div;
  if (len > p.max_len) len = p.max_len;
  return len < 0 ? 0 : len;
}

__device__ __forceinline__ int32_t map_id(const Params& p, int r, int slot) {
  return p.idx_map ? p.idx_map[(size_t)r * p.idx_map_stride + slot] : slot;
}

// Keys of a row or chunk staged once into LDS (vector loads); all passes then run from
// LDS.  Up to kStageMax keys are staged; longer rows are read from global memory.
constexpr int kStageMax = 32768;

__device__ __forceinline__ void stage_keys(const float* scores, int n, int force, uint32_t* keys) {
  const bool vec = (((uintptr_t)scores) & 15u) == 0;
  const int n4 = vec ? n / 4 : 0;
  for (int i = threadIdx.x; i < n4; i += kThreads) {
    const float4 v = reinterpret_cast<const float4*>(scores)[i];
    keys[4 * i] = float_key(v.x); keys[4 * i + 1] = float_key(v.y);
    keys[4 * i + 2] = float_key(v.z); keys[4 * i + 3] = float_key(v.w);
  }
  for (int i = 4 * n4 + threadIdx.x; i < n; i += kThreads) keys[i] = float_key(scores[i]);
  __syncthreads();
  if (force >= 0 && threadIdx.x == 0) keys[force] = 0xffffffffu;
  __syncthreads();
}

// single level: one workgroup per row
__global__ void __launch_bounds__(kThreads) topk_single(Params p, int stage_cap) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  uint32_t* skeys = reinterpret_cast<uint32_t*>(smem_raw + sizeof(Smem));
  const int r = blockIdx.x;
  const int n = row_len(p, r);
  int32_t* out = p.out_idx + (size_t)r * p.k;
  if (n <= p.k) {
    for (int i = threadIdx.x; i < p.k; i += kThreads) out[i] = i < n ? map_id(p, r, i) : -1;
    return;
  }
  const float* row = p.scores + (size_t)r * p.row_stride;
  const int force = p.force_last ? n - 1 : -1;
  RowSrc src{row, nullptr, force};
  if (n <= stage_cap) {
    stage_keys(row, n, force, skeys);
    src = RowSrc{nullptr, skeys, -1};
  }
  uint32_t T, take;
  radix_threshold(src, n, p.k, sm, &T, &take);
  ordered_compact(src, n, p.k, T, take, sm, [&](uint32_t pos, int i, uint32_t) { out[pos] = map_id(p, r, i); });
}

// two-level, first level: grid (rows, nchunks); chunk c of row r -> ws[r][c*k .. c*k+k)
__global__ void __launch_bounds__(kThreads) topk_chunk(Params p, int stage_cap) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  uint32_t* skeys = reinterpret_cast<uint32_t*>(smem_raw + sizeof(Smem));
  const int r = blockIdx.x, c = blockIdx.y;
  const int n = row_len(p, r);
  const int c0 = c * p.chunk;
  const int len = max(0, min(p.chunk, n - c0));
  uint32_t* ok = p.ws_keys + ((size_t)r * p.nchunks + c) * p.k;
  int32_t* os = p.ws_slot + ((size_t)r * p.nchunks + c) * p.k;
  const int force = (p.force_last && n > 0 && n - 1 >= c0 && n - 1 < c0 + p.chunk) ? (n - 1 - c0) : -1;
  const float* row = p.scores + (size_t)r * p.row_stride + c0;
  RowSrc src{row, nullptr, force};
  if (len <= p.k) {
    for (int i = threadIdx.x; i < p.k; i += kThreads) {
      ok[i] = i < len ? src.key(i) : 0u;
      os[i] = i < len ? c0 + i : -1;
    }
    return;
  }
  if (len <= stage_cap) {
    stage_keys(row, len, force, skeys);
    src = RowSrc{nullptr, skeys, -1};
  }
  uint32_t T, take;
  radix_threshold(src, len, p.k, sm, &T, &take);
  ordered_compact(src, len, p.k, T, take, sm, [&](uint32_t pos, int i, uint32_t key) {
    ok[pos] = key;
    os[pos] = c0 + i;
  });
}

// two-level, second level: one workgroup per row over nchunks*k pairs; key 0 marks padding
__global__ void __launch_bounds__(kThreads) topk_merge(Params p, int stage_cap) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  uint32_t* skeys = reinterpret_cast<uint32_t*>(smem_raw + sizeof(Smem));
  const int r = blockIdx.x;
  const int n = row_len(p, r);
  int32_t* out = p.out_idx + (size_t)r * p.k;
  const int32_t* slots = p.ws_slot + (size_t)r * p.nchunks * p.k;
  if (n <= p.k) {
    for (int i = threadIdx.x; i < p.k; i += kThreads) out[i] = i < n ? map_id(p, r, i) : -1;
    return;
  }
  const int m = p.nchunks * p.k;
  const uint32_t* gkeys = p.ws_keys + (size_t)r * m;
  RowSrc src{nullptr, gkeys, -1};
  if (m <= stage_cap) {
    const uint4* g4 = reinterpret_cast<const uint4*>(gkeys);  // k is a multiple of 4 here or not:
    if ((m & 3) == 0 && (((uintptr_t)gkeys) & 15u) == 0) {
      for (int i = threadIdx.x; i < m / 4; i += kThreads) reinterpret_cast<uint4*>(skeys)[i] = g4[i];
    } else {
      for (int i = threadIdx.x; i < m; i += kThreads) skeys[i] = gkeys[i];
    }
    __syncthreads();
    src = RowSrc{nullptr, skeys, -1};
  }
  uint32_t T, take;
  radix_threshold(src, m, p.k, sm, &T, &take);
  ordered_compact(src, m, p.k, T, take, sm, [&](uint32_t pos, int i, uint32_t) {
    const int sl = slots[i];
    out[pos] = sl >= 0 ? map_id(p, r, sl) : -1;
  });
}

// expand selected blocks (ascending, -1 padded, the latest visible block included) into
// positions; one workgroup per row
__global__ void __launch_bounds__(kThreads) hier_expand(int n_keep, int block, const int32_t* sel,
                                                         const int32_t* q_pos, int N, int m,
                                                         int32_t* cand, int32_t* count) {
  const int r = blockIdx.x;
  const int t = q_pos[r];
  int nv = t >= 0 ? t / m : 0;
  if (nv > N) nv = N;
  const int32_t* s = sel + (size_t)r * n_keep;
  int32_t* o = cand + (size_t)r * n_keep * block;
  const int total = n_keep * block;
  for (int q = threadIdx.x; q < total; q += kThreads) {
    const int bi = q / block, u = q % block;
    const int blk = s[bi];
    const int pos = blk >= 0 ? blk * block + u : -1;
    // only the latest (highest, last-listed) block can be partial; its tail maps to -1 and
    // sits at the end of the list, so the valid positions stay contiguous and ascending
    o[q] = (pos >= 0 && pos < nv) ? pos : -1;
  }
  if (threadIdx.x == 0) {
    const int nb = (nv + block - 1) / block;
    const int kept = nb < n_keep ? nb : n_keep;
    count[r] = kept == 0 ? 0 : (kept - 1) * block + (nv - (nb - 1) * block);
  }
}

__global__ void copy_i32(const int32_t* src, int32_t* dst, size_t n) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) dst[i] = src[i];
}

int pick_chunk(int max_len, int k) {
  // chunk size: a power of two >= 8192 such that the merge row (nchunks*k) stays <= 16384
  int chunk = 8192;
  while ((long long)((max_len + chunk - 1) / chunk) * k > 16384 && chunk < (1 << 30)) chunk *= 2;
  return chunk;
}

}  // namespace

size_t topk_workspace_bytes(int rows, int k, int max_len) {
  if (max_len <= kSingleMax) return 0;
  const int chunk = pick_chunk(max_len, k);
  const size_t nchunks = (size_t)(max_len + chunk - 1) / chunk;
  return (size_t)rows * nchunks * k * (sizeof(uint32_t) + sizeof(int32_t));
}

static hipError_t set_lds(const void* fn, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  // every pointer a kernel dereferences must be set
  if (!a.out_idx || (a.max_len > 0 && !a.scores) || (!a.counts && !a.q_pos) ||
      (a.max_len > kSingleMax && (!a.ws || a.ws_bytes < topk_workspace_bytes(a.rows, a.k, a.max_len))))
    return hipErrorInvalidValue;
  Params p{};
  p.rows = a.rows; p.k = a.k; p.scores = a.scores; p.row_stride = a.row_stride;
  p.counts = a.counts; p.q_pos = a.q_pos; p.N = a.N; p.m = a.m; p.len_div = a.len_div;
  p.force_last = a.force_last; p.idx_map = a.idx_map; p.idx_map_stride = a.idx_map_stride;
  p.out_idx = a.out_idx;
  p.max_len = a.max_len;
  hipError_t e;
  if (a.max_len <= kSingleMax) {
    const int cap = a.max_len < kStageMax ? a.max_len : kStageMax;
    const size_t lds = sizeof(Smem) + (size_t)cap * 4;
    if ((e = set_lds((const void*)topk_single, lds)) != hipSuccess) return e;
    ScopedProf pr(s, "topk_single");
    hipLaunchKernelGGL(topk_single, dim3(a.rows), dim3(kThreads), lds, s, p, cap);
    return hipGetLastError();
  }
  p.chunk = pick_chunk(a.max_len, a.k);
  p.nchunks = (a.max_len + p.chunk - 1) / p.chunk;
  p.ws_keys = (uint32_t*)a.ws;
  p.ws_slot = (int32_t*)((char*)a.ws + (size_t)a.rows * p.nchunks * a.k * sizeof(uint32_t));
  {
    const int cap = p.chunk < kStageMax ? p.chunk : kStageMax;
    const size_t lds = sizeof(Smem) + (size_t)cap * 4;
    if ((e = set_lds((const void*)topk_chunk, lds)) != hipSuccess) return e;
    ScopedProf pr(s, "topk_chunk");
    hipLaunchKernelGGL(topk_chunk, dim3(a.rows, p.nchunks), dim3(kThreads), lds, s, p, cap);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    const int m = p.nchunks * a.k;
    const int cap = m < kStageMax ? m : kStageMax;
    const size_t lds = sizeof(Smem) + (size_t)cap * 4;
    if ((e = set_lds((const void*)topk_merge, lds)) != hipSuccess) return e;
    ScopedProf pr(s, "topk_merge");
    hipLaunchKernelGGL(topk_merge, dim3(a.rows), dim3(kThreads), lds, s, p, cap);
  }
  return hipGetLastError();
}

hipError_t launch_hier_expand(int rows, int n_keep, int block, const int32_t* sel_blocks,
                              const int32_t* q_pos, int N, int m, int32_t* out_cand,
                              int32_t* out_count, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (!sel_blocks || !q_pos || !out_cand || !out_count) return hipErrorInvalidValue;
  ScopedProf pr(s, "hier_expand");
  hipLaunchKernelGGL(hier_expand, dim3(rows), dim3(kThreads), 0, s, n_keep, block, sel_blocks, q_pos,
                     N, m, out_cand, out_count);
  return hipGetLastError();
}

hipError_t launch_copy_idx(const int32_t* src, int32_t* dst, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  if (!src || !dst) return hipErrorInvalidValue;
  ScopedProf pr(s, "reuse_copy");
  const size_t blocks = (n + 255) / 256;
  const int grid = (int)(blocks < 4096 ? blocks : 4096);
  hipLaunchKernelGGL(copy_i32, dim3(grid), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

}  // namespace csa2
