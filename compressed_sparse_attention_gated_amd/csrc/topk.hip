// Exact top-k selection ([DSA-to-CSA notes] eq. (17)) by radix select, and the expansion
// of selected blocks into the hierarchical candidate pool ([CSA2 column]
// "解码器里的分层索引"; [Evolution blog] §4.4).
//
// Scores become order-preserving uint32 keys (-0 maps to +0).  Range-adaptive histogram
// passes (at most 2048 LDS bins each, over the live key range) find the exact k-th largest
// key T and how many keys equal to T are taken (topk_core.h).  A compaction then walks the
// row in index order: per-segment counts, one block scan, and a wave scan inside each
// segment give every selected element its output slot, so the output is ascending and
// ties go to the lower index, deterministically.
//
// Rows of up to 16,384 keys are loaded from their scores straight into registers and
// selected there (the LDS holds only histograms); longer rows up to kSingleMax are staged
// in LDS or read from global memory.  Rows longer than kSingleMax use two levels: chunks of
// a row are reduced to their own top-k (exact: the global top-k is contained in the union
// of the chunks' top-k), written as (key, slot) pairs in index order, then topk_merge
// selects from the pairs, pruned by each chunk's first-pass bound; slot order of the pairs
// equals index order, so the tie rule carries over.

#include "common.h"
#include "internal.h"
#include "topk_core.h"

namespace csa2 {
namespace {

constexpr int kThreads = 256;       // single rows and chunks
constexpr int kMergeThreads = 1024; // merge rows (few workgroups, long rows)
constexpr int kSingleMax = 32768;
constexpr size_t kLdsMax = 160 * 1024;  // LDS per workgroup on gfx950
constexpr int kWideBelow = 256;          // fewer workgroups than this: 1024 threads each

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
  uint2* ws_bound;    // [rows, nchunks]: (bound, count) - count keys of the chunk are >= bound
  const int32_t* id_base;  // [rows] or null: reported id = slot + id_base[row]
};



__device__ __forceinline__ int row_len(const Params& p, int r) {
  int len;
  if (p.counts) {
    len = p.counts[r];
  } else {
    const int t = p.q_pos[r];
    len = t >= 0 ? t / p.m : 0;
    const int cap = p.id_base ? p.N - min(max(p.id_base[r], 0), p.N) : p.N;
    if (len > cap) len = cap;
  }
  if (p.len_div > 1) len = (len + p.len_div - 1) / p.len_div;
  if (len > p.max_len) len = p.max_len;
  return len < 0 ? 0 : len;
}

__device__ __forceinline__ int32_t map_id(const Params& p, int r, int slot) {
  if (p.idx_map) return p.idx_map[(size_t)r * p.idx_map_stride + slot];
  return p.id_base ? slot + min(max(p.id_base[r], 0), p.N) : slot;
}

// Keys of a row or chunk staged once into LDS (vector loads); all passes then run from
// LDS.  Up to kStageMax keys are staged; longer rows are read from global memory.
constexpr int kStageMax = 32768;
// Rows of up to kRegSingle keys are selected from registers (16 rows of 4 keys per thread
// at 256 threads); the LDS then holds only the selection state.
constexpr int kRegSingle = 16384;
constexpr int kRegThreads = 512;  // workgroup size of register rows when there are many rows

template <int kT>
__device__ __forceinline__ void stage_keys(const float* scores, int n, int force, uint32_t* keys) {
  const bool vec = (((uintptr_t)scores) & 15u) == 0;
  const int n4 = vec ? n / 4 : 0;
  for (int i = threadIdx.x; i < n4; i += kT) {
    const float4 v = reinterpret_cast<const float4*>(scores)[i];
    keys[4 * i] = float_key(v.x); keys[4 * i + 1] = float_key(v.y);
    keys[4 * i + 2] = float_key(v.z); keys[4 * i + 3] = float_key(v.w);
  }
  for (int i = 4 * n4 + threadIdx.x; i < n; i += kT) keys[i] = float_key(scores[i]);
  __syncthreads();
  if (force >= 0 && threadIdx.x == 0) keys[force] = 0xffffffffu;
  __syncthreads();
}

// Selected positions are first collected in LDS (sel[pos] = i) and mapped / written after
// one barrier, so the id map (Reindex) is read with all loads in flight at once.  Used
// when k <= kDeferMax and the LDS has room; otherwise each selection is written directly.
constexpr int kDeferMax = 4096;

__host__ __device__ __forceinline__ size_t smem_keys_off(size_t smem_bytes) { return (smem_bytes + 15) & ~(size_t)15; }

// single level: one workgroup per row
template <int kT>
// 512-thread rows: at most 80 VGPRs, so that three workgroups share a CU
__global__ void __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(kT == 512 ? 6 : 1)))
topk_single(Params p, int stage_cap, int defer) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  TopkSmem<kT>& sm = *reinterpret_cast<TopkSmem<kT>*>(smem_raw);
  uint32_t* skeys = reinterpret_cast<uint32_t*>(smem_raw + smem_keys_off(sizeof(TopkSmem<kT>)));
  int32_t* sel = reinterpret_cast<int32_t*>(skeys + ((stage_cap + 3) & ~3));
  // the last rows first: in a causal prefill they are the longest, so the short ones fill
  // the tail of the launch
  const int r = (int)gridDim.x - 1 - (int)blockIdx.x;
  const int n = row_len(p, r);
  int32_t* out = p.out_idx + (size_t)r * p.k;
  if (n <= p.k) {
    for (int i = threadIdx.x; i < p.k; i += kT) out[i] = i < n ? map_id(p, r, i) : -1;
    return;
  }
  const float* row = p.scores + (size_t)r * p.row_stride;
  const int force = p.force_last ? n - 1 : -1;
  uint32_t T, take;
  auto direct = [=](uint32_t pos, int i, uint32_t) { out[pos] = map_id(p, r, i); };
  if (n <= kRegSingle) {
    // the row's keys go straight from its scores into registers; LDS holds only the
    // histograms, so several rows' workgroups share a CU
    constexpr int kJ = kRegSingle / (4 * kT);
    KeyRegs<kT, kJ> kr;
    key_regs_load_scores(kr, row, n, force);
    radix_threshold<kT>(kr, n, p.k, sm, &T, &take);
    if (T != 0u && p.k <= 2 * kTopkBins) {
      // selected positions staged in the histogram space, then mapped and stored coalesced
      int32_t* ssel = reinterpret_cast<int32_t*>(&sm.hist[0][0]);
      ordered_compact_regs(kr, p.k, T, take, sm, [=](uint32_t pos, int i, uint32_t) { ssel[pos] = i; });
      lds_barrier();
      for (int q = threadIdx.x; q < p.k; q += kT) out[q] = map_id(p, r, ssel[q]);
    } else if (T != 0u) {
      ordered_compact_regs(kr, p.k, T, take, sm, direct);
    } else {  // slots past n could tie with T = 0: compact from the scores, which stop at n
      ordered_compact<kT>(KeysScores{row, force}, n, p.k, T, take, sm, direct);
    }
    return;
  }
  auto deferred = [&](uint32_t pos, int i, uint32_t) { sel[pos] = i; };
  if (n <= stage_cap) {
    stage_keys<kT>(row, n, force, skeys);
    const KeysLds src{skeys};
    radix_threshold<kT>(src, n, p.k, sm, &T, &take);
    if (defer) ordered_compact<kT>(src, n, p.k, T, take, sm, deferred);
    else ordered_compact<kT>(src, n, p.k, T, take, sm, direct);
  } else {
    const KeysScores src{row, force};
    radix_threshold<kT>(src, n, p.k, sm, &T, &take);
    if (defer) ordered_compact<kT>(src, n, p.k, T, take, sm, deferred);
    else ordered_compact<kT>(src, n, p.k, T, take, sm, direct);
  }
  if (defer) {
    __syncthreads();
    for (int q = threadIdx.x; q < p.k; q += kT) out[q] = map_id(p, r, sel[q]);
  }
}

// two-level, first level: grid (rows, nchunks); chunk c of row r -> ws[r][c*k .. c*k+k)
template <int kT>
__global__ void __launch_bounds__(kT) topk_chunk(Params p, int stage_cap) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  TopkSmem<kT>& sm = *reinterpret_cast<TopkSmem<kT>*>(smem_raw);
  uint32_t* skeys = reinterpret_cast<uint32_t*>(smem_raw + smem_keys_off(sizeof(TopkSmem<kT>)));
  const int r = blockIdx.x, c = blockIdx.y;
  const int n = row_len(p, r);
  const int c0 = c * p.chunk;
  const int len = max(0, min(p.chunk, n - c0));
  uint32_t* ok = p.ws_keys + ((size_t)r * p.nchunks + c) * p.k;
  int32_t* os = p.ws_slot + ((size_t)r * p.nchunks + c) * p.k;
  uint2* ob = p.ws_bound + (size_t)r * p.nchunks + c;
  const int force = (p.force_last && n > 0 && n - 1 >= c0 && n - 1 < c0 + p.chunk) ? (n - 1 - c0) : -1;
  const float* row = p.scores + (size_t)r * p.row_stride + c0;
  if (len <= p.k) {
    const KeysScores src{row, force};
    for (int i = threadIdx.x; i < p.k; i += kT) {
      ok[i] = i < len ? src.key(i) : 0u;
      os[i] = i < len ? c0 + i : -1;
    }
    if (threadIdx.x == 0) *ob = make_uint2(0u, (uint32_t)len);  // every key >= 0
    return;
  }
  uint32_t T, take, L2, g2;
  const int k2 = bound_rank(p.k, p.nchunks);
  auto emit = [&](uint32_t pos, int i, uint32_t key) {
    ok[pos] = key;
    os[pos] = c0 + i;
  };
  if (len <= stage_cap) {
    stage_keys<kT>(row, len, force, skeys);
    const KeysLds src{skeys};
    radix_threshold<kT>(src, len, p.k, sm, &T, &take, k2, &L2, &g2);
    if (threadIdx.x == 0) *ob = make_uint2(L2, g2);
    ordered_compact<kT>(src, len, p.k, T, take, sm, emit);
  } else {
    const KeysScores src{row, force};
    radix_threshold<kT>(src, len, p.k, sm, &T, &take, k2, &L2, &g2);
    if (threadIdx.x == 0) *ob = make_uint2(L2, g2);
    ordered_compact<kT>(src, len, p.k, T, take, sm, emit);
  }
}

// two-level, second level: one workgroup per row over nchunks*k (key, slot) pairs; key 0
// marks padding (below every real key).
//
// Pruned form (rows of at most kPruneMax pairs, chunk bounds present): the chunk bounds
// give a key L with at least k candidates >= L, so L <= the row's k-th largest key and
// every key below L can be dropped.  The survivors are gathered in index order into LDS,
// and the selection runs over them alone.
constexpr int kPruneMax = 16384;

__global__ void __launch_bounds__(kMergeThreads) topk_merge(Params p, int stage_cap, int defer, int prune) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  TopkSmem<kMergeThreads>& sm = *reinterpret_cast<TopkSmem<kMergeThreads>*>(smem_raw);
  uint32_t* skeys = reinterpret_cast<uint32_t*>(smem_raw + smem_keys_off(sizeof(TopkSmem<kMergeThreads>)));
  const int cap4 = (stage_cap + 3) & ~3;
  int32_t* sidx = reinterpret_cast<int32_t*>(skeys + cap4);  // pruned form: survivor -> its slot
  int32_t* sel = prune ? sidx + cap4 : reinterpret_cast<int32_t*>(skeys + cap4);
  const int r = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = row_len(p, r);
  int32_t* out = p.out_idx + (size_t)r * p.k;
  const int32_t* slots = p.ws_slot + (size_t)r * p.nchunks * p.k;
  if (n <= p.k) {
    for (int i = threadIdx.x; i < p.k; i += kMergeThreads) out[i] = i < n ? map_id(p, r, i) : -1;
    return;
  }
  const int m = p.nchunks * p.k;
  const uint32_t* gkeys = p.ws_keys + (size_t)r * m;
  uint32_t T, take;
  if (prune) {
    // this thread's pairs [16t, 16t + 16): loads issued first, in flight during the bound
    constexpr int kPer = kPruneMax / kMergeThreads;
    const int i0 = kPer * threadIdx.x;
    uint32_t kk[kPer];
    int32_t ks[kPer];  // their slots
    if ((m & 3) == 0) {
#pragma unroll
      for (int q = 0; q < kPer / 4; ++q) {
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        int4 w = make_int4(-1, -1, -1, -1);
        if (i0 + 4 * q < m) {
          v = reinterpret_cast<const uint4*>(gkeys + i0)[q];
          w = reinterpret_cast<const int4*>(slots + i0)[q];
        }
        kk[4 * q] = v.x; kk[4 * q + 1] = v.y; kk[4 * q + 2] = v.z; kk[4 * q + 3] = v.w;
        ks[4 * q] = w.x; ks[4 * q + 1] = w.y; ks[4 * q + 2] = w.z; ks[4 * q + 3] = w.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        kk[j] = i0 + j < m ? gkeys[i0 + j] : 0u;
        ks[j] = i0 + j < m ? slots[i0 + j] : -1;
      }
    }
    // L: the largest chunk bound such that the chunks with bounds >= it hold >= k keys at
    // or above it.  The bounds are staged in LDS (the survivor arrays are free until the
    // survivors are written, after a barrier below).
    uint2* sb = reinterpret_cast<uint2*>(skeys);  // nchunks <= m <= the two arrays' 2*cap4 words / 2
    const uint2* bd = p.ws_bound + (size_t)r * p.nchunks;
    for (int c = threadIdx.x; c < p.nchunks; c += kMergeThreads) sb[c] = bd[c];
    __syncthreads();
    uint32_t best = 0;
    for (int c = threadIdx.x; c < p.nchunks; c += kMergeThreads) {
      const uint32_t lc = sb[c].x;
      uint32_t held = 0;
      for (int j = 0; j < p.nchunks; ++j) {
        const uint2 b = sb[j];
        if (b.x >= lc) held += b.y;
      }
      if (held >= (uint32_t)p.k) best = max(best, lc);
    }
    best = wave_umax(best);
    if (lane == 0) sm.whi[wave] = best;
    __syncthreads();
    uint32_t L = 0;
#pragma unroll
    for (int w = 0; w < TopkSmem<kMergeThreads>::kW; ++w) L = max(L, sm.whi[w]);
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) cnt += (i0 + j < m && kk[j] >= L) ? 1u : 0u;
    uint32_t ns;
    uint32_t pos = block_excl_scan<kMergeThreads>(cnt, &ns, sm);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (i0 + j < m && kk[j] >= L) {
        skeys[pos] = kk[j];
        sidx[pos] = ks[j];
        ++pos;
      }
    }
    __syncthreads();
    const KeysLds src{skeys};
    radix_threshold<kMergeThreads>(src, (int)ns, p.k, sm, &T, &take);
    ordered_compact<kMergeThreads>(src, (int)ns, p.k, T, take, sm,
                                   [&](uint32_t q, int j, uint32_t) { sel[q] = sidx[j]; });
    __syncthreads();
    for (int q = threadIdx.x; q < p.k; q += kMergeThreads) {
      const int sl = sel[q];
      out[q] = sl >= 0 ? map_id(p, r, sl) : -1;
    }
    return;
  }
  auto direct = [&](uint32_t pos, int i, uint32_t) {
    const int sl = slots[i];
    out[pos] = sl >= 0 ? map_id(p, r, sl) : -1;
  };
  auto deferred = [&](uint32_t pos, int i, uint32_t) { sel[pos] = i; };
  if (m <= stage_cap) {
    if ((m & 3) == 0) {
      for (int i = threadIdx.x; i < m / 4; i += kMergeThreads)
        reinterpret_cast<uint4*>(skeys)[i] = reinterpret_cast<const uint4*>(gkeys)[i];
    } else {
      for (int i = threadIdx.x; i < m; i += kMergeThreads) skeys[i] = gkeys[i];
    }
    __syncthreads();
    const KeysLds src{skeys};
    radix_threshold<kMergeThreads>(src, m, p.k, sm, &T, &take);
    if (defer) ordered_compact<kMergeThreads>(src, m, p.k, T, take, sm, deferred);
    else ordered_compact<kMergeThreads>(src, m, p.k, T, take, sm, direct);
  } else {
    const KeysGlobal src{gkeys};
    radix_threshold<kMergeThreads>(src, m, p.k, sm, &T, &take);
    if (defer) ordered_compact<kMergeThreads>(src, m, p.k, T, take, sm, deferred);
    else ordered_compact<kMergeThreads>(src, m, p.k, T, take, sm, direct);
  }
  if (defer) {
    __syncthreads();
    for (int q = threadIdx.x; q < p.k; q += kMergeThreads) {
      const int sl = slots[sel[q]];
      out[q] = sl >= 0 ? map_id(p, r, sl) : -1;
    }
  }
}

// LDS of a merge launch and whether it takes the pruned form
static size_t merge_lds(int m, int k, bool have_bounds, int* cap_out, int* defer_out, int* prune_out) {
  const size_t base = smem_keys_off(sizeof(TopkSmem<kMergeThreads>));
  const int cap = m < kStageMax ? m : kStageMax;
  const size_t cap4 = (size_t)((cap + 3) & ~3);
  const bool prune = have_bounds && m <= kPruneMax && base + 2 * cap4 * 4 + (size_t)k * 4 <= kLdsMax;
  size_t lds;
  int defer = 0;
  if (prune) {
    lds = base + 2 * cap4 * 4 + (size_t)k * 4;
  } else {
    lds = base + cap4 * 4;
    defer = k <= kDeferMax && lds + (size_t)k * 4 <= kLdsMax;
    if (defer) lds += (size_t)k * 4;
  }
  *cap_out = cap;
  *defer_out = defer;
  *prune_out = prune;
  return lds;
}

// expand selected blocks (ascending, -1 padded, the latest visible block included) into
// positions; grid (rows, ceil(n_keep*block / 256)), one position per thread
__global__ void __launch_bounds__(kThreads) hier_expand(int n_keep, int block, const int32_t* __restrict__ sel,
                                                         const int32_t* __restrict__ q_pos, int N, int m,
                                                         int32_t* __restrict__ cand, int32_t* __restrict__ count) {
  const int r = blockIdx.x;
  const int t = q_pos[r];
  int nv = t >= 0 ? t / m : 0;
  if (nv > N) nv = N;
  const int total = n_keep * block;
  const int q = blockIdx.y * kThreads + threadIdx.x;
  if (q < total) {
    const int blk = sel[(size_t)r * n_keep + q / block];
    const int pos = blk >= 0 ? blk * block + q % block : -1;
    // only the latest (highest, last-listed) block can be partial; its tail maps to -1 and
    // sits at the end of the list, so the valid positions stay contiguous and ascending
    cand[(size_t)r * total + q] = (pos >= 0 && pos < nv) ? pos : -1;
  }
  if (blockIdx.y == 0 && threadIdx.x == 0) {
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
  return (size_t)rows * nchunks * k * (sizeof(uint32_t) + sizeof(int32_t)) + (size_t)rows * nchunks * sizeof(uint2);
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
  p.out_idx = a.out_idx; p.id_base = a.id_base;
  p.max_len = a.max_len;
  hipError_t e;
  if (a.max_len <= kSingleMax) {
    // rows that fit the registers need no staged keys (and stage their selection in the
    // histogram space)
    const bool regs = a.max_len <= kRegSingle;
    const int cap = regs ? 0 : (a.max_len < kStageMax ? a.max_len : kStageMax);
    const bool wide = a.rows < kWideBelow;
    size_t lds = smem_keys_off(wide ? sizeof(TopkSmem<kMergeThreads>) : sizeof(TopkSmem<kThreads>)) + (size_t)((cap + 3) & ~3) * 4;
    const int defer = !regs && a.k <= kDeferMax && lds + (size_t)a.k * 4 <= kLdsMax;
    if (defer) lds += (size_t)a.k * 4;
    ScopedProf pr(s, "topk_single");
    if (regs && !wide) {  // many register rows: 512 threads, half the keys per thread
      hipLaunchKernelGGL(topk_single<kRegThreads>, dim3(a.rows), dim3(kRegThreads),
                         smem_keys_off(sizeof(TopkSmem<kRegThreads>)), s, p, 0, 0);
    } else if (wide) {
      if ((e = set_lds((const void*)topk_single<kMergeThreads>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(topk_single<kMergeThreads>, dim3(a.rows), dim3(kMergeThreads), lds, s, p, cap, defer);
    } else {
      if ((e = set_lds((const void*)topk_single<kThreads>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(topk_single<kThreads>, dim3(a.rows), dim3(kThreads), lds, s, p, cap, defer);
    }
    return hipGetLastError();
  }
  p.chunk = pick_chunk(a.max_len, a.k);
  p.nchunks = (a.max_len + p.chunk - 1) / p.chunk;
  p.ws_keys = (uint32_t*)a.ws;
  p.ws_slot = (int32_t*)((char*)a.ws + (size_t)a.rows * p.nchunks * a.k * sizeof(uint32_t));
  p.ws_bound = (uint2*)((char*)p.ws_slot + (size_t)a.rows * p.nchunks * a.k * sizeof(int32_t));
  {
    const int cap = p.chunk < kStageMax ? p.chunk : kStageMax;
    const bool wide = (long long)a.rows * p.nchunks < kWideBelow;
    const size_t lds =
        smem_keys_off(wide ? sizeof(TopkSmem<kMergeThreads>) : sizeof(TopkSmem<kThreads>)) + (size_t)((cap + 3) & ~3) * 4;
    ScopedProf pr(s, "topk_chunk");
    if (wide) {
      if ((e = set_lds((const void*)topk_chunk<kMergeThreads>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(topk_chunk<kMergeThreads>, dim3(a.rows, p.nchunks), dim3(kMergeThreads), lds, s, p, cap);
    } else {
      if ((e = set_lds((const void*)topk_chunk<kThreads>, lds)) != hipSuccess) return e;
      hipLaunchKernelGGL(topk_chunk<kThreads>, dim3(a.rows, p.nchunks), dim3(kThreads), lds, s, p, cap);
    }
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    int cap, defer, prune;
    const size_t lds = merge_lds(p.nchunks * a.k, a.k, true, &cap, &defer, &prune);
    if ((e = set_lds((const void*)topk_merge, lds)) != hipSuccess) return e;
    ScopedProf pr(s, "topk_merge");
    hipLaunchKernelGGL(topk_merge, dim3(a.rows), dim3(kMergeThreads), lds, s, p, cap, defer, prune);
  }
  return hipGetLastError();
}

hipError_t launch_topk_merge(const TopkArgs& a, int nchunks, uint32_t* keys, int32_t* slots, uint2* bounds,
                             hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (!a.out_idx || !keys || !slots || (!a.counts && !a.q_pos)) return hipErrorInvalidValue;
  Params p{};
  p.rows = a.rows; p.k = a.k; p.counts = a.counts; p.q_pos = a.q_pos; p.N = a.N; p.m = a.m;
  p.len_div = a.len_div; p.force_last = a.force_last; p.idx_map = a.idx_map;
  p.idx_map_stride = a.idx_map_stride; p.out_idx = a.out_idx; p.max_len = a.max_len; p.id_base = a.id_base;
  p.nchunks = nchunks; p.ws_keys = keys; p.ws_slot = slots; p.ws_bound = bounds;
  int cap, defer, prune;
  const size_t lds = merge_lds(nchunks * a.k, a.k, bounds != nullptr, &cap, &defer, &prune);
  hipError_t e = set_lds((const void*)topk_merge, lds);
  if (e != hipSuccess) return e;
  ScopedProf pr(s, "topk_merge");
  hipLaunchKernelGGL(topk_merge, dim3(a.rows), dim3(kMergeThreads), lds, s, p, cap, defer, prune);
  return hipGetLastError();
}

hipError_t launch_hier_expand(int rows, int n_keep, int block, const int32_t* sel_blocks,
                              const int32_t* q_pos, int N, int m, int32_t* out_cand,
                              int32_t* out_count, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (!sel_blocks || !q_pos || !out_cand || !out_count) return hipErrorInvalidValue;
  ScopedProf pr(s, "hier_expand");
  const int total = n_keep * block;
  hipLaunchKernelGGL(hier_expand, dim3(rows, (total + kThreads - 1) / kThreads), dim3(kThreads), 0, s, n_keep,
                     block, sel_blocks, q_pos, N, m, out_cand, out_count);
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
