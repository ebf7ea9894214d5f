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
#include "topk_core.h"

namespace csa2 {
namespace {

constexpr int kThreads = 256;       // single rows and chunks
constexpr int kMergeThreads = 1024; // merge rows (few workgroups, long rows)
constexpr int kSingleMax = 32768;

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

// single level: one workgroup per row
__global__ void __launch_bounds__(kThreads) topk_single(Params p, int stage_cap) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  TopkSmem<kThreads>& sm = *reinterpret_cast<TopkSmem<kThreads>*>(smem_raw);
  uint32_t* skeys = reinterpret_cast<uint32_t*>(smem_raw + ((sizeof(TopkSmem<kThreads>) + 15) & ~(size_t)15));
  const int r = blockIdx.x;
  const int n = row_len(p, r);
  int32_t* out = p.out_idx + (size_t)r * p.k;
  if (n <= p.k) {
    for (int i = threadIdx.x; i < p.k; i += kThreads) out[i] = i < n ? map_id(p, r, i) : -1;
    return;
  }
  const float* row = p.scores + (size_t)r * p.row_stride;
  const int force = p.force_last ? n - 1 : -1;
  uint32_t T, take;
  auto emit = [&](uint32_t pos, int i, uint32_t) { out[pos] = map_id(p, r, i); };
  if (n <= stage_cap) {
    stage_keys<kThreads>(row, n, force, skeys);
    const KeysLds src{skeys};
    radix_threshold<kThreads>(src, n, p.k, sm, &T, &take);
    ordered_compact<kThreads>(src, n, p.k, T, take, sm, emit);
  } else {
    const KeysScores src{row, force};
    radix_threshold<kThreads>(src, n, p.k, sm, &T, &take);
    ordered_compact<kThreads>(src, n, p.k, T, take, sm, emit);
  }
}

// two-level, first level: grid (rows, nchunks); chunk c of row r -> ws[r][c*k .. c*k+k)
__global__ void __launch_bounds__(kThreads) topk_chunk(Params p, int stage_cap) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  TopkSmem<kThreads>& sm = *reinterpret_cast<TopkSmem<kThreads>*>(smem_raw);
  uint32_t* skeys = reinterpret_cast<uint32_t*>(smem_raw + ((sizeof(TopkSmem<kThreads>) + 15) & ~(size_t)15));
  const int r = blockIdx.x, c = blockIdx.y;
  const int n = row_len(p, r);
  const int c0 = c * p.chunk;
  const int len = max(0, min(p.chunk, n - c0));
  uint32_t* ok = p.ws_keys + ((size_t)r * p.nchunks + c) * p.k;
  int32_t* os = p.ws_slot + ((size_t)r * p.nchunks + c) * p.k;
  const int force = (p.force_last && n > 0 && n - 1 >= c0 && n - 1 < c0 + p.chunk) ? (n - 1 - c0) : -1;
  const float* row = p.scores + (size_t)r * p.row_stride + c0;
  if (len <= p.k) {
    const KeysScores src{row, force};
    for (int i = threadIdx.x; i < p.k; i += kThreads) {
      ok[i] = i < len ? src.key(i) : 0u;
      os[i] = i < len ? c0 + i : -1;
    }
    return;
  }
  uint32_t T, take;
  auto emit = [&](uint32_t pos, int i, uint32_t key) {
    ok[pos] = key;
    os[pos] = c0 + i;
  };
  if (len <= stage_cap) {
    stage_keys<kThreads>(row, len, force, skeys);
    const KeysLds src{skeys};
    radix_threshold<kThreads>(src, len, p.k, sm, &T, &take);
    ordered_compact<kThreads>(src, len, p.k, T, take, sm, emit);
  } else {
    const KeysScores src{row, force};
    radix_threshold<kThreads>(src, len, p.k, sm, &T, &take);
    ordered_compact<kThreads>(src, len, p.k, T, take, sm, emit);
  }
}

// two-level, second level: one workgroup per row over nchunks*k (key, slot) pairs; key 0
// marks padding (below every real key)
__global__ void __launch_bounds__(kMergeThreads) topk_merge(Params p, int stage_cap) {
  extern __shared__ __align__(16) uint8_t smem_raw[];
  TopkSmem<kMergeThreads>& sm = *reinterpret_cast<TopkSmem<kMergeThreads>*>(smem_raw);
  uint32_t* skeys = reinterpret_cast<uint32_t*>(smem_raw + ((sizeof(TopkSmem<kMergeThreads>) + 15) & ~(size_t)15));
  const int r = blockIdx.x;
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
  auto emit = [&](uint32_t pos, int i, uint32_t) {
    const int sl = slots[i];
    out[pos] = sl >= 0 ? map_id(p, r, sl) : -1;
  };
  if (m <= stage_cap) {
    if ((m & 3) == 0 && (((uintptr_t)gkeys) & 15u) == 0) {
      for (int i = threadIdx.x; i < m / 4; i += kMergeThreads)
        reinterpret_cast<uint4*>(skeys)[i] = reinterpret_cast<const uint4*>(gkeys)[i];
    } else {
      for (int i = threadIdx.x; i < m; i += kMergeThreads) skeys[i] = gkeys[i];
    }
    __syncthreads();
    const KeysLds src{skeys};
    radix_threshold<kMergeThreads>(src, m, p.k, sm, &T, &take);
    ordered_compact<kMergeThreads>(src, m, p.k, T, take, sm, emit);
  } else {
    const KeysLds src{gkeys};
    radix_threshold<kMergeThreads>(src, m, p.k, sm, &T, &take);
    ordered_compact<kMergeThreads>(src, m, p.k, T, take, sm, emit);
  }
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
    const size_t lds = ((sizeof(TopkSmem<kThreads>) + 15) & ~(size_t)15) + (size_t)cap * 4;
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
    const size_t lds = ((sizeof(TopkSmem<kThreads>) + 15) & ~(size_t)15) + (size_t)cap * 4;
    if ((e = set_lds((const void*)topk_chunk, lds)) != hipSuccess) return e;
    ScopedProf pr(s, "topk_chunk");
    hipLaunchKernelGGL(topk_chunk, dim3(a.rows, p.nchunks), dim3(kThreads), lds, s, p, cap);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    const int m = p.nchunks * a.k;
    const int cap = m < kStageMax ? m : kStageMax;
    const size_t lds = ((sizeof(TopkSmem<kMergeThreads>) + 15) & ~(size_t)15) + (size_t)cap * 4;
    if ((e = set_lds((const void*)topk_merge, lds)) != hipSuccess) return e;
    ScopedProf pr(s, "topk_merge");
    hipLaunchKernelGGL(topk_merge, dim3(a.rows), dim3(kMergeThreads), lds, s, p, cap);
  }
  return hipGetLastError();
}

hipError_t launch_topk_merge(const TopkArgs& a, int nchunks, uint32_t* keys, int32_t* slots, hipStream_t s) {
  if (a.rows == 0) return hipSuccess;
  if (!a.out_idx || !keys || !slots || (!a.counts && !a.q_pos)) return hipErrorInvalidValue;
  Params p{};
  p.rows = a.rows; p.k = a.k; p.counts = a.counts; p.q_pos = a.q_pos; p.N = a.N; p.m = a.m;
  p.len_div = a.len_div; p.force_last = a.force_last; p.idx_map = a.idx_map;
  p.idx_map_stride = a.idx_map_stride; p.out_idx = a.out_idx; p.max_len = a.max_len;
  p.nchunks = nchunks; p.ws_keys = keys; p.ws_slot = slots;
  const int m = nchunks * a.k;
  const int cap = m < kStageMax ? m : kStageMax;
  const size_t lds = ((sizeof(TopkSmem<kMergeThreads>) + 15) & ~(size_t)15) + (size_t)cap * 4;
  hipError_t e = set_lds((const void*)topk_merge, lds);
  if (e != hipSuccess) return e;
  ScopedProf pr(s, "topk_merge");
  hipLaunchKernelGGL(topk_merge, dim3(a.rows), dim3(kMergeThreads), lds, s, p, cap);
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
