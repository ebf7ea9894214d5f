// Internal interface between the host API (api.cpp) and the kernel launchers (*.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <string>

#include "../../include/csa2.h"

namespace csa2 {

// kernel timing hooks (no-ops unless csa2_profile_enable(1) on this thread)
void prof_begin(hipStream_t s, const char* name);
void prof_end(hipStream_t s);

struct ScopedProf {
  hipStream_t s;
  ScopedProf(hipStream_t st, const char* name) : s(st) { prof_begin(st, name); }
  ~ScopedProf() { prof_end(s); }
};

// ---- grouped output projection (proj.hip)
hipError_t launch_out_proj(const csa2_out_proj_desc& d, hipStream_t s);
// ---- compressor (compress.hip)
hipError_t launch_compress(const csa2_compress_desc& d, hipStream_t s);

// ---- indexer scan (index.hip)
struct ScanArgs {
  int B, T, H_I, d_I, N, m, block;
  const void* q_idx;
  const float* w;
  const int32_t* q_pos;
  csa2_dtype k_dtype;
  const void* k_idx;
  const uint8_t *k_codes, *k_scales;
  const int32_t *cand, *n_cand;  // REINDEX: score slots of cand instead of entries 0..n_vis-1
  int cand_stride;
  float* scores;          // [B*T, row_stride]
  int64_t row_stride;
  float* block_max;       // [B*T, nblk] or null (FULL only)
  int nblk;
  const int32_t* ent_base;  // [B*T] or null: a query's entries start at this id (packed samples)
  const uint8_t* q_scales;  // non-null: q_I in MXFP4 (q_idx holds the codes), with an MXFP4 K_I
};
hipError_t launch_index_scan(const ScanArgs& a, hipStream_t s);

// ---- top-k selection (topk.hip)
// Rows of fp32 scores; row r has length len(r) given either by the causal rule
// (q_pos, m, N) or by counts[r]; idx_map (optional) maps a slot to the reported id.
struct TopkArgs {
  int rows, k;
  const float* scores;
  int64_t row_stride;
  // row length: if counts != null, len = counts[r]; else len = min(N, floor(q_pos[r]/m))
  // (with `len_div` > 1 meaning ceil(len / len_div), used for block rows)
  const int32_t* counts;
  const int32_t* q_pos;
  int N, m, len_div;
  int force_last;          // 1: the row's last slot always wins (hierarchical pool)
  const int32_t* idx_map;  // [rows, idx_map_stride] or null
  int64_t idx_map_stride;
  int32_t* out_idx;        // [rows, k]
  int max_len;             // upper bound of len over rows (sizes the launch)
  void* ws;                // workspace for the two-level path
  size_t ws_bytes;
  const int32_t* id_base;  // [rows] or null: reported id = slot + id_base[row] (packed samples;
                           // the row length is also clamped to N - id_base[row])
};
size_t topk_workspace_bytes(int rows, int k, int max_len);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);

// second level only: rows of nchunks*k (key, slot) pairs already written by a first level,
// with one (bound, count) pair per chunk: `count` keys of the chunk are >= `bound`
hipError_t launch_topk_merge(const TopkArgs& a, int nchunks, uint32_t* keys, int32_t* slots, uint2* bounds,
                             hipStream_t s);

// fused decode scan + chunk-local top-k (FULL mode, one query per sequence): the scan
// writes (key, slot) pairs of each chunk's top-k; topk_merge finishes.  Returns the chunk
// size used through *chunk_out and the number of chunks through *nchunks_out.
int scan_select_chunk(int rows, int N, int k);
// Longest chunk the fused scan + chunk top-k handles: its keys (4 bytes each) and the
// selection state share one workgroup's 160 KiB of LDS.
constexpr int kMaxSelectChunk = 32768;
hipError_t launch_index_scan_select(const ScanArgs& a, int k, int chunk, int nchunks, uint32_t* keys,
                                    int32_t* slots, uint2* bounds, hipStream_t s);

// expand selected blocks (ascending, -1 padded) into candidate positions
hipError_t launch_hier_expand(int rows, int n_keep, int block, const int32_t* sel_blocks,
                              const int32_t* q_pos, int N, int m, int32_t* out_cand,
                              int32_t* out_count, hipStream_t s);

hipError_t launch_copy_idx(const int32_t* src, int32_t* dst, size_t n, hipStream_t s);

// ---- sparse attention (attn.hip)
size_t attn_workspace_bytes(const csa2_attn_desc& d);
hipError_t launch_attn(const csa2_attn_desc& d, void* ws, size_t ws_bytes, hipStream_t s);

}  // namespace csa2
