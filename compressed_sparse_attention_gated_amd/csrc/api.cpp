// Host side of the libcsa2 C ABI: argument validation (all of it before any launch),
// workspace sizing, mode dispatch, the thread-local last-error string and the optional
// per-kernel event timing.

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/csa2.h"
#include "internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}
int ok() {
  g_err.clear();
  return CSA2_OK;
}
int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(CSA2_ERR_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool pow2_upto(int v, int hi) { return v >= 1 && v <= hi && (v & (v - 1)) == 0; }
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// --------------------------------------------------------------- kernel timing
struct ProfRec {
  std::string name;
  hipEvent_t a, b;
  hipStream_t s;
};
thread_local bool g_prof_on = false;
thread_local std::vector<ProfRec> g_prof;
thread_local std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace csa2 {
void prof_begin(hipStream_t s, const char* name) {
  if (!g_prof_on) return;
  ProfRec r{name, take_event(), take_event(), s};
  if (r.a) (void)hipEventRecord(r.a, s);
  g_prof.push_back(r);
}
void prof_end(hipStream_t s) {
  if (!g_prof_on || g_prof.empty()) return;
  ProfRec& r = g_prof.back();
  if (r.b) (void)hipEventRecord(r.b, s);
}
}  // namespace csa2

using namespace csa2;

// The integer a caller stored in an enum-typed field or argument.  Reading such an object
// as its enum type is undefined when the value is none of the enumerators, so every check
// reads the raw integer first and rejects unknown values before the field is used.
template <class E>
static int raw(const E& f) {
  static_assert(sizeof(E) == sizeof(int), "the C enums of the ABI are int-sized");
  int v;
  std::memcpy(&v, &f, sizeof v);
  return v;
}

extern "C" {

int csa2_version(void) { return CSA2_VERSION; }
const char* csa2_last_error(void) { return g_err.c_str(); }

int csa2_profile_enable(int on) {
  g_prof_on = on != 0;
  return CSA2_OK;
}

int csa2_profile_collect(csa2_kernel_time* out, int max) {
  int n = 0;
  int rc = CSA2_OK;
  for (ProfRec& r : g_prof) {
    float ms = -1.f;
    if (r.a && r.b && hipEventSynchronize(r.b) == hipSuccess) {
      if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) ms = -1.f;
    } else {
      rc = CSA2_ERR_HIP;
    }
    if (out && n < max) {
      std::memset(out[n].name, 0, sizeof out[n].name);
      std::strncpy(out[n].name, r.name.c_str(), sizeof out[n].name - 1);
      out[n].ms = ms;
      ++n;
    }
    if (r.a) g_event_pool.push_back(r.a);
    if (r.b) g_event_pool.push_back(r.b);
  }
  g_prof.clear();
  if (rc != CSA2_OK) return fail(rc, "profile: an event could not be synchronised");
  ok();
  return n;
}

// --------------------------------------------------------------- compress
static int check_compress(const csa2_compress_desc* d) {
  if (!d) return fail(CSA2_ERR_INVALID, "compress: null descriptor");
  if (d->B < 0 || d->n < 0 || d->m < 1) return fail(CSA2_ERR_INVALID, "compress: need B >= 0, n >= 0, m >= 1");
  if (d->c < 8 || d->c > 512 || d->c % 8 != 0 || !pow2_upto(d->c / 8, 64))
    return fail(CSA2_ERR_UNSUPPORTED, "compress: c=%d unsupported (c/8 must be a power of two, 8 <= c <= 512)", d->c);
  if (raw(d->dtype) != CSA2_F32 && raw(d->dtype) != CSA2_BF16)
    return fail(CSA2_ERR_UNSUPPORTED, "compress: dtype must be F32 or BF16");
  if (d->overlap != 0 && d->overlap != 1) return fail(CSA2_ERR_INVALID, "compress: overlap must be 0 or 1");
  if (d->rope_dims < 0 || d->rope_dims > d->c || d->rope_dims % 2)
    return fail(CSA2_ERR_INVALID, "compress: rope_dims must be even and in [0, c]");
  if (d->rope_dims > 0 && !(d->rope_theta > 0.f)) return fail(CSA2_ERR_INVALID, "compress: rope_theta must be > 0");
  if (d->norm && !(d->eps >= 0.f)) return fail(CSA2_ERR_INVALID, "compress: eps must be >= 0");
  const long long n_ent = (long long)d->B * (d->n / d->m);
  if (n_ent == 0 && !(d->cu_seqlens && d->out_cu_entries)) return CSA2_OK;
  if (!d->ca || !d->za) return fail(CSA2_ERR_INVALID, "compress: ca and za are required");
  if (!d->out && !d->out_codes) return fail(CSA2_ERR_INVALID, "compress: out or out_codes is required");
  if (!d->out_codes != !d->out_scales)
    return fail(CSA2_ERR_INVALID, "compress: out_codes and out_scales go together");
  if (d->out_codes && d->c % 16 != 0)
    return fail(CSA2_ERR_UNSUPPORTED, "compress: FP4 planes need c %% 16 == 0");
  if (!d->ik_codes != !d->ik_scales) return fail(CSA2_ERR_INVALID, "compress: ik_codes and ik_scales go together");
  if (d->ik_codes && !d->w_ik) return fail(CSA2_ERR_INVALID, "compress: ik_codes need w_ik");
  if (d->q_rows < 0) return fail(CSA2_ERR_INVALID, "compress: q_rows must be >= 0");
  if (d->overlap && (!d->cb || !d->zb)) return fail(CSA2_ERR_INVALID, "compress: overlap needs cb and zb");
  if (!d->cb0 != !d->zb0) return fail(CSA2_ERR_INVALID, "compress: cb0 and zb0 go together");
  if (d->cu_seqlens) {
    if (d->B != 1) return fail(CSA2_ERR_INVALID, "compress: packed samples (cu_seqlens) need B == 1");
    if (d->n_samples < 1 || d->n_samples > CSA2_MAX_PACKED_SAMPLES)
      return fail(CSA2_ERR_INVALID, "compress: n_samples must be in [1, %d]", CSA2_MAX_PACKED_SAMPLES);
    if (d->cb0) return fail(CSA2_ERR_INVALID, "compress: cb0 / zb0 do not combine with cu_seqlens");
  }
  if (d->cb0 && !d->overlap) return fail(CSA2_ERR_INVALID, "compress: cb0 and zb0 need overlap");
  if (d->w_ik) {
    if (!d->out_ik && !d->ik_codes) return fail(CSA2_ERR_INVALID, "compress: w_ik needs out_ik or ik_codes");
    if (d->d_index != 32 && d->d_index != 64 && d->d_index != 128)
      return fail(CSA2_ERR_UNSUPPORTED, "compress: d_index must be 32, 64 or 128");
    if (d->c * d->d_index < 1024)
      return fail(CSA2_ERR_UNSUPPORTED, "compress: the projection needs c * d_index >= 1024");
  }
  const int64_t n_per = d->n / d->m;
  if (d->out_batch_stride != 0 && d->out_batch_stride < d->c)
    return fail(CSA2_ERR_INVALID, "compress: out_batch_stride smaller than one row");
  if (!d->dst_row && d->out_batch_stride != 0 && d->out_batch_stride < n_per * d->c)
    return fail(CSA2_ERR_INVALID, "compress: out_batch_stride smaller than (n/m)*c");
  if (d->w_ik && d->out_ik_batch_stride != 0 && d->out_ik_batch_stride < d->d_index)
    return fail(CSA2_ERR_INVALID, "compress: out_ik_batch_stride smaller than one row");
  if (!d->dst_row && d->w_ik && d->out_ik_batch_stride != 0 && d->out_ik_batch_stride < n_per * d->d_index)
    return fail(CSA2_ERR_INVALID, "compress: out_ik_batch_stride smaller than (n/m)*d_index");
  return CSA2_OK;
}

int csa2_compress(const csa2_compress_desc* d, void* stream) {
  int rc = check_compress(d);
  if (rc != CSA2_OK) return rc;
  if ((long long)d->B * (d->n / d->m) == 0 && !(d->cu_seqlens && d->out_cu_entries)) return ok();
  return hip_status(launch_compress(*d, (hipStream_t)stream), "compress");
}

// --------------------------------------------------------------- index + top-k
// q_dtype 0 (a zeroed field) reads as BF16
static bool q_is_bf16(const csa2_index_desc* d) { return raw(d->q_dtype) == CSA2_BF16 || raw(d->q_dtype) == 0; }

// md: the mode argument as the caller passed it (its raw integer)
static int check_index(const csa2_index_desc* d, int md) {
  if (!d) return fail(CSA2_ERR_INVALID, "index: null descriptor");
  if (md != CSA2_MODE_FULL && md != CSA2_MODE_REINDEX && md != CSA2_MODE_REUSE)
    return fail(CSA2_ERR_INVALID, "index: unknown mode %d", md);
  if (d->B < 0 || d->T < 0) return fail(CSA2_ERR_INVALID, "index: need B, T >= 0");
  if (d->k < 1) return fail(CSA2_ERR_INVALID, "index: k must be >= 1");
  if (d->k > 4096) return fail(CSA2_ERR_UNSUPPORTED, "index: k > 4096");
  const long long rows = (long long)d->B * d->T;
  if (md == CSA2_MODE_REUSE) {
    if (rows && (!d->src_idx || !d->out_idx)) return fail(CSA2_ERR_INVALID, "index: REUSE needs src_idx and out_idx");
    return CSA2_OK;
  }
  if (d->H_I < 1 || d->H_I > 64) return fail(CSA2_ERR_UNSUPPORTED, "index: H_I must be in [1, 64]");
  if (d->d_I != 32 && d->d_I != 64 && d->d_I != 128) return fail(CSA2_ERR_UNSUPPORTED, "index: d_I must be 32, 64 or 128");
  if (d->N < 0 || d->m < 1) return fail(CSA2_ERR_INVALID, "index: need N >= 0, m >= 1");
  if (raw(d->k_dtype) != CSA2_BF16 && raw(d->k_dtype) != CSA2_MXFP4)
    return fail(CSA2_ERR_UNSUPPORTED, "index: K_I dtype must be BF16 or MXFP4");
  if (!q_is_bf16(d) && raw(d->q_dtype) != CSA2_MXFP4)
    return fail(CSA2_ERR_UNSUPPORTED, "index: q_I dtype must be BF16 or MXFP4");
  if (d->q_dtype == CSA2_MXFP4 && d->k_dtype != CSA2_MXFP4)
    return fail(CSA2_ERR_UNSUPPORTED, "index: an MXFP4 q_I needs an MXFP4 K_I");
  if (rows == 0) return CSA2_OK;
  if (!d->q_idx || !d->w || !d->q_pos || !d->out_idx) return fail(CSA2_ERR_INVALID, "index: q_idx, w, q_pos, out_idx are required");
  if (d->q_dtype == CSA2_MXFP4 && !d->q_scales) return fail(CSA2_ERR_INVALID, "index: q_scales required for an MXFP4 q_I");
  if (d->N > 0) {
    if (d->k_dtype == CSA2_BF16 && !d->k_idx) return fail(CSA2_ERR_INVALID, "index: k_idx required for BF16 K_I");
    if (d->k_dtype == CSA2_MXFP4 && (!d->k_codes || !d->k_scales))
      return fail(CSA2_ERR_INVALID, "index: k_codes and k_scales required for MXFP4 K_I");
  }
  if (md == CSA2_MODE_FULL && d->out_block_max && !pow2_upto(d->block, 32))
    return fail(CSA2_ERR_UNSUPPORTED, "index: block must be a power of two <= 32");
  if (d->ent_base && md != CSA2_MODE_FULL)
    return fail(CSA2_ERR_INVALID, "index: ent_base (packed samples) is for FULL mode only");
  if (md == CSA2_MODE_REINDEX) {
    if (!d->cand || !d->n_cand || d->cand_stride < 1) return fail(CSA2_ERR_INVALID, "index: REINDEX needs cand, n_cand, cand_stride >= 1");
    if (d->N == 0) return fail(CSA2_ERR_INVALID, "index: REINDEX with N == 0");
  }
  if ((long long)d->N * 1 > (1LL << 30)) return fail(CSA2_ERR_UNSUPPORTED, "index: N too large");
  return CSA2_OK;
}

// decode-style FULL calls (few queries per sequence, long rows) fuse the chunk-local
// top-k into the scan; the workspace then holds (key, slot) pairs instead of scores
static bool use_fused(const csa2_index_desc* d, csa2_mode mode) {
  return mode == CSA2_MODE_FULL && !d->ent_base && d->T < 8 && d->N > 8192 &&
         scan_select_chunk((int)(d->B * d->T), d->N, d->k) <= kMaxSelectChunk;
}

static size_t index_ws(const csa2_index_desc* d, csa2_mode mode) {
  const size_t rows = (size_t)d->B * d->T;
  if (mode == CSA2_MODE_REUSE || rows == 0) return 0;
  if (use_fused(d, mode)) {
    const int chunk = scan_select_chunk((int)(d->B * d->T), d->N, d->k);
    const size_t nchunks = (size_t)(d->N + chunk - 1) / chunk;
    return align256(rows * nchunks * d->k * sizeof(uint32_t)) + align256(rows * nchunks * d->k * sizeof(int32_t)) +
           align256(rows * nchunks * sizeof(uint2));
  }
  const int len = mode == CSA2_MODE_FULL ? d->N : d->cand_stride;
  size_t bytes = 0;
  if (!d->out_scores) bytes += align256(rows * (size_t)len * sizeof(float));
  bytes += align256(topk_workspace_bytes((int)rows, d->k, len));
  return bytes;
}

size_t csa2_index_workspace_bytes(const csa2_index_desc* d, csa2_mode mode) {
  if (check_index(d, raw(mode)) != CSA2_OK) return 0;
  return index_ws(d, mode);
}

int csa2_index_topk(const csa2_index_desc* d, csa2_mode mode, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_index(d, raw(mode));
  if (rc != CSA2_OK) return rc;
  hipStream_t s = (hipStream_t)stream;
  const long long rows = (long long)d->B * d->T;
  if (rows == 0) return ok();
  if (mode == CSA2_MODE_REUSE) {
    if (d->src_idx == d->out_idx) return ok();
    return hip_status(launch_copy_idx(d->src_idx, d->out_idx, (size_t)rows * d->k, s), "index/reuse");
  }
  const size_t need = index_ws(d, mode);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(CSA2_ERR_WORKSPACE, "index: workspace of %zu bytes required, %zu given", need, ws_bytes);
  if (use_fused(d, mode)) {
    const int chunk = scan_select_chunk((int)(d->B * d->T), d->N, d->k);
    const int nchunks = (d->N + chunk - 1) / chunk;
    uint32_t* keys = (uint32_t*)ws;
    int32_t* slots = (int32_t*)((char*)ws + align256((size_t)rows * nchunks * d->k * sizeof(uint32_t)));
    uint2* bounds = (uint2*)((char*)slots + align256((size_t)rows * nchunks * d->k * sizeof(int32_t)));
    ScanArgs a{};
    a.B = d->B; a.T = d->T; a.H_I = d->H_I; a.d_I = d->d_I; a.N = d->N; a.m = d->m;
    a.block = d->block > 0 ? d->block : 1;
    a.q_idx = d->q_idx; a.w = d->w; a.q_pos = d->q_pos; a.k_dtype = d->k_dtype; a.k_idx = d->k_idx;
    a.k_codes = d->k_codes; a.k_scales = d->k_scales;
    a.q_scales = d->q_dtype == CSA2_MXFP4 ? d->q_scales : nullptr;
    a.scores = d->out_scores; a.row_stride = d->N;
    a.block_max = d->out_block_max;
    a.nblk = (d->N + a.block - 1) / a.block;
    hipError_t e = launch_index_scan_select(a, d->k, chunk, nchunks, keys, slots, bounds, s);
    if (e != hipSuccess) return hip_status(e, "index/scan_select");
    TopkArgs t{};
    t.rows = (int)rows; t.k = d->k; t.q_pos = d->q_pos; t.N = d->N; t.m = d->m; t.len_div = 1;
    t.out_idx = d->out_idx; t.max_len = d->N;
    return hip_status(launch_topk_merge(t, nchunks, keys, slots, bounds, s), "index/topk_merge");
  }
  const int len = mode == CSA2_MODE_FULL ? d->N : d->cand_stride;
  char* wp = (char*)ws;
  float* scores = d->out_scores;
  if (!scores) {
    scores = (float*)wp;
    wp += align256((size_t)rows * len * sizeof(float));
  }
  void* tk_ws = wp;
  const size_t tk_bytes = topk_workspace_bytes((int)rows, d->k, len);

  if (len > 0) {
    ScanArgs a{};
    a.B = d->B; a.T = d->T; a.H_I = d->H_I; a.d_I = d->d_I; a.N = d->N; a.m = d->m;
    a.block = d->block > 0 ? d->block : 1;
    a.q_idx = d->q_idx; a.w = d->w; a.q_pos = d->q_pos; a.k_dtype = d->k_dtype; a.k_idx = d->k_idx;
    a.k_codes = d->k_codes; a.k_scales = d->k_scales;
    a.q_scales = d->q_dtype == CSA2_MXFP4 ? d->q_scales : nullptr;
    a.cand = mode == CSA2_MODE_REINDEX ? d->cand : nullptr;
    a.n_cand = mode == CSA2_MODE_REINDEX ? d->n_cand : nullptr;
    a.cand_stride = d->cand_stride;
    a.scores = scores; a.row_stride = len;
    a.block_max = mode == CSA2_MODE_FULL ? d->out_block_max : nullptr;
    a.nblk = (d->N + a.block - 1) / a.block;
    a.ent_base = mode == CSA2_MODE_FULL ? d->ent_base : nullptr;
    hipError_t e = launch_index_scan(a, s);
    if (e != hipSuccess) return hip_status(e, "index/scan");
  }
  TopkArgs t{};
  t.rows = (int)rows; t.k = d->k; t.scores = scores; t.row_stride = len;
  t.out_idx = d->out_idx;
  if (mode == CSA2_MODE_FULL) {
    t.q_pos = d->q_pos; t.N = d->N; t.m = d->m; t.id_base = d->ent_base;
  } else {
    t.counts = d->n_cand; t.idx_map = d->cand; t.idx_map_stride = d->cand_stride;
  }
  t.len_div = 1;
  t.max_len = len;
  t.ws = tk_ws; t.ws_bytes = tk_bytes;
  return hip_status(launch_topk(t, s), "index/topk");
}

// --------------------------------------------------------------- index + top-k, no allocation
// The workspace of csa2_index_topk_noalloc lives in this file-scope device array, one copy
// per GPU, held until the process ends.  In host code the array's name is only a stand-in:
// its device address comes from hipGetSymbolAddress, once per device, with that device
// current, and only that address is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[CSA2_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the current device's copy of `scratch` (resolved on first use on that device)
hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" int csa2_index_topk_noalloc(const csa2_index_desc* d, csa2_mode mode, void* stream) {
  int rc = check_index(d, raw(mode));
  if (rc != CSA2_OK) return rc;
  const size_t need = index_ws(d, mode);
  if (need > CSA2_NOALLOC_SCRATCH_BYTES)
    return fail(CSA2_ERR_WORKSPACE, "index (no-alloc): this call needs %zu bytes of scratch, the static array holds %zu",
                need, (size_t)CSA2_NOALLOC_SCRATCH_BYTES);
  if (need == 0) return csa2_index_topk(d, mode, nullptr, 0, stream);
  void* ws = nullptr;
  hipError_t e = scratch_of_current_device(&ws);
  if (e != hipSuccess) return hip_status(e, "index (no-alloc): scratch address");
  return csa2_index_topk(d, mode, ws, CSA2_NOALLOC_SCRATCH_BYTES, stream);
}

// --------------------------------------------------------------- hierarchical pool
static int check_hier(const csa2_hier_desc* d) {
  if (!d) return fail(CSA2_ERR_INVALID, "hier: null descriptor");
  if (d->B < 0 || d->T < 0 || d->N < 0 || d->m < 1) return fail(CSA2_ERR_INVALID, "hier: need B, T, N >= 0, m >= 1");
  if (!pow2_upto(d->block, 32)) return fail(CSA2_ERR_UNSUPPORTED, "hier: block must be a power of two <= 32");
  if (d->n_keep < 1 || d->n_keep > 4096) return fail(CSA2_ERR_UNSUPPORTED, "hier: n_keep must be in [1, 4096]");
  if ((long long)d->B * d->T == 0) return CSA2_OK;
  if (!d->q_pos || !d->block_max || !d->out_cand || !d->out_count)
    return fail(CSA2_ERR_INVALID, "hier: q_pos, block_max, out_cand, out_count are required");
  return CSA2_OK;
}

static size_t hier_ws(const csa2_hier_desc* d) {
  const size_t rows = (size_t)d->B * d->T;
  if (rows == 0) return 0;
  const int nblk = (d->N + d->block - 1) / d->block;
  return align256(rows * d->n_keep * sizeof(int32_t)) + align256(topk_workspace_bytes((int)rows, d->n_keep, nblk));
}

size_t csa2_hier_workspace_bytes(const csa2_hier_desc* d) {
  if (check_hier(d) != CSA2_OK) return 0;
  return hier_ws(d);
}

int csa2_hier_candidates(const csa2_hier_desc* d, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_hier(d);
  if (rc != CSA2_OK) return rc;
  const long long rows = (long long)d->B * d->T;
  if (rows == 0) return ok();
  const size_t need = hier_ws(d);
  if (!ws || ws_bytes < need) return fail(CSA2_ERR_WORKSPACE, "hier: workspace of %zu bytes required, %zu given", need, ws_bytes);
  hipStream_t s = (hipStream_t)stream;
  const int nblk = (d->N + d->block - 1) / d->block;
  int32_t* sel = (int32_t*)ws;
  char* tk_ws = (char*)ws + align256((size_t)rows * d->n_keep * sizeof(int32_t));
  TopkArgs t{};
  t.rows = (int)rows; t.k = d->n_keep; t.scores = d->block_max; t.row_stride = nblk;
  t.q_pos = d->q_pos; t.N = d->N; t.m = d->m; t.len_div = d->block; t.force_last = 1;
  t.out_idx = sel; t.max_len = nblk; t.ws = tk_ws;
  t.ws_bytes = topk_workspace_bytes((int)rows, d->n_keep, nblk);
  hipError_t e = launch_topk(t, s);
  if (e != hipSuccess) return hip_status(e, "hier/topk");
  return hip_status(launch_hier_expand((int)rows, d->n_keep, d->block, sel, d->q_pos, d->N, d->m, d->out_cand,
                                       d->out_count, s),
                    "hier/expand");
}

// --------------------------------------------------------------- attention
static int check_attn(const csa2_attn_desc* d) {
  if (!d) return fail(CSA2_ERR_INVALID, "attn: null descriptor");
  if (d->B < 0 || d->T < 0 || d->H < 0 || d->k < 0 || d->N < 0) return fail(CSA2_ERR_INVALID, "attn: negative size");
  if (d->c < 16 || d->c % 16 != 0) return fail(CSA2_ERR_INVALID, "attn: c must be a positive multiple of 16");
  if (d->c > 512) return fail(CSA2_ERR_UNSUPPORTED, "attn: c > 512");
  if (d->rope_dims < 0 || d->rope_dims > d->c || d->rope_dims % 2) return fail(CSA2_ERR_INVALID, "attn: rope_dims must be even and in [0, c]");
  if (d->rope_dims > 0 && !(d->rope_theta > 0.f)) return fail(CSA2_ERR_INVALID, "attn: rope_theta must be > 0");
  if (d->q_norm && !(d->eps >= 0.f)) return fail(CSA2_ERR_INVALID, "attn: eps must be >= 0");
  if (raw(d->q_dtype) != CSA2_F32 && raw(d->q_dtype) != CSA2_BF16)
    return fail(CSA2_ERR_UNSUPPORTED, "attn: q dtype must be F32 or BF16");
  if (raw(d->kv_dtype) != CSA2_F32 && raw(d->kv_dtype) != CSA2_BF16 && raw(d->kv_dtype) != CSA2_FP4_E4M3)
    return fail(CSA2_ERR_UNSUPPORTED, "attn: kv dtype must be F32, BF16 or FP4");
  if (d->kv_dtype != d->q_dtype && !(d->kv_dtype == CSA2_FP4_E4M3 && d->q_dtype == CSA2_BF16))
    return fail(CSA2_ERR_UNSUPPORTED, "attn: kv dtype must equal q dtype, or be FP4 with bf16 q");
  if (d->num_splits < 0) return fail(CSA2_ERR_INVALID, "attn: num_splits must be >= 0");
  if ((long long)d->B * d->T * d->H == 0) return CSA2_OK;
  if (!d->q || !d->q_pos || !d->out) return fail(CSA2_ERR_INVALID, "attn: q, q_pos and out are required");
  if (d->dense_m < 0) return fail(CSA2_ERR_INVALID, "attn: dense_m must be >= 0");
  if (d->dense_m > 0 && d->idx) return fail(CSA2_ERR_INVALID, "attn: dense attention takes no idx");
  if (d->dense_m == 0 && d->k > 0 && !d->idx) return fail(CSA2_ERR_INVALID, "attn: idx required when k > 0");
  if (d->k > 0 && d->N > 0) {
    if (d->kv_dtype == CSA2_FP4_E4M3 && (!d->kv_codes || !d->kv_scales))
      return fail(CSA2_ERR_INVALID, "attn: FP4 kv needs kv_codes and kv_scales");
    if (d->kv_dtype != CSA2_FP4_E4M3 && !d->kv) return fail(CSA2_ERR_INVALID, "attn: kv required");
  }
  if (d->win) {
    if ((!d->win_pos0 && !d->win_row0) || d->Lw < 0 || d->n_win < 0)
      return fail(CSA2_ERR_INVALID, "attn: window needs win_pos0 (or win_row0), Lw >= 0, n_win >= 0");
  }
  if (d->win_row0 && !d->win) return fail(CSA2_ERR_INVALID, "attn: win_row0 without a window");
  return CSA2_OK;
}

size_t csa2_attn_workspace_bytes(const csa2_attn_desc* d) {
  if (check_attn(d) != CSA2_OK) return 0;
  return attn_workspace_bytes(*d);
}

int csa2_sparse_attn(const csa2_attn_desc* d, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_attn(d);
  if (rc != CSA2_OK) return rc;
  if ((long long)d->B * d->T * d->H == 0) return ok();
  const size_t need = attn_workspace_bytes(*d);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(CSA2_ERR_WORKSPACE, "attn: workspace of %zu bytes required, %zu given", need, ws_bytes);
  return hip_status(launch_attn(*d, ws, ws_bytes, (hipStream_t)stream), "attn");
}

}  // extern "C"

// --------------------------------------------------------------- output projection
static int check_out_proj(const csa2_out_proj_desc* d) {
  if (!d) return fail(CSA2_ERR_INVALID, "out_proj: null descriptor");
  if (d->M < 0 || d->n_h < 1 || d->c < 1 || d->g < 1 || d->d_g < 1 || d->d < 1)
    return fail(CSA2_ERR_INVALID, "out_proj: need M >= 0 and positive n_h, c, g, d_g, d");
  if (d->n_h % d->g != 0) return fail(CSA2_ERR_INVALID, "out_proj: n_h must be a multiple of g");
  if ((long long)d->c * (d->n_h / d->g) % 64 != 0 || (long long)d->g * d->d_g % 64 != 0)
    return fail(CSA2_ERR_UNSUPPORTED, "out_proj: c*n_h/g and g*d_g must be multiples of 64");
  if (d->M == 0) return CSA2_OK;
  if (!d->o || !d->w1 || !d->w2 || !d->mid || !d->out)
    return fail(CSA2_ERR_INVALID, "out_proj: o, w1, w2, mid and out are required");
  return CSA2_OK;
}

int csa2_out_proj(const csa2_out_proj_desc* d, void* stream) {
  int rc = check_out_proj(d);
  if (rc != CSA2_OK) return rc;
  if (d->M == 0) return ok();
  return hip_status(launch_out_proj(*d, (hipStream_t)stream), "out_proj");
}
