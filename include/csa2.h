/* csa2.h - C ABI of libcsa2, the MI355X (gfx950) CSA2 compressed-sparse-attention hot path.
 *
 * The operations follow three web pages (cited by title and section / equation):
 *   [CSA2 column]      daiw.org, "CSA2：跨层共享的压缩稀疏注意力" (DeepSeek V4.1 Flash column)
 *   [Evolution blog]   0xnullpath, "DeepSeek 的 Attention 演进 -【DSA、CSA、CSA2】"
 *   [DSA-to-CSA notes] wineandchord, "从 DSA 到 CSA/HCA：先压缩时间轴，再决定怎样寻址"
 *
 * Conventions shared by every call
 *   - Every pointer is caller-owned device memory unless stated otherwise; the library
 *     allocates nothing and keeps no state between calls (apart from the optional,
 *     thread-local kernel-timing record).
 *   - Work is enqueued on the caller's stream `stream` (a hipStream_t; NULL = the null
 *     stream).  No call synchronises the host.
 *   - Tensors are dense, row-major, with the shapes given ([B, T, H, c] means c fastest).
 *   - bf16 values are IEEE bfloat16 bit patterns; fp32 accumulation everywhere; bf16
 *     outputs are rounded to nearest even.
 *   - Indices are int32 entry ids within their sequence; -1 marks an empty slot.
 *   - Return value: CSA2_OK, or a negative csa2_status.  Argument checks (null pointers,
 *     sizes, unsupported combinations, workspace size) all happen before any launch; on
 *     error nothing is enqueued and csa2_last_error() describes the problem.
 *     CSA2_ERR_HIP means a launch error reported by the HIP runtime.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA2_VERSION 4 /* 2: write-path, packed-sample, dense-attention and projection fields;
                          3: per-query sample bounds of index and attention over packed streams;
                          4: MXFP4 indexer queries (q_dtype, q_scales) */
#define CSA2_MAX_PACKED_SAMPLES 4096

#if defined(__GNUC__) || defined(__clang__)
#define CSA2_API __attribute__((visibility("default")))
#else
#define CSA2_API
#endif

typedef enum {
  CSA2_OK = 0,
  CSA2_ERR_INVALID = -1,     /* null required pointer, bad size, missing mode input */
  CSA2_ERR_UNSUPPORTED = -2, /* valid but not implemented: dtype combination or shape */
  CSA2_ERR_HIP = -3,         /* HIP runtime error at launch */
  CSA2_ERR_WORKSPACE = -4    /* workspace pointer NULL or smaller than *_workspace_bytes */
} csa2_status;

typedef enum {
  CSA2_F32 = 0,
  CSA2_BF16 = 1,
  /* main-KV rows in 4-bit E2M1 with one E4M3 scale per 16 channels, stored as two
   * planes: codes [.., c/2] (element 2i in the low nibble of byte i) and scales [.., c/16].
   * 512 channels -> 256 + 32 = 288 bytes per entry ([CSA2 column], "890 字节是怎么来的"). */
  CSA2_FP4_E4M3 = 2,
  /* indexer-K rows in MXFP4: E2M1 codes [.., d/2] plus one E8M0 scale per 32 values
   * [.., d/32]; 128 dims -> 64 + 4 = 68 bytes per entry (same section). */
  CSA2_MXFP4 = 3
} csa2_dtype;

/* Per-layer mode ([CSA2 column], "三种模式：谁算、谁复用"; [Evolution blog] §4.3). */
typedef enum {
  CSA2_MODE_FULL = 0,    /* score every visible entry with this layer's indexer, keep top-k */
  CSA2_MODE_REINDEX = 1, /* score only the candidate pool with this layer's indexer, keep top-k */
  CSA2_MODE_REUSE = 2    /* no indexer: the indices of the upstream Full/Reindex layer */
} csa2_mode;

/* ------------------------------------------------------------------ compressor
 * csa2_compress: the gated per-channel softmax compressor with its write epilogue.
 *   Non-overlap ([Evolution blog] §4.1; HCA eq. (22)-(23) of [DSA-to-CSA notes]):
 *     entry i of sequence b pools tokens [m*i, m*i+m): for each channel, weights are a
 *     softmax over the m logits Z^a + B^a, applied to C^a.  m = 1 is the identity.
 *   Overlap (CSA, [DSA-to-CSA notes] eq. (11)-(12)): 2m candidates per channel, the
 *     current block via (C^a, Z^a + B^a) and the previous block via (C^b, Z^b + B^b);
 *     entry 0's history has logits -inf and values 0.
 *   Epilogue ([Evolution blog] §4.1): optional RMSNorm (unit gain, eps), optional
 *     indexer-K projection K_I = x_hat * W_ik of the normalised, not yet rotated entry,
 *     then RoPE on the last rope_dims channels at position pos0[b] + m*i (adjacent pairs
 *     (c-r+2u, c-r+2u+1), angle = pos * theta^(-2u/r)).
 *   Only complete blocks are compressed: n/m entries (floor); a ragged tail is ignored.
 * Arguments:
 *   B, n, c, m: sequences, tokens per sequence, channels, block size (m >= 1).
 *   dtype: F32 or BF16, the type of ca/za/cb/zb, out and w_ik/out_ik.
 *   ca, za [B, n, c] required; cb, zb [B, n, c] required iff overlap.
 *   ba, bb: fp32 [m, c] position biases or NULL (= 0); bb used only with overlap.
 *   pos0: int32 [B] position of token 0 of each sequence, or NULL (= 0).
 *   out: [B, n/m, c] at out + b*out_batch_stride (elements; 0 means (n/m)*c).
 *   w_ik: [c, d_index] or NULL; out_ik: [B, n/m, d_index] (batch stride out_ik_batch_stride,
 *     0 means (n/m)*d_index).
 * Write path into the decode cache (the 4-bit cache rows of [CSA2 column], "890 字节是怎么来的":
 * 512 main-KV channels in 288 bytes, 128 indexer-K dims in 68 bytes; [Evolution blog] §4.1
 * stores an entry after its norm and position encoding, then quantised):
 *   dst_row: int32 [B] or NULL (= 0).  Entry i of sequence b goes to row dst_row[b] + i of
 *     every output buffer, so a decode step appends its new entry at the cache's length.
 *     For m > 1 the caller keeps the tokens of the open block and calls with the block once
 *     it is complete; with overlap it passes the previous block's C^b, Z^b rows as cb0, zb0.
 *   cb0, zb0: [B, m, c] of dtype, or NULL: with overlap, the C^b, Z^b rows of the block
 *     before entry 0, which then pools them as its history like every later entry (NULL:
 *     entry 0 is the first block of its sequence and has no history).
 *   out_codes, out_scales: if non-NULL, the entries (after RMSNorm and RoPE) are also
 *     written as FP4_E4M3 planes, codes [B, q_rows, c/2] and E4M3 scales [B, q_rows, c/16]:
 *     per 16 channels scale = E4M3(amax / 6) and code = E2M1(x / scale), both rounded to
 *     nearest with ties to the even code, codes saturated at +-6; scale 0 gives zero codes.
 *   ik_codes, ik_scales: if non-NULL (with w_ik), K_I is also written as MXFP4 planes,
 *     codes [B, q_rows, d_index/2] and E8M0 scales [B, q_rows, d_index/32]: per 32 values
 *     the exponent e = floor(log2 amax) - 2 (clamped to [-127, 127]), code = E2M1(x / 2^e)
 *     rounded as above; an all-zero group gets scale byte 127 and zero codes.
 *   q_rows: rows per sequence of the quantised planes (0 = n/m).
 *   out (and out_ik) may be NULL when the quantised planes are requested instead; at least
 *   one output of the entries is required, and w_ik needs out_ik or the MXFP4 planes.
 *   Rows outside an output's capacity (out_batch_stride / c, out_ik_batch_stride / d_index,
 *   q_rows) or below 0 are not written.  Every rounding decision is exact: the same fp32
 *   entry values always give the same bytes.
 * Packed samples ([DSA-to-CSA notes]: samples packed into one token stream must not share a
 * compression window, and a tail shorter than m is not completed by the next sample):
 *   cu_seqlens: NULL, or int32 [n_samples + 1] device offsets: sample s holds tokens
 *     [cu_seqlens[s], cu_seqlens[s+1]) of the stream (B must be 1).  Each sample is
 *     compressed on its own: its floor(len/m) entries follow those of the samples before it,
 *     its positions start at pos0[s] (pos0 is then per sample; NULL = 0), and its first entry
 *     has no history.  Offsets are clamped into [0, n] and made non-decreasing.
 *   n_samples: 1 .. CSA2_MAX_PACKED_SAMPLES.  cb0 / zb0 are not accepted with cu_seqlens.
 *   out_cu_entries: NULL or int32 [n_samples + 1]: receives the samples' entry offsets (the
 *     last one is the number of entries written).
 * Supported: c/8 a power of two, 8 <= c <= 512 (c % 16 == 0 for FP4 planes); rope_dims even
 * and <= c; with w_ik, d_index in {32, 64, 128} and c * d_index >= 1024.
 */
typedef struct {
  int B, n, c, m, overlap;
  csa2_dtype dtype;
  const void *ca, *za, *cb, *zb;
  const float *ba, *bb;
  const int32_t *pos0;
  int norm;
  float eps;
  int rope_dims;
  float rope_theta;
  void *out;
  int64_t out_batch_stride;
  const void *w_ik;
  int d_index;
  void *out_ik;
  int64_t out_ik_batch_stride;
  const int32_t *dst_row;
  uint8_t *out_codes, *out_scales;
  uint8_t *ik_codes, *ik_scales;
  int64_t q_rows;
  const void *cb0, *zb0;
  const int32_t *cu_seqlens;
  int n_samples;
  int32_t *out_cu_entries;
} csa2_compress_desc;

CSA2_API int csa2_compress(const csa2_compress_desc *d, void *stream);

/* ------------------------------------------------------------------ indexer + top-k
 * csa2_index_topk: lightning-indexer scores and top-k selection, in one of three modes.
 *   Score ([DSA-to-CSA notes] eq. (16)): I[t,s] = sum_h w[t,h] * ReLU(q_I[t,h] . K_I[s]).
 *   Visibility ([DSA-to-CSA notes] "因果边界与短滑窗"): entry j is visible to query
 *     position t iff t >= m*(j+1), i.e. n_vis(t) = min(N, floor(t/m)).
 *   Top-k ([DSA-to-CSA notes] eq. (17)): the min(k, n_vis) highest scores; ties go to the
 *     lower entry id (-0 equals +0); out_idx lists the chosen ids ascending, padded with -1.
 *   FULL: score all visible entries, optionally also the block maxima over `block`
 *     consecutive entries (only visible entries count; [CSA2 column], "解码器里的分层索引").
 *   REINDEX: score only cand[b,t,0:n_cand[b,t]] (ascending entry ids, all visible) with
 *     this layer's q_I/w, keep the top-k by (score desc, id asc) ([Evolution blog] §4.4).
 *   REUSE: out_idx = src_idx (no work if they are the same pointer).
 * Arguments:
 *   B sequences, T queries per sequence, H_I heads, d_I dims, N entries per sequence.
 *   q_idx: bf16 [B, T, H_I, d_I]; w: fp32 [B, T, H_I]; q_pos: int32 [B, T].
 *   k_dtype BF16: k_idx bf16 [B, N, d_I].  k_dtype MXFP4: k_codes [B, N, d_I/2] and
 *     k_scales [B, N, d_I/32] (bytes).
 *   cand: int32 [B, T, cand_stride], n_cand: int32 [B, T] (REINDEX).
 *   src_idx: int32 [B, T, k] (REUSE).  out_idx: int32 [B, T, k] (all modes).
 *   out_block_max: fp32 [B, T, ceil(N/block)] or NULL (FULL); entries of blocks with no
 *     visible position are left unwritten.
 *   out_scores: fp32 [B, T, N] (FULL) or [B, T, cand_stride] (REINDEX), or NULL; only
 *     visible / candidate slots are written.
 *   ws, ws_bytes: device workspace of at least csa2_index_workspace_bytes(d, mode).
 *   ent_base: NULL, or int32 [B, T] (FULL only): packed samples.  The entries of a query's
 *     own sample start at id ent_base[b,t] of the stream's entries (csa2_compress with
 *     cu_seqlens reports them in out_cu_entries), q_pos is the query's position within its
 *     sample, and it sees entries ent_base + [0, n_vis) with n_vis = min(N - ent_base,
 *     floor(q_pos/m)): no entry of another sample ([DSA-to-CSA notes], checklist "怎样验证":
 *     the indexer mask must not cross a sample boundary).  out_idx holds stream entry ids;
 *     out_scores / out_block_max are indexed by the sample-local slot.
 *   q_dtype: CSA2_BF16 (a zeroed field, 0, reads the same) for the q_idx layout above, or
 *     CSA2_MXFP4 with an MXFP4 K_I: q_idx then holds E2M1 codes [B, T, H_I, d_I/2] (dim 2i
 *     in the low nibble of byte i) and q_scales E8M0 bytes [B, T, H_I, d_I/32], the indexer
 *     QK path in FP4 on both sides ([DSA-to-CSA notes], "Lightning Indexer" and "数值与
 *     kernel": the indexer QK path is quantised to FP4).  Scores are the fp32 sums of the
 *     exact products of the decoded values, as with a bf16 q_I.  Other values of q_dtype,
 *     or MXFP4 with a BF16 K_I, fail with CSA2_ERR_UNSUPPORTED; a missing q_scales with
 *     CSA2_ERR_INVALID.
 * Supported: H_I <= 64 (heads beyond H_I are zero-padded internally), d_I in {32, 64, 128},
 *   block in {1, 2, 4, 8, 16, 32}, k <= 4096.
 */
typedef struct {
  int B, T, H_I, d_I, N, m, k;
  const void *q_idx;
  const float *w;
  const int32_t *q_pos;
  csa2_dtype k_dtype;
  const void *k_idx;
  const uint8_t *k_codes, *k_scales;
  const int32_t *cand, *n_cand;
  int cand_stride;
  const int32_t *src_idx;
  int32_t *out_idx;
  float *out_block_max;
  int block;
  float *out_scores;
  const int32_t *ent_base;
  csa2_dtype q_dtype;
  const uint8_t *q_scales;
} csa2_index_desc;

CSA2_API size_t csa2_index_workspace_bytes(const csa2_index_desc *d, csa2_mode mode);
CSA2_API int csa2_index_topk(const csa2_index_desc *d, csa2_mode mode, void *ws, size_t ws_bytes, void *stream);

/* csa2_index_topk_noalloc: csa2_index_topk without a workspace argument, for callers that
 *   cannot allocate device memory (code under HIP graph capture, tight serving loops,
 *   harnesses that forbid hipMalloc).  Same descriptor, modes, results and errors; the
 *   workspace is a static device array of CSA2_NOALLOC_SCRATCH_BYTES held by the library on
 *   each GPU it runs on until the process ends.  Calls needing more than that (see
 *   csa2_index_workspace_bytes) fail with CSA2_ERR_WORKSPACE before anything is enqueued:
 *   decode-shaped FULL calls (up to ~500 queries of 1M entries) fit, whole-prefill score
 *   matrices do not.  The call allocates nothing.  Every call on one GPU shares that GPU's
 *   array: calls that overlap in time on one GPU (other streams, other threads) race. */
#define CSA2_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
CSA2_API int csa2_index_topk_noalloc(const csa2_index_desc *d, csa2_mode mode, void *stream);

/* ------------------------------------------------------------------ hierarchical pool
 * csa2_hier_candidates: the decoder's hierarchical candidate pool ([CSA2 column],
 *   "解码器里的分层索引"; [Evolution blog] §4.4).  For each query: blocks
 *   0 .. ceil(n_vis/block)-1 with scores block_max; the latest visible block is always
 *   kept and the other n_keep-1 blocks are chosen by (score desc, block asc); the output
 *   lists the visible positions of the chosen blocks in ascending order.
 * Arguments:
 *   B, T, N, m: as for csa2_index_topk; n_vis = min(N, floor(q_pos/m)).
 *   block_max: fp32 [B, T, ceil(N/block)] (from csa2_index_topk FULL).
 *   out_cand: int32 [B, T, n_keep*block], -1 padded; out_count: int32 [B, T].
 *   ws, ws_bytes: workspace of at least csa2_hier_workspace_bytes(d).
 * Supported: n_keep <= 4096, block in {1, 2, 4, 8, 16, 32}.
 */
typedef struct {
  int B, T, N, m, block, n_keep;
  const int32_t *q_pos;
  const float *block_max;
  int32_t *out_cand;
  int32_t *out_count;
} csa2_hier_desc;

CSA2_API size_t csa2_hier_workspace_bytes(const csa2_hier_desc *d);
CSA2_API int csa2_hier_candidates(const csa2_hier_desc *d, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ sparse shared-KV MQA
 * csa2_sparse_attn: attention of every query head over its selected entries plus its
 *   sliding window ([DSA-to-CSA notes] eq. (18)-(19), (27) and "Shared-KV MQA";
 *   [CSA2 column] "保留了 CSA 的骨架").  For query (b,t) at position p = q_pos[b,t], head h:
 *     q_hat  = RoPE_p(RMSNorm(q[b,t,h]))          (RMSNorm if q_norm; unit gain, eps)
 *     rows   = kv[b, idx[b,t,j]] for idx != -1, then the window rows win[b, i] whose
 *              position win_pos0[b] + i lies in [p - window + 1, p]
 *     z_j    = scale * q_hat . row_j              (scale 0 means 1/sqrt(c))
 *     out    = sum_j e^{z_j} row_j / (sum_j e^{z_j} + e^{sink[h]}),
 *              then the last rope_dims channels rotated by -p.
 *   Each row is both key and value and is used as stored: RMSNorm and RoPE of the KV
 *   rows belong to the write path (csa2_compress).  With no rows, out = 0.
 * Arguments:
 *   q_dtype F32 or BF16: q [B, T, H, c], out [B, T, H, c] and win [B, Lw, c] share it.
 *   kv_dtype: q_dtype (kv [B, N, c]) or FP4_E4M3 (kv_codes [B, N, c/2], kv_scales [B, N, c/16]).
 *   idx: int32 [B, T, k]; ids outside [0, N) other than -1 are an error of the caller
 *     and are treated as empty.
 *   win: NULL or [B, Lw, c] with win_pos0 int32 [B]; window = n_win (0 = no window).
 *   sink: fp32 [H] or NULL (no sink term).  out_mass: fp32 [B, T, H] or NULL: receives
 *     sum_j p_j, the probability mass on real rows.
 *   ws, ws_bytes: workspace of at least csa2_attn_workspace_bytes(d) (split partials).
 *   dense_m: 0 for the selected entries of idx.  > 0 for dense attention over every
 *     visible entry, the HCA form ([DSA-to-CSA notes] eq. (20)-(26): a heavily compressed
 *     history, m' = 128 in V4, read in full without an indexer): idx must be NULL, k is
 *     ignored, and the rows are entries 0 .. n_vis-1 with n_vis = min(N, floor(p / dense_m))
 *     (an entry is visible once its block of dense_m tokens has ended: "因果边界与短滑窗"),
 *     then the window rows as above.
 *   win_row0: NULL, or int32 [B, T]: packed samples.  The window buffer win[b] holds the
 *     stream's per-token rows, and row win_row0[b,t] holds position 0 of the query's own
 *     sample (q_pos is the position within that sample).  The window is then the rows
 *     win_row0 + x for x in [max(0, p - window + 1), p], clipped to [0, Lw): it never
 *     reaches into the sample before ([DSA-to-CSA notes], checklist "怎样验证": the sliding
 *     window must not cross a sample boundary).  win_pos0 is not read.
 * Supported: c % 16 == 0, c <= 512, rope_dims even and <= c; FP4 needs bf16 q.
 *   The MFMA paths run for bf16 q, c == 512, H % 32 == 0, rope_dims <= 128; other shapes
 *   use a generic fp32 kernel with the same semantics.
 */
typedef struct {
  int B, T, H, c, k, N;
  int rope_dims;
  float rope_theta, eps, scale;
  int q_norm;
  csa2_dtype q_dtype;
  const void *q;
  const int32_t *q_pos;
  csa2_dtype kv_dtype;
  const void *kv;
  const uint8_t *kv_codes, *kv_scales;
  const int32_t *idx;
  const void *win;
  int Lw;
  const int32_t *win_pos0;
  int n_win;
  const float *sink;
  void *out;
  float *out_mass;
  int num_splits; /* row-range splits per query (0 = chosen by the library); a tuning knob
                     that does not change results beyond fp32 rounding order */
  int dense_m;
  const int32_t *win_row0;
} csa2_attn_desc;

CSA2_API size_t csa2_attn_workspace_bytes(const csa2_attn_desc *d);
CSA2_API int csa2_sparse_attn(const csa2_attn_desc *d, void *ws, size_t ws_bytes, void *stream);

/* ------------------------------------------------------------------ utilities */
CSA2_API int csa2_version(void);
/* Thread-local description of the last error of a csa2_* call on this thread ("" if none). */
CSA2_API const char *csa2_last_error(void);

/* Kernel timing ([DSA-to-CSA notes] "数值与 kernel": time every component).
 * csa2_profile_enable(1) makes every later launch on this thread be bracketed by two HIP
 * events recorded on the launch's stream; csa2_profile_collect waits for them and copies
 * up to `max` (name, milliseconds) records in launch order, then clears the record.
 * Returns the number of records written, or a negative csa2_status. */
typedef struct {
  char name[48];
  float ms;
} csa2_kernel_time;

CSA2_API int csa2_profile_enable(int on);
CSA2_API int csa2_profile_collect(csa2_kernel_time *out, int max);

/* ------------------------------------------------------------------ output projection
 * csa2_out_proj: the grouped output projection that follows the core attention ([DSA-to-CSA
 *   notes], section "Grouped output projection"): the n_h heads are split into g groups of
 *   n_h/g consecutive heads; group j's c*n_h/g output values are projected to d_g, and the
 *   concatenation of the g results (g*d_g values) is projected to d.
 * Arguments (all bf16, fp32 accumulation, results rounded to nearest even):
 *   o: [M, n_h, c], the attention output of M query tokens (csa2_sparse_attn's out).
 *   w1: [g, d_g, c*n_h/g]: group j's projection stored (output, input): mid_j = o_j w1[j]^T.
 *   w2: [d, g*d_g], likewise: out = mid w2^T.
 *   mid: [M, g*d_g], caller-provided: receives the first level (the second reads it back).
 *   out: [M, d].
 * Supported: n_h % g == 0; c*n_h/g and g*d_g multiples of 64.
 */
typedef struct {
  int M, n_h, c, g, d_g, d;
  const void *o, *w1, *w2;
  void *mid, *out;
} csa2_out_proj_desc;

CSA2_API int csa2_out_proj(const csa2_out_proj_desc *d, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
